// e4m3fn encoding shared by the quantiser and the fused SwiGLU epilogue:
// the code of x / s for a block scale s, with x / s correctly rounded (IEEE
// fp32) and then rounded to the nearest e4m3fn value.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Magnitude code of an fp32 a = |v| (sign bit clear) in e4m3fn, round to
// nearest even, saturating.  Finite e4m3fn values: subnormals m * 2^-9
// (m < 8), normals (1 + m/8) * 2^(e-7) for exponent field e = 1..15 except
// the NaN pattern 1111.111; the largest finite value is 448 (1111.110).
static __device__ __forceinline__ uint32_t e4m3_mag(uint32_t a) {
  if (a > 0x7F800000u) return 0x7Fu;  // NaN
  // from 464 (halfway between 448 and the next step, 480, which e4m3fn does
  // not have) a tie to the even mantissa already gives 448; above it
  // everything saturates to 448
  if (a >= 0x43E80000u) return 0x7Eu;
  if (a < 0x3C800000u) {  // below 2^-6: the subnormal grid, step 2^-9
    // |v| * 2^9 is exact; rint rounds half to even; 8 lands on 2^-6 (0x08)
    return (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  // normal: keep 3 of the 23 fraction bits, round the other 20 half to even;
  // a carry out of the mantissa moves into the exponent field as it should
  uint32_t code = ((((a >> 23) - 127u + 7u) << 3) | ((a >> 20) & 7u));
  const uint32_t rem = a & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1u;
  return code;
}

// Codes x / s for one block.  x / s, correctly rounded, without a division
// per element: with the correctly rounded reciprocal rs of s, q0 = x rs and
// one exact-residual correction q0 + (x - q0 s) rs give the correctly rounded
// quotient as long as the residual does not underflow.  Blocks with
// amax < 2^-60 are first scaled by 2^64 (x and s alike: the quotient does not
// change), which keeps every element that can reach a non-zero code clear of
// underflow.  Checked exhaustively on MI355X: the e4m3 code equals that of
// the IEEE quotient for every pair of positive bf16 values x <= amax.  An
// infinite scale (a block holding an infinity) takes the division itself.
// The code's sign is x's (s > 0): NaN and -0 keep their sign.
struct E4m3Quotient {
  float s, kk, sk, rs;
  bool exact_div;
  __device__ __forceinline__ E4m3Quotient(float amax, float scale)
      : s(scale), kk(amax < 0x1p-60f ? 0x1p64f : 1.f) {
    sk = s * kk;
    rs = 1.f / sk;
    exact_div = !(s < __builtin_inff());
  }
  __device__ __forceinline__ uint32_t code(float v) const {
    float q;
    if (exact_div) {
      q = v / s;
    } else {
      const float vk = v * kk, q0 = vk * rs;
      q = __builtin_fmaf(__builtin_fmaf(-q0, sk, vk), rs, q0);
    }
    return e4m3_mag(__float_as_uint(q) & 0x7FFFFFFFu) | ((__float_as_uint(v) >> 24) & 0x80u);
  }
};
