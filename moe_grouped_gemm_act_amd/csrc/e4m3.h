// e4m3fn encoding shared by the quantiser and the fused SwiGLU epilogue:
// the code of x / s for a block scale s, with x / s correctly rounded (IEEE
// fp32) and then rounded to the nearest e4m3fn value, ties to even,
// magnitudes past 448 saturating to 448, NaN to the NaN code; each code
// carries the sign of x.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// x / s correctly rounded, without a division per element: with the
// correctly rounded reciprocal rs of s, q0 = x rs and one exact-residual
// correction q0 + (x - q0 s) rs give the correctly rounded quotient as long
// as the residual does not underflow.  This is Markstein's FMA quotient
// correction (P. W. Markstein, "Computation of elementary functions on the
// IBM RISC System/6000 processor", IBM J. Res. Develop. 34(1), 1990): the
// residual x - q0 s is exact in one fused multiply-add, and one more FMA
// with the correctly rounded reciprocal rounds the quotient correctly.  Blocks with amax < 2^-60 are first
// scaled by 2^64 (x and s alike: the quotient does not change), which keeps
// every element that can reach a non-zero code clear of underflow.  A scale
// of 0 (an underflowed amax / 448) or infinity (a block holding an infinity)
// takes x * (1 / s), which is x / s there: +-inf or NaN, and +-0 or NaN.
// Checked exhaustively on MI355X: the resulting e4m3 code equals that of
// the IEEE quotient for every pair of positive bf16 values x <= amax.
struct E4m3Quotient {
  float kk, sk, rs;
  bool special;
  __device__ __forceinline__ E4m3Quotient(float amax, float s)
      : kk(amax < 0x1p-60f ? 0x1p64f : 1.f) {
    sk = s * kk;
    rs = 1.f / sk;
    special = !(s > 0.f && s < __builtin_inff());
  }
  __device__ __forceinline__ float quotient(float v) const {
    const float vk = v * kk, q0 = vk * rs;
    const float q = __builtin_fmaf(__builtin_fmaf(-q0, sk, vk), rs, q0);
    return special ? v * rs : q;
  }
};

// Saturation to the largest finite e4m3fn value; NaN passes (the compare is
// false for it).
static __device__ __forceinline__ float e4m3_sat(float q) {
  return __builtin_fabsf(q) > 448.f ? __builtin_copysignf(448.f, q) : q;
}

// Four codes, byte i from quotient qi, packed little-endian.  The hardware
// conversion (v_cvt_pk_fp8_f32, OCP e4m3fn on gfx950) rounds to nearest
// even; checked on MI355X against a bit-level encoder for every fp32 value
// of magnitude below 464.  Past 448 it would give NaN, hence the saturation
// first.  It writes NaN as 0xFF whatever the sign, so each code takes its
// sign bit from xi (qi has the sign of xi for every other input).
static __device__ __forceinline__ uint32_t e4m3_pack4(float q0, float q1, float q2, float q3,
                                                      float x0, float x1, float x2, float x3) {
  uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(q0), e4m3_sat(q1), 0, false);
  c = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(q2), e4m3_sat(q3), c, true);
  const uint32_t sg = ((__float_as_uint(x0) >> 24) & 0x80u) | ((__float_as_uint(x1) >> 16) & 0x8000u) |
                      ((__float_as_uint(x2) >> 8) & 0x800000u) | (__float_as_uint(x3) & 0x80000000u);
  return (c & 0x7F7F7F7Fu) | sg;
}
