// 1x128 activation quantisation for gfx950: bf16 [M][K] -> e4m3fn codes
// [M][K] and fp32 scales [K/128][M], the layout the GEMM reads.
//
// The pages leave the FP8 conversion of activations to the caller (kakushin,
// "Hvorfor FP8 og FP4 er interessant": scales, rounding and memory layout
// must be handled right for low precision to work).  With the 1x128
// granularity the GEMM reads, each 128-wide K block x of a row gets
//   s = amax|x| / 448        (IEEE fp32 division; 1 for an all-zero block;
//                             NaN elements take no part in the maximum)
// and codes e4m3(x / s): IEEE fp32 division, then the nearest e4m3fn value,
// ties to the even code, magnitudes past 448 saturating to 448, NaN to the
// NaN code; every code takes the sign of x.
//
// HBM-bound: 2 bytes read and 1 written per element, plus 4 per 128.  A
// workgroup takes 64 rows of one K block; four threads share a row (32
// elements, four 16-byte loads each) and meet in a two-step lane exchange
// for the block maximum; the 64 scales of the block are one contiguous run
// of sa.  (One wave per row with 1 KB row reads measured slower.)

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8gemm.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t qrsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

// Magnitude code of an fp32 a = |v| (sign bit clear) in e4m3fn, round to
// nearest even, saturating.  Finite e4m3fn values: subnormals m * 2^-9
// (m < 8), normals (1 + m/8) * 2^(e-7) for exponent field e = 1..15 except
// the NaN pattern 1111.111; the largest finite value is 448 (1111.110).
__device__ __forceinline__ uint32_t e4m3_mag(uint32_t a) {
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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

constexpr int QROWS = 64;  // rows per workgroup

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t *X, uint8_t *A, float *sa,
                                                    int M, int K) {
  const int tid = threadIdx.x, row = tid >> 2, q = tid & 3;
  const int kb = blockIdx.y, m = blockIdx.x * QROWS + row;
  const bool live = m < M;
  // elements [kb*128 + q*32, +32) of row m: four 16-byte loads; rows past M
  // read out of range (zeros, no traffic)
  const __amdgpu_buffer_rsrc_t rx = qrsrc(X, (uint32_t)M * K * 2);
  const uint32_t off = live ? ((uint32_t)m * K + kb * 128 + q * 32) * 2 : 0x80000000u;
  u32x4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + i * 16, 0, 0));
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[i * 8 + 2 * j] = bf16_lo(w[i][j]);
      x[i * 8 + 2 * j + 1] = bf16_hi(w[i][j]);
    }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));  // NaN operands are skipped
  // the four threads of a row are lanes 4r' .. 4r'+3 of the wave
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const float s = amax == 0.f ? 1.f : amax / 448.f;
  // x / s, correctly rounded, without a division per element: with the
  // correctly rounded reciprocal rs of s, q0 = x rs and one exact-residual
  // correction q0 + (x - q0 s) rs gives the correctly rounded quotient as long
  // as the residual does not underflow.  Blocks with amax < 2^-60 are first
  // scaled by 2^64 (x and s alike: the quotient does not change), which keeps
  // every element that can reach a non-zero code clear of underflow.  Checked
  // exhaustively on MI355X: the e4m3 code equals that of the IEEE quotient
  // for every pair of positive bf16 values x <= amax.  An infinite scale (a
  // block holding an infinity) takes the division itself.
  const float kk = amax < 0x1p-60f ? 0x1p64f : 1.f;
  const float sk = s * kk, rs = 1.f / sk;
  const bool exact_div = !(s < __builtin_inff());
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w4 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = x[4 * i + e];
      float qv;
      if (exact_div) {
        qv = v / s;
      } else {
        const float vk = v * kk, q0 = vk * rs;
        qv = __builtin_fmaf(__builtin_fmaf(-q0, sk, vk), rs, q0);
      }
      // the code's sign is x's (s > 0): NaN and -0 keep their sign
      const uint32_t code =
          e4m3_mag(__float_as_uint(qv) & 0x7FFFFFFFu) | ((__float_as_uint(v) >> 24) & 0x80u);
      w4 |= code << (8 * e);
    }
    c[i] = w4;
  }
  if (live) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(A + (size_t)m * K + kb * 128 + q * 32);
    dst[0] = u32x4{c[0], c[1], c[2], c[3]};
    dst[1] = u32x4{c[4], c[5], c[6], c[7]};
    if (q == 0) sa[(size_t)kb * M + m] = s;
  }
}

}  // namespace

extern "C" int quantize_fp8_1x128(const void *X, void *A, float *sa, int M, int K, void *stream) {
  if (M < 0 || K < 0) return FP8GEMM_INVALID_ARG;
  if (M == 0 || K == 0) return FP8GEMM_OK;
  if (!X || !A || !sa) return FP8GEMM_INVALID_ARG;
  if (K % 128 != 0) return FP8GEMM_UNSUPPORTED_SHAPE;
  if ((long long)M * K * 2 >= (1LL << 31)) return FP8GEMM_UNSUPPORTED_SHAPE;
  if (reinterpret_cast<uintptr_t>(X) % 16 || reinterpret_cast<uintptr_t>(A) % 16 ||
      reinterpret_cast<uintptr_t>(sa) % 4)
    return FP8GEMM_MISALIGNED;
  hipLaunchKernelGGL(quant_kernel, dim3((M + QROWS - 1) / QROWS, K / 128), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t *>(X),
                     static_cast<uint8_t *>(A), sa, M, K);
  return hipGetLastError() == hipSuccess ? FP8GEMM_OK : FP8GEMM_LAUNCH_FAILED;
}
