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
// of sa.  (One wave per row with 1 KB row reads measured slower.)  The grid
// runs K blocks fastest, so the workgroups in flight read whole rows
// together: 9-20% faster than row groups fastest at K = 16384, 18432 and
// 1536 (8% slower at K = 7168).  Codes and scales go out with plain stores:
// the GEMM reads them next, and the quantise-then-GEMM pair measured the same
// or faster with them than with non-temporal stores.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "e4m3.h"
#include "fp8gemm.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t qrsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

constexpr int QROWS = 64;  // rows per workgroup

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t *X, uint8_t *A, float *sa,
                                                    int M, int K) {
  const int tid = threadIdx.x, row = tid >> 2, q = tid & 3;
  const int kb = blockIdx.x, m = blockIdx.y * QROWS + row;
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
  const E4m3Quotient qd(amax, s);
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    c[i] = e4m3_pack4(qd.quotient(x[4 * i]), qd.quotient(x[4 * i + 1]), qd.quotient(x[4 * i + 2]),
                      qd.quotient(x[4 * i + 3]), x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  if (live) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(A + (size_t)m * K + kb * 128 + q * 32);
    // plain stores: the GEMM that follows reads these codes and scales (the
    // quantise-then-GEMM pair measured the same or faster than with
    // non-temporal stores)
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
  if ((M + QROWS - 1) / QROWS > 65535) return FP8GEMM_UNSUPPORTED_SHAPE;
  const uint16_t *x = static_cast<const uint16_t *>(X);
  uint8_t *a = static_cast<uint8_t *>(A);
  void *args[] = {&x, &a, &sa, &M, &K};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&quant_kernel),
                                       dim3(K / 128, (M + QROWS - 1) / QROWS), dim3(256), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8GEMM_OK : FP8GEMM_LAUNCH_FAILED;
}
