// libfp8gemm: FP8 e4m3fn NT GEMM with 1x128 / 128x128 fp32 block scales and
// bf16 output, dense and MoE grouped (contiguous, masked), for gfx950.
//
// Method (DeepGEMM pages, GeekNews summary "Topic Body"): FP8 GEMM with the
// fine-grained scaling of DeepSeek-V3; the tensor-core partial sum of each
// scale block is "promoted" into a higher-precision accumulator on the
// general-purpose cores because FP8 tensor-core accumulation is imprecise.
// The pages describe that schedule for Hopper (TMA staging, warp
// specialisation, JIT per shape); none of that is reused.  Here:
//
//   * one v_mfma_scale_f32_16x16x128_f8f6f4 (E8M0 scales fixed at 2^0)
//     covers a whole 128-wide K block of a 16x16 output sub-tile, so its fp32
//     result IS the block's partial sum: promotion is one VALU FMA per output
//     element per block, acc += p * (sa * sb), with no extra accumulator tile;
//   * the MFMA computes the TRANSPOSED sub-tile (weights as the first
//     operand), so the 4 results a lane holds share one activation row m and
//     four consecutive weight rows n inside one 128-row scale block: the
//     combined scale sa[kb][m] * sb[n/128][kb] is one register per lane per
//     sub-tile column, and the bf16 results of a lane are 8 contiguous bytes
//     of a row of D;
//   * A and B tiles are staged global -> registers -> LDS in a two-stage
//     ring with an XOR swizzle of the 16-byte chunks so that fragment reads
//     are bank-conflict free;
//   * the K order inside a block is irrelevant to the sum, so each lane's
//     32-byte MFMA operand is two 16-byte chunks (c, c+4) of the 128-byte
//     row and A and B use the same chunk mapping.
//
// The grouped layouts reuse the same body (GeekNews "성능 평가"): contiguous
// tiles look up their expert from m_indices; masked tiles read the expert's
// device-side row count and tiles past it exit before loading anything.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>

#include "fp8gemm.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 128;        // K block = one scale block = one MFMA's K
constexpr int THREADS = 256;   // 4 waves of 64

enum Layout { DENSE = 0, CONTIG = 1, MASKED = 2 };

struct Args {
  const uint8_t *A;
  const float *sa;
  const uint8_t *B;
  const float *sb;
  uint16_t *D;
  int M, N, K, G;
  const int32_t *idx;  // m_indices (CONTIG) or masked_m (MASKED)
  int tiles_m, tiles_n;
};

// XOR key of an LDS row: 16-byte chunk c of row r sits at position
// c ^ key(r).  Rows r and r+1 share a 256-byte bank window and rows r, r+8
// share banks; this key makes any 8 consecutive rows, and the 8 even / 8 odd
// rows of a 16-row fragment, hit distinct chunks.  It depends on r mod 16
// only, so every 16-row fragment of a tile has the same per-lane pattern and
// the compiler can address all of them from one base with immediate offsets.
__device__ __forceinline__ int row_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int chunk_pos(int chunk, int row) { return (chunk ^ row_key(row)) << 4; }

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ v8i frag(const uint8_t *row_ptr, int row, int g) {
  u32x4 lo = *reinterpret_cast<const u32x4 *>(row_ptr + chunk_pos(g, row));
  u32x4 hi = *reinterpret_cast<const u32x4 *>(row_ptr + chunk_pos(g + 4, row));
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Block tile BM (rows of A / D) x BN (rows of B / columns of D), 4 waves in
// a 2 x 2 grid, each wave owning (BM/2) x (BN/2).
template <int BM, int BN, int LAYOUT>
__global__ __launch_bounds__(THREADS) void gemm_kernel(Args a) {
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 16, TN = WN / 16;
  constexpr int CA = BM * 8 / THREADS, CB = BN * 8 / THREADS;  // 16-byte chunks per thread
  static_assert(CA >= 1 && CB >= 1 && WN <= 128 && 128 % WN == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BM + BN) * BK];
  __shared__ int s_group;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int tile = blockIdx.x;
  const int m0 = (tile % a.tiles_m) * BM, n0 = (tile / a.tiles_m) * BN;
  const int M = a.M, N = a.N, K = a.K;
  const int Kb = K / BK, Nb = (N + 127) / 128;

  const uint8_t *A = a.A, *B = a.B;
  const float *sa = a.sa, *sb = a.sb;
  uint16_t *D = a.D;
  int mvalid = M, g = 0;
  if (LAYOUT == MASKED) {
    g = blockIdx.y;
    const int c = a.idx[g];
    mvalid = c < 0 ? 0 : (c > M ? M : c);
    if (m0 >= mvalid) return;  // whole tile masked: nothing loaded, nothing written
    A += (size_t)g * M * K;
    sa += (size_t)g * Kb * M;
    D += (size_t)g * M * N;
  }
  if (LAYOUT == CONTIG) {
    if (tid == 0) s_group = -1;
    __syncthreads();
    if (tid < BM && m0 + tid < M) {
      const int v = a.idx[m0 + tid];
      if (v >= 0 && v < a.G) atomicMax(&s_group, v);
    }
    __syncthreads();
    g = s_group;
    if (g < 0) return;  // all padding
  }
  if (LAYOUT != DENSE) {
    B += (size_t)g * N * K;
    sb += (size_t)g * Nb * Kb;
  }

  // global -> LDS chunk assignment: chunk c = tid + 256 i covers row c/8,
  // 16-byte column c%8; 8 consecutive threads read one 128-byte line.
  const uint8_t *gsrc[CA + CB];
  int ldst[CA + CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + THREADS * i, r = c >> 3, col = c & 7;
    const int row = min(m0 + r, M - 1);
    gsrc[i] = A + (size_t)row * K + col * 16;
    ldst[i] = r * BK + chunk_pos(col, r);
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + THREADS * i, r = c >> 3, col = c & 7;
    const int row = min(n0 + r, N - 1);
    gsrc[CA + i] = B + (size_t)row * K + col * 16;
    ldst[CA + i] = BM * BK + r * BK + chunk_pos(col, r);
  }
  u32x4 stage[CA + CB];

  const int fr = lane & 15, fg = lane >> 4;
  int srow[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) srow[t] = min(m0 + wm * WM + t * 16 + fr, M - 1);
  const int nb = min((n0 + wn * WN) / 128, Nb - 1);
  const float *sbp = sb + (size_t)nb * Kb;

  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  if (Kb > 0) {
#pragma unroll
    for (int i = 0; i < CA + CB; ++i) stage[i] = *reinterpret_cast<const u32x4 *>(gsrc[i]);
#pragma unroll
    for (int i = 0; i < CA + CB; ++i) *reinterpret_cast<u32x4 *>(&smem[0][ldst[i]]) = stage[i];
  }
  __syncthreads();

  for (int kb = 0; kb < Kb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < Kb) {
#pragma unroll
      for (int i = 0; i < CA + CB; ++i)
        stage[i] = *reinterpret_cast<const u32x4 *>(gsrc[i] + (size_t)(kb + 1) * BK);
    }
    const float sbv = sbp[kb];
    float s[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) s[t] = sa[(size_t)kb * M + srow[t]] * sbv;

    const uint8_t *As = smem[cur], *Bs = smem[cur] + BM * BK;
    v8i bfr[TN], afr[TM];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int row = wn * WN + t * 16 + fr;
      bfr[t] = frag(Bs + row * BK, row, fg);
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int row = wm * WM + t * 16 + fr;
      afr[t] = frag(As + row * BK, row, fg);
    }
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bfr[i], afr[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], s[j], acc[i][j][r]);
      }

    if (kb + 1 < Kb) {
#pragma unroll
      for (int i = 0; i < CA + CB; ++i)
        *reinterpret_cast<u32x4 *>(&smem[cur ^ 1][ldst[i]]) = stage[i];
    }
    __syncthreads();
  }

  // epilogue: lane holds D[m][n .. n+3] for each (sub-tile row i, column j)
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = m0 + wm * WM + j * 16 + fr;
    bool ok = m < mvalid;
    if (LAYOUT == CONTIG) ok = m < M && a.idx[m] == g;
    if (!ok) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int n = n0 + wn * WN + i * 16 + 4 * fg;
      uint16_t *dp = D + (size_t)m * N + n;
      const uint32_t b0 = bf16_bits(acc[i][j][0]), b1 = bf16_bits(acc[i][j][1]);
      const uint32_t b2 = bf16_bits(acc[i][j][2]), b3 = bf16_bits(acc[i][j][3]);
      if ((N & 3) == 0 && n + 3 < N) {
        *reinterpret_cast<u32x2 *>(dp) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
      } else {
        if (n < N) dp[0] = (uint16_t)b0;
        if (n + 1 < N) dp[1] = (uint16_t)b1;
        if (n + 2 < N) dp[2] = (uint16_t)b2;
        if (n + 3 < N) dp[3] = (uint16_t)b3;
      }
    }
  }
}

// Direct-to-LDS loads (global_load_lds): each lane's `bytes` from global
// memory land at lds + lane * bytes.  Kept in a device function: written in a
// kernel template, the builtin makes the host pass drop the kernel's stub.
__device__ __forceinline__ void dma16(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (vmcnt: bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their no-wait maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }

// ---------------------------------------------------------------------------
// Large-M kernel (prefill and MoE grouped shapes): compute bound.
//
// Block tile BN = WGN * TN * 16 weight rows by BM = WGM * TM * 16 activation
// rows.  Six waves: four compute waves in a WGN x WGM grid, each owning a
// (TN * 16) x (TM * 16) tile (per K block it reads TN + TM operand fragments
// from LDS for TN * TM MFMAs), and two loader waves.  The loaders move each
// K block's activation rows, weight rows and activation scales with
// direct-to-LDS loads (global_load_lds: 16 bytes per lane, one 128-byte row
// per 8 lanes, the lane -> source mapping applying the XOR swizzle) into a
// ring of STAGES slots, STAGES - 1 blocks ahead, and wait for them with an
// explicit vmcnt; one bare barrier per K block hands a slot over.  Because
// vector-memory counters are per wave, the compute waves never wait on the
// loads in flight (they issue none), and the loaders never stall on LDS
// reads.  The weight scales of the tile's K range sit in LDS, loaded once.
constexpr int TK_THREADS = 384;

template <int WGN, int WGM, int TN, int TM, int STAGES, int LAYOUT>
__global__ __launch_bounds__(TK_THREADS) void tile_kernel(Args a) {
  constexpr int BN = WGN * TN * 16, BM = WGM * TM * 16;
  constexpr int ROWS = BM + BN;
  constexpr int SLOT = ROWS * BK + BM * 4;  // operand rows, then the BM activation scales
  constexpr int OCT = ROWS / 8;             // 1 KB row groups per slot
  constexpr int DMA = OCT / 2;              // row-group loads per loader wave per slot
  constexpr int SDMA = BM / 128;            // 64-float scale loads per loader wave per slot
  constexpr int PER_G = DMA + SDMA;         // vector memory instructions per loader per slot
  constexpr int MAXKB = 160;                // K <= 20480 for the weight-scale preload
  static_assert(WGN * WGM == 4 && OCT % 2 == 0 && BM % 128 == 0 && 128 % (TN * 16) == 0,
                "tile shape");
  static_assert(PER_G * (STAGES - 1) < 64, "loads in flight per loader must fit vmcnt");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES][SLOT];
  __shared__ float s_sb[BN > 128 ? 2 : 1][MAXKB];
  __shared__ int s_group;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fg = lane >> 4;
  const int M = a.M, N = a.N, K = a.K, Kb = K / BK, Nb = (N + 127) / 128;

  // tile order: workgroup ids are dealt to the 8 XCDs round robin; give each
  // XCD a contiguous run of tiles, walked GROUPN weight tiles at a time with
  // the activation tiles inside, so concurrent tiles on one XCD share panels
  constexpr int GROUPN = 4;
  const int T = a.tiles_m * a.tiles_n;
  int tile = blockIdx.x;
  {
    const int x = tile % 8, l = tile / 8, per = T / 8, rem = T % 8;
    tile = x * per + min(x, rem) + l;
  }
  int tn, tm;
  {
    const int gsz = GROUPN * a.tiles_m, grp = tile / gsz, in = tile % gsz;
    const int gw = min(GROUPN, a.tiles_n - grp * GROUPN);
    tn = grp * GROUPN + in % gw;
    tm = in / gw;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  const uint8_t *A = a.A, *B = a.B;
  const float *sa = a.sa, *sb = a.sb;
  uint16_t *D = a.D;
  int mvalid = M, g = 0;
  if (LAYOUT == MASKED) {
    g = blockIdx.y;
    const int c = a.idx[g];
    mvalid = c < 0 ? 0 : (c > M ? M : c);
    if (m0 >= mvalid) return;  // whole tile masked: nothing loaded, nothing written
    A += (size_t)g * M * K;
    sa += (size_t)g * Kb * M;
    D += (size_t)g * M * N;
  }
  if (LAYOUT == CONTIG) {
    if (tid == 0) s_group = -1;
    __syncthreads();
    if (tid < BM && m0 + tid < M) {
      const int v = a.idx[m0 + tid];
      if (v >= 0 && v < a.G) atomicMax(&s_group, v);
    }
    __syncthreads();
    g = s_group;
    if (g < 0) return;  // all padding
  }
  if (LAYOUT != DENSE) {
    B += (size_t)g * N * K;
    sb += (size_t)g * Nb * Kb;
  }
  for (int i = tid; i < (BN > 128 ? 2 : 1) * Kb; i += TK_THREADS) {
    const int h = i / Kb, kb = i % Kb;
    s_sb[h][kb] = sb[(size_t)min(n0 / 128 + h, Nb - 1) * Kb + kb];
  }

  if (wave >= 4) {
    // ---------------- loader waves ----------------
    const int L = wave - 4;
    // q-th row-group load: rows (L + 2q) * 8 .. + 7 of the slot; lane l ->
    // row + l / 8, physical chunk l % 8 holding logical chunk (l % 8) ^ key(row)
    uint32_t off[DMA];  // byte offsets from A (rows < BM) or B (the rest); < 2^31
#pragma unroll
    for (int q = 0; q < DMA; ++q) {
      const int r = (L + 2 * q) * 8 + (lane >> 3);
      const int col = (lane & 7) ^ row_key(r);
      off[q] = (uint32_t)(r < BM ? min(m0 + r, M - 1) : min(n0 + r - BM, N - 1)) * K + col * 16;
    }
    uint32_t soff[SDMA];  // scale floats (L + 2j) * 64 + lane of the tile's rows
#pragma unroll
    for (int j = 0; j < SDMA; ++j) soff[j] = (uint32_t)min(m0 + (L + 2 * j) * 64 + lane, M - 1);
    // G(t): K block t (clamped: blocks past the end re-read the last one and
    // are never consumed) -> slot t % STAGES
#define TK_G(t)                                                                               \
  do {                                                                                        \
    const int kb_ = min((t), Kb - 1);                                                         \
    uint8_t *sl_ = lds[(t) % STAGES];                                                         \
    _Pragma("unroll") for (int q = 0; q < DMA; ++q)                                          \
        dma16(((L + 2 * q) * 8 < BM ? A : B) + off[q] + (uint32_t)kb_ * BK,                   \
              sl_ + (L + 2 * q) * 1024);                                                      \
    _Pragma("unroll") for (int j = 0; j < SDMA; ++j)                                          \
        dma4(sa + soff[j] + (uint32_t)kb_ * M, sl_ + ROWS * BK + (L + 2 * j) * 256);          \
  } while (0)
    __syncthreads();  // weight scales visible (before any load is in flight: this
                      // barrier drains the vector-memory queue)
    if (Kb > 0) {
#pragma unroll
      for (int t = 0; t < STAGES - 1; ++t) TK_G(t);
    }
    for (int t0 = 0; t0 < Kb; t0 += STAGES) {
#pragma unroll
      for (int u = 0; u < STAGES; ++u) {
        const int t = t0 + u;
        if (t >= Kb) break;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_G * (STAGES - 2)));  // my loads of block t landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // ... and everyone's; all compute waves are past block t - 1
        asm volatile("" ::: "memory");
        TK_G(t + STAGES - 1);
      }
    }
#undef TK_G
    __builtin_amdgcn_s_waitcnt(0);  // nothing may still write LDS when the workgroup ends
    return;
  }

  // ---------------- compute waves ----------------
  const int wn = wave % WGN, wm = wave / WGN;
  const int hsb = (wn * TN * 16) / 128;  // which weight-scale block this wave's rows use
  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // weight scales visible

  for (int t0 = 0; t0 < Kb; t0 += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int t = t0 + u;
      if (t >= Kb) break;
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();  // block t is in slot u
      asm volatile("" ::: "memory");
      const uint8_t *sl = lds[u];
      const float *ssl = reinterpret_cast<const float *>(sl + ROWS * BK);
      const float sbv = s_sb[hsb][t];
      v8i bfr[TN];
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int row = BM + (wn * TN + i) * 16 + fr;
        bfr[i] = frag(sl + row * BK, row, fg);
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int row = (wm * TM + j) * 16 + fr;
        const v8i afr = frag(sl + row * BK, row, fg);
        const float sc = ssl[row] * sbv;
        v4f pr[TN];
#pragma unroll
        for (int i = 0; i < TN; ++i)
          pr[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bfr[i], afr, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[i][r], sc, acc[i][j][r]);
      }
    }
  }

#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = m0 + (wm * TM + j) * 16 + fr;
    bool ok = m < mvalid;
    if (LAYOUT == CONTIG) ok = m < M && a.idx[m] == g;
    if (!ok) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int n = n0 + (wn * TN + i) * 16 + 4 * fg;
      uint16_t *dp = D + (size_t)m * N + n;
      const uint32_t b0 = bf16_bits(acc[i][j][0]), b1 = bf16_bits(acc[i][j][1]);
      const uint32_t b2 = bf16_bits(acc[i][j][2]), b3 = bf16_bits(acc[i][j][3]);
      if ((N & 3) == 0 && n + 3 < N) {
        *reinterpret_cast<u32x2 *>(dp) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
      } else {
        if (n < N) dp[0] = (uint16_t)b0;
        if (n + 1 < N) dp[1] = (uint16_t)b1;
        if (n + 2 < N) dp[2] = (uint16_t)b2;
        if (n + 3 < N) dp[3] = (uint16_t)b3;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-M kernel (decode shapes, M <= 128): the weights are the HBM stream.
//
// A workgroup owns MROWS = 16 * MG activation rows, BN = 64 * NBW weight
// rows and a range of K blocks; wave w owns weight rows [w BN/4, (w+1) BN/4)
// and all activation rows.  Each K block's activation and weight tiles are
// read with whole 128-byte rows per 8 lanes (a wave instruction covers 8
// full lines: the L1 path sustains about 3.5x the bandwidth it gives to
// MFMA-fragment-shaped requests, which touch 16 half lines each) into a
// two-slot swizzled LDS ring, staged through registers two blocks ahead;
// the MFMA fragments are then read from LDS.  Loads past the end of the K
// range use buffer offsets beyond the resource, which return zeros without
// touching memory.
//
// When the output alone gives too few workgroups to cover the chip, K is
// also split over `splits` workgroups per output tile: each writes its fp32
// partial tile to a workspace with coherent (sc1) stores, waits for them to
// land, and counts in on a per-tile counter; the last to arrive reads the
// other partials with coherent loads, adds all of them in split order,
// rounds to bf16, stores, and re-arms the counter.  The result is
// deterministic, and no agent-wide cache writeback or invalidate is issued
// (those flush the whole L2 of an XCD).
struct SkArgs {
  const uint8_t *A;
  const float *sa;
  const uint8_t *B;
  const float *sb;
  uint16_t *D;
  int M, N, K;
  int splits, kb_per_split;
  float *ws;
  unsigned *counters;
};

constexpr uint32_t OOB = 0x80000000u;  // buffer offset past any resource: reads zeros
#ifndef SK_RS
#define SK_RS 2  // register sets: K blocks staged ahead (deeper measured slower on MI355X)
#endif

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

template <int MG, int NBW, int RS>
__global__ __launch_bounds__(THREADS) void skinny_kernel(SkArgs a) {
  constexpr int MROWS = 16 * MG, BN = 64 * NBW;
  constexpr int U = RS % 2 == 0 ? RS : 2 * RS;  // loop unroll: register set and LDS slot indices static
  constexpr int CH = (MROWS + BN) * 8 / THREADS;  // 16-byte chunks per thread per K block
  constexpr int CHA = MROWS * 8 / THREADS;         // of which activation chunks (the first ones)
  constexpr int SLOT = (MROWS + BN) * BK;
  static_assert(MROWS * 8 % THREADS == 0 && BN * 8 % THREADS == 0 && 128 % BN == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][SLOT];
  __shared__ float ssa[2][THREADS];  // sa of the slot's K block; entries >= MROWS unused
  __shared__ float ssb[2][THREADS];  // sb of the slot's K block, replicated (no ALU on loads
                                     // before they reach LDS: the compiler would hoist it)
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fg = lane >> 4;
  const int ntile = blockIdx.x, split = blockIdx.y, mtile = blockIdx.z;
  const int n0 = ntile * BN, m0 = mtile * MROWS;
  const int M = a.M, N = a.N, K = a.K, Kb = K / BK;
  const int kb0 = split * a.kb_per_split;
  const int kb1 = min(Kb, kb0 + a.kb_per_split);
  const int nk = max(kb1 - kb0, 0);

  const __amdgpu_buffer_rsrc_t ra = rsrc(a.A, (uint32_t)M * K);
  const __amdgpu_buffer_rsrc_t rb = rsrc(a.B, (uint32_t)N * K);
  const __amdgpu_buffer_rsrc_t rs = rsrc(a.sa, (uint32_t)M * Kb * 4);
  // chunk i of this thread: row r = c / 8 of the slot (activation rows first), 16-byte column c % 8
  uint32_t goff[CH];
  int loff[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + THREADS * i, r = c >> 3, col = c & 7;
    const int grow = r < MROWS ? min(m0 + r, M - 1) : min(n0 + r - MROWS, N - 1);
    goff[i] = (uint32_t)grow * K + col * 16;
    loff[i] = r * BK + chunk_pos(col, r);
  }
  const uint32_t soff = (uint32_t)min(m0 + tid, M - 1) * 4;
  const __amdgpu_buffer_rsrc_t rsb = rsrc(a.sb + (size_t)(n0 / 128) * Kb, (uint32_t)Kb * 4);

  u32x4 st[RS][CH];
  float sst[RS], sbt[RS];
  // G(t): global -> registers, K block kb0 + t, register set t % RS (zeros past the range)
#define SK_G(t)                                                                               \
  do {                                                                                        \
    const bool ok_ = (t) < nk;                                                                \
    const uint32_t ko_ = ok_ ? (uint32_t)(kb0 + (t)) * BK : OOB;                              \
    sst[(t) % RS] = __builtin_bit_cast(                                                       \
        float, __builtin_amdgcn_raw_buffer_load_b32(                                          \
                   rs, ok_ ? soff + (uint32_t)(kb0 + (t)) * M * 4 : OOB, 0, 0));              \
    sbt[(t) % RS] = __builtin_bit_cast(                                                       \
        float, __builtin_amdgcn_raw_buffer_load_b32(                                          \
                   rsb, ok_ ? (uint32_t)(kb0 + (t)) * 4 : OOB, 0, 0));                        \
    _Pragma("unroll") for (int i = 0; i < CH; ++i) st[(t) % RS][i] = __builtin_bit_cast(     \
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(i < CHA ? ra : rb, goff[i] + ko_, 0, 0)); \
  } while (0)
  // W(t): register set t % RS -> LDS slot t & 1
#define SK_W(t)                                                                               \
  do {                                                                                        \
    _Pragma("unroll") for (int i = 0; i < CH; ++i)                                            \
        *reinterpret_cast<u32x4 *>(&lds[(t) & 1][loff[i]]) = st[(t) % RS][i];                 \
    ssa[(t) & 1][tid] = sst[(t) % RS];                                                        \
    ssb[(t) & 1][tid] = sbt[(t) % RS]; /* the same value in every entry */                    \
  } while (0)

  v4f acc[NBW][MG];
#pragma unroll
  for (int j = 0; j < NBW; ++j)
#pragma unroll
    for (int i = 0; i < MG; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};

  // Block t: loaded G(t) RS - 1 iterations before it is written to LDS,
  // W(t) one iteration before it is used.
#pragma unroll
  for (int t = 0; t < RS; ++t) SK_G(t);
  SK_W(0);
  SK_G(RS);
  for (int t = 0; t < nk; t += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {  // t % U == 0, so every set / slot index below is static
      const int tt = t + u;
      __syncthreads();      // slot tt&1 written; nobody still reads slot (tt+1)&1
      SK_W(tt + 1);
      SK_G(tt + 1 + RS);
      const uint8_t *sl = lds[u & 1];
      v8i bfr[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int row = MROWS + (wave * NBW + j) * 16 + fr;
        bfr[j] = frag(sl + row * BK, row, fg);
      }
#pragma unroll
      for (int i = 0; i < MG; ++i) {
        const int row = i * 16 + fr;
        const v8i afr = frag(sl + row * BK, row, fg);
        const float s = ssa[u & 1][row] * ssb[u & 1][row];
        v4f pr[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          pr[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bfr[j], afr, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][i][r] = __builtin_fmaf(pr[j][r], s, acc[j][i][r]);
      }
    }
  }
#undef SK_G
#undef SK_W

  if (a.splits > 1) {
    const int tile = mtile * gridDim.x + ntile;
    constexpr int PER = THREADS * NBW * MG * 4;  // floats per partial tile
    float *part = a.ws + (size_t)tile * a.splits * PER;
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int i = 0; i < MG; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __hip_atomic_store(part + (size_t)split * PER + (((j * MG + i) * 4 + r) * THREADS + tid),
                             acc[j][i][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // the partial has landed before this workgroup counts in
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(a.splits - 1);
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int i = 0; i < MG; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float t = 0.f;
          for (int s = 0; s < a.splits; ++s)
            t += s == split ? acc[j][i][r]
                            : __hip_atomic_load(
                                  part + (size_t)s * PER + (((j * MG + i) * 4 + r) * THREADS + tid),
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          acc[j][i][r] = t;
        }
    if (tid == 0) __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

#pragma unroll
  for (int i = 0; i < MG; ++i) {
    const int m = m0 + i * 16 + fr;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int n = n0 + (wave * NBW + j) * 16 + 4 * fg;
      uint16_t *dp = a.D + (size_t)m * N + n;
      const uint32_t b0 = bf16_bits(acc[j][i][0]), b1 = bf16_bits(acc[j][i][1]);
      const uint32_t b2 = bf16_bits(acc[j][i][2]), b3 = bf16_bits(acc[j][i][3]);
      if ((N & 3) == 0 && n + 3 < N) {
        *reinterpret_cast<u32x2 *>(dp) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
      } else {
        if (n < N) dp[0] = (uint16_t)b0;
        if (n + 1 < N) dp[1] = (uint16_t)b1;
        if (n + 2 < N) dp[2] = (uint16_t)b2;
        if (n + 3 < N) dp[3] = (uint16_t)b3;
      }
    }
  }
}

int cdiv(int a, int b) { return (a + b - 1) / b; }

// ---- split-K workspace: one per (device, stream), made on first need ------
// Holds fp32 partial tiles and per-tile arrival counters (zeroed once here,
// re-armed by the kernels).  Never allocated while the stream is capturing:
// such calls run without a K split instead.
constexpr size_t WS_FLOATS = size_t(16) << 20;  // 64 MB of partials
constexpr int WS_COUNTERS = 1 << 16;

struct Workspace {
  float *part = nullptr;
  unsigned *counters = nullptr;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

const Workspace *workspace(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto it = g_ws.find({dev, s});
  if (it != g_ws.end()) return &it->second;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
  Workspace w;
  if (hipMalloc(reinterpret_cast<void **>(&w.part), WS_FLOATS * sizeof(float)) != hipSuccess)
    return nullptr;
  if (hipMalloc(reinterpret_cast<void **>(&w.counters), WS_COUNTERS * sizeof(unsigned)) != hipSuccess ||
      hipMemsetAsync(w.counters, 0, WS_COUNTERS * sizeof(unsigned), s) != hipSuccess) {
    (void)hipFree(w.part);
    return nullptr;
  }
  return &(g_ws[{dev, s}] = w);
}

// Optional override for tuning sweeps: FP8GEMM_SKINNY="nbw,splits" (nbw: 16-row
// weight groups per wave, 1 or 2).
bool skinny_override(int *nbw, int *splits) {
  const char *e = getenv("FP8GEMM_SKINNY");
  return e && sscanf(e, "%d,%d", nbw, splits) == 2 && (*nbw == 1 || *nbw == 2) && *splits >= 1;
}

template <int MG, int NBW>
int launch_skinny(SkArgs a, int m_tiles, int n_tiles, hipStream_t stream) {
  void *kargs[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&skinny_kernel<MG, NBW, SK_RS>),
                                 dim3(n_tiles, a.splits, m_tiles), dim3(THREADS), kargs, 0, stream);
  return e == hipSuccess ? FP8GEMM_OK : FP8GEMM_LAUNCH_FAILED;
}

// Dense GEMM with at most 128 activation rows per m-tile.
int run_skinny(const uint8_t *A, const float *sa, const uint8_t *B, const float *sb, uint16_t *D,
               int M, int N, int K, hipStream_t stream) {
  const int MG = M <= 64 ? 4 : 8;
  const int m_tiles = cdiv(M, 16 * MG);
  const int Kb = K / BK;
  int nbw = 1, splits = 1;
  if (!skinny_override(&nbw, &splits)) {
    // measured on MI355X (decode shapes, weights streamed from HBM): one
    // 16-row weight group per wave; a two-way K split pays for its partial
    // exchange only when there are few output tiles
    nbw = 1;
    const int tiles = cdiv(N, 64) * m_tiles;
    splits = tiles < 100 ? 2 : 1;
  }
  const int n_tiles = cdiv(N, 64 * nbw);
  splits = std::max(1, std::min(splits, std::max(Kb, 1)));
  const int kps = Kb > 0 ? cdiv(Kb, splits) : 0;
  splits = Kb > 0 ? cdiv(Kb, kps) : 1;
  SkArgs a{A, sa, B, sb, D, M, N, K, splits, kps, nullptr, nullptr};
  if (splits > 1) {
    const Workspace *w = workspace(stream);
    const size_t need = (size_t)n_tiles * m_tiles * splits * 16 * MG * 64 * nbw;
    if (!w || need > WS_FLOATS || n_tiles * m_tiles > WS_COUNTERS) {
      a.splits = 1;
      a.kb_per_split = Kb;
    } else {
      a.ws = w->part;
      a.counters = w->counters;
    }
  }
  if (MG == 4)
    return nbw == 2 ? launch_skinny<4, 2>(a, m_tiles, n_tiles, stream)
                    : launch_skinny<4, 1>(a, m_tiles, n_tiles, stream);
  return nbw == 2 ? launch_skinny<8, 2>(a, m_tiles, n_tiles, stream)
                  : launch_skinny<8, 1>(a, m_tiles, n_tiles, stream);
}

template <int WGN, int WGM, int TN, int TM, int STAGES, int LAYOUT>
int launch_tile(Args a, int groups, hipStream_t stream) {
  a.tiles_m = cdiv(a.M, WGM * TM * 16);
  a.tiles_n = cdiv(a.N, WGN * TN * 16);
  void *kargs[] = {&a};
  hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void *>(&tile_kernel<WGN, WGM, TN, TM, STAGES, LAYOUT>),
      dim3(a.tiles_m * a.tiles_n, groups), dim3(TK_THREADS), kargs, 0, stream);
  return e == hipSuccess ? FP8GEMM_OK : FP8GEMM_LAUNCH_FAILED;
}

template <int BM, int BN, int LAYOUT>
int launch(Args a, int groups, hipStream_t stream) {
  a.tiles_m = cdiv(a.M, BM);
  a.tiles_n = cdiv(a.N, BN);
  void *kargs[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&gemm_kernel<BM, BN, LAYOUT>),
                                 dim3(a.tiles_m * a.tiles_n, groups), dim3(THREADS), kargs, 0,
                                 stream);
  return e == hipSuccess ? FP8GEMM_OK : FP8GEMM_LAUNCH_FAILED;
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Checks shared by the three calls.  Runs before any HIP call.
int check_common(const void *A, const float *sa, const void *B, const float *sb, const void *D,
                 int M, int N, int K, long long a_elems, long long b_elems, long long d_elems) {
  if (M < 0 || N < 0 || K < 0) return FP8GEMM_INVALID_ARG;
  if (M == 0 || N == 0) return -1;  // empty: nothing to do, success
  if (!D) return FP8GEMM_INVALID_ARG;
  if (K > 0 && (!A || !sa || !B || !sb)) return FP8GEMM_INVALID_ARG;  // K == 0 reads nothing
  if (K % BK != 0) return FP8GEMM_UNSUPPORTED_SHAPE;
  const long long lim = 1LL << 31;
  if (a_elems >= lim || b_elems >= lim || d_elems >= lim) return FP8GEMM_UNSUPPORTED_SHAPE;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || !aligned(sa, 4) || !aligned(sb, 4))
    return FP8GEMM_MISALIGNED;
  return FP8GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_fp8_1x128_128x128_bf16(const void *A, const float *sa, const void *B, const float *sb,
                                void *D, int M, int N, int K, void *stream) {
  const int st = check_common(A, sa, B, sb, D, M, N, K, (long long)M * K, (long long)N * K,
                              (long long)M * N);
  if (st != FP8GEMM_OK) return st < 0 ? FP8GEMM_OK : st;
  Args a{static_cast<const uint8_t *>(A), sa, static_cast<const uint8_t *>(B), sb,
         static_cast<uint16_t *>(D), M, N, K, 1, nullptr, 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= 128)
    return run_skinny(a.A, sa, a.B, sb, a.D, M, N, K, s);
  if (K > 20480) return launch<128, 128, DENSE>(a, 1, s);
  return launch_tile<2, 2, 4, 8, 3, DENSE>(a, 1, s);
}

int grouped_contiguous(const void *A, const float *sa, const void *B, const float *sb, void *D,
                       int M, int N, int K, int G, void *stream, const int32_t *m_indices) {
  if (G < 1) return FP8GEMM_INVALID_ARG;
  const int st = check_common(A, sa, B, sb, D, M, N, K, (long long)M * K,
                              (long long)G * N * K, (long long)M * N);
  if (st != FP8GEMM_OK) return st < 0 ? FP8GEMM_OK : st;
  if (!m_indices) return FP8GEMM_INVALID_ARG;
  if (!aligned(m_indices, 4)) return FP8GEMM_MISALIGNED;
  if (M % 128 != 0) return FP8GEMM_UNSUPPORTED_SHAPE;
  Args a{static_cast<const uint8_t *>(A), sa, static_cast<const uint8_t *>(B), sb,
         static_cast<uint16_t *>(D), M, N, K, G, m_indices, 0, 0};
  if (K > 20480) return launch<128, 128, CONTIG>(a, 1, static_cast<hipStream_t>(stream));
  return launch_tile<4, 1, 4, 8, 3, CONTIG>(a, 1, static_cast<hipStream_t>(stream));
}

int grouped_masked(const void *A, const float *sa, const void *B, const float *sb, void *D,
                   int M, int N, int K, int G, void *stream, const int32_t *masked_m,
                   int expected_m) {
  if (G < 1 || expected_m < 0) return FP8GEMM_INVALID_ARG;
  const int st = check_common(A, sa, B, sb, D, M, N, K, (long long)G * M * K,
                              (long long)G * N * K, (long long)G * M * N);
  if (st != FP8GEMM_OK) return st < 0 ? FP8GEMM_OK : st;
  if (!masked_m) return FP8GEMM_INVALID_ARG;
  if (!aligned(masked_m, 4)) return FP8GEMM_MISALIGNED;
  if (G > 65535) return FP8GEMM_UNSUPPORTED_SHAPE;
  Args a{static_cast<const uint8_t *>(A), sa, static_cast<const uint8_t *>(B), sb,
         static_cast<uint16_t *>(D), M, N, K, G, masked_m, 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (expected_m <= 64 || K > 20480) return launch<64, 128, MASKED>(a, G, s);
  return launch_tile<2, 2, 4, 8, 3, MASKED>(a, G, s);
}

const char *fp8gemm_status_string(int status) {
  switch (status) {
    case FP8GEMM_OK: return "ok";
    case FP8GEMM_INVALID_ARG: return "invalid argument (null pointer, negative size, G < 1 or expected_m < 0)";
    case FP8GEMM_UNSUPPORTED_SHAPE: return "unsupported shape (K % 128 != 0, contiguous M % 128 != 0, or too large)";
    case FP8GEMM_MISALIGNED: return "misaligned pointer (A, B, D need 16 bytes; scales and indices 4)";
    case FP8GEMM_LAUNCH_FAILED: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
