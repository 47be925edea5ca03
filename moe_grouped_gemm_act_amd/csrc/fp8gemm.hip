// libfp8gemm: FP8 e4m3fn NT GEMM with 1x128 / 128x128 fp32 block scales and
// bf16 output, dense and MoE grouped (contiguous, masked), for gfx950.
//
// Method (DeepGEMM pages, GeekNews summary "Topic Body"): FP8 GEMM with the
// fine-grained scaling of DeepSeek-V3; the tensor-core partial sum of each
// scale block is added (promoted) into a higher-precision accumulator on the
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
//   * A and B tiles are staged into an LDS ring by dedicated loader waves
//     with direct-to-LDS loads (the Hopper design's asynchronous copies and
//     warp specialisation become wave roles on one workgroup barrier), with
//     an XOR swizzle of the 16-byte chunks so that fragment reads are
//     bank-conflict free;
//   * decode shapes (M <= 128) stream the weights from HBM: the same kernel
//     with 32- to 128-row weight tiles sized to fill the CUs and, where the
//     output alone gives too few tiles, a deterministic split of K summed by
//     a second kernel;
//   * large M: 256 x 128 tiles with eight compute waves (two per SIMD, so
//     one wave's promotion FMAs run beside the other's MFMAs); a partly
//     filled last wave of tiles is split over K; calls with many tiles and
//     short K run as a persistent walk, one workgroup per CU, whose loaders
//     prefetch across tiles;
//   * the K order inside a block is irrelevant to the sum, so each lane's
//     32-byte MFMA operand is two 16-byte chunks (c, c+4) of the 128-byte
//     row and A and B use the same chunk mapping.
//
// The grouped layouts reuse the same body (GeekNews "성능 평가"): contiguous
// tiles look up their expert from m_indices; masked tiles read the expert's
// device-side row count and tiles past it exit before loading anything (or,
// for long K, the walk visits the live tiles only, the experts listed by
// load).  The fused SwiGLU + 1x128
// requantisation epilogue and a BF16 variant without scales run on the same
// kernels.

#include <hip/hip_runtime.h>
#include <atomic>
#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <vector>

#include "e4m3.h"
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
  int splits, kb_per_split;  // K split over workgroups (tile kernel, dense only); 1 and K/128 otherwise
  float *ws;                 // split-K partial planes [splits][M][N] (splits > 1)
  uint8_t *act;              // fused SwiGLU: e4m3 codes of y [M][N/2] (masked [G][M][N/2]) ...
  float *act_scale;          // ... and their 1x128 scales [N/256][M] ([G][N/256][M])
  // tail split (dense, large M): tiles past full_tiles are split over K into
  // tail_splits items of tail_kb blocks each, whose fp32 partials go to ws
  // tile by tile and are summed by tail_reduce_kernel
  int full_tiles, tail_splits, tail_kb;
};

// XOR key of an LDS row: 16-byte chunk c of row r sits at position
// c ^ key(r).  A fragment read has lane l at row base + l % 16, chunk l / 16
// (and + 4); with key(r) = (r >> 1) & 7 these ds_read_b128 accesses are free
// of bank conflicts on gfx950 (measured with the SQ_LDS_BANK_CONFLICT
// counter: zero, against half of all LDS cycles for a key that separates
// only rows 8 apart).  It depends on r mod 16 only, so every 16-row fragment
// of a tile has the same per-lane pattern: the FP8 K block forms two
// per-lane offsets once and reads each fragment at a constant offset from
// them.
__device__ __forceinline__ int row_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int chunk_pos(int chunk, int row) { return (chunk ^ row_key(row)) << 4; }

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// chunk h (0: first 16 bytes, 1: second) of a fragment as 8 bf16 values
__device__ __forceinline__ bf16x8 bf_half(const v8i &v, int h) {
  const u32x4 x = h ? u32x4{(unsigned)v[4], (unsigned)v[5], (unsigned)v[6], (unsigned)v[7]}
                    : u32x4{(unsigned)v[0], (unsigned)v[1], (unsigned)v[2], (unsigned)v[3]};
  return __builtin_bit_cast(bf16x8, x);
}

// a fragment from its two 16-byte halves' addresses
__device__ __forceinline__ v8i frag_at(const uint8_t *plo, const uint8_t *phi) {
  const u32x4 lo = *reinterpret_cast<const u32x4 *>(plo);
  const u32x4 hi = *reinterpret_cast<const u32x4 *>(phi);
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

__device__ __forceinline__ v8i frag(const uint8_t *row_ptr, int row, int g) {
  u32x4 lo = *reinterpret_cast<const u32x4 *>(row_ptr + chunk_pos(g, row));
  u32x4 hi = *reinterpret_cast<const u32x4 *>(row_ptr + chunk_pos(g + 4, row));
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Fallback kernel for shapes the tile kernel does not take (K > 20480, past
// its weight-scale preload; masked calls with small expected counts, where
// 64-row tiles waste less): A and B staged global -> registers -> LDS in a
// two-slot ring.
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

// Buffer resource over [p, p + bytes): raw buffer loads past the end return
// zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}
constexpr uint32_t OOB = 0x80000000u;  // buffer offset past any resource: reads zeros

// Direct-to-LDS buffer loads (buffer_load ... lds): each lane's `bytes` at
// byte offset `off` of the resource land at lds + lane * bytes; an offset
// past the resource writes zeros and moves no data.  Kept in device
// functions: written in a kernel template, the builtin makes the host pass
// drop the kernel's stub.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                           off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4,
                                           off, 0, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (vmcnt: bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their no-wait maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }

// ---------------------------------------------------------------------------
// Tile kernel: every shape except the fallbacks below.
//
// Block tile BN = WGN * TN * 16 weight rows by BM = WGM * TM * 16 activation
// rows.  Four compute waves in a WGN x WGM grid each own a (TN * 16) x
// (TM * 16) tile (per K block they read TN + TM operand fragments from LDS
// for TN * TM MFMAs); NLD loader waves move each K block's activation rows,
// weight rows and activation scales with direct-to-LDS loads
// (global_load_lds: 16 bytes per lane, one 128-byte row per 8 lanes, the
// lane -> source mapping applying the XOR swizzle) into a ring of STAGES
// slots, STAGES - 1 blocks ahead, and wait for them with an explicit vmcnt;
// one bare barrier per K block hands a slot over.  Because vector-memory
// counters are per wave, the compute waves never wait on the loads in flight
// (they issue none), and the loaders never stall on LDS reads.  The weight
// scales of the tile's K range sit in LDS, loaded once.
//
// Large M (prefill, grouped): 128 x 256 or 256 x 128 tiles, MFMA bound.
// Small M (decode): the weights are the HBM stream and the output gives few
// tiles, so K may be split over `splits` workgroups per output tile.  Each
// split then writes its fp32 partial tile to its own plane of a workspace
// and ends; splitk_reduce_kernel, launched next on the same stream, adds the
// planes in split order and rounds to bf16, spread over the whole chip.  The
// result is deterministic, and nothing waits on another workgroup.
// The lane id computed anew where it is called (the compiler cannot merge it
// with an earlier copy), so a lane-derived value needed after the K loop
// need not be kept live through it, where the compute waves use every
// register.
__device__ __forceinline__ int fresh_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Pieces of a compute wave's work shared by the tile kernel and the
// persistent walk below.  A compute wave (wn, wm) of a WGN-wide grid owns
// weight rows (wn TN + i) 16 + 0..15 and activation rows (wm TM + j) 16 +
// 0..15 of the block tile; slot rows 0..BM-1 are activations, BM.. weights.

// Product k = j * TN + i of a K block (activation group j, weight group i)
// comes from one MFMA; it is promoted lag MFMAs later, when it has long
// landed, so the promotion FMAs issue in the shadow of the next MFMAs instead
// of waiting on the one just issued.  Products sit in a ring of `ring`
// registers; TN * TM is a multiple of it, so slots and the promotion of the
// previous block's last products line up across blocks.  Lag 2 in a ring of
// 4; tiles of two products per block (narrow decode tiles) use lag 1 in a
// ring of 2.
template <int TN, int TM>
constexpr int ring_size() { return (TN * TM) % 4 == 0 ? 4 : 2; }

// One FP8 K block from slot `sl` (activation scales after the operand rows),
// with the wave's weight scale sbv (TWOB: fragment i takes sbv_hi instead
// when bit i of himask is set, its rows lying in the next 128-row weight
// block): acc += (sa sb) (A_blk B_blk^T), the last
// LAG products carried to the next block (or fp8_flush).  The next activation
// fragment and its scale are read from LDS one group ahead.  Large tiles
// (WGN > 1) read only their first two weight fragments before the first MFMA
// and the rest one MFMA ahead of use, so the compute waves, released together
// by the barrier, do not all queue their whole fragment reads on the LDS at
// once.
template <int WGN, int TN, int TM, int BM, bool TWOB = false>
__device__ __forceinline__ void fp8_kblock(const uint8_t *sl, float sbv, float sbv_hi, unsigned himask,
                                           int wn, int wm, int fr, int fg, v4f (&acc)[TN][TM],
                                           v4f (&ring)[ring_size<TN, TM>()], float (&sc_last)[2]) {
  constexpr int RING = ring_size<TN, TM>(), LAG = RING / 2;
  constexpr int ROWS = BM + WGN * TN * 16;
  static_assert((TN * TM) % RING == 0 && LAG < RING && LAG <= TN, "product ring");
  // Every fragment row is 16 q + fr, so its swizzle depends on fr alone: two
  // per-lane offsets (one per 16-byte half) locate every fragment of the
  // wave, and a fragment's row group is a constant offset from them (four
  // address adds per block; the rest are immediate offsets).
  const int lo = fr * BK + chunk_pos(fg, fr), hi = fr * BK + chunk_pos(fg + 4, fr);
  const uint8_t *pa = sl + wm * TM * 16 * BK, *pb = sl + (BM + wn * TN * 16) * BK;
  const uint8_t *palo = pa + lo, *pahi = pa + hi, *pblo = pb + lo, *pbhi = pb + hi;
  const float *ssl = reinterpret_cast<const float *>(sl + ROWS * BK) + wm * TM * 16 + fr;
  v8i bfr[TN], afr[2];
  float scb[TM], sch[TM];  // activation scale times the weight scale sbv, and times sbv_hi
  constexpr int B0 = WGN > 1 && TN > 2 ? 2 : TN;
  constexpr int G = 16 * BK;  // bytes per 16-row group
#pragma unroll
  for (int i = 0; i < B0; ++i) bfr[i] = frag_at(pblo + i * G, pbhi + i * G);
  afr[0] = frag_at(palo, pahi);
  scb[0] = ssl[0] * sbv;
  sch[0] = TWOB ? ssl[0] * sbv_hi : scb[0];
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    if (j + 1 < TM) {
      afr[(j + 1) & 1] = frag_at(palo + (j + 1) * G, pahi + (j + 1) * G);
      scb[j + 1] = ssl[(j + 1) * 16] * sbv;
      sch[j + 1] = TWOB ? ssl[(j + 1) * 16] * sbv_hi : scb[j + 1];
    }
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      if (j == 0 && i + B0 < TN) {
        asm volatile("" ::: "memory");  // keeps the read after the MFMAs before it
        bfr[i + B0] = frag_at(pblo + (i + B0) * G, pbhi + (i + B0) * G);
      }
      const int k = j * TN + i;
      ring[k % RING] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          bfr[i], afr[j & 1], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
      const int kp = k - LAG;                      // product promoted now
      const int kq = kp >= 0 ? kp : kp + TN * TM;  // its index in its own block
      const bool hi = TWOB && ((himask >> (kq % TN)) & 1u);
      const float sp = kp >= 0 ? (hi ? sch[kq / TN] : scb[kq / TN]) : sc_last[hi ? 1 : 0];
      v4f &ap = acc[kq % TN][kq / TN];
      const v4f &pp = ring[(kq + RING) % RING];
#pragma unroll
      for (int r = 0; r < 4; ++r) ap[r] = __builtin_fmaf(pp[r], sp, ap[r]);
    }
  }
  sc_last[0] = scb[TM - 1];
  sc_last[1] = sch[TM - 1];
}

// the last block's last lag products
template <int TN, int TM, bool TWOB = false>
__device__ __forceinline__ void fp8_flush(v4f (&acc)[TN][TM], const v4f (&ring)[ring_size<TN, TM>()],
                                          const float (&sc_last)[2], unsigned himask) {
  constexpr int RING = ring_size<TN, TM>(), LAG = RING / 2;
#pragma unroll
  for (int k = TN * TM - LAG; k < TN * TM; ++k) {
    const float sp = sc_last[TWOB && ((himask >> (k % TN)) & 1u) ? 1 : 0];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc[k % TN][k / TN][r] = __builtin_fmaf(ring[k % RING][r], sp, acc[k % TN][k / TN][r]);
  }
}

// SwiGLU weight tiles (256 rows for 128 outputs of y = silu(g) u): row rw of
// the tile is gate row (rw < 32 within each 64-row group) or the matching up
// row, so a compute wave's fragments i < 2 hold gate values and i + 2 the up
// values of the same 32 outputs, in the same lanes.  Weight row in B of tile
// row rw, for output tile tn of I = N / 2 outputs.
__device__ __forceinline__ int swiglu_row(int rw, int tn, int I) {
  return ((rw & 32) ? I : 0) + tn * 128 + (rw >> 6) * 32 + (rw & 31);
}

// SwiGLU epilogue of one compute wave (wn, wm) of a 256 x BM tile: y for its
// 32 outputs in registers, the rows' maxima over the tile's 128 outputs
// through s_rmax (4 x BM floats; one workgroup barrier, which every wave of
// the workgroup, loaders included, must take at the same point), then the
// e4m3 codes of y / s with s = amax|y| / 448 for each row and its scale.
// Rows: m < mvalid (CONTIG: rows whose index names expert g).
template <int TM, int BM, int LAYOUT>
__device__ __forceinline__ void swiglu_epilogue(v4f (&acc)[4][TM], float *s_rmax, uint8_t *act,
                                                float *act_scale, const int32_t *idx, int g, int M,
                                                int I, int mvalid, int m0, int tn, int wn, int wm) {
  const int lid = fresh_lane_id();
  const int fr = lid & 15, fg = lid >> 4;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = acc[i][j][r];
        // silu(g) = g / (1 + e^-g): hardware exponential and reciprocal
        acc[i][j][r] = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * acc[i + 2][j][r];
        mx = fmaxf(mx, fabsf(acc[i][j][r]));  // NaN is skipped, as in the quantiser
      }
    // the row's other values of this wave sit in lanes fr + 16, + 32, + 48
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (fg == 0) s_rmax[wn * BM + (wm * TM + j) * 16 + fr] = mx;
  }
  __syncthreads();  // every wave's row maxima
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int ml = (wm * TM + j) * 16 + fr, m = m0 + ml;
    const float amax = fmaxf(fmaxf(s_rmax[ml], s_rmax[BM + ml]), fmaxf(s_rmax[2 * BM + ml], s_rmax[3 * BM + ml]));
    const float sc = amax == 0.f ? 1.f : amax / 448.f;
    const E4m3Quotient qd(amax, sc);
    bool ok = m < mvalid;
    if (LAYOUT == CONTIG) ok = m < M && idx[m] == g;
    if (!ok) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint32_t *>(act + (size_t)m * I + tn * 128 + wn * 32 + i * 16 + 4 * fg) =
          e4m3_pack4(qd.quotient(acc[i][j][0]), qd.quotient(acc[i][j][1]), qd.quotient(acc[i][j][2]),
                     qd.quotient(acc[i][j][3]), acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    if (wn == 0 && fg == 0) act_scale[(size_t)tn * M + m] = sc;
  }
}

// One BF16 K block (64 elements, 128 bytes a row).  No scales, so products
// accumulate straight in the MFMA's own accumulator.  A lane's two 16-byte
// chunks of a block row hold elements 8g..8g+7 and 32+8g..32+8g+7 (g = lane
// / 16): exactly the operands of two 16x16x32 bf16 MFMAs, over the block's
// first and second 32 elements.  All sub-tiles take the first half before
// the second, so no MFMA waits on the one just issued.
template <int TN, int TM, int BM>
__device__ __forceinline__ void bf16_kblock(const uint8_t *sl, int wn, int wm, int fr, int fg,
                                            v4f (&acc)[TN][TM]) {
  v8i bfr[TN], afr[TM];
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int row = BM + (wn * TN + i) * 16 + fr;
    bfr[i] = frag(sl + row * BK, row, fg);
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int row = (wm * TM + j) * 16 + fr;
    afr[j] = frag(sl + row * BK, row, fg);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int i = 0; i < TN; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf_half(bfr[i], h), bf_half(afr[j], h),
                                                            acc[i][j], 0, 0, 0);
}

// The wave's part of a BM x BN fp32 tile, row-major, at pt (tail-split parts).
template <int TN, int TM, int BN>
__device__ __forceinline__ void store_part(const v4f (&acc)[TN][TM], float *pt, int wn, int wm,
                                           int fr, int fg) {
#pragma unroll
  for (int j = 0; j < TM; ++j)
#pragma unroll
    for (int i = 0; i < TN; ++i)
      *reinterpret_cast<v4f *>(pt + ((wm * TM + j) * 16 + fr) * BN + (wn * TN + i) * 16 + 4 * fg) =
          acc[i][j];
}

// The wave's part of the output tile at (m0, n0) as bf16: rows below mvalid
// (CONTIG: rows whose index names expert g).
template <int TN, int TM, int LAYOUT>
__device__ __forceinline__ void store_bf16(const v4f (&acc)[TN][TM], uint16_t *D, const int32_t *idx,
                                           int g, int M, int N, int mvalid, int m0, int n0, int wn,
                                           int wm, int fr, int fg) {
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = m0 + (wm * TM + j) * 16 + fr;
    bool ok = m < mvalid;
    if (LAYOUT == CONTIG) ok = m < M && idx[m] == g;
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

template <int WGN, int WGM, int TN, int TM, int STAGES, int NLD, bool KSPLIT, bool ACT, int LAYOUT,
          bool BF = false>
__global__ __launch_bounds__((WGN * WGM + NLD) * 64) void tile_kernel(Args a) {
  constexpr int BN = WGN * TN * 16, BM = WGM * TM * 16;
  constexpr int ROWS = BM + BN;
  // BF: bf16 operands with no scales; a "K block" is then 128 bytes = 64 elements
  constexpr int SLOT = ROWS * BK + (BF ? 0 : BM * 4);  // operand rows, then the BM activation scales
  constexpr int OCT = ROWS / 8;             // 1 KB row groups per slot
  constexpr int DMA = OCT / NLD;            // row-group loads per loader wave per slot
  constexpr int SG = BM / 64;               // 64-float activation-scale loads per slot
  constexpr int SPL = BF ? 0 : (SG + NLD - 1) / NLD; // of which per loader (spares repeat one: same bytes, same place)
  constexpr int PER_G = DMA + SPL;          // vector memory instructions per loader per slot
  constexpr int MAXKB = 160;                // K <= 20480 for the weight-scale preload
  constexpr int NCW = WGN * WGM;            // compute waves
  constexpr int CT = NCW * 64;              // compute threads
  // a wave's weight rows lie in one 128-row scale block, or (TWOB: one wave
  // column of 96 rows) in at most two
  static_assert((NCW == 4 || NCW == 8) && OCT % NLD == 0 && BM % 64 == 0 && BN % 32 == 0 &&
                    (128 % (TN * 16) == 0 || (WGN == 1 && BN == 96)),
                "tile shape");
  constexpr bool TWOB = ACT || BN % 128 == 96;  // a wave reads two weight-scale blocks
  static_assert(PER_G * (STAGES - 1) < 64, "loads in flight per loader must fit vmcnt");
  // ACT (fused SwiGLU): the tile's 256 weight rows are 128 gate rows and the
  // 128 matching up rows, interleaved 32 by 32 (swiglu_row); its output is
  // 128 columns of y
  static_assert(!ACT || (BN == 256 && WGN == 4 && TN == 4 && BM <= 128), "SwiGLU tile shape");
  static_assert(!(ACT && BF), "the fused SwiGLU takes FP8 operands");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES][SLOT];
  __shared__ float s_sb[BN > 128 || TWOB ? 2 : 1][BF ? 1 : MAXKB];
  __shared__ float s_rmax[ACT ? 4 * BM : 1];  // ACT: row maxima of y per wave column
  __shared__ int s_group;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fg = lane >> 4;
  const int M = a.M, N = a.N, K = a.K, Nb = (N + 127) / 128;
  const int RB = BF ? 2 * K : K, Kb = RB / BK;  // operand row bytes, K blocks

  // work order: workgroup ids are dealt to the 8 XCDs round robin; give each
  // XCD a contiguous run of (split, tile) items, walked GROUPN weight tiles
  // at a time with the activation tiles inside, so concurrent tiles on one
  // XCD share panels
  constexpr int GROUPN = 4;
  const int T = a.tiles_m * a.tiles_n, S = KSPLIT ? a.splits : 1;
  // Tail split: when the last wave of tiles would leave most CUs idle, the
  // tiles past full_tiles are split over K.  Their items take the highest
  // workgroup ids, which are dispatched last, once CUs free up, round robin
  // over the XCDs; the full tiles keep the XCD-aware order below.
  const bool tail = !KSPLIT && LAYOUT == DENSE && a.tail_splits > 1 && (int)blockIdx.x >= a.full_tiles;
  int item = blockIdx.x, split, tile;
  if (tail) {
    const int r = item - a.full_tiles;
    tile = a.full_tiles + r / a.tail_splits;
    split = r % a.tail_splits;
  } else {
    const int TS = (!KSPLIT && a.tail_splits > 1) ? a.full_tiles : T * S;
    const int x = item % 8, l = item / 8, per = TS / 8, rem = TS % 8;
    item = x * per + min(x, rem) + l;
    split = item / T;
    tile = item % T;
  }
  int tn, tm;
  {
    const int gsz = GROUPN * a.tiles_m, grp = tile / gsz, in = tile % gsz;
    const int gw = min(GROUPN, a.tiles_n - grp * GROUPN);
    tn = grp * GROUPN + in % gw;
    tm = in / gw;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbps = tail ? a.tail_kb : a.kb_per_split;
  const int kb0 = split * kbps, nk = max(0, min(Kb - kb0, kbps));

  const uint8_t *A = a.A, *B = a.B;
  const float *sa = a.sa, *sb = a.sb;
  uint16_t *D = a.D;
  uint8_t *act = a.act;
  float *act_scale = a.act_scale;
  int mvalid = M, g = 0;
  if (LAYOUT == MASKED) {
    g = blockIdx.y;
    const int c = a.idx[g];
    mvalid = c < 0 ? 0 : (c > M ? M : c);
    if (m0 >= mvalid) return;  // whole tile masked: nothing loaded, nothing written
    A += (size_t)g * M * RB;
    if (!BF) sa += (size_t)g * Kb * M;
    D += (size_t)g * M * N;
    act += (size_t)g * M * (N / 2);
    act_scale += (size_t)g * (N / 256) * M;
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
    B += (size_t)g * N * RB;
    if (!BF) sb += (size_t)g * Nb * Kb;
  }
  if (wave >= NCW) {
    // ---------------- loader waves ----------------
    const int L = wave - NCW;
    const int lane = ACT ? fresh_lane_id() : tid & 63;
    constexpr int QA = BM / 8 / NLD;  // loads q < QA are activation row groups, the rest weights
    static_assert((BM / 8) % NLD == 0, "row groups split evenly between A and B");
    const __amdgpu_buffer_rsrc_t ra = rsrc(A, (uint32_t)M * RB);
    const __amdgpu_buffer_rsrc_t rb = rsrc(B, (uint32_t)N * RB);
    const __amdgpu_buffer_rsrc_t rs = rsrc(sa, (uint32_t)M * Kb * 4);
    // q-th row-group load: rows (L + NLD q) * 8 .. + 7 of the slot; lane l ->
    // row + l / 8, physical chunk l % 8 holding logical chunk (l % 8) ^ key(row).
    // Rows past the valid ones (activation rows >= mvalid, weight rows >= N)
    // read out of range: zeros, no memory traffic; they are never stored.
    uint32_t off[DMA];  // byte offsets into A (q < QA) or B
#pragma unroll
    for (int q = 0; q < DMA; ++q) {
      const int r = (L + NLD * q) * 8 + (lane >> 3);
      const int col = (lane & 7) ^ row_key(r);
      if (q < QA) {
        off[q] = m0 + r < mvalid ? (uint32_t)(m0 + r) * RB + col * 16 : OOB;
      } else {
        const int rw = r - BM;  // weight row of the tile
        const int grow = ACT ? swiglu_row(rw, tn, N / 2) : n0 + rw;
        off[q] = grow < N ? (uint32_t)grow * RB + col * 16 : OOB;
      }
    }
    uint32_t soff[SPL > 0 ? SPL : 1];  // byte offsets of scale floats 64 j + lane of the tile's rows
    int sdst[SPL > 0 ? SPL : 1];
#pragma unroll
    for (int jj = 0; jj < SPL; ++jj) {
      const int j = (L + NLD * jj) % SG;
      soff[jj] = m0 + j * 64 + lane < mvalid ? (uint32_t)(m0 + j * 64 + lane) * 4 : OOB;
      sdst[jj] = ROWS * BK + j * 256;
    }
    // G(t): K block kb0 + t (clamped: blocks past the range re-read the last
    // one and are never consumed) -> slot t % STAGES
#define TK_G(t)                                                                               \
  do {                                                                                        \
    const int kb_ = kb0 + min((t), nk - 1);                                                   \
    uint8_t *sl_ = lds[(t) % STAGES];                                                         \
    _Pragma("unroll") for (int q = 0; q < DMA; ++q)                                          \
        dma16(q < QA ? ra : rb, off[q] + (uint32_t)kb_ * BK, sl_ + (L + NLD * q) * 1024);     \
    _Pragma("unroll") for (int jj = 0; jj < SPL; ++jj)                                        \
        dma4(rs, soff[jj] + (uint32_t)kb_ * M * 4, sl_ + sdst[jj]);                           \
  } while (0)
    if (nk > 0) {
#pragma unroll
      for (int t = 0; t < STAGES - 1; ++t) TK_G(t);
    }
    for (int t0 = 0; t0 < nk; t0 += STAGES) {
#pragma unroll
      for (int u = 0; u < STAGES; ++u) {
        const int t = t0 + u;
        if (t >= nk) break;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_G * (STAGES - 2)));  // my loads of block t landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // ... and everyone's; all compute waves are past block t - 1
        asm volatile("" ::: "memory");
        TK_G(t + STAGES - 1);
      }
    }
#undef TK_G
    __builtin_amdgcn_s_waitcnt(0);  // nothing may still write LDS when the workgroup ends
    if (ACT) __syncthreads();  // the SwiGLU epilogue's barrier
    return;
  }

  // ---------------- compute waves ----------------
  const int wn = wave % WGN, wm = wave / WGN;
  // which weight-scale block this wave's rows use (ACT: gate block 0, up block 1)
  const int hsb = ACT ? 0 : (wn * TN * 16) / 128;
  // TWOB: the fragments whose rows use the second block (ACT: the up
  // fragments 2 and 3; 96-row tiles: rows past the tile's first 128-row
  // boundary)
  unsigned himask = ACT ? 0xCu : 0u;
  if (!ACT && TWOB) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
      if ((n0 & 127) + i * 16 >= 128) himask |= 1u << i;
  }
  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // masked layout: a wave whose activation rows all lie past masked_m has
  // nothing to compute and only takes the barriers (a compile-time no-op for
  // the other layouts, whose loop measured 3% slower with the branch)
  const bool idle = LAYOUT == MASKED && m0 + wm * TM * 16 >= mvalid;
  if constexpr (BF) {
    for (int t0 = 0; t0 < nk; t0 += STAGES) {
#pragma unroll
      for (int u = 0; u < STAGES; ++u) {
        const int t = t0 + u;
        if (t >= nk) break;
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // block t is in slot u
        asm volatile("" ::: "memory");
        if (!idle) bf16_kblock<TN, TM, BM>(lds[u], wn, wm, fr, fg, acc);
      }
    }
  } else {
    // the weight scales of the K range go to LDS while the loaders start; the
    // first K-block barrier publishes them
    for (int i = tid; i < (BN > 128 || TWOB ? 2 : 1) * nk; i += CT) {
      const int h = i / nk, t = i % nk;
      const int blk = ACT ? (h == 0 ? tn : N / 256 + tn) : min(n0 / 128 + h, Nb - 1);
      s_sb[h][t] = sb[(size_t)blk * Kb + kb0 + t];
    }
    __builtin_amdgcn_s_waitcnt(0);
    v4f ring[ring_size<TN, TM>()];
#pragma unroll
    for (int q = 0; q < ring_size<TN, TM>(); ++q) ring[q] = v4f{0.f, 0.f, 0.f, 0.f};
    float sc_last[2] = {0.f, 0.f};  // scales of the previous block's last activation group
    for (int t0 = 0; t0 < nk; t0 += STAGES) {
#pragma unroll
      for (int u = 0; u < STAGES; ++u) {
        const int t = t0 + u;
        if (t >= nk) break;
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // block t is in slot u
        asm volatile("" ::: "memory");
        // ACT: the slot's offset goes through an empty asm, so the compiler
        // adds it at each read instead of keeping every slot's fragment
        // addresses in registers through the loop
        int so = u * SLOT;
        if (ACT) asm volatile("" : "+s"(so));
        if (!idle)
          fp8_kblock<WGN, TN, TM, BM, TWOB>(&lds[0][0] + so, s_sb[hsb][t], s_sb[TWOB ? 1 : hsb][t],
                                            himask, wn, wm, fr, fg, acc, ring, sc_last);
      }
    }
    fp8_flush<TN, TM, TWOB>(acc, ring, sc_last, himask);
  }

  if constexpr (ACT) {
    // fused SwiGLU and 1x128 requantisation of y = silu(g) u
    swiglu_epilogue<TM, BM, LAYOUT>(acc, s_rmax, act, act_scale, a.idx, g, M, N / 2, mvalid, m0, tn,
                                    wn, wm);
    return;
  }

  if (tail) {
    // this K part of a tail tile: its fp32 partial tile goes to workspace
    // slot (tail tile, split), BM x BN floats, row-major within the tile
    store_part<TN, TM, BN>(acc, a.ws + ((size_t)(tile - a.full_tiles) * a.tail_splits + split) * (BM * BN),
                           wn, wm, fr, fg);
    return;
  }
  if (S > 1) {
    // this split's fp32 partial goes to its own [M][N] plane of the
    // workspace; splitk_reduce_kernel (next on the stream) sums the planes
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + (wm * TM + j) * 16 + fr;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int n = n0 + (wn * TN + i) * 16 + 4 * fg;
        float *pp = a.ws + ((size_t)split * M + m) * N + n;
        if ((N & 3) == 0 && n + 3 < N) {
          *reinterpret_cast<v4f *>(pp) = acc[i][j];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) pp[r] = acc[i][j][r];
        }
      }
    }
    return;
  }
  store_bf16<TN, TM, LAYOUT>(acc, D, a.idx, g, M, N, mvalid, m0, n0, wn, wm, fr, fg);
}
// ---------------------------------------------------------------------------
// Persistent tile walk for the large tiles (dense and contiguous calls with
// more tiles than CUs): one workgroup per CU takes items b, b + P, b + 2P, ...
// of the same item list the tile kernel runs as separate workgroups (whole
// tiles in XCD order, then, for dense calls, the K parts of a split last
// wave; P is a multiple of 8, so every item of a workgroup stays on its
// XCD).  The loader waves run one producer cursor over the workgroup's K
// blocks of all its items, STAGES - 1 blocks ahead of the compute waves: the
// next tile's first blocks load while the compute waves finish a tile and
// store it.  The weight scales of each block travel in its slot with the
// activation scales (every loader loads the same two floats, so all loaders
// keep one count of loads per slot), so nothing is preloaded per tile.
// Contiguous layout: each item's expert is found for all of the workgroup's
// items at once, before any load.  Masked layout: the list holds only the
// live tiles, expert by expert (ceil(masked_m[g] / BM) activation tiles by
// the weight tiles), up to 64 experts ordered by load so that each XCD's run
// pairs a loaded expert with a light one; every workgroup builds the order
// and the experts' offsets into the list from masked_m on the device, and
// finds an item's expert by binary search.
// ACT (fused SwiGLU, 256 x 128 tiles of interleaved gate/up rows): after a
// tile's last block every wave, loaders included, takes one more barrier
// for the epilogue's row maxima (swiglu_epilogue); the LDS ring is not used
// by the epilogue, so the prefetch of the next tile goes on.
constexpr int WALK_MAXIT = 256;  // items per workgroup, at most (contiguous)
constexpr int WALK_MAXG = 512;   // experts, at most (masked)

template <int WGN, int WGM, int TN, int TM, int STAGES, int NLD, int LAYOUT, bool BF, bool ACT = false>
__global__ __launch_bounds__((WGN * WGM + NLD) * 64) void walk_kernel(Args a) {
  constexpr int BN = WGN * TN * 16, BM = WGM * TM * 16;
  constexpr int ROWS = BM + BN;
  constexpr int SBOFF = ROWS * BK + BM * 4;          // FP8: the block's weight scales
  constexpr int SLOT = BF ? ROWS * BK : SBOFF + 256;  // operand rows, activation scales, weight scales
  constexpr int OCT = ROWS / 8;
  constexpr int DMA = OCT / NLD;
  constexpr int SG = BM / 64;
  constexpr int SPL = BF ? 0 : (SG + NLD - 1) / NLD;
  constexpr int PER_G = DMA + SPL + (BF ? 0 : 1);  // vector memory instructions per loader per slot
  constexpr int NCW = WGN * WGM, NT = (NCW + NLD) * 64;
  static_assert((NCW == 4 || NCW == 8) && OCT % NLD == 0 && BM % 64 == 0 && BN % 64 == 0 &&
                    BN <= 256 && 128 % (TN * 16) == 0 && (BM / 8) % NLD == 0,
                "tile shape");
  static_assert(PER_G * (STAGES - 1) < 64, "loads in flight per loader must fit vmcnt");
  static_assert(LAYOUT != CONTIG || BM <= 128, "one expert per activation tile");
  static_assert(!ACT || (BN == 256 && WGN == 4 && TN == 4 && BM <= 128 && !BF), "SwiGLU tile shape");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES][SLOT];
  __shared__ int s_grp[LAYOUT == CONTIG ? WALK_MAXIT : 1];
  __shared__ float s_rmax[ACT ? 4 * BM : 1];  // ACT: row maxima of y per wave column
  // masked: the experts in list order (s_perm[r]: the expert at position
  // r), the items before position r (s_pre[r]) and expert g's valid rows
  // (s_mv[g])
  __shared__ int s_pre[LAYOUT == MASKED ? WALK_MAXG + 1 : 1];
  __shared__ int s_mv[LAYOUT == MASKED ? WALK_MAXG : 1];
  __shared__ int s_perm[LAYOUT == MASKED ? WALK_MAXG : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = a.M, N = a.N, K = a.K, Nb = (N + 127) / 128;
  const int RB = BF ? 2 * K : K, Kb = RB / BK;
  if (LAYOUT == MASKED) {
    // the live tiles: expert g has ceil(min(max(masked_m[g], 0), M) / BM)
    // activation tiles by tiles_n weight tiles.  Up to 64 experts are listed
    // heaviest, lightest, second heaviest, second lightest, ... (by valid
    // rows; ties by index), so each XCD's run of the list (below) pairs a
    // heavily loaded expert with a lightly loaded one instead of taking
    // neighbours in index order; more experts keep index order.  A
    // wave-wide prefix sum over the list, 64 at a time, gives each
    // position's first item.
    if (wave == 0) {
      const int lane = tid & 63;
      const bool pair = a.G <= 64;
      for (int base = 0; base < a.G; base += 64) {
        const int g = base + lane;
        int mv = -1;
        if (g < a.G) {
          const int v = a.idx[g];
          mv = v < 0 ? 0 : (v > M ? M : v);
          s_mv[g] = mv;
        }
        int pos = g;
        if (pair) {
          int rank = 0;
          for (int h = 0; h < a.G; ++h) {
            const int mh = __shfl(mv, h, 64);
            rank += (mh > mv || (mh == mv && h < g)) ? 1 : 0;
          }
          pos = rank < (a.G + 1) / 2 ? 2 * rank : 2 * (a.G - 1 - rank) + 1;
        }
        if (g < a.G) s_perm[pos] = g;
      }
      __builtin_amdgcn_s_waitcnt(0);  // s_perm and s_mv written before this wave reads them
      __builtin_amdgcn_wave_barrier();
      int carry = 0;
      for (int base = 0; base < a.G; base += 64) {
        const int r = base + lane;
        int c = 0;
        if (r < a.G) c = (s_mv[s_perm[r]] + BM - 1) / BM * a.tiles_n;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_up(c, d, 64);
          if (lane >= d) c += y;
        }
        if (r < a.G) s_pre[r + 1] = carry + c;
        carry += __shfl(c, 63, 64);
      }
      if (lane == 0) s_pre[0] = 0;
    }
    __syncthreads();
  }
  const int T = a.tiles_m * a.tiles_n;
  const bool tsplit = LAYOUT == DENSE && a.tail_splits > 1;
  // whole tiles (masked: the live ones, counted on the device); then the tail parts
  const int F = LAYOUT == MASKED ? s_pre[a.G] : tsplit ? a.full_tiles : T;
  const int NI = F + (tsplit ? (T - F) * a.tail_splits : 0);
  const int P = gridDim.x, b = blockIdx.x;
  const int nit = b < NI ? (NI - b + P - 1) / P : 0;

  struct Item {
    int tile, split, m0, n0, kb0, nk, g, mvalid;
    bool tail;
  };
  // item k of this workgroup, at position b + k P of the list
  auto item = [&](int k) {
    constexpr int GROUPN = 4;
    const int pos = b + k * P;
    Item it;
    it.tail = pos >= F;
    if (it.tail) {
      const int r = pos - F;
      it.tile = F + r / a.tail_splits;
      it.split = r % a.tail_splits;
    } else {
      const int x = pos % 8, l = pos / 8, per = F / 8, rem = F % 8;
      it.tile = x * per + min(x, rem) + l;
      it.split = 0;
    }
    int tiles_m = a.tiles_m, tile = it.tile;
    it.g = 0;
    it.mvalid = M;
    if (LAYOUT == MASKED) {
      // the list position holding live tile `tile`: the last r with
      // s_pre[r] <= tile; its expert
      int lo = 0, hi = a.G - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= tile) lo = mid;
        else hi = mid - 1;
      }
      it.g = s_perm[lo];
      it.mvalid = s_mv[it.g];
      tiles_m = (s_pre[lo + 1] - s_pre[lo]) / a.tiles_n;
      tile -= s_pre[lo];
    }
    const int gsz = GROUPN * tiles_m, grp = tile / gsz, in = tile % gsz;
    const int gw = min(GROUPN, a.tiles_n - grp * GROUPN);
    it.n0 = (grp * GROUPN + in % gw) * BN;
    it.m0 = (in / gw) * BM;
    const int kbps = it.tail ? a.tail_kb : Kb;
    it.kb0 = it.split * kbps;
    it.nk = max(0, min(Kb - it.kb0, kbps));
    return it;
  };

  if (LAYOUT == CONTIG) {
    // each item's expert: the largest valid index among its rows (one expert
    // per 128-row block by contract; every row is checked again at store
    // time), -1 when they are all padding
    for (int k = tid; k < nit; k += NT) s_grp[k] = -1;
    __syncthreads();
    for (int e = tid; e < nit * BM; e += NT) {
      const int m = item(e / BM).m0 + e % BM;
      if (m < M) {
        const int v = a.idx[m];
        if (v >= 0 && v < a.G) atomicMax(&s_grp[e / BM], v);
      }
    }
    __syncthreads();
  }
  // expert of item k (0 for dense), -1: nothing to do
  auto group = [&](int k) { return LAYOUT == CONTIG ? s_grp[k] : 0; };

  if (wave >= NCW) {
    // ---------------- loader waves ----------------
    const int L = wave - NCW, lane = tid & 63;
    constexpr int QA = BM / 8 / NLD;  // loads q < QA are activation row groups, the rest weights
    __amdgpu_buffer_rsrc_t ra = rsrc(a.A, (uint32_t)M * RB), rb = ra, rs = ra, rsb = ra;
    if (!BF) rs = rsrc(a.sa, (uint32_t)M * Kb * 4);
    uint32_t off[DMA], soff[SPL > 0 ? SPL : 1], sboff = OOB;
    int sdst[SPL > 0 ? SPL : 1];
#pragma unroll
    for (int jj = 0; jj < SPL; ++jj) sdst[jj] = ROWS * BK + ((L + NLD * jj) % SG) * 256;
    int pk = -1, pt = 0, pnk = 0, pkb0 = 0;  // producer: item, block in it, its count and first block
    // move the producer to the next item with work; past the last one, every
    // load goes out of range (zeros, no traffic), so each slot still counts
    // PER_G loads per loader
    auto advance = [&]() {
      for (++pk; pk < nit; ++pk) {
        if (group(pk) < 0) continue;
        const Item it = item(pk);
        const int g = LAYOUT == MASKED ? it.g : group(pk);
        if (LAYOUT == MASKED) {
          ra = rsrc(a.A + (size_t)g * M * RB, (uint32_t)M * RB);
          if (!BF) rs = rsrc(a.sa + (size_t)g * Kb * M, (uint32_t)M * Kb * 4);
        }
        if (LAYOUT != DENSE) {
          rb = rsrc(a.B + (size_t)g * N * RB, (uint32_t)N * RB);
          if (!BF) rsb = rsrc(a.sb + (size_t)g * Nb * Kb, (uint32_t)Nb * Kb * 4);
        } else {
          rb = rsrc(a.B, (uint32_t)N * RB);
          if (!BF) rsb = rsrc(a.sb, (uint32_t)Nb * Kb * 4);
        }
        // q-th row-group load: rows (L + NLD q) * 8 .. + 7 of the slot; lane l
        // -> row + l / 8, physical chunk l % 8 holding logical chunk
        // (l % 8) ^ key(row); rows past M or N read out of range
#pragma unroll
        for (int q = 0; q < DMA; ++q) {
          const int r = (L + NLD * q) * 8 + (lane >> 3);
          const int col = (lane & 7) ^ row_key(r);
          const int grow = q < QA ? it.m0 + r : ACT ? swiglu_row(r - BM, it.n0 / BN, N / 2) : it.n0 + r - BM;
          off[q] = grow < (q < QA ? it.mvalid : N) ? (uint32_t)grow * RB + col * 16 : OOB;
        }
        if (!BF) {
#pragma unroll
          for (int jj = 0; jj < SPL; ++jj) {
            const int m = it.m0 + ((L + NLD * jj) % SG) * 64 + lane;
            soff[jj] = m < it.mvalid ? (uint32_t)m * 4 : OOB;
          }
          // lane h < BN / 128: the scale row of the tile's h-th 128-row weight
          // block (ACT: the gate block, then the up block)
          const int blk = ACT ? (lane == 0 ? it.n0 / BN : N / 256 + it.n0 / BN) : min(it.n0 / 128 + lane, Nb - 1);
          sboff = lane < BN / 128 ? (uint32_t)blk * Kb * 4 : OOB;
        }
        pkb0 = it.kb0;
        pnk = it.nk;
        pt = 0;
        return;
      }
      pnk = 0;
      pt = 0;
    };
    auto produce = [&](int s) {
      if (pt == pnk && pk < nit) advance();
      const bool real = pt < pnk;
      const uint32_t kb = real ? (uint32_t)(pkb0 + pt) : 0u;
      uint8_t *sl = &lds[0][0] + s * SLOT;
#pragma unroll
      for (int q = 0; q < DMA; ++q) dma16(q < QA ? ra : rb, real ? off[q] + kb * BK : OOB, sl + (L + NLD * q) * 1024);
#pragma unroll
      for (int jj = 0; jj < SPL; ++jj) dma4(rs, real ? soff[jj] + kb * M * 4 : OOB, sl + sdst[jj]);
      if (!BF) dma4(rsb, real ? sboff + kb * 4 : OOB, sl + SBOFF);
      pt += real ? 1 : 0;
    };
    int ps = 0;  // slot the producer fills next
#pragma unroll
    for (int q = 0; q < STAGES - 1; ++q) {
      produce(ps);
      ps = ps + 1 == STAGES ? 0 : ps + 1;
    }
    for (int k = 0; k < nit; ++k) {
      if (group(k) < 0) continue;
      const int nk = item(k).nk;
      for (int t = 0; t < nk; ++t) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_G * (STAGES - 2)));  // my loads of this block landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // ... and everyone's; all compute waves are past the previous block
        asm volatile("" ::: "memory");
        produce(ps);
        ps = ps + 1 == STAGES ? 0 : ps + 1;
      }
      // ACT: the SwiGLU epilogue's barrier; the next item's first blocks are
      // already in flight
      if (ACT) __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0);  // nothing may still write LDS when the workgroup ends
    return;
  }

  // ---------------- compute waves ----------------
  const int lane = tid & 63, fr = lane & 15, fg = lane >> 4;
  const int wn = wave % WGN, wm = wave / WGN;
  // which of the slot's weight scales this wave's rows use (ACT: gate 0, up 1)
  const int hsb = ACT ? 0 : (wn * TN * 16) / 128;
  int cs = 0;                            // slot of the next block
  for (int k = 0; k < nit; ++k) {
    if (group(k) < 0) continue;  // all padding: nothing loaded, nothing written
    const Item it = item(k);
    const int g = LAYOUT == MASKED ? it.g : group(k);
    v4f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    // masked layout: all of this wave's activation rows past masked_m:
    // barriers only
    const bool idle = LAYOUT == MASKED && it.m0 + wm * TM * 16 >= it.mvalid;
    if constexpr (BF) {
      for (int t = 0; t < it.nk; ++t) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // this item's block t is in slot cs
        asm volatile("" ::: "memory");
        if (!idle) bf16_kblock<TN, TM, BM>(&lds[0][0] + cs * SLOT, wn, wm, fr, fg, acc);
        cs = cs + 1 == STAGES ? 0 : cs + 1;
      }
    } else {
      v4f ring[ring_size<TN, TM>()];
#pragma unroll
      for (int q = 0; q < ring_size<TN, TM>(); ++q) ring[q] = v4f{0.f, 0.f, 0.f, 0.f};
      float sc_last[2] = {0.f, 0.f};
      for (int t = 0; t < it.nk; ++t) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // this item's block t is in slot cs
        asm volatile("" ::: "memory");
        const uint8_t *sl = &lds[0][0] + cs * SLOT;
        const float *sbs = reinterpret_cast<const float *>(sl + SBOFF);
        if (!idle)
          fp8_kblock<WGN, TN, TM, BM, ACT>(sl, sbs[hsb], sbs[ACT ? 1 : hsb], ACT ? 0xCu : 0u, wn, wm,
                                           fr, fg, acc, ring, sc_last);
        cs = cs + 1 == STAGES ? 0 : cs + 1;
      }
      fp8_flush<TN, TM, ACT>(acc, ring, sc_last, ACT ? 0xCu : 0u);
    }
    if constexpr (ACT) {
      const int I = N / 2;
      swiglu_epilogue<TM, BM, LAYOUT>(
          acc, s_rmax, a.act + (LAYOUT == MASKED ? (size_t)g * M * I : 0),
          a.act_scale + (LAYOUT == MASKED ? (size_t)g * (N / 256) * M : 0), a.idx, g, M, I,
          it.mvalid, it.m0, it.n0 / BN, wn, wm);
    } else if (it.tail) {
      store_part<TN, TM, BN>(acc, a.ws + ((size_t)(it.tile - F) * a.tail_splits + it.split) * (BM * BN),
                             wn, wm, fr, fg);
    } else {
      store_bf16<TN, TM, LAYOUT>(acc, a.D + (LAYOUT == MASKED ? (size_t)g * M * N : 0), a.idx, g, M,
                                 N, it.mvalid, it.m0, it.n0, wn, wm, fr, fg);
    }
  }
}

// Split-K reduction (decode): D[m][n] = bf16(sum over s, in split order, of
// ws[s][m][n]).  One thread per 4 consecutive columns of a row; the planes
// are fetched NB at a time with buffer loads (NB = S up to 8, so no load is
// wasted; planes past S in a last batch read out of range: zeros, no
// traffic), so the loads of one thread are issued together.  (Eight loads a
// batch for every S cost 0.2-0.3 us more per call at S = 4 and 6:
// out-of-range loads still take the CU's memory request slots.)
template <int NB>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *ws, uint16_t *D, int M,
                                                            int N, int S) {
  const int nq = (N + 3) / 4;
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  if (q >= (long long)M * nq) return;
  const int m = (int)(q / nq), n = (int)(q % nq) * 4;
  const uint32_t plane = (uint32_t)M * N * 4;
  const __amdgpu_buffer_rsrc_t r = rsrc(ws, plane * (uint32_t)S);
  const bool vec = (N & 3) == 0;
  const uint32_t off = ((uint32_t)m * N + n) * 4;
  v4f sum = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += NB) {
    v4f p[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const uint32_t o = s0 + k < S ? off + (uint32_t)(s0 + k) * plane : OOB;
      if (vec) {
        p[k] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p[k][e] = n + e < N ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                              r, o == OOB ? OOB : o + 4 * e, 0, 0))
                              : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (s0 + k >= S) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] = s0 + k == 0 ? p[k][e] : sum[e] + p[k][e];
    }
  }
  uint16_t *dp = D + (size_t)m * N + n;
  const uint32_t b0 = bf16_bits(sum[0]), b1 = bf16_bits(sum[1]);
  const uint32_t b2 = bf16_bits(sum[2]), b3 = bf16_bits(sum[3]);
  if (vec) {
    *reinterpret_cast<u32x2 *>(dp) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
  } else {
    if (n < N) dp[0] = (uint16_t)b0;
    if (n + 1 < N) dp[1] = (uint16_t)b1;
    if (n + 2 < N) dp[2] = (uint16_t)b2;
    if (n + 3 < N) dp[3] = (uint16_t)b3;
  }
}

// Tail-split reduction: tail tile t (of R) has S partial tiles of BM x BN
// floats in ws; D gets their sum in split order, rounded to bf16.  One
// thread per 4 consecutive columns of a tile row; the tile's position comes
// from the same GROUPN walk as the tile kernel's.
template <int BM, int BN>
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float *ws, uint16_t *D, int M, int N,
                                                          int full_tiles, int S, int tiles_m,
                                                          int tiles_n) {
  constexpr int GROUPN = 4, QT = BM * BN / 4;
  const int q = blockIdx.x * 256 + threadIdx.x;
  const int t = q / QT, e = q % QT;  // tail tile, quad inside it (grid: whole tiles)
  const int tile = full_tiles + t;
  const int gsz = GROUPN * tiles_m, grp = tile / gsz, in = tile % gsz;
  const int gw = min(GROUPN, tiles_n - grp * GROUPN);
  const int ml = e / (BN / 4), nl = (e % (BN / 4)) * 4;
  const int m = (in / gw) * BM + ml, n = (grp * GROUPN + in % gw) * BN + nl;
  if (m >= M || n >= N) return;
  const float *p = ws + (size_t)t * S * (BM * BN) + ml * BN + nl;
  v4f sum = *reinterpret_cast<const v4f *>(p);
  for (int s = 1; s < S; ++s) sum += *reinterpret_cast<const v4f *>(p + (size_t)s * (BM * BN));
  uint16_t *dp = D + (size_t)m * N + n;
  const uint32_t b0 = bf16_bits(sum[0]), b1 = bf16_bits(sum[1]), b2 = bf16_bits(sum[2]),
                 b3 = bf16_bits(sum[3]);
  if ((N & 3) == 0 && n + 3 < N) {
    *reinterpret_cast<u32x2 *>(dp) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
  } else {
    dp[0] = (uint16_t)b0;
    if (n + 1 < N) dp[1] = (uint16_t)b1;
    if (n + 2 < N) dp[2] = (uint16_t)b2;
    if (n + 3 < N) dp[3] = (uint16_t)b3;
  }
}

int cdiv(int a, int b) { return (a + b - 1) / b; }

// ---- split-K workspace -------------------------------------------------
// The fp32 partials of a split call (decode planes, or the tail parts of a
// large-M call) live in a library-owned workspace of WS_BYTES, which every
// default plan fits (decode: splits x M x N <= 256 x 128 x 128 floats = 16 MB;
// tail: at most 256 parts of 256 x 128 floats = 32 MB).
//   * Eager calls (stream not capturing) share ONE workspace per device,
//     allocated on first need.  Its users are ordered on the GPU: a call on a
//     stream other than the last user's first makes its stream wait for the
//     event the last user recorded after its kernels, then records the event
//     itself.  So split calls on different streams run one after the other
//     (never on the same partials at once), and memory does not grow with the
//     number of streams.
//   * Calls made while their stream is being captured into a graph take a
//     workspace of their own for that capture (one per capture and capturing
//     stream, shared by the capture's split calls on that stream, which the
//     stream orders).  It comes from the device's list of workspaces released
//     by graphs that have been destroyed, else from hipMalloc with this
//     thread's capture mode exchanged to relaxed for the allocation (an
//     allocation is not a stream operation; global mode forbids it only as
//     potentially unsafe).  The graph holds it through a user object whose
//     release (when the graph and every executable made from it are
//     destroyed) puts it back on the list; the release callback makes no HIP
//     call.  A replay therefore never shares partials with eager calls or with
//     another graph.
//   * When no workspace can be had, the call runs without a K split (the
//     same results within the tolerance, slower).
// (Graph memory nodes from a captured hipMallocAsync would be the plain
// route; on this runtime a second launch of such a graph faulted, so they
// are not used.)
constexpr size_t WS_BYTES = size_t(32) << 20;
constexpr size_t WS_FLOATS = WS_BYTES / sizeof(float);
constexpr int MAX_DEV = 64;

struct DeviceWs {
  std::mutex mu;  // eager workspace and event; held across an eager split call's launches
  float *eager = nullptr;
  hipEvent_t done = nullptr;     // recorded after the last eager user's kernels
  hipStream_t last = nullptr;    // the stream that recorded it
  bool recorded = false;
  // capture workspaces; guarded by cap_mu, never held across a HIP call, so
  // the user-object release callback may take it
  std::mutex cap_mu;
  std::map<std::pair<unsigned long long, hipStream_t>, float *> live;  // (capture id, stream)
  std::vector<float *> spare;    // released by destroyed graphs, reusable
};
DeviceWs g_dev_ws[MAX_DEV];

struct CaptureWsRecord {  // owned by the user object
  int dev;
  unsigned long long id;
  hipStream_t stream;
  float *ptr;
};

void release_capture_ws(void *p) {  // user-object destructor: no HIP calls
  CaptureWsRecord *r = static_cast<CaptureWsRecord *>(p);
  DeviceWs &d = g_dev_ws[r->dev];
  {
    std::lock_guard<std::mutex> lk(d.cap_mu);
    d.live.erase({r->id, r->stream});
    d.spare.push_back(r->ptr);
  }
  delete r;
}

// A workspace held for one call.  acquire() returns false when the call must
// run unsplit; release() (after the call's launches) completes the eager
// ordering.
struct WsLease {
  float *ptr = nullptr;
  DeviceWs *eager_dev = nullptr;  // set for eager leases: d.mu is held until release
  hipStream_t stream = nullptr;

  bool acquire(hipStream_t s) {
    stream = s;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) {
      (void)hipGetLastError();
      return false;
    }
    DeviceWs &d = g_dev_ws[dev];
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    unsigned long long id = 0;
    hipGraph_t graph = nullptr;
    const hipGraphNode_t *deps = nullptr;
    size_t ndeps = 0;
    if (hipStreamGetCaptureInfo_v2(s, &cs, &id, &graph, &deps, &ndeps) != hipSuccess) {
      (void)hipGetLastError();  // handled: no split
      return false;
    }
    if (cs == hipStreamCaptureStatusActive) return acquire_capture(d, dev, id, graph);
    if (cs != hipStreamCaptureStatusNone) return false;  // an invalidated capture
    d.mu.lock();
    if (!d.eager) {
      if (hipMalloc(reinterpret_cast<void **>(&d.eager), WS_BYTES) != hipSuccess) {
        (void)hipGetLastError();  // handled: no split
        d.eager = nullptr;
        d.mu.unlock();
        return false;
      }
    }
    if (!d.done && hipEventCreateWithFlags(&d.done, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      d.done = nullptr;
      d.mu.unlock();
      return false;
    }
    if (d.recorded && d.last != s && hipStreamWaitEvent(s, d.done, 0) != hipSuccess) {
      (void)hipGetLastError();
      d.mu.unlock();
      return false;
    }
    ptr = d.eager;
    eager_dev = &d;
    return true;
  }

  bool acquire_capture(DeviceWs &d, int dev, unsigned long long id, hipGraph_t graph) {
    {
      std::lock_guard<std::mutex> lk(d.cap_mu);
      auto it = d.live.find({id, stream});
      if (it != d.live.end()) {
        ptr = it->second;
        return true;
      }
      if (!d.spare.empty()) {
        ptr = d.spare.back();
        d.spare.pop_back();
      }
    }
    if (!ptr) {
      hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
      if (hipThreadExchangeStreamCaptureMode(&mode) != hipSuccess) {
        (void)hipGetLastError();
        return false;
      }
      const hipError_t e = hipMalloc(reinterpret_cast<void **>(&ptr), WS_BYTES);
      hipStreamCaptureMode back = mode;
      (void)hipThreadExchangeStreamCaptureMode(&back);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        ptr = nullptr;
        return false;
      }
    }
    CaptureWsRecord *r = new CaptureWsRecord{dev, id, stream, ptr};
    hipUserObject_t uo = nullptr;
    if (hipUserObjectCreate(&uo, r, release_capture_ws, 1, hipUserObjectNoDestructorSync) != hipSuccess) {
      (void)hipGetLastError();
      std::lock_guard<std::mutex> lk(d.cap_mu);
      d.spare.push_back(ptr);
      delete r;
      ptr = nullptr;
      return false;
    }
    {
      std::lock_guard<std::mutex> lk(d.cap_mu);
      d.live[{id, stream}] = ptr;
    }
    if (hipGraphRetainUserObject(graph, uo, 1, hipGraphUserObjectMove) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipUserObjectRelease(uo, 1);  // runs release_capture_ws: back on the list
      ptr = nullptr;
      return false;
    }
    return true;
  }

  // after the call's launches (whatever their status)
  void release() {
    if (!eager_dev) return;
    DeviceWs &d = *eager_dev;
    if (hipEventRecord(d.done, stream) == hipSuccess) {
      d.recorded = true;
      d.last = stream;
    } else {
      // the next user on another stream cannot be ordered after this call:
      // wait for it here (eager only, and only on a runtime error)
      (void)hipGetLastError();
      (void)hipStreamSynchronize(stream);
      (void)hipGetLastError();
      d.recorded = false;
    }
    eager_dev = nullptr;
    d.mu.unlock();
  }
  ~WsLease() { release(); }
};

// ---- fixed scratch of the allocation-free entry point --------------------
// A file-scope device array: each GPU the library runs on holds its own copy
// from module load until the process ends.  Host code must not pass the
// array's name to a kernel (on the host it names a stand-in, not device
// memory): the address comes from hipGetSymbolAddress, once per device with
// that device current, and is kept per device.  Every call of that entry
// point on a GPU shares the array; it keeps the last call's partials, which
// every call overwrites before reading (nothing in it must start at zero).
constexpr size_t SCRATCH_FLOATS = WS_FLOATS;  // 32 MB: every default plan fits
static __device__ __align__(256) float scratch[SCRATCH_FLOATS];

std::mutex g_scratch_mu;
float *g_scratch_ptr[MAX_DEV];

// the current device's address of `scratch`, or nullptr on a runtime error
float *scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    // a symbol lookup, no stream operation: allowed while a stream captures
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    const bool exchanged = hipThreadExchangeStreamCaptureMode(&mode) == hipSuccess;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (exchanged) (void)hipThreadExchangeStreamCaptureMode(&mode);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = static_cast<float *>(p);
  }
  return g_scratch_ptr[dev];
}

template <int WGN, int WGM, int TN, int TM, int STAGES, int NLD, int LAYOUT, bool KSPLIT = false,
          bool ACT = false, bool BF = false>
int launch_tile(Args a, int groups, hipStream_t stream) {
  a.tiles_m = cdiv(a.M, WGM * TM * 16);
  a.tiles_n = cdiv(a.N, WGN * TN * 16);
  if (!KSPLIT) {
    a.splits = 1;
    a.kb_per_split = (BF ? 2 * a.K : a.K) / BK;
  }
  void *kargs[] = {&a};
  hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void *>(
          &tile_kernel<WGN, WGM, TN, TM, STAGES, NLD, KSPLIT, ACT, LAYOUT, BF>),
      dim3(a.tiles_m * a.tiles_n * a.splits, groups), dim3((WGN * WGM + NLD) * 64), kargs, 0,
      stream);
  return e == hipSuccess ? FP8GEMM_OK : FP8GEMM_LAUNCH_FAILED;
}

// Dense GEMM with M <= 128 (decode): the tile kernel with a deep ring, four
// loader waves, 64 weight rows per tile and a K split sized so that the
// (split, tile) items cover the chip.
// Optional override for tuning sweeps: FP8GEMM_DECODE="bn,stages,splits[,waves]".
struct DecodeCfg {
  int bn, stages, splits, waves;
};

// Instances built: four compute waves with (bn, stages) in {(64,4), (64,6),
// (128,4), (96,4), (32,4)} for both activation tile heights; eight compute
// waves with four slots for bn = 128, and for bn = 64 with 128 activation
// rows.
bool decode_built(int bn, int stages, int bm, int waves) {
  if (waves == 8) return stages == 4 && (bn == 128 || (bn == 64 && bm == 128));
  return waves == 4 &&
         ((bn == 64 && (stages == 4 || stages == 6)) || ((bn == 128 || bn == 96 || bn == 32) && stages == 4));
}

// Default (measured on MI355X over the decode shapes, weights streamed from
// HBM): four slots; 64 weight rows per tile unless the output alone gives
// 384 or more such tiles, then 128 (fewer activation re-reads per weight
// byte); a K split only when the tiles alone leave CUs idle, with (tiles x
// splits) kept within one wave of 256 workgroups and at least 9 K blocks per
// split, since the partial planes and their reduction cost about 3 us.
DecodeCfg decode_config(int M, int N, int Kb, bool bf) {
  const int bm = M <= 64 ? 64 : 128;
  const char *e = getenv("FP8GEMM_DECODE");
  DecodeCfg o{0, 0, 0, 4};
  if (e && sscanf(e, "%d,%d,%d,%d", &o.bn, &o.stages, &o.splits, &o.waves) >= 3 && o.splits >= 1 &&
      decode_built(o.bn, o.stages, bm, o.waves))
    return o;
  const int tiles64 = cdiv(N, 64);
  DecodeCfg c{tiles64 >= 384 ? 128 : 64, 4, 1, 4};
  const int tiles = cdiv(N, c.bn) * cdiv(M, bm);
  c.splits = std::max(1, std::min(256 / std::max(tiles, 1), Kb / 9));
  // K too short to split but half the CUs idle: 32-row weight tiles double
  // the workgroups without partials (64 and 128 x 7168 x 2048: 8.5 -> 7.3 and
  // 11.0 -> 9.4 us; each workgroup streams half the weights and the same
  // activations)
  if (c.splits == 1 && c.bn == 64 && 2 * tiles <= 256) {
    c.bn = 32;
    return c;
  }
  // no K split and 96-row tiles fill more of the chip in one wave (N = 24576:
  // 256 tiles instead of 192 of 128 rows)
  const int tiles96 = cdiv(N, 96) * cdiv(M, bm);
  if (c.splits == 1 && tiles96 <= 256 && tiles96 > tiles) {
    c.bn = 96;
    return c;
  }
  // eight compute waves (two per SIMD, so one's promotion FMAs overlap the
  // other's MFMAs) where the tile has the rows for them and K is not split
  // (measured 2-4% with 128-row tiles at 24576x1536 and 64-row tiles at
  // 128x7168x2048, which now take the narrower tiles above; slower with a K
  // split); FP8 only: BF16 has no promotion
  if (!bf && c.splits == 1 && decode_built(c.bn, 4, bm, 8)) c.waves = 8;
  return c;
}

// BF: bf16 operands, K blocks of 64 elements (128 bytes)
// fixed_ws: a caller-provided scratch of SCRATCH_FLOATS (the allocation-free
// entry point); nullptr: the library workspace (WsLease)
template <bool BF>
int run_decode(Args a, hipStream_t stream, float *fixed_ws = nullptr) {
  const int Kb = (BF ? 2 * a.K : a.K) / BK;
  DecodeCfg c = decode_config(a.M, a.N, Kb, BF);
  const int bm = a.M <= 64 ? 64 : 128;
  int splits = std::max(1, std::min(c.splits, std::max(Kb, 1)));
  const int kps = Kb > 0 ? cdiv(Kb, splits) : 0;
  splits = Kb > 0 ? cdiv(Kb, kps) : 1;
  a.splits = splits;
  a.kb_per_split = kps;
  WsLease ws;  // held until the reduction is enqueued
  if (splits > 1) {
    const size_t need = (size_t)splits * a.M * a.N;
    if (fixed_ws) {
      if (need > SCRATCH_FLOATS) return FP8GEMM_SCRATCH_EXCEEDED;
      a.ws = fixed_ws;
    } else if (need > WS_FLOATS || !ws.acquire(stream)) {
      a.splits = 1;
      a.kb_per_split = Kb;
    } else {
      a.ws = ws.ptr;
    }
  }
  int st = FP8GEMM_LAUNCH_FAILED;  // unreachable: decode_config returns built instances only
  if (c.waves == 8) {
    if (c.bn == 128)
      st = bm == 64 ? launch_tile<2, 4, 4, 1, 4, 4, DENSE, true, false, BF>(a, 1, stream)
                    : launch_tile<2, 4, 4, 2, 4, 4, DENSE, true, false, BF>(a, 1, stream);
    else
      st = launch_tile<2, 4, 2, 2, 4, 4, DENSE, true, false, BF>(a, 1, stream);
  }
#define DEC(BN_, ST_)                                                                     \
  if (c.waves == 4 && c.bn == BN_ && c.stages == ST_)                                     \
    st = bm == 64 ? launch_tile<1, 4, BN_ / 16, 1, ST_, 4, DENSE, true, false, BF>(a, 1, stream) \
                  : launch_tile<1, 4, BN_ / 16, 2, ST_, 4, DENSE, true, false, BF>(a, 1, stream);
  DEC(64, 4)
  DEC(64, 6)
  DEC(128, 4)
  DEC(96, 4)
  DEC(32, 4)
#undef DEC
  if (st != FP8GEMM_OK || a.splits == 1) return st;
  const long long quads = (long long)a.M * cdiv(a.N, 4);
  const dim3 grid((unsigned)((quads + 255) / 256));
  // the launch's own status (hipGetLastError would also report an earlier
  // call's error)
  void *rargs[] = {&a.ws, &a.D, &a.M, &a.N, &a.splits};
  const void *red = nullptr;
  switch (std::min(a.splits, 8)) {
#define RED(NB_)                                                                   \
  case NB_: red = reinterpret_cast<const void *>(&splitk_reduce_kernel<NB_>); break;
    RED(2) RED(3) RED(4) RED(5) RED(6) RED(7) RED(8)
#undef RED
    default: return FP8GEMM_LAUNCH_FAILED;  // unreachable: splits > 1 here
  }
  return hipLaunchKernel(red, grid, dim3(256), rargs, 0, stream) == hipSuccess ? FP8GEMM_OK
                                                                             : FP8GEMM_LAUNCH_FAILED;
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

// Workgroups of the persistent walk: the device's CUs, rounded down to a
// multiple of the 8 XCDs (one workgroup per CU: the walk's ring takes most
// of a CU's LDS).  Cached per device.
int walk_workgroups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev].load(std::memory_order_relaxed) > 0)
    return cache[dev].load(std::memory_order_relaxed);
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  n = n / 8 * 8;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}
// The walk for calls with more tiles than CUs and operand rows of at most
// 8 KB (FP8 K <= 8192, BF16 K <= 4096).  Measured against one workgroup per
// tile: 9% faster at FP8 K = 1536, 2-4% on the contiguous K = 7168 calls,
// 2-3% slower at K = 16384 and 18432, where a tile's fixed costs are a small
// share of its time and the walk's runtime slot indexing costs a little in
// every block.  Plain masked calls keep one workgroup per (tile, expert)
// unless FP8GEMM_WALK=2: their walk over the live tiles measured the same per
// call and up to 3% slower over the two masked workload calls (the masked
// SwiGLU call walks by default).  FP8GEMM_WALK=0 turns the walk off
// everywhere (tuning overrides).
bool walk_enabled(int row_bytes, bool masked = false) {
  const char *e = getenv("FP8GEMM_WALK");
  if (e && e[0] == '0') return false;
  if (masked && !(e && e[0] == '2')) return false;
  return row_bytes <= 8192;
}

// a.tiles_m / tiles_n and the tail fields set; P workgroups
template <int WGN, int WGM, int TN, int TM, int STAGES, int NLD, int LAYOUT, bool BF, bool ACT = false>
hipError_t launch_walk(Args &a, int P, hipStream_t stream) {
  void *kargs[] = {&a};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(&walk_kernel<WGN, WGM, TN, TM, STAGES, NLD, LAYOUT, BF, ACT>),
      dim3(P), dim3((WGN * WGM + NLD) * 64), kargs, 0, stream);
}

// Dense M > 128 with one large tile per CU.  When the tiles leave a last
// wave of R <= 128 tiles for the 256 CUs, those R tiles are split over K into
// S = min(8, 256 / R) parts (each at least 4 K blocks) that run as the last
// items of the same grid, and tail_reduce_kernel adds the parts.  Without a
// workspace the tail is not split.
template <int WGN, int WGM, int TN, int TM, int STAGES, int NLD, bool BF = false>
int launch_dense_large(Args a, hipStream_t stream, float *fixed_ws = nullptr) {
  constexpr int BN = WGN * TN * 16, BM = WGM * TM * 16;
  const int tiles_m = cdiv(a.M, BM), tiles_n = cdiv(a.N, BN), T = tiles_m * tiles_n;
  const int Kb = (BF ? 2 * a.K : a.K) / BK, R = T % 256;
  int S = R > 0 && R <= 128 ? std::min(8, 256 / R) : 1;
  while (S > 1 && cdiv(Kb, S) < 4) --S;
  WsLease ws;  // held until the tail reduction is enqueued
  if (S > 1) {
    const size_t need = (size_t)R * S * BM * BN;
    if (fixed_ws) {
      if (need > SCRATCH_FLOATS) return FP8GEMM_SCRATCH_EXCEEDED;
    } else if (need > WS_FLOATS || !ws.acquire(stream)) {
      S = 1;
    }
  }
  // more tiles than CUs: the persistent walk over the same items
  const int P = walk_workgroups();
  const bool walk = walk_enabled(BF ? 2 * a.K : a.K) && P >= 8 && T > P;
  a.tiles_m = tiles_m;
  a.tiles_n = tiles_n;
  a.splits = 1;
  a.kb_per_split = Kb;
  if (S <= 1) {
    if (!walk) return launch_tile<WGN, WGM, TN, TM, STAGES, NLD, DENSE, false, false, BF>(a, 1, stream);
    return launch_walk<WGN, WGM, TN, TM, STAGES, NLD, DENSE, BF>(a, P, stream) == hipSuccess
               ? FP8GEMM_OK
               : FP8GEMM_LAUNCH_FAILED;
  }
  const int kb = cdiv(Kb, S);
  a.full_tiles = T - R;
  a.tail_splits = cdiv(Kb, kb);
  a.tail_kb = kb;
  a.ws = fixed_ws ? fixed_ws : ws.ptr;
  hipError_t er;
  if (walk) {
    er = launch_walk<WGN, WGM, TN, TM, STAGES, NLD, DENSE, BF>(a, P, stream);
  } else {
    void *kargs[] = {&a};
    er = hipLaunchKernel(
        reinterpret_cast<const void *>(
            &tile_kernel<WGN, WGM, TN, TM, STAGES, NLD, false, false, DENSE, BF>),
        dim3(a.full_tiles + R * a.tail_splits), dim3((WGN * WGM + NLD) * 64), kargs, 0, stream);
  }
  if (er != hipSuccess) return FP8GEMM_LAUNCH_FAILED;
  int tm = tiles_m, tn = tiles_n;
  void *rargs[] = {&a.ws, &a.D, &a.M, &a.N, &a.full_tiles, &a.tail_splits, &tm, &tn};
  er = hipLaunchKernel(reinterpret_cast<const void *>(&tail_reduce_kernel<BM, BN>),
                       dim3(R * (BM * BN / 4) / 256), dim3(256), rargs, 0, stream);
  return er == hipSuccess ? FP8GEMM_OK : FP8GEMM_LAUNCH_FAILED;
}

// Contiguous layout, 256 x 128 tiles: the persistent walk when there are
// more tiles than CUs (and few enough per workgroup for its expert table)
template <bool BF>
int launch_contig_large(Args a, hipStream_t stream) {
  const int P = walk_workgroups();
  a.tiles_m = cdiv(a.M, 128);
  a.tiles_n = cdiv(a.N, 256);
  const int T = a.tiles_m * a.tiles_n;
  if (!walk_enabled(BF ? 2 * a.K : a.K) || P < 8 || T <= P || cdiv(T, P) > WALK_MAXIT)
    return launch_tile<4, 2, 4, 4, 3, 4, CONTIG, false, false, BF>(a, 1, stream);
  a.splits = 1;
  a.kb_per_split = (BF ? 2 * a.K : a.K) / BK;
  return launch_walk<4, 2, 4, 4, 3, 4, CONTIG, BF>(a, P, stream) == hipSuccess ? FP8GEMM_OK
                                                                              : FP8GEMM_LAUNCH_FAILED;
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

// The dense call; fixed: the split-K partials go to `scratch` (the
// allocation-free entry point) instead of the library workspace.
int dense_fp8(const void *A, const float *sa, const void *B, const float *sb, void *D, int M, int N,
              int K, void *stream, bool fixed) {
  const int st = check_common(A, sa, B, sb, D, M, N, K, (long long)M * K, (long long)N * K,
                              (long long)M * N);
  if (st != FP8GEMM_OK) return st < 0 ? FP8GEMM_OK : st;
  float *fws = nullptr;
  if (fixed && !(fws = scratch_ptr())) return FP8GEMM_LAUNCH_FAILED;
  Args a{static_cast<const uint8_t *>(A), sa, static_cast<const uint8_t *>(B), sb,
         static_cast<uint16_t *>(D), M, N, K, 1, nullptr, 0, 0, 1, K / BK, nullptr};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= 128 && K <= 20480) return run_decode<false>(a, s, fws);
  if (K > 20480) return launch<128, 128, DENSE>(a, 1, s);
  // 256 weight rows x 128 activation rows, eight compute waves (two per
  // SIMD, so one wave's promotion FMAs run under the other's MFMAs) and four
  // loader waves (measured 1.5-2% faster on the prefill shapes than 128 x
  // 256 tiles); FP8GEMM_LARGE=6 selects the four-compute-wave layout
  const char *e = getenv("FP8GEMM_LARGE");
  if (e && e[0] == '6') return launch_tile<2, 2, 4, 8, 3, 2, DENSE>(a, 1, s);
  return launch_dense_large<4, 2, 4, 4, 3, 4>(a, s, fws);
}

}  // namespace

extern "C" {

int gemm_fp8_1x128_128x128_bf16(const void *A, const float *sa, const void *B, const float *sb,
                                void *D, int M, int N, int K, void *stream) {
  return dense_fp8(A, sa, B, sb, D, M, N, K, stream, false);
}

int gemm_fp8_1x128_128x128_bf16_noalloc(const void *A, const float *sa, const void *B,
                                        const float *sb, void *D, int M, int N, int K,
                                        void *stream) {
  return dense_fp8(A, sa, B, sb, D, M, N, K, stream, true);
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
         static_cast<uint16_t *>(D), M, N, K, G, m_indices, 0, 0, 1, K / BK, nullptr};
  if (K > 20480) return launch<128, 128, CONTIG>(a, 1, static_cast<hipStream_t>(stream));
  // 256 weight rows x 128 activation rows (one expert per 128-row block),
  // eight compute waves and four loader waves
  const char *e = getenv("FP8GEMM_LARGE");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (e && e[0] == '6') return launch_tile<4, 1, 4, 8, 3, 2, CONTIG>(a, 1, s);
  return launch_contig_large<false>(a, s);
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
         static_cast<uint16_t *>(D), M, N, K, G, masked_m, 0, 0, 1, K / BK, nullptr};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K > 20480) return launch<64, 128, MASKED>(a, G, s);
  // measured on MI355X (G = 16, 256-row capacity, counts ~ U[0, 256]):
  // eight compute waves (two per SIMD overlap promotion FMAs with MFMAs),
  // four loader waves; 64-row activation tiles when the hint says counts are
  // small; for short K 256 weight rows, which halve the activation re-reads
  // and the tiles' fixed costs
  if (expected_m <= 64) return launch_tile<1, 4, 8, 1, 4, 4, MASKED>(a, G, s);
  const int P = walk_workgroups();
  const char *we = getenv("FP8GEMM_WALK"), *mt = getenv("FP8GEMM_MASKED");
  // the persistent walk over the live tiles (up to WALK_MAXG experts, rows
  // of at most 8 KB); FP8GEMM_WALK=0 turns it off, =2 also walks K <= 4096
  const bool walk = !(we && we[0] == '0') && P >= 8 && G <= WALK_MAXG && K <= 8192;
  const bool walk_all = walk && we && we[0] == '2';
  if (K > 4096 && !(mt && mt[0] == '0')) {
    // 256 activation rows (a whole expert of a 256-row capacity) by 128
    // weight rows, walked over the live tiles: each expert's weight tile is
    // streamed once, not once per 128-row activation tile, and compute waves
    // whose 64 rows lie past masked_m skip their MFMAs (G = 16 x 256 x 4096
    // x 7168: 123 us, against 126 us for 128-row activation tiles; the walk
    // and one workgroup per tile measure the same)
    if (!walk) return launch_tile<2, 4, 4, 4, 3, 4, MASKED>(a, G, s);
    a.tiles_m = cdiv(M, 256);
    a.tiles_n = cdiv(N, 128);
    return launch_walk<2, 4, 4, 4, 3, 4, MASKED, false>(a, P, s) == hipSuccess ? FP8GEMM_OK
                                                                               : FP8GEMM_LAUNCH_FAILED;
  }
  if (K <= 4096) {
    // 256 weight rows by 128 activation rows, one workgroup per (tile,
    // expert), dead tiles exiting at once (the walk measured 2-4% slower at
    // 16 x 256 x 7168 x 2048)
    if (!walk_all) return launch_tile<4, 2, 4, 4, 3, 4, MASKED>(a, G, s);
    a.tiles_m = cdiv(M, 128);
    a.tiles_n = cdiv(N, 256);
    return launch_walk<4, 2, 4, 4, 3, 4, MASKED, false>(a, P, s) == hipSuccess ? FP8GEMM_OK
                                                                               : FP8GEMM_LAUNCH_FAILED;
  }
  // K > 4096 with FP8GEMM_MASKED=0 (tuning override): 128 x 128 tiles
  if (!walk_all) return launch_tile<2, 4, 4, 2, 4, 4, MASKED>(a, G, s);
  a.tiles_m = cdiv(M, 128);
  a.tiles_n = cdiv(N, 128);
  return launch_walk<2, 4, 4, 2, 4, 4, MASKED, false>(a, P, s) == hipSuccess ? FP8GEMM_OK
                                                                             : FP8GEMM_LAUNCH_FAILED;
}

// Grouped GEMM with B_g = [W_gate; W_up] (N = 2I rows) and the SwiGLU and
// 1x128 requantisation fused into the epilogue; shared checks.
static int check_swiglu(const void *A, const float *sa, const void *B, const float *sb,
                        const void *Y, const float *sy, int M, int I, int K, int G,
                        const int32_t *idx, long long a_elems, long long y_elems) {
  if (G < 1 || I < 0) return FP8GEMM_INVALID_ARG;
  const int st = check_common(A, sa, B, sb, Y, M, 2 * I, K, a_elems, (long long)G * 2 * I * K,
                              y_elems);
  if (st != FP8GEMM_OK) return st;
  if (!sy || !idx) return FP8GEMM_INVALID_ARG;
  if (!aligned(sy, 4) || !aligned(idx, 4)) return FP8GEMM_MISALIGNED;
  if (I % 128 != 0 || K > 20480) return FP8GEMM_UNSUPPORTED_SHAPE;
  return FP8GEMM_OK;
}

int grouped_contiguous_swiglu_fp8(const void *A, const float *sa, const void *B, const float *sb,
                                  void *Y, float *sy, int M, int I, int K, int G, void *stream,
                                  const int32_t *m_indices) {
  const int st = check_swiglu(A, sa, B, sb, Y, sy, M, I, K, G, m_indices, (long long)M * K,
                              (long long)M * I);
  if (st != FP8GEMM_OK) return st < 0 ? FP8GEMM_OK : st;
  if (M % 128 != 0) return FP8GEMM_UNSUPPORTED_SHAPE;
  Args a{static_cast<const uint8_t *>(A), sa, static_cast<const uint8_t *>(B), sb, nullptr, M,
         2 * I, K, G, m_indices, 0, 0, 1, K / BK, nullptr, static_cast<uint8_t *>(Y), sy};
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the persistent walk as for the plain contiguous call
  const int P = walk_workgroups();
  const int T = (M / 128) * (I / 128);
  if (!walk_enabled(K) || P < 8 || T <= P || cdiv(T, P) > WALK_MAXIT)
    return launch_tile<4, 2, 4, 4, 3, 4, CONTIG, false, true>(a, 1, s);
  a.tiles_m = M / 128;
  a.tiles_n = I / 128;
  return launch_walk<4, 2, 4, 4, 3, 4, CONTIG, false, true>(a, P, s) == hipSuccess ? FP8GEMM_OK
                                                                                  : FP8GEMM_LAUNCH_FAILED;
}

int grouped_masked_swiglu_fp8(const void *A, const float *sa, const void *B, const float *sb,
                              void *Y, float *sy, int M, int I, int K, int G, void *stream,
                              const int32_t *masked_m, int expected_m) {
  if (expected_m < 0) return FP8GEMM_INVALID_ARG;
  const int st = check_swiglu(A, sa, B, sb, Y, sy, M, I, K, G, masked_m, (long long)G * M * K,
                              (long long)G * M * I);
  if (st != FP8GEMM_OK) return st < 0 ? FP8GEMM_OK : st;
  if (G > 65535) return FP8GEMM_UNSUPPORTED_SHAPE;
  Args a{static_cast<const uint8_t *>(A), sa, static_cast<const uint8_t *>(B), sb, nullptr, M,
         2 * I, K, G, masked_m, 0, 0, 1, K / BK, nullptr, static_cast<uint8_t *>(Y), sy};
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the walk over the live tiles: 13% faster than one workgroup per (tile,
  // expert) here (the plain masked call measured level)
  const int P = walk_workgroups();
  if (!walk_enabled(K) || P < 8 || G > WALK_MAXG)
    return launch_tile<4, 2, 4, 4, 3, 4, MASKED, false, true>(a, G, s);
  a.tiles_m = cdiv(M, 128);
  a.tiles_n = I / 128;
  return launch_walk<4, 2, 4, 4, 3, 4, MASKED, false, true>(a, P, s) == hipSuccess ? FP8GEMM_OK
                                                                                  : FP8GEMM_LAUNCH_FAILED;
}

// BF16 GEMM without scales: shared checks (sizes in elements; bytes are twice)
static int check_bf16(const void *A, const void *B, const void *D, int M, int N, int K,
                      long long a_elems, long long b_elems, long long d_elems) {
  if (M < 0 || N < 0 || K < 0) return FP8GEMM_INVALID_ARG;
  if (M == 0 || N == 0) return -1;  // empty: nothing to do, success
  if (!D) return FP8GEMM_INVALID_ARG;
  if (K > 0 && (!A || !B)) return FP8GEMM_INVALID_ARG;
  if (K % 64 != 0) return FP8GEMM_UNSUPPORTED_SHAPE;
  const long long lim = 1LL << 30;  // 2^31 bytes
  if (a_elems >= lim || b_elems >= lim || d_elems >= lim) return FP8GEMM_UNSUPPORTED_SHAPE;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16)) return FP8GEMM_MISALIGNED;
  return FP8GEMM_OK;
}

int gemm_bf16_nt(const void *A, const void *B, void *D, int M, int N, int K, void *stream) {
  const int st = check_bf16(A, B, D, M, N, K, (long long)M * K, (long long)N * K,
                            (long long)M * N);
  if (st != FP8GEMM_OK) return st < 0 ? FP8GEMM_OK : st;
  Args a{static_cast<const uint8_t *>(A), nullptr, static_cast<const uint8_t *>(B), nullptr,
         static_cast<uint16_t *>(D), M, N, K, 1, nullptr, 0, 0, 1, 2 * K / BK, nullptr};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= 128) return run_decode<true>(a, s);
  return launch_dense_large<2, 4, 4, 4, 3, 4, true>(a, s);
}

int grouped_contiguous_bf16(const void *A, const void *B, void *D, int M, int N, int K, int G,
                            void *stream, const int32_t *m_indices) {
  if (G < 1) return FP8GEMM_INVALID_ARG;
  const int st = check_bf16(A, B, D, M, N, K, (long long)M * K, (long long)G * N * K,
                            (long long)M * N);
  if (st != FP8GEMM_OK) return st < 0 ? FP8GEMM_OK : st;
  if (!m_indices) return FP8GEMM_INVALID_ARG;
  if (!aligned(m_indices, 4)) return FP8GEMM_MISALIGNED;
  if (M % 128 != 0) return FP8GEMM_UNSUPPORTED_SHAPE;
  Args a{static_cast<const uint8_t *>(A), nullptr, static_cast<const uint8_t *>(B), nullptr,
         static_cast<uint16_t *>(D), M, N, K, G, m_indices, 0, 0, 1, 2 * K / BK, nullptr};
  return launch_contig_large<true>(a, static_cast<hipStream_t>(stream));
}

int grouped_masked_bf16(const void *A, const void *B, void *D, int M, int N, int K, int G,
                        void *stream, const int32_t *masked_m, int expected_m) {
  if (G < 1 || expected_m < 0) return FP8GEMM_INVALID_ARG;
  const int st = check_bf16(A, B, D, M, N, K, (long long)G * M * K, (long long)G * N * K,
                            (long long)G * M * N);
  if (st != FP8GEMM_OK) return st < 0 ? FP8GEMM_OK : st;
  if (!masked_m) return FP8GEMM_INVALID_ARG;
  if (!aligned(masked_m, 4)) return FP8GEMM_MISALIGNED;
  if (G > 65535) return FP8GEMM_UNSUPPORTED_SHAPE;
  Args a{static_cast<const uint8_t *>(A), nullptr, static_cast<const uint8_t *>(B), nullptr,
         static_cast<uint16_t *>(D), M, N, K, G, masked_m, 0, 0, 1, 2 * K / BK, nullptr};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (expected_m <= 64)
    return launch_tile<1, 4, 8, 1, 4, 4, MASKED, false, false, true>(a, G, s);
  return launch_tile<1, 4, 8, 2, 4, 4, MASKED, false, false, true>(a, G, s);
}

const char *fp8gemm_status_string(int status) {
  switch (status) {
    case FP8GEMM_OK: return "ok";
    case FP8GEMM_INVALID_ARG: return "invalid argument (null pointer, negative size, G < 1 or expected_m < 0)";
    case FP8GEMM_UNSUPPORTED_SHAPE: return "unsupported shape (K % 128 != 0, contiguous M % 128 != 0, or too large)";
    case FP8GEMM_MISALIGNED: return "misaligned pointer (A, B, D need 16 bytes; scales and indices 4)";
    case FP8GEMM_LAUNCH_FAILED: return "kernel launch failed";
    case FP8GEMM_SCRATCH_EXCEEDED: return "the call's plan needs more than the 32 MB fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

}  // extern "C"
