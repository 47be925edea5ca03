/*
 * fp8ref — the CPU oracle for the FP8 block-scaled NT GEMM and its two MoE
 * grouped layouts, the 1x128 activation quantiser, the grouped GEMM with a
 * fused SwiGLU, and the BF16 GEMM without scales.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg use it; the product path never does.  It shares
 * no source with the GPU library.
 *
 * What it computes (DeepGEMM pages: GeekNews summary "Topic Body", the bullet
 * on fine-grained scaling from DeepSeek-V3, and "성능 평가" for the dense and
 * the two grouped layouts; flashmla.net "Quick Start Guide" for the
 * fp8 x fp8 -> bf16 "nt" operation name):
 *
 *   D[m,n] = bf16( sum_kb  (sa[kb][m] * sb[n/128][kb]) *
 *                          sum_{k in block kb} dec(A[m,k]) * dec(B[n,k]) )
 *
 * A [M,K] and B [N,K] hold OCP e4m3fn codes (K contiguous, "NT"), sa holds one
 * fp32 scale per (row, 128-wide K block) stored K-block-major ([K/128][M]),
 * sb one fp32 scale per 128x128 block of B ([ceil(N/128)][K/128]), D is
 * row-major bf16 bits.
 *
 * Evaluation order, fixed so the result is exact up to one final rounding:
 *   1. each 128-element block sum is formed in fp64; every e4m3 value is an
 *      integer multiple of 2^-9 no larger than 448 in magnitude, so every
 *      product is a multiple of 2^-18 below 2^18 and a 128-term sum stays
 *      below 2^43 * 2^-18: the fp64 block sum is exact in any order;
 *   2. sa*sb is formed in fp64 (exact: 24-bit x 24-bit significands);
 *   3. the term (sa*sb)*blocksum and the sum over kb (ascending) are fp64;
 *   4. one round-to-nearest-even to bf16, written out from IEEE-754.
 * The pages' "promotion" (tensor-core partial sums folded into a CUDA-core
 * fp32 accumulator, GeekNews "Topic Body") is a schedule for reaching this
 * value on the GPU; the oracle needs none, it is exact up to step 4.
 *
 * Parity pins for every exported function live in tests/ (run without a GPU).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef MUTANT
#define MUTANT 0 /* non-zero only in the pin tests' planted-mistake builds */
#endif

/* ---- e4m3fn decode table (OCP 8-bit floating point spec, E4M3) ----------
 * sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
 * subnormal (m * 2^-9); no infinities; S.1111.111 is NaN; max 448. */
static double dec_tab[256];
static pthread_once_t dec_once = PTHREAD_ONCE_INIT;

static void build_dec_tab(void) {
  for (int c = 0; c < 256; ++c) {
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
      v = NAN;
    else if (e == 0)
      v = ldexp((double)m, -9);
    else
      v = ldexp(1.0 + m / 8.0, e - 7);
    dec_tab[c] = s ? -v : v;
  }
}

static const double *dec(void) {
  pthread_once(&dec_once, build_dec_tab);
  return dec_tab;
}

double fp8ref_e4m3_value(int code) { return dec()[code & 255]; }

/* ---- bf16 round-to-nearest-even from fp64 (IEEE-754 binary16-brain:
 * 8 exponent bits as binary32, 8-bit significand incl. the hidden bit).
 * One rounding, no detour through binary32. NaN -> quiet NaN with the sign
 * kept; overflow -> infinity. */
uint16_t fp8ref_bf16_rne(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0 : 0x7FC0);
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int e;
  frexp(a, &e);              /* a in [2^(e-1), 2^e) */
  int lo = e - 1;            /* unbiased exponent of a */
  if (lo < -126) lo = -126;  /* bf16 subnormals share the 2^-126 binade quantum */
  double q = ldexp(1.0, lo - 7); /* spacing of bf16 values in this binade */
#if MUTANT == 4 /* planted mistake: rounds through binary32 first (double rounding) */
  a = (double)(float)a;
#endif
  double r = nearbyint(a / q) * q; /* a/q is exact (power-of-two q); RNE */
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
  /* r is now exactly a bf16 value, hence exactly a binary32 value */
  float f = (float)r;
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return sign | (uint16_t)(bits >> 16);
}

/* exact 128-term block dot product of two e4m3 code rows */
double fp8ref_block_dot(const uint8_t *a, const uint8_t *b) {
  const double *t = dec();
  double s = 0.0;
#if MUTANT == 1 /* planted mistake: last element of each block dropped */
  for (int k = 0; k < 127; ++k) s += t[a[k]] * t[b[k]];
#else
  for (int k = 0; k < 128; ++k) s += t[a[k]] * t[b[k]];
#endif
  return s;
}

/* One output element.  arow/brow: K codes; sa_col: &sa[0][m] with stride
 * sa_stride between K blocks; sb_row: &sb[n/128][0]. */
static double element(const uint8_t *arow, const float *sa_col, long sa_stride,
                      const uint8_t *brow, const float *sb_row, int Kb) {
  double acc = 0.0;
  for (int kb = 0; kb < Kb; ++kb) {
#if MUTANT == 2 /* planted mistake: weight scale taken from block 0 for every kb */
    double scale = (double)sa_col[(long)kb * sa_stride] * (double)sb_row[0];
#elif MUTANT == 3 /* planted mistake: activation scale read as [M][Kb] */
    double scale = (double)sa_col[(long)kb] * (double)sb_row[kb];
#else
    double scale = (double)sa_col[(long)kb * sa_stride] * (double)sb_row[kb];
#endif
    acc += scale * fp8ref_block_dot(arow + (long)kb * 128, brow + (long)kb * 128);
  }
  return acc;
}

/* ---- problem description shared by the threaded drivers ---------------- */
enum { DENSE = 0, CONTIG = 1, MASKED = 2 };

typedef struct {
  int kind;
  const uint8_t *A, *B;
  const float *sa, *sb;
  uint16_t *D;
  double *D64;
  int M, N, K, G;
  const int32_t *m_indices, *masked_m;
  long row_begin, row_end; /* rows of the flattened output: dense/contig m, masked g*M+m */
  uint8_t *act;            /* SwiGLU form (N = 2I): codes [rows][I] and scales ... */
  float *act_scale;        /* ... [G or 1][I/128][M]; D and D64 unused */
  const uint16_t *A16, *B16; /* BF16 form: bf16 operands, no scales (A, B, sa, sb unused) */
} job_t;

static void bf16_row(const job_t *j, long row);

static void swiglu_row(const job_t *j, const uint8_t *A, const float *sa, const uint8_t *B,
                       const float *sb, long row, long m, long g);

static void do_row(const job_t *j, long row) {
  int Kb = j->K / 128, Nb = (j->N + 127) / 128;
  const uint8_t *A = j->A, *B = j->B;
  const float *sa = j->sa, *sb = j->sb;
  long M = j->M, N = j->N, K = j->K;
  long m = row;
  if (j->kind == CONTIG) {
    int g = j->m_indices[row];
#if MUTANT == 5 /* planted mistake: padding rows computed with expert 0 */
    if (g < 0 || g >= j->G) g = 0;
#endif
    if (g < 0 || g >= j->G) return; /* padding row: untouched */
    B += (long)g * N * K;
    sb += (long)g * Nb * Kb;
  } else if (j->kind == MASKED) {
    long g = row / M;
    m = row % M;
    int valid = j->masked_m[g];
    if (valid < 0) valid = 0;
    if (valid > j->M) valid = j->M;
    if (m >= valid) return; /* masked row: untouched */
    A += g * M * K;
    sa += g * (long)Kb * M;
    B += g * N * K;
    sb += g * (long)Nb * Kb;
  }
  if (j->act) {
    swiglu_row(j, A, sa, B, sb, row, m, j->kind == MASKED ? row / M : 0);
    return;
  }
  for (long n = 0; n < N; ++n) {
#if MUTANT == 6 /* planted mistake: B read transposed-in-blocks (column n uses row n^1) */
    long nn = (n ^ 1) < N ? (n ^ 1) : n;
    double v = element(A + m * K, sa + m, M, B + nn * K, sb + (n / 128) * Kb, Kb);
#else
    double v = element(A + m * K, sa + m, M, B + n * K, sb + (n / 128) * Kb, Kb);
#endif
    if (j->D) j->D[row * N + n] = fp8ref_bf16_rne(v);
    if (j->D64) j->D64[row * N + n] = v;
  }
}

static void *worker(void *arg) {
  const job_t *j = (const job_t *)arg;
  for (long r = j->row_begin; r < j->row_end; ++r) {
    if (j->A16)
      bf16_row(j, r);
    else
      do_row(j, r);
  }
  return NULL;
}

static int run(job_t base, long rows, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (rows < threads) threads = rows > 0 ? (int)rows : 1;
  pthread_t tid[256];
  int live[256];
  job_t jobs[256];
  long per = (rows + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    jobs[t] = base;
    jobs[t].row_begin = t * per;
    jobs[t].row_end = (t + 1) * per < rows ? (t + 1) * per : rows;
    live[t] = 0;
    if (jobs[t].row_begin >= jobs[t].row_end) continue;
    if (pthread_create(&tid[t], NULL, worker, &jobs[t]) == 0)
      live[t] = 1;
    else
      worker(&jobs[t]); /* could not start a thread: do the rows here */
  }
  for (int t = 0; t < threads; ++t)
    if (live[t]) pthread_join(tid[t], NULL);
  return 0;
}

static int bad_dims(int M, int N, int K) { return M < 0 || N < 0 || K < 0 || K % 128 != 0; }

/* Dense: D [M,N] bits (nullable), D64 [M,N] unrounded values (nullable). */
int fp8ref_gemm(const uint8_t *A, const float *sa, const uint8_t *B, const float *sb,
                uint16_t *D, double *D64, int M, int N, int K, int threads) {
  if (bad_dims(M, N, K)) return 1;
  job_t j = {DENSE, A, B, sa, sb, D, D64, M, N, K, 1, NULL, NULL, 0, 0};
  return run(j, M, threads);
}

/* M-axis contiguous grouping: B [G,N,K], sb [G,Nb,Kb], m_indices [M]; a row
 * whose index is outside [0,G) is left untouched (GeekNews "성능 평가",
 * contiguous layout: groups stacked along M, N and K shared). */
int fp8ref_grouped_contiguous(const uint8_t *A, const float *sa, const uint8_t *B,
                              const float *sb, uint16_t *D, double *D64, int M, int N,
                              int K, int G, const int32_t *m_indices, int threads) {
  if (bad_dims(M, N, K) || G < 1) return 1;
  job_t j = {CONTIG, A, B, sa, sb, D, D64, M, N, K, G, m_indices, NULL, 0, 0};
  return run(j, M, threads);
}

/* Masked grouping: A [G,M,K], sa [G,Kb,M], B [G,N,K], sb [G,Nb,Kb],
 * D [G,M,N]; only rows m < clamp(masked_m[g], 0, M) are written (GeekNews
 * "성능 평가", masked layout: a mask tensor says how much work each expert
 * has, and only that is computed). */
int fp8ref_grouped_masked(const uint8_t *A, const float *sa, const uint8_t *B,
                          const float *sb, uint16_t *D, double *D64, int M, int N, int K,
                          int G, const int32_t *masked_m, int threads) {
  if (bad_dims(M, N, K) || G < 1) return 1;
  job_t j = {MASKED, A, B, sa, sb, D, D64, M, N, K, G, NULL, masked_m, 0, 0};
  return run(j, (long)G * M, threads);
}

/* Sampled evaluation for sizes where the full output is too slow: value of
 * D at npts points.  For the dense and contiguous layouts a point is (m, n)
 * (g ignored; contiguous looks g up in m_indices and reports NaN bits 0xFFFF
 * for a row that is not written); for the masked layout a point is (g, m, n)
 * and is evaluated whether or not the row is masked (callers choose rows
 * below masked_m). kind: 0 dense, 1 contiguous, 2 masked. */
int fp8ref_points(int kind, const uint8_t *A, const float *sa, const uint8_t *B,
                  const float *sb, int M, int N, int K, int G, const int32_t *m_indices,
                  long npts, const int64_t *pg, const int64_t *pm, const int64_t *pn,
                  uint16_t *out, double *out64) {
  if (bad_dims(M, N, K)) return 1;
  int Kb = K / 128, Nb = (N + 127) / 128;
  for (long i = 0; i < npts; ++i) {
    long m = pm[i], n = pn[i], g = 0;
    const uint8_t *Ag = A, *Bg = B;
    const float *sag = sa, *sbg = sb;
    if (kind == CONTIG) {
      g = m_indices[m];
      if (g < 0 || g >= G) {
        if (out) out[i] = 0xFFFF;
        if (out64) out64[i] = NAN;
        continue;
      }
    } else if (kind == MASKED) {
      g = pg[i];
      Ag += g * (long)M * K;
      sag += g * (long)Kb * M;
    }
    if (kind != DENSE) {
      Bg += g * (long)N * K;
      sbg += g * (long)Nb * Kb;
    }
    double v = element(Ag + m * (long)K, sag + m, M, Bg + n * (long)K, sbg + (n / 128) * Kb, Kb);
    if (out) out[i] = fp8ref_bf16_rne(v);
    if (out64) out64[i] = v;
  }
  return 0;
}

/* ---- 1x128 activation quantisation (the step before the GEMM) ----------
 * The pages leave the FP8 conversion of activations to the caller (kakushin,
 * "Hvorfor FP8 og FP4 er interessant": scales, rounding and layout have to be
 * handled right for low precision to work).  With the 1x128 granularity this
 * library reads, each 128-wide K block x of a row gets one fp32 scale
 *   s = amax|x| / 448   (fp32 division; 1 when the block is all zero;
 *                        NaN elements do not take part in the maximum)
 * and codes e4m3(x / s), the division in fp32 and the encoding to the
 * nearest e4m3fn value, the code's sign being x's.  Input is bf16 bits
 * [M][K]; codes are [M][K], scales are stored K-block-major, sa[kb][m], as
 * the GEMM reads them. */

/* Nearest e4m3fn code to v, written as the definition: a search over the
 * finite codes of v's sign; a tie goes to the even code (mantissa LSB 0);
 * magnitudes past 448 take 448 (the largest finite value); NaN gives the
 * NaN code of its sign. */
uint8_t fp8ref_e4m3_encode(float v) {
  if (isnan(v)) return signbit(v) ? 0xFF : 0x7F;
  const double *d = dec();
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs((double)v);
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    const double diff = fabs(d[c] - a);
#if MUTANT == 7 /* planted mistake: ties go to the larger code */
    if (diff < bestd || diff == bestd) {
#else
    if (diff < bestd || (diff == bestd && (c & 1) == 0)) {
#endif
      best = c;
      bestd = diff;
    }
  }
  return (uint8_t)(sign | best);
}

static float bf16_to_float(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int fp8ref_quantize_1x128(const uint16_t *x, int M, int K, uint8_t *codes, float *sa) {
  if (M < 0 || K < 0 || K % 128 != 0) return 1;
  const int Kb = K / 128;
  for (long m = 0; m < M; ++m)
    for (int kb = 0; kb < Kb; ++kb) {
      const uint16_t *xb = x + m * (long)K + kb * 128;
      float amax = 0.0f;
      for (int k = 0; k < 128; ++k) {
        const float a = fabsf(bf16_to_float(xb[k]));
        if (a > amax) amax = a; /* false for NaN: NaN is skipped */
      }
#if MUTANT == 8 /* planted mistake: scale amax / 447 */
      const float s = amax == 0.0f ? 1.0f : amax / 447.0f;
#else
      const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
#endif
      sa[(long)kb * M + m] = s;
      /* the code's sign is x's: that is the quotient's sign for any s > 0,
       * and it also fixes the sign of the NaN an infinite element gives
       * (inf / inf), which IEEE arithmetic leaves open */
      for (int k = 0; k < 128; ++k) {
        const float xk = bf16_to_float(xb[k]);
        codes[m * (long)K + kb * 128 + k] =
            (uint8_t)(fp8ref_e4m3_encode(fabsf(xk / s)) | (signbit(xk) ? 0x80 : 0x00));
      }
    }
  return 0;
}

/* ---- grouped GEMM with a fused SwiGLU and 1x128 requantisation ----------
 * The step after the grouped GEMM in an MoE expert (kakushin, "Hva gjør
 * DeepGEMM?": the fused MoE flow includes the activation).  B_g holds
 * [W_gate; W_up]: rows 0..I-1 gate, rows I..2I-1 up (N = 2I, I % 128 == 0).
 * For a computed row m (the GEMM's rules: contiguous m_indices[m] in [0,G),
 * masked m < clamp(masked_m[g], 0, M)) and n < I:
 *   g = GEMM(m, n), u = GEMM(m, I + n)   the GEMM oracle's exact values,
 *   y = silu(g) * u = g u / (1 + e^-g)   in fp64, rounded once to fp32;
 * each 128-wide block of y is then quantised like fp8ref_quantize_1x128
 * (s = amax|y| / 448 in fp32, codes of y / s, the sign of y).  Codes are
 * [M][I] (masked [G][M][I]); scales [I/128][M] (masked [G][I/128][M]); rows
 * not computed keep their previous contents. */
static void swiglu_row(const job_t *j, const uint8_t *A, const float *sa, const uint8_t *B,
                       const float *sb, long row, long m, long g) {
  const long M = j->M, K = j->K, I = j->N / 2;
  const int Kb = j->K / 128;
  float y[128];
  for (long b = 0; b < I / 128; ++b) {
    float amax = 0.0f;
    for (long c = 0; c < 128; ++c) {
      const long n = b * 128 + c;
      const double gv = element(A + m * K, sa + m, M, B + n * K, sb + (n / 128) * Kb, Kb);
      const double uv = element(A + m * K, sa + m, M, B + (I + n) * K, sb + ((I + n) / 128) * Kb, Kb);
#if MUTANT == 9 /* planted mistake: gate and up swapped */
      y[c] = (float)(uv / (1.0 + exp(-uv)) * gv);
#else
      y[c] = (float)(gv / (1.0 + exp(-gv)) * uv);
#endif
      const float a = fabsf(y[c]);
      if (a > amax) amax = a;
    }
    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
    j->act_scale[(g * (I / 128) + b) * M + m] = s;
    for (long c = 0; c < 128; ++c)
      j->act[row * I + b * 128 + c] =
          (uint8_t)(fp8ref_e4m3_encode(fabsf(y[c] / s)) | (signbit(y[c]) ? 0x80 : 0x00));
  }
}

int fp8ref_swiglu_quant(int kind, const uint8_t *A, const float *sa, const uint8_t *B,
                        const float *sb, int M, int I, int K, int G, const int32_t *idx,
                        uint8_t *codes, float *scales, int threads) {
  if (bad_dims(M, 2 * I, K) || I % 128 != 0 || G < 1 || (kind != CONTIG && kind != MASKED))
    return 1;
  job_t j;
  memset(&j, 0, sizeof j);
  j.kind = kind;
  j.A = A;
  j.B = B;
  j.sa = sa;
  j.sb = sb;
  j.M = M;
  j.N = 2 * I;
  j.K = K;
  j.G = G;
  j.m_indices = kind == CONTIG ? idx : NULL;
  j.masked_m = kind == MASKED ? idx : NULL;
  j.act = codes;
  j.act_scale = scales;
  return run(j, kind == MASKED ? (long)G * M : (long)M, threads);
}


/* ---- BF16 NT GEMM, no scales --------------------------------------------
 * The pages list BF16 beside FP8 and FP4 among the library's number formats,
 * with the same plain and grouped GEMM forms (kakushin, "Hva gjør
 * DeepGEMM?", its first two items).  With no block scales the operation is
 * the plain product
 *   D[m,n] = bf16( sum_k A[m,k] * B[n,k] )
 * A [M,K] and B [N,K] bf16 bits (K contiguous, "NT"), D [M,N] bf16 bits; the
 * contiguous and masked layouts are the FP8 calls' without their scales
 * (B [G,N,K]; masked A [G,M,K] and D [G,M,N]), with the same row rules.
 * Every product of two bf16 values is exact in fp64 (8-bit significands);
 * the sum runs over k ascending in fp64, then one rounding to bf16 as
 * above.  Any K >= 0 is accepted (K = 0 gives zeros). */
static double bf16_val(uint16_t b) { return (double)bf16_to_float(b); }

static double bf16_dot(const uint16_t *a, const uint16_t *b, long K) {
  double s = 0.0;
#if MUTANT == 10 /* planted mistake: the last product of the sum dropped */
  for (long k = 0; k + 1 < K; ++k) s += bf16_val(a[k]) * bf16_val(b[k]);
#else
  for (long k = 0; k < K; ++k) s += bf16_val(a[k]) * bf16_val(b[k]);
#endif
  return s;
}

static void bf16_row(const job_t *j, long row) {
  const long M = j->M, N = j->N, K = j->K;
  const uint16_t *A = j->A16, *B = j->B16;
  long m = row;
  if (j->kind == CONTIG) {
    const int g = j->m_indices[row];
    if (g < 0 || g >= j->G) return; /* padding row: untouched */
    B += (long)g * N * K;
  } else if (j->kind == MASKED) {
    const long g = row / M;
    m = row % M;
    int valid = j->masked_m[g];
    if (valid < 0) valid = 0;
    if (valid > j->M) valid = j->M;
    if (m >= valid) return; /* masked row: untouched */
    A += g * M * K;
    B += g * N * K;
  }
  for (long n = 0; n < N; ++n) {
#if MUTANT == 11 /* planted mistake: B read as if stored [K][N] */
    double v = 0.0;
    for (long k = 0; k < K; ++k) v += bf16_val(A[m * K + k]) * bf16_val(B[k * N + n]);
#else
    const double v = bf16_dot(A + m * K, B + n * K, K);
#endif
    if (j->D) j->D[row * N + n] = fp8ref_bf16_rne(v);
    if (j->D64) j->D64[row * N + n] = v;
  }
}

/* kind: 0 dense (G = 1, idx unused), 1 contiguous (idx = m_indices [M]),
 * 2 masked (idx = masked_m [G]).  D / D64 nullable as in fp8ref_gemm. */
int fp8ref_gemm_bf16(int kind, const uint16_t *A, const uint16_t *B, uint16_t *D, double *D64,
                     int M, int N, int K, int G, const int32_t *idx, int threads) {
  if (M < 0 || N < 0 || K < 0 || G < 1 || kind < DENSE || kind > MASKED) return 1;
  if (kind != DENSE && !idx) return 1;
  job_t j;
  memset(&j, 0, sizeof j);
  j.kind = kind;
  j.A16 = A;
  j.B16 = B;
  j.D = D;
  j.D64 = D64;
  j.M = M;
  j.N = N;
  j.K = K;
  j.G = kind == DENSE ? 1 : G;
  j.m_indices = kind == CONTIG ? idx : NULL;
  j.masked_m = kind == MASKED ? idx : NULL;
  return run(j, kind == MASKED ? (long)G * M : (long)M, threads);
}
