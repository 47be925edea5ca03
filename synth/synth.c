/*
 * synth — seeded synthetic inputs for the FP8 block-scaled GEMM.  It produces
 * e4m3fn codes plus fp32 block scales from N(0,1) draws; it holds none of the
 * GEMM's arithmetic and is shared by the tests, the smoke check and the
 * benchmark (the GPU library and the CPU oracle both consume its output).
 *
 * Random numbers: a counter-based generator, so every element's value depends
 * only on (seed, element index) and not on the thread count.  Each draw is
 * the SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) applied to
 * key(seed) + (counter + 1) * golden_gamma; two such uniforms feed the
 * Box-Muller transform (cosine branch only).
 *
 * Quantisation (the caller's job on the pages: kakushin.no "Hvorfor FP8 og
 * FP4 er interessant" says users must convert to FP8 themselves): the amax
 * of every scale block over its valid elements sets scale = amax / 448 in
 * fp32 (1.0 for an all-zero block); every element is divided by its scale in
 * fp32 and rounded to the nearest e4m3fn value, ties to even, saturating at
 * +-448 (OCP 8-bit floating point spec, E4M3).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static const uint64_t GAMMA = 0x9E3779B97F4A7C15ULL;

static double uniform01(uint64_t key, uint64_t ctr) {
  uint64_t z = mix64(key + (ctr + 1) * GAMMA);
  return ((double)(z >> 11) + 0.5) * (1.0 / 9007199254740992.0); /* (0,1) */
}

/* N(0,1) draw number `idx` of stream `seed` */
static float normal_at(uint64_t seed, uint64_t idx) {
  uint64_t key = mix64(seed * GAMMA + 0x632BE59BD9B4E019ULL);
  double u1 = uniform01(key, 2 * idx);
  double u2 = uniform01(key, 2 * idx + 1);
  return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

void synth_normal(uint64_t seed, uint64_t offset, int64_t n, float *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = normal_at(seed, offset + (uint64_t)i);
}

/* float -> e4m3fn code, round to nearest even, saturating at 448 */
uint8_t synth_e4m3_encode(float xf) {
  if (isnan(xf)) return 0x7F;
  uint8_t sign = signbit(xf) ? 0x80 : 0;
  double a = fabs((double)xf);
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int E = e - 1;          /* floor(log2 a) */
  if (E < -6) E = -6;     /* subnormal binade has the 2^-6 binade's spacing */
  double q = ldexp(1.0, E - 3);
  double r = nearbyint(a / q) * q;
  if (r == 0.0) return sign;
  if (r >= 448.0) return sign | 0x7E;
  frexp(r, &e);
  int Er = e - 1;
  if (Er < -6) return sign | (uint8_t)(r / ldexp(1.0, -9)); /* subnormal: m * 2^-9 */
  int mant = (int)(r / ldexp(1.0, Er) * 8.0) - 8;
  return sign | (uint8_t)(((Er + 7) << 3) | mant);
}

/* ---- activations: one scale per (row, 128-wide K block) --------------- */
typedef struct {
  uint64_t seed, offset;
  int M, K;
  const float *row_mult;
  uint8_t *codes;
  float *sa; /* [K/128][M] */
  int r0, r1;
} act_job;

static void *act_worker(void *p) {
  act_job *j = (act_job *)p;
  float x[128];
  int Kb = j->K / 128;
  for (int m = j->r0; m < j->r1; ++m) {
    float mult = j->row_mult ? j->row_mult[m] : 1.0f;
    for (int kb = 0; kb < Kb; ++kb) {
      uint64_t base = j->offset + (uint64_t)m * j->K + (uint64_t)kb * 128;
      float amax = 0.0f;
      for (int k = 0; k < 128; ++k) {
        x[k] = normal_at(j->seed, base + k) * mult;
        float a = fabsf(x[k]);
        if (a > amax) amax = a;
      }
      float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
      j->sa[(int64_t)kb * j->M + m] = scale;
      uint8_t *dst = j->codes + (int64_t)m * j->K + (int64_t)kb * 128;
      for (int k = 0; k < 128; ++k) dst[k] = synth_e4m3_encode(x[k] / scale);
    }
  }
  return NULL;
}

/* codes [M][K], sa [K/128][M]; draws use indices offset + m*K + k;
 * row_mult (nullable) multiplies row m's draws before quantisation. */
int synth_act(uint64_t seed, uint64_t offset, int M, int K, const float *row_mult,
              uint8_t *codes, float *sa, int threads) {
  if (M < 0 || K < 0 || K % 128) return 1;
  if (threads < 1) threads = 1;
  if (threads > 128) threads = 128;
  pthread_t tid[128];
  act_job jobs[128];
  int live[128];
  int per = (M + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    act_job j = {seed, offset, M, K, row_mult, codes, sa, t * per, (t + 1) * per};
    if (j.r1 > M) j.r1 = M;
    jobs[t] = j;
    live[t] = 0;
    if (j.r0 >= j.r1) continue;
    if (pthread_create(&tid[t], NULL, act_worker, &jobs[t]) == 0)
      live[t] = 1;
    else
      act_worker(&jobs[t]);
  }
  for (int t = 0; t < threads; ++t)
    if (live[t]) pthread_join(tid[t], NULL);
  return 0;
}

/* ---- weights: one scale per 128x128 block ------------------------------ */
typedef struct {
  uint64_t seed, offset;
  int N, K;
  uint8_t *codes;
  float *sb; /* [ceil(N/128)][K/128] */
  int b0, b1; /* row-block range */
} w_job;

static void *w_worker(void *p) {
  w_job *j = (w_job *)p;
  static __thread float x[128 * 128];
  int Kb = j->K / 128;
  for (int nb = j->b0; nb < j->b1; ++nb) {
    int rows = j->N - nb * 128 < 128 ? j->N - nb * 128 : 128;
    for (int kb = 0; kb < Kb; ++kb) {
      float amax = 0.0f;
      for (int r = 0; r < rows; ++r) {
        uint64_t base = j->offset + (uint64_t)(nb * 128 + r) * j->K + (uint64_t)kb * 128;
        for (int k = 0; k < 128; ++k) {
          float v = normal_at(j->seed, base + k);
          x[r * 128 + k] = v;
          float a = fabsf(v);
          if (a > amax) amax = a;
        }
      }
      float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
      j->sb[(int64_t)nb * Kb + kb] = scale;
      for (int r = 0; r < rows; ++r) {
        uint8_t *dst = j->codes + (int64_t)(nb * 128 + r) * j->K + (int64_t)kb * 128;
        for (int k = 0; k < 128; ++k) dst[k] = synth_e4m3_encode(x[r * 128 + k] / scale);
      }
    }
  }
  return NULL;
}

/* codes [N][K], sb [ceil(N/128)][K/128]; draws use indices offset + n*K + k */
int synth_weight(uint64_t seed, uint64_t offset, int N, int K, uint8_t *codes, float *sb,
                 int threads) {
  if (N < 0 || K < 0 || K % 128) return 1;
  int Nb = (N + 127) / 128;
  if (threads < 1) threads = 1;
  if (threads > 128) threads = 128;
  pthread_t tid[128];
  w_job jobs[128];
  int live[128];
  int per = (Nb + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    w_job j = {seed, offset, N, K, codes, sb, t * per, (t + 1) * per};
    if (j.b1 > Nb) j.b1 = Nb;
    jobs[t] = j;
    live[t] = 0;
    if (j.b0 >= j.b1) continue;
    if (pthread_create(&tid[t], NULL, w_worker, &jobs[t]) == 0)
      live[t] = 1;
    else
      w_worker(&jobs[t]);
  }
  for (int t = 0; t < threads; ++t)
    if (live[t]) pthread_join(tid[t], NULL);
  return 0;
}
