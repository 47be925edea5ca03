/* Host-only sanitizer pass (AddressSanitizer + UndefinedBehaviorSanitizer,
 * gcc): builds the CPU oracle and the seeded generator from their sources
 * into one program and drives every function on small inputs with ragged
 * shapes, grouped layouts, out-of-range indices and counts, and the
 * quantiser's special values.  Exits 0 when every call returns its success
 * status; the sanitizers abort on any memory or undefined-behaviour error.
 * Test infrastructure only (run by tests/test_host_sanitizers.py). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int synth_act(uint64_t, uint64_t, int, int, const float *, uint8_t *, float *, int);
int synth_weight(uint64_t, uint64_t, int, int, uint8_t *, float *, int);
void synth_normal(uint64_t, uint64_t, int64_t, float *);
uint8_t synth_e4m3_encode(float);
double fp8ref_e4m3_value(int);
uint16_t fp8ref_bf16_rne(double);
double fp8ref_block_dot(const uint8_t *, const uint8_t *);
int fp8ref_gemm(const uint8_t *, const float *, const uint8_t *, const float *, uint16_t *, double *, int,
                int, int, int);
int fp8ref_grouped_contiguous(const uint8_t *, const float *, const uint8_t *, const float *, uint16_t *,
                              double *, int, int, int, int, const int32_t *, int);
int fp8ref_grouped_masked(const uint8_t *, const float *, const uint8_t *, const float *, uint16_t *,
                          double *, int, int, int, int, const int32_t *, int);
int fp8ref_points(int, const uint8_t *, const float *, const uint8_t *, const float *, int, int, int, int,
                  const int32_t *, long, const int64_t *, const int64_t *, const int64_t *, uint16_t *,
                  double *);
uint8_t fp8ref_e4m3_encode(float);
int fp8ref_quantize_1x128(const uint16_t *, int, int, uint8_t *, float *);
int fp8ref_swiglu_quant(int, const uint8_t *, const float *, const uint8_t *, const float *, int, int, int,
                        int, const int32_t *, uint8_t *, float *, int);
int fp8ref_gemm_bf16(int, const uint16_t *, const uint16_t *, uint16_t *, double *, int, int, int, int,
                     const int32_t *, int);

#define REQUIRE(x)                                                  \
  do {                                                              \
    if (!(x)) {                                                     \
      fprintf(stderr, "failed: %s (line %d)\n", #x, __LINE__);      \
      return 1;                                                     \
    }                                                               \
  } while (0)

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

int main(void) {
  /* exact-size heap buffers, so any out-of-bounds access is reported */
  const int G = 3, M = 130, N = 200, K = 384, Kb = 3, Nb = 2;
  uint8_t *A = xmalloc((size_t)G * M * K), *B = xmalloc((size_t)G * N * K);
  float *sa = xmalloc(sizeof(float) * G * Kb * M), *sb = xmalloc(sizeof(float) * G * Nb * Kb);
  float *mult = xmalloc(sizeof(float) * M);
  for (int m = 0; m < M; ++m) mult[m] = m % 7 == 0 ? 50.f : 1.f;
  for (int g = 0; g < G; ++g) {
    REQUIRE(synth_act(11 + g, 0, M, K, mult, A + (size_t)g * M * K, sa + (size_t)g * Kb * M, 3) == 0);
    REQUIRE(synth_weight(21 + g, 0, N, K, B + (size_t)g * N * K, sb + (size_t)g * Nb * Kb, 2) == 0);
  }
  REQUIRE(synth_act(1, 0, 5, 100, NULL, A, sa, 1) != 0); /* K % 128 != 0 is refused */
  float nrm[17];
  synth_normal(5, 3, 17, nrm);
  REQUIRE(synth_e4m3_encode(NAN) == 0x7F && synth_e4m3_encode(-1e9f) == 0xFE);

  for (int c = 0; c < 256; ++c) (void)fp8ref_e4m3_value(c);
  REQUIRE(fp8ref_bf16_rne(1.0) == 0x3F80 && fp8ref_bf16_rne(NAN) == 0x7FC0);
  REQUIRE(fp8ref_bf16_rne(-INFINITY) == 0xFF80 && fp8ref_bf16_rne(1e300) == 0x7F80);
  REQUIRE(fp8ref_block_dot(A, B) == fp8ref_block_dot(A, B));

  uint16_t *D = xmalloc(sizeof(uint16_t) * G * M * N);
  double *D64 = xmalloc(sizeof(double) * G * M * N);
  REQUIRE(fp8ref_gemm(A, sa, B, sb, D, D64, M, N, K, 4) == 0);
  REQUIRE(fp8ref_gemm(A, sa, B, sb, D, NULL, 1, 1, K, 1) == 0);
  REQUIRE(fp8ref_gemm(A, sa, B, sb, D, NULL, M, N, 0, 2) == 0); /* K = 0: zeros */

  int32_t *idx = xmalloc(sizeof(int32_t) * M);
  for (int m = 0; m < M; ++m) idx[m] = m < 40 ? 2 : m < 90 ? -1 : m < 120 ? 0 : (m == 125 ? 99 : 1);
  REQUIRE(fp8ref_grouped_contiguous(A, sa, B, sb, D, D64, M, N, K, G, idx, 3) == 0);
  int32_t mm[3] = {-4, 77, 1000};
  REQUIRE(fp8ref_grouped_masked(A, sa, B, sb, D, D64, M, N, K, G, mm, 5) == 0);

  enum { P = 9 };
  int64_t pg[P] = {0, 1, 2, 2, 0, 1, 1, 2, 0}, pm[P] = {0, 76, 129, 0, 129, 1, 5, 64, 7},
          pn[P] = {0, 199, 128, 127, 5, 100, 0, 1, 199};
  uint16_t pout[P];
  double p64[P];
  REQUIRE(fp8ref_points(0, A, sa, B, sb, M, N, K, 1, NULL, P, pg, pm, pn, pout, p64) == 0);
  REQUIRE(fp8ref_points(1, A, sa, B, sb, M, N, K, G, idx, P, pg, pm, pn, pout, p64) == 0);
  REQUIRE(fp8ref_points(2, A, sa, B, sb, M, N, K, G, mm, P, pg, pm, pn, pout, NULL) == 0);

  REQUIRE(fp8ref_e4m3_encode(NAN) == 0x7F && fp8ref_e4m3_encode(448.f) == 0x7E);
  uint16_t *X = xmalloc(sizeof(uint16_t) * M * K);
  for (int i = 0; i < M * K; ++i) X[i] = (uint16_t)((i * 2654435761u) >> 16);
  X[3] = 0x7FC0;
  X[200] = 0x7F80;
  X[300] = 0x8000;
  uint8_t *codes = xmalloc((size_t)M * K);
  float *qs = xmalloc(sizeof(float) * Kb * M);
  REQUIRE(fp8ref_quantize_1x128(X, M, K, codes, qs) == 0);
  REQUIRE(fp8ref_quantize_1x128(X, M, 100, codes, qs) != 0);

  const int I = 128;  /* SwiGLU: B rows 2I = 256 per expert */
  uint8_t *B2 = xmalloc((size_t)G * 2 * I * K);
  float *sb2 = xmalloc(sizeof(float) * G * 2 * Kb * 1);
  for (int g = 0; g < G; ++g)
    REQUIRE(synth_weight(31 + g, 0, 2 * I, K, B2 + (size_t)g * 2 * I * K, sb2 + (size_t)g * 2 * Kb, 1) == 0);
  uint8_t *Y = xmalloc((size_t)G * M * I);
  float *sy = xmalloc(sizeof(float) * G * (I / 128) * M);
  REQUIRE(fp8ref_swiglu_quant(1, A, sa, B2, sb2, M, I, K, G, idx, Y, sy, 3) == 0);
  REQUIRE(fp8ref_swiglu_quant(2, A, sa, B2, sb2, M, I, K, G, mm, Y, sy, 3) == 0);

  uint16_t *Ab = xmalloc(sizeof(uint16_t) * G * M * 192), *Bb = xmalloc(sizeof(uint16_t) * G * N * 192);
  for (int i = 0; i < G * M * 192; ++i) Ab[i] = (uint16_t)(0x3C00 + (i % 97));
  for (int i = 0; i < G * N * 192; ++i) Bb[i] = (uint16_t)(0xBC00 + (i % 89));
  REQUIRE(fp8ref_gemm_bf16(0, Ab, Bb, D, D64, M, N, 192, 1, NULL, 2) == 0);
  REQUIRE(fp8ref_gemm_bf16(1, Ab, Bb, D, NULL, M, N, 192, G, idx, 2) == 0);
  REQUIRE(fp8ref_gemm_bf16(2, Ab, Bb, D, D64, M, N, 192, G, mm, 2) == 0);

  free(A); free(B); free(sa); free(sb); free(mult); free(D); free(D64); free(idx); free(X);
  free(codes); free(qs); free(B2); free(sb2); free(Y); free(sy); free(Ab); free(Bb);
  puts("sanitize driver ok");
  return 0;
}
