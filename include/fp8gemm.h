/*
 * libfp8gemm — FP8 (OCP e4m3fn) NT GEMM with fine-grained block scaling and
 * bf16 output, plus its two MoE grouped layouts, for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (DeepGEMM pages: GeekNews summary "Topic Body", which names
 * DeepSeek-V3 fine-grained scaling and the dense and MoE grouped GEMMs;
 * flashmla.net "Quick Start Guide", whose operation name reads
 * fp8 x fp8 -> bf16, "nt"):
 *
 *   D[m,n] = bf16( sum_kb  sa[kb][m] * sb[n/128][kb] *
 *                          sum_{k = 128kb}^{128kb+127}  A[m,k] * B[n,k] )
 *
 * "NT": A is [M,K] and B is [N,K], both with K contiguous; D = A * B^T.
 * The caller supplies FP8 data and any transposition (kakushin.no, "Hvorfor
 * FP8 og FP4 er interessant").  The 1x128 activation / 128x128 weight scale
 * granularity is the reading this library implements; the pages say only
 * "fine-grained".
 *
 * Common conventions for every call below
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the
 *    library keeps no reference after the call returns.
 *  - Layouts are row-major with no padding:
 *      A  : e4m3fn codes, 1 byte each        sa : fp32, [K/128][M] (M contiguous)
 *      B  : e4m3fn codes, 1 byte each        sb : fp32, [ceil(N/128)][K/128]
 *      D  : bf16 bit patterns, 2 bytes each
 *    The last scale block of B covers only the rows that exist when N is not
 *    a multiple of 128.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls are asynchronous on it: a return of FP8GEMM_OK means the work was
 *    enqueued.  No call synchronises or reads device memory on the host, so
 *    every call may be captured into a HIP graph.
 *  - Library-owned memory: the dense calls (FP8 and BF16) may split K over
 *    several workgroups: with M <= 128 for every tile, and with larger M for
 *    the tiles of a last, partly filled wave.  They then enqueue two kernels
 *    (partial products, then their sum in a fixed order, so results are
 *    deterministic) and keep the fp32 partials in a 32 MB library workspace:
 *      . calls made outside graph capture share one workspace per device,
 *        allocated with hipMalloc on first need and kept until the process
 *        ends.  Its users are ordered on the GPU: a call on a stream other
 *        than the previous user's makes its stream wait (hipStreamWaitEvent)
 *        for an event recorded after that user's kernels, so split calls on
 *        different streams never share partials at once (they run one after
 *        the other) and memory does not grow with the number of streams;
 *      . calls captured into a HIP graph use a workspace of that capture
 *        (one per capture and capturing stream), taken from workspaces that
 *        destroyed graphs gave back, else allocated during the capture with
 *        hipMalloc (the thread's capture mode is switched to relaxed for that
 *        one call and restored).  The graph holds it through a user object:
 *        it returns to the library when the graph and every executable
 *        instantiated from it have been destroyed.  A replay, on any stream,
 *        therefore never shares partials with eager calls or other graphs.
 *    If no workspace can be had, the call runs without a K split (the same
 *    results within the tolerance, slower).
 *  - Results are rounded once, fp32 -> bf16, to nearest even; NaN inputs give
 *    NaN outputs.
 *  - Argument errors are reported synchronously, before anything is launched,
 *    as a non-zero status; nothing is written then.  No C++ exception crosses
 *    this interface.  Device-resident index data is never checked on the host
 *    (that would need a synchronisation): its out-of-range values have the
 *    defined meanings given per call.
 *  - Constraints: M, N, K >= 0; K % 128 == 0; A, B and D 16-byte aligned;
 *    sa and sb 4-byte aligned.  M == 0 or N == 0 returns FP8GEMM_OK without
 *    launching; K == 0 writes zeros (an empty sum).
 *  - Calls on different streams may overlap, except that split calls made
 *    outside capture are ordered through the device workspace as above.
 *    Calls on one stream are ordered by the stream.
 */
#ifndef FP8GEMM_H
#define FP8GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fp8gemm_status {
  FP8GEMM_OK = 0,
  FP8GEMM_INVALID_ARG = 1,       /* null pointer for a non-empty problem, negative size, G < 1, expected_m < 0 */
  FP8GEMM_UNSUPPORTED_SHAPE = 2, /* K % 128 != 0; contiguous layout with M % 128 != 0; sizes past 2^31 elements */
  FP8GEMM_MISALIGNED = 3,        /* A, B or D not 16-byte aligned, sa or sb not 4-byte aligned */
  FP8GEMM_LAUNCH_FAILED = 4,     /* the HIP runtime refused one of the call's own launches (an
                                    error left by an earlier HIP call is not reported) */
  FP8GEMM_SCRATCH_EXCEEDED = 5   /* allocation-free entry point only: the call's plan needs more
                                    than its fixed scratch (32 MB) */
};

/*
 * Dense GEMM.  A [M,K], sa [K/128][M], B [N,K], sb [ceil(N/128)][K/128],
 * D [M,N].  Every element of D is written.
 */
int gemm_fp8_1x128_128x128_bf16(const void *A, const float *sa, const void *B, const float *sb,
                                void *D, int M, int N, int K, void *stream);

/*
 * Allocation-free form of the dense GEMM, for callers that cannot allocate
 * device memory: code under HIP graph capture that must not call hipMalloc,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * layouts, kernels and results as gemm_fp8_1x128_128x128_bf16 (bit for bit,
 * where that call gets a workspace); the only difference is where a split
 * call keeps its fp32 partials: a fixed 32 MB device array of the library
 * (one per GPU, created when the library's code is loaded on it and held
 * until the process ends), whose address is looked up on the first call on
 * each device.  The call allocates nothing and calls no allocating routine.
 * Every split call of this entry point on one GPU uses the same array:
 * calls that overlap on one GPU (on different streams, or graph replays)
 * race on it and give wrong results; calls ordered on one stream are safe.
 * Nothing in the array needs clearing (each call overwrites the partials it
 * reads).  Every default plan fits 32 MB; a plan that needs more (possible
 * only through a tuning override) returns FP8GEMM_SCRATCH_EXCEEDED before
 * anything is launched.
 */
int gemm_fp8_1x128_128x128_bf16_noalloc(const void *A, const float *sa, const void *B,
                                        const float *sb, void *D, int M, int N, int K,
                                        void *stream);

/*
 * M-axis contiguous grouped GEMM (GeekNews "성능 평가", contiguous layout:
 * the experts' rows are stacked along M and share N and K).
 *   A [M,K] and sa [K/128][M] hold all experts' rows; B [G][N,K] and
 *   sb [G][ceil(N/128)][K/128] hold one weight matrix per expert; D [M,N].
 *   m_indices [M] (int32, device) gives each row's expert.  Row m is computed
 *   with expert m_indices[m]; a row whose index is outside [0,G) (e.g. -1
 *   for padding) is not written and keeps its previous contents.
 * Contract: M % 128 == 0, and each aligned 128-row block of A holds rows of
 * at most one expert (expert segments start at multiples of 128; padding
 * rows may sit anywhere).  A block that breaks it is computed for the
 * largest valid expert index among its rows; its rows of other experts are
 * not written.
 */
int grouped_contiguous(const void *A, const float *sa, const void *B, const float *sb, void *D,
                       int M, int N, int K, int G, void *stream, const int32_t *m_indices);

/*
 * Masked grouped GEMM (GeekNews "성능 평가", masked layout: for graph
 * replay, where the host cannot know each expert's token count, a device
 * mask says how many rows of each expert are real and only those are
 * computed).
 *   A [G][M,K], sa [G][K/128][M], B [G][N,K], sb [G][ceil(N/128)][K/128],
 *   D [G][M,N]; M is the per-expert row capacity.
 *   masked_m [G] (int32, device): expert g's rows m < clamp(masked_m[g], 0, M)
 *   are computed and written; its other rows keep their previous contents.
 *   expected_m (host, >= 0) is a hint of the typical masked_m used to choose
 *   tile shapes; it never changes which elements are written or their values
 *   beyond the stated tolerance.
 */
int grouped_masked(const void *A, const float *sa, const void *B, const float *sb, void *D,
                   int M, int N, int K, int G, void *stream, const int32_t *masked_m,
                   int expected_m);

/*
 * 1x128 activation quantisation: the FP8 conversion the pages leave to the
 * caller (kakushin.no, "Hvorfor FP8 og FP4 er interessant"), producing the A
 * and sa operands of the calls above.
 *   X [M,K] bf16 bits (device, read); A [M,K] e4m3fn codes (device, written);
 *   sa [K/128][M] fp32 (device, written; M contiguous as the GEMM reads it).
 *   For each row m and 128-wide K block x:
 *     s = amax|x| / 448 (IEEE fp32 division; 1 for an all-zero block; NaN
 *         elements take no part in the maximum),
 *     A = the e4m3fn value nearest to x / s (IEEE fp32 division), ties to the
 *         even code, magnitudes past 448 saturating to 448, NaN to the NaN
 *         code; the sign bit of every code is the sign of x (so -0 stays
 *         -0, and an infinite element, whose block scale is infinite, gives
 *         the NaN code of its own sign).
 * Constraints: K % 128 == 0; X and A 16-byte aligned, sa 4-byte aligned;
 * M * K * 2 < 2^31.  M == 0 or K == 0 returns FP8GEMM_OK without launching.
 * Allocates nothing; asynchronous on `stream` like the calls above.
 */
int quantize_fp8_1x128(const void *X, void *A, float *sa, int M, int K, void *stream);

/*
 * Grouped GEMM with the expert's activation fused into its epilogue: the
 * linear layer and the activation that the pages' fused MoE flow chains
 * (kakushin.no, "Hva gjør DeepGEMM?", the Mega MoE item).  The pages name no
 * activation; this is the SwiGLU reading, followed by the 1x128 FP8
 * requantisation the next expert GEMM reads, so y never goes to memory in
 * a wider type.
 *   Each expert's weights B_g [2I,K] stack the gate projection (rows 0..I-1)
 *   over the up projection (rows I..2I-1), with sb_g [2I/128][K/128].  With
 *   h = the fp32 block-scaled sum of the calls above, taken before any bf16
 *   rounding,
 *     y[m,n] = silu(h[m,n]) * h[m,I+n],   silu(x) = x / (1 + e^-x),  n < I,
 *   is quantised per row and 128-wide block of n as quantize_fp8_1x128
 *   quantises x (the same scale and code rules, applied to the fp32 y):
 *   codes Y [.., I] and scales sy [I/128][M] (M contiguous).  y is formed
 *   in fp32 with the hardware exponential and reciprocal, from h as the
 *   MFMA block sums give it, so it is not the exact y: a code may be one
 *   step off where the exact y / s lies near a rounding midpoint (about 0.1%
 *   of codes on random data), and a scale a few fp32 ulps off.
 * Rows are selected as in the grouped calls above; rows not computed keep
 * their previous codes and scales.  No bf16 output is written.
 * Constraints beyond the grouped calls: I % 128 == 0 and K <= 20480
 * (FP8GEMM_UNSUPPORTED_SHAPE otherwise); sy 4-byte aligned; Y 16-byte
 * aligned.  Allocates nothing.
 */
/* Contiguous layout: A [M,K], sa [K/128][M], B [G][2I,K],
 * sb [G][2I/128][K/128], m_indices [M]; Y [M,I], sy [I/128][M]. */
int grouped_contiguous_swiglu_fp8(const void *A, const float *sa, const void *B, const float *sb,
                                  void *Y, float *sy, int M, int I, int K, int G, void *stream,
                                  const int32_t *m_indices);

/* Masked layout: A [G][M,K], sa [G][K/128][M], B [G][2I,K],
 * sb [G][2I/128][K/128], masked_m [G]; Y [G][M,I], sy [G][I/128][M]. */
int grouped_masked_swiglu_fp8(const void *A, const float *sa, const void *B, const float *sb,
                              void *Y, float *sy, int M, int I, int K, int G, void *stream,
                              const int32_t *masked_m, int expected_m);

/*
 * BF16 NT GEMM without scales: the pages list BF16 beside FP8 among the
 * library's number formats, with the same plain and grouped GEMM forms
 * (kakushin.no, "Hva gjør DeepGEMM?", its first two items).
 *   D[m,n] = bf16( sum_k A[m,k] * B[n,k] ), fp32 accumulation in the MFMA.
 * A, B and D hold bf16 bit patterns (2 bytes each), row-major, K contiguous
 * in A and B.  Layouts and row rules are those of the FP8 calls above with
 * the scales removed: dense A [M,K], B [N,K], D [M,N]; contiguous adds
 * B [G][N,K] and m_indices [M]; masked has A [G][M,K], B [G][N,K],
 * D [G][M,N] and masked_m [G].  Conventions as above (device pointers,
 * asynchronous on `stream`, errors before any launch, the same workspace
 * rule for the dense call with M <= 128).
 * Constraints: K % 64 == 0 (FP8GEMM_UNSUPPORTED_SHAPE otherwise); every
 * tensor below 2^31 bytes; A, B and D 16-byte aligned.  M == 0 or N == 0
 * returns FP8GEMM_OK without launching; K == 0 writes zeros.
 */
int gemm_bf16_nt(const void *A, const void *B, void *D, int M, int N, int K, void *stream);

int grouped_contiguous_bf16(const void *A, const void *B, void *D, int M, int N, int K, int G,
                            void *stream, const int32_t *m_indices);

int grouped_masked_bf16(const void *A, const void *B, void *D, int M, int N, int K, int G,
                        void *stream, const int32_t *masked_m, int expected_m);

/* Static, human-readable text for a status code (never NULL). */
const char *fp8gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8GEMM_H */
