"""The five synthetic workloads, shaped like the pages' DeepSeek-V3/R1
inference GEMMs (GeekNews "성능 평가": dense shapes from prefill and decode
without tensor parallelism; flashmla.net "Performance That Speaks Volumes":
64x2112x7168, 4 experts x 8192x4096x7168, 4096x7168x16384).

All values are seeded N(0,1) draws quantised to e4m3fn with 1x128 activation
and 128x128 weight amax/448 scales (see synth.c).  Seeds are
1000 * workload + variant.  Each builder returns numpy arrays in the library's
layouts.
"""
from . import act, contiguous_indices, grouped_act, grouped_weight, heavy_rows, masked_counts, weight

SMALL = (128, 256, 512)  # dense M, N, K: the quick parity case
DECODE_NK = ((2112, 7168), (24576, 1536), (7168, 2048), (4096, 7168))
DECODE_SHAPES = tuple((M, N, K) for M in (64, 128) for (N, K) in DECODE_NK)
PREFILL_SHAPES = tuple((4096, N, K) for (N, K) in ((7168, 16384), (2112, 7168), (24576, 1536),
                                                    (7168, 18432)))
CONTIG_CASES = ((4, 32768, 4096, 7168, True), (8, 32768, 4096, 7168, False))  # G, rows, N, K, uniform
MASKED_CASES = ((16, 256, 4096, 7168), (16, 256, 7168, 2048))  # G, M (capacity), N, K
MASKED_EXPECTED_M = 128


def dense(seed, M, N, K, heavy=False, threads=None):
    """A [M,K], sa [K/128,M], B [N,K], sb [Nb,Kb]; heavy=True scales 1% of
    activation rows by 50 before quantisation (the prefill workload)."""
    rm = heavy_rows(seed + 7, M) if heavy else None
    A, sa = act(seed, M, K, row_mult=rm, threads=threads)
    B, sb = weight(seed + 1, N, K, threads=threads)
    return {"A": A, "sa": sa, "B": B, "sb": sb, "M": M, "N": N, "K": K}


def contiguous(seed, G, rows, N, K, uniform, threads=None):
    idx, segs = contiguous_indices(seed + 3, G, rows, uniform)
    A, sa = act(seed, rows, K, threads=threads)
    B, sb = grouped_weight(seed + 1, G, N, K, threads=threads)
    return {"A": A, "sa": sa, "B": B, "sb": sb, "m_indices": idx, "segments": segs,
            "M": rows, "N": N, "K": K, "G": G}


def masked(seed, G, M, N, K, threads=None):
    A, sa = grouped_act(seed, G, M, K, threads=threads)
    B, sb = grouped_weight(seed + 1, G, N, K, threads=threads)
    mm = masked_counts(seed + 5, G, M)
    return {"A": A, "sa": sa, "B": B, "sb": sb, "masked_m": mm, "M": M, "N": N, "K": K, "G": G,
            "expected_m": MASKED_EXPECTED_M}
