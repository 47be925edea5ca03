"""GPU parity of the grouped GEMM with fused SwiGLU and 1x128 requantisation
against the oracle, on identical seeded inputs.

Rows that are not computed (padding rows of the contiguous layout, rows past
masked_m) must keep their sentinel codes and scales bit for bit.  On computed
rows the kernel's y is not the exact one: its h comes from MFMA block sums
and fp32 promotion, and silu uses the hardware exponential and reciprocal.
So, with y the exact value from the oracle's fp64 GEMM and t = y / s in the
kernel's code units:
  - each scale s agrees with the oracle's to 1e-4 relative (s follows the
    block's largest |y|);
  - each code's value lies within half an e4m3 step of t, plus 1e-4 |t|, plus
    1e-4 of the block's largest |t| (448).  The last term covers the error of
    h, which the MFMA's 128-product block sums make of the order of 1e-5 of
    the block maximum (measured: at most 2.5e-5 over these cases);
  - at most 1% of the codes differ from the oracle's (measured: about 0.1%,
    all where t lies near a rounding midpoint).
"""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_act_amd as fg
import oracle
from synth import contiguous_indices, grouped_act, grouped_weight, masked_counts
from synth import act as synth_act
from synth import workloads as W
from parity_util import to_gpu

pytestmark = pytest.mark.gpu

# kernel y against exact y: fp32 error relative to |y| and to the block's largest |y|
Y_REL, Y_ABS = 1e-4, 1e-4
CODE_SENT = 0x7F               # the NaN code: never produced from finite inputs
SCALE_SENT = np.uint32(0x7FBFFFFF)


def announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def e4m3_values():
    return np.array([oracle.e4m3_value(c) for c in range(256)], np.float64)


E4M3 = None


def decode(codes):
    global E4M3
    if E4M3 is None:
        E4M3 = e4m3_values()
    return E4M3[codes]


def sentinels(lead, M, I):
    Y = np.full((*lead, M, I), CODE_SENT, np.uint8)
    sy = np.full((*lead, I // 128, M), SCALE_SENT, np.uint32).view(np.float32)
    return Y, sy


def silu_mul(h, I):
    """exact y from fp64 GEMM values h [..., 2I]"""
    g, u = h[..., :I], h[..., I:]
    return g / (1.0 + np.exp(-g)) * u


def half_step(t):
    """half the spacing of the e4m3fn grid at |t| (t in code units)"""
    a = np.maximum(np.abs(t), 2.0 ** -6)  # the subnormal range has the spacing of the smallest binade
    return 2.0 ** (np.floor(np.log2(a)) - 4)


def check_rows(Yk, syk, Yo, syo, y64, what):
    """Yk, Yo [R, I] codes; syk, syo [I/128, R]; y64 [R, I] exact y."""
    R, I = Yk.shape
    assert (Yk != CODE_SENT).all() and np.isfinite(syk).all(), f"{what}: computed row left unwritten"
    rel = np.abs(syk.astype(np.float64) - syo) / syo
    assert rel.max() <= 1e-4, f"{what}: scale off by {rel.max():.2e} relative"
    sk = np.repeat(syk.T.astype(np.float64), 128, axis=1)          # [R, I] kernel scale per element
    amax = np.repeat(np.abs(y64).reshape(R, I // 128, 128).max(axis=2), 128, axis=1)
    t = y64 / sk                                                    # exact y in the kernel's code units
    err = np.abs(decode(Yk) - t)
    budget = half_step(t) + Y_REL * np.abs(t) + Y_ABS * amax / sk
    over = err > budget
    excess = (err - half_step(t)) / (amax / sk)   # error beyond rounding, relative to the block maximum
    differ = Yk != Yo
    announce(f"{what}: {differ.sum()} of {Yk.size} codes differ from the oracle's; "
             f"largest error beyond rounding {max(excess.max(), 0):.2e} of the block maximum")
    if over.any():
        r, c = np.argwhere(over)[0]
        raise AssertionError(f"{what}: {over.sum()} codes outside the bound; first at row {r} col {c}: "
                             f"t={t[r, c]:.6g} kernel {decode(Yk[r, c])} oracle {decode(Yo[r, c])} "
                             f"block max t={amax[r, c] / sk[r, c]:.6g}")
    assert differ.mean() <= 0.01, f"{what}: {differ.mean():.3%} of codes differ from the oracle's"


def gpu_contig(A, sa, B, sb, idx):
    M, I = A.shape[0], B.shape[1] // 2
    Y0, sy0 = sentinels((), M, I)
    Y, sy = to_gpu(Y0), to_gpu(sy0)
    fg.grouped_contiguous_swiglu_fp8(to_gpu(A), to_gpu(sa), to_gpu(B), to_gpu(sb), to_gpu(idx), Y, sy)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), sy.cpu().numpy()


def gpu_masked(A, sa, B, sb, mm, expected_m=64):
    G, M, I = A.shape[0], A.shape[1], B.shape[1] // 2
    Y0, sy0 = sentinels((G,), M, I)
    Y, sy = to_gpu(Y0), to_gpu(sy0)
    fg.grouped_masked_swiglu_fp8(to_gpu(A), to_gpu(sa), to_gpu(B), to_gpu(sb), to_gpu(mm),
                                 expected_m, Y, sy)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), sy.cpu().numpy()


def oracle_rows(A, sa, B, sb, idx):
    """oracle codes, scales and exact y of the rows of a contiguous-layout
    problem (rows with an index outside [0, G) come back as sentinels)"""
    M, I = A.shape[0], B.shape[1] // 2
    Yo, syo = sentinels((), M, I)
    oracle.swiglu_quant("contiguous", A, sa, B, sb, idx, Yo, syo)
    _, h = oracle.grouped_contiguous(A, sa, B, sb, idx, np.zeros((M, 2 * I), np.uint16), want64=True)
    return Yo, syo, silu_mul(h, I)


def check_rows_chunked(Yk, syk, Yo, syo, y64, what, chunk=4096):
    """check_rows over row chunks (bounded memory for whole workloads)"""
    R = Yk.shape[0]
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        check_rows(Yk[r0:r1], np.ascontiguousarray(syk[:, r0:r1]), Yo[r0:r1],
                   np.ascontiguousarray(syo[:, r0:r1]), y64[r0:r1],
                   what if R <= chunk else f"{what} rows {r0}..{r1 - 1}")


def compare_contig(A, sa, B, sb, idx, Yk, syk, what):
    Yo, syo, y64 = oracle_rows(A, sa, B, sb, idx)
    G = B.shape[0]
    live = (idx >= 0) & (idx < G)
    assert (Yk[~live] == CODE_SENT).all(), f"{what}: a padding row was written"
    assert (syk[:, ~live].view(np.uint32) == SCALE_SENT).all(), f"{what}: a padding scale was written"
    if live.any():
        check_rows_chunked(Yk[live], syk[:, live], Yo[live], syo[:, live], y64[live], what)


@pytest.mark.parametrize("G,rows,I,K,uniform", [
    (2, 256, 128, 256, True),      # one weight tile per expert
    (3, 768, 384, 1280, False),    # odd tile count along I, padded segments
    (4, 1024, 256, 512, False),
])
def test_contiguous_small_full(G, rows, I, K, uniform):
    seed = 9000 + G * 10 + I
    announce(f"swiglu contiguous G={G} rows={rows} I={I} K={K} seed {seed}")
    idx, _ = contiguous_indices(seed + 3, G, rows, uniform)
    A, sa = synth_act(seed, rows, K)
    B, sb = grouped_weight(seed + 1, G, 2 * I, K)
    Yk, syk = gpu_contig(A, sa, B, sb, idx)
    compare_contig(A, sa, B, sb, idx, Yk, syk, f"contiguous G={G} I={I} K={K}")


def test_contiguous_all_padding_block_and_bad_indices():
    """a 128-row block of padding, an index past G and a negative index other
    than -1 leave their rows untouched"""
    G, rows, I, K = 2, 512, 256, 384
    seed = 9100
    idx = np.full(rows, -1, np.int32)
    idx[0:100] = 0
    idx[256:400] = 1
    idx[400:450] = 7    # past G
    idx[450:470] = -5
    announce("swiglu contiguous padding and bad indices")
    A, sa = synth_act(seed, rows, K)
    B, sb = grouped_weight(seed + 1, G, 2 * I, K)
    Yk, syk = gpu_contig(A, sa, B, sb, idx)
    compare_contig(A, sa, B, sb, idx, Yk, syk, "contiguous padding")


def test_contiguous_k_zero():
    """K = 0: every h is an empty sum, so y = 0, codes 0 and scales 1"""
    G, rows, I = 2, 256, 128
    idx = np.repeat(np.arange(G, dtype=np.int32), rows // G)
    A, sa = np.zeros((rows, 0), np.uint8), np.zeros((0, rows), np.float32)
    B, sb = np.zeros((G, 2 * I, 0), np.uint8), np.zeros((G, 2 * I // 128, 0), np.float32)
    announce("swiglu contiguous K=0")
    Yk, syk = gpu_contig(A, sa, B, sb, idx)
    assert (Yk == 0).all() and (syk == 1.0).all()


def masked_case(seed, G, M, I, K, mm):
    A, sa = grouped_act(seed, G, M, K)
    B, sb = grouped_weight(seed + 1, G, 2 * I, K)
    return A, sa, B, sb, np.asarray(mm, np.int32)


def compare_masked(A, sa, B, sb, mm, Yk, syk, what, rows_per_group=None, seed=0):
    """oracle on all valid rows (or a sample of rows_per_group per expert),
    through the contiguous oracle with each row's expert as its index"""
    G, M = A.shape[0], A.shape[1]
    valid = np.clip(mm, 0, M)
    live = np.arange(M)[None, :] < valid[:, None]
    assert (Yk[~live] == CODE_SENT).all(), f"{what}: a masked row was written"
    assert (np.transpose(syk, (0, 2, 1))[~live].view(np.uint32) == SCALE_SENT).all(), \
        f"{what}: a masked scale was written"
    rng = np.random.default_rng(seed)
    pg, pm = [], []
    for g in range(G):
        ms = np.arange(valid[g])
        if rows_per_group is not None and ms.size > rows_per_group:
            edge = [0, valid[g] - 1] + [m for m in (63, 64, 127, 128) if m < valid[g]]
            ms = np.unique(np.concatenate([edge, rng.choice(ms, rows_per_group, replace=False)]))
        pg += [g] * len(ms)
        pm += list(ms)
    if not pg:
        return
    pg, pm = np.array(pg), np.array(pm)
    As = np.ascontiguousarray(A[pg, pm])
    sas = np.ascontiguousarray(sa[pg, :, pm].T)
    idx = pg.astype(np.int32)
    Yo, syo, y64 = oracle_rows(As, sas, B, sb, idx)
    check_rows_chunked(Yk[pg, pm], np.ascontiguousarray(syk[pg, :, pm].T), Yo, syo, y64, what)


@pytest.mark.parametrize("G,M,I,K,mm", [
    (4, 192, 256, 384, [0, 192, 77, 500]),       # empty, full, ragged, clamped to M
    (3, 128, 384, 640, [-3, 1, 128]),            # negative -> 0, a single row
    (2, 320, 128, 1024, [300, 129]),             # ragged last activation tile
])
def test_masked_small_full(G, M, I, K, mm):
    seed = 9200 + G + M
    announce(f"swiglu masked G={G} M={M} I={I} K={K} masked_m={mm} seed {seed}")
    A, sa, B, sb, mm = masked_case(seed, G, M, I, K, mm)
    for expected_m in (0, 64, M):  # the hint must not change the result
        Yk, syk = gpu_masked(A, sa, B, sb, mm, expected_m)
        compare_masked(A, sa, B, sb, mm, Yk, syk, f"masked G={G} M={M} expected_m={expected_m}")


@pytest.mark.parametrize("G", [70, 600])
def test_masked_many_experts(G):
    """More experts than one wave scans at once (70: the walk over live
    tiles) and than the walk takes (600: one workgroup per tile and expert);
    counts of every kind, tiny experts."""
    M, I, K = 40, 128, 256
    seed = 9300 + G
    rng = np.random.default_rng(seed)
    mm = rng.integers(-3, M + 5, G).astype(np.int32)
    mm[:3] = [0, M, 1]
    announce(f"swiglu masked many experts G={G}")
    A, sa, B, sb, mm = masked_case(seed, G, M, I, K, mm)
    Yk, syk = gpu_masked(A, sa, B, sb, mm, 32)
    compare_masked(A, sa, B, sb, mm, Yk, syk, f"masked G={G}", rows_per_group=4, seed=seed)


@pytest.mark.parametrize("case", range(len(W.CONTIG_CASES)))
def test_contiguous_workload_full(case):
    """the gate/up projection of the contiguous workloads (4 experts x 8192
    rows, and 8 uneven padded experts; 32768 rows, I = 2048, K = 7168):
    every padding row untouched, every routed row's codes and scales checked
    against the oracle"""
    G, rows, N, K, uniform = W.CONTIG_CASES[case]
    I = N // 2
    seed = 3000 + 100 * case
    announce(f"swiglu contiguous full size G={G} rows={rows} I={I} K={K} seed {seed}")
    d = W.contiguous(seed, G, rows, N, K, uniform)
    Yk, syk = gpu_contig(d["A"], d["sa"], d["B"], d["sb"], d["m_indices"])
    idx = d["m_indices"]
    live = (idx >= 0) & (idx < G)
    assert (Yk[live] != CODE_SENT).all() and np.isfinite(syk[:, live]).all()
    compare_contig(d["A"], d["sa"], d["B"], d["sb"], idx, Yk, syk, f"contiguous G={G} full size")


def test_masked_workload_full():
    """the masked workload's gate/up projection (16 experts, 256-row
    capacity, I = 2048, K = 7168): every valid row of every expert"""
    G, M, N, K = W.MASKED_CASES[0]
    I = N // 2
    seed = 4000
    announce(f"swiglu masked full size G={G} M={M} I={I} K={K} seed {seed}")
    d = W.masked(seed, G, M, N, K)
    Yk, syk = gpu_masked(d["A"], d["sa"], d["B"], d["sb"], d["masked_m"], d["expected_m"])
    compare_masked(d["A"], d["sa"], d["B"], d["sb"], d["masked_m"], Yk, syk, "masked full size")


def test_moe_layer_chain():
    """The calls compose as an MoE expert layer: quantise the activations,
    gate/up projection with the fused SwiGLU and requantisation, down
    projection.  The quantiser matches the oracle bit for bit; the down
    projection, fed the GPU's codes and scales in the layout the SwiGLU call
    writes them, matches the oracle's GEMM on those operands; padding rows are
    never written."""
    from parity_util import SENTINEL, assert_close, bits
    G, rows, K, I, N = 3, 128 * 4, 512, 256, 384
    seed = 9400
    idx, _ = contiguous_indices(seed, G, rows, False)
    x = np.random.default_rng(seed).standard_normal((rows, K)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    W13, s13 = grouped_weight(seed + 1, G, 2 * I, K)
    W2, s2 = grouped_weight(seed + 2, G, N, I)
    announce("MoE layer chain: quantise -> gate/up + SwiGLU -> down")
    A, sa = fg.quantize_fp8_1x128(xb.cuda())
    Y, sy = fg.grouped_contiguous_swiglu_fp8(A, sa, to_gpu(W13), to_gpu(s13), to_gpu(idx))
    D = torch.full((rows, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    fg.grouped_contiguous(Y, sy, to_gpu(W2), to_gpu(s2), to_gpu(idx), D)
    torch.cuda.synchronize()
    codes, osa = oracle.quantize_1x128(xb.view(torch.int16).numpy().view(np.uint16))
    assert (A.cpu().numpy() == codes).all() and (sa.cpu().numpy() == osa).all()
    Yh, syh = Y.cpu().numpy(), sy.cpu().numpy()
    live = (idx >= 0) & (idx < G)
    ref = oracle.grouped_contiguous(Yh, syh, W2, s2, idx, np.full((rows, N), SENTINEL, np.uint16))
    got = bits(D)
    assert (got[~live] == SENTINEL).all(), "a padding row was written"
    assert_close(got[live], ref[live], "down projection of the SwiGLU output")
