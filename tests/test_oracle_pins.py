"""Pins for the CPU oracle: what the pages and the mathematics fix, checked
without a GPU and without re-using the oracle's own code.

Each pin is chosen so a plausible mistake in the oracle fails it; the
planted-mistake tests at the bottom compile the oracle with such mistakes
and check that at least one pin fails for each.
"""
import math
import os
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

# ---------------------------------------------------------------- helpers ----


def torch_e4m3_values():
    """All 256 e4m3fn codes decoded by PyTorch's float8_e4m3fn (an
    independent implementation of the OCP format)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


TV = torch_e4m3_values()
FINITE = np.array([c for c in range(256) if not math.isnan(TV[c])], dtype=np.uint8)


def frac_value(code):
    return Fraction(float(TV[code]))


def exact_bf16_bits(x: Fraction) -> int:
    """Round an exact rational to bf16, ties to even, by exact comparisons."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    r = a / q
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * q
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    f32 = np.array([float(val)], np.float32)
    return sign | int(f32.view(np.uint32)[0] >> 16)


def exact_gemm_bits(A, sa, B, sb):
    """Whole-result brute force in exact rationals (tiny sizes only)."""
    M, K = A.shape
    N = B.shape[0]
    Kb = K // 128
    out = np.zeros((M, N), np.uint16)
    fa = [[frac_value(c) for c in row] for row in A]
    fb = [[frac_value(c) for c in row] for row in B]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for kb in range(Kb):
                blk = sum(fa[m][k] * fb[n][k] for k in range(kb * 128, kb * 128 + 128))
                tot += Fraction(float(sa[kb, m])) * Fraction(float(sb[n // 128, kb])) * blk
            out[m, n] = exact_bf16_bits(tot)
    return out


def rand_codes(rng, shape, finite=True):
    pool = FINITE if finite else np.arange(256, dtype=np.uint8)
    return rng.choice(pool, size=shape).astype(np.uint8)


def bits_to_f32(b):
    return oracle.bf16_bits_to_float(b)


def read_table(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ------------------------------------------------------ P1: e4m3 decoding ----


def test_e4m3_anchors_from_spec(golden_dir):
    for code, val in read_table(os.path.join(golden_dir, "e4m3fn_anchors.txt")):
        c = int(code, 16)
        got = oracle.e4m3_value(c)
        if val == "nan":
            assert math.isnan(got), code
            continue
        want = float.fromhex(val) if "p" in val else float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e4m3_all_codes_match_torch():
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan_g, nan_t = np.isnan(got), np.isnan(TV)
    assert (nan_g == nan_t).all() and nan_g.sum() == 2
    assert (got[~nan_g] == TV[~nan_t]).all()
    assert (np.signbit(got[~nan_g]) == np.signbit(TV[~nan_t])).all()


def test_e4m3_monotone_and_symmetric():
    pos = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))
    for c in range(0x7F):
        assert oracle.e4m3_value(c | 0x80) == -oracle.e4m3_value(c)


# ------------------------------------------------------ bf16 rounding -------


def test_bf16_anchors(golden_dir):
    for lit, hexbits in read_table(os.path.join(golden_dir, "bf16_rne_anchors.txt")):
        assert oracle.bf16_rne(float(lit)) == int(hexbits, 16), lit


def test_bf16_rounding_brute_force():
    rng = np.random.default_rng(7)
    mags = np.concatenate([
        rng.uniform(-1, 1, 4000) * 2.0 ** rng.integers(-140, 127, 4000),
        rng.standard_normal(4000),
    ])
    for x in mags:
        x = float(x)
        assert oracle.bf16_rne(x) == exact_bf16_bits(Fraction(x)), x


def test_bf16_ties_exhaustive_one_binade():
    # every tie point between consecutive bf16 values in [1, 2)
    for mant in range(128):
        lo = 1 + mant / 128
        tie = lo + 1 / 256
        want = 0x3F80 + mant + (mant % 2)  # to the even neighbour
        assert oracle.bf16_rne(tie) == want
        assert oracle.bf16_rne(math.nextafter(tie, 3)) == 0x3F80 + mant + 1
        assert oracle.bf16_rne(math.nextafter(tie, 0)) == 0x3F80 + mant


# ------------------------------------------------------ P2: block exactness -


def test_block_dot_exact_integer():
    rng = np.random.default_rng(11)
    ints = (TV * 512).round()  # every finite e4m3 value is an integer multiple of 2^-9
    assert np.all(ints[np.isfinite(TV)] == TV[np.isfinite(TV)] * 512)
    for _ in range(300):
        a = rand_codes(rng, 128)
        b = rand_codes(rng, 128)
        want = sum(int(ints[x]) * int(ints[y]) for x, y in zip(a, b))
        assert oracle.block_dot(a, b) == want / 2 ** 18


def test_block_dot_worst_case():
    a = np.full(128, 0x7E, np.uint8)
    assert oracle.block_dot(a, a) == 128 * 448.0 ** 2
    b = np.where(np.arange(128) % 2 == 0, 0x7E, 0xFE).astype(np.uint8)
    assert oracle.block_dot(a, b) == 0.0
    assert oracle.block_dot(b, b) == 128 * 448.0 ** 2


def test_nan_propagates():
    rng = np.random.default_rng(3)
    A = rand_codes(rng, (2, 256))
    B = rand_codes(rng, (3, 256))
    A[1, 200] = 0x7F
    sa = np.ones((2, 2), np.float32)
    sb = np.ones((1, 2), np.float32)
    D = oracle.gemm(A, sa, B, sb)
    f = bits_to_f32(D)
    assert np.isnan(f[1]).all() and not np.isnan(f[0]).any()


# ------------------------------------------------------ P3: whole result ----


@pytest.mark.parametrize("M,N,K,seed", [(3, 5, 128, 1), (4, 131, 256, 2), (2, 3, 512, 3)])
def test_tiny_gemm_exact_rational(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rand_codes(rng, (M, K))
    B = rand_codes(rng, (N, K))
    sa = rng.uniform(0.001, 2, (K // 128, M)).astype(np.float32)
    sb = rng.uniform(0.001, 2, ((N + 127) // 128, K // 128)).astype(np.float32)
    D = oracle.gemm(A, sa, B, sb)
    if N > 128:  # a few columns on both sides of the scale-block boundary
        for c in [0, 1, 127, 128, 129, N - 1]:
            w = exact_gemm_bits(A, sa, B[c:c + 1], sb[c // 128:c // 128 + 1])
            assert (D[:, c] == w[:, 0]).all(), c
    else:
        assert (D == exact_gemm_bits(A, sa, B, sb)).all()


def test_dequantize_then_matmul_fp64():
    """Independent formulation: scale every element first, then one matmul."""
    rng = np.random.default_rng(5)
    M, N, K = 37, 300, 512
    A, sa = synth.act(101, M, K)
    B, sb = synth.weight(102, N, K)
    D, D64 = oracle.gemm(A, sa, B, sb, want64=True)
    Ad = TV[A] * np.repeat(sa.T.astype(np.float64), 128, axis=1)
    Bd = TV[B] * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    ref = Ad @ Bd.T
    assert np.allclose(D64, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # bf16 of the independent value agrees except where fp64 error meets a tie
    ref_bits = np.array([exact_bf16_bits(Fraction(float(v))) for v in ref.ravel()[:3000]])
    assert (ref_bits == D.ravel()[:3000]).mean() > 0.999
    del rng


# ------------------------------------------------------ P4: identity / perm -


def test_identity_and_permutation_exact():
    rng = np.random.default_rng(9)
    M, N, K = 128, 200, 256
    B = rand_codes(rng, (N, K))
    sb = (2.0 ** rng.integers(-3, 4, ((N + 127) // 128, K // 128))).astype(np.float32)
    perm = rng.permutation(K)[:M]
    A = np.zeros((M, K), np.uint8)
    A[np.arange(M), perm] = 0x38  # 1.0
    sa = np.ones((K // 128, M), np.float32)
    D = oracle.gemm(A, sa, B, sb)
    n = np.arange(N)
    want = TV[B[:, perm]].T * sb[n // 128][:, perm // 128].T  # [M, N]
    want_bits = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # e4m3 values times powers of two have at most 4 significant bits: exact in bf16
    assert (bits_to_f32(want_bits) == want).all()
    # compare values: a zero product's sign is not part of the definition
    assert (bits_to_f32(D) == bits_to_f32(want_bits)).all()


# ------------------------------------------------------ P5: power-of-two ----


def test_power_of_two_scales_linearity():
    M, N, K = 16, 2112, 256
    A, sa = synth.act(201, M, K)
    B, sb = synth.weight(202, N, K)
    D1 = oracle.gemm(A, sa, B, sb)
    D2 = oracle.gemm(A, sa * 2, B, sb)
    f1, f2 = bits_to_f32(D1), bits_to_f32(D2)
    assert (f2 == 2 * f1).all()
    sb2 = sb.copy()
    sb2[16] *= 4  # the partial block: columns 2048..2111
    D3 = oracle.gemm(A, sa, B, sb2)
    f3 = bits_to_f32(D3)
    assert (f3[:, :2048] == f1[:, :2048]).all()
    assert (f3[:, 2048:] == 4 * f1[:, 2048:]).all()
    # one K block's activation scale for one row only affects that row
    sa3 = sa.copy()
    sa3[1, 5] *= 0.5
    f4 = bits_to_f32(oracle.gemm(A, sa3, B, sb))
    rows = np.arange(M) != 5
    assert (f4[rows] == f1[rows]).all() and (f4[5] != f1[5]).any()


def test_exact_small_values_power_of_two_scales():
    """codes in {0, +-0.5, +-1, +-1.5, +-2}, power-of-two scales: exact sums."""
    rng = np.random.default_rng(13)
    M, N, K = 64, 192, 512
    pool = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x3C, 0xBC, 0x40, 0xC0], np.uint8)
    A = rng.choice(pool, (M, K))
    B = rng.choice(pool, (N, K))
    sa = (2.0 ** rng.integers(-2, 3, (K // 128, M))).astype(np.float32)
    sb = (2.0 ** rng.integers(-2, 3, (2, K // 128))).astype(np.float32)
    D, D64 = oracle.gemm(A, sa, B, sb, want64=True)
    ints = np.rint(TV[A] * 2) @ np.rint(TV[B] * 2).T  # exact integer check of one scale set
    assert np.all(np.abs(D64) < 2 ** 20)
    # recompute exactly per block in integers
    tot = np.zeros((M, N))
    for kb in range(K // 128):
        s = slice(kb * 128, kb * 128 + 128)
        blk = np.rint(TV[A[:, s]] * 2) @ np.rint(TV[B[:, s]] * 2).T / 4
        tot += blk * sa[kb][:, None] * sb[np.arange(N) // 128, kb][None, :]
    assert (tot == D64).all()
    del ints


# ------------------------------------------------------ P6: grouped layouts -


def test_contiguous_rows_equal_dense_with_their_expert():
    G, N, K = 3, 160, 256
    idx, segs = synth.contiguous_indices(31, G, 128 * 5, uniform=False)
    M = idx.shape[0]
    A, sa = synth.act(301, M, K)
    B, sb = synth.grouped_weight(302, G, N, K)
    sentinel = np.full((M, N), 0x7FBF, np.uint16)
    D = oracle.grouped_contiguous(A, sa, B, sb, idx, sentinel.copy())
    for g in range(G):
        Dg = oracle.gemm(A, sa, B[g], sb[g])
        rows = idx == g
        assert (D[rows] == Dg[rows]).all()
    assert (D[idx < 0] == 0x7FBF).all()
    assert (idx < 0).sum() > 0


def test_contiguous_out_of_range_index_is_padding():
    G, N, K, M = 2, 64, 128, 256
    A, sa = synth.act(311, M, K)
    B, sb = synth.grouped_weight(312, G, N, K)
    idx = np.zeros(M, np.int32)
    idx[128:] = 1
    idx[5], idx[200], idx[201] = -1, 2, 99
    D = oracle.grouped_contiguous(A, sa, B, sb, idx, np.full((M, N), 0x7FBF, np.uint16))
    for r in (5, 200, 201):
        assert (D[r] == 0x7FBF).all()
    assert (D[(idx >= 0) & (idx < G)] != 0x7FBF).all()


def test_routing_probe_reveals_expert():
    """B_g = 2^g * (identity-like), A rows = unit vectors: D shows g exactly."""
    G, N, K, M = 4, 128, 128, 512
    B = np.zeros((G, N, K), np.uint8)
    B[:, np.arange(N), np.arange(K)] = 0x38
    sb = np.stack([np.full((1, 1), 2.0 ** g, np.float32) for g in range(G)])
    A = np.zeros((M, K), np.uint8)
    A[np.arange(M), np.arange(M) % K] = 0x38
    sa = np.ones((1, M), np.float32)
    idx = (np.arange(M) // 128).astype(np.int32)[::-1].copy()
    D = oracle.grouped_contiguous(A, sa, B, sb, idx, np.zeros((M, N), np.uint16))
    f = bits_to_f32(D)
    for m in range(M):
        assert f[m, m % K] == 2.0 ** idx[m] and np.count_nonzero(f[m]) == 1


def test_masked_full_equals_dense_and_zero_untouched():
    G, M, N, K = 3, 96, 130, 256
    A, sa = synth.grouped_act(401, G, M, K)
    B, sb = synth.grouped_weight(402, G, N, K)
    mm = np.array([M, 0, 37], np.int32)
    D = oracle.grouped_masked(A, sa, B, sb, mm, np.full((G, M, N), 0x7FBF, np.uint16))
    assert (D[0] == oracle.gemm(A[0], sa[0], B[0], sb[0])).all()
    assert (D[1] == 0x7FBF).all()
    D2 = oracle.gemm(A[2], sa[2], B[2], sb[2])
    assert (D[2, :37] == D2[:37]).all() and (D[2, 37:] == 0x7FBF).all()


def test_masked_counts_clamped():
    G, M, N, K = 2, 64, 64, 128
    A, sa = synth.grouped_act(411, G, M, K)
    B, sb = synth.grouped_weight(412, G, N, K)
    D = oracle.grouped_masked(A, sa, B, sb, np.array([M + 50, -7], np.int32),
                              np.full((G, M, N), 0x7FBF, np.uint16))
    assert (D[0] == oracle.gemm(A[0], sa[0], B[0], sb[0])).all()
    assert (D[1] == 0x7FBF).all()


def test_points_equal_full_output():
    rng = np.random.default_rng(17)
    M, N, K = 50, 260, 384
    A, sa = synth.act(501, M, K)
    B, sb = synth.weight(502, N, K)
    D = oracle.gemm(A, sa, B, sb)
    pm = rng.integers(0, M, 200)
    pn = rng.integers(0, N, 200)
    assert (oracle.points("dense", A, sa, B, sb, pm, pn) == D[pm, pn]).all()
    G = 2
    Ag, sag = synth.grouped_act(503, G, M, K)
    Bg, sbg = synth.grouped_weight(504, G, N, K)
    Dm = oracle.grouped_masked(Ag, sag, Bg, sbg, np.array([M, M], np.int32),
                               np.zeros((G, M, N), np.uint16))
    pg = rng.integers(0, G, 200)
    assert (oracle.points("masked", Ag, sag, Bg, sbg, pm, pn, pg=pg) == Dm[pg, pm, pn]).all()
    idx = np.where(np.arange(M) < 25, 0, 1).astype(np.int32)
    idx[3] = -1
    Dc = oracle.grouped_contiguous(A, sa, Bg, sbg, idx, np.zeros((M, N), np.uint16))
    got = oracle.points("contiguous", A, sa, Bg, sbg, pm, pn, m_indices=idx)
    ok = idx[pm] >= 0
    assert (got[ok] == Dc[pm, pn][ok]).all() and (got[~ok] == 0xFFFF).all()


def test_empty_problems():
    A = np.zeros((0, 128), np.uint8)
    B = np.zeros((5, 128), np.uint8)
    D = oracle.gemm(A, np.zeros((1, 0), np.float32), B, np.ones((1, 1), np.float32))
    assert D.shape == (0, 5)
    # K = 0: an empty sum, every element is +0
    D = oracle.gemm(np.zeros((3, 0), np.uint8), np.zeros((0, 3), np.float32),
                    np.zeros((4, 0), np.uint8), np.zeros((1, 0), np.float32))
    assert (D == 0).all()


# ------------------------------------------- 1x128 activation quantiser ----


def torch_e4m3_bits(v):
    """PyTorch's own float32 -> float8_e4m3fn conversion (round to nearest
    even; callers keep |v| below the overflow threshold)."""
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_of(x):
    """float32 array -> bf16 bits (round to nearest even) and its exact value"""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16), t.to(torch.float32).numpy()


def test_e4m3_encode_round_trips_every_code():
    for c in FINITE:
        assert oracle.e4m3_encode(TV[c]) == c if not (c == 0x80) else oracle.e4m3_encode(-0.0) == 0x80


def test_e4m3_encode_ties_go_to_even():
    pos = [c for c in FINITE if c < 0x7F]
    for c in pos[:-1]:
        mid = (TV[c] + TV[c + 1]) / 2  # exact in fp32
        assert np.float32(mid) == mid
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even, hex(c)
        assert oracle.e4m3_encode(-mid) == even | 0x80


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(31)
    mag = 2.0 ** rng.uniform(-12, np.log2(448), 20000)
    v = (mag * rng.choice([-1, 1], mag.size)).astype(np.float32)
    got = np.array([oracle.e4m3_encode(x) for x in v], np.uint8)
    assert (got == torch_e4m3_bits(v)).all()


def test_e4m3_encode_saturates_and_nan():
    for v in (448.0, 449.0, 463.99, 464.0, 1e6, float("inf")):
        assert oracle.e4m3_encode(v) == 0x7E and oracle.e4m3_encode(-v) == 0xFE
    assert oracle.e4m3_encode(float("nan")) in (0x7F, 0xFF)


def test_quantize_1x128_definition():
    rng = np.random.default_rng(32)
    M, K = 6, 512
    xb, x = bf16_of(rng.standard_normal((M, K)).astype(np.float32) * 3)
    x[2, 128:256] = 0.0
    xb[2, 128:256] = 0  # an all-zero block
    xb[4, 10] = np.uint16(0x7FC0)  # a NaN element (skipped by the maximum)
    x[4, 10] = np.nan
    codes, sa = oracle.quantize_1x128(xb)
    for m in range(M):
        for kb in range(K // 128):
            blk = x[m, kb * 128:(kb + 1) * 128]
            amax = np.float32(np.nanmax(np.abs(blk)))
            s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0))
            assert sa[kb, m] == s
            q = (blk / s).astype(np.float32)
            ok = ~np.isnan(q)
            assert (codes[m, kb * 128:(kb + 1) * 128][ok] == torch_e4m3_bits(q[ok])).all()
            assert (codes[m, kb * 128:(kb + 1) * 128][~ok] & 0x7F == 0x7F).all()
            if amax > 0:  # the block's largest magnitude lands on +-448
                j = int(np.nanargmax(np.abs(blk)))
                assert codes[m, kb * 128 + j] & 0x7F == 0x7E
    assert (sa[1, 2] == 1.0) and (codes[2, 128:256] == 0).all()


def test_quantize_1x128_error_bound():
    rng = np.random.default_rng(33)
    xb, x = bf16_of((rng.standard_normal((8, 1024)) * np.exp(rng.uniform(-8, 8, (8, 1)))).astype(np.float32))
    codes, sa = oracle.quantize_1x128(xb)
    deq = TV[codes] * np.repeat(sa.T, 128, axis=1)
    # normal e4m3 values carry 3 fraction bits: half a step is 2^-4 relative;
    # below 2^-6 (in units of the scale) the step is 2^-9
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.repeat(sa.T, 128, axis=1) * 2.0 ** -10)
    assert (np.abs(deq - x) <= bound * (1 + 1e-6)).all()


# ------------------------------- grouped GEMM + SwiGLU + requantisation ----


def independent_swiglu_quant(A, sa, Bg, sbg):
    """dequantise, fp64 matmul, y = g u / (1 + e^-g) rounded to fp32, then the
    1x128 quantisation through numpy and PyTorch's float8 cast"""
    M, K = A.shape
    I = Bg.shape[0] // 2
    Ad = TV[A] * np.repeat(sa.T.astype(np.float64), 128, axis=1)
    Bd = TV[Bg] * np.repeat(np.repeat(sbg.astype(np.float64), 128, axis=1), 128, axis=0)[:2 * I]
    h = Ad @ Bd.T
    g, u = h[:, :I], h[:, I:]
    with np.errstate(over="ignore"):  # e^-g overflows for very negative g: silu -> -0
        y = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    codes = np.empty((M, I), np.uint8)
    scales = np.empty((I // 128, M), np.float32)
    for b in range(I // 128):
        blk = y[:, b * 128:(b + 1) * 128]
        amax = np.abs(blk).max(axis=1)
        s = np.where(amax == 0, np.float32(1), (amax / np.float32(448)).astype(np.float32)).astype(np.float32)
        scales[b] = s
        q = np.abs((blk / s[:, None]).astype(np.float32))
        codes[:, b * 128:(b + 1) * 128] = torch_e4m3_bits(q) | np.where(np.signbit(blk), 0x80, 0).astype(np.uint8)
    return codes, scales


def test_swiglu_quant_matches_independent_chain():
    rng = np.random.default_rng(41)
    G, M, I, K = 2, 6, 256, 384
    A = rand_codes(rng, (M, K))
    sa = rng.uniform(0.01, 0.1, (K // 128, M)).astype(np.float32)
    B = rand_codes(rng, (G, 2 * I, K))
    sb = rng.uniform(0.01, 0.1, (G, 2 * I // 128, K // 128)).astype(np.float32)
    idx = np.array([0, 1, -1, 1, 0, 0], np.int32)
    codes = np.full((M, I), 0xAB, np.uint8)
    scales = np.full((I // 128, M), -7.0, np.float32)
    oracle.swiglu_quant("contiguous", A, sa, B, sb, idx, codes, scales)
    for m in range(M):
        if idx[m] < 0:  # padding row: untouched
            assert (codes[m] == 0xAB).all() and (scales[:, m] == -7.0).all()
            continue
        c, sc = independent_swiglu_quant(A[m:m + 1], sa[:, m:m + 1], B[idx[m]], sb[idx[m]])
        assert (codes[m] == c[0]).all() and (scales[:, m] == sc[:, 0]).all()


def test_swiglu_quant_masked_rows_and_zero_gate():
    rng = np.random.default_rng(42)
    G, M, I, K = 2, 5, 128, 256
    A = rand_codes(rng, (G, M, K))
    sa = rng.uniform(0.01, 0.1, (G, K // 128, M)).astype(np.float32)
    B = rand_codes(rng, (G, 2 * I, K))
    B[1, :I] = 0  # expert 1's gate rows are zero: silu(0) = 0 everywhere
    sb = rng.uniform(0.01, 0.1, (G, 2, K // 128)).astype(np.float32)
    mm = np.array([3, 9], np.int32)  # 9 is clamped to M
    codes = np.full((G, M, I), 0xAB, np.uint8)
    scales = np.full((G, I // 128, M), -7.0, np.float32)
    oracle.swiglu_quant("masked", A, sa, B, sb, mm, codes, scales)
    assert (codes[0, 3:] == 0xAB).all() and (scales[0, :, 3:] == -7.0).all()
    assert (codes[1] & 0x7F == 0).all() and (scales[1] == 1.0).all()  # y == 0: scale 1, zero codes
    c, sc = independent_swiglu_quant(A[0, :3], sa[0, :, :3], B[0], sb[0])
    assert (codes[0, :3] == c).all() and (scales[0, :, :3] == sc).all()


# ------------------------------------------------------------- BF16 GEMM ----


def rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 values will do


def bf16_exact_bits(A, B):
    """D = bf16(A B^T) by exact rationals (tiny sizes only)."""
    fa = [[Fraction(float(v)) for v in row] for row in bits_to_f32(A)]
    fb = [[Fraction(float(v)) for v in row] for row in bits_to_f32(B)]
    return np.array([[exact_bf16_bits(sum((x * y for x, y in zip(ra, rb)), Fraction(0)))
                      for rb in fb] for ra in fa], np.uint16).reshape(len(fa), len(fb))


@pytest.mark.parametrize("M,N,K,seed", [(3, 5, 64, 1), (2, 3, 7, 2), (4, 4, 130, 3)])
def test_bf16_gemm_exact_rational(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A, B = rand_bf16(rng, (M, K)), rand_bf16(rng, (N, K), 4.0)
    assert (oracle.gemm_bf16("dense", A, B) == bf16_exact_bits(A, B)).all()


def test_bf16_gemm_matches_numpy_float64_matmul():
    """a library matmul of the decoded values; products of bf16 values are
    exact in fp64 and these sums stay exact, so the bits agree"""
    rng = np.random.default_rng(11)
    A, B = rand_bf16(rng, (40, 256)), rand_bf16(rng, (24, 256))
    ref = bits_to_f32(A).astype(np.float64) @ bits_to_f32(B).astype(np.float64).T
    want = np.array([oracle.bf16_rne(v) for v in ref.ravel()], np.uint16).reshape(ref.shape)
    got, d64 = oracle.gemm_bf16("dense", A, B, want64=True)
    assert (got == want).all()
    assert np.array_equal(d64, ref)


def test_bf16_identity_and_zero_k():
    rng = np.random.default_rng(12)
    B = rand_bf16(rng, (6, 64))
    eye = np.zeros((64, 64), np.uint16)
    eye[np.arange(64), np.arange(64)] = 0x3F80  # 1.0
    assert (oracle.gemm_bf16("dense", eye, B) == B.T).all()  # bf16 values pass through exactly
    D = oracle.gemm_bf16("dense", np.zeros((3, 0), np.uint16), np.zeros((2, 0), np.uint16))
    assert (D == 0).all()


def test_bf16_grouped_rows():
    rng = np.random.default_rng(13)
    G, M, N, K = 3, 8, 5, 64
    A, B = rand_bf16(rng, (M, K)), rand_bf16(rng, (G, N, K))
    idx = np.array([0, 2, -1, 1, 7, 1, 0, -4], np.int32)
    D = oracle.gemm_bf16("contiguous", A, B, idx, out=np.full((M, N), 0x7FBF, np.uint16))
    for m, g in enumerate(idx):
        if 0 <= g < G:
            assert (D[m] == oracle.gemm_bf16("dense", A[m:m + 1], B[g])[0]).all()
        else:
            assert (D[m] == 0x7FBF).all()
    Am = rand_bf16(rng, (G, M, K))
    mm = np.array([8, 0, 30], np.int32)  # full, empty, clamped to M
    Dm = oracle.gemm_bf16("masked", Am, B, mm, out=np.full((G, M, N), 0x7FBF, np.uint16))
    assert (Dm[0] == oracle.gemm_bf16("dense", Am[0], B[0])).all()
    assert (Dm[1] == 0x7FBF).all()
    assert (Dm[2] == oracle.gemm_bf16("dense", Am[2], B[2])).all()


# ------------------------------------------------------ planted mistakes ----

MUTANTS = {
    1: "drops the last element of every K block",
    2: "uses the first K block's weight scale for every block",
    3: "reads the activation scales as [M][K/128]",
    4: "rounds to bf16 through binary32 (double rounding)",
    5: "computes padding rows of the contiguous layout with expert 0",
    6: "pairs output column n with weight row n^1",
    7: "rounds e4m3 ties towards the larger code",
    8: "quantises with scale amax / 447",
    9: "swaps the gate and up halves of the SwiGLU",
    10: "drops the last product of a BF16 dot product",
    11: "reads the BF16 weights as [K][N]",
}


def _pins_pass(lib):
    """A compact run of the pins above against one oracle build; returns the
    names of the pins that fail."""
    failed = []
    rng = np.random.default_rng(1)
    # whole-result brute force (exact rationals)
    M, N, K = 3, 4, 256
    A = rand_codes(rng, (M, K))
    B = rand_codes(rng, (N, K))
    sa = rng.uniform(0.01, 2, (K // 128, M)).astype(np.float32)
    sb = rng.uniform(0.01, 2, (1, K // 128)).astype(np.float32)
    if not (oracle.gemm(A, sa, B, sb, lib=lib) == exact_gemm_bits(A, sa, B, sb)).all():
        failed.append("exact_rational")
    # bf16 anchors
    if oracle.bf16_rne(1 + 2 ** -8 + 2 ** -50, lib=lib) != 0x3F81:
        failed.append("bf16_anchor")
    # contiguous padding untouched
    idx = np.array([0] * 100 + [-1] * 28, np.int32)
    A2, sa2 = synth.act(7, 128, 128)
    B2, sb2 = synth.grouped_weight(8, 1, 16, 128)
    D = oracle.grouped_contiguous(A2, sa2, B2, sb2, idx, np.full((128, 16), 0x7FBF, np.uint16),
                                  lib=lib)
    if not (D[100:] == 0x7FBF).all():
        failed.append("padding_untouched")
    # e4m3 tie: halfway between 1.0 (0x38) and 1.125 (0x39) goes to the even code
    if oracle.e4m3_encode(1.0625, lib=lib) != 0x38:
        failed.append("e4m3_tie")
    # quantiser scale: a block whose largest magnitude is 896 has scale exactly 2
    xb = np.zeros((1, 128), np.uint16)
    xb[0, 5] = np.uint16(0x4460)  # bf16 896.0
    codes, sa = oracle.quantize_1x128(xb, lib=lib)
    if sa[0, 0] != 2.0 or codes[0, 5] != 0x7E:
        failed.append("quantise_scale")
    # SwiGLU: one row, one block; against the independent chain
    A3 = rand_codes(rng, (1, 128))
    B3 = rand_codes(rng, (1, 256, 128))
    sa3 = np.full((1, 1), 0.05, np.float32)
    sb3 = np.full((1, 2, 1), 0.05, np.float32)
    c3 = np.zeros((1, 128), np.uint8)
    s3 = np.zeros((1, 1), np.float32)
    oracle.swiglu_quant("contiguous", A3, sa3, B3, sb3, np.zeros(1, np.int32), c3, s3, lib=lib)
    ci, si = independent_swiglu_quant(A3, sa3, B3[0], sb3[0])
    if not ((c3 == ci).all() and (s3 == si).all()):
        failed.append("swiglu")
    # BF16 GEMM: exact rationals on a tiny problem
    A4, B4 = rand_bf16(rng, (2, 6)), rand_bf16(rng, (3, 6))
    if not (oracle.gemm_bf16("dense", A4, B4, lib=lib) == bf16_exact_bits(A4, B4)).all():
        failed.append("bf16_exact")
    return failed


@pytest.fixture(scope="module")
def mutant_libs():
    d = tempfile.mkdtemp(prefix="fp8ref_mutants_")
    libs = {}
    for k in MUTANTS:
        out = os.path.join(d, f"libfp8ref_m{k}.so")
        subprocess.run(oracle.build_command(out=out, defines=[f"MUTANT={k}"]), check=True)
        libs[k] = oracle.load(out)
    return libs


def test_clean_oracle_passes_compact_pins():
    assert _pins_pass(oracle.load()) == []


@pytest.mark.parametrize("k", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant_libs, k):
    assert _pins_pass(mutant_libs[k]) != [], MUTANTS[k]
