"""Seeded random shapes through the GEMM entry points, the fused SwiGLU calls
and the quantiser, against the oracle: ragged M, N and K, group counts,
padding patterns, valid-row counts and size hints that the fixed cases do
not cover.  Each case draws its shape from its own seed (printed before the
call), so a failure names a reproducible case.  Tolerance and the
written-row rules are those of the fixed parity tests."""
import os
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_act_amd as fg
import oracle
import synth
from parity_util import SENTINEL, assert_close, bits, sentinel_out, to_gpu

pytestmark = pytest.mark.gpu
# cases per family (a longer sweep: FP8GEMM_RANDOM_CASES=n)
CASES = int(os.environ.get("FP8GEMM_RANDOM_CASES", "12"))
DENSE_M = (1, 2, 7, 33, 64, 65, 100, 128, 129, 200, 255, 300, 513)


def announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def rng(case, salt):
    return np.random.default_rng(90000 + 1000 * salt + case)


def contiguous_layout(r, G, blocks):
    """m_indices for `blocks` 128-row blocks: each block holds one expert's
    leading rows (the rest padding, -1 or an out-of-range index) or is all
    padding"""
    idx = np.full(128 * blocks, -1, np.int32)
    for b in range(blocks):
        if r.random() < 0.15:
            continue  # a whole padding block
        n = int(r.integers(1, 129))
        idx[128 * b:128 * b + n] = int(r.integers(0, G))
        if n < 128 and r.random() < 0.3:
            idx[128 * b + n] = G + int(r.integers(0, 3))  # out of range: padding
    return idx


def bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("case", range(CASES))
def test_random_dense(case):
    r = rng(case, 0)
    M, N, K = int(r.choice(DENSE_M)), int(r.integers(1, 900)), 128 * int(r.integers(1, 24))
    seed = 91000 + case
    announce(f"random dense case {case}: {M}x{N}x{K} seed {seed}")
    A, sa = synth.act(seed, M, K)
    B, sb = synth.weight(seed + 1, N, K)
    D = sentinel_out((M, N))
    fg.gemm_fp8_1x128_128x128_bf16(to_gpu(A), to_gpu(sa), to_gpu(B), to_gpu(sb), D)
    torch.cuda.synchronize()
    assert_close(bits(D), oracle.gemm(A, sa, B, sb), f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("case", range(CASES))
def test_random_contiguous(case):
    r = rng(case, 1)
    G, blocks = int(r.integers(1, 7)), int(r.integers(1, 12))
    N, K = int(r.integers(1, 700)), 128 * int(r.integers(1, 16))
    idx = contiguous_layout(r, G, blocks)
    M = idx.size
    seed = 92000 + case
    announce(f"random contiguous case {case}: G={G} {M}x{N}x{K} seed {seed}")
    A, sa = synth.act(seed, M, K)
    B, sb = synth.grouped_weight(seed + 1, G, N, K)
    D = sentinel_out((M, N))
    fg.grouped_contiguous(to_gpu(A), to_gpu(sa), to_gpu(B), to_gpu(sb), to_gpu(idx), D)
    torch.cuda.synchronize()
    got = bits(D)
    ref = oracle.grouped_contiguous(A, sa, B, sb, idx, np.full((M, N), SENTINEL, np.uint16))
    valid = (idx >= 0) & (idx < G)
    assert (got[~valid] == SENTINEL).all(), "a padding row was written"
    assert (got[valid] != SENTINEL).all(), "a valid row was not written"
    if valid.any():
        assert_close(got[valid], ref[valid], f"contiguous G={G} {M}x{N}x{K}")


@pytest.mark.parametrize("case", range(CASES))
def test_random_masked(case):
    r = rng(case, 2)
    G, M = int(r.integers(1, 9)), int(r.integers(1, 300))
    N, K = int(r.integers(1, 700)), 128 * int(r.integers(1, 60))  # past 4096 too
    mm = r.integers(-5, M + 6, size=G).astype(np.int32)
    expected_m = int(r.choice([0, 32, 64, 128, 300]))
    seed = 93000 + case
    announce(f"random masked case {case}: G={G} {M}x{N}x{K} expected_m={expected_m} seed {seed}")
    A, sa = synth.grouped_act(seed, G, M, K)
    B, sb = synth.grouped_weight(seed + 1, G, N, K)
    D = sentinel_out((G, M, N))
    fg.grouped_masked(to_gpu(A), to_gpu(sa), to_gpu(B), to_gpu(sb), to_gpu(mm), expected_m, D)
    torch.cuda.synchronize()
    got = bits(D)
    ref = oracle.grouped_masked(A, sa, B, sb, mm, np.full((G, M, N), SENTINEL, np.uint16))
    live = np.arange(M)[None, :] < np.clip(mm, 0, M)[:, None]
    assert (got[~live] == SENTINEL).all(), "a masked row was written"
    assert (got[live] != SENTINEL).all(), "a valid row was not written"
    if live.any():
        assert_close(got[live], ref[live], f"masked G={G} {M}x{N}x{K}")


@pytest.mark.parametrize("case", range(CASES))
def test_random_bf16(case):
    r = rng(case, 3)
    kind = ("dense", "contiguous", "masked")[case % 3]
    N, K = int(r.integers(1, 600)), 64 * int(r.integers(1, 30))
    seed = 94000 + case
    if kind == "dense":
        M = int(r.choice(DENSE_M))
        A = bf16_bits(synth.normal(seed, M * K).reshape(M, K))
        B = bf16_bits(synth.normal(seed + 1, N * K).reshape(N, K) * 0.5)
        announce(f"random bf16 dense case {case}: {M}x{N}x{K} seed {seed}")
        D = sentinel_out((M, N))
        fg.gemm_bf16_nt(bf16_dev(A), bf16_dev(B), D)
        torch.cuda.synchronize()
        assert_close(bits(D), oracle.gemm_bf16("dense", A, B), f"bf16 dense {M}x{N}x{K}")
    elif kind == "contiguous":
        G, blocks = int(r.integers(1, 6)), int(r.integers(1, 10))
        idx = contiguous_layout(r, G, blocks)
        M = idx.size
        A = bf16_bits(synth.normal(seed, M * K).reshape(M, K))
        B = bf16_bits(synth.normal(seed + 1, G * N * K).reshape(G, N, K) * 0.5)
        announce(f"random bf16 contiguous case {case}: G={G} {M}x{N}x{K} seed {seed}")
        D = sentinel_out((M, N))
        fg.grouped_contiguous_bf16(bf16_dev(A), bf16_dev(B), to_gpu(idx), D)
        torch.cuda.synchronize()
        got = bits(D)
        want = oracle.gemm_bf16("contiguous", A, B, idx, out=np.full((M, N), SENTINEL, np.uint16))
        valid = (idx >= 0) & (idx < G)
        assert (got[~valid] == SENTINEL).all() and (got[valid] != SENTINEL).all()
        if valid.any():
            assert_close(got[valid], want[valid], f"bf16 contiguous G={G} {M}x{N}x{K}")
    else:
        G, M = int(r.integers(1, 7)), int(r.integers(1, 260))
        mm = r.integers(-3, M + 4, size=G).astype(np.int32)
        expected_m = int(r.choice([0, 64, 256]))
        A = bf16_bits(synth.normal(seed, G * M * K).reshape(G, M, K))
        B = bf16_bits(synth.normal(seed + 1, G * N * K).reshape(G, N, K) * 0.5)
        announce(f"random bf16 masked case {case}: G={G} {M}x{N}x{K} seed {seed}")
        D = sentinel_out((G, M, N))
        fg.grouped_masked_bf16(bf16_dev(A), bf16_dev(B), to_gpu(mm), expected_m, D)
        torch.cuda.synchronize()
        got = bits(D)
        want = oracle.gemm_bf16("masked", A, B, mm, out=np.full((G, M, N), SENTINEL, np.uint16))
        live = np.arange(M)[None, :] < np.clip(mm, 0, M)[:, None]
        assert (got[~live] == SENTINEL).all() and (got[live] != SENTINEL).all()
        if live.any():
            assert_close(got[live], want[live], f"bf16 masked G={G} {M}x{N}x{K}")


@pytest.mark.parametrize("case", range(CASES))
def test_random_quantise(case):
    r = rng(case, 4)
    M, K = int(r.integers(1, 400)), 128 * int(r.integers(1, 40))
    seed = 95000 + case
    announce(f"random quantise case {case}: {M}x{K} seed {seed}")
    x = synth.normal(seed, M * K).reshape(M, K) * np.exp(synth.normal(seed + 1, M).reshape(M, 1) * 2)
    xb = bf16_bits(x)
    A, sa = fg.quantize_fp8_1x128(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_1x128(xb)
    assert (A.cpu().numpy() == codes).all()
    assert (sa.cpu().numpy().view(np.uint32) == scales.view(np.uint32)).all()


@pytest.mark.parametrize("case", range(CASES))
def test_random_swiglu(case):
    """the fused SwiGLU + 1x128 requantisation, contiguous and masked, under
    the SwiGLU tests' own bounds (scales, codes within half a step plus the
    fp32 error of h, at most 1% of codes differing)"""
    from test_gpu_swiglu import compare_contig, compare_masked, gpu_contig, gpu_masked
    r = rng(case, 5)
    I, K = 128 * int(r.integers(1, 5)), 128 * int(r.integers(1, 40))
    seed = 96000 + case
    if case % 2 == 0:
        G, blocks = int(r.integers(1, 6)), int(r.integers(1, 9))
        idx = contiguous_layout(r, G, blocks)
        M = idx.size
        announce(f"random swiglu contiguous case {case}: G={G} rows={M} I={I} K={K} seed {seed}")
        A, sa = synth.act(seed, M, K)
        B, sb = synth.grouped_weight(seed + 1, G, 2 * I, K)
        Yk, syk = gpu_contig(A, sa, B, sb, idx)
        compare_contig(A, sa, B, sb, idx, Yk, syk, f"swiglu contiguous G={G} I={I} K={K}")
    else:
        G, M = int(r.integers(1, 7)), int(r.integers(1, 260))
        mm = r.integers(-3, M + 4, size=G).astype(np.int32)
        expected_m = int(r.choice([0, 64, 256]))
        announce(f"random swiglu masked case {case}: G={G} M={M} I={I} K={K} seed {seed}")
        A, sa = synth.grouped_act(seed, G, M, K)
        B, sb = synth.grouped_weight(seed + 1, G, 2 * I, K)
        Yk, syk = gpu_masked(A, sa, B, sb, mm, expected_m)
        compare_masked(A, sa, B, sb, mm, Yk, syk, f"swiglu masked G={G} M={M} I={I} K={K}")
