"""GPU parity of the BF16 GEMM without scales (dense, contiguous, masked)
against the oracle, on identical seeded inputs.

Tolerance as for the FP8 calls (parity_util): the kernel accumulates in
fp32 inside the MFMA, the oracle in fp64, and both round once to bf16.
Inputs of small integers make every fp32 intermediate exact, and then the
results must match bit for bit; which rows are written is always checked bit
for bit against a sentinel fill.
"""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_act_amd as fg
import oracle
import synth
from parity_util import SENTINEL, assert_close, bits

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rand_bf16(seed, shape, scale=1.0):
    return bf16_bits(synth.normal(seed, int(np.prod(shape))).reshape(shape) * scale)


def small_int_bf16(seed, shape):
    """values in {-2, ..., 2}: products and K <= 2^20 term sums are exact in fp32"""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.integers(-2, 3, size=shape).astype(np.float32))


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def sentinel(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def gpu_dense(A, B):
    D = sentinel((A.shape[0], B.shape[0]))
    fg.gemm_bf16_nt(dev(A), dev(B), D)
    torch.cuda.synchronize()
    return bits(D)


def gpu_contig(A, B, idx):
    D = sentinel((A.shape[0], B.shape[1]))
    fg.grouped_contiguous_bf16(dev(A), dev(B), torch.from_numpy(idx).cuda(), D)
    torch.cuda.synchronize()
    return bits(D)


def gpu_masked(A, B, mm, expected_m):
    D = sentinel((A.shape[0], A.shape[1], B.shape[1]))
    fg.grouped_masked_bf16(dev(A), dev(B), torch.from_numpy(mm).cuda(), expected_m, D)
    torch.cuda.synchronize()
    return bits(D)


# ------------------------------------------------------------------ dense ----


@pytest.mark.parametrize("M,N,K", [
    (128, 256, 512),     # a few tiles
    (200, 300, 320),     # ragged in M and N, K not a multiple of 128
    (1, 130, 64),        # one row, one K block
    (64, 2112, 7168),    # decode shape: K split over workgroups
    (128, 4096, 1536),   # decode shape, 128 rows
    (300, 520, 2048),    # large-M kernel with ragged tiles
])
def test_dense_full(M, N, K):
    seed = 11000 + M + N + K
    announce(f"bf16 dense {M}x{N}x{K} seed {seed}")
    A, B = rand_bf16(seed, (M, K)), rand_bf16(seed + 1, (N, K), 0.5)
    assert_close(gpu_dense(A, B), oracle.gemm_bf16("dense", A, B), f"bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (256, 384, 1024), (96, 200, 512)])
def test_dense_exact_small_integers(M, N, K):
    announce(f"bf16 dense exact {M}x{N}x{K}")
    A, B = small_int_bf16(1, (M, K)), small_int_bf16(2, (N, K))
    got, want = gpu_dense(A, B), oracle.gemm_bf16("dense", A, B)
    assert (got == want).all(), f"{(got != want).sum()} elements differ"


@pytest.mark.parametrize("cfg", ["96,4,1", "32,4,2", "128,4,1,8"])
@pytest.mark.parametrize("M,N,K", [(64, 300, 512), (128, 2112, 640)])
def test_dense_decode_variants(M, N, K, cfg, monkeypatch):
    """BF16 decode instances beyond the defaults (tuning override)."""
    monkeypatch.setenv("FP8GEMM_DECODE", cfg)
    seed = 11600 + M + N
    announce(f"bf16 decode {cfg} {M}x{N}x{K}")
    A, B = rand_bf16(seed, (M, K)), rand_bf16(seed + 1, (N, K), 0.5)
    assert_close(gpu_dense(A, B), oracle.gemm_bf16("dense", A, B), f"bf16 decode {cfg}")


def test_dense_k_zero_and_empty():
    announce("bf16 dense K=0")
    D = gpu_dense(np.zeros((130, 0), np.uint16), np.zeros((70, 0), np.uint16))
    assert (D == 0).all()
    E = torch.empty((0, 5), dtype=torch.bfloat16, device="cuda")
    fg.gemm_bf16_nt(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                    torch.empty((5, 64), dtype=torch.bfloat16, device="cuda"), E)


def test_grouped_k_zero():
    """K = 0 in both grouped layouts: valid rows are empty sums (zero), the
    others keep their sentinel"""
    G, N = 3, 130
    idx = np.full(128 * 2, -1, np.int32)
    idx[:90] = 2
    idx[128:200] = 0
    idx[200:210] = 5  # out of range
    announce("bf16 contiguous K=0")
    got = gpu_contig(np.zeros((idx.size, 0), np.uint16), np.zeros((G, N, 0), np.uint16), idx)
    valid = (idx >= 0) & (idx < G)
    assert (got[valid] == 0).all() and (got[~valid] == SENTINEL).all()
    mm = np.array([0, 77, 300], np.int32)
    M = 130
    announce("bf16 masked K=0")
    got = gpu_masked(np.zeros((G, M, 0), np.uint16), np.zeros((G, N, 0), np.uint16), mm, 64)
    live = np.arange(M)[None, :] < np.clip(mm, 0, M)[:, None]
    assert (got[live] == 0).all() and (got[~live] == SENTINEL).all()


def test_dense_prefill_shape_full():
    M, N, K = 4096, 2112, 7168
    announce(f"bf16 dense {M}x{N}x{K}")
    A, B = rand_bf16(11100, (M, K)), rand_bf16(11101, (N, K), 0.5)
    D = gpu_dense(A, B)
    from parity_util import assert_close_full
    assert_close_full(D, oracle.gemm_bf16("dense", A, B), "bf16 prefill")


@pytest.mark.parametrize("walk", ["default", "0"])
def test_dense_persistent_walk(walk, monkeypatch):
    """9 x 30 = 270 tiles of 128 x 256: the persistent walk, with a tail split
    of the last 14 tiles, and one workgroup per tile."""
    if walk != "default":
        monkeypatch.setenv("FP8GEMM_WALK", walk)
    M, N, K = 2304, 3840, 512
    announce(f"bf16 walk {walk} dense {M}x{N}x{K}")
    A, B = rand_bf16(11050, (M, K)), rand_bf16(11051, (N, K), 0.5)
    assert_close(gpu_dense(A, B), oracle.gemm_bf16("dense", A, B), f"bf16 walk {walk}")


@pytest.mark.parametrize("walk", ["default", "0"])
def test_contiguous_persistent_walk(walk, monkeypatch):
    if walk != "default":
        monkeypatch.setenv("FP8GEMM_WALK", walk)
    G, rows, N, K = 4, 128 * 18, 4096, 256  # 18 x 16 = 288 tiles
    announce(f"bf16 walk {walk} contiguous G={G} rows={rows}")
    idx, _ = synth.contiguous_indices(11070, G, rows, False)
    A, B = rand_bf16(11071, (rows, K)), rand_bf16(11072, (G, N, K), 0.5)
    got = gpu_contig(A, B, idx)
    want = oracle.gemm_bf16("contiguous", A, B, idx, out=np.full((rows, N), SENTINEL, np.uint16))
    live = (idx >= 0) & (idx < G)
    assert (got[~live] == SENTINEL).all(), "a padding row was written"
    assert_close(got[live], want[live], f"bf16 walk {walk} contiguous")


# ------------------------------------------------------------- grouped ----


@pytest.mark.parametrize("G,rows,N,K,uniform", [(3, 768, 384, 512, False), (4, 1024, 256, 1024, True)])
def test_contiguous_full(G, rows, N, K, uniform):
    seed = 11200 + G
    announce(f"bf16 contiguous G={G} rows={rows} N={N} K={K}")
    idx, _ = synth.contiguous_indices(seed + 3, G, rows, uniform)
    idx = idx.copy()
    idx[5:9] = G + 3  # out-of-range indices: rows not written
    A, B = rand_bf16(seed, (rows, K)), rand_bf16(seed + 1, (G, N, K), 0.5)
    got = gpu_contig(A, B, idx)
    want = oracle.gemm_bf16("contiguous", A, B, idx, out=np.full((rows, N), SENTINEL, np.uint16))
    live = (idx >= 0) & (idx < G)
    assert (got[~live] == SENTINEL).all(), "a padding row was written"
    assert_close(got[live], want[live], "bf16 contiguous")


@pytest.mark.parametrize("G,M,N,K,mm", [
    (4, 192, 256, 384, [0, 192, 77, 500]),
    (3, 320, 130, 640, [-3, 1, 300]),
])
def test_masked_full(G, M, N, K, mm):
    seed = 11300 + G + M
    mm = np.array(mm, np.int32)
    A, B = rand_bf16(seed, (G, M, K)), rand_bf16(seed + 1, (G, N, K), 0.5)
    want = oracle.gemm_bf16("masked", A, B, mm, out=np.full((G, M, N), SENTINEL, np.uint16))
    valid = np.clip(mm, 0, M)
    live = np.arange(M)[None, :] < valid[:, None]
    for expected_m in (0, 64, M):  # the hint never changes the result
        announce(f"bf16 masked G={G} M={M} N={N} K={K} expected_m={expected_m}")
        got = gpu_masked(A, B, mm, expected_m)
        assert (got[~live] == SENTINEL).all(), "a masked row was written"
        assert_close(got[live], want[live], f"bf16 masked expected_m={expected_m}")


def test_masked_exact_small_integers():
    G, M, N, K = 2, 256, 512, 1024
    announce("bf16 masked exact")
    mm = np.array([256, 131], np.int32)
    A, B = small_int_bf16(5, (G, M, K)), small_int_bf16(6, (G, N, K))
    got = gpu_masked(A, B, mm, 128)
    want = oracle.gemm_bf16("masked", A, B, mm, out=np.full((G, M, N), SENTINEL, np.uint16))
    assert (got == want).all()
