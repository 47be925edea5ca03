"""The allocation-free dense entry point (fixed device scratch, nothing
allocated) against the regular dense entry point, through the C ABI: two
calls in a row, the second on a smaller input, each equal to the regular
call's output bit for bit and within the oracle tolerance; large-M calls with
a tail split; a plan past the scratch is rejected before any launch."""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_act_amd as fg
import oracle
from synth import workloads as W
from parity_util import assert_close, bits, sentinel_out, to_gpu

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def inputs(seed, M, N, K):
    d = W.dense(seed, M, N, K)
    return d, tuple(to_gpu(d[k]) for k in ("A", "sa", "B", "sb"))


def test_noalloc_two_calls_equal_the_regular_call():
    # 128x4096x7168: 4 K splits (8 MB of partials); then 64x2112x7168: 7 splits
    cases = [(9500, 128, 4096, 7168), (9501, 64, 2112, 7168)]
    prepared = [inputs(*c) for c in cases]
    outs = [sentinel_out((M, N)) for _, M, N, _ in cases]
    torch.cuda.synchronize()
    for (seed, M, N, K), (_, t), D in zip(cases, prepared, outs):
        announce(f"noalloc dense {M}x{N}x{K} seed {seed}")
        fg.gemm_fp8_1x128_128x128_bf16_noalloc(*t, D)  # back to back, no sync between
    torch.cuda.synchronize()
    for (seed, M, N, K), (d, t), D in zip(cases, prepared, outs):
        R = sentinel_out((M, N))
        fg.gemm_fp8_1x128_128x128_bf16(*t, R)
        torch.cuda.synchronize()
        got, ref = bits(D), bits(R)
        assert (got == ref).all(), f"{M}x{N}x{K}: differs from the regular call"
        assert_close(got, ref, f"noalloc {M}x{N}x{K} vs regular")
        assert_close(got, oracle.gemm(d["A"], d["sa"], d["B"], d["sb"]), f"noalloc {M}x{N}x{K} vs oracle")


def test_noalloc_large_m_tail_split():
    # 1100x7400x2048: the persistent walk with 5 tail tiles in 4 parts; then
    # a smaller 300x520x2048 whose 9 tiles are all split
    for seed, M, N, K in ((9510, 1100, 7400, 2048), (9511, 300, 520, 2048)):
        announce(f"noalloc dense {M}x{N}x{K} seed {seed}")
        d, t = inputs(seed, M, N, K)
        D, R = sentinel_out((M, N)), sentinel_out((M, N))
        fg.gemm_fp8_1x128_128x128_bf16_noalloc(*t, D)
        fg.gemm_fp8_1x128_128x128_bf16(*t, R)
        torch.cuda.synchronize()
        assert (bits(D) == bits(R)).all(), f"{M}x{N}x{K}: differs from the regular call"
        assert_close(bits(D), oracle.gemm(d["A"], d["sa"], d["B"], d["sb"]), f"noalloc {M}x{N}x{K}")


def test_noalloc_rejects_a_plan_past_the_scratch(monkeypatch):
    """a tuning override asking for 8 splits of 128x24576 partials (100 MB)
    is rejected before any launch; the regular call runs it unsplit"""
    M, N, K = 128, 24576, 2048
    d, t = inputs(9520, M, N, K)
    monkeypatch.setenv("FP8GEMM_DECODE", "64,4,15")
    D = sentinel_out((M, N))
    torch.cuda.synchronize()
    announce("noalloc plan past the scratch")
    with pytest.raises(fg.Fp8GemmError) as e:
        fg.gemm_fp8_1x128_128x128_bf16_noalloc(*t, D)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert (bits(D) == 0x7FBF).all(), "nothing may be written"
    fg.gemm_fp8_1x128_128x128_bf16(*t, D)
    torch.cuda.synchronize()
    assert_close(bits(D), oracle.gemm(d["A"], d["sa"], d["B"], d["sb"]), "regular call, override unsplit")


def test_noalloc_under_graph_capture():
    """The allocation-free call captured into a graph (no allocation during
    the capture): every replay, with eager calls of the same shape in
    between, equals the regular call's result bit for bit."""
    M, N, K = 128, 4096, 7168
    d, t = inputs(9530, M, N, K)
    R = sentinel_out((M, N))
    fg.gemm_fp8_1x128_128x128_bf16(*t, R)
    torch.cuda.synchronize()
    ref = bits(R)
    s = torch.cuda.Stream()
    D = sentinel_out((M, N))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    announce("noalloc under graph capture 128x4096x7168")
    with torch.cuda.graph(g, stream=s):
        fg.gemm_fp8_1x128_128x128_bf16_noalloc(*t, D)
    E = sentinel_out((M, N))
    for r in range(3):
        D.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        assert (bits(D) == ref).all(), f"replay {r}"
        fg.gemm_fp8_1x128_128x128_bf16_noalloc(*t, E)  # eager, ordered after the replay
        torch.cuda.synchronize()
        assert (bits(E) == ref).all()
