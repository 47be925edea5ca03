"""HIP-graph capture of every entry point beyond the dense GEMM (whose
split-K replay is tested with the parity cases): each graph is replayed
several times, with the output cleared and eager launches of the same call
in between, and every replay must equal the eager result bit for bit (all
kernels are deterministic: no atomics, fixed summation order)."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_act_amd as fg
import synth
from synth import workloads as W
from parity_util import to_gpu

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def hip_runtime():
    """The HIP runtime the process has loaded (skip if there is not exactly one)."""
    torch.zeros(1, device="cuda")
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    if len(paths) != 1:
        pytest.skip(f"HIP runtimes loaded: {sorted(paths)}")
    lib = ctypes.CDLL(paths.pop())
    for fn in (lib.hipStreamCreate, lib.hipStreamSynchronize, lib.hipStreamDestroy):
        fn.restype = ctypes.c_int
    lib.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    return lib


def replay_equals_eager(what, call, outs):
    """call() launches on the current stream into `outs`; returns after
    checking three replays of its captured graph against the eager result."""
    s = torch.cuda.Stream()
    for o in outs:
        o.zero_()  # rows a call does not write (padding, masked) must compare equal too
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        call()
    s.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for r in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"{what}: replay {r} differs"
        with torch.cuda.stream(s):
            call()  # eager work between replays
        s.synchronize()
    announce(f"{what}: 3 replays equal the eager result")


def test_graph_quantize():
    M, K = 300, 1024
    x = synth.normal(8800, M * K).reshape(M, K)
    X = torch.from_numpy(x).to(torch.bfloat16).cuda()
    A = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
    replay_equals_eager("quantize 300x1024", lambda: fg.quantize_fp8_1x128(X, A, sa), [A, sa])


def test_graph_masked_fp8():
    d = W.masked(8810, 4, 192, 512, 1024)
    A, sa, B, sb = (to_gpu(d[k]) for k in ("A", "sa", "B", "sb"))
    mm = to_gpu(d["masked_m"])
    D = torch.empty((4, 192, 512), dtype=torch.bfloat16, device="cuda")
    replay_equals_eager("masked 4x192x512x1024",
                        lambda: fg.grouped_masked(A, sa, B, sb, mm, 96, D), [D])


def test_graph_masked_fp8_walk():
    """K > 4096: the masked call walks its live tiles (256-row activation
    tiles, expert offsets built from masked_m on the device) by default"""
    d = W.masked(8812, 5, 256, 384, 4352)
    d["masked_m"] = np.array([256, 0, 129, 7, 300], np.int32)
    A, sa, B, sb = (to_gpu(d[k]) for k in ("A", "sa", "B", "sb"))
    mm = to_gpu(d["masked_m"])
    D = torch.empty((5, 256, 384), dtype=torch.bfloat16, device="cuda")
    replay_equals_eager("masked walk 5x256x384x4352",
                        lambda: fg.grouped_masked(A, sa, B, sb, mm, 128, D), [D])


def test_graph_swiglu_contiguous_and_masked():
    G, rows, I, K = 3, 768, 256, 1024
    idx, _ = synth.contiguous_indices(8823, G, rows, False)
    A, sa = synth.act(8820, rows, K)
    B, sb = synth.grouped_weight(8821, G, 2 * I, K)
    tA, tsa, tB, tsb, tidx = to_gpu(A), to_gpu(sa), to_gpu(B), to_gpu(sb), to_gpu(idx)
    Y = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    sy = torch.empty((I // 128, rows), dtype=torch.float32, device="cuda")
    replay_equals_eager("contiguous swiglu 768x512x1024",
                        lambda: fg.grouped_contiguous_swiglu_fp8(tA, tsa, tB, tsb, tidx, Y, sy), [Y, sy])
    Am, sam = synth.grouped_act(8830, G, 192, K)
    mm = to_gpu(np.array([192, 5, 0], np.int32))
    tAm, tsam = to_gpu(Am), to_gpu(sam)
    Ym = torch.empty((G, 192, I), dtype=torch.uint8, device="cuda")
    sym = torch.empty((G, I // 128, 192), dtype=torch.float32, device="cuda")
    replay_equals_eager("masked swiglu 3x192x512x1024",
                        lambda: fg.grouped_masked_swiglu_fp8(tAm, tsam, tB, tsb, mm, 64, Ym, sym), [Ym, sym])


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (300, 520, 640)])
def test_graph_bf16_dense(M, N, K):
    """the first shape takes the split-K decode path (workspace + reduction)"""
    a = torch.from_numpy(synth.normal(8840, M * K).reshape(M, K)).to(torch.bfloat16).cuda()
    b = torch.from_numpy(synth.normal(8841, N * K).reshape(N, K)).to(torch.bfloat16).cuda()
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    replay_equals_eager(f"bf16 {M}x{N}x{K}", lambda: fg.gemm_bf16_nt(a, b, D), [D])


def test_capture_takes_its_own_workspace():
    """A split-K shape captured on a fresh stream before any eager call: the
    capture takes a workspace of its own (allocated during the capture), so
    every replay, with eager calls of the same shape in between, equals the
    eager result bit for bit and matches the oracle."""
    import oracle
    from parity_util import assert_close, bits, sentinel_out
    M, N, K = 64, 2112, 7168
    d = W.dense(8850, M, N, K)
    A, sa, B, sb = (to_gpu(d[k]) for k in ("A", "sa", "B", "sb"))
    s = torch.cuda.Stream()
    D = sentinel_out((M, N))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fg.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, D)
    De = sentinel_out((M, N))
    fg.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, De)
    torch.cuda.synchronize()
    eager = bits(De)
    for r in range(3):
        D.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        assert (bits(D) == eager).all(), f"replay {r}"
        fg.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, De)
        torch.cuda.synchronize()
    assert_close(eager, oracle.gemm(d["A"], d["sa"], d["B"], d["sb"]), "captured first")
    announce("capture before any eager call: own workspace, replays equal eager and oracle")


def test_graph_replay_beside_eager_calls_on_another_stream():
    """A graph of split calls (decode planes and a large-M tail split)
    captured on stream A is replayed on stream B while eager split calls run
    on stream A, with no synchronisation between them: both results equal
    the same calls made one at a time."""
    from parity_util import bits, sentinel_out
    shapes = [(128, 4096, 7168, 8880), (1100, 7400, 2048, 8881), (64, 2112, 7168, 8882),
              (300, 520, 2048, 8883)]
    ins = []
    for M, N, K, seed in shapes:
        d = W.dense(seed, M, N, K)
        ins.append(((to_gpu(d["A"]), to_gpu(d["sa"]), to_gpu(d["B"]), to_gpu(d["sb"])), (M, N)))
    ref = []
    for args, mn in ins:
        D = sentinel_out(mn)
        fg.gemm_fp8_1x128_128x128_bf16(*args, D)
        torch.cuda.synchronize()
        ref.append(bits(D))
    sa_, sb_ = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [sentinel_out(mn) for _, mn in ins]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=sa_):  # the graph: shapes 0 and 1
        for (args, _), D in zip(ins[:2], outs[:2]):
            fg.gemm_fp8_1x128_128x128_bf16(*args, D)
    for o in outs:
        o.zero_()
    torch.cuda.synchronize()
    announce("graph on stream B beside eager split calls on stream A")
    for _ in range(6):
        with torch.cuda.stream(sb_):
            g.replay()
        with torch.cuda.stream(sa_):  # eager: shapes 2 and 3
            for (args, _), D in zip(ins[2:], outs[2:]):
                fg.gemm_fp8_1x128_128x128_bf16(*args, D)
    torch.cuda.synchronize()
    for i, (D, r) in enumerate(zip(outs, ref)):
        assert (bits(D) == r).all(), f"shape {shapes[i][:3]} differs from its serial result"


def test_workspace_memory_flat():
    """Split calls on 100 HIP streams, each created, used and destroyed in
    turn (free device memory falls by under 8 MB: no workspace per stream),
    and 12 graphs of a split call captured, replayed and destroyed in turn
    (under 32 MB: destroyed graphs give their workspace back)."""
    import gc
    import time
    from parity_util import sentinel_out
    M, N, K = 128, 2112, 7168
    d = W.dense(8890, M, N, K)
    A, sa, B, sb = (to_gpu(d[k]) for k in ("A", "sa", "B", "sb"))
    D = sentinel_out((M, N))
    fg.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, D)  # the device's eager workspace exists
    torch.cuda.synchronize()
    hip = hip_runtime()

    def stream_cycle():
        """a HIP stream created, used for a split call and destroyed"""
        h = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(h)) == 0
        s = torch.cuda.ExternalStream(h.value)
        fg.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, D, stream=s)
        assert hip.hipStreamSynchronize(h) == 0
        assert hip.hipStreamDestroy(h) == 0

    stream_cycle()  # the runtime's own first-use costs
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(100):
        stream_cycle()
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free0 - free1 <= (8 << 20), f"100 streams: free memory fell by {(free0 - free1) >> 20} MB"
    s = torch.cuda.Stream()
    for i in range(12):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fg.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, D)
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        del g
        gc.collect()
        torch.cuda.synchronize()
        time.sleep(0.02)  # the graph's release callback may run on a runtime thread
        if i == 0:
            free2 = torch.cuda.mem_get_info()[0]
    free3 = torch.cuda.mem_get_info()[0]
    assert free2 - free3 <= (32 << 20), f"11 more graphs: free memory fell by {(free2 - free3) >> 20} MB"
    announce(f"memory: streams {(free0 - free1) >> 20} MB, graphs {(free2 - free3) >> 20} MB")


def test_two_streams_split_k_concurrently():
    """Split-K calls on two streams interleaved with no synchronisation: the
    device's one eager workspace orders them on the GPU, so both results equal
    the same calls made one after the other."""
    from parity_util import bits, sentinel_out
    shapes = [(64, 2112, 7168, 8860), (128, 4096, 7168, 8861)]
    ins = []
    for M, N, K, seed in shapes:
        d = W.dense(seed, M, N, K)
        ins.append(((to_gpu(d["A"]), to_gpu(d["sa"]), to_gpu(d["B"]), to_gpu(d["sb"])), (M, N)))
    ref = []
    for (A, sa, B, sb), (M, N) in ins:
        D = sentinel_out((M, N))
        fg.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, D)
        torch.cuda.synchronize()
        ref.append(bits(D))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [sentinel_out(mn) for _, mn in ins]
    torch.cuda.synchronize()
    for _ in range(5):  # interleave launches on the two streams
        for (args, _), s, D in zip(ins, streams, outs):
            with torch.cuda.stream(s):
                fg.gemm_fp8_1x128_128x128_bf16(*args, D)
    torch.cuda.synchronize()
    for D, r in zip(outs, ref):
        assert (bits(D) == r).all()
    announce("two streams: split-K results equal the serial ones")


def test_host_threads_share_the_workspace():
    """Four host threads, each with its own stream, call split-K decode and
    tail-split large-M GEMMs at once (the binding releases the GIL in the
    library call): the device workspace's lease serialises them on the GPU,
    and every result equals the same call made alone."""
    import threading
    from parity_util import bits, sentinel_out
    shapes = [(64, 2112, 7168, 8880), (128, 4096, 7168, 8881), (1100, 7400, 2048, 8882)]
    ins, ref = [], []
    for M, N, K, seed in shapes:
        d = W.dense(seed, M, N, K)
        args = (to_gpu(d["A"]), to_gpu(d["sa"]), to_gpu(d["B"]), to_gpu(d["sb"]))
        D = sentinel_out((M, N))
        fg.gemm_fp8_1x128_128x128_bf16(*args, D)
        torch.cuda.synchronize()
        ins.append((args, (M, N)))
        ref.append(bits(D))
    nthreads, rounds = 4, 6
    streams = [torch.cuda.Stream() for _ in range(nthreads)]
    outs = [[sentinel_out(mn) for _, mn in ins] for _ in range(nthreads)]
    torch.cuda.synchronize()
    errors = []

    def work(t):
        try:
            with torch.cuda.stream(streams[t]):
                for r in range(rounds):
                    for i in range(len(ins)):
                        k = (i + t + r) % len(ins)  # threads start on different calls
                        fg.gemm_fp8_1x128_128x128_bf16(*ins[k][0], outs[t][k])
        except Exception as e:  # reported in the main thread
            errors.append(repr(e))

    announce(f"{nthreads} host threads, {rounds} rounds of {len(ins)} calls each")
    threads = [threading.Thread(target=work, args=(t,)) for t in range(nthreads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(nthreads):
        for k in range(len(ins)):
            assert (bits(outs[t][k]) == ref[k]).all(), f"thread {t}, call {k}"


def test_graph_persistent_walk_calls():
    """The persistent walk under capture: a dense call with a tail split
    (its partials in the capture's own workspace), a contiguous call and
    a contiguous SwiGLU call, each with more tiles than CUs."""
    d = W.dense(8870, 1100, 7400, 2048)  # 261 tiles: 256 whole + 5 split in 4
    A, sa, B, sb = (to_gpu(d[k]) for k in ("A", "sa", "B", "sb"))
    D = torch.empty((1100, 7400), dtype=torch.bfloat16, device="cuda")
    replay_equals_eager("walk dense 1100x7400x2048", lambda: fg.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, D), [D])
    c = W.contiguous(8871, 5, 128 * 20, 4352, 256, uniform=False)  # 20 x 17 tiles
    cA, csa, cB, csb, cidx = (to_gpu(c[k]) for k in ("A", "sa", "B", "sb", "m_indices"))
    Dc = torch.empty((c["M"], c["N"]), dtype=torch.bfloat16, device="cuda")
    replay_equals_eager("walk contiguous 2560x4352x256",
                        lambda: fg.grouped_contiguous(cA, csa, cB, csb, cidx, Dc), [Dc])
    G, rows, I, K = 4, 128 * 20, 2048, 256  # 20 x 16 tiles
    idx, _ = synth.contiguous_indices(8873, G, rows, False)
    sA, ssa = synth.act(8874, rows, K)
    sB, ssb = synth.grouped_weight(8875, G, 2 * I, K)
    tA, tsa, tB, tsb, tidx = to_gpu(sA), to_gpu(ssa), to_gpu(sB), to_gpu(ssb), to_gpu(idx)
    Y = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    sy = torch.empty((I // 128, rows), dtype=torch.float32, device="cuda")
    replay_equals_eager("walk contiguous swiglu 2560x4096x256",
                        lambda: fg.grouped_contiguous_swiglu_fp8(tA, tsa, tB, tsb, tidx, Y, sy), [Y, sy])
