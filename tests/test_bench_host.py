"""Host-side pieces of the benchmark (no GPU): the one-GPU guard, the
algorithmic byte and FLOP counts the roofline divides by, and how the
profile summarizer groups library dispatches into calls."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_dense_bytes_counts_each_operand_once():
    # 64 x 2112 x 7168: A, B, the 1x128 activation scales, the 128x128
    # weight scales (17 row blocks, N = 2112 is ragged) and the bf16 output
    M, N, K = 64, 2112, 7168
    Kb, Nb = 56, 17
    want = M * K + N * K + 4 * M * Kb + 4 * Nb * Kb + 2 * M * N
    assert bench.dense_bytes(M, N, K) == want == 15_886_048


def test_grouped_cost_counts_valid_rows_and_live_experts():
    N, K = 4096, 7168
    flop, by = bench.grouped_cost([0, 128, 5, 0], N, K)
    rows, live, Kb, Nb = 133, 2, 56, 32
    assert flop == 2.0 * rows * N * K
    assert by == rows * K + 4 * rows * Kb + live * (N * K + 4 * Nb * Kb) + 2 * rows * N


def _row(name, disp):
    return {"Kernel_Name": name, "Dispatch_Id": disp}


def test_launch_grouping_attaches_reductions_to_their_tile_kernel():
    rows = [
        _row("void (anonymous namespace)::tile_kernel<1, 4, 4, 1, 4, 4, true, false, 0, false>(Args)", 1),
        _row("(anonymous namespace)::splitk_reduce_kernel(float const*, unsigned short*, int, int, int)", 2),
        _row("void (anonymous namespace)::walk_kernel<4, 2, 4, 4, 3, 4, 0, false>(Args)", 3),
        _row("void (anonymous namespace)::tail_reduce_kernel<128, 256>(float const*, ...)", 4),
        _row("void (anonymous namespace)::tile_kernel<4, 2, 4, 4, 3, 4, false, false, 1, false>(Args)", 5),
        _row("(anonymous namespace)::quant_kernel(unsigned short const*, ...)", 6),
    ]
    groups = bench._launches(rows)
    assert [[r["Dispatch_Id"] for r in g] for g in groups] == [[1, 2], [3, 4], [5], [6]]
    assert all(bench._ours(r["Kernel_Name"]) for r in rows)
    assert not bench._ours("void at::native::vectorized_elementwise_kernel<4, ...>")


def test_workload_calls_cover_the_configured_shapes():
    from synth import workloads as W
    dec = bench.workload_calls("small")
    assert [c.label for c in dec] == ["dense 128x256x512"]
    assert dec[0].bytes == bench.dense_bytes(*W.SMALL) and dec[0].flop == 2.0 * 128 * 256 * 512
    assert set(bench.WORKLOAD_TEXT) >= {"decode", "prefill", "contiguous", "masked", "quant",
                                         "swiglu", "bf16", "small"}
    assert bench.MEMORY_BOUND == {"decode", "small", "masked", "quant"}


def test_dispatch_order_maps_calls_and_timed_replays():
    """The summarizer's reading of the bench's launch order: eager pass over
    the rotation copies, warm-up and timed step replays (all calls in order),
    then per call (reps + 1) graph replays of `copies` launches, the first
    untimed; only those timed per-call replays count for the profile's
    duration."""
    line = {"per_call": [{}, {}], "config": {"rotating_copies": 3}, "warmup": 2, "steps": 20}
    nc, copies, reps = 2, 3, 5  # reps = max(3, min(50, 20 // 4))
    head = nc * (copies + 2 + 20)
    n = head + nc * (reps + 1) * copies
    calls = bench._call_of_dispatches(n, line)
    timed = bench._timed_per_call(n, line)
    assert calls[:head] == [i % nc for i in range(head)]
    assert not any(timed[:head])
    for c in range(nc):
        block = range(head + c * (reps + 1) * copies, head + (c + 1) * (reps + 1) * copies)
        assert all(calls[i] == c for i in block)
        flags = [timed[i] for i in block]
        assert flags == [False] * copies + [True] * (reps * copies)
