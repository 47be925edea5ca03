"""Throughput of the FP8 block-scaled GEMM path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the hot path over one batch of the workload: one GEMM
call per shape of the workload, inputs already resident in HBM.  The default
workload is the decode-shaped dense set (M in {64, 128} x (N, K) in
{(2112,7168), (24576,1536), (7168,2048), (4096,7168)}), which is memory-bound:
`value` is algorithmic bytes moved per second (GB/s) over the timed steps,
counting A, B, the scales and D once per call.  Every step uses a different
copy of the inputs (rotating sets totalling > 1 GB) so weights come from HBM,
not from the 256 MB last-level cache.

Rank 0 prints one JSON line.  Extra fields: per-shape kernel times from HIP
events recorded around every launch in the timed region on the launch
stream, the roofline of the dominant shape's kernel, and the CPU oracle timed
on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOPS & % of FP8 MFMA peak (HBM GB/s for small M)"
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0  # dense FP8 MFMA, MI355X published figure
ROTATE_BYTES = 1 << 30


def dense_bytes(M, N, K):
    Kb, Nb = K // 128, (N + 127) // 128
    return M * K + N * K + 4 * M * Kb + 4 * Nb * Kb + 2 * M * N


def workload_shapes(name):
    from synth import workloads as W
    if name == "decode":
        return [("dense", M, N, K, False) for (M, N, K) in W.DECODE_SHAPES]
    if name == "prefill":
        return [("dense", M, N, K, True) for (M, N, K) in W.PREFILL_SHAPES]
    if name == "small":
        return [("dense",) + W.SMALL + (False,)]
    raise SystemExit(f"unknown workload {name}")


WORKLOAD_TEXT = {
    "decode": "dense decode-shaped FP8 GEMM, M in {64,128} x (N,K) in {(2112,7168),(24576,1536),(7168,2048),(4096,7168)}",
    "prefill": "dense prefill-shaped FP8 GEMM, M=4096 x (N,K) in {(7168,16384),(2112,7168),(24576,1536),(7168,18432)}, 1% rows x50",
    "small": "dense FP8 GEMM 128x256x512",
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU form "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_grouped_gemm_act_amd as fg
    from synth import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shapes = workload_shapes(args.workload)

    # inputs: one seeded set per shape, cloned on the GPU into rotating copies
    sets = []
    total = 0
    host = []
    for i, (_, M, N, K, heavy) in enumerate(shapes):
        d = W.dense(2000 + i if args.workload == "decode" else 3000 + i, M, N, K, heavy=heavy)
        host.append(d)
        t = {k: torch.from_numpy(d[k]).to(dev) for k in ("A", "sa", "B", "sb")}
        t["D"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        sets.append([t])
        total += dense_bytes(M, N, K)
    copies = max(1, min(64, -(-ROTATE_BYTES // total)))
    for s in sets:
        for _ in range(copies - 1):
            s.append({k: v.clone() for k, v in s[0].items()})
    torch.cuda.synchronize()

    def step(j, events=None):
        for i, s in enumerate(sets):
            t = s[j % copies]
            if events is not None:
                events[i][0].record()
            fg.gemm_fp8_1x128_128x128_bf16(t["A"], t["sa"], t["B"], t["sb"], t["D"])
            if events is not None:
                events[i][1].record()

    for j in range(args.warmup):
        step(j)
    torch.cuda.synchronize()

    # timed region: wall clock around exactly K steps; events on the launch
    # stream (torch's current stream, which the binding launches on)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)] for _ in shapes]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        step(j, [ev[i][j] for i in range(len(shapes))])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_shape = []
    for i, (_, M, N, K, _) in enumerate(shapes):
        ms = np.array([a.elapsed_time(b) for a, b in ev[i]])
        avg_s = float(ms.mean()) * 1e-3
        by, fl = dense_bytes(M, N, K), 2.0 * M * N * K
        per_shape.append({"M": M, "N": N, "K": K, "avg_us": avg_s * 1e6,
                          "median_us": float(np.median(ms)) * 1e3,
                          "GBps": by / avg_s / 1e9, "TFLOPS": fl / avg_s / 1e12,
                          "bytes": by, "flop": fl})
    dom = max(per_shape, key=lambda r: r["avg_us"])
    step_bytes = sum(r["bytes"] for r in per_shape)
    step_flop = sum(r["flop"] for r in per_shape)
    memory_bound = args.workload in ("decode", "small")
    gbps = step_bytes * args.steps / wall / 1e9
    tflops = step_flop * args.steps / wall / 1e12
    if memory_bound:
        roof = {"bound": "hbm", "achieved": dom["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": dom["GBps"] / PEAK_HBM_GBS, "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": dom["TFLOPS"], "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": dom["TFLOPS"] / PEAK_FP8_TFLOPS, "traffic": None}
    roof["kernel"] = f"dense {dom['M']}x{dom['N']}x{dom['K']}"
    roof["avg_us"] = dom["avg_us"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host, shapes, args.cpu_seconds, memory_bound)

    line = {
        "metric": METRIC,
        "value": gbps if memory_bound else tflops,
        "unit": "GB/s" if memory_bound else "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)", "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "shapes": len(shapes),
                   "rotating_copies": copies, "parallelism": "none (1 GPU)"},
        "tflops": tflops,
        "frac_fp8_peak": tflops / PEAK_FP8_TFLOPS,
        "gbps": gbps,
        "frac_hbm_peak": gbps / PEAK_HBM_GBS,
        "per_shape": per_shape,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(host, shapes, budget_s, memory_bound):
    """The oracle, as it stands, on whole outputs of the workload's shapes
    (in order) until about budget_s seconds of wall time have been spent."""
    import numpy as np

    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    done, by, fl = [], 0, 0.0
    for d, (_, M, N, K, _) in zip(host, shapes):
        if done and time.perf_counter() - t0 > budget_s:
            break
        # whole output rows, as many as the remaining budget allows at an
        # assumed 2e8 multiply-adds per second per thread
        left = max(0.5, budget_s - (time.perf_counter() - t0))
        rows = max(1, min(M, int(left * 2e8 * threads / (N * K))))
        A, sa = d["A"][:rows], np.ascontiguousarray(d["sa"][:, :rows])
        oracle.gemm(A, sa, d["B"], d["sb"], threads=threads)
        done.append(f"{rows}x{N}x{K}")
        by += dense_bytes(rows, N, K)  # algorithmic bytes of the computed slice
        fl += 2.0 * rows * N * K
    dt = time.perf_counter() - t0
    val = by / dt / 1e9 if memory_bound else fl / dt / 1e12
    return {"value": val, "unit": "GB/s" if memory_bound else "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": dt, "gflops": fl / dt / 1e9,
            "sample": "full outputs (all columns) of the first rows of each shape: " + ", ".join(done)}


if __name__ == "__main__":
    main()
