"""Throughput of the FP8 block-scaled GEMM path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the hot path over one batch of the workload: one GEMM
call per shape of the workload, inputs already resident in HBM, launched as a
HIP graph replay.  With no --workload, the headline is the largest workload,
the MoE grouped GEMM in the M-axis contiguous layout (G=4 experts x 8192 rows
and G=8 uneven experts, 32768 rows, N=4096, K=7168), which is MFMA-bound:
`value` is algorithmic FLOP per second (TFLOP/s) over the K timed steps.  The
same line then carries, under `per_config`, the other workloads timed the same
way in the same run: decode (M in {64,128}, HBM-bound, GB/s), prefill (M=4096,
TFLOP/s) and masked (G=16, HBM-bound, GB/s).  Every step uses a different copy
of the inputs where one copy is under 1 GB (rotating sets totalling > 1 GB) so
weights come from HBM, not from the 256 MB last-level cache.

Rank 0 prints one JSON line.  Extra fields: per-shape kernel times (HIP
events on the launch stream around back-to-back graph replays of that
shape's kernel), the roofline of the dominant shape's kernel (with the
committed rocprofv3 trace's mean duration of the same call beside it), and
the CPU oracle timed on a bounded sample of the same workload on every host
core.
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
PEAK_BF16_TFLOPS = 2500.0  # dense BF16 MFMA, MI355X published figure
ROTATE_BYTES = 1 << 30


def dense_bytes(M, N, K):
    Kb, Nb = K // 128, (N + 127) // 128
    return M * K + N * K + 4 * M * Kb + 4 * Nb * Kb + 2 * M * N


def grouped_cost(rows_per_group, N, K):
    """Algorithmic FLOP and bytes of a grouped call: only valid rows, and the
    weights of experts that have at least one row."""
    Kb, Nb = K // 128, (N + 127) // 128
    rows = sum(rows_per_group)
    live = sum(1 for r in rows_per_group if r > 0)
    flop = 2.0 * rows * N * K
    by = rows * K + 4 * rows * Kb + live * (N * K + 4 * Nb * Kb) + 2 * rows * N
    return flop, by


class Call:
    """One GEMM call of a workload: seeded host inputs, device copies, cost."""

    def __init__(self, kind, d, label, flop, by):
        self.kind, self.d, self.label, self.flop, self.bytes = kind, d, label, flop, by

    def to_device(self, torch, dev):
        if self.kind == "bf16":
            t = {k: torch.from_numpy(self.d[k].view("int16")).view(torch.bfloat16).to(dev) for k in ("A", "B")}
            t["D"] = torch.empty((self.d["M"], self.d["N"]), dtype=torch.bfloat16, device=dev)
            return t
        if self.kind == "quant":
            X = torch.from_numpy(self.d["X"].view("int16")).view(torch.bfloat16).to(dev)
            M, K = self.d["M"], self.d["K"]
            return {"X": X, "A": torch.empty((M, K), dtype=torch.uint8, device=dev),
                    "sa": torch.empty((K // 128, M), dtype=torch.float32, device=dev)}
        base = self.kind.replace("_swiglu", "")
        keys = ["A", "sa", "B", "sb"] + (["m_indices"] if base == "contiguous" else []) \
            + (["masked_m"] if base == "masked" else [])
        t = {k: torch.from_numpy(self.d[k]).to(dev) for k in keys}
        lead = (self.d["G"],) if base == "masked" else ()
        M, N = self.d["M"], self.d["N"]
        if self.kind.endswith("_swiglu"):
            t["Y"] = torch.empty((*lead, M, N // 2), dtype=torch.uint8, device=dev)
            t["sy"] = torch.empty((*lead, N // 256, M), dtype=torch.float32, device=dev)
        else:
            t["D"] = torch.empty((*lead, M, N), dtype=torch.bfloat16, device=dev)
        return t

    def launch(self, fg, t):
        if self.kind == "bf16":
            fg.gemm_bf16_nt(t["A"], t["B"], t["D"])
        elif self.kind == "quant":
            fg.quantize_fp8_1x128(t["X"], t["A"], t["sa"])
        elif self.kind == "dense":
            fg.gemm_fp8_1x128_128x128_bf16(t["A"], t["sa"], t["B"], t["sb"], t["D"])
        elif self.kind == "contiguous":
            fg.grouped_contiguous(t["A"], t["sa"], t["B"], t["sb"], t["m_indices"], t["D"])
        elif self.kind == "contiguous_swiglu":
            fg.grouped_contiguous_swiglu_fp8(t["A"], t["sa"], t["B"], t["sb"], t["m_indices"],
                                             t["Y"], t["sy"])
        elif self.kind == "masked_swiglu":
            fg.grouped_masked_swiglu_fp8(t["A"], t["sa"], t["B"], t["sb"], t["masked_m"],
                                         self.d["expected_m"], t["Y"], t["sy"])
        else:
            fg.grouped_masked(t["A"], t["sa"], t["B"], t["sb"], t["masked_m"], self.d["expected_m"], t["D"])


def workload_calls(name):
    import numpy as np
    from synth import workloads as W
    calls = []
    if name in ("decode", "prefill", "small"):
        shapes = {"decode": W.DECODE_SHAPES, "prefill": W.PREFILL_SHAPES, "small": (W.SMALL,)}[name]
        for i, (M, N, K) in enumerate(shapes):
            seed = {"decode": 2000, "prefill": 3000, "small": 1000}[name] + i
            d = W.dense(seed, M, N, K, heavy=name == "prefill")
            calls.append(Call("dense", d, f"dense {M}x{N}x{K}", 2.0 * M * N * K, dense_bytes(M, N, K)))
    elif name == "contiguous":
        for i, (G, rows, N, K, uniform) in enumerate(W.CONTIG_CASES):
            d = W.contiguous(4000 + i, G, rows, N, K, uniform)
            counts = np.bincount(d["m_indices"][d["m_indices"] >= 0], minlength=G)
            flop, by = grouped_cost(counts.tolist(), N, K)
            calls.append(Call("contiguous", d, f"contiguous G={G} {rows}x{N}x{K}", flop, by + 4 * rows))
    elif name == "quant":
        import torch
        import synth
        for i, (M, N, K) in enumerate(W.PREFILL_SHAPES):
            x = synth.normal(6000 + i, M * K).reshape(M, K)
            x[synth.heavy_rows(6007 + i, M) > 1] *= 50
            xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            d = {"X": xb, "M": M, "K": K}
            calls.append(Call("quant", d, f"quantize {M}x{K}", 0.0, 3 * M * K + 4 * M * (K // 128)))
    elif name == "bf16":
        import torch
        import synth
        for i, (M, N, K) in enumerate(W.PREFILL_SHAPES):
            def b16(seed, shape, scale):
                x = synth.normal(seed, shape[0] * shape[1]).reshape(shape) * scale
                return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            d = {"A": b16(7000 + 10 * i, (M, K), 1.0), "B": b16(7001 + 10 * i, (N, K), 0.5),
                 "M": M, "N": N, "K": K}
            calls.append(Call("bf16", d, f"bf16 {M}x{N}x{K}", 2.0 * M * N * K, 2 * (M * K + N * K + M * N)))
    elif name == "swiglu":
        # the experts' gate/up projection (N = 2I = 4096, K = 7168) with the
        # SwiGLU and 1x128 requantisation fused: codes [rows, I] and scales
        # [I/128, rows] are written instead of a bf16 D
        for i, (G, rows, N, K, uniform) in enumerate(W.CONTIG_CASES):
            d = W.contiguous(4000 + i, G, rows, N, K, uniform)
            counts = np.bincount(d["m_indices"][d["m_indices"] >= 0], minlength=G)
            flop, by = grouped_cost(counts.tolist(), N, K)
            by += int(counts.sum()) * (N // 2 + 4 * (N // 256) - 2 * N) + 4 * rows
            calls.append(Call("contiguous_swiglu", d, f"contiguous+swiglu G={G} {rows}x{N}x{K}", flop, by))
        G, M, N, K = W.MASKED_CASES[0]
        d = W.masked(5000, G, M, N, K)
        live = np.clip(d["masked_m"], 0, M)
        flop, by = grouped_cost(live.tolist(), N, K)
        by += int(live.sum()) * (N // 2 + 4 * (N // 256) - 2 * N) + 4 * G
        calls.append(Call("masked_swiglu", d, f"masked+swiglu G={G} {M}x{N}x{K}", flop, by))
    elif name == "masked":
        for i, (G, M, N, K) in enumerate(W.MASKED_CASES):
            d = W.masked(5000 + i, G, M, N, K)
            flop, by = grouped_cost(np.clip(d["masked_m"], 0, M).tolist(), N, K)
            calls.append(Call("masked", d, f"masked G={G} {M}x{N}x{K}", flop, by + 4 * G))
    else:
        raise SystemExit(f"unknown workload {name}")
    return calls


WORKLOAD_TEXT = {
    "decode": "dense decode-shaped FP8 GEMM, M in {64,128} x (N,K) in {(2112,7168),(24576,1536),(7168,2048),(4096,7168)}",
    "prefill": "dense prefill-shaped FP8 GEMM, M=4096 x (N,K) in {(7168,16384),(2112,7168),(24576,1536),(7168,18432)}, 1% rows x50",
    "small": "dense FP8 GEMM 128x256x512",
    "contiguous": "MoE grouped FP8 GEMM, M-axis contiguous: G=4 x 8192 rows and G=8 uneven (32768 padded rows), N=4096, K=7168",
    "masked": "MoE grouped FP8 GEMM, masked: G=16, 256 rows/expert, masked_m ~ U[0,256], (N,K) in {(4096,7168),(7168,2048)}",
    "swiglu": "MoE gate/up projection with SwiGLU and 1x128 FP8 requantisation fused: contiguous G=4 x 8192 rows and G=8 uneven (32768 padded rows), masked G=16 x 256 rows; N=2I=4096, K=7168",
    "bf16": "dense BF16 GEMM without scales (fp32 accumulate, bf16 out), M=4096 x (N,K) in {(7168,16384),(2112,7168),(24576,1536),(7168,18432)}",
    "quant": "1x128 FP8 quantisation of bf16 activations, M=4096 x K in {16384,7168,1536,18432} (the prefill A operands), 1% rows x50",
}
MEMORY_BOUND = {"decode", "small", "masked", "quant"}
DEFAULT_WORKLOAD = "contiguous"  # the largest configuration: the headline
EXTRA_WORKLOADS = ("decode", "prefill", "masked")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOAD_TEXT),
                    help=f"time this workload only (default: {DEFAULT_WORKLOAD}, with "
                         + ", ".join(EXTRA_WORKLOADS) + " under per_config)")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="with the default workload, skip the per_config workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the GEMM: copy a MIB-sized buffer 5 times (a plain copy "
                         "kernel of known size, used to calibrate rocprofv3 byte counters)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="no GPU: turn the rocprofv3 outputs of the profiling commands (see "
                         "profile_commands) under DIR into profiles/<workload>.md and "
                         "profiles/<workload>.traffic.json")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload or DEFAULT_WORKLOAD)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU form "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)
        return

    import moe_grouped_gemm_act_amd as fg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    workload = args.workload or DEFAULT_WORKLOAD
    head = measure(torch, fg, workload, args.steps, args.warmup, dev, stream)
    per_config = None
    if args.workload is None and not args.no_extra_configs:
        per_config = {}
        for w in EXTRA_WORKLOADS:
            r = measure(torch, fg, w, args.steps, args.warmup, dev, stream)
            per_config[w] = {k: r[k] for k in ("workload", "value", "unit", "ms_per_step", "frac",
                                               "rotating_copies", "per_call", "roofline")}
    calls = head.pop("calls")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(calls, args.cpu_seconds, head["memory_bound"])

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (fp32 accumulate)" if workload == "bf16" else "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[workload], "calls": len(head["per_call"]),
                   "rotating_copies": head["rotating_copies"], "parallelism": "none (1 GPU)"},
        "tflops": head["tflops"],
        "frac_fp8_peak": head["tflops"] / PEAK_FP8_TFLOPS,
        "frac_mfma_peak": head["tflops"] / (PEAK_BF16_TFLOPS if workload == "bf16" else PEAK_FP8_TFLOPS),
        "gbps": head["gbps"],
        "frac_hbm_peak": head["gbps"] / PEAK_HBM_GBS,
        "per_call": head["per_call"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
    }
    if per_config is not None:
        line["per_config"] = per_config
    print(json.dumps(line), flush=True)


def measure(torch, fg, workload, steps, warmup, dev, stream):
    """Time one workload: W warm-up and K timed graph replays of its step,
    then each call on its own; returns the figures (and the calls)."""
    calls = workload_calls(workload)

    # inputs: one seeded set per call, cloned on the GPU into rotating copies
    sets, total = [], 0
    for c in calls:
        sets.append([c.to_device(torch, dev)])
        total += c.bytes
    copies = max(1, min(64, -(-ROTATE_BYTES // total)))
    for s_ in sets:
        for _ in range(copies - 1):
            s_.append({k: v.clone() for k, v in s_[0].items()})
    torch.cuda.synchronize()

    def launch(i, j):
        calls[i].launch(fg, sets[i][j % copies])

    # Steps run as HIP graph replays (one graph per rotation set, all calls in
    # order), so the timed region measures the GPU, not Python launch cost.
    with torch.cuda.stream(stream):
        for j in range(copies):  # eager pass first (any library set-up happens outside capture)
            for i in range(len(calls)):
                launch(i, j)
    stream.synchronize()
    step_graphs = []
    for j in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(len(calls)):
                launch(i, j)
        step_graphs.append(g)
    with torch.cuda.stream(stream):
        for j in range(warmup):
            step_graphs[j % copies].replay()
    stream.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for j in range(steps):
            step_graphs[j % copies].replay()
    stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-call kernel duration: HIP events on the launch stream around
    # back-to-back replays of a graph holding `copies` launches of that call
    per_call = []
    reps = max(3, min(50, steps // 4))
    for i, c in enumerate(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(copies):
                launch(i, j)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            g.replay()
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
        stream.synchronize()
        avg_s = a.elapsed_time(b) * 1e-3 / (reps * copies)
        per_call.append({"call": c.label, "avg_us": avg_s * 1e6, "GBps": c.bytes / avg_s / 1e9,
                         "TFLOPS": c.flop / avg_s / 1e12, "bytes": c.bytes, "flop": c.flop})
        del g
    del step_graphs, sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    dom = max(per_call, key=lambda r: r["avg_us"])
    step_bytes = sum(c.bytes for c in calls)
    step_flop = sum(c.flop for c in calls)
    memory_bound = workload in MEMORY_BOUND
    gbps = step_bytes * steps / wall / 1e9
    tflops = step_flop * steps / wall / 1e12
    if memory_bound:
        roof = {"bound": "hbm", "achieved": dom["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": dom["GBps"] / PEAK_HBM_GBS, "traffic": None}
    else:
        peak = PEAK_BF16_TFLOPS if workload == "bf16" else PEAK_FP8_TFLOPS
        roof = {"bound": "mfma", "achieved": dom["TFLOPS"], "peak": peak,
                "unit": "TFLOP/s", "frac": dom["TFLOPS"] / peak, "traffic": None}
    roof["kernel"] = dom["call"]
    roof["avg_us"] = dom["avg_us"]
    prof = profiled_call(dom["call"])
    roof["traffic"] = prof and prof["traffic"]
    if prof and prof.get("trace_avg_us"):
        # the committed rocprofv3 kernel trace of the same call (same kernel
        # sources): its mean duration and the fraction it gives
        t = prof["trace_avg_us"] * 1e-6
        units = dom["bytes"] / 1e9 if memory_bound else dom["flop"] / 1e12
        roof["profile"] = {"source": prof["source"], "trace_avg_us": prof["trace_avg_us"],
                           "frac": units / t / roof["peak"],
                           "live_over_trace": dom["avg_us"] / prof["trace_avg_us"],
                           # the clock the call ran at in the profiled run (SQ busy cycles
                           # per shader array over the traced duration) and its MFMA busy
                           # fraction per cycle
                           "sclk_ghz": prof.get("sclk_ghz"), "mfma_busy": prof.get("mfma_busy")}
    value = gbps if memory_bound else tflops
    return {"workload": WORKLOAD_TEXT[workload], "value": value,
            "unit": "GB/s" if memory_bound else "TFLOP/s", "ms_per_step": wall / steps * 1e3,
            "frac": value / (PEAK_HBM_GBS if memory_bound else roof["peak"]),
            "tflops": tflops, "gbps": gbps, "rotating_copies": copies, "per_call": per_call,
            "roofline": roof, "memory_bound": memory_bound, "calls": calls}


def source_sha256():
    """sha256 over what the library's code is made from: the kernel sources
    (csrc/*.hip then csrc/*.h, in name order), then the build script with its
    compiler flags."""
    import glob
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "moe_grouped_gemm_act_amd")
    csrc = os.path.join(pkg, "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        h.update(open(f, "rb").read())
    h.update(open(os.path.join(pkg, "build.py"), "rb").read())
    return h.hexdigest()


def profile_commands(workload, out="gpurun_out/prof"):
    """The rocprofv3 runs a profile summary is built from (run from the
    repository root after `cd /tmp && export TMPDIR=/tmp`)."""
    w = workload
    b = f"python3 bench.py --workload {w} --no-cpu-baseline"
    return [
        ("kt", f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/{w}/kt -o {w} -- {b} --steps 20 --warmup 5"),
        ("fetch", f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/{w}/fetch -o {w} -- {b} --steps 2 --warmup 1"),
        ("write", f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/{w}/write -o {w} -- {b} --steps 2 --warmup 1"),
        ("sq", f"rocprofv3 --pmc SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT --output-format csv -d {out}/{w}/sq -o {w} -- {b} --steps 2 --warmup 1"),
        ("cfetch", f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/copy/fetch -o copy -- python3 bench.py --copy-probe 1024"),
        ("cwrite", f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/copy/write -o copy -- python3 bench.py --copy-probe 1024"),
    ]


_PRIMARY = ("tile_kernel", "walk_kernel", "gemm_kernel", "quant_kernel")
_FOLLOWER = ("splitk_reduce_kernel", "tail_reduce_kernel")  # run right after their call's tile kernel


def _ours(name):
    return any(k in name for k in _PRIMARY + _FOLLOWER)


def _launches(rows):
    """Group library dispatches (in dispatch order) into call launches: each
    primary kernel plus the split-K reduction that follows it, if any."""
    out = []
    for r in rows:
        if any(k in r["Kernel_Name"] for k in _FOLLOWER) and out:
            out[-1].append(r)
        else:
            out.append([r])
    return out


def _call_of_dispatches(n, line):
    """Map the i-th library dispatch of a bench run to its call index, from the
    bench's fixed launch order: eager pass over every rotation copy, warm-up
    and timed graph replays (all calls in order), then per call (reps + 1)
    replays of a graph holding `copies` launches of that call."""
    nc, copies = len(line["per_call"]), line["config"]["rotating_copies"]
    reps = max(3, min(50, line["steps"] // 4))
    head = nc * (copies + line["warmup"] + line["steps"])
    tail = nc * (reps + 1) * copies
    if n != head + tail:
        raise SystemExit(f"profile has {n} library dispatches, bench order implies {head + tail}")
    return [i % nc if i < head else (i - head) // ((reps + 1) * copies) for i in range(n)]


def _timed_per_call(n, line):
    """For each library dispatch of a bench run (the order of
    _call_of_dispatches): whether it belongs to the timed replays of the
    per-call phase, the launches the bench's own per-call figure covers (not
    the first replay of each call's graph, nor the step replays, which
    include the clock's settling after start-up)."""
    nc, copies = len(line["per_call"]), line["config"]["rotating_copies"]
    reps = max(3, min(50, line["steps"] // 4))
    head = nc * (copies + line["warmup"] + line["steps"])
    return [i >= head and (i - head) % ((reps + 1) * copies) >= copies for i in range(n)]


def _last_json(path):
    for ln in reversed(open(path).read().splitlines()):
        if ln.startswith("{"):
            return json.loads(ln)
    raise SystemExit(f"no JSON line in {path}")


def summarize_profile(d, workload):
    import csv
    import glob
    import statistics as st
    w = workload
    sha = source_sha256()

    def rows(pattern):
        f = glob.glob(os.path.join(d, pattern))
        if len(f) != 1:
            raise SystemExit(f"expected one file for {pattern}, found {f}")
        return list(csv.DictReader(open(f[0])))

    kt = _launches(sorted((r for r in rows(f"{w}/kt/*kernel_trace.csv") if _ours(r["Kernel_Name"])),
                          key=lambda r: int(r["Dispatch_Id"])))
    kline = _last_json(os.path.join(d, w, "kt.log"))
    kcall = _call_of_dispatches(len(kt), kline)
    ktimed = _timed_per_call(len(kt), kline)
    labels = [c["call"] for c in kline["per_call"]]

    def counter(sub):
        rs = _launches(sorted((r for r in rows(f"{w}/{sub}/*counter_collection.csv")
                               if _ours(r["Kernel_Name"])), key=lambda r: int(r["Dispatch_Id"])))
        line = _last_json(os.path.join(d, w, f"{sub}.log"))
        cc = _call_of_dispatches(len(rs), line)
        out = {}
        for grp, c in zip(rs, cc):
            out.setdefault(c, []).append(sum(float(r["Counter_Value"]) for r in grp) * 1024)
        return out

    def copy_scale(sub, name):
        rs = [r for r in rows(f"copy/{sub}/*counter_collection.csv") if "copyBuffer" in r["Kernel_Name"]]
        kib = st.mean(float(r["Counter_Value"]) for r in rs)
        return (1 << 30) / (kib * 1024), kib

    def sq_counters():
        """per call: mean over launches of each SQ counter (summed over the
        launch's kernels), from the multi-counter pass; None if not taken"""
        if not glob.glob(os.path.join(d, w, "sq", "*counter_collection.csv")):
            return None
        by_disp = {}
        for r in rows(f"{w}/sq/*counter_collection.csv"):
            if _ours(r["Kernel_Name"]):
                e = by_disp.setdefault(int(r["Dispatch_Id"]), {"Kernel_Name": r["Kernel_Name"]})
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        grps = _launches([by_disp[k] for k in sorted(by_disp)])
        cc = _call_of_dispatches(len(grps), _last_json(os.path.join(d, w, "sq.log")))
        out = {}
        for grp, c in zip(grps, cc):
            tot = {}
            for e in grp:
                for k, v in e.items():
                    if k != "Kernel_Name":
                        tot[k] = tot.get(k, 0.0) + v
            out.setdefault(c, []).append(tot)
        return {c: {k: st.mean(t[k] for t in v) for k in v[0]} for c, v in out.items()}

    fscale, fkib = copy_scale("fetch", "FETCH_SIZE")
    wscale, wkib = copy_scale("write", "WRITE_SIZE")
    fetch, write = counter("fetch"), counter("write")
    sq = sq_counters()
    sq_table = []
    if sq:
        agent = [r for r in rows(f"{w}/sq/*agent_info.csv") if int(r.get("Simd_Count") or 0) > 0][0]
        n_simd, n_arr = int(agent["Simd_Count"]), int(agent["Array_Count"])
    table, traffic = [], {}
    import re
    for i, lab in enumerate(labels):
        grps = [g for g, c in zip(kt, kcall) if c == i]
        # a launch's time: its kernels' durations (a split call's reduction included)
        def dur(g):
            return sum((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000 for r in g)
        durs = [dur(g) for g in grps]
        # the launches the bench's per-call figure times, traced
        timed = [dur(g) for g, c, t in zip(kt, kcall, ktimed) if c == i and t]
        r0 = grps[0][0]
        names = []
        for r in grps[0]:
            m = re.search(r"(tile_kernel|walk_kernel|gemm_kernel|tail_reduce_kernel)<[^>]*>|splitk_reduce_kernel|quant_kernel", r["Kernel_Name"])
            names.append(m.group(0) if m else r["Kernel_Name"])
        name = " + ".join(names)
        grid = (int(r0["Grid_Size_X"]) // int(r0["Workgroup_Size_X"]), int(r0["Grid_Size_Y"]))
        fb = st.mean(fetch[i]) * fscale
        wb = st.mean(write[i]) * wscale
        alg = kline["per_call"][i]["bytes"]
        traffic[lab] = {"fetch_bytes": fb, "write_bytes": wb, "trace_avg_us": st.mean(timed),
                        "trace_all_avg_us": st.mean(durs)}
        if sq and i in sq:
            q = sq[i]
            busy = q["SQ_BUSY_CYCLES"] / n_arr  # per shader array: the launch's cycles
            traffic[lab]["sclk_ghz"] = busy / (st.mean(durs) * 1e3)
            traffic[lab]["mfma_busy"] = q["SQ_VALU_MFMA_BUSY_CYCLES"] / n_simd / busy
            sq_table.append(f"| {lab} | {q['SQ_VALU_MFMA_BUSY_CYCLES'] / n_simd / busy:.3f} | "
                            f"{q['SQ_LDS_BANK_CONFLICT'] / max(q['SQ_LDS_IDX_ACTIVE'], 1):.3f} | "
                            f"{busy / (st.mean(durs) * 1e3):.2f} |")
        table.append(f"| {lab} | `{name}` | {grid[0]},{grid[1]} | {len(durs)} | {st.mean(durs):.2f} | "
                     f"{st.median(durs):.2f} | {min(durs):.2f} | {st.mean(timed):.2f} | "
                     f"{kline['per_call'][i]['avg_us']:.2f} | "
                     f"{fb / 1e6:.2f} | {wb / 1e6:.2f} | {alg / 1e6:.2f} | {(fb + wb) / alg:.2f} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    cmds = "\n".join(f"    {c}" for _, c in profile_commands(w))
    md = f"""# rocprofv3: {w} workload

Workload: {WORKLOAD_TEXT[w]}; seeded synthetic inputs, {kline['config']['rotating_copies']} rotating
input copies (> 1 GB) so the weights come from HBM.  Library sha256 `{sha}`
(moe_grouped_gemm_act_amd/csrc/*.hip, then *.h, in name order, then build.py with its flags).

Commands (repository root, one MI355X, after `cd /tmp && export TMPDIR=/tmp`), then
`python3 bench.py --workload {w} --summarize-profile gpurun_out/prof` to write this file:

{cmds}

Per call: kernel trace durations (all launches of that call in the traced bench run; a
split-K or tail-split call's launch is its tile kernel plus the reduction kernel, durations added);
"timed avg us": the mean over the traced launches that the bench's per-call figure times (its
graph replays after the first, past the start-up phase in which the clock settles), the
duration `bench.py` quotes beside its live figure; the bench's own HIP-event average for the
same call in that run (launch gaps included, and stretched by the tracer); and HBM bytes per
launch from the two counter runs, scaled by the copy calibration below; grid is the first
kernel's.  "ratio" = measured HBM bytes / algorithmic bytes (A, B, scales and D once each).

| call | kernel | grid (x,y) | launches | avg us | median us | min us | timed avg us | bench avg us | FETCH (MB) | WRITE (MB) | algorithmic (MB) | ratio |
|---|---|---|---|---|---|---|---|---|---|---|---|---|
""" + "\n".join(table) + f"""

Calibration: a 1 GiB device copy (`__amd_rocclr_copyBuffer`) reads FETCH_SIZE {fkib:.0f} KiB and
WRITE_SIZE {wkib:.0f} KiB per dispatch: scale factors {fscale:.3f} (fetch) and {wscale:.3f} (write).
"""
    if sq_table:
        md += f"""
SQ counters (the `sq` pass, means over launches).  "MFMA busy" =
SQ_VALU_MFMA_BUSY_CYCLES / {n_simd} SIMDs over SQ_BUSY_CYCLES / {n_arr} shader arrays (the
launch's own cycles); "LDS conflicts" = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; "GHz" = those
busy cycles over the traced mean duration (the clock the launch ran at, approximately).

| call | MFMA busy | LDS conflicts | GHz |
|---|---|---|---|
""" + "\n".join(sq_table) + "\n"
    open(os.path.join(ROOT, "profiles", f"{w}.md"), "w").write(md)
    json.dump({"source_sha256": sha, "fetch_scale": fscale, "write_scale": wscale, "kernels": traffic},
              open(os.path.join(ROOT, "profiles", f"{w}.traffic.json"), "w"), indent=1)
    print(md)


def profiled_call(kernel):
    """From the committed profile summaries, for the call `kernel`, only when
    they were taken on the kernel sources as they are now (else None): HBM
    bytes per launch (calibrated rocprofv3 FETCH_SIZE + WRITE_SIZE) and the
    kernel trace's mean launch duration."""
    import glob
    sha = source_sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.traffic.json"))):
        d = json.load(open(f))
        k = d.get("kernels", {}).get(kernel)
        if d.get("source_sha256") == sha and k:
            return {"traffic": {"bytes": k["fetch_bytes"] + k["write_bytes"], "fetch_bytes": k["fetch_bytes"],
                                "write_bytes": k["write_bytes"], "source": os.path.basename(f)},
                    "trace_avg_us": k.get("trace_avg_us"), "source": os.path.basename(f),
                    "sclk_ghz": k.get("sclk_ghz"), "mfma_busy": k.get("mfma_busy")}
    return None


def host_cpu():
    """The host's cores this process may run on, and the CPU model."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    quota = None
    try:  # cgroup v2 CPU quota, if one is set
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()
        if q != "max":
            quota = int(q) / int(per)
    except (OSError, ValueError):
        pass
    return cores, model, quota


def cpu_baseline(calls, budget_s, memory_bound):
    """The oracle, as it stands, on whole output rows of the workload's dense
    calls (in order, repeated) until about budget_s seconds of wall time have
    been spent; grouped calls are sampled as dense GEMMs of one expert."""
    import numpy as np

    import oracle
    cores, model, quota = host_cpu()
    threads = max(1, min(256, cores))  # every core this process may use (the oracle's cap is 256)
    granted = min(threads, quota) if quota else threads
    t0 = time.perf_counter()
    done, by, fl, passes = [], 0, 0.0, 0
    while True:
        for c in calls:
            d = c.d
            if c.kind == "quant":
                M, K = d["X"].shape
                left = max(0.2, budget_s - (time.perf_counter() - t0))
                rows = max(1, min(M, int(left * 2e6 / K)))  # the oracle encodes ~2e6 values/s
                oracle.quantize_1x128(np.ascontiguousarray(d["X"][:rows]))
                if passes == 0:
                    done.append(f"quantize {rows}x{K}")
                by += 3 * rows * K + 4 * rows * (K // 128)
                if time.perf_counter() - t0 > budget_s:
                    break
                continue
            if c.kind == "bf16":
                A, B = d["A"], d["B"]
                M, K = A.shape
                N = B.shape[0]
                left = max(0.2, budget_s - (time.perf_counter() - t0))
                rows = max(1, min(M, int(left * 3e8 * granted / (N * K))))
                oracle.gemm_bf16("dense", A[:rows], B, threads=threads)
                if passes == 0:
                    done.append(f"{rows}x{N}x{K}")
                by += 2 * (rows * K + N * K + rows * N)
                fl += 2.0 * rows * N * K
                if time.perf_counter() - t0 > budget_s:
                    break
                continue
            A, sa, B, sb = d["A"], d["sa"], d["B"], d["sb"]
            if c.kind.startswith("masked"):
                A, sa = A[0], sa[0]
            if c.kind != "dense":
                B, sb = B[0], sb[0]
            M, K = A.shape
            N = B.shape[0]
            # whole output rows, as many as the remaining budget allows at an
            # assumed 1e9 multiply-adds per second per core actually granted
            left = max(0.2, budget_s - (time.perf_counter() - t0))
            rows = max(1, min(M, int(left * 1e9 * granted / (N * K))))
            sa_r = np.ascontiguousarray(sa[:, :rows])
            if c.kind.endswith("_swiglu"):  # one expert's rows through the fused oracle
                I = N // 2
                oracle.swiglu_quant("contiguous", A[:rows], sa_r, B[None], sb[None],
                                    np.zeros(rows, np.int32), np.empty((rows, I), np.uint8),
                                    np.empty((I // 128, rows), np.float32), threads=threads)
                by += rows * K + 4 * rows * (K // 128) + N * K + 4 * (N // 128) * (K // 128) \
                    + rows * I + 4 * rows * (I // 128)
            else:
                oracle.gemm(A[:rows], sa_r, B, sb, threads=threads)
                by += dense_bytes(rows, N, K)  # algorithmic bytes of the computed slice
            if passes == 0:
                done.append(f"{rows}x{N}x{K}")
            fl += 2.0 * rows * N * K
            if time.perf_counter() - t0 > budget_s:
                break
        passes += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    val = by / dt / 1e9 if memory_bound else fl / dt / 1e12
    # the oracle's GEMM runs on `threads` host threads, its quantiser on one
    used = 1 if all(c.kind == "quant" for c in calls) else threads
    return {"value": val, "unit": "GB/s" if memory_bound else "TFLOP/s", "cores": used,
            "kind": "oracle", "seconds": dt, "gflops": fl / dt / 1e9,
            "host": {"cores_available": cores, "cpu_model": model, "cgroup_cpu_quota": quota},
            "sample": f"{passes} pass(es) over whole output rows of each call (first pass: "
                      + ", ".join(done) + f"), stopped after about {budget_s:.0f} s"}


if __name__ == "__main__":
    main()
