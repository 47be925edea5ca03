"""Launch status: each call reports the status of its own launches, not an
error that an earlier, unrelated HIP call left in the thread's last-error
slot (here a failed allocation made just before the call)."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_act_amd as fg
import synth
from synth import workloads as W
from parity_util import bits, sentinel_out, to_gpu

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def hip_runtime():
    """The HIP runtime the process has loaded (skip if there is not exactly one)."""
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    if len(paths) != 1:
        pytest.skip(f"HIP runtimes loaded: {sorted(paths)}")
    return ctypes.CDLL(paths.pop())


def test_earlier_hip_error_is_not_reported():
    torch.zeros(1, device="cuda")  # the runtime is loaded and initialised
    hip = hip_runtime()
    d = W.dense(8900, 64, 2112, 7168)  # decode: split-K planes and a reduction kernel
    A, sa, B, sb = (to_gpu(d[k]) for k in ("A", "sa", "B", "sb"))
    D = sentinel_out((64, 2112))
    t = W.dense(8901, 1100, 7400, 2048)  # large M: 261 tiles, the last 5 split over K
    tA, tsa, tB, tsb = (to_gpu(t[k]) for k in ("A", "sa", "B", "sb"))
    tD = sentinel_out((1100, 7400))
    X = torch.from_numpy(synth.normal(8902, 300 * 1024).reshape(300, 1024)).to(torch.bfloat16).cuda()
    QA = torch.empty((300, 1024), dtype=torch.uint8, device="cuda")
    Qs = torch.empty((8, 300), dtype=torch.float32, device="cuda")
    calls = [
        ("dense 64x2112x7168", lambda: fg.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, D), D),
        ("dense 1100x7400x2048", lambda: fg.gemm_fp8_1x128_128x128_bf16(tA, tsa, tB, tsb, tD), tD),
        ("quantize 300x1024", lambda: fg.quantize_fp8_1x128(X, QA, Qs), QA),
    ]
    ref = []
    for what, call, out in calls:  # eager first: the workspace exists before the failed allocation
        call()
        torch.cuda.synchronize()
        ref.append(bits(out) if out.dtype == torch.bfloat16 else out.cpu().numpy())
    for (what, call, out), r in zip(calls, ref):
        p = ctypes.c_void_p()
        assert hip.hipMalloc(ctypes.byref(p), ctypes.c_size_t(1 << 62)) != 0
        try:
            call()  # the binding raises on a non-zero status
        finally:
            hip.hipGetLastError()  # leave no error behind for the next torch launch
        torch.cuda.synchronize()
        got = bits(out) if out.dtype == torch.bfloat16 else out.cpu().numpy()
        assert np.array_equal(got, r), what
        announce(f"{what}: status OK after an unrelated failed allocation")
