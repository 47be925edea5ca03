"""Build libfp8gemm.so in-tree with hipcc for gfx950 (ahead of time; no JIT)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("fp8gemm.hip", "quant.hip")]
LIB = os.path.join(HERE, "libfp8gemm.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the AMDGPU register-pressure trackers in the machine scheduler: 1% on the
    # contiguous MoE calls (32768 x 4096 x 7168), the other workloads level
    "-mllvm", "-amdgpu-use-amdgpu-trackers",
    "-Wall", "-Wno-unused-command-line-argument",
]


def command(out=LIB, extra=()):
    return ["hipcc", *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-o", out, *SRCS]


def build(out=LIB, extra=()):
    tmp = out + ".tmp"
    subprocess.run(command(tmp, extra), check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
