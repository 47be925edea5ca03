"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the oracle and the seeded generator built from their sources with gcc, and
the HIP library's host side (argument validation, which runs before any HIP
call) built with the sanitizers on its host pass only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")


def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    subprocess.run(["gcc", "-O1", "-std=c11", *SAN, "-o", exe,
                    os.path.join(ROOT, "tests", "sanitize_driver.c"),
                    os.path.join(ROOT, "oracle", "fp8ref.c"), os.path.join(ROOT, "synth", "synth.c"),
                    "-lpthread", "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitize driver ok" in r.stdout


VALIDATION_DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include "fp8gemm.h"
#define REQ(x) do { if (!(x)) { fprintf(stderr, "failed: %s\n", #x); return 1; } } while (0)
int main(void) {
  char *P = (char *)0x10000, *O = (char *)0x10004;
  const float *F = (const float *)0x10000;
  const int32_t *I = (const int32_t *)0x10000;
  REQ(gemm_fp8_1x128_128x128_bf16(P, F, P, F, P, -1, 64, 128, 0) == FP8GEMM_INVALID_ARG);
  REQ(gemm_fp8_1x128_128x128_bf16(P, F, P, F, P, 64, 64, 100, 0) == FP8GEMM_UNSUPPORTED_SHAPE);
  REQ(gemm_fp8_1x128_128x128_bf16(O, F, P, F, P, 64, 64, 128, 0) == FP8GEMM_MISALIGNED);
  REQ(gemm_fp8_1x128_128x128_bf16(P, F, P, F, P, 1 << 20, 64, 1 << 12, 0) == FP8GEMM_UNSUPPORTED_SHAPE);
  REQ(gemm_fp8_1x128_128x128_bf16(0, 0, 0, 0, 0, 0, 64, 128, 0) == FP8GEMM_OK);
  REQ(gemm_fp8_1x128_128x128_bf16_noalloc(P, F, P, F, 0, 64, 64, 128, 0) == FP8GEMM_INVALID_ARG);
  REQ(grouped_contiguous(P, F, P, F, P, 200, 64, 128, 2, 0, I) == FP8GEMM_UNSUPPORTED_SHAPE);
  REQ(grouped_contiguous(P, F, P, F, P, 256, 64, 128, 0, 0, I) == FP8GEMM_INVALID_ARG);
  REQ(grouped_masked(P, F, P, F, P, 256, 64, 128, 4, 0, I, -1) == FP8GEMM_INVALID_ARG);
  REQ(grouped_masked(P, F, P, F, P, 1, 64, 128, 1 << 16, 0, I, 0) == FP8GEMM_UNSUPPORTED_SHAPE);
  REQ(quantize_fp8_1x128(P, P, (float *)F, 64, 100, 0) == FP8GEMM_UNSUPPORTED_SHAPE);
  REQ(grouped_contiguous_swiglu_fp8(P, F, P, F, P, (float *)F, 256, 100, 128, 2, 0, I) == FP8GEMM_UNSUPPORTED_SHAPE);
  REQ(grouped_masked_swiglu_fp8(P, F, P, F, P, (float *)F, 256, 128, 128, 2, 0, I, -3) == FP8GEMM_INVALID_ARG);
  REQ(gemm_bf16_nt(P, P, P, 64, 64, 100, 0) == FP8GEMM_UNSUPPORTED_SHAPE);
  REQ(grouped_contiguous_bf16(P, P, P, 100, 64, 64, 2, 0, I) == FP8GEMM_UNSUPPORTED_SHAPE);
  REQ(grouped_masked_bf16(P, P, P, 64, 64, 64, 0, 0, I, 0) == FP8GEMM_INVALID_ARG);
  for (int s = 0; s < 8; ++s) REQ(fp8gemm_status_string(s) != 0);
  puts("validation driver ok");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")
def test_host_validation_under_sanitizers(tmp_path):
    """Every call below fails validation, so no HIP call is made; the
    library's host code runs instrumented (the device code is compiled as
    usual, without sanitizers)."""
    drv = tmp_path / "validate.c"
    drv.write_text(VALIDATION_DRIVER)
    exe = str(tmp_path / "validate")
    csrc = os.path.join(ROOT, "moe_grouped_gemm_act_amd", "csrc")
    host_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        host_san += ["-Xarch_host", f]
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O1", "-std=c++17", "-g",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
                    "-I", os.path.join(ROOT, "include"), "-o", exe,
                    "-x", "c++", str(drv), "-x", "hip", os.path.join(csrc, "fp8gemm.hip"),
                    os.path.join(csrc, "quant.hip")], check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validation driver ok" in r.stdout
