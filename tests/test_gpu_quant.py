"""GPU parity of the 1x128 activation quantiser against the oracle: codes and
scales are integer / exactly-rounded results, so they must match bit for bit
(both sides divide in IEEE fp32 and round to the nearest e4m3fn value)."""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_act_amd as fg
import oracle
import synth

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def gpu_quant(xb, stream=None):
    X = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    A, sa = fg.quantize_fp8_1x128(X, stream=stream)
    torch.cuda.synchronize()
    return A.cpu().numpy(), sa.cpu().numpy()


def check(xb, what):
    codes, sa = oracle.quantize_1x128(xb)
    A, gsa = gpu_quant(xb)
    assert (A == codes).all(), f"{what}: {(A != codes).sum()} codes differ"
    assert (gsa.view(np.uint32) == sa.view(np.uint32)).all(), f"{what}: scales differ"


@pytest.mark.parametrize("M,K", [(1, 128), (64, 256), (100, 640), (129, 1024), (300, 2048)])
def test_quant_random_full(M, K):
    seed = 7000 + M + K
    announce(f"quant {M}x{K} seed {seed}")
    x = synth.normal(seed, M * K).reshape(M, K) * np.exp(
        synth.normal(seed + 1, M).reshape(M, 1) * 3).astype(np.float32)
    check(bf16_bits(x), f"{M}x{K}")


def test_quant_special_blocks():
    """exact ties (block maximum 448 makes the scale 1, so x / s = x), the
    subnormal grid, an all-zero block, NaN and infinity"""
    K = 128 * 6
    x = np.zeros((3, K), np.float32)
    mids = np.array([1.0625, 1.1875, 3.25, 0.0029296875, 0.0048828125, 13.0, 208.0, 440.0], np.float32)
    for r in range(3):
        x[r, 0] = 448.0
        x[r, 1:1 + mids.size] = mids * (1 if r != 1 else -1)
        x[r, 128:256] = np.float32(2.0 ** -12) * np.arange(128)  # tiny values, largest 127 * 2^-12
        x[r, 256:384] = 0.0  # all zero
        x[r, 384:512] = np.linspace(-3, 3, 128)
        x[r, 640:768] = np.linspace(-1e30, 1e30, 128)
    xb = bf16_bits(x)
    xb[0, 400] = 0x7FC0  # NaN inside a block
    xb[1, 520] = 0x7F80  # +inf: the scale becomes inf
    xb[2, 401] = 0xFFC0  # a negative NaN keeps its sign
    xb[2, 402] = 0x8000  # -0 encodes as -0
    xb[0, 700:702] = [0x0080, 0x8001]  # tiny elements beside 1e30-sized ones
    announce("quant special blocks")
    check(xb, "special blocks")


def test_quant_prefill_activation_full():
    M, K = 4096, 7168
    x = synth.normal(7100, M * K).reshape(M, K)
    x[synth.heavy_rows(7107, M) > 1] *= 50
    xb = bf16_bits(x)
    announce("quant 4096x7168")
    A, gsa = gpu_quant(xb)
    codes, sa = oracle.quantize_1x128(xb)
    assert (A == codes).all()
    assert (gsa.view(np.uint32) == sa.view(np.uint32)).all()


def test_quant_stream_and_determinism():
    x = bf16_bits(synth.normal(7200, 256 * 1024).reshape(256, 1024))
    a1, s1 = gpu_quant(x)
    a2, s2 = gpu_quant(x, stream=torch.cuda.Stream())
    assert (a1 == a2).all() and (s1 == s2).all()


def test_quant_feeds_the_gemm():
    """quantise -> GEMM on the GPU equals the oracle GEMM of the oracle's
    quantisation (same bytes, so the GEMM tolerance applies)"""
    from parity_util import assert_close
    M, N, K = 96, 384, 1024
    xa = bf16_bits(synth.normal(7300, M * K).reshape(M, K))
    B, sb = synth.weight(7301, N, K)
    X = torch.from_numpy(xa.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    A, sa = fg.quantize_fp8_1x128(X)
    D = fg.gemm_fp8_1x128_128x128_bf16(A, sa, torch.from_numpy(B).to("cuda:0"),
                                       torch.from_numpy(sb).to("cuda:0"))
    torch.cuda.synchronize()
    codes, osa = oracle.quantize_1x128(xa)
    ref = oracle.gemm(codes, osa, B, sb)
    assert_close(D.view(torch.int16).cpu().numpy().view(np.uint16), ref, "quantise + gemm")
