"""Helpers shared by the GPU parity tests: moving seeded inputs to the GPU,
reading bf16 results back as bit patterns, and the tolerance check.

Tolerance (stated for this GEMM): every compared element satisfies
|out - ref| <= 8e-3 * |ref| + 1e-3 * rms(ref), and the relative Frobenius
error ||out - ref|| / ||ref|| <= 1e-3, where ref is the oracle's value
rounded once to bf16 and rms/norms run over the compared elements.  NaN must
appear exactly where the oracle has NaN.
"""
import numpy as np
import torch

import oracle

SENTINEL = 0x7FBF  # a NaN bit pattern the kernels never produce (their NaN is 0x7FC0)
REL_ELEM, ABS_RMS, FROB = 8e-3, 1e-3, 1e-3


def to_gpu(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def sentinel_out(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def bits(D):
    return D.view(torch.int16).cpu().numpy().view(np.uint16)


def f32(b):
    return oracle.bf16_bits_to_float(b)


def assert_close(out_bits, ref_bits, what=""):
    out_bits = np.asarray(out_bits).ravel()
    ref_bits = np.asarray(ref_bits).ravel()
    o, r = f32(out_bits).astype(np.float64), f32(ref_bits).astype(np.float64)
    nan_o, nan_r = np.isnan(o), np.isnan(r)
    assert (nan_o == nan_r).all(), f"{what}: NaN pattern differs at {np.flatnonzero(nan_o != nan_r)[:10]}"
    o, r = o[~nan_r], r[~nan_r]
    if r.size == 0:
        return
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(o - r)
    bound = REL_ELEM * np.abs(r) + ABS_RMS * rms
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, (f"{what}: {bad.size} elements out of tolerance; first {bad[:5]} "
                           f"out={o[bad[:5]]} ref={r[bad[:5]]}")
    nr = float(np.linalg.norm(r))
    frob = float(np.linalg.norm(o - r)) / nr if nr > 0 else float(np.linalg.norm(o - r))
    assert frob <= FROB, f"{what}: relative Frobenius error {frob:.3e}"
    return frob
