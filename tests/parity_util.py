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


def assert_close_full(out_bits, ref_bits, what="", chunk=1 << 23):
    """assert_close over arrays of any size, in chunks: the same element bound
    (with rms(ref) over all compared elements) and the relative Frobenius
    error over all of them.  Returns the Frobenius error."""
    o_all = np.asarray(out_bits).reshape(-1)
    r_all = np.asarray(ref_bits).reshape(-1)
    assert o_all.shape == r_all.shape, f"{what}: shapes differ"
    n = r_all.size
    sq, cnt = 0.0, 0
    for i in range(0, n, chunk):
        o, r = f32(o_all[i:i + chunk]), f32(r_all[i:i + chunk])
        nan_o, nan_r = np.isnan(o), np.isnan(r)
        assert (nan_o == nan_r).all(), \
            f"{what}: NaN pattern differs at {i + np.flatnonzero(nan_o != nan_r)[:10]}"
        r = r[~nan_r].astype(np.float64)
        sq += float(np.dot(r, r))
        cnt += r.size
    if cnt == 0:
        return 0.0
    rms = (sq / cnt) ** 0.5
    esq, bad, first = 0.0, 0, None
    for i in range(0, n, chunk):
        o, r = f32(o_all[i:i + chunk]).astype(np.float64), f32(r_all[i:i + chunk]).astype(np.float64)
        keep = ~np.isnan(r)
        o, r, pos = o[keep], r[keep], np.flatnonzero(keep) + i
        e = np.abs(o - r)
        esq += float(np.dot(e, e))
        over = np.flatnonzero(e > REL_ELEM * np.abs(r) + ABS_RMS * rms)
        if over.size and first is None:
            first = (pos[over[:5]], o[over[:5]], r[over[:5]])
        bad += over.size
    assert bad == 0, (f"{what}: {bad} of {cnt} elements out of tolerance; first at flat index "
                      f"{first[0]} out={first[1]} ref={first[2]}")
    frob = esq ** 0.5 / sq ** 0.5 if sq > 0 else esq ** 0.5
    assert frob <= FROB, f"{what}: relative Frobenius error {frob:.3e} over {cnt} elements"
    return frob


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
