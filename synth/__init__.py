"""Seeded synthetic inputs for the FP8 block-scaled GEMM (see synth.c).

Produces e4m3fn codes (uint8) with fp32 block scales in the layouts the
library takes: activations [M, K] with scales [K/128, M]; weights [N, K] with
scales [ceil(N/128), K/128]; grouped tensors stack a leading G axis.  Holds
no GEMM arithmetic; the quantiser is the caller-side FP8 conversion that the
pages leave to the user (kakushin.no, "Hvorfor FP8 og FP4 er interessant").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build_command():
    return ["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-o", _LIB, _SRC,
            "-lpthread", "-lm"]


def build():
    subprocess.run(build_command(), check=True)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
        lib.synth_act.argtypes = [u64, u64, i32, i32, vp, vp, vp, i32]
        lib.synth_act.restype = i32
        lib.synth_weight.argtypes = [u64, u64, i32, i32, vp, vp, i32]
        lib.synth_weight.restype = i32
        lib.synth_normal.argtypes = [u64, u64, ctypes.c_int64, vp]
        lib.synth_normal.restype = None
        lib.synth_e4m3_encode.argtypes = [ctypes.c_float]
        lib.synth_e4m3_encode.restype = ctypes.c_uint8
        _lib = lib
    return _lib


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def normal(seed, n, offset=0):
    out = np.empty(n, np.float32)
    _load().synth_normal(seed, offset, n, _ptr(out))
    return out


def e4m3_encode(x: float) -> int:
    return int(_load().synth_e4m3_encode(float(x)))


def act(seed, M, K, row_mult=None, offset=0, threads=None):
    """Activations: codes [M, K] uint8 and sa [K/128, M] float32."""
    assert K % 128 == 0
    codes = np.empty((M, K), np.uint8)
    sa = np.empty((K // 128, M), np.float32)
    rm = None
    if row_mult is not None:
        rm = np.ascontiguousarray(row_mult, dtype=np.float32)
        assert rm.shape == (M,)
    rc = _load().synth_act(seed, offset, M, K, _ptr(rm) if rm is not None else None,
                           _ptr(codes), _ptr(sa), threads or default_threads())
    assert rc == 0
    return codes, sa


def weight(seed, N, K, offset=0, threads=None):
    """Weights: codes [N, K] uint8 and sb [ceil(N/128), K/128] float32."""
    assert K % 128 == 0
    codes = np.empty((N, K), np.uint8)
    sb = np.empty(((N + 127) // 128, K // 128), np.float32)
    rc = _load().synth_weight(seed, offset, N, K, _ptr(codes), _ptr(sb),
                              threads or default_threads())
    assert rc == 0
    return codes, sb


def grouped_act(seed, G, M, K, threads=None):
    """Masked-layout activations: A [G, M, K], sa [G, K/128, M]."""
    A = np.empty((G, M, K), np.uint8)
    sa = np.empty((G, K // 128, M), np.float32)
    for g in range(G):
        A[g], sa[g] = act(seed, M, K, offset=g * M * K, threads=threads)
    return A, sa


def grouped_weight(seed, G, N, K, threads=None):
    """Per-expert weights: B [G, N, K], sb [G, ceil(N/128), K/128]."""
    B = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, (N + 127) // 128, K // 128), np.float32)
    for g in range(G):
        B[g], sb[g] = weight(seed, N, K, offset=g * N * K, threads=threads)
    return B, sb


def heavy_rows(seed, M, frac=0.01, mult=50.0):
    """Row multipliers: round(frac*M) rows, picked by a seeded shuffle, get `mult`."""
    rng = np.random.Generator(np.random.Philox(seed))
    count = int(round(frac * M))
    rows = rng.permutation(M)[:count]
    out = np.ones(M, np.float32)
    out[rows] = mult
    return out


def contiguous_indices(seed, G, total, uniform):
    """m_indices for the M-axis contiguous layout.

    Expert segments start at multiples of 128 and together cover `total` rows.
    uniform=True: equal segments with no padding.  Otherwise G seeded segment
    lengths (multiples of 128, each >= 128) and a seeded 0..127-row padded tail
    in each segment (index -1).  Returns (m_indices int32 [total], segments)
    where segments is a list of (start, padded_len, valid_len).
    """
    assert total % 128 == 0 and total // 128 >= G
    if uniform:
        assert total % (128 * G) == 0
        lens = [total // G] * G
        valid = list(lens)
    else:
        rng = np.random.Generator(np.random.Philox(seed))
        blocks = total // 128
        cuts = np.sort(rng.choice(np.arange(1, blocks), size=G - 1, replace=False))
        sizes = np.diff(np.concatenate([[0], cuts, [blocks]]))
        lens = [int(s) * 128 for s in sizes]
        pads = rng.integers(0, 128, size=G)
        valid = [lens[g] - int(pads[g]) for g in range(G)]
    idx = np.full(total, -1, np.int32)
    segs = []
    start = 0
    for g in range(G):
        idx[start:start + valid[g]] = g
        segs.append((start, lens[g], valid[g]))
        start += lens[g]
    return idx, segs


def masked_counts(seed, G, M):
    """masked_m[g] uniform over 0..M inclusive."""
    rng = np.random.Generator(np.random.Philox(seed))
    return rng.integers(0, M + 1, size=G).astype(np.int32)
