"""CPU oracle for the FP8 block-scaled NT GEMM (ctypes over fp8ref.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU library never does and
shares no code with it.

Every function takes numpy arrays in the library's layouts (A [M,K] uint8
e4m3fn codes, sa [K/128, M] fp32, B [N,K] uint8, sb [ceil(N/128), K/128]
fp32; grouped forms add a leading G axis as described per function) and
returns bf16 bit patterns as uint16 (and, on request, the unrounded fp64
values).  The definition it follows is spelled out in fp8ref.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8ref.c")
_LIB = os.path.join(_HERE, "libfp8ref.so")
_lib = None


def build_command(src=_SRC, out=_LIB, defines=()):
    return (["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC"]
            + [f"-D{d}" for d in defines] + ["-o", out, src, "-lpthread", "-lm"])


def build():
    subprocess.run(build_command(), check=True)


def _bind(lib):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
    lib.fp8ref_e4m3_value.argtypes = [i32]
    lib.fp8ref_e4m3_value.restype = ctypes.c_double
    lib.fp8ref_bf16_rne.argtypes = [ctypes.c_double]
    lib.fp8ref_bf16_rne.restype = ctypes.c_uint16
    lib.fp8ref_block_dot.argtypes = [vp, vp]
    lib.fp8ref_block_dot.restype = ctypes.c_double
    lib.fp8ref_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32]
    lib.fp8ref_grouped_contiguous.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32]
    lib.fp8ref_grouped_masked.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32]
    lib.fp8ref_e4m3_encode.argtypes = [ctypes.c_float]
    lib.fp8ref_e4m3_encode.restype = ctypes.c_uint8
    lib.fp8ref_quantize_1x128.argtypes = [vp, i32, i32, vp, vp]
    lib.fp8ref_quantize_1x128.restype = i32
    lib.fp8ref_swiglu_quant.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, i32]
    lib.fp8ref_swiglu_quant.restype = i32
    lib.fp8ref_points.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, i64, vp, vp,
                                  vp, vp, vp]
    lib.fp8ref_gemm_bf16.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32]
    for f in (lib.fp8ref_gemm, lib.fp8ref_grouped_contiguous, lib.fp8ref_grouped_masked,
              lib.fp8ref_points, lib.fp8ref_gemm_bf16):
        f.restype = i32
    return lib


def load(path=_LIB):
    """Load (building first if absent) the oracle library; `path` lets tests
    load a separately compiled variant."""
    global _lib
    if path != _LIB:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _threads(threads):
    return threads or max(1, min(16, os.cpu_count() or 1))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def e4m3_value(code, lib=None):
    return (lib or load()).fp8ref_e4m3_value(int(code))


def bf16_rne(x, lib=None):
    return int((lib or load()).fp8ref_bf16_rne(float(x)))


def block_dot(a, b, lib=None):
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    assert a.shape == (128,) and b.shape == (128,)
    return (lib or load()).fp8ref_block_dot(_p(a), _p(b))


def gemm(A, sa, B, sb, want64=False, out=None, threads=None, lib=None):
    """Dense: D[m,n] for A [M,K], sa [K/128,M], B [N,K], sb [ceil(N/128),K/128]."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K and sa.shape == (K // 128, M) and sb.shape == ((N + 127) // 128, K // 128)
    D = out if out is not None else np.zeros((M, N), np.uint16)
    D64 = np.full((M, N), np.nan) if want64 else None
    rc = (lib or load()).fp8ref_gemm(_p(A), _p(sa), _p(B), _p(sb), _p(D), _p(D64), M, N, K,
                                     _threads(threads))
    assert rc == 0
    return (D, D64) if want64 else D


def grouped_contiguous(A, sa, B, sb, m_indices, out, want64=False, threads=None, lib=None):
    """A [M,K], sa [K/128,M], B [G,N,K], sb [G,Nb,Kb], m_indices [M] int32.
    Rows with an index outside [0,G) keep whatever `out` holds."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    idx = _c(m_indices, np.int32)
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    assert out.dtype == np.uint16 and out.shape == (M, N) and out.flags.c_contiguous
    D64 = np.full((M, N), np.nan) if want64 else None
    rc = (lib or load()).fp8ref_grouped_contiguous(_p(A), _p(sa), _p(B), _p(sb), _p(out),
                                                   _p(D64), M, N, K, G, _p(idx),
                                                   _threads(threads))
    assert rc == 0
    return (out, D64) if want64 else out


def grouped_masked(A, sa, B, sb, masked_m, out, want64=False, threads=None, lib=None):
    """A [G,M,K], sa [G,K/128,M], B [G,N,K], sb [G,Nb,Kb], masked_m [G] int32.
    Rows m >= clamp(masked_m[g], 0, M) keep whatever `out` [G,M,N] holds."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    mm = _c(masked_m, np.int32)
    G, M, K = A.shape
    N = B.shape[1]
    assert out.dtype == np.uint16 and out.shape == (G, M, N) and out.flags.c_contiguous
    D64 = np.full((G, M, N), np.nan) if want64 else None
    rc = (lib or load()).fp8ref_grouped_masked(_p(A), _p(sa), _p(B), _p(sb), _p(out),
                                               _p(D64), M, N, K, G, _p(mm),
                                               _threads(threads))
    assert rc == 0
    return (out, D64) if want64 else out


def points(kind, A, sa, B, sb, pm, pn, pg=None, m_indices=None, want64=False, lib=None):
    """Values at sample points.  kind 'dense' | 'contiguous' | 'masked'.
    Shapes as in the full functions; for 'masked' pass pg (group of each point).
    Contiguous points on rows that are not written come back as 0xFFFF."""
    k = {"dense": 0, "contiguous": 1, "masked": 2}[kind]
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    K = A.shape[-1]
    M = A.shape[-2]
    N = B.shape[-2]
    G = B.shape[0] if kind != "dense" else 1
    pm, pn = _c(pm, np.int64), _c(pn, np.int64)
    pg = _c(pg if pg is not None else np.zeros_like(pm), np.int64)
    idx = _c(m_indices, np.int32) if m_indices is not None else None
    out = np.zeros(len(pm), np.uint16)
    o64 = np.zeros(len(pm)) if want64 else None
    rc = (lib or load()).fp8ref_points(k, _p(A), _p(sa), _p(B), _p(sb), M, N, K, G, _p(idx),
                                       len(pm), _p(pg), _p(pm), _p(pn), _p(out), _p(o64))
    assert rc == 0
    return (out, o64) if want64 else out


def bf16_bits_to_float(bits):
    """bf16 bit patterns (uint16) -> float32 values (exact widening)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_encode(v, lib=None):
    """Nearest e4m3fn code to the fp32 value v (ties to the even code,
    saturating at 448, NaN to the NaN code)."""
    return int((lib or load()).fp8ref_e4m3_encode(float(np.float32(v))))


def quantize_1x128(x_bf16_bits, lib=None):
    """x: uint16 bf16 bits [M, K] -> (codes uint8 [M, K], sa float32 [K/128, M])."""
    x = _c(x_bf16_bits, np.uint16)
    M, K = x.shape
    codes = np.empty((M, K), np.uint8)
    sa = np.empty((K // 128, M), np.float32)
    rc = (lib or load()).fp8ref_quantize_1x128(_p(x), M, K, _p(codes), _p(sa))
    if rc:
        raise ValueError("fp8ref_quantize_1x128: bad shape")
    return codes, sa


def swiglu_quant(kind, A, sa, B, sb, idx, codes, scales, threads=None, lib=None):
    """Grouped GEMM with B_g = [W_gate; W_up] (2I rows), SwiGLU and 1x128
    requantisation of y = silu(g) * u.  kind "contiguous": A [M,K],
    sa [K/128,M], idx = m_indices [M], codes [M,I], scales [I/128,M];
    kind "masked": A [G,M,K], sa [G,K/128,M], idx = masked_m [G],
    codes [G,M,I], scales [G,I/128,M].  codes / scales are updated in place
    (rows not computed keep their contents) and returned."""
    k = {"contiguous": 1, "masked": 2}[kind]
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    idx = _c(idx, np.int32)
    G, N2, K = B.shape
    I = N2 // 2
    M = A.shape[0] if kind == "contiguous" else A.shape[1]
    assert codes.flags.c_contiguous and scales.flags.c_contiguous
    rc = (lib or load()).fp8ref_swiglu_quant(k, _p(A), _p(sa), _p(B), _p(sb), M, I, K, G, _p(idx),
                                              _p(codes), _p(scales), _threads(threads))
    if rc:
        raise ValueError("fp8ref_swiglu_quant: bad arguments")
    return codes, scales



def gemm_bf16(kind, A, B, idx=None, out=None, want64=False, threads=None, lib=None):
    """BF16 NT GEMM without scales, D = bf16(A B^T) per row.  kind 'dense':
    A [M,K], B [N,K]; 'contiguous': A [M,K], B [G,N,K], idx = m_indices [M];
    'masked': A [G,M,K], B [G,N,K], idx = masked_m [G].  A and B hold bf16
    bits (uint16).  `out` (bf16 bits, [M,N] or [G,M,N]) is updated in place:
    rows not computed keep their contents.  Returns out (and the unrounded
    fp64 values, NaN where not computed, with want64)."""
    k = {"dense": 0, "contiguous": 1, "masked": 2}[kind]
    A, B = _c(A, np.uint16), _c(B, np.uint16)
    if kind == "masked":
        G, M, K = A.shape
    else:
        (M, K), G = A.shape, (B.shape[0] if kind == "contiguous" else 1)
    N = B.shape[-2]
    shape = (G, M, N) if kind == "masked" else (M, N)
    if out is None:
        out = np.zeros(shape, np.uint16)
    assert out.shape == shape and out.dtype == np.uint16 and out.flags.c_contiguous
    D64 = np.full(shape, np.nan) if want64 else None
    ix = _c(idx, np.int32) if idx is not None else None
    rc = (lib or load()).fp8ref_gemm_bf16(k, _p(A), _p(B), _p(out), _p(D64), M, N, K, G, _p(ix),
                                          _threads(threads))
    if rc:
        raise ValueError("fp8ref_gemm_bf16: bad arguments")
    return (out, D64) if want64 else out
