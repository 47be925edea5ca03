"""Python binding for libfp8gemm (FP8 e4m3 1x128/128x128 block-scaled NT GEMM,
bf16 output; dense, M-axis contiguous grouped and masked grouped).

Argument marshalling only: every step runs in the HIP kernels of
libfp8gemm.so, built in-tree by ``moe_grouped_gemm_act_amd.build``.  PyTorch
provides device memory and the current HIP stream.  There is no fallback: if
the library is missing, importing the functions raises.

Layouts (row-major, contiguous): A [M,K] and B [N,K] hold e4m3fn codes
(torch.uint8 or torch.float8_e4m3fn); sa [K/128, M] and sb [ceil(N/128), K/128]
are float32; D is bfloat16 [M,N].  Grouped forms add a leading G axis as in
include/fp8gemm.h.

Example (one MoE layer's expert GEMMs on device tensors)::

    import moe_grouped_gemm_act_amd as fg
    A, sa = fg.quantize_fp8_1x128(x)                # x: bf16 [rows, K]
    Y, sy = fg.grouped_contiguous_swiglu_fp8(A, sa, W13, s13, m_indices)
    D = fg.grouped_contiguous(Y, sy, W2, s2, m_indices)  # bf16 [rows, N]

W13 holds each expert's [W_gate; W_up] rows (2I of them), W2 the down
projection; s13 and s2 are their 128x128 block scales.  Every call enqueues
on the current stream and may be captured into a HIP graph.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch  # loads the HIP runtime this library binds to (same SONAME)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8gemm.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "fp8gemm.h")

__all__ = ["gemm_fp8_1x128_128x128_bf16", "gemm_fp8_1x128_128x128_bf16_noalloc",
           "grouped_contiguous", "grouped_masked",
           "quantize_fp8_1x128", "grouped_contiguous_swiglu_fp8", "grouped_masked_swiglu_fp8",
           "gemm_bf16_nt", "grouped_contiguous_bf16", "grouped_masked_bf16",
           "fp8gemm_status_string", "Fp8GemmError", "load_library",
           "LIB_PATH"]


class Fp8GemmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libfp8gemm status {status}: {msg}")
        self.status = status


_lib = None


def load_library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.gemm_fp8_1x128_128x128_bf16.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp]
        lib.gemm_fp8_1x128_128x128_bf16_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp]
        lib.grouped_contiguous.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp]
        lib.grouped_masked.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, i32]
        lib.quantize_fp8_1x128.argtypes = [vp, vp, vp, i32, i32, vp]
        lib.grouped_contiguous_swiglu_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                      vp, vp]
        lib.grouped_masked_swiglu_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp,
                                                  vp, i32]
        lib.gemm_bf16_nt.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        lib.grouped_contiguous_bf16.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
        lib.grouped_masked_bf16.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, i32]
        for f in (lib.gemm_fp8_1x128_128x128_bf16, lib.gemm_fp8_1x128_128x128_bf16_noalloc,
                  lib.grouped_contiguous, lib.grouped_masked,
                  lib.quantize_fp8_1x128, lib.grouped_contiguous_swiglu_fp8,
                  lib.grouped_masked_swiglu_fp8, lib.gemm_bf16_nt, lib.grouped_contiguous_bf16,
                  lib.grouped_masked_bf16):
            f.restype = i32
        lib.fp8gemm_status_string.argtypes = [i32]
        lib.fp8gemm_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def declared_functions():
    """Names of the functions include/fp8gemm.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def fp8gemm_status_string(status: int) -> str:
    return load_library().fp8gemm_status_string(int(status)).decode()


def _check(status):
    if status != 0:
        raise Fp8GemmError(status, fp8gemm_status_string(status))


def _codes(t, name):
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must hold e4m3fn codes (uint8 or float8_e4m3fn), got {t.dtype}")
    return t


def _dev(*ts):
    dev = ts[0].device
    for t in ts:
        if t.device != dev or t.device.type != "cuda":
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream, dev):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, D=None, stream=None):
    """D[M,N] (bf16) = block-scaled A[M,K] * B[N,K]^T; returns D."""
    A, B = _codes(A, "A"), _codes(B, "B")
    M, K = A.shape
    N = B.shape[0]
    if D is None:
        D = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _shape(B, (N, K), "B")
    _shape(sa, (K // 128, M), "sa")
    _shape(sb, ((N + 127) // 128, K // 128), "sb")
    _shape(D, (M, N), "D")
    if sa.dtype != torch.float32 or sb.dtype != torch.float32 or D.dtype != torch.bfloat16:
        raise TypeError("sa, sb must be float32 and D bfloat16")
    dev = _dev(A, sa, B, sb, D)
    _check(load_library().gemm_fp8_1x128_128x128_bf16(
        _p(A), _p(sa), _p(B), _p(sb), _p(D), M, N, K, _stream(stream, dev)))
    return D


def gemm_fp8_1x128_128x128_bf16_noalloc(A, sa, B, sb, D, stream=None):
    """The allocation-free form of gemm_fp8_1x128_128x128_bf16: same result,
    split-K partials in the library's fixed device scratch, nothing allocated
    (D must be given).  Calls that overlap on one GPU race on the scratch."""
    A, B = _codes(A, "A"), _codes(B, "B")
    M, K = A.shape
    N = B.shape[0]
    _shape(B, (N, K), "B")
    _shape(sa, (K // 128, M), "sa")
    _shape(sb, ((N + 127) // 128, K // 128), "sb")
    _shape(D, (M, N), "D")
    if sa.dtype != torch.float32 or sb.dtype != torch.float32 or D.dtype != torch.bfloat16:
        raise TypeError("sa, sb must be float32 and D bfloat16")
    dev = _dev(A, sa, B, sb, D)
    _check(load_library().gemm_fp8_1x128_128x128_bf16_noalloc(
        _p(A), _p(sa), _p(B), _p(sb), _p(D), M, N, K, _stream(stream, dev)))
    return D


def grouped_contiguous(A, sa, B, sb, m_indices, D=None, stream=None):
    """M-axis contiguous grouping: A [M,K], sa [K/128,M], B [G,N,K],
    sb [G,ceil(N/128),K/128], m_indices [M] int32; rows whose index is outside
    [0,G) are not written.  Returns D [M,N]."""
    A, B = _codes(A, "A"), _codes(B, "B")
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    if D is None:
        D = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _shape(B, (G, N, K), "B")
    _shape(sa, (K // 128, M), "sa")
    _shape(sb, (G, (N + 127) // 128, K // 128), "sb")
    _shape(m_indices, (M,), "m_indices")
    _shape(D, (M, N), "D")
    if m_indices.dtype != torch.int32:
        raise TypeError("m_indices must be int32")
    dev = _dev(A, sa, B, sb, m_indices, D)
    _check(load_library().grouped_contiguous(
        _p(A), _p(sa), _p(B), _p(sb), _p(D), M, N, K, G, _stream(stream, dev), _p(m_indices)))
    return D


def grouped_masked(A, sa, B, sb, masked_m, expected_m, D=None, stream=None):
    """Masked grouping: A [G,M,K], sa [G,K/128,M], B [G,N,K],
    sb [G,ceil(N/128),K/128], masked_m [G] int32 (device); only rows
    m < masked_m[g] of D [G,M,N] are written.  Returns D."""
    A, B = _codes(A, "A"), _codes(B, "B")
    G, M, K = A.shape
    N = B.shape[1]
    if D is None:
        D = torch.empty((G, M, N), dtype=torch.bfloat16, device=A.device)
    _shape(B, (G, N, K), "B")
    _shape(sa, (G, K // 128, M), "sa")
    _shape(sb, (G, (N + 127) // 128, K // 128), "sb")
    _shape(masked_m, (G,), "masked_m")
    _shape(D, (G, M, N), "D")
    if masked_m.dtype != torch.int32:
        raise TypeError("masked_m must be int32")
    dev = _dev(A, sa, B, sb, masked_m, D)
    _check(load_library().grouped_masked(
        _p(A), _p(sa), _p(B), _p(sb), _p(D), M, N, K, G, _stream(stream, dev), _p(masked_m),
        int(expected_m)))
    return D


def quantize_fp8_1x128(X, A=None, sa=None, stream=None):
    """1x128 quantisation of bf16 activations X [M,K]: returns (A [M,K] e4m3fn
    codes as uint8, sa [K/128,M] float32), the operands of the GEMM calls."""
    M, K = X.shape
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    if A is None:
        A = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    if sa is None:
        sa = torch.empty((K // 128, M), dtype=torch.float32, device=X.device)
    A = _codes(A, "A")
    _shape(A, (M, K), "A")
    _shape(sa, (K // 128, M), "sa")
    if sa.dtype != torch.float32:
        raise TypeError("sa must be float32")
    dev = _dev(X, A, sa)
    _check(load_library().quantize_fp8_1x128(_p(X), _p(A), _p(sa), M, K, _stream(stream, dev)))
    return A, sa


def _swiglu_outputs(Y, sy, lead, M, I, dev):
    if Y is None:
        Y = torch.empty((*lead, M, I), dtype=torch.uint8, device=dev)
    if sy is None:
        sy = torch.empty((*lead, I // 128, M), dtype=torch.float32, device=dev)
    Y = _codes(Y, "Y")
    _shape(Y, (*lead, M, I), "Y")
    _shape(sy, (*lead, I // 128, M), "sy")
    if sy.dtype != torch.float32:
        raise TypeError("sy must be float32")
    return Y, sy


def grouped_contiguous_swiglu_fp8(A, sa, B, sb, m_indices, Y=None, sy=None, stream=None):
    """Contiguous grouping with SwiGLU and 1x128 requantisation fused:
    A [M,K], sa [K/128,M], B [G,2I,K] (gate rows over up rows),
    sb [G,2I/128,K/128], m_indices [M] int32.  Returns (Y [M,I] e4m3fn codes
    as uint8, sy [I/128,M] float32); rows whose index is outside [0,G) are
    not written."""
    A, B = _codes(A, "A"), _codes(B, "B")
    M, K = A.shape
    G, N2 = B.shape[0], B.shape[1]
    I = N2 // 2
    _shape(B, (G, 2 * I, K), "B")
    _shape(sa, (K // 128, M), "sa")
    _shape(sb, (G, (2 * I + 127) // 128, K // 128), "sb")
    _shape(m_indices, (M,), "m_indices")
    if m_indices.dtype != torch.int32:
        raise TypeError("m_indices must be int32")
    Y, sy = _swiglu_outputs(Y, sy, (), M, I, A.device)
    dev = _dev(A, sa, B, sb, m_indices, Y, sy)
    _check(load_library().grouped_contiguous_swiglu_fp8(
        _p(A), _p(sa), _p(B), _p(sb), _p(Y), _p(sy), M, I, K, G, _stream(stream, dev),
        _p(m_indices)))
    return Y, sy


def grouped_masked_swiglu_fp8(A, sa, B, sb, masked_m, expected_m, Y=None, sy=None, stream=None):
    """Masked grouping with SwiGLU and 1x128 requantisation fused:
    A [G,M,K], sa [G,K/128,M], B [G,2I,K], sb [G,2I/128,K/128], masked_m [G]
    int32.  Returns (Y [G,M,I] codes, sy [G,I/128,M]); only rows
    m < masked_m[g] are written."""
    A, B = _codes(A, "A"), _codes(B, "B")
    G, M, K = A.shape
    I = B.shape[1] // 2
    _shape(B, (G, 2 * I, K), "B")
    _shape(sa, (G, K // 128, M), "sa")
    _shape(sb, (G, (2 * I + 127) // 128, K // 128), "sb")
    _shape(masked_m, (G,), "masked_m")
    if masked_m.dtype != torch.int32:
        raise TypeError("masked_m must be int32")
    Y, sy = _swiglu_outputs(Y, sy, (G,), M, I, A.device)
    dev = _dev(A, sa, B, sb, masked_m, Y, sy)
    _check(load_library().grouped_masked_swiglu_fp8(
        _p(A), _p(sa), _p(B), _p(sb), _p(Y), _p(sy), M, I, K, G, _stream(stream, dev),
        _p(masked_m), int(expected_m)))
    return Y, sy


def _bf16(t, name):
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    return t


def gemm_bf16_nt(A, B, D=None, stream=None):
    """D[M,N] = bf16(A[M,K] B[N,K]^T), all bfloat16, fp32 accumulation; returns D."""
    A, B = _bf16(A, "A"), _bf16(B, "B")
    M, K = A.shape
    N = B.shape[0]
    if D is None:
        D = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _shape(B, (N, K), "B")
    _shape(_bf16(D, "D"), (M, N), "D")
    dev = _dev(A, B, D)
    _check(load_library().gemm_bf16_nt(_p(A), _p(B), _p(D), M, N, K, _stream(stream, dev)))
    return D


def grouped_contiguous_bf16(A, B, m_indices, D=None, stream=None):
    """BF16 contiguous grouping: A [M,K], B [G,N,K], m_indices [M] int32;
    rows whose index is outside [0,G) are not written.  Returns D [M,N]."""
    A, B = _bf16(A, "A"), _bf16(B, "B")
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    if D is None:
        D = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _shape(B, (G, N, K), "B")
    _shape(m_indices, (M,), "m_indices")
    _shape(_bf16(D, "D"), (M, N), "D")
    if m_indices.dtype != torch.int32:
        raise TypeError("m_indices must be int32")
    dev = _dev(A, B, m_indices, D)
    _check(load_library().grouped_contiguous_bf16(_p(A), _p(B), _p(D), M, N, K, G,
                                                  _stream(stream, dev), _p(m_indices)))
    return D


def grouped_masked_bf16(A, B, masked_m, expected_m, D=None, stream=None):
    """BF16 masked grouping: A [G,M,K], B [G,N,K], masked_m [G] int32; only
    rows m < masked_m[g] of D [G,M,N] are written.  Returns D."""
    A, B = _bf16(A, "A"), _bf16(B, "B")
    G, M, K = A.shape
    N = B.shape[1]
    if D is None:
        D = torch.empty((G, M, N), dtype=torch.bfloat16, device=A.device)
    _shape(B, (G, N, K), "B")
    _shape(masked_m, (G,), "masked_m")
    _shape(_bf16(D, "D"), (G, M, N), "D")
    if masked_m.dtype != torch.int32:
        raise TypeError("masked_m must be int32")
    dev = _dev(A, B, masked_m, D)
    _check(load_library().grouped_masked_bf16(_p(A), _p(B), _p(D), M, N, K, G,
                                              _stream(stream, dev), _p(masked_m), int(expected_m)))
    return D
