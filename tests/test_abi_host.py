"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments synchronously, before any HIP call
(every call below fails validation, so nothing is launched)."""
import ctypes

import pytest

import moe_grouped_gemm_act_amd as fg

OK, INVALID, SHAPE, MISALIGNED = 0, 1, 2, 3
P = ctypes.c_void_p(0x10000)       # aligned non-null stand-in; never dereferenced
P_ODD = ctypes.c_void_p(0x10004)   # 4-byte but not 16-byte aligned
NUL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return fg.load_library()


def test_exports_every_declared_function(lib):
    names = fg.declared_functions()
    assert set(names) == {"gemm_fp8_1x128_128x128_bf16", "gemm_fp8_1x128_128x128_bf16_noalloc",
                          "grouped_contiguous",
                          "grouped_masked", "quantize_fp8_1x128",
                          "grouped_contiguous_swiglu_fp8", "grouped_masked_swiglu_fp8",
                          "gemm_bf16_nt", "grouped_contiguous_bf16", "grouped_masked_bf16",
                          "fp8gemm_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(6):
        assert fg.fp8gemm_status_string(s) != "unknown status"
    assert fg.fp8gemm_status_string(99) == "unknown status"


def dense(lib, A=P, sa=P, B=P, sb=P, D=P, M=64, N=64, K=128):
    return lib.gemm_fp8_1x128_128x128_bf16(A, sa, B, sb, D, M, N, K, NUL)


def test_dense_validation(lib):
    assert dense(lib, M=-1) == INVALID
    assert dense(lib, N=-5) == INVALID
    assert dense(lib, K=-128) == INVALID
    assert dense(lib, A=NUL) == INVALID
    assert dense(lib, sb=NUL) == INVALID
    assert dense(lib, D=NUL) == INVALID
    assert dense(lib, K=100) == SHAPE
    assert dense(lib, K=129) == SHAPE
    assert dense(lib, A=P_ODD) == MISALIGNED
    assert dense(lib, D=P_ODD) == MISALIGNED
    assert dense(lib, sa=ctypes.c_void_p(0x10002)) == MISALIGNED
    assert dense(lib, M=1 << 20, K=1 << 12) == SHAPE  # 2^32 elements
    # empty problems succeed without launching, even with null pointers
    assert dense(lib, A=NUL, sa=NUL, B=NUL, sb=NUL, D=NUL, M=0) == OK
    assert dense(lib, A=NUL, sa=NUL, B=NUL, sb=NUL, D=NUL, N=0) == OK


def test_dense_noalloc_validation(lib):
    """the allocation-free dense call validates exactly as the dense call"""
    def call(A=P, sa=P, B=P, sb=P, D=P, M=64, N=64, K=128):
        return lib.gemm_fp8_1x128_128x128_bf16_noalloc(A, sa, B, sb, D, M, N, K, NUL)
    for kw, want in (({"M": -1}, INVALID), ({"A": NUL}, INVALID), ({"D": NUL}, INVALID),
                     ({"K": 100}, SHAPE), ({"A": P_ODD}, MISALIGNED),
                     ({"M": 1 << 20, "K": 1 << 12}, SHAPE)):
        assert call(**kw) == want == dense(lib, **kw), kw
    assert call(A=NUL, sa=NUL, B=NUL, sb=NUL, D=NUL, M=0) == OK


def test_contiguous_validation(lib):
    def call(G=2, M=256, K=128, idx=P, A=P):
        return lib.grouped_contiguous(A, P, P, P, P, M, 64, K, G, NUL, idx)
    assert call(G=0) == INVALID
    assert call(idx=NUL) == INVALID
    assert call(M=200) == SHAPE
    assert call(K=64) == SHAPE
    assert call(idx=ctypes.c_void_p(0x10001)) == MISALIGNED
    assert call(A=P_ODD) == MISALIGNED
    assert lib.grouped_contiguous(NUL, NUL, NUL, NUL, NUL, 0, 64, 128, 2, NUL, NUL) == OK


def test_masked_validation(lib):
    def call(G=4, M=256, K=128, mm=P, expected=128):
        return lib.grouped_masked(P, P, P, P, P, M, 64, K, G, NUL, mm, expected)
    assert call(G=0) == INVALID
    assert call(expected=-1) == INVALID
    assert call(mm=NUL) == INVALID
    assert call(K=130) == SHAPE
    assert call(G=1 << 16, M=1, K=128) == SHAPE
    assert lib.grouped_masked(NUL, NUL, NUL, NUL, NUL, 0, 64, 128, 4, NUL, NUL, 0) == OK


def test_quantize_validation(lib):
    def call(X=P, A=P, sa=P, M=64, K=256):
        return lib.quantize_fp8_1x128(X, A, sa, M, K, NUL)
    assert call(M=-1) == INVALID
    assert call(X=NUL) == INVALID
    assert call(sa=NUL) == INVALID
    assert call(K=130) == SHAPE
    assert call(M=1 << 20, K=1 << 12) == SHAPE  # M * K * 2 past 2^31
    assert call(X=P_ODD) == MISALIGNED
    assert call(A=P_ODD) == MISALIGNED
    assert call(sa=ctypes.c_void_p(0x10002)) == MISALIGNED
    assert call(X=NUL, A=NUL, sa=NUL, M=0) == OK  # empty: nothing launched


def test_swiglu_validation(lib):
    def contig(G=2, M=256, I=256, K=256, Y=P, sy=P, idx=P):
        return lib.grouped_contiguous_swiglu_fp8(P, P, P, P, Y, sy, M, I, K, G, NUL, idx)

    def masked(G=2, M=256, I=256, K=256, Y=P, sy=P, mm=P, expected=64):
        return lib.grouped_masked_swiglu_fp8(P, P, P, P, Y, sy, M, I, K, G, NUL, mm, expected)
    for call in (contig, masked):
        assert call(G=0) == INVALID
        assert call(I=-128) == INVALID
        assert call(sy=NUL) == INVALID
        assert call(Y=NUL) == INVALID
        assert call(I=64) == SHAPE      # I must be a whole number of 128-wide blocks
        assert call(I=192) == SHAPE
        assert call(K=20608) == SHAPE   # past the kernel's K range
        assert call(K=100) == SHAPE
        assert call(Y=P_ODD) == MISALIGNED
        assert call(sy=ctypes.c_void_p(0x10002)) == MISALIGNED
        assert call(M=0, Y=NUL, sy=NUL) == OK  # empty: nothing launched
        assert call(I=0, Y=NUL, sy=NUL) == OK
    assert contig(idx=NUL) == INVALID
    assert contig(M=200) == SHAPE
    assert masked(mm=NUL) == INVALID
    assert masked(expected=-1) == INVALID
    assert masked(G=1 << 16, M=1, K=128) == SHAPE


def test_bf16_validation(lib):
    def dense(A=P, B=P, D=P, M=64, N=64, K=128):
        return lib.gemm_bf16_nt(A, B, D, M, N, K, NUL)

    def contig(G=2, M=256, K=128, idx=P, A=P):
        return lib.grouped_contiguous_bf16(A, P, P, M, 64, K, G, NUL, idx)

    def masked(G=4, M=256, K=128, mm=P, expected=64, D=P):
        return lib.grouped_masked_bf16(P, P, D, M, 64, K, G, NUL, mm, expected)
    assert dense(M=-1) == INVALID
    assert dense(A=NUL) == INVALID
    assert dense(D=NUL) == INVALID
    assert dense(K=96) == SHAPE        # K must be a multiple of 64
    assert dense(A=P_ODD) == MISALIGNED
    assert dense(D=P_ODD) == MISALIGNED
    assert dense(M=1 << 16, K=1 << 14) == SHAPE  # A past 2^31 bytes
    assert dense(A=NUL, B=NUL, D=NUL, M=0) == OK
    assert dense(A=NUL, B=NUL, D=NUL, N=0) == OK
    assert contig(G=0) == INVALID
    assert contig(idx=NUL) == INVALID
    assert contig(M=200) == SHAPE
    assert contig(K=32) == SHAPE
    assert contig(idx=ctypes.c_void_p(0x10001)) == MISALIGNED
    assert contig(A=P_ODD) == MISALIGNED
    assert masked(G=0) == INVALID
    assert masked(expected=-1) == INVALID
    assert masked(mm=NUL) == INVALID
    assert masked(K=100) == SHAPE
    assert masked(D=P_ODD) == MISALIGNED
    assert masked(G=1 << 16, M=1, K=64) == SHAPE


def test_binding_rejects_bad_tensors():
    import torch
    A = torch.zeros((4, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):  # CPU tensors are refused before the library is called
        fg.gemm_fp8_1x128_128x128_bf16(A, torch.zeros((1, 4)), torch.zeros((8, 128), dtype=torch.uint8),
                                       torch.zeros((1, 1)), D=torch.zeros((4, 8), dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        fg.gemm_fp8_1x128_128x128_bf16(A.float(), None, None, None)
