"""Python access to the C oracle (oracle/gemm_ref.c).

TEST INFRASTRUCTURE ONLY (see the package docstring).

All matrices are numpy arrays of uint16 encodings (binary16 or bfloat16),
contiguous and row-major:
  A [M, K];  B [N, K] for the NT form, [K, N] for the NN form;  C [M, N].

The arithmetic itself lives in gemm_ref.c; this module only marshals arrays.
Sources for what is computed are cited there (TileLang tutorial chapter 11,
sections 1.1 and 3.6; the code/04 README's correctness criterion; the
"Stage 04 - GEMM" notes for the NN form).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16 = 0
BF16 = 1
_B_NK = 0
_B_KN = 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_decode.argtypes = [ctypes.c_uint16, ctypes.c_int]
        lib.oracle_decode.restype = ctypes.c_float
        lib.oracle_encode_rne.argtypes = [ctypes.c_float, ctypes.c_int]
        lib.oracle_encode_rne.restype = ctypes.c_uint16
        lib.oracle_decode_array.argtypes = [u16p, f32p, ctypes.c_int64, ctypes.c_int]
        lib.oracle_decode_array.restype = None
        lib.oracle_encode_array.argtypes = [f32p, u16p, ctypes.c_int64, ctypes.c_int]
        lib.oracle_encode_array.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_gemm_rows.argtypes = [u16p, u16p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int, u16p, f32p, i64p]
        lib.oracle_gemm_rows.restype = ctypes.c_int
        lib.oracle_gemm_points.argtypes = [u16p, u16p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_int, i64p, i64p, ctypes.c_int64,
                                           u16p, f32p]
        lib.oracle_gemm_points.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle matrices are uint16 encodings, got %s" % a.dtype)
    return a


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def decode(bits, dtype: int) -> np.ndarray:
    """Exact binary32 values of an array of 16-bit encodings."""
    bits = _u16(np.asarray(bits, dtype=np.uint16))
    out = np.empty(bits.shape, dtype=np.float32)
    _load().oracle_decode_array(_ptr(bits, ctypes.c_uint16), _ptr(out, ctypes.c_float), bits.size, dtype)
    return out


def encode(values, dtype: int) -> np.ndarray:
    """Round binary32 values to 16-bit encodings, ties to even."""
    values = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    out = np.empty(values.shape, dtype=np.uint16)
    _load().oracle_encode_array(_ptr(values, ctypes.c_float), _ptr(out, ctypes.c_uint16), values.size, dtype)
    return out


def _gemm_rows(A, B, b_layout, M, N, K, dtype, m_begin, m_end, want_sums, relu=False):
    A = _u16(A)
    B = _u16(B)
    if A.size != M * K or B.size != N * K:
        raise ValueError("operand sizes do not match M, N, K")
    rows = m_end - m_begin
    C = np.empty((rows, N), dtype=np.uint16)
    S = np.empty((rows, N), dtype=np.float32) if want_sums else None
    cnt = ctypes.c_int64(0)
    rc = _load().oracle_gemm_rows(_ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16), b_layout,
                                  M, N, K, dtype, m_begin, m_end, int(bool(relu)), _ptr(C, ctypes.c_uint16),
                                  _ptr(S, ctypes.c_float) if want_sums else None, ctypes.byref(cnt))
    if rc != 0:
        raise ValueError("oracle_gemm_rows rejected its arguments")
    return C, S, cnt.value


def gemm_nt(A, B, dtype: int, rows=None, return_sums=False, return_count=False, relu=False):
    """C = round(A[M,K] . B[N,K]^T) with ascending-k binary32 accumulation.

    rows=(m_begin, m_end) restricts the computation to those rows of C.
    relu=True applies the ReLU epilogue (s > 0 ? s : +0) to each binary32 sum
    before the rounding (TileLang tutorial, chapter 11, section 4.6).
    Returns C (and, on request, the binary32 sums and the multiply-add count).
    """
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    m0, m1 = rows if rows is not None else (0, M)
    C, S, cnt = _gemm_rows(A, B, _B_NK, M, N, K, dtype, m0, m1, return_sums, relu)
    out = (C,)
    if return_sums:
        out += (S,)
    if return_count:
        out += (cnt,)
    return out[0] if len(out) == 1 else out


def gemm_nn(A, B, dtype: int, rows=None, return_sums=False, return_count=False, relu=False):
    """C = round(A[M,K] . B[K,N]) with ascending-k binary32 accumulation
    (relu as for gemm_nt)."""
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    m0, m1 = rows if rows is not None else (0, M)
    C, S, cnt = _gemm_rows(A, B, _B_KN, M, N, K, dtype, m0, m1, return_sums, relu)
    out = (C,)
    if return_sums:
        out += (S,)
    if return_count:
        out += (cnt,)
    return out[0] if len(out) == 1 else out


def gemm_points(A, B, layout: str, dtype: int, rows, cols, return_sums=False, relu=False):
    """Elements C[rows[i], cols[i]], each as an ascending-k binary32 dot product.

    layout is "nt" (B [N,K]) or "nn" (B [K,N]); relu as for gemm_nt.
    """
    A = _u16(A)
    B = _u16(B)
    M, K = A.shape
    if layout == "nt":
        N = B.shape[0]
        b_layout = _B_NK
    elif layout == "nn":
        N = B.shape[1]
        b_layout = _B_KN
    else:
        raise ValueError("layout must be 'nt' or 'nn'")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in shape")
    C = np.empty(rows.shape, dtype=np.uint16)
    S = np.empty(rows.shape, dtype=np.float32)
    rc = _load().oracle_gemm_points(_ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16), b_layout,
                                    M, N, K, dtype, int(bool(relu)), _ptr(rows, ctypes.c_int64),
                                    _ptr(cols, ctypes.c_int64),
                                    rows.size, _ptr(C, ctypes.c_uint16), _ptr(S, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle_gemm_points rejected its arguments")
    return (C, S) if return_sums else C
