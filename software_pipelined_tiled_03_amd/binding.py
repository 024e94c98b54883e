"""Python binding of the C-ABI library declared in include/pipegemm.h.

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  The library
must have been built (software_pipelined_tiled_03_amd/build.py); if it is
missing, every call raises -- there is no fallback path.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libpipegemm.so")

GEMM_F16 = 0
GEMM_BF16 = 1
GEMM_NT = 0
GEMM_NN = 1

GEMM_OK = 0
GEMM_ERR_ARG = 1
GEMM_ERR_LDS_BUDGET = 2
GEMM_ERR_UNSUPPORTED = 3
GEMM_ERR_ALIGN = 4
GEMM_ERR_HIP = 5

STATUS_NAMES = {GEMM_OK: "GEMM_OK", GEMM_ERR_ARG: "GEMM_ERR_ARG", GEMM_ERR_LDS_BUDGET: "GEMM_ERR_LDS_BUDGET",
                GEMM_ERR_UNSUPPORTED: "GEMM_ERR_UNSUPPORTED", GEMM_ERR_ALIGN: "GEMM_ERR_ALIGN",
                GEMM_ERR_HIP: "GEMM_ERR_HIP"}


class GemmError(Exception):
    """Base class; .status holds the gemm_status code."""

    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


class GemmArgumentError(GemmError, ValueError):
    pass


class LdsBudgetError(GemmError, ValueError):
    """num_stages x (block_M + block_N) x block_K x 2 bytes exceeds the LDS limit."""


class UnsupportedConfigError(GemmError, ValueError):
    pass


class AlignmentError(GemmError, ValueError):
    pass


class GemmHipError(GemmError, RuntimeError):
    pass


_EXC = {GEMM_ERR_ARG: GemmArgumentError, GEMM_ERR_LDS_BUDGET: LdsBudgetError,
        GEMM_ERR_UNSUPPORTED: UnsupportedConfigError, GEMM_ERR_ALIGN: AlignmentError, GEMM_ERR_HIP: GemmHipError}

_lib = None


def load():
    """Load the C-ABI library (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("pipegemm library not built: %s is missing "
                           "(run `python software_pipelined_tiled_03_amd/build.py`)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    for name in ("gemm_nt", "gemm_nn", "gemm_nt_relu", "gemm_nn_relu"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32, i32, vp]
        f.restype = i32
    lib.gemm_stamped.argtypes = [i32, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.gemm_stamped.restype = i32
    lib.gemm_lds_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.gemm_lds_bytes.restype = i64
    lib.gemm_lds_budget.argtypes = []
    lib.gemm_lds_budget.restype = i64
    lib.gemm_check.argtypes = [i32, i64, i64, i64, i32, i32, i32, i32, i32, i32, i32, i64]
    lib.gemm_check.restype = i32
    lib.gemm_last_error.argtypes = []
    lib.gemm_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().gemm_last_error().decode()


def _raise_for(status):
    if status != GEMM_OK:
        raise _EXC.get(status, GemmError)(status, last_error())


# --- raw C-ABI mirrors (same names and arguments as the header) -------------

def gemm_nt_raw(A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads, hip_stream):
    """gemm_nt on raw device addresses; returns the status code."""
    return load().gemm_nt(A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                          hip_stream)


def gemm_nn_raw(A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads, hip_stream):
    """gemm_nn on raw device addresses; returns the status code."""
    return load().gemm_nn(A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                          hip_stream)


def gemm_nt_relu_raw(A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads, hip_stream):
    """gemm_nt_relu on raw device addresses; returns the status code."""
    return load().gemm_nt_relu(A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                               hip_stream)


def gemm_nn_relu_raw(A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads, hip_stream):
    """gemm_nn_relu on raw device addresses; returns the status code."""
    return load().gemm_nn_relu(A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                               hip_stream)


def gemm_stamped_raw(layout, A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                     hip_stream, stamps):
    """gemm_stamped on raw device addresses; returns the status code."""
    return load().gemm_stamped(layout, A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead,
                               threads, hip_stream, stamps)


def gemm_lds_bytes(block_M, block_N, block_K, num_stages, dtype=GEMM_F16, a_lead=0) -> int:
    return int(load().gemm_lds_bytes(block_M, block_N, block_K, num_stages, a_lead, dtype))


def gemm_lds_budget() -> int:
    v = int(load().gemm_lds_budget())
    if v < 0:
        raise GemmHipError(GEMM_ERR_HIP, last_error())
    return v


def gemm_check(layout, M, N, K, dtype, block_M, block_N, block_K, num_stages, threads, lds_budget, a_lead=0) -> int:
    """Validation only (status code); lds_budget > 0 touches no device."""
    return int(load().gemm_check(layout, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                                 lds_budget))


# --- torch convenience wrappers --------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return GEMM_F16
    if t.dtype == torch.bfloat16:
        return GEMM_BF16
    raise GemmArgumentError(GEMM_ERR_ARG, "dtype must be float16 or bfloat16, got %s" % t.dtype)


def _gemm(layout, A, B, out, block, num_stages, threads, stream, a_lead, relu=False, stamps=None):
    import torch
    if A.dim() != 2 or B.dim() != 2:
        raise GemmArgumentError(GEMM_ERR_ARG, "A and B must be 2-D")
    if not (A.is_cuda and B.is_cuda):
        raise GemmArgumentError(GEMM_ERR_ARG, "A and B must be device tensors")
    if A.device != B.device:
        raise GemmArgumentError(GEMM_ERR_ARG, "A and B are on different devices (%s, %s)" % (A.device, B.device))
    if not (A.is_contiguous() and B.is_contiguous()):
        raise GemmArgumentError(GEMM_ERR_ARG, "A and B must be contiguous row-major")
    if A.dtype != B.dtype:
        raise GemmArgumentError(GEMM_ERR_ARG, "A and B dtypes differ")
    M, K = A.shape
    if layout == GEMM_NT:
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K:
        raise GemmArgumentError(GEMM_ERR_ARG, "inner dimensions differ: %d vs %d" % (K, Kb))
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    elif (out.shape != (M, N) or out.dtype != A.dtype or not out.is_contiguous() or out.device != A.device):
        raise GemmArgumentError(GEMM_ERR_ARG, "out must be a contiguous (M, N) tensor of A's dtype and device")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    bm, bn, bk = block
    lib = load()
    if relu:
        fn = lib.gemm_nt_relu if layout == GEMM_NT else lib.gemm_nn_relu
    else:
        fn = lib.gemm_nt if layout == GEMM_NT else lib.gemm_nn
    with torch.cuda.device(A.device):
        if stamps is not None:
            st = lib.gemm_stamped(layout, A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, _dtype_code(A), bm, bn,
                                  bk, num_stages, int(a_lead), threads, stream, stamps.data_ptr())
        else:
            st = fn(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, _dtype_code(A), bm, bn, bk, num_stages,
                    int(a_lead), threads, stream)
    _raise_for(st)
    return out


def gemm_stamped(layout, A, B, out=None, block=(128, 128, 32), num_stages=3, threads=256, stream=None, a_lead=0,
                 stamps=None):
    """gemm_nt / gemm_nn (layout GEMM_NT / GEMM_NN) that also writes six clock
    counters per workgroup into `stamps` (an int64 device tensor of at least
    6 x grid elements; allocated when None).  Returns (C, stamps)."""
    import torch
    M, K = A.shape
    N = B.shape[0] if layout == GEMM_NT else B.shape[1]
    grid = -(-M // block[0]) * -(-N // block[1])
    if stamps is None:
        stamps = torch.zeros(6 * grid, dtype=torch.int64, device=A.device)
    elif (stamps.dtype != torch.int64 or not stamps.is_contiguous() or stamps.numel() < 6 * grid
          or stamps.device != A.device):
        raise GemmArgumentError(GEMM_ERR_ARG, "stamps must be a contiguous int64 device tensor of >= 6 x grid values")
    out = _gemm(layout, A, B, out, block, num_stages, threads, stream, a_lead, stamps=stamps)
    return out, stamps


def gemm_nt(A, B, out=None, block=(128, 128, 32), num_stages=3, threads=256, stream=None, a_lead=0, relu=False):
    """C = A[M,K] @ B[N,K]^T on the GPU (fp16/bf16 in, fp32 accumulate, C in A's dtype);
    relu=True fuses ReLU into the store (gemm_nt_relu)."""
    return _gemm(GEMM_NT, A, B, out, block, num_stages, threads, stream, a_lead, relu)


def gemm_nn(A, B, out=None, block=(128, 128, 32), num_stages=3, threads=256, stream=None, a_lead=0, relu=False):
    """C = A[M,K] @ B[K,N] on the GPU (fp16/bf16 in, fp32 accumulate, C in A's dtype);
    relu=True fuses ReLU into the store (gemm_nn_relu)."""
    return _gemm(GEMM_NN, A, B, out, block, num_stages, threads, stream, a_lead, relu)


# --- attention (include/pipeattn.h) -------------------------------------------

_attn_declared = False


def _attn_lib():
    global _attn_declared
    lib = load()
    if not _attn_declared:
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, ctypes.c_float, i32, i32,
                                 i32, i32, vp]
        lib.attn_fwd.restype = i32
        lib.attn_lds_bytes.argtypes = [i32, i32, i32]
        lib.attn_lds_bytes.restype = i64
        lib.attn_check.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, i32, i32, i32, i32, i64]
        lib.attn_check.restype = i32
        ip = ctypes.POINTER(i32)
        lib.attn_default_config.argtypes = [i64, i64, i64, i64, i32, ip, ip, ip, ip]
        lib.attn_default_config.restype = i32
        _attn_declared = True
    return lib


def attn_fwd_raw(Q, K, V, O, batch, heads, kv_heads, seq_q, seq_kv, dim, dtype, is_causal, scale, block_M, block_N,
                 num_stages, threads, hip_stream):
    """attn_fwd on raw device addresses; returns the status code."""
    return _attn_lib().attn_fwd(Q, K, V, O, batch, heads, kv_heads, seq_q, seq_kv, dim, dtype, is_causal, scale,
                                block_M, block_N, num_stages, threads, hip_stream)


def attn_lds_bytes(block_N, dim, num_stages) -> int:
    return int(_attn_lib().attn_lds_bytes(block_N, dim, num_stages))


def attn_check(batch, heads, kv_heads, seq_q, seq_kv, dim, dtype, is_causal, block_M, block_N, num_stages, threads,
               lds_budget) -> int:
    """Validation only (status code); lds_budget > 0 touches no device."""
    return int(_attn_lib().attn_check(batch, heads, kv_heads, seq_q, seq_kv, dim, dtype, is_causal, block_M,
                                      block_N, num_stages, threads, lds_budget))


def attn_default_config(batch, heads, seq_q, dim, is_causal):
    """(block_M, block_N, num_stages, threads) of the gfx950 default table
    for these sizes (attn_default_config in include/pipeattn.h)."""
    out = [ctypes.c_int32() for _ in range(4)]
    st = _attn_lib().attn_default_config(batch, heads, seq_q, dim, int(is_causal), *[ctypes.byref(x) for x in out])
    _raise_for(st)
    return tuple(x.value for x in out)


def attention(Q, K, V, causal=False, scale=0.0, out=None, block_M=None, block_N=None, num_stages=None, threads=None,
              stream=None):
    """O = softmax(scale Q K^T [causal]) V on the GPU.  Q [B, H, Sq, D], K and V
    [B, Hkv, Skv, D] contiguous fp16/bf16 device tensors; O like Q.  With
    block_M left at None the tile comes from attn_default_config for these
    sizes (block_N, num_stages and threads, if given, still apply); with
    block_M given, the others default to 64 keys, 2 stages and one 32-query
    block per wave."""
    import torch
    if Q.dim() != 4 or K.dim() != 4 or V.dim() != 4:
        raise GemmArgumentError(GEMM_ERR_ARG, "Q, K and V must be 4-D [batch, heads, seq, dim]")
    if not (Q.is_cuda and K.is_cuda and V.is_cuda):
        raise GemmArgumentError(GEMM_ERR_ARG, "Q, K and V must be device tensors")
    if not (Q.device == K.device == V.device):
        raise GemmArgumentError(GEMM_ERR_ARG, "Q, K and V are not all on one device")
    if not (Q.is_contiguous() and K.is_contiguous() and V.is_contiguous()):
        raise GemmArgumentError(GEMM_ERR_ARG, "Q, K and V must be contiguous")
    if not (Q.dtype == K.dtype == V.dtype):
        raise GemmArgumentError(GEMM_ERR_ARG, "Q, K and V dtypes differ")
    B, H, Sq, D = Q.shape
    if K.shape != V.shape or K.shape[0] != B or K.shape[3] != D:
        raise GemmArgumentError(GEMM_ERR_ARG, "K and V must be [batch, kv_heads, seq_kv, dim] matching Q")
    Hkv, Skv = K.shape[1], K.shape[2]
    dflt = attn_default_config(B, H, Sq, D, causal) if block_M is None else (block_M, 64, 2, 0)
    block_M, block_N, num_stages, threads = (d if v is None else v
                                             for v, d in zip((block_M, block_N, num_stages, threads), dflt))
    if out is None:
        out = torch.empty_like(Q)
    elif out.shape != Q.shape or out.dtype != Q.dtype or not out.is_contiguous() or out.device != Q.device:
        raise GemmArgumentError(GEMM_ERR_ARG, "out must be a contiguous tensor shaped like Q")
    if stream is None:
        stream = torch.cuda.current_stream(Q.device).cuda_stream
    with torch.cuda.device(Q.device):
        st = attn_fwd_raw(Q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr(), B, H, Hkv, Sq, Skv, D,
                          _dtype_code(Q), int(bool(causal)), float(scale), block_M, block_N, num_stages, threads,
                          stream)
    _raise_for(st)
    return out
