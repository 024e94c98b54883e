"""Configuration space, pre-pruning and tuning of the pipelined GEMM.

The TileLang tutorial's tuning workflow (chapter 11, sections 3.5-3.8, 5.3):
a configuration space given as a list or as a function of the problem size;
candidates pre-pruned of tiles that do not divide the problem and of
over-budget combinations; "wasted" spaces (every candidate infeasible, or a
single legal one that leaves nothing to rank, or keys the kernel does not
take) reported before anything runs; every candidate measured on the same
operands; and the result fixed as a per-device default, with a switch that
turns tuning off.

The enumeration, pruning, timing and the gfx950 default table run in the
C-ABI library (gemm_configs, gemm_prune, gemm_tune, gemm_default_config);
this module turns config dicts into gemm_config records and back.
"""
import ctypes

from . import binding as _b

#: The tuned parameters and their defaults (the tutorial's kernel signature
#: defaults for the first five; threads 256 is this library's default).
DEFAULTS = dict(block_M=128, block_N=128, block_K=32, num_stages=3, a_lead=0, threads=256)
_FIELDS = ("block_M", "block_N", "block_K", "num_stages", "a_lead", "threads")
GEMM_PRUNE_NODIV = 16
#: status of a legal candidate that the cost model ranked below the measured top
RANKED_OUT = 17
STATUS_TEXT = {_b.GEMM_OK: "ok", GEMM_PRUNE_NODIV: "tile does not divide the problem",
               RANKED_OUT: "ranked below the measured top by the cost model",
               _b.GEMM_ERR_LDS_BUDGET: "over the LDS budget", _b.GEMM_ERR_UNSUPPORTED: "no kernel built",
               _b.GEMM_ERR_ALIGN: "misaligned", _b.GEMM_ERR_ARG: "bad argument"}


class GemmConfig(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in _FIELDS]


class TuningSpaceError(ValueError):
    """The configuration space cannot be tuned (every candidate infeasible, or
    only one legal candidate)."""


_declared = False


def _lib():
    global _declared
    lib = _b.load()
    if not _declared:
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        pc = ctypes.POINTER(GemmConfig)
        lib.gemm_configs.argtypes = [i32, i32, pc, i32]
        lib.gemm_configs.restype = i32
        lib.gemm_prune.argtypes = [i32, i64, i64, i64, i32, pc, i32, i64, ctypes.POINTER(i32)]
        lib.gemm_prune.restype = i32
        lib.gemm_tune.argtypes = [i32, vp, vp, vp, i64, i64, i64, i32, pc, ctypes.POINTER(i32), i32, i32, i32, vp,
                                  ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
        lib.gemm_tune.restype = i32
        lib.gemm_default_config.argtypes = [i32, i64, i64, i64, i32, pc]
        lib.gemm_default_config.restype = i32
        lib.gemm_rank.argtypes = [i64, i64, i64, pc, i32, ctypes.POINTER(ctypes.c_double)]
        lib.gemm_rank.restype = i32
        _declared = True
    return lib


def _as_dict(c):
    return {f: int(getattr(c, f)) for f in _FIELDS}


def _layout_code(layout):
    if layout in (_b.GEMM_NT, "nt", "NT"):
        return _b.GEMM_NT
    if layout in (_b.GEMM_NN, "nn", "NN"):
        return _b.GEMM_NN
    raise ValueError("layout must be 'nt' or 'nn', got %r" % (layout,))


def built_configs(layout="nt", dtype=_b.GEMM_F16):
    """Every configuration the library has a kernel for (gemm_configs)."""
    lib = _lib()
    lc = _layout_code(layout)
    n = lib.gemm_configs(lc, dtype, None, 0)
    if n < 0:
        raise _b.GemmArgumentError(_b.GEMM_ERR_ARG, _b.last_error())
    arr = (GemmConfig * n)()
    lib.gemm_configs(lc, dtype, arr, n)
    return [_as_dict(c) for c in arr]


def default_config(layout, M, N, K, dtype=_b.GEMM_F16):
    """The configuration used without tuning on gfx950 (gemm_default_config)."""
    c = GemmConfig()
    st = _lib().gemm_default_config(_layout_code(layout), M, N, K, dtype, ctypes.byref(c))
    _b._raise_for(st)
    return _as_dict(c)


def expand(configs, M, N, K):
    """The candidate list: `configs` may be a list of dicts or a callable
    taking (M, N, K) and returning one (chapter 11, section 3.5).  Missing keys
    take DEFAULTS; a key the kernel does not take is an error (section 5.3)."""
    if callable(configs):
        configs = configs(M, N, K)
    out = []
    for c in configs:
        unused = set(c) - set(_FIELDS)
        if unused:
            raise ValueError("Unused keys in config: %s" % sorted(unused))
        d = dict(DEFAULTS)
        d.update({k: int(v) for k, v in c.items()})
        out.append(d)
    return out


def prune(layout, M, N, K, dtype, configs, lds_budget=0):
    """Pre-prune (gemm_prune): returns a status code per candidate and the
    number left legal.  lds_budget 0 = the current device's."""
    n = len(configs)
    arr = (GemmConfig * max(n, 1))(*[GemmConfig(*[c[f] for f in _FIELDS]) for c in configs])
    status = (ctypes.c_int32 * max(n, 1))()
    legal = _lib().gemm_prune(_layout_code(layout), M, N, K, dtype, arr, n, lds_budget, status)
    if legal < 0:
        raise _b.GemmArgumentError(_b.GEMM_ERR_ARG, _b.last_error())
    return [int(status[i]) for i in range(n)], legal


def model_costs(M, N, K, configs):
    """The analytic cost (gemm_rank, modelled microseconds) of each config."""
    n = len(configs)
    arr = (GemmConfig * max(n, 1))(*[GemmConfig(*[c[f] for f in _FIELDS]) for c in configs])
    cost = (ctypes.c_double * max(n, 1))()
    _b._raise_for(_lib().gemm_rank(M, N, K, arr, n, cost))
    return [float(cost[i]) for i in range(n)]


def rank(layout, M, N, K, dtype=_b.GEMM_F16, configs=None, lds_budget=163840):
    """The legal candidates ordered by the cost model, cheapest first, as
    (config, modelled microseconds) pairs (chapter 11, section 3.9: the model
    orders the search; equal costs mean it cannot tell them apart and only
    measurement can).  Pure host with the default budget (gfx950's 160 KiB);
    lds_budget 0 takes the current device's."""
    cands = expand(built_configs(layout, dtype) if configs is None else configs, M, N, K)
    status, _ = prune(layout, M, N, K, dtype, cands, lds_budget)
    legal = [c for c, s in zip(cands, status) if s == _b.GEMM_OK]
    costs = model_costs(M, N, K, legal)
    order = sorted(range(len(legal)), key=lambda i: (costs[i], i))
    return [(legal[i], costs[i]) for i in order]


def plan(layout, M, N, K, dtype, configs=None, lds_budget=0, allow_single=False):
    """Expand and pre-prune the space, and reject a wasted one before anything
    runs (chapter 11, section 5.3).  Returns (candidates, statuses)."""
    cands = expand(built_configs(layout, dtype) if configs is None else configs, M, N, K)
    status, legal = prune(layout, M, N, K, dtype, cands, lds_budget)
    if legal == 0:
        why = {}
        for s in status:
            why[STATUS_TEXT.get(s, s)] = why.get(STATUS_TEXT.get(s, s), 0) + 1
        raise TuningSpaceError("every candidate is infeasible (%d requested: %s)" % (len(cands), why))
    if legal == 1 and not allow_single:
        raise TuningSpaceError("only one legal configuration: tuning cannot rank anything")
    return cands, status


class TuneResult:
    """The tutorial's AutotuneResult: the winning config, its latency, and the
    whole table (config, status, ms) for inspection."""

    def __init__(self, config, latency_ms, table):
        self.config = config
        self.latency = latency_ms
        self.table = table

    def __repr__(self):
        return "TuneResult(config=%r, latency=%.4f ms, %d candidates)" % (self.config, self.latency,
                                                                        len(self.table))


def tune(A, B, layout="nt", configs=None, warmup=25, reps=100, out=None, stream=None, allow_single=False, top=None):
    """Measure every legal candidate on A, B (device tensors) and return the
    fastest (gemm_tune).  out receives C (every candidate writes the same C).

    top=k measures only the k legal candidates the cost model ranks cheapest
    (gemm_rank); the others are reported with status RANKED_OUT."""
    import torch

    lc = _layout_code(layout)
    if A.dim() != 2 or B.dim() != 2 or not (A.is_cuda and B.is_cuda) or A.dtype != B.dtype:
        raise _b.GemmArgumentError(_b.GEMM_ERR_ARG, "A and B must be 2-D device tensors of one dtype")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise _b.GemmArgumentError(_b.GEMM_ERR_ARG, "A and B must be contiguous row-major")
    M, K = A.shape
    N = B.shape[0] if lc == _b.GEMM_NT else B.shape[1]
    if (B.shape[1] if lc == _b.GEMM_NT else B.shape[0]) != K:
        raise _b.GemmArgumentError(_b.GEMM_ERR_ARG, "inner dimensions differ")
    dtype = _b._dtype_code(A)
    cands, status = plan(lc, M, N, K, dtype, configs, 0, allow_single)
    if top is not None:
        if int(top) < 1:
            raise ValueError("top must be at least 1")
        legal = [i for i, s in enumerate(status) if s == _b.GEMM_OK]
        costs = model_costs(M, N, K, [cands[i] for i in legal])
        keep = set(legal[j] for j in sorted(range(len(legal)), key=lambda j: (costs[j], j))[:int(top)])
        status = [s if (s != _b.GEMM_OK or i in keep) else RANKED_OUT for i, s in enumerate(status)]
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    elif out.shape != (M, N) or out.dtype != A.dtype or not out.is_contiguous() or out.device != A.device:
        raise _b.GemmArgumentError(_b.GEMM_ERR_ARG, "out must be a contiguous (M, N) tensor of A's dtype and device")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    n = len(cands)
    arr = (GemmConfig * n)(*[GemmConfig(*[c[f] for f in _FIELDS]) for c in cands])
    st_arr = (ctypes.c_int32 * n)(*status)
    ms = (ctypes.c_float * n)()
    best = ctypes.c_int32(-1)
    with torch.cuda.device(A.device):
        st = _lib().gemm_tune(lc, A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, dtype, arr, st_arr, n,
                              warmup, reps, stream, ms, ctypes.byref(best))
    _b._raise_for(st)
    table = [(cands[i], status[i], float(ms[i]) if status[i] == _b.GEMM_OK else None) for i in range(n)]
    return TuneResult(cands[best.value], float(ms[best.value]), table)


def time_config(A, B, config, layout="nt", warmup=5, reps=30, out=None, stream=None):
    """Mean milliseconds per launch of one configuration on A, B, timed by the
    library's own loop (gemm_tune with a single candidate: `warmup`
    launches, then `reps` back-to-back launches between two HIP events), so a
    small problem measures its kernels rather than the host's per-call cost.
    The tile need not divide the problem (edge tiles are masked)."""
    import torch

    lc = _layout_code(layout)
    M, K = A.shape
    N = B.shape[0] if lc == _b.GEMM_NT else B.shape[1]
    c = dict(DEFAULTS, **config)
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    arr = (GemmConfig * 1)(GemmConfig(*[c[f] for f in _FIELDS]))
    st_arr = (ctypes.c_int32 * 1)(_b.GEMM_OK)
    ms = (ctypes.c_float * 1)()
    best = ctypes.c_int32(-1)
    with torch.cuda.device(A.device):
        st = _lib().gemm_tune(lc, A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, _b._dtype_code(A), arr, st_arr,
                              1, warmup, reps, stream, ms, ctypes.byref(best))
    _b._raise_for(st)
    return float(ms[0])


_tuned = {}


def matmul(A, B, layout="nt", autotune=False, out=None, stream=None, relu=False):
    """C = A @ B^T (layout 'nt', B [N,K]) or A @ B ('nn', B [K,N]); relu=True
    fuses ReLU into the store.

    autotune=False uses default_config (the fixed gfx950 table).  autotune=True
    tunes once per (layout, M, N, K, dtype) in this process and then reuses the
    winner: the first call pays for the search, later calls do not
    (chapter 11, section 3.8)."""
    lc = _layout_code(layout)
    M, K = A.shape
    N = B.shape[0] if lc == _b.GEMM_NT else B.shape[1]
    dtype = _b._dtype_code(A)
    if autotune:
        key = (lc, M, N, K, dtype)
        if key not in _tuned:
            _tuned[key] = tune(A, B, lc, warmup=3, reps=10, out=out, stream=stream).config
        cfg = _tuned[key]
    else:
        cfg = default_config(lc, M, N, K, dtype)
    fn = _b.gemm_nt if lc == _b.GEMM_NT else _b.gemm_nn
    return fn(A, B, out=out, block=(cfg["block_M"], cfg["block_N"], cfg["block_K"]), num_stages=cfg["num_stages"],
              threads=cfg["threads"], stream=stream, a_lead=cfg["a_lead"], relu=relu)
