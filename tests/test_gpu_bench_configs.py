"""GPU parity at full size in every launch configuration the benchmark times:
each sweep point of bench.py (workload, tile, threads, ring depth, a_lead) and
the headline, on the benchmark's own seeded inputs, against the oracle on
sampled whole rows of C (tile-boundary rows and random ones, every column).

Within one sweep (same tile and thread count) every ring depth must also give
the same C bit for bit: the ring changes when tiles arrive, never the order
in which a wave accumulates.
"""
import numpy as np
import pytest

import bench
from software_pipelined_tiled_03_amd import binding as pg
from software_pipelined_tiled_03_amd import inputs

import attn_error_model as em
from test_gpu_parity import assert_close, dev, host, sample_rows

pytestmark = pytest.mark.gpu

H = bench.HEADLINE
POINTS = list(bench.SWEEPS) + [("headline", H["workload"], H["block"], H["threads"],
                                ("%d%s" % (H["num_stages"], "+A" if H["a_lead"] else ""),))]

_operands = {}


def _workload(name, og):
    """Seeded inputs on the device and the oracle's sampled rows, once per workload."""
    if name not in _operands:
        _operands.clear()
        w = inputs.workload(name)
        A, B = w.make()
        rows = sample_rows(w.M, 256, seed=len(name), extra=6)
        fn = og.gemm_nt if w.layout == "nt" else og.gemm_nn
        # a row of C depends only on the same row of A
        want = fn(np.ascontiguousarray(A[rows]), B, w.dtype)
        dA = dev(A, w.dtype).view(w.M, w.K)
        dB = dev(B, w.dtype).view(B.shape)
        _operands[name] = (w, dA, dB, rows, want)
    return _operands[name]


@pytest.mark.parametrize("point", POINTS, ids=lambda p: p[0])
def test_bench_configuration_full_size(oracle_gemm, point):
    label, wl, block, threads, depths = point
    w, dA, dB, rows, want = _workload(wl, oracle_gemm)
    fn = pg.gemm_nt if w.layout == "nt" else pg.gemm_nn
    first = None
    for d in depths:
        s, lead = bench.parse_depth(d)
        print("bench point %s %s S=%s" % (label, wl, d), flush=True)
        C = fn(dA, dB, block=block, num_stages=s, threads=threads, a_lead=lead)
        got = host(C)
        assert_close(got[rows], want, w.dtype, oracle_gemm, "%s S=%s" % (label, d))
        if first is None:
            first = got
        else:
            assert np.array_equal(got, first), "%s: S=%s changed the result" % (label, d)


@pytest.mark.parametrize("point", bench.ATTENTION, ids=lambda p: "%s_bm%d_bn%d_t%d" % ((p[0],) + p[1]))
def test_bench_attention_configuration_full_size(point):
    import torch

    from oracle import attention as oatt
    from oracle import gemm as og

    name, (bm, bn, th), depths = point
    w = inputs.attention_workload(name)
    Q, K, V = w.make()
    dQ, dK, dV = (dev(x, w.dtype) for x in (Q, K, V))
    rng = np.random.default_rng(bm + bn + th)
    picks = [(0, 0), (w.batch - 1, w.heads - 1), (w.batch // 2, 7)]
    rows = np.unique(np.concatenate([[0, 1, bm - 1, bm, w.seq_q - 1], rng.integers(0, w.seq_q, 6)]))
    want = {bh: oatt.attention_rows(Q, K, V, w.dtype, bh[0], bh[1], rows, causal=w.causal) for bh in picks}
    wts = {bh: oatt.attention_rows_weights(Q, K, V, w.dtype, bh[0], bh[1], rows, causal=w.causal) for bh in picks}
    first = None
    for s in depths:
        print("bench attention point %s bm%d bn%d t%d S=%d" % (name, bm, bn, th, s), flush=True)
        O = pg.attention(dQ, dK, dV, causal=w.causal, block_M=bm, block_N=bn, num_stages=s, threads=th)
        torch.cuda.synchronize()
        got = host(O)
        for (b, h), ref in want.items():
            g = og.decode(got[b, h, rows], w.dtype).astype(np.float64)
            assert np.isfinite(g).all(), "%s S=%d: non-finite output" % (name, s)
            R, A = wts[(b, h)]
            bad = em.violations(g, ref, R, A, w.dtype, w.seq_kv, ref.shape[-1])
            assert not bad.any(), "%s S=%d b=%d h=%d: %d elements outside the bound, max err %.3g" % (
                name, s, b, h, int(bad.sum()), np.abs(g - ref).max())
        if first is None:
            first = got
        else:
            assert np.array_equal(got, first), "%s: S=%d changed the result" % (name, s)
