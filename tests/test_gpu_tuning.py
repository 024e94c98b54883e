"""GPU tests of the tuning front end: every legal candidate of the built space
runs on the same operands, the winner's C matches the oracle, and every
candidate writes the same C bit for bit (the accumulation order over K does
not depend on the configuration)."""
import numpy as np
import pytest
import torch

import software_pipelined_tiled_03_amd as pg
from software_pipelined_tiled_03_amd import inputs
from software_pipelined_tiled_03_amd import tuning as pt

pytestmark = pytest.mark.gpu

F16, BF16 = inputs.F16, inputs.BF16
TORCH_DT = {F16: torch.float16, BF16: torch.bfloat16}


def dev(u16, dtype):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(TORCH_DT[dtype])


def host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def close(got, want, dtype, og):
    g = og.decode(got, dtype).astype(np.float64)
    w = og.decode(want, dtype).astype(np.float64)
    return bool((np.abs(g - w) <= 1e-2 + 1e-2 * np.abs(w)).all())


@pytest.mark.parametrize("layout,dtype", [("nt", F16), ("nn", BF16)])
def test_tune_full_space_1024(oracle_gemm, layout, dtype):
    M = N = K = 1024
    w = inputs.custom(layout, dtype, M, N, K, seed=77 + dtype)
    A, B = w.make()
    dA, dB = dev(A, dtype).view(M, K), dev(B, dtype).view(B.shape)
    res = pg.tune(dA, dB, layout, warmup=2, reps=5)
    torch.cuda.synchronize()
    legal = [(c, ms) for c, s, ms in res.table if s == 0]
    assert len(legal) == len(pg.built_configs(layout, dtype))
    assert all(ms is not None and ms > 0 for _, ms in legal)
    assert res.latency == min(ms for _, ms in legal) and res.config in [c for c, _ in legal]
    want = (oracle_gemm.gemm_nt if layout == "nt" else oracle_gemm.gemm_nn)(A, B, dtype)
    fn = pg.gemm_nt if layout == "nt" else pg.gemm_nn
    first = None
    for c, _ in legal:
        out = fn(dA, dB, block=(c["block_M"], c["block_N"], c["block_K"]), num_stages=c["num_stages"],
                 threads=c["threads"], a_lead=c["a_lead"])
        got = host(out)
        if first is None:
            first = got
            assert close(got, want, dtype, oracle_gemm), "first candidate %s" % c
        else:
            assert np.array_equal(got, first), "candidate %s wrote a different C" % c


def test_tune_writes_c_and_reports_pruned_candidates(oracle_gemm):
    M = N = K = 1024
    w = inputs.workload("nt_f16_1024")
    A, B = w.make()
    dA, dB = dev(A, F16).view(M, K), dev(B, F16).view(N, K)
    space = [dict(block_M=256, block_N=256, block_K=64, num_stages=s, a_lead=l) for s in (1, 2, 3) for l in (0, 1)]
    out = torch.full((M, N), 9.0, dtype=torch.float16, device="cuda")
    res = pg.tune(dA, dB, "nt", configs=space, warmup=1, reps=3, out=out)
    torch.cuda.synchronize()
    status = [s for _, s, _ in res.table]
    # S=1 with a_lead is an argument error; S=3 is over 160 KiB with or without the lead tile
    assert status == [0, pg.binding.GEMM_ERR_ARG, 0, 0, pg.binding.GEMM_ERR_LDS_BUDGET,
                      pg.binding.GEMM_ERR_LDS_BUDGET]
    assert [ms is None for _, _, ms in res.table] == [False, True, False, False, True, True]
    assert close(host(out), oracle_gemm.gemm_nt(A, B, F16), F16, oracle_gemm)


def test_ragged_problem_has_no_dividing_tile():
    # the tutorial's pre-pruning drops tiles that do not divide the problem: no built tile divides 4000
    dA = torch.empty((4000, 3000), dtype=torch.float16, device="cuda")
    dB = torch.empty((5000, 3000), dtype=torch.float16, device="cuda")
    with pytest.raises(pg.TuningSpaceError, match="infeasible"):
        pg.tune(dA, dB, "nt")


def test_matmul_tunes_once_then_reuses(monkeypatch, oracle_gemm):
    M = N = K = 1024
    w = inputs.workload("nt_f16_1024")
    A, B = w.make()
    dA, dB = dev(A, F16).view(M, K), dev(B, F16).view(N, K)
    calls = []
    real = pt.tune

    def counting(*a, **k):
        calls.append(1)
        return real(*a, **k)

    monkeypatch.setattr(pt, "tune", counting)
    pt._tuned.clear()
    c1 = host(pg.matmul(dA, dB, "nt", autotune=True))
    c2 = host(pg.matmul(dA, dB, "nt", autotune=True))
    c3 = host(pg.matmul(dA, dB, "nt", autotune=False))
    assert len(calls) == 1
    assert np.array_equal(c1, c2) and np.array_equal(c1, c3)
    assert close(c1, oracle_gemm.gemm_nt(A, B, F16), F16, oracle_gemm)


def test_tune_top_measures_only_the_models_choice(oracle_gemm):
    M = N = K = 1024
    w = inputs.custom("nt", F16, M, N, K, seed=91)
    A, B = w.make()
    dA, dB = dev(A, F16).view(M, K), dev(B, F16).view(N, K)
    res = pg.tune(dA, dB, "nt", warmup=2, reps=5, top=6)
    measured = [(c, ms) for c, s, ms in res.table if s == 0]
    ranked_out = [c for c, s, _ in res.table if s == pt.RANKED_OUT]
    assert len(measured) == 6 and all(ms > 0 for _, ms in measured)
    top6 = [c for c, _ in pg.rank("nt", M, N, K)[:6]]
    assert sorted(map(str, (c for c, _ in measured))) == sorted(map(str, top6))
    assert len(ranked_out) == len(pg.rank("nt", M, N, K)) - 6
    assert res.config in top6


def test_rank_orders_a_measured_table():
    # a cheap shape: the model's first choice is within 15 % of the measured best
    M, N, K = 4096, 4096, 512
    A = (torch.rand(M, K, device="cuda") * 2 - 1).half()
    B = (torch.rand(N, K, device="cuda") * 2 - 1).half()
    # an 18 us kernel: enough launches per candidate (about 1 ms) that power
    # management transitions do not decide the ordering
    res = pg.tune(A, B, "nt", warmup=20, reps=60)
    measured = {str(c): ms for c, s, ms in res.table if s == 0}
    first = pg.rank("nt", M, N, K)[0][0]
    assert measured[str(first)] <= 1.15 * res.latency, (first, measured[str(first)], res.config, res.latency)
