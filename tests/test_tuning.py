"""Tuning front end on the CPU: the built configuration space, pre-pruning
against the oracle's budget rule and divisibility filter (TileLang tutorial,
chapter 11, section 3.7: 214 of 216 legal at 228 KiB for 4096^3), the wasted
spaces of section 5.3, and the gfx950 default table.  No device is touched
(every call passes an explicit LDS budget)."""
import itertools

import pytest

import software_pipelined_tiled_03_amd as pg
from oracle import budget as obudget
from software_pipelined_tiled_03_amd import binding as pb
from software_pipelined_tiled_03_amd import tuning as pt

MI355X = 160 * 1024
F16, BF16 = pg.GEMM_F16, pg.GEMM_BF16


def pages_grid():
    keys = ("block_M", "block_N", "block_K", "num_stages", "threads")
    return [dict(zip(keys, v)) for v in itertools.product((64, 128, 256), (64, 128, 256), (16, 32, 64),
                                                          (1, 2, 3, 4), (128, 256))]


def key(c):
    return (c["block_M"], c["block_N"], c["block_K"], c["num_stages"], c["threads"])


@pytest.mark.parametrize("layout,dtype", [("nt", F16), ("nn", BF16)])
def test_built_space_is_all_legal_where_tiles_divide(layout, dtype):
    cands = pg.built_configs(layout, dtype)
    assert len(cands) >= 50
    assert len({tuple(c.values()) for c in cands}) == len(cands)
    for c in cands:
        assert pg.gemm_lds_bytes(c["block_M"], c["block_N"], c["block_K"], c["num_stages"], dtype,
                                 a_lead=c["a_lead"]) <= MI355X
    status, legal = pg.prune(layout, 4096, 4096, 4096, dtype, cands, MI355X)
    assert legal == len(cands) and set(status) == {0}


@pytest.mark.parametrize("budget,rejected", [(obudget.H100_BUDGET, 2), (MI355X, 8)])
def test_prune_agrees_with_the_oracle_on_the_pages_grid(budget, rejected):
    grid = pages_grid()
    status, legal = pg.prune("nt", 4096, 4096, 4096, F16, pt.expand(grid, 4096, 4096, 4096), budget)
    _, olegal, orej = obudget.grid_configs(4096, 4096, 4096, budget)
    over = {key(c) for c, s in zip(grid, status) if s == pb.GEMM_ERR_LDS_BUDGET}
    assert over == {key(c) for c in orej} and len(over) == rejected
    within = {key(c) for c, s in zip(grid, status) if s != pb.GEMM_ERR_LDS_BUDGET}
    assert within == {key(c) for c in olegal}
    # what the budget allows but no kernel is built for (64-wide tiles, block_K 16) is not legal here
    assert all(s in (0, pb.GEMM_ERR_LDS_BUDGET, pb.GEMM_ERR_UNSUPPORTED) for s in status)
    assert 0 < legal < len(within)


def test_prune_drops_tiles_that_do_not_divide_first():
    grid = pages_grid()
    M, N, K = 4000, 5000, 3000
    status, _ = pg.prune("nt", M, N, K, F16, pt.expand(grid, M, N, K), obudget.H100_BUDGET)
    nodiv = {key(c) for c, s in zip(grid, status) if s == pt.GEMM_PRUNE_NODIV}
    want = {key(c) for c in grid if M % c["block_M"] or N % c["block_N"] or K % c["block_K"]}
    assert nodiv == want
    # 256x256x64 S4 does not divide 4000 either: it is dropped as not dividing, before the budget
    assert (256, 256, 64, 4, 256) in nodiv


def test_wasted_spaces_are_rejected_before_running():
    over = [dict(block_M=256, block_N=256, block_K=64, num_stages=s) for s in (3, 4)]
    with pytest.raises(pg.TuningSpaceError, match="infeasible"):
        pg.plan("nt", 4096, 4096, 4096, F16, over, MI355X)
    single = [dict(block_M=256, block_N=256, block_K=64, num_stages=2)]
    with pytest.raises(pg.TuningSpaceError, match="only one legal"):
        pg.plan("nt", 4096, 4096, 4096, F16, single, MI355X)
    cands, status = pg.plan("nt", 4096, 4096, 4096, F16, single, MI355X, allow_single=True)
    assert status == [0]
    with pytest.raises(ValueError, match="Unused keys in config"):
        pg.plan("nt", 4096, 4096, 4096, F16, [dict(block_M=128, num_stage=3)], MI355X)


def test_configs_may_be_a_function_of_the_problem():
    def space(M, N, K):
        return [dict(block_M=bm, block_N=bn, block_K=64, num_stages=s) for bm in (128, 256) for bn in (128, 256)
                for s in (2, 3) if M % bm == 0]
    cands, status = pg.plan("nt", 4096, 4096, 4096, F16, space, MI355X)
    assert len(cands) == 8
    # defaults fill the keys a candidate leaves out
    assert all(c["threads"] == 256 and c["a_lead"] == 0 for c in cands)
    # 256x256x64 at S3 is over 160 KiB
    assert sum(s == pb.GEMM_ERR_LDS_BUDGET for s in status) == 1


@pytest.mark.parametrize("shape", [(4096, 4096, 4096), (1024, 1024, 1024), (2048, 2048, 2048), (8192, 512, 1024),
                                   (4000, 5000, 3000), (512, 512, 65536), (128, 128, 128), (1, 1, 8),
                                   (16384, 16384, 512), (3072, 3072, 3072), (6144, 2048, 2048)])
@pytest.mark.parametrize("layout,dtype", [("nt", F16), ("nn", BF16)])
def test_default_config_is_a_built_legal_configuration(shape, layout, dtype):
    M, N, K = shape
    if layout == "nn" and N % 8:
        pytest.skip("the NN form needs N % 8 == 0")
    c = pg.default_config(layout, M, N, K, dtype)
    st = pg.gemm_check(0 if layout == "nt" else 1, M, N, K, dtype, c["block_M"], c["block_N"], c["block_K"],
                       c["num_stages"], c["threads"], MI355X, a_lead=c["a_lead"])
    assert st == 0, pg.last_error()
    # the cheapest of the per-tile table entries under the cost model
    table = [dict(block_M=256, block_N=256, block_K=64, num_stages=2, a_lead=1, threads=512),
             dict(block_M=256, block_N=128, block_K=64, num_stages=3, a_lead=0, threads=256),
             dict(block_M=128, block_N=256, block_K=64, num_stages=3, a_lead=0, threads=512),
             dict(block_M=128, block_N=128, block_K=64, num_stages=3, a_lead=0, threads=512),
             dict(block_M=64, block_N=128, block_K=64, num_stages=4, a_lead=0, threads=256)]
    costs = pt.model_costs(M, N, K, table)
    assert c == table[min(range(len(table)), key=lambda i: (costs[i], i))]


def test_default_config_of_the_headline_problem():
    assert pg.default_config("nt", 4096, 4096, 4096) == dict(block_M=256, block_N=256, block_K=64, num_stages=2,
                                                             a_lead=1, threads=512)
    assert pg.default_config("nt", 8192, 8192, 1024)["threads"] == 512
    assert pg.default_config("nt", 2048, 2048, 2048)["block_M"] == 128
    # the small grids (1024^3, long K on a 512 x 512 C) take the 64 x 128 tile
    assert pg.default_config("nt", 1024, 1024, 1024)["block_M"] == 64
    assert pg.default_config("nt", 512, 512, 65536)["block_M"] == 64


# ---------------------------------------------------------------------------
# The analytic cost model (gemm_rank; chapter 11, section 3.9: it orders the
# search, measurement decides).  The pages print no model, so these checks are
# of its arguments, its ordering contract, and the monotonicity its own
# definition implies; how well it orders real measurements is a GPU test.

def test_rank_rejects_bad_arguments():
    bad = dict(pt.DEFAULTS, threads=96)
    with pytest.raises(pb.GemmArgumentError):
        pt.model_costs(1024, 1024, 1024, [bad])
    with pytest.raises(pb.GemmArgumentError):
        pt.model_costs(-1, 1024, 1024, [dict(pt.DEFAULTS)])
    with pytest.raises(pb.GemmArgumentError):
        pt.model_costs(1024, 1024, 1024, [dict(pt.DEFAULTS, a_lead=2)])


@pytest.mark.parametrize("shape", [(4096, 4096, 4096), (2048, 2048, 2048), (1024, 1024, 8192), (128, 128, 128)])
def test_rank_orders_exactly_the_legal_candidates(shape):
    M, N, K = shape
    ranked = pg.rank("nt", M, N, K)
    status, legal = pg.prune("nt", M, N, K, F16, pg.built_configs("nt", F16), MI355X)
    assert len(ranked) == legal
    costs = [c for _, c in ranked]
    assert costs == sorted(costs) and all(c > 0 for c in costs)
    assert ranked == pg.rank("nt", M, N, K)   # deterministic


def test_rank_more_ring_depth_is_never_modelled_slower():
    # at one workgroup per compute unit (256x256 tiles); where a deeper ring
    # lowers the occupancy the model may rightly prefer the shallower one
    for tile, depths in [((256, 256, 32), range(1, 6)), ((256, 256, 64), range(1, 3))]:
        for threads in (256, 512):
            cfgs = [dict(block_M=tile[0], block_N=tile[1], block_K=tile[2], num_stages=s, a_lead=0, threads=threads)
                    for s in depths]
            costs = pt.model_costs(4096, 4096, 4096, cfgs)
            assert all(b <= a for a, b in zip(costs, costs[1:])), (tile, threads, costs)
            assert costs[0] > costs[1]   # S = 1 serialises copy, latency and compute


def test_rank_scales_with_the_problem():
    c = dict(block_M=256, block_N=256, block_K=64, num_stages=2, a_lead=1, threads=512)
    a, b = pt.model_costs(4096, 4096, 4096, [c])[0], pt.model_costs(4096, 4096, 8192, [c])[0]
    assert 1.9 < b / a < 2.05          # twice the K tiles, the same fixed store and launch
    w1, w2 = pt.model_costs(4096, 4096, 4096, [c])[0], pt.model_costs(8192, 4096, 4096, [c])[0]
    assert 1.95 < w2 / w1 < 2.05       # twice the rounds of workgroups


def test_rank_first_choice_at_4096_is_the_measured_fastest():
    # the measured winner of the 4096^3 fp16 NT tuning table on MI355X
    assert pg.rank("nt", 4096, 4096, 4096)[0][0] == pg.default_config("nt", 4096, 4096, 4096)
