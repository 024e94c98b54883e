"""Pins for the oracle's on-chip budget arithmetic against the pages' worked
examples (tests/golden/budget_228kib.txt)."""
from oracle import budget
from tests.conftest import golden_lines


def _golden():
    return golden_lines("budget_228kib.txt")


def test_budget_value_is_228_kib():
    (b,) = [int(r[1]) for r in _golden() if r[0] == "budget"]
    assert b == budget.H100_BUDGET == 233472


def test_per_stage_and_max_stages():
    for r in _golden():
        if r[0] == "per_stage":
            bm, bn, bk, want = map(int, r[1:])
            assert budget.stage_bytes(bm, bn, bk) == want
        if r[0] == "max_stages":
            bm, bn, bk, want = map(int, r[1:])
            assert budget.max_stages(bm, bn, bk, budget.H100_BUDGET) == want


def test_footprint_table():
    rows = [r for r in _golden() if r[0] == "footprint"]
    table = budget.footprint_table(256, 256, 64, [int(r[4]) for r in rows], budget.H100_BUDGET)
    for r, got in zip(rows, table):
        assert got.bytes == int(r[5])
        assert f"{got.kib:.1f}" == r[6]
        assert got.fits == (r[7] == "fits")
        assert f"{got.percent:.0f}" == r[8]


def test_kib_at_depth():
    for r in _golden():
        if r[0] == "kib_at":
            bm, bn, bk, s, kib = map(int, r[1:])
            assert budget.lds_bytes(bm, bn, bk, s) == kib * 1024


def test_pruned_grid_counts_and_rejects():
    (g,) = [r for r in _golden() if r[0] == "grid"]
    M, N, K, req, legal, rej = map(int, g[1:])
    r, l, j = budget.grid_configs(M, N, K, budget.H100_BUDGET)
    assert (len(r), len(l), len(j)) == (req, legal, rej)
    want = sorted(tuple(map(int, x[1:])) for x in _golden() if x[0] == "rejected")
    got = sorted((c["block_M"], c["block_N"], c["block_K"], c["num_stages"], c["threads"]) for c in j)
    assert got == want


def test_mi355x_budget_grid():
    # Same grid against the 160 KiB gfx950 LDS limit (not a figure from the
    # pages; follows from the same formula): 208 legal, 8 rejected.
    r, l, j = budget.grid_configs(4096, 4096, 4096, budget.MI355X_BUDGET)
    assert (len(r), len(l), len(j)) == (216, 208, 8)
    got = {(c["block_M"], c["block_N"], c["block_K"], c["num_stages"]) for c in j}
    assert got == {(128, 256, 64, 4), (256, 128, 64, 4), (256, 256, 64, 3), (256, 256, 64, 4)}


def test_divisibility_prunes_before_budget():
    # 4000 is not a multiple of 64, so no tile of the grid divides M: every
    # candidate is pruned before the budget is even consulted
    r, l, j = budget.grid_configs(4000, 4096, 4096, budget.H100_BUDGET)
    assert len(r) == 216 and len(l) == 0 and len(j) == 0
