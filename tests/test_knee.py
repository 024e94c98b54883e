"""The knee reduction (oracle/knee.py): the pages' pipeline model fed with
measured parameters.  Checked here without a GPU: on per-depth periods that
the model itself generates from known latency, compute, issue and occupancy,
the reduction recovers those parameters and the knees; the closed-form knee
agrees with the pages' worked example (latency 30, compute 20 -> depth 3)."""
import json

import pytest

from oracle import knee, timeline


def synthetic_sweep(bm, bn, bk, th, C_scale, L, rate, depths, M=4096, N=4096):
    """Rows as bench.py writes them, with periods from the model itself."""
    C = knee.compute_cycles(bm, bn, bk, th)
    I = (bm + bn) * bk * 2 / rate
    rows = {}
    for s in depths:
        o = knee.occupancy(bm, bn, bk, th, s, 0, M, N)
        p = knee.predicted_period(C, L, I, s, o) if s > 1 else L + C
        rows[str(s)] = dict(loop_cycles_per_k_tile=p, tflops=1000.0 * o / p, clock_ghz=2.0)
    return rows


def longk_rows(bk, rate):
    C = knee.compute_cycles(128, 128, bk, 512)
    I = (128 + 128) * bk * 2 / rate
    return {str(s): dict(loop_cycles_per_k_tile=max(C, I, (900 + C) / s) if s > 1 else 900 + C, tflops=1.0)
            for s in (1, 2, 4, 6)}


def test_parameters_and_knees_are_recovered():
    sweeps = {
        "cfg5b_longk_tile128x128x64_t512": longk_rows(64, 40.0),
        "cfg5b_longk_tile128x128x32_t512": longk_rows(32, 32.0),
        "tile256x256x32_t512": synthetic_sweep(256, 256, 32, 512, 1, 1500.0, 40.0, (1, 2, 3, 4)),
        "tile256x256x64_t512": synthetic_sweep(256, 256, 64, 512, 1, 2300.0, 40.0, (1, 2)),
    }
    results, rates = knee.analyse(sweeps)
    assert rates[64] == pytest.approx(40.0) and rates[32] == pytest.approx(32.0)
    by = {r["label"]: r for r in results}
    r = by["tile256x256x32_t512"]
    assert r["C"] == 1024 and r["L"] == pytest.approx(1500.0)
    # 1 + ceil(1500 / 1024) = 3; the model's curve stops falling at 3 as well
    assert r["closed_form_knee"] == 3 and r["predicted_knee"] == 3 and r["measured_knee"] == 3
    for p in r["depths"]:
        assert p["measured"] == pytest.approx(p["predicted"], rel=1e-6)
    assert by["tile256x256x64_t512"]["predicted_knee"] == 2


def test_occupancy_limits():
    # 128 x 128 x 32 on 4 waves: three workgroups by registers (136 per lane ->
    # 3 waves per SIMD), three by LDS at S = 3 (48 KiB), one at S = 6 (96 KiB)
    assert knee.occupancy(128, 128, 32, 256, 3, 0, 4096, 4096) == 3
    assert knee.occupancy(128, 128, 32, 256, 6, 0, 4096, 4096) == 1
    # 8 waves, two per SIMD at 92 registers (5 waves per SIMD): two workgroups
    assert knee.occupancy(128, 128, 32, 512, 2, 0, 4096, 4096) == 2
    # the 256-wide tiles: one workgroup per compute unit
    assert knee.occupancy(256, 256, 64, 512, 2, 1, 4096, 4096) == 1
    # 16 tiles on 256 compute units: at most one each
    assert knee.occupancy(128, 128, 32, 256, 3, 0, 512, 512) == 1


def test_closed_form_knee_of_the_pages_example():
    # chapter 11, section 1.3: latency 30, compute 20 -> minimum sufficient depth 3
    assert timeline.min_depth(30, 20) == 3
    periods = [(s, knee.predicted_period(20, 30, 1, s, 1)) for s in range(1, 7)]
    assert knee.knee(periods) == 3


def test_reads_a_profile_block(tmp_path):
    rows = {"tile256x256x64_t512": {"1": {"loop_cycles_per_k_tile": 4329, "tflops": 960.0}}}
    md = tmp_path / "p.md"
    md.write_text("# x\n\n```json\n%s\n```\n" % json.dumps(rows))
    assert knee.load_rows(str(md)) == rows
