"""Host-side checks of bench.py's contract (no GPU): the one-GPU refusal, the
ring-depth notation, the headline configuration's validity and the lookup of
profiled HBM traffic by kernel-source hash."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("text,want", [("1", (1, 0)), ("3", (3, 0)), ("2+A", (2, 1)), ("3+A", (3, 1))])
def test_ring_depth_notation(text, want):
    assert bench.parse_depth(text) == want


def test_headline_configuration_passes_validation():
    import software_pipelined_tiled_03_amd as pg

    h = bench.HEADLINE
    bm, bn, bk = h["block"]
    # pure host validation against the gfx950 budget: no device is touched
    assert pg.gemm_check(pg.GEMM_NT, 4096, 4096, 4096, pg.GEMM_F16, bm, bn, bk, h["num_stages"], h["threads"],
                         163840, a_lead=h["a_lead"]) == 0


def test_every_sweep_point_is_a_valid_configuration():
    import software_pipelined_tiled_03_amd as pg
    from software_pipelined_tiled_03_amd import inputs

    for label, wl, block, threads, depths in bench.SWEEPS:
        w = inputs.workload(wl)
        for d in depths:
            s, lead = bench.parse_depth(d)
            layout = pg.GEMM_NT if w.layout == "nt" else pg.GEMM_NN
            st = pg.gemm_check(layout, w.M, w.N, w.K, w.dtype, block[0], block[1], block[2], s, threads, 163840,
                               a_lead=lead)
            assert st == 0, (label, d, st)


def test_every_attention_point_is_a_valid_configuration():
    import software_pipelined_tiled_03_amd as pg
    from software_pipelined_tiled_03_amd import inputs

    seen = set()
    for name, (bm, bn, th), depths in bench.ATTENTION:
        w = inputs.attention_workload(name)
        for s in depths:
            st = pg.attn_check(w.batch, w.heads, w.kv_heads, w.seq_q, w.seq_kv, w.dim, w.dtype, int(w.causal), bm, bn,
                               s, th, 163840)
            assert st == 0, (name, bm, bn, th, s, st, pg.last_error())
            assert (name, bm, bn, th, s) not in seen, "timed twice: %s" % ((name, bm, bn, th, s),)
            seen.add((name, bm, bn, th, s))


def test_profiled_traffic_is_used_only_for_the_profiled_sources(monkeypatch):
    h = bench.HEADLINE
    args = (h["block"], h["num_stages"], h["a_lead"], h["threads"])
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic(*args) is None
    # the hash recorded in the headline profile, if one is committed, brings back its figure
    path = os.path.join(bench.PROFILES, "gemm_nt_f16_4096_256x256x64_s2a_t512.md")
    if not os.path.exists(path):
        pytest.skip("no headline profile committed")
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip()
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: fields["source_sha256"])
    assert bench.measured_traffic(*args) == int(fields["hbm_bytes_per_launch"])
    # compulsory traffic 2(MK + NK + MN) is a lower bound for what a launch moves
    assert int(fields["hbm_bytes_per_launch"]) >= 2 * 3 * 4096 * 4096


def _profile_hash(name):
    for line in open(os.path.join(bench.PROFILES, name)):
        if line.startswith("- source_sha256"):
            return line.split(":", 1)[1].strip()
    raise AssertionError("%s carries no source_sha256 line" % name)


@pytest.mark.parametrize("name", ["gemm_nt_f16_4096_256x256x64_s2a_t512.md", "stage_sweep_4096.md",
                                  "stage_sweep_small_ragged_longk.md"])
def test_committed_gemm_profiles_match_the_kernel_sources(name):
    # a kernel change must come with new profiles, or the bench line's traffic goes null
    assert _profile_hash(name) == bench.kernel_source_hash(), "%s was taken from other kernel sources" % name


def test_committed_attention_profile_matches_the_kernel_sources():
    assert _profile_hash("attention_fwd_sweep.md") == bench.attention_source_hash()


def test_shape_ceiling_counts_rounds_of_the_compute_units():
    # 4096^3 at 256 x 256: 256 tiles, one round, no padding
    assert bench.shape_ceiling(4096, 4096, 4096, (256, 256, 64)) == pytest.approx(bench.PEAK_TFLOPS)
    # 1024^3 at 128 x 128: 64 tiles on 256 compute units
    assert bench.shape_ceiling(1024, 1024, 1024, (128, 128, 32)) == pytest.approx(bench.PEAK_TFLOPS * 0.25)
    # 4000 x 5000 at 256 x 256: 16 x 20 = 320 tiles take two rounds (the second a quarter full),
    # times the useful fraction of the padded work
    useful = 4000 * 5000 * 3000 / (4096 * 5120 * 3008)
    assert bench.shape_ceiling(4000, 5000, 3000, (256, 256, 64)) == pytest.approx(
        bench.PEAK_TFLOPS * 320 / 512 * (4000 * 5000 * 3000) / (4096 * 5120 * 3008))
    assert bench.shape_ceiling(4000, 5000, 3000, (128, 128, 32)) == pytest.approx(bench.PEAK_TFLOPS * useful)
    # 512 x 512 x 65536 at 128 x 128: 16 workgroups
    assert bench.shape_ceiling(512, 512, 65536, (128, 128, 32)) == pytest.approx(bench.PEAK_TFLOPS / 16)


def test_stamp_summary_reduces_clock_phases_and_residency():
    import torch

    # 16 workgroups, 2 GHz everywhere but XCD 3 at 1.5 GHz; 1000 cycles of
    # prologue, 64000 of loop (nk = 64), 2000 of epilogue; 10 us of real time
    # at 2 GHz, all starting together
    rows = []
    for w in range(16):
        f = 1.5 if w % 8 == 3 else 2.0
        total = 67000
        rt = total / f / 10.0  # 10 ns ticks
        rows.append([0, 1000, 65000, total, 100, 100 + rt])
    st = bench.stamp_summary(torch.tensor(rows, dtype=torch.float64).to(torch.int64), 64, flops=2.0 * 256 * 4096 * 67000,
                             ms=67000 / 2.0 / 1e6 * 1.0)
    assert st["clock_ghz_per_xcd"][3] == pytest.approx(1.5, abs=1e-3)
    assert st["clock_ghz_per_xcd"][0] == pytest.approx(2.0, abs=1e-3)
    assert st["clock_ghz_min_xcd"] == pytest.approx(1.5, abs=1e-3)
    assert st["loop_cycles_per_k_tile"] == pytest.approx(1000.0)
    assert st["prologue_us"] == pytest.approx(0.5, abs=1e-3)      # 1000 cycles at 2 GHz (median)
    # 16 workgroups on 256 compute units: 1/16 resident per CU on average over the span
    assert st["wgs_resident_per_cu"] == pytest.approx(16 / 256 * (14 * 33.5 + 2 * 44.667) / 16 / 44.667, abs=0.01)
    # utilisation: the stamped launches' own time (ms), else the launch's own
    # span (44.667 us here), at the mean clock (14 x 2.0 + 2 x 1.5) / 16 GHz
    flops, clock = 2.0 * 256 * 4096 * 67000, (14 * 2.0 + 2 * 1.5) / 16
    assert st["mfma_util_at_clock"] == pytest.approx(flops / 33.5e-6 / (256 * 4096 * clock * 1e9), rel=1e-3)
    st = bench.stamp_summary(torch.tensor(rows, dtype=torch.float64).to(torch.int64), 64, flops=flops)
    assert st["mfma_util_at_clock"] == pytest.approx(flops / 44.667e-6 / (256 * 4096 * clock * 1e9), rel=1e-3)
