"""The stage-count knee: the pages' pipeline model, fed with parameters taken
from measurements, predicts each sweep's period per ring depth before it is
compared with the measured one.

TEST INFRASTRUCTURE: analysis of measurements (run by hand and by tests/),
never on the product path.

Model.  TileLang tutorial, chapter 11: section 1.2 names three separately
measured quantities (the cost of issuing one round's copies, the latency from
issue until the data has arrived, and one round's compute), section 1.3
schedules copy -> compute rounds greedily over `stages` buffers (implemented in
oracle/timeline.py), and section 2.2 gives its steady period
max(compute, issue, (latency + compute) / depth); the knee is the depth past
which the period stops falling, 1 + ceil(latency / compute) when compute
dominates issue.

Parameters, per sweep (one tile, one thread count, ring depths S), in shader
cycles of one workgroup's K tile:
  C  compute: the K tile's MFMA cycles on the SIMDs the workgroup occupies,
     2 block_M block_N block_K / (1024 min(waves, 4)) (1024 flop per cycle per
     SIMD, both MFMA shapes);
  L  latency: the measured S = 1 period minus C (S = 1 copies, waits and then
     computes, so its period is latency + compute);
  I  issue: the K tile's bytes (block_M + block_N) block_K 2 divided by the
     copy rate one compute unit sustains, measured on the long-K shape
     512 x 512 x 65536 (16 workgroups, one per compute unit, deepest ring of
     each of its sweeps), per block_K;
  o  workgroups per compute unit, fixed before the run: the least of the LDS
     limit floor(160 KiB / ring bytes), the register limit (waves per SIMD
     that the compiler's register count allows, divided by the workgroup's
     waves per SIMD) and the tiles per compute unit ceil(tiles / 256).
The predicted period of one workgroup at depth S is the model's steady
compute interval (timeline.simulate with issue I, latency L, compute C, S
buffers), floored by o C and o I: o workgroups share a compute unit's
matrix cores and its copy path.  The measured period is the clock-stamped
launch's K-loop cycles per K tile (median over workgroups).  Both are
compared per compute unit: the workgroup's period divided by o (cycles per K
tile the compute unit completes), which is what throughput follows when o
changes with S.

Knees: the predicted knee is the least S whose predicted per-unit period is
within 3 % of the least predicted over the sweep's depths; the measured knee
the same over the measured per-unit periods (and, beside it, over the
measured TFLOP/s, which also carry the clock's change with S); the
closed-form knee is 1 + ceil(L / C).

Usage: python -m oracle.knee <bench JSON line file | profile .md with a
```json block of per-depth rows>   -> a markdown table per sweep.
"""
import json
import math
import re
import sys

from . import timeline

LDS_BYTES = 160 * 1024
CUS = 256
VGPRS_PER_LANE = 512  # per SIMD lane, shared by the waves resident on the SIMD

# Registers per lane (arch + accumulation VGPRs, the compiler's .vgpr_count for
# the gfx950 build) of each built tile: (block_M, block_N, block_K, threads).
# tests/test_assembly.py checks this table against the compiled kernels.
REG_COUNT = {
    (64, 128, 64, 256): 80, (128, 128, 32, 128): 264, (128, 128, 32, 256): 136, (128, 128, 32, 512): 92,
    (128, 128, 64, 256): 136, (128, 128, 64, 512): 94, (128, 256, 32, 256): 264, (128, 256, 64, 256): 264,
    (128, 256, 64, 512): 152, (256, 128, 32, 256): 264, (256, 128, 32, 512): 143, (256, 128, 64, 256): 264,
    (256, 256, 32, 256): 512, (256, 256, 32, 512): 240, (256, 256, 64, 256): 512, (256, 256, 64, 512): 246,
}

LABEL = re.compile(r"tile(\d+)x(\d+)x(\d+)_t(\d+)")
SHAPES = {"nt_f16_4096": (4096, 4096, 4096), "nn_bf16_4096": (4096, 4096, 4096),
          "nt_f16_longk_512x512x65536": (512, 512, 65536)}


def parse_label(label):
    """'nn_bf16_tile256x128x32_t512' -> (256, 128, 32, 512)."""
    m = LABEL.search(label)
    if not m:
        raise ValueError("no tile in sweep label %r" % label)
    return tuple(int(x) for x in m.groups())


def compute_cycles(bm, bn, bk, threads):
    return 2.0 * bm * bn * bk / (1024.0 * min(threads // 64, 4))


def reg_waves_per_simd(bm, bn, bk, threads):
    """Waves per SIMD the register count allows (allocation granule 8)."""
    v = REG_COUNT[(bm, bn, bk, threads)]
    return VGPRS_PER_LANE // (-(-v // 8) * 8)


def occupancy(bm, bn, bk, threads, stages, lead, M, N):
    """Workgroups per compute unit, fixed before the run (see the module docstring)."""
    s = max(stages, 1)
    ring = ((s + lead) * bm + s * bn) * bk * 2
    by_lds = LDS_BYTES // ring
    waves = threads // 64
    per_simd = max(1, waves // 4)          # this workgroup's waves on each SIMD it uses
    simds = min(waves, 4)
    by_regs = (reg_waves_per_simd(bm, bn, bk, threads) // per_simd) * (4 // simds)
    tiles = -(-M // bm) * -(-N // bn)
    return max(1, min(by_lds, by_regs, -(-tiles // CUS)))


def predicted_period(C, L, I, stages, o, iterations=64):
    sched = timeline.simulate(iterations, I, L, C, stages)
    return max(sched.compute_iv, o * C, o * I)


def knee(periods, tol=0.03):
    """Least depth whose period is within tol (3 %) of the least period; with
    tol None the values are negated throughputs, within 3 % of the largest."""
    if tol is None:
        best = max(-p for _, p in periods)
        return min(s for s, p in periods if -p >= best * 0.97)
    best = min(p for _, p in periods)
    return min(s for s, p in periods if p <= best * (1 + tol))


def load_rows(path):
    """The per_num_stages sweeps of a bench.py JSON line, or of a ```json
    block in a profile summary (one JSON object: label -> depth -> row)."""
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if m:
        return json.loads(m.group(1))
    line = [l for l in text.strip().splitlines() if l.startswith("{")][-1]
    return json.loads(line)["per_num_stages"]


def issue_rates(sweeps):
    """Copy bytes per cycle one compute unit sustains, per block_K, from the
    long-K sweeps (the deepest ring of each build; the best build per block_K)."""
    rates = {}
    for label, rows in sweeps.items():
        if "longk" not in label or not isinstance(rows, dict):
            continue
        bm, bn, bk, th = parse_label(label)
        deepest = max(rows, key=lambda d: int(d.split("+")[0]))
        r = (bm + bn) * bk * 2 / rows[deepest]["loop_cycles_per_k_tile"]
        rates[bk] = max(rates.get(bk, 0.0), r)
    return rates


def workload_of(label):
    if "longk" in label:
        return "nt_f16_longk_512x512x65536"
    return "nn_bf16_4096" if label.startswith("nn_") else "nt_f16_4096"


def analyse(sweeps):
    """One result per sweep with a plain (no a_lead) S = 1 point and at least
    two plain depths: the parameters, and per depth o, the measured and
    predicted periods and TFLOP/s."""
    rates = issue_rates(sweeps)
    out = []
    for label, rows in sweeps.items():
        if not isinstance(rows, dict) or "1" not in rows:
            continue
        wl = workload_of(label)
        if label.startswith(("cfg1", "cfg2", "cfg5a", "shard")) or wl not in SHAPES:
            continue
        M, N, K = SHAPES[wl]
        bm, bn, bk, th = parse_label(label)
        if bk not in rates:
            continue
        C = compute_cycles(bm, bn, bk, th)
        o1 = occupancy(bm, bn, bk, th, 1, 0, M, N)
        P1 = rows["1"]["loop_cycles_per_k_tile"]
        L = max(0.0, P1 - C)
        I = (bm + bn) * bk * 2 / rates[bk]
        depths = sorted(int(d) for d in rows if "+" not in d)
        per = []
        for s in depths:
            r = rows[str(s)]
            o = occupancy(bm, bn, bk, th, s, 0, M, N)
            pred = predicted_period(C, L, I, s, o)
            per.append(dict(S=s, o=o, measured=round(r["loop_cycles_per_k_tile"] / o, 1),
                            predicted=round(pred / o, 1), tflops=r["tflops"], clock_ghz=r.get("clock_ghz"),
                            copy_rate=round((bm + bn) * bk * 2 * o / r["loop_cycles_per_k_tile"], 1)))
        out.append(dict(label=label, C=C, L=round(L, 1), I=round(I, 1), o1=o1,
                        closed_form_knee=1 + math.ceil(L / C) if C > 0 else None,
                        predicted_knee=knee([(p["S"], p["predicted"]) for p in per]),
                        measured_knee=knee([(p["S"], p["measured"]) for p in per]),
                        measured_knee_tflops=knee([(p["S"], -p["tflops"]) for p in per], tol=None),
                        depths=per))
    return out, rates


def markdown(results, rates):
    lines = ["Copy rate per compute unit (long-K, deepest ring): " +
             ", ".join("block_K %d: %.1f B/cycle" % (k, v) for k, v in sorted(rates.items())), ""]
    lines.append("| sweep | C | L | I | knee: closed form / model / measured (cycles) / measured (TFLOP/s) | "
                 "per S: o, measured / predicted cycles per K tile per compute unit, copy B/cycle per unit |")
    lines.append("|---|---|---|---|---|---|")
    for r in results:
        cells = "; ".join("S=%d o=%d %.0f / %.0f, %.1f" % (p["S"], p["o"], p["measured"], p["predicted"],
                                                            p["copy_rate"]) for p in r["depths"])
        lines.append("| %s | %.0f | %.0f | %.0f | %s / %d / %d / %d | %s |" % (
            r["label"], r["C"], r["L"], r["I"], r["closed_form_knee"], r["predicted_knee"], r["measured_knee"],
            r["measured_knee_tflops"], cells))
    return "\n".join(lines)


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    if len(argv) != 1:
        print(__doc__.split("Usage:")[1].strip(), file=sys.stderr)
        return 2
    results, rates = analyse(load_rows(argv[0]))
    print(markdown(results, rates))
    return 0


if __name__ == "__main__":
    sys.exit(main())
