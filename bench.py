"""Benchmark of the software-pipelined tiled GEMM on one MI355X.

A step is one GEMM call, C = A[M,K] . B^T, on inputs already resident in
HBM.  The headline workload is the 4096^3 fp16 NT GEMM; `value` is its
throughput in TFLOP/s (2MNK / t) with the fastest configuration (256x256x64
tile, two stages plus a leading A tile, 8 waves).  The line also carries the
num_stages sweep of the 128x128x32 tile (the tutorial's default) and of the
256x256 tiles (each point timed by the library's own launch loop, with the
clock, phase times and cycles per K tile of one clock-stamped launch), the
roofline of the kernel (MFMA bound, measured with HIP events on the launch
stream), the shader clock the headline ran at with its MFMA utilisation at
that clock, and the CPU oracle timed on a bounded row sample of the same GEMM
together with the element-wise parity of the headline's C.

The attention forward pass (the KV-length loop on the same ring) is swept
per ring depth on its workloads and reported under "attention".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep] [--no-cpu-baseline]
                       [--no-attention | --attention] [--no-clock] [--workload W --block BMxBNxBK
                       --stages S[+A] --threads T] [--tune-tables] [--oracle-table] [--sustain SECONDS]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2500.0     # MI355X dense fp16/bf16 MFMA, published
HEADLINE = dict(workload="nt_f16_4096", block=(256, 256, 64), num_stages=2, a_lead=1, threads=512)
# (label, workload, block, threads, ring depths); a depth "S+A" is num_stages S with a_lead = 1
SWEEPS = [
    # the smaller and ragged shapes first (one workgroup, 64 workgroups, ragged
    # edges, a long K loop on 16 CUs), so that the full-chip 4096^3 sweeps and
    # the headline that follows them run under the same sustained load
    ("cfg1_128_tile128x128x32_t256", "nt_f16_128", (128, 128, 32), 256, ("1",)),
    ("cfg2_1024_tile128x128x32_t256", "nt_f16_1024", (128, 128, 32), 256, ("1", "2", "3")),
    ("cfg2_1024_tile64x128x64_t256", "nt_f16_1024", (64, 128, 64), 256, ("2", "3", "4")),
    ("cfg5a_ragged_tile128x128x32_t256", "nt_f16_ragged_4000x5000x3000", (128, 128, 32), 256, ("3",)),
    ("cfg5a_ragged_tile256x256x64_t512", "nt_f16_ragged_4000x5000x3000", (256, 256, 64), 512, ("2", "2+A")),
    ("cfg5b_longk_tile128x128x32_t256", "nt_f16_longk_512x512x65536", (128, 128, 32), 256, ("1", "2", "3", "4", "6")),
    # the same 16 workgroups with 8 waves each (two per SIMD), at block_K 32 and 64
    ("cfg5b_longk_tile128x128x32_t512", "nt_f16_longk_512x512x65536", (128, 128, 32), 512, ("1", "2", "3", "4", "6")),
    ("cfg5b_longk_tile128x128x64_t512", "nt_f16_longk_512x512x65536", (128, 128, 64), 512, ("1", "2", "3", "4", "5")),
    # the gfx950 default for this shape: twice the workgroups of the 128-wide tiles
    ("cfg5b_longk_tile64x128x64_t256", "nt_f16_longk_512x512x65536", (64, 128, 64), 256, ("2", "3", "4", "6")),
    # one GPU's share of 4096^3 over 8 GPUs (512 x 4096 x 4096): 256, 128 or 32 workgroups
    ("shard8_tile64x128x64_t256", "nt_f16_shard8_512x4096x4096", (64, 128, 64), 256, ("2", "3", "4", "6")),
    ("shard8_tile128x128x64_t256", "nt_f16_shard8_512x4096x4096", (128, 128, 64), 256, ("2", "3", "4")),
    ("shard8_tile128x128x32_t512", "nt_f16_shard8_512x4096x4096", (128, 128, 32), 512, ("2", "3", "4")),
    ("shard8_tile128x256x64_t256", "nt_f16_shard8_512x4096x4096", (128, 256, 64), 256, ("2", "3")),
    ("shard8_tile256x256x64_t512", "nt_f16_shard8_512x4096x4096", (256, 256, 64), 512, ("2+A",)),
    ("tile128x128x32_t128", "nt_f16_4096", (128, 128, 32), 128, ("1", "2", "3", "4", "6")),
    ("tile128x128x32_t256", "nt_f16_4096", (128, 128, 32), 256, ("1", "2", "3", "4", "6")),
    ("tile128x128x32_t512", "nt_f16_4096", (128, 128, 32), 512, ("1", "2", "3", "4", "6")),
    ("tile256x256x32_t256", "nt_f16_4096", (256, 256, 32), 256, ("1", "2", "3", "4", "5", "2+A", "3+A")),
    ("tile256x256x32_t512", "nt_f16_4096", (256, 256, 32), 512, ("1", "2", "3", "4", "2+A", "3+A")),
    ("tile256x256x64_t256", "nt_f16_4096", (256, 256, 64), 256, ("1", "2", "2+A")),
    ("tile256x256x64_t512", "nt_f16_4096", (256, 256, 64), 512, ("1", "2", "2+A")),
    ("nn_bf16_tile128x128x32_t256", "nn_bf16_4096", (128, 128, 32), 256, ("1", "2", "3", "4", "6")),
    ("nn_bf16_tile128x256x64_t256", "nn_bf16_4096", (128, 256, 64), 256, ("1", "2", "3")),
    ("nn_bf16_tile256x128x32_t256", "nn_bf16_4096", (256, 128, 32), 256, ("1", "2", "3", "4", "6")),
    # the same two tiles on 8 waves (16x16x32 MFMAs, two waves per SIMD)
    ("nn_bf16_tile128x256x64_t512", "nn_bf16_4096", (128, 256, 64), 512, ("1", "2", "3", "3+A")),
    ("nn_bf16_tile256x128x32_t512", "nn_bf16_4096", (256, 128, 32), 512, ("1", "2", "3", "4", "6")),
    ("nn_bf16_tile256x256x64_t256", "nn_bf16_4096", (256, 256, 64), 256, ("2", "2+A")),
    ("nn_bf16_tile256x256x64_t512", "nn_bf16_4096", (256, 256, 64), 512, ("2", "2+A")),
]


def parse_depth(d):
    """'3' -> (3, 0); '2+A' -> (2, 1)."""
    d = str(d)
    return (int(d[:-2]), 1) if d.endswith("+A") else (int(d), 0)
# The attention KV-length loop on the same ring: (workload, (block_M, block_N, threads), ring depths)
ATTENTION = [
    ("attn_f16_b4_h32_s4096_d128", (256, 64, 512), (1, 2, 3, 4)),
    ("attn_f16_b4_h32_s4096_d128_causal", (256, 64, 512), (1, 2, 3, 4)),
    ("attn_f16_b4_h32_s4096_d128", (256, 128, 512), (1, 2)),
    ("attn_f16_b4_h32_s4096_d128_causal", (256, 128, 512), (1, 2)),
    # the pages' fixed flashattn configuration: block_M 128, block_N 128, 2 stages, 256 threads
    ("attn_f16_b4_h32_s4096_d128", (128, 128, 256), (1, 2)),
    ("attn_f16_b4_h32_s4096_d128_causal", (128, 128, 256), (1, 2)),
    # 4 waves: two workgroups share a compute unit where the ring fits in half the LDS
    ("attn_f16_b4_h32_s4096_d128", (128, 64, 256), (1, 2, 3, 4)),
    ("attn_f16_b4_h32_s4096_d128_causal", (128, 64, 256), (1, 2)),
    ("attn_f16_b4_h32_s4096_d128", (256, 64, 256), (1, 2, 3, 4)),
    ("attn_f16_b4_h32_s4096_d128_causal", (256, 64, 256), (1, 2, 3, 4)),
    # bf16, causal, 32 query heads on 8 KV heads
    ("attn_bf16_b2_h32_kv8_s2048_d128_causal", (256, 128, 512), (1, 2)),
    ("attn_bf16_b2_h32_kv8_s2048_d128_causal", (256, 64, 512), (2, 3, 4)),
    # head dimension 64
    ("attn_f16_b4_h32_s4096_d64", (256, 128, 512), (1, 2, 3, 4)),
    ("attn_f16_b4_h32_s4096_d64", (256, 64, 512), (2, 3, 4)),
    ("attn_f16_b4_h32_s4096_d64_causal", (256, 128, 512), (2, 3, 4)),
    # two 32-query blocks per wave, 8 waves (fits the registers at D = 64)
    ("attn_f16_b4_h32_s4096_d64", (512, 64, 512), (2, 3, 4)),
    ("attn_f16_b4_h32_s4096_d64", (512, 128, 512), (2,)),
    ("attn_f16_b4_h32_s4096_d64_causal", (512, 64, 512), (2, 3, 4)),
    # 4 waves at D = 64, one and two 32-query blocks per wave
    ("attn_f16_b4_h32_s4096_d64", (128, 64, 256), (1, 2, 3)),
    ("attn_f16_b4_h32_s4096_d64_causal", (128, 64, 256), (1, 2, 3)),
    ("attn_f16_b4_h32_s4096_d64", (256, 64, 256), (2, 3)),
    ("attn_f16_b4_h32_s4096_d64_causal", (256, 64, 256), (2, 3)),
]
PROFILES = os.path.join(ROOT, "profiles")


KERNEL_SOURCES = ("pipegemm_kernel.hpp", "pipegemm_kernels.hip", "pipegemm_launch.hpp", "pipegemm_layout.hpp")


def kernel_source_hash():
    """sha256 of the device-code sources the kernels are built from (the
    kernel template, its layouts and schedule, and its instantiations; the
    host-side validation and tuning code does not change what a launch
    moves)."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "software_pipelined_tiled_03_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


ATTN_SOURCES = ("attn_kernel.hpp", "attn_kernels.hip", "attn_launch.hpp", "attn_map.hpp", "pipegemm_kernel.hpp",
                "pipegemm_layout.hpp")


def attention_source_hash():
    """sha256 over the contents, in this order, of the device-code sources
    the attention kernel is built from (its own files and the GEMM headers it
    takes the ring and layouts from), then the compiler flags only its units
    get (build.ATTN_FLAGS)."""
    import hashlib

    from software_pipelined_tiled_03_amd import build

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "software_pipelined_tiled_03_amd", "csrc")
    for name in ATTN_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    h.update(" ".join(build.ATTN_FLAGS).encode())
    return h.hexdigest()


def measured_traffic(block, stages, a_lead, threads):
    """HBM bytes per launch from a committed rocprofv3 summary of this exact
    kernel configuration, or None if there is none or the kernel sources
    changed since it was taken.  The summary carries lines
    `config: <BMxBNxBK> S=<s>[+A] threads=<t>`, `source_sha256: <hex>` and
    `hbm_bytes_per_launch: <int>`."""
    want = "%dx%dx%d S=%d%s threads=%d" % (block[0], block[1], block[2], stages, "+A" if a_lead else "", threads)
    src = kernel_source_hash()
    if not os.path.isdir(PROFILES):
        return None
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        fields = {}
        with open(os.path.join(PROFILES, name)) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip("-* `")] = v.strip(" `\n")
        if fields.get("config") == want and fields.get("source_sha256") == src and "hbm_bytes_per_launch" in fields:
            return int(fields["hbm_bytes_per_launch"])
    return None


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _device_inputs(w):
    import numpy as np
    import torch

    from software_pipelined_tiled_03_amd import inputs

    A, B = w.make()
    tdt = torch.float16 if w.dtype == inputs.F16 else torch.bfloat16
    dA = torch.from_numpy(A.view(np.int16)).cuda().view(tdt)
    dB = torch.from_numpy(B.view(np.int16)).cuda().view(tdt)
    return A, B, dA, dB


LDS_PER_CU = 163840
CUS = 256


def shape_ceiling(M, N, K, block):
    """The most a shape can reach on this tile, in TFLOP/s: the nominal peak
    times the fraction of compute-unit time its grid can fill (the tiles go
    out in ceil(tiles / 256) rounds over the 256 compute units; a tile keeps
    at most one compute unit busy) and the fraction of the padded tile work
    that is useful (ragged edges)."""
    bm, bn, bk = block
    tm, tn, nk = -(-M // bm), -(-N // bn), -(-K // bk)
    tiles = tm * tn
    rounds = -(-tiles // CUS)
    return PEAK_TFLOPS * tiles / (rounds * CUS) * (M * N * K) / (tm * bm * tn * bn * nk * bk)


def stamp_summary(stamps, nk, flops=None, ms=None):
    """Reduce gemm_stamped's six counters per workgroup (cycles at start,
    after the prologue, after the K loop and at the end; 100 MHz real time at
    start and end): the shader clock (mean over workgroups, and per XCD =
    workgroup id mod 8), the median prologue, K-loop and epilogue times, the
    K-loop cycles per K tile (median over workgroups), the workgroups resident
    per compute unit on average (summed workgroup time over the span times
    256), and with `flops` the MFMA utilisation at the measured clock:
    2MNK / time / (256 CUs x 4096 flop x clock), with the time taken from the
    stamped launches themselves (`ms`, their event time per launch, or without
    it the stamped launch's own span), never from other launches: the clock
    under this load moves by 10 % and more between windows a few
    milliseconds apart, so a clock from one window and a time from another
    give a ratio that is off by as much."""
    import numpy as np

    s = stamps.view(-1, 6).cpu().numpy().astype(np.float64)
    cyc, rt = s[:, 3] - s[:, 0], s[:, 5] - s[:, 4]
    ok = rt > 0
    clk = np.where(ok, cyc / np.where(ok, rt, 1) * 0.1, np.nan)  # GHz
    clock = float(np.nanmean(clk))
    xcd = np.arange(len(s)) % 8
    per_xcd = [round(float(np.nanmean(clk[xcd == x])), 3) if (xcd == x).any() else None for x in range(8)]
    to_us = lambda c: float(np.median(c / clk)) / 1e3
    span_us = float(s[:, 5].max() - s[:, 4].min()) / 100.0
    out = dict(clock_ghz=round(clock, 3), clock_ghz_per_xcd=per_xcd,
               clock_ghz_min_xcd=round(float(np.nanmin([c for c in per_xcd if c is not None])), 3),
               prologue_us=round(to_us(s[:, 1] - s[:, 0]), 3), loop_us=round(to_us(s[:, 2] - s[:, 1]), 3),
               epilogue_us=round(to_us(s[:, 3] - s[:, 2]), 3),
               loop_cycles_per_k_tile=round(float(np.median(s[:, 2] - s[:, 1])) / max(nk, 1), 1),
               wg_span_us=round(span_us, 3),
               wgs_resident_per_cu=round(float(rt.sum()) / 100.0 / (span_us * CUS), 2) if span_us > 0 else None)
    t_ms = ms if ms else (span_us * 1e-3 if span_us > 0 else None)
    if flops is not None and t_ms:
        out["mfma_util_at_clock"] = round(flops / (t_ms * 1e-3) / (CUS * 4096 * clock * 1e9), 4)
    return out


def time_gemm(fn, dA, dB, C, block, stages, threads, steps, warmup, a_lead=0, relu=False):
    """Average milliseconds per call over `steps` back-to-back launches."""
    import torch

    for _ in range(warmup):
        fn(dA, dB, out=C, block=block, num_stages=stages, threads=threads, a_lead=a_lead, relu=relu)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn(dA, dB, out=C, block=block, num_stages=stages, threads=threads, a_lead=a_lead, relu=relu)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def launch_distribution(fn, dA, dB, C, block, stages, threads, a_lead=0, reps=100, warmup=25, scrub=None):
    """Per-launch durations (HIP events around each single launch on the
    current stream): median, min and p90 in ms.  With `scrub` (a device byte
    tensor larger than the last-level caches) every timed launch is preceded by
    a write of the whole scrub buffer outside its events, so A and B start cold."""
    import torch

    for _ in range(warmup):
        fn(dA, dB, out=C, block=block, num_stages=stages, threads=threads, a_lead=a_lead)
    stream = torch.cuda.current_stream()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(pairs):
        if scrub is not None:
            scrub.fill_(i & 0xFF)
        e0.record(stream)
        fn(dA, dB, out=C, block=block, num_stages=stages, threads=threads, a_lead=a_lead)
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)
    return dict(median_ms=round(t[len(t) // 2], 5), min_ms=round(t[0], 5),
                p90_ms=round(t[min(len(t) - 1, (9 * len(t)) // 10)], 5))


def attention_sweep(steps=10, warmup=3):
    """TFLOP/s (4 B H D x visible query-key pairs / t) of the attention kernel
    per ring depth on the ATTENTION workloads."""
    import numpy as np
    import torch

    import software_pipelined_tiled_03_amd as pg
    from software_pipelined_tiled_03_amd import inputs

    out = {}
    tensors = {}
    for name, (bm, bn, th), depths in ATTENTION:
        w = inputs.attention_workload(name)
        if name not in tensors:
            tdt = torch.float16 if w.dtype == inputs.F16 else torch.bfloat16
            tensors[name] = [torch.from_numpy(x.view(np.int16)).cuda().view(tdt) for x in w.make()]
        dQ, dK, dV = tensors[name]
        O = torch.empty_like(dQ)
        row = {}
        for s in depths:
            def call():
                pg.attention(dQ, dK, dV, causal=w.causal, out=O, block_M=bm, block_N=bn, num_stages=s, threads=th)
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                call()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            row[str(s)] = dict(tflops=round(w.flops / ms / 1e9, 1), ms=round(ms, 4),
                               lds_bytes=pg.attn_lds_bytes(bn, 128, s))
            _log("attention %s bm%d bn%d S=%d: %.1f TFLOP/s" % (name, bm, bn, s, w.flops / ms / 1e9))
        out["%s_bm%d_bn%d_t%d" % (name, bm, bn, th)] = row
    del tensors
    return out


def cpu_baseline(w, A, B, rows, gpu_c=None):
    """The CPU oracle (as it stands) on the first `rows` rows of C.  With
    `gpu_c` (the headline launch's C as 16-bit encodings) the same rows are
    also compared with the oracle's: max abs / rel error and the count outside
    |gpu - oracle| <= 1e-2 + 1e-2 |oracle|."""
    import numpy as np

    from oracle import gemm as og

    fn = og.gemm_nt if w.layout == "nt" else og.gemm_nn
    fn(A, B, w.dtype, rows=(0, 1))  # load / warm
    t0 = time.perf_counter()
    ref = fn(A, B, w.dtype, rows=(0, rows))
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    out = dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=og.num_threads(), kind="oracle",
               sample="rows 0..%d of C (%d x %d x %d, %s), %.1f GFLOP in %.2f s"
                      % (rows - 1, w.M, w.N, w.K, w.layout.upper(), flops / 1e9, dt))
    if gpu_c is not None:
        want = og.decode(ref, w.dtype).astype(np.float64)
        got = og.decode(gpu_c[:rows], w.dtype).astype(np.float64)
        err = np.abs(got - want)
        out["parity_rows"] = rows
        out["parity_elements"] = int(err.size)
        out["parity_outside_tolerance"] = int((err > 1e-2 + 1e-2 * np.abs(want)).sum())
        out["parity_max_abs_err"] = float(err.max())
        out["parity_max_rel_err"] = float((err / np.maximum(np.abs(want), 1e-3)).max())
    return out


# Shapes of the tuning tables that fix the gfx950 default table (NT fp16)
TUNE_SHAPES = [(512, 512, 65536), (1024, 1024, 1024), (1024, 1024, 8192), (2048, 2048, 2048), (3072, 3072, 3072),
               (4096, 4096, 4096), (4096, 4096, 512), (6144, 2048, 2048), (2048, 6144, 2048), (8192, 8192, 1024),
               (8192, 8192, 8192), (16384, 4096, 4096)]


def tune_tables(passes=1):
    """Every built configuration measured on each TUNE_SHAPES problem (NT fp16,
    uniform[-1,1] from inputs.custom with seed 7M + 3N + K), after settling
    launches of the default configuration; each candidate gets about 3 ms of
    warm-up launches and 3 ms of timed launches (at least 10 and 30), so a
    short kernel is not timed inside the power manager's transitions.  One
    JSON line per shape and pass: the tuned winner, the default table's pick
    (gemm_default_config), the cost model's first choice (gemm_rank), their
    measured times, and every candidate's time."""
    import numpy as np
    import torch

    import software_pipelined_tiled_03_amd as pg
    from software_pipelined_tiled_03_amd import inputs

    for M, N, K in TUNE_SHAPES:
        A, B = inputs.custom("nt", inputs.F16, M, N, K, seed=7 * M + 3 * N + K).make()
        dA = torch.from_numpy(A.view(np.int16)).cuda().view(torch.float16)
        dB = torch.from_numpy(B.view(np.int16)).cuda().view(torch.float16)
        C = torch.empty((M, N), dtype=torch.float16, device="cuda")
        d = pg.default_config("nt", M, N, K)
        t = pg.tuning.time_config(dA, dB, d, warmup=200, reps=50, out=C)
        warm, reps = max(10, int(3.0 / t)), max(30, int(3.0 / t))
        first = pg.rank("nt", M, N, K)[0][0]
        for p in range(passes):
            res = pg.tune(dA, dB, "nt", warmup=warm, reps=reps, out=C)
            ms = {tuple(sorted(c.items())): v for c, st, v in res.table if st == 0}
            row = dict(shape=[M, N, K], passes=p, legal=len(ms), warmup=warm, reps=reps, best=res.config,
                       best_ms=round(res.latency, 5), default=d, default_ms=round(ms[tuple(sorted(d.items()))], 5),
                       model_first=first, model_first_ms=round(ms[tuple(sorted(first.items()))], 5),
                       table=[[c["block_M"], c["block_N"], c["block_K"], c["num_stages"], c["a_lead"], c["threads"],
                               round(v, 5)] for c, st, v in res.table if st == 0])
            row["default_over_best"] = round(row["default_ms"] / row["best_ms"], 4)
            row["model_first_over_best"] = round(row["model_first_ms"] / row["best_ms"], 4)
            print(json.dumps(row), flush=True)
            _log("tune %dx%dx%d pass %d: best %.4f ms, default %.4f ms (x%.3f), model first x%.3f"
                 % (M, N, K, p, row["best_ms"], row["default_ms"], row["default_over_best"],
                    row["model_first_over_best"]))
        del dA, dB, C
    return 0


# Oracle timing table: (workload, timed runs, also on one thread)
ORACLE_TABLE = [
    ("nt_f16_128", 3, True),
    ("nt_f16_1024", 3, True),
    ("nt_f16_4096", 1, False),
    ("nn_bf16_4096", 1, False),
    ("nt_f16_ragged_4000x5000x3000", 1, False),
    ("nt_f16_longk_512x512x65536", 3, True),
]


def oracle_table_worker(one_thread):
    """Times the CPU oracle (whole C, every row) on each workload of
    ORACLE_TABLE; with one_thread only on the workloads marked for it.  Runs
    in its own process so that OMP_NUM_THREADS is read at the oracle's load."""
    if one_thread:
        os.environ["OMP_NUM_THREADS"] = "1"
    from oracle import gemm as og
    from software_pipelined_tiled_03_amd import inputs

    rows = []
    for name, runs, single in ORACLE_TABLE:
        if one_thread and not single:
            continue
        w = inputs.workload(name)
        A, B = w.make()
        fn = og.gemm_nt if w.layout == "nt" else og.gemm_nn
        fn(A, B, w.dtype, rows=(0, 1))
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            fn(A, B, w.dtype)
            ts.append(time.perf_counter() - t0)
        t = sorted(ts)[len(ts) // 2]
        rows.append(dict(workload=name, threads=og.num_threads(), runs=runs, seconds=round(t, 4),
                         gflops=round(2.0 * w.M * w.N * w.K / t / 1e9, 2)))
        _log("oracle %s on %d thread(s): %.3f s, %.2f GFLOP/s" % (name, og.num_threads(), t, rows[-1]["gflops"]))
    return rows


def oracle_table():
    """The CPU oracle's timing on every GEMM workload, on all host cores and on
    one thread; prints one JSON line.  No GPU is used."""
    import platform
    import subprocess

    rows = []
    for one in (0, 1):
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-table-worker", str(one)],
                           capture_output=True, text=True, check=True)
        rows += json.loads(r.stdout.strip().splitlines()[-1])
    model = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    print(json.dumps({"oracle_table": rows, "host": {"nproc": os.cpu_count(), "cpu_model": model}}), flush=True)
    return 0


def sustain(call, flops, seconds):
    """`call` (one launch) back to back for `seconds` windows of about one
    second each (HIP events around each; the first, of 100 launches, sizes
    the others), one JSON line per window."""
    import torch

    per_window = None
    for sec in range(seconds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = per_window or 100
        t0 = time.time()
        e0.record()
        for _ in range(n):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        if per_window is None:
            per_window = max(100, int(1000.0 / ms))
        print(json.dumps({"sustain_s": sec, "launches": n, "ms_per_launch": round(ms, 5),
                          "tflops": round(flops / ms / 1e9, 1), "wall_s": round(time.time() - t0, 3)}), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle", type=int, default=500,
                    help="back-to-back launches of the timed configuration before its warmup (power settling)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--attention", action="store_true", help="run the attention sweep even with --no-sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-clock", action="store_true", help="skip the clock-stamped launches after the headline")
    ap.add_argument("--workload", default=HEADLINE["workload"], help="one of inputs.WORKLOADS")
    ap.add_argument("--block", default=None, help="tile as BMxBNxBK (default: the headline tile)")
    ap.add_argument("--stages", default=None, help="ring depth, e.g. 3 or 2+A (num_stages 2 with a_lead)")
    ap.add_argument("--threads", type=int, default=None)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--oracle-table", action="store_true",
                    help="only time the CPU oracle on every GEMM workload (all cores and one thread); no GPU")
    ap.add_argument("--oracle-table-worker", type=int, default=None, help=argparse.SUPPRESS)
    ap.add_argument("--tune-tables", action="store_true",
                    help="only measure every built configuration on the tuning shapes (one JSON line per shape)")
    ap.add_argument("--sustain", type=int, default=0,
                    help="only run the headline configuration (with --attention: the attention forward pass of the "
                         "first attention workload, default tile) back to back for this many windows of about a "
                         "second (at most 120), one JSON line per window: a steady load for reading board power "
                         "and clocks beside it")
    args = ap.parse_args()

    if args.oracle_table_worker is not None:
        print(json.dumps(oracle_table_worker(bool(args.oracle_table_worker))), flush=True)
        return 0
    if args.oracle_table:
        return oracle_table()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this GEMM runs on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch

    import software_pipelined_tiled_03_amd as pg
    from software_pipelined_tiled_03_amd import inputs

    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        return 1
    pg.load()

    if args.tune_tables:
        return tune_tables(passes=2)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 5}))
        return 0

    if args.sustain and args.attention:
        import numpy as np
        aw = inputs.attention_workload(ATTENTION[0][0])
        dQ, dK, dV = [torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16) for x in aw.make()]
        O = torch.empty_like(dQ)
        # the default tile for these sizes (attn_default_config)
        return sustain(lambda: pg.attention(dQ, dK, dV, causal=aw.causal, out=O), aw.flops, min(args.sustain, 120))

    w = inputs.workload(args.workload)
    A, B, dA, dB = _device_inputs(w)
    fn = pg.gemm_nt if w.layout == "nt" else pg.gemm_nn
    C = torch.empty((w.M, w.N), dtype=dA.dtype, device="cuda")
    flops = 2.0 * w.M * w.N * w.K

    if args.sustain:
        hb, hs, hl, ht = HEADLINE["block"], HEADLINE["num_stages"], HEADLINE["a_lead"], HEADLINE["threads"]
        return sustain(lambda: fn(dA, dB, out=C, block=hb, num_stages=hs, threads=ht, a_lead=hl), flops,
                       min(args.sustain, 120))

    sweep = {}
    if not args.no_sweep:
        operands = {w.name: (dA, dB, C, fn)}
        for label, wl, block, th, stages in SWEEPS:
            if wl not in operands:
                ws = inputs.workload(wl)
                _, _, sA, sB = _device_inputs(ws)
                operands[wl] = (sA, sB, torch.empty((ws.M, ws.N), dtype=sA.dtype, device="cuda"),
                                pg.gemm_nt if ws.layout == "nt" else pg.gemm_nn)
            sA, sB, sC, sfn = operands[wl]
            lay = "nt" if sfn is pg.gemm_nt else "nn"
            sM, sK, sN = sA.shape[0], sA.shape[1], sC.shape[1]
            sflops = 2.0 * sM * sN * sK
            row = {}
            for d in stages:
                s, lead = parse_depth(d)
                cfg = dict(block_M=block[0], block_N=block[1], block_K=block[2], num_stages=s, a_lead=lead,
                           threads=th)
                # the library's own timing loop (no per-call host cost in the figure)
                ms = pg.tuning.time_config(sA, sB, cfg, layout=lay, warmup=5, reps=30, out=sC)
                # one more launch with clock stamps: clock, phases, cycles per K tile
                _, stamps = pg.gemm_stamped(pg.GEMM_NT if lay == "nt" else pg.GEMM_NN, sA, sB, out=sC, block=block,
                                            num_stages=s, threads=th, a_lead=lead)
                st = stamp_summary(stamps, -(-sK // block[2]), sflops)
                lds = pg.gemm_lds_bytes(block[0], block[1], block[2], s, a_lead=lead)
                row[d] = dict(tflops=round(sflops / ms / 1e9, 1),
                              pct_peak=round(100 * sflops / ms / 1e9 / PEAK_TFLOPS, 1),
                              pct_shape_ceiling=round(100 * sflops / ms / 1e9 / shape_ceiling(sM, sN, sK, block), 1),
                              lds_bytes=lds, wgs_per_cu_by_lds=LDS_PER_CU // lds, us=round(ms * 1e3, 2),
                              clock_ghz=st["clock_ghz"], mfma_util_at_clock=st.get("mfma_util_at_clock"),
                              loop_cycles_per_k_tile=st["loop_cycles_per_k_tile"],
                              wgs_resident_per_cu=st["wgs_resident_per_cu"],
                              copy_bytes_per_cycle_per_wg=round((block[0] + block[1]) * block[2] * 2
                                                                / st["loop_cycles_per_k_tile"], 2),
                              prologue_us=st["prologue_us"], epilogue_us=st["epilogue_us"],
                              # the stamped launch's own span (first workgroup start to last
                              # workgroup end): kernel time without launch gaps, which set
                              # `us` for the smallest shapes
                              kernel_us=st["wg_span_us"],
                              tflops_kernel=round(sflops / st["wg_span_us"] / 1e6, 1) if st["wg_span_us"] else None)
                _log("sweep %s S=%s: %.1f TFLOP/s at %.2f GHz, %.0f cycles per K tile"
                     % (label, d, sflops / ms / 1e9, st["clock_ghz"], st["loop_cycles_per_k_tile"]))
            sweep[label] = row
        rej = None
        nA, nB, nC, nfn = operands.get("nn_bf16_4096", (None, None, None, None))
        if nfn is not None:
            try:
                nfn(nA, nB, out=nC, block=(256, 256, 64), num_stages=4, threads=256)
            except pg.LdsBudgetError as e:
                rej = str(e)
        sweep["nn_bf16_256x256x64_S4_rejected"] = rej
        del operands

    block = tuple(int(x) for x in args.block.split("x")) if args.block else HEADLINE["block"]
    if args.stages is not None:
        stages, a_lead = parse_depth(args.stages)
    else:
        stages, a_lead = HEADLINE["num_stages"], HEADLINE["a_lead"]
    threads = args.threads if args.threads is not None else HEADLINE["threads"]
    # settle: the power manager needs a few tens of milliseconds of sustained
    # load before the clock holds steady (from idle the first launches run
    # boosted, then dip well below the sustained rate), so the timed launches
    # follow `settle` back-to-back launches whatever ran before them
    ms = time_gemm(fn, dA, dB, C, block, stages, threads, steps=args.steps, warmup=args.settle + args.warmup,
                   a_lead=a_lead)
    tflops = flops / ms / 1e9
    # the headline's C (16-bit encodings), for the parity check of the CPU-baseline leg
    import numpy as np
    headline_c = None if args.no_cpu_baseline else C.view(torch.int16).cpu().numpy().view(np.uint16)
    _log("headline %s tile %s S=%d%s threads=%d: %.3f ms, %.1f TFLOP/s"
         % (w.name, block, stages, "+A" if a_lead else "", threads, ms, tflops))

    # the same configuration, right after the timed launches, with clock
    # stamps: the shader clock the chip actually ran at (it is power-limited
    # with random operands), per XCD, and the MFMA utilisation at that clock
    clock = None
    if not args.no_clock:
        layout_code = pg.GEMM_NT if w.layout == "nt" else pg.GEMM_NN
        grid = -(-w.M // block[0]) * -(-w.N // block[1])
        stamps = torch.zeros(6 * grid, dtype=torch.int64, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            pg.gemm_stamped(layout_code, dA, dB, out=C, block=block, num_stages=stages, threads=threads,
                            a_lead=a_lead, stamps=stamps)
        e1.record()
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / reps
        # utilisation of these stamped launches: their clock and their own time
        clock = stamp_summary(stamps, -(-w.K // block[2]), flops, sms)
        clock["launches"] = reps
        clock["ms_per_launch"] = round(sms, 5)
        _log("clock %.3f GHz (XCDs %s), MFMA utilisation at that clock %.3f; prologue %.2f us, loop %.2f us, "
             "epilogue %.2f us" % (clock["clock_ghz"], clock["clock_ghz_per_xcd"], clock["mfma_util_at_clock"],
                                  clock["prologue_us"], clock["loop_us"], clock["epilogue_us"]))

    # per-launch distribution of the same configuration, warm and with the
    # caches scrubbed (512 MiB written between launches: twice the MALL)
    per_launch = None
    if not args.no_sweep:
        warm = launch_distribution(fn, dA, dB, C, block, stages, threads, a_lead=a_lead)
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold = launch_distribution(fn, dA, dB, C, block, stages, threads, a_lead=a_lead, scrub=scrub)
        del scrub
        for d in (warm, cold):
            d["median_tflops"] = round(flops / d["median_ms"] / 1e9, 1)
        per_launch = {"reps": 100, "warmup": 25, "warm": warm, "cold_scrub_512mib": cold}
        _log("per launch: warm median %.4f ms (min %.4f, p90 %.4f); cold median %.4f ms"
             % (warm["median_ms"], warm["min_ms"], warm["p90_ms"], cold["median_ms"]))

    attn = attention_sweep() if args.attention or not (args.no_attention or args.no_sweep) else None

    # the fused GEMM+ReLU epilogue in the same configuration
    relu_ms = time_gemm(fn, dA, dB, C, block, stages, threads, steps=max(10, args.steps // 2), warmup=args.warmup,
                        a_lead=a_lead, relu=True)
    _log("headline with fused ReLU: %.3f ms, %.1f TFLOP/s" % (relu_ms, flops / relu_ms / 1e9))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, A, B, min(args.cpu_rows, w.M), gpu_c=headline_c)
        _log("cpu oracle: %.4f TFLOP/s on %d threads" % (cpu["value"], cpu["cores"]))

    out = {
        "metric": "TFLOP/s (2MNK/t) and % of MFMA peak at 4096^3 fp16, per num_stages",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_launches": args.settle,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "f16" if w.dtype == inputs.F16 else "bf16",
        "data": "synthetic",
        "config": {"workload": "GEMM %s %dx%dx%d %s, fp32 accumulate" % (
                       w.layout.upper(), w.M, w.N, w.K, "fp16 uniform[-1,1]" if w.dtype == inputs.F16 else "bf16 normal(0,1)"),
                   "M": w.M, "N": w.N, "K": w.K, "layout": w.layout.upper(), "block": "%dx%dx%d" % tuple(block),
                   "num_stages": stages, "a_lead": a_lead, "threads": threads},
        "pct_peak": round(100 * tflops / PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(block, stages, a_lead, threads)},
        "cpu_baseline": cpu,
        "per_num_stages": sweep,
        "fused_relu": {"tflops": round(flops / relu_ms / 1e9, 2), "ms_per_step": round(relu_ms, 5)},
        "per_launch": per_launch,
        "clock": clock,
        "attention": attn,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
