"""GPU parity: the HIP path (called through the C-ABI binding) against the CPU
oracle, element by element, on the same seeded inputs.

Tolerance: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| for every compared element
(the correctness criterion of the code/04 README of the TileLang tutorial:
rtol = atol = 1e-2, fp16 in, fp32 accumulate).  Several results are correct:
the oracle sums k in ascending order, the matrix cores in their own order, so
only the tolerance is compared -- except where the exact result is
representable (identity B), which must match bit for bit, and across ring
depths, which must not change the GPU's own result at all (the pipeline only
changes when tiles arrive, never the accumulation order).
"""
import numpy as np
import pytest
import torch

from software_pipelined_tiled_03_amd import binding as pg
from software_pipelined_tiled_03_amd import inputs

pytestmark = pytest.mark.gpu

RTOL = ATOL = 1e-2
F16, BF16 = inputs.F16, inputs.BF16
TORCH_DT = {F16: torch.float16, BF16: torch.bfloat16}


def dev(u16, dtype):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(TORCH_DT[dtype])


def host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run(layout, A, B, dtype, M, N, K, block, stages, threads, out=None, a_lead=0):
    dA, dB = dev(A, dtype), dev(B, dtype)
    fn = pg.gemm_nt if layout == "nt" else pg.gemm_nn
    C = fn(dA.view(M, K), dB.view(B.shape), out=out, block=block, num_stages=stages, threads=threads,
           a_lead=a_lead)
    torch.cuda.synchronize()
    return host(C)


def assert_close(got, want, dtype, og, what=""):
    g = og.decode(got, dtype).astype(np.float64)
    w = og.decode(want, dtype).astype(np.float64)
    assert np.isfinite(g).all(), "non-finite GPU output " + what
    err = np.abs(g - w)
    bad = err > ATOL + RTOL * np.abs(w)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d elements outside tolerance; first %s; max err %.3g"
                             % (what, int(bad.sum()), bad.size, idx.tolist(), err.max()))


def sample_rows(M, tile_m, seed, extra=8):
    rng = np.random.default_rng(seed)
    rows = {0, 1, tile_m - 1, tile_m, M // 2, M - 2, M - 1}
    rows |= set(int(r) for r in rng.integers(0, M, extra))
    return sorted(r for r in rows if 0 <= r < M)


def oracle_rows(og, layout, A, B, dtype, rows):
    fn = og.gemm_nt if layout == "nt" else og.gemm_nn
    return np.concatenate([fn(A, B, dtype, rows=(r, r + 1)) for r in rows])


# --------------------------------------------------------------------------
# The measured workloads

def test_nt_f16_128_single_stage(oracle_gemm):
    w = inputs.workload("nt_f16_128")
    A, B = w.make()
    got = run("nt", A, B, F16, w.M, w.N, w.K, (128, 128, 32), 1, 256)
    assert_close(got, oracle_gemm.gemm_nt(A, B, F16), F16, oracle_gemm, "128^3 S=1")


def test_nt_f16_1024_stages_1_2_3(oracle_gemm):
    w = inputs.workload("nt_f16_1024")
    A, B = w.make()
    want = oracle_gemm.gemm_nt(A, B, F16)
    outs = []
    for s in (1, 2, 3):
        got = run("nt", A, B, F16, w.M, w.N, w.K, (128, 128, 32), s, 256)
        assert_close(got, want, F16, oracle_gemm, "1024^3 S=%d" % s)
        outs.append(got)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), "ring depth changed the result"


@pytest.mark.parametrize("threads", [128, 256, 512])
def test_nt_f16_4096_stage_sweep(oracle_gemm, threads):
    w = inputs.workload("nt_f16_4096")
    A, B = w.make()
    rows = sample_rows(w.M, 128, 3)
    want = oracle_rows(oracle_gemm, "nt", A, B, F16, rows)
    first = None
    for s in (1, 2, 3, 4, 6):
        got = run("nt", A, B, F16, w.M, w.N, w.K, (128, 128, 32), s, threads)
        assert_close(got[rows], want, F16, oracle_gemm, "4096^3 S=%d threads=%d" % (s, threads))
        if first is None:
            first = got
        else:
            assert np.array_equal(got, first), "S=%d changed the result" % s


@pytest.mark.parametrize("block", [(128, 128, 32), (128, 256, 64), (256, 128, 32)])
def test_nn_bf16_4096_tiles(oracle_gemm, block):
    w = inputs.workload("nn_bf16_4096")
    A, B = w.make()
    rows = sample_rows(w.M, block[0], 4)
    want = oracle_rows(oracle_gemm, "nn", A, B, BF16, rows)
    got = run("nn", A, B, BF16, w.M, w.N, w.K, block, 3, 256)
    assert_close(got[rows], want, BF16, oracle_gemm, "NN bf16 4096^3 tile %s" % (block,))


def test_nn_bf16_4096_over_budget_rejected():
    w = inputs.workload("nn_bf16_4096")
    dA = torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((w.K, w.N), dtype=torch.bfloat16, device="cuda")
    out = torch.full((w.M, w.N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pg.LdsBudgetError):
        pg.gemm_nn(dA, dB, out=out, block=(256, 256, 64), num_stages=4, threads=256)
    assert "LDS budget" in pg.last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "C was touched by a rejected call"


@pytest.mark.parametrize("threads", [256, 512])
def test_nt_f16_4096_leading_a_ring(oracle_gemm, threads):
    # 256x256x64: two stages plus one leading A tile fill the 160 KiB exactly
    w = inputs.workload("nt_f16_4096")
    A, B = w.make()
    rows = sample_rows(w.M, 256, 8)
    want = oracle_rows(oracle_gemm, "nt", A, B, F16, rows)
    got0 = run("nt", A, B, F16, w.M, w.N, w.K, (256, 256, 64), 2, threads)
    got1 = run("nt", A, B, F16, w.M, w.N, w.K, (256, 256, 64), 2, threads, a_lead=1)
    assert_close(got1[rows], want, F16, oracle_gemm, "4096^3 256x256x64 S=2 a_lead threads=%d" % threads)
    assert np.array_equal(got0, got1), "a_lead changed the result"


def test_ragged_4000x5000x3000(oracle_gemm):
    w = inputs.workload("nt_f16_ragged_4000x5000x3000")
    A, B = w.make()
    rows = sample_rows(w.M, 128, 5)
    want = oracle_rows(oracle_gemm, "nt", A, B, F16, rows)
    got = run("nt", A, B, F16, w.M, w.N, w.K, (128, 128, 32), 3, 256)
    assert_close(got[rows], want, F16, oracle_gemm, "ragged 4000x5000x3000")


def test_long_k_512x512x65536(oracle_gemm):
    w = inputs.workload("nt_f16_longk_512x512x65536")
    A, B = w.make()
    rows = sample_rows(w.M, 128, 6, extra=4)
    want = oracle_rows(oracle_gemm, "nt", A, B, F16, rows)
    first = None
    for s, lead in ((1, 0), (2, 0), (3, 0), (4, 0), (6, 0), (2, 1), (3, 1), (4, 1)):
        got = run("nt", A, B, F16, w.M, w.N, w.K, (128, 128, 32), s, 256, a_lead=lead)
        assert_close(got[rows], want, F16, oracle_gemm, "long K S=%d a_lead=%d" % (s, lead))
        if first is None:
            first = got
        else:
            assert np.array_equal(got, first)
    got = run("nt", A, B, F16, w.M, w.N, w.K, (256, 256, 64), 2, 512, a_lead=1)
    assert_close(got[rows], want, F16, oracle_gemm, "long K 256x256x64 S=2 a_lead")


def test_one_gpu_share_512x4096x4096(oracle_gemm):
    # rows 0..511 of the 4096^3 problem, in the configurations the bench sweeps;
    # in the headline configuration the share is bit for bit the same rows of
    # the whole product (a C tile does not depend on the tiles beside it)
    w = inputs.workload("nt_f16_shard8_512x4096x4096")
    A, B = w.make()
    rows = sample_rows(w.M, 128, 7, extra=4)
    want = oracle_rows(oracle_gemm, "nt", A, B, F16, rows)
    for block, s, th, lead in (((128, 128, 64), 3, 256, 0), ((128, 128, 32), 3, 512, 0), ((128, 256, 64), 2, 256, 0),
                               ((256, 256, 64), 2, 512, 1)):
        got = run("nt", A, B, F16, w.M, w.N, w.K, block, s, th, a_lead=lead)
        assert_close(got[rows], want, F16, oracle_gemm, "shard %s S=%d threads=%d" % (block, s, th))
    full = inputs.workload("nt_f16_4096")
    Af, Bf = full.make()
    whole = run("nt", Af, Bf, F16, full.M, full.N, full.K, (256, 256, 64), 2, 512, a_lead=1)
    assert np.array_equal(got, whole[:512]), "the share differs from the same rows of the whole product"


# --------------------------------------------------------------------------
# Every built tile, both layouts and dtypes, on a shape ragged in M, N and K

TILES = [(64, 128, 64, 256), (128, 128, 32, 128), (128, 128, 32, 256), (128, 128, 32, 512), (128, 128, 64, 256),
         (128, 128, 64, 512),
         (128, 256, 32, 256), (128, 256, 64, 256), (128, 256, 64, 512), (256, 128, 32, 256), (256, 128, 32, 512),
         (256, 128, 64, 256),
         (256, 256, 32, 256), (256, 256, 32, 512), (256, 256, 64, 256), (256, 256, 64, 512)]


@pytest.mark.parametrize("tile", TILES, ids=lambda t: "%dx%dx%d_t%d" % t)
@pytest.mark.parametrize("layout,dtype", [("nt", F16), ("nt", BF16), ("nn", F16), ("nn", BF16)])
def test_every_tile_ragged(oracle_gemm, tile, layout, dtype):
    bm, bn, bk, th = tile
    M, N, K = 2 * bm + 37, 2 * bn + 24, 5 * bk + 8   # ragged edges in all three dimensions
    wl = inputs.custom(layout, dtype, M, N, K, seed=bm * 7 + bn * 3 + bk + th + 97 * dtype)
    A, B = wl.make()
    fn = oracle_gemm.gemm_nt if layout == "nt" else oracle_gemm.gemm_nn
    want = fn(A, B, dtype)
    budget = 160 * 1024
    first = None
    for s, lead in ((1, 0), (2, 0), (3, 0), (2, 1), (3, 1)):
        if (s * (bm + bn) + lead * bm) * bk * 2 > budget:
            continue
        got = run(layout, A, B, dtype, M, N, K, (bm, bn, bk), s, th, a_lead=lead)
        what = "%s dtype=%d tile %s S=%d a_lead=%d" % (layout, dtype, tile, s, lead)
        assert_close(got, want, dtype, oracle_gemm, what)
        if first is None:
            first = got
        else:
            assert np.array_equal(got, first), what + " differs from S=1"


# --------------------------------------------------------------------------
# Exact cases, edge cases, invariants

@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_identity_b_is_exact(oracle_gemm, layout):
    M = K = 256
    A = inputs.random_matrix((M, K), 11, F16)
    I = np.eye(K, dtype=np.float32).astype(np.float16).view(np.uint16)
    got = run(layout, A, I, F16, M, K, K, (128, 128, 32), 3, 256)
    assert np.array_equal(got, A)


def test_k_zero_writes_zeros():
    out = torch.full((64, 96), 3.0, dtype=torch.float16, device="cuda")
    dA = torch.empty((64, 0), dtype=torch.float16, device="cuda")
    dB = torch.empty((96, 0), dtype=torch.float16, device="cuda")
    pg.gemm_nt(dA, dB, out=out, block=(128, 128, 32), num_stages=2)
    torch.cuda.synchronize()
    assert bool((out == 0).all())


@pytest.mark.parametrize("block,stages,threads,lead", [((128, 128, 32), 3, 256, 0), ((256, 256, 64), 2, 512, 1),
                                                       ((128, 128, 32), 1, 256, 0)])
def test_stamped_launch_writes_the_same_c_and_sane_counters(block, stages, threads, lead):
    w = inputs.workload("nt_f16_1024")
    A, B = w.make()
    dA, dB = dev(A, F16).view(w.M, w.K), dev(B, F16).view(w.N, w.K)
    plain = pg.gemm_nt(dA, dB, block=block, num_stages=stages, threads=threads, a_lead=lead)
    C, stamps = pg.gemm_stamped(pg.GEMM_NT, dA, dB, block=block, num_stages=stages, threads=threads, a_lead=lead)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), C.view(torch.int16))
    grid = (w.M // block[0]) * (w.N // block[1])
    s = stamps.view(-1, 6).cpu().numpy().astype(np.int64)
    assert s.shape == (grid, 6)
    # cycles: start <= after prologue <= after the K loop <= end; real time advances
    assert (s[:, 0] <= s[:, 1]).all() and (s[:, 1] <= s[:, 2]).all() and (s[:, 2] <= s[:, 3]).all()
    assert (s[:, 4] < s[:, 5]).all()
    clk = (s[:, 3] - s[:, 0]) / (s[:, 5] - s[:, 4]) * 0.1   # GHz
    assert 0.3 < float(np.median(clk)) < 3.0


def test_empty_m_or_n_is_a_noop():
    dA = torch.ones((0, 64), dtype=torch.float16, device="cuda")
    dB = torch.ones((32, 64), dtype=torch.float16, device="cuda")
    assert pg.gemm_nt(dA, dB).shape == (0, 32)
    dA = torch.ones((16, 64), dtype=torch.float16, device="cuda")
    dB = torch.ones((0, 64), dtype=torch.float16, device="cuda")
    assert pg.gemm_nt(dA, dB).shape == (16, 0)


def test_tiny_shape(oracle_gemm):
    A = inputs.random_matrix((1, 8), 12, F16)
    B = inputs.random_matrix((1, 8), 13, F16)
    got = run("nt", A, B, F16, 1, 1, 8, (128, 128, 32), 2, 256)
    assert_close(got, oracle_gemm.gemm_nt(A, B, F16), F16, oracle_gemm, "1x1x8")


def test_writes_stay_inside_c(oracle_gemm):
    # C sits inside a larger buffer; the guard regions around it must survive
    M, N, K = 200, 136, 96
    A = inputs.random_matrix((M, K), 14, F16)
    B = inputs.random_matrix((N, K), 15, F16)
    pad = 4096
    buf = torch.full((pad + M * N + pad,), -5.0, dtype=torch.float16, device="cuda")
    C = buf[pad:pad + M * N].view(M, N)
    pg.gemm_nt(dev(A, F16).view(M, K), dev(B, F16).view(N, K), out=C, block=(128, 128, 32), num_stages=3)
    torch.cuda.synchronize()
    assert bool((buf[:pad] == -5.0).all()) and bool((buf[pad + M * N:] == -5.0).all())
    assert_close(host(C), oracle_gemm.gemm_nt(A, B, F16), F16, oracle_gemm, "guarded C")


def test_odd_n_scalar_epilogue(oracle_gemm):
    M, N, K = 130, 67, 40   # N % 4 != 0: scalar stores
    A = inputs.random_matrix((M, K), 16, F16)
    B = inputs.random_matrix((N, K), 17, F16)
    got = run("nt", A, B, F16, M, N, K, (128, 128, 32), 2, 256)
    assert_close(got, oracle_gemm.gemm_nt(A, B, F16), F16, oracle_gemm, "odd N")


def test_repeated_runs_bit_identical():
    w = inputs.workload("nt_f16_1024")
    A, B = w.make()
    dA, dB = dev(A, F16).view(1024, 1024), dev(B, F16).view(1024, 1024)
    outs = [host(pg.gemm_nt(dA, dB, block=(256, 256, 64), num_stages=2)) for _ in range(3)]
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])


def test_runs_on_callers_stream(oracle_gemm):
    w = inputs.workload("nt_f16_1024")
    A, B = w.make()
    dA, dB = dev(A, F16).view(1024, 1024), dev(B, F16).view(1024, 1024)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = pg.gemm_nt(dA, dB, block=(128, 128, 32), num_stages=4)
    s.synchronize()
    assert_close(host(C), oracle_gemm.gemm_nt(A, B, F16), F16, oracle_gemm, "side stream")


def test_alignment_and_argument_errors():
    dA = torch.empty((64, 20), dtype=torch.float16, device="cuda")
    dB = torch.empty((64, 20), dtype=torch.float16, device="cuda")
    with pytest.raises(pg.AlignmentError):
        pg.gemm_nt(dA, dB)          # K = 20 is not a multiple of 8
    dA = torch.empty((64, 32), dtype=torch.float16, device="cuda")
    dB = torch.empty((64, 32), dtype=torch.float16, device="cuda")
    with pytest.raises(pg.UnsupportedConfigError):
        pg.gemm_nt(dA, dB, block=(64, 64, 32))
    with pytest.raises(pg.GemmArgumentError):
        pg.gemm_nt(dA, dB, threads=100)
    assert pg.gemm_lds_budget() == 160 * 1024


# --------------------------------------------------------------------------
# The fused ReLU epilogue (gemm_nt_relu / gemm_nn_relu)

def run_relu(layout, A, B, dtype, M, N, K, block, stages, threads, a_lead=0):
    dA, dB = dev(A, dtype), dev(B, dtype)
    fn = pg.gemm_nt if layout == "nt" else pg.gemm_nn
    C = fn(dA.view(M, K), dB.view(B.shape), block=block, num_stages=stages, threads=threads, a_lead=a_lead,
           relu=True)
    torch.cuda.synchronize()
    return host(C)


def relu_of(bits, dtype, og):
    return np.where(og.decode(bits, dtype) > 0, bits, np.uint16(0))


@pytest.mark.parametrize("tile", [(128, 128, 32, 256), (256, 256, 64, 256), (128, 256, 64, 256)],
                         ids=lambda t: "%dx%dx%d_t%d" % t)
@pytest.mark.parametrize("layout,dtype", [("nt", F16), ("nn", BF16)])
def test_relu_ragged(oracle_gemm, tile, layout, dtype):
    bm, bn, bk, th = tile
    M, N, K = 2 * bm + 37, 2 * bn + 24, 5 * bk + 8
    wl = inputs.custom(layout, dtype, M, N, K, seed=311 + bm + bn + bk + dtype)
    A, B = wl.make()
    fn = oracle_gemm.gemm_nt if layout == "nt" else oracle_gemm.gemm_nn
    want = fn(A, B, dtype, relu=True)
    plain = run(layout, A, B, dtype, M, N, K, (bm, bn, bk), 2, th)
    got = run_relu(layout, A, B, dtype, M, N, K, (bm, bn, bk), 2, th)
    assert_close(got, want, dtype, oracle_gemm, "relu %s %s" % (layout, tile))
    # the fused epilogue is exactly ReLU of the kernel's own result
    assert np.array_equal(got, relu_of(plain, dtype, oracle_gemm))
    assert (got == 0).any() and (got != 0).any()


def test_relu_headline_configuration(oracle_gemm):
    w = inputs.workload("nt_f16_4096")
    A, B = w.make()
    rows = sample_rows(w.M, 256, 21, extra=4)
    want = np.concatenate([oracle_gemm.gemm_nt(A, B, F16, rows=(r, r + 1), relu=True) for r in rows])
    got = run_relu("nt", A, B, F16, w.M, w.N, w.K, (256, 256, 64), 2, 512, a_lead=1)
    assert_close(got[rows], want, F16, oracle_gemm, "relu 4096^3 256x256x64 S=2+A")
    plain = run("nt", A, B, F16, w.M, w.N, w.K, (256, 256, 64), 2, 512, a_lead=1)
    assert np.array_equal(got, relu_of(plain, F16, oracle_gemm))


def test_relu_nan_sum_gives_positive_zero(oracle_gemm):
    M, N, K = 64, 128, 64
    A = inputs.random_matrix((M, K), 22, F16)
    B = inputs.random_matrix((N, K), 23, F16)
    A[5, 7] = 0x7E00   # quiet NaN: row 5 of C is NaN, and +0 after the epilogue
    plain = run("nt", A, B, F16, M, N, K, (128, 128, 32), 2, 256)
    got = run_relu("nt", A, B, F16, M, N, K, (128, 128, 32), 2, 256)
    assert np.isnan(oracle_gemm.decode(plain[5], F16)).all()
    assert (got[5] == 0).all()
    assert_close(np.delete(got, 5, axis=0), np.delete(oracle_gemm.gemm_nt(A, B, F16, relu=True), 5, axis=0), F16,
                 oracle_gemm, "relu rows without NaN")
