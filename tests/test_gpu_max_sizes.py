"""GPU parity at the largest sizes the 32-bit buffer offsets accept: a
workgroup's A or B panel, its rows of C, and one attention head's Q and O
just under 2 GiB each (the limits gemm_check and attn_check enforce).

The GEMM operands are +-1, so every fp32 partial sum is an integer below
2^24 and exact whatever the summation order: C must equal the exact sum,
rounded once to fp16 (the oracle's rounding), bit for bit.  The attention
rows are checked against the float64 oracle within the error-model bound, and
the rows past the last query must keep their canary (the last block's padding
rows have store offsets past 2^31, which the kernel drops)."""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import gemm as og
from software_pipelined_tiled_03_amd import binding as pg
from software_pipelined_tiled_03_amd import inputs

import attn_error_model as em

pytestmark = pytest.mark.gpu

LIM = 1 << 31
ONE, MINUS_ONE = 0x3C00, 0xBC00  # fp16 encodings of +1 and -1


def signs(shape, seed):
    """+-1 as int8, and as fp16 on the GPU."""
    s = (np.random.default_rng(seed).integers(0, 2, size=shape, dtype=np.int8) * 2 - 1).astype(np.int8)
    bits = np.where(s > 0, ONE, MINUS_ONE).astype(np.uint16)
    return s, torch.from_numpy(bits.view(np.int16)).cuda().view(torch.float16)


def exact_fp16(sums):
    return og.encode(np.asarray(sums, dtype=np.float32), inputs.F16)


def host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_k_at_the_operand_panel_limit():
    # a 128-row panel of A (and of B) is 128 K 2 bytes: just under 2 GiB
    M, N, K = 128, 128, LIM // (2 * 128) - 8
    assert pg.gemm_check(pg.GEMM_NT, M, N, K, pg.GEMM_F16, 128, 128, 32, 3, 256, 160 * 1024) == pg.GEMM_OK
    a, dA = signs((M, K), 1201)
    b, dB = signs((N, K), 1202)
    C = pg.gemm_nt(dA, dB, block=(128, 128, 32), num_stages=3, threads=256)
    torch.cuda.synchronize()
    got = host(C)
    for r in (0, 77, M - 1):
        # a.b for +-1 vectors: K minus twice the number of differing signs
        want = K - 2 * np.count_nonzero(b != a[r], axis=1)
        assert np.array_equal(got[r], exact_fp16(want)), "row %d" % r


@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_n_at_the_c_rows_limit(layout):
    # a workgroup's 128 rows of C are 128 N 2 bytes: just under 2 GiB
    M, N, K = 128, LIM // (2 * 128) - 8, 64
    lay = pg.GEMM_NT if layout == "nt" else pg.GEMM_NN
    assert pg.gemm_check(lay, M, N, K, pg.GEMM_F16, 128, 128, 32, 3, 256, 160 * 1024) == pg.GEMM_OK
    a, dA = signs((M, K), 1203)
    b, dB = signs((N, K) if layout == "nt" else (K, N), 1204 + (layout == "nn"))
    fn = pg.gemm_nt if layout == "nt" else pg.gemm_nn
    C = fn(dA, dB, block=(128, 128, 32), num_stages=3, threads=256)
    torch.cuda.synchronize()
    bf = b.astype(np.float32)
    for r in (0, M - 1):
        want = (bf @ a[r].astype(np.float32)) if layout == "nt" else (a[r].astype(np.float32) @ bf)
        got = C[r].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, exact_fp16(want)), "%s row %d" % (layout, r)


def test_attention_query_rows_at_the_limit():
    # one head's Q and O are Sq x 128 x 2 bytes: just under 2 GiB; Sq is not a
    # multiple of block_M, so the last block has padding rows
    Sq, Skv, D = LIM // (2 * 128) - 8, 64, 128
    assert Sq % 256 != 0
    assert pg.attn_check(1, 1, 1, Sq, Skv, D, pg.GEMM_F16, 0, 256, 128, 2, 512, 160 * 1024) == pg.GEMM_OK
    g = torch.Generator(device="cuda")
    g.manual_seed(1205)
    q = torch.randn((1, 1, Sq, D), generator=g, device="cuda", dtype=torch.float32).half()
    w = inputs.attention_custom(inputs.F16, 1, 1, 1, 256, Skv, D, False, seed=1206)
    _, K, V = w.make()
    k = torch.from_numpy(K.view(np.int16)).cuda().view(torch.float16)
    v = torch.from_numpy(V.view(np.int16)).cuda().view(torch.float16)
    big = torch.full((Sq + 512, D), 7.0, dtype=torch.float16, device="cuda")
    out = big[:Sq].view(1, 1, Sq, D)
    pg.attention(q, k, v, out=out, block_M=256, block_N=128, num_stages=2, threads=512)
    torch.cuda.synchronize()
    assert bool((big[Sq:] == 7.0).all()), "a store landed past the last query row"
    rows = np.array([0, 1, 255, 256, Sq // 2, Sq - 249, Sq - 248, Sq - 2, Sq - 1])
    Qs = q[0, 0, torch.from_numpy(rows).cuda()].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    Qs = Qs[None, None]
    idx = np.arange(len(rows))
    want = oatt.attention_rows(Qs, K, V, inputs.F16, 0, 0, idx)
    R, A = oatt.attention_rows_weights(Qs, K, V, inputs.F16, 0, 0, idx)
    got = og.decode(host(out[0, 0, torch.from_numpy(rows).cuda()]), inputs.F16).astype(np.float64)
    bad = em.violations(got, want, R, A, inputs.F16, Skv, D)
    assert not bad.any(), "%d of %d outside the bound" % (int(bad.sum()), bad.size)
