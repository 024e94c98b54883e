"""GPU parity of the attention forward pass (the KV-length loop on the same
pipelined LDS ring) against the float64 oracle, element by element, within
the error bound of tests/attn_error_model.py: (3 u_in + u_out + 2 Skv u32 +
2 D u32 A_i) sum_j P_ij |V_jd|, derived from the kernel's arithmetic (fp32
scores and sums, P rounded to the input dtype for the second product and the
row sum, output rounded); a CPU test shows it rejects one dropped key tile and a shifted causal
diagonal.  The result must not depend on the ring depth."""
import numpy as np
import pytest
import torch

import software_pipelined_tiled_03_amd as pg
from oracle import attention as oatt
from oracle import gemm as og
from software_pipelined_tiled_03_amd import inputs

import attn_error_model as em

pytestmark = pytest.mark.gpu

F16, BF16 = inputs.F16, inputs.BF16
TORCH_DT = {F16: torch.float16, BF16: torch.bfloat16}
# (block_M, block_N, threads); 256 queries on 256 threads = two 32-query blocks per wave
TILES = [(128, 64, 256), (256, 64, 512), (128, 128, 256), (256, 128, 512), (256, 64, 256)]


def dev(u16, dtype):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(TORCH_DT[dtype])


def host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run(w, Q, K, V, tile, stages, scale=0.0):
    bm, bn, th = tile
    O = pg.attention(dev(Q, w.dtype), dev(K, w.dtype), dev(V, w.dtype), causal=w.causal, scale=scale, block_M=bm,
                     block_N=bn, num_stages=stages, threads=th)
    torch.cuda.synchronize()
    return host(O)


def weights(Q, K, V, dtype, causal, scale=None):
    """(R, A) of the error bound for every (b, h, row), stacked like O."""
    B, H, Sq, D = Q.shape
    R = np.empty((B, H, Sq, D))
    A = np.empty((B, H, Sq))
    for b in range(B):
        for h in range(H):
            R[b, h], A[b, h] = oatt.attention_rows_weights(Q, K, V, dtype, b, h, np.arange(Sq), causal, scale)
    return R, A


def assert_close(got_bits, want, R, A, dtype, skv, what):
    g = og.decode(got_bits, dtype).astype(np.float64)
    assert np.isfinite(g).all(), what + ": non-finite output"
    D = want.shape[-1]
    bad = em.violations(g.reshape(-1, D), want.reshape(-1, D), R.reshape(-1, D), A.reshape(-1), dtype, skv, D)
    err = np.abs(g - want)
    assert not bad.any(), "%s: %d of %d outside the bound, max err %.3g" % (what, int(bad.sum()), bad.size, err.max())


@pytest.mark.parametrize("tile", TILES, ids=lambda t: "bm%d_bn%d_t%d" % t)
@pytest.mark.parametrize("dtype,causal", [(F16, False), (F16, True), (BF16, True)])
def test_ragged_every_tile_every_depth(tile, dtype, causal):
    # 300 queries and keys: ragged against block_M and block_N; 4 query heads on 2 KV heads
    w = inputs.attention_custom(dtype, 2, 4, 2, 300, 300, 128, causal, seed=700 + dtype + 2 * causal + tile[1])
    Q, K, V = w.make()
    want = oatt.attention(Q, K, V, dtype, causal=causal)
    R, A = weights(Q, K, V, dtype, causal)
    first = None
    for s in (1, 2, 3, 4):
        if pg.attn_check(2, 4, 2, 300, 300, 128, dtype, int(causal), tile[0], tile[1], s, tile[2], 160 * 1024):
            continue
        got = run(w, Q, K, V, tile, s)
        assert_close(got, want, R, A, dtype, 300, "tile %s S=%d" % (tile, s))
        if first is None:
            first = got
        else:
            assert np.array_equal(got, first), "ring depth %d changed the result" % s


@pytest.mark.parametrize("Sq,Skv", [(200, 333), (1, 77), (130, 1), (64, 64)])
def test_unequal_and_tiny_lengths(Sq, Skv):
    w = inputs.attention_custom(F16, 1, 2, 1, Sq, Skv, 128, False, seed=800 + Sq + Skv)
    Q, K, V = w.make()
    want = oatt.attention(Q, K, V, F16)
    R, A = weights(Q, K, V, F16, False)
    assert_close(run(w, Q, K, V, (128, 64, 256), 2), want, R, A, F16, Skv, "Sq=%d Skv=%d" % (Sq, Skv))


def test_explicit_scale():
    w = inputs.attention_custom(BF16, 1, 2, 2, 257, 257, 128, True, seed=900)
    Q, K, V = w.make()
    want = oatt.attention(Q, K, V, BF16, causal=True, scale=0.3)
    R, A = weights(Q, K, V, BF16, True, 0.3)
    assert_close(run(w, Q, K, V, (256, 64, 512), 3, scale=0.3), want, R, A, BF16, 257, "scale 0.3")


@pytest.mark.parametrize("tile", [(128, 64, 256), (256, 64, 256), (256, 128, 512)], ids=lambda t: "bm%d_bn%d_t%d" % t)
@pytest.mark.parametrize("name", ["attn_f16_b4_h32_s4096_d128", "attn_f16_b4_h32_s4096_d128_causal",
                                  "attn_bf16_b2_h32_kv8_s2048_d128_causal"])
def test_full_size_sampled_rows(name, tile):
    w = inputs.attention_workload(name)
    Q, K, V = w.make()
    got = run(w, Q, K, V, tile, 2)
    rng = np.random.default_rng(11)
    for b, h in [(0, 0), (w.batch - 1, w.heads - 1), (w.batch // 2, 5)]:
        rows = np.unique(np.concatenate([[0, 1, 127, 128, w.seq_q - 1], rng.integers(0, w.seq_q, 8)]))
        want = oatt.attention_rows(Q, K, V, w.dtype, b, h, rows, causal=w.causal)
        R, A = oatt.attention_rows_weights(Q, K, V, w.dtype, b, h, rows, causal=w.causal)
        assert_close(got[b, h, rows], want, R, A, w.dtype, w.seq_kv, "%s b=%d h=%d" % (name, b, h))


def test_errors_leave_output_untouched():
    q = torch.zeros((1, 3, 64, 128), dtype=torch.float16, device="cuda")
    k = torch.zeros((1, 2, 64, 128), dtype=torch.float16, device="cuda")
    out = torch.full_like(q, 5.0)
    with pytest.raises(pg.GemmArgumentError):
        pg.attention(q, k, k, out=out)     # 3 heads on 2 KV heads
    with pytest.raises(pg.LdsBudgetError):
        pg.attention(q[:, :2], k, k, out=out[:, :2].contiguous(), block_N=128, num_stages=3)
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())


def scaled_keys(K, dtype, profile):
    """K with key j multiplied by 2^e_j (exact in the dtype): e_j rising from
    0 to 6 over the sequence ("grow": the row max keeps moving, by less and by
    more than 2^8 in the exponent from tile to tile) or falling from 6 to 0
    ("shrink": the first tile holds the max)."""
    S = K.shape[2]
    e = (7 * np.arange(S)) // S
    if profile == "shrink":
        e = 6 - e
    k = og.decode(K, dtype).astype(np.float32) * np.exp2(e.astype(np.float32))[None, None, :, None]
    return og.encode(k, dtype)


@pytest.mark.parametrize("profile", ["grow", "shrink"])
@pytest.mark.parametrize("dtype,causal", [(F16, False), (F16, True), (BF16, False)])
def test_reference_max_moves_across_tiles(profile, dtype, causal):
    # key magnitudes change by powers of two along the sequence, so the
    # softmax's reference max is moved (O and l rescaled) on some tiles and
    # kept on others, with P up to 256
    w = inputs.attention_custom(dtype, 1, 2, 1, 1024, 1024, 128, causal, seed=950 + dtype + 2 * causal)
    Q, K, V = w.make()
    K = scaled_keys(K, dtype, profile)
    want = oatt.attention(Q, K, V, dtype, causal=causal)
    R, A = weights(Q, K, V, dtype, causal)
    first = None
    for tile, s in (((256, 128, 512), 2), ((256, 64, 512), 4), ((128, 64, 256), 3)):
        got = run(w, Q, K, V, tile, s)
        assert_close(got, want, R, A, dtype, 1024, "%s tile %s S=%d" % (profile, tile, s))
        if tile[1] == 64:
            if first is None:
                first = got
            else:
                assert np.array_equal(got, first), "the result depends on the workgroup shape at block_N 64"


@pytest.mark.parametrize("tile", [(256, 128, 512), (256, 64, 256), (128, 64, 256)], ids=lambda t: "bm%d_bn%d_t%d" % t)
def test_rows_past_sq_are_not_written(tile):
    # O inside a larger buffer: 300 query rows per head is ragged against
    # block_M, so the last query block has padding rows, whose stores must be
    # dropped; the rows after the last head must keep their canary
    w = inputs.attention_custom(F16, 1, 2, 1, 300, 300, 128, False, seed=990)
    Q, K, V = w.make()
    q, k, v = dev(Q, F16), dev(K, F16), dev(V, F16)
    big = torch.full((2 * 300 + 512, 128), 7.0, dtype=torch.float16, device="cuda")
    out = big[:600].view(1, 2, 300, 128)
    bm, bn, th = tile
    pg.attention(q, k, v, out=out, block_M=bm, block_N=bn, num_stages=2, threads=th)
    torch.cuda.synchronize()
    assert bool((big[600:] == 7.0).all()), "a store landed past the last query row"
    want = oatt.attention(Q, K, V, F16)
    R, A = weights(Q, K, V, F16, False)
    assert_close(host(out), want, R, A, F16, 300, "tile %s" % (tile,))


# at D = 64 two 32-query blocks per wave also fit with two waves per SIMD
TILES_D64 = TILES + [(512, 64, 512), (512, 128, 512)]


@pytest.mark.parametrize("tile", TILES_D64, ids=lambda t: "bm%d_bn%d_t%d" % t)
@pytest.mark.parametrize("dtype,causal", [(F16, True), (BF16, False)])
def test_head_dim_64_every_tile_every_depth(tile, dtype, causal):
    # D = 64: one K half, V rows of 128 bytes with their own swizzle; ragged
    # lengths, 4 query heads on 2 KV heads
    w = inputs.attention_custom(dtype, 2, 4, 2, 300, 300, 64, causal, seed=1300 + dtype + 2 * causal + tile[1])
    Q, K, V = w.make()
    want = oatt.attention(Q, K, V, dtype, causal=causal)
    R, A = weights(Q, K, V, dtype, causal)
    first = None
    for s in (1, 2, 3, 4):
        if pg.attn_check(2, 4, 2, 300, 300, 64, dtype, int(causal), tile[0], tile[1], s, tile[2], 160 * 1024):
            continue
        got = run(w, Q, K, V, tile, s)
        assert_close(got, want, R, A, dtype, 300, "D=64 tile %s S=%d" % (tile, s))
        if first is None:
            first = got
        else:
            assert np.array_equal(got, first), "ring depth %d changed the result" % s


@pytest.mark.parametrize("B,H,Hkv", [(3, 6, 3), (1, 5, 5), (2, 12, 4), (2, 8, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_every_work_item_once(B, H, Hkv, causal):
    # head counts that are not multiples of the 8 XCDs, query heads sharing KV
    # heads (all of them one KV head in the last case), and several query
    # blocks per head: every (head, query block) must
    # be computed by exactly one workgroup in both work orders, so O starts as
    # NaN and every element must come out finite and inside the bound
    w = inputs.attention_custom(F16, B, H, Hkv, 700, 700, 128, causal, seed=1300 + 7 * B + H + causal)
    Q, K, V = w.make()
    want = oatt.attention(Q, K, V, F16, causal=causal)
    R, A = weights(Q, K, V, F16, causal)
    for bm, bn, th in [(256, 128, 512), (256, 64, 512)]:
        O = torch.full((B, H, 700, 128), float("nan"), dtype=torch.float16, device="cuda")
        pg.attention(dev(Q, F16), dev(K, F16), dev(V, F16), causal=causal, out=O, block_M=bm, block_N=bn,
                     num_stages=2, threads=th)
        torch.cuda.synchronize()
        assert_close(host(O), want, R, A, F16, 700, "B=%d H=%d Hkv=%d tile %d x %d" % (B, H, Hkv, bm, bn))


@pytest.mark.parametrize("B,H,Hkv,S,D,causal", [(1, 4, 4, 600, 128, False), (2, 4, 2, 600, 128, True),
                                                 (1, 4, 4, 600, 64, True), (1, 2, 2, 1100, 64, False)])
def test_default_configuration(B, H, Hkv, S, D, causal):
    # no tile arguments: the configuration comes from attn_default_config
    w = inputs.attention_custom(F16, B, H, Hkv, S, S, D, causal, seed=1400 + S + D + causal)
    Q, K, V = w.make()
    want = oatt.attention(Q, K, V, F16, causal=causal)
    R, A = weights(Q, K, V, F16, causal)
    O = pg.attention(dev(Q, F16), dev(K, F16), dev(V, F16), causal=causal)
    torch.cuda.synchronize()
    assert_close(host(O), want, R, A, F16, S, "default configuration %s" % (pg.attn_default_config(B, H, S, D,
                                                                                                     causal),))
