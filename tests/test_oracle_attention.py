"""Pins for the attention oracle against facts that do not depend on it: the
library's float64 scaled-dot-product attention, closed forms (uniform
weights give running means of V; a single key gives V itself), invariances
(a key shift along a direction orthogonal to every query, repeated heads in a
group), and the flop count."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as oatt
from oracle import gemm as og
from software_pipelined_tiled_03_amd import inputs

F16, BF16 = inputs.F16, inputs.BF16


def enc(x, dtype):
    return og.encode(np.asarray(x, dtype=np.float32), dtype)


def rand(shape, seed, dtype):
    return enc(np.random.default_rng(seed).standard_normal(shape), dtype)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("B,H,Hkv,S,D", [(1, 2, 2, 7, 8), (2, 4, 2, 33, 16), (1, 6, 1, 20, 32)])
def test_matches_library_sdpa_in_float64(B, H, Hkv, S, D, dtype, causal):
    Q = rand((B, H, S, D), 1, dtype)
    K = rand((B, Hkv, S, D), 2, dtype)
    V = rand((B, Hkv, S, D), 3, dtype)
    got = oatt.attention(Q, K, V, dtype, causal=causal)
    q = torch.from_numpy(og.decode(Q, dtype).astype(np.float64))
    k = torch.from_numpy(og.decode(K, dtype).astype(np.float64)).repeat_interleave(H // Hkv, dim=1)
    v = torch.from_numpy(og.decode(V, dtype).astype(np.float64)).repeat_interleave(H // Hkv, dim=1)
    want = F.scaled_dot_product_attention(q, k, v, is_causal=causal).numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_average_the_visible_values(causal):
    S, D = 9, 4
    Q = enc(np.zeros((1, 1, S, D)), F16)
    K = rand((1, 1, S, D), 4, F16)
    V = rand((1, 1, S, D), 5, F16)
    v = og.decode(V, F16).astype(np.float64)[0, 0]
    want = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None] if causal else np.tile(v.mean(axis=0), (S, 1))
    assert np.allclose(oatt.attention(Q, K, V, F16, causal=causal)[0, 0], want, rtol=0, atol=1e-12)


def test_single_key_returns_its_value():
    Q = rand((2, 3, 5, 8), 6, BF16)
    K = rand((2, 3, 1, 8), 7, BF16)
    V = rand((2, 3, 1, 8), 8, BF16)
    got = oatt.attention(Q, K, V, BF16)
    want = np.broadcast_to(og.decode(V, BF16).astype(np.float64), got.shape)
    assert np.array_equal(got, want)


def test_first_causal_row_is_the_first_value():
    Q = rand((1, 2, 6, 16), 9, F16)
    K = rand((1, 2, 6, 16), 10, F16)
    V = rand((1, 2, 6, 16), 11, F16)
    got = oatt.attention(Q, K, V, F16, causal=True)
    assert np.array_equal(got[:, :, 0], og.decode(V, F16).astype(np.float64)[:, :, 0])


def test_large_scale_picks_the_best_matching_key():
    # orthonormal-ish keys: query i equals key perm[i], so with a huge scale
    # the softmax is one-hot on that key
    D = S = 8
    perm = np.random.default_rng(12).permutation(S)
    K = enc(np.eye(S)[None, None], F16)
    Q = enc(np.eye(S)[perm][None, None], F16)
    V = rand((1, 1, S, D), 13, F16)
    got = oatt.attention(Q, K, V, F16, scale=100.0)
    assert np.allclose(got[0, 0], og.decode(V, F16).astype(np.float64)[0, 0][perm], rtol=0, atol=1e-30)


def test_key_shift_orthogonal_to_queries_changes_nothing():
    # adding c to every key changes every score of a query by q.c; with q.c = 0 nothing changes
    S, D = 12, 8
    q = np.random.default_rng(14).standard_normal((S, D))
    q[:, -1] = 0.0
    c = np.zeros(D)
    c[-1] = 3.0
    k = np.random.default_rng(15).integers(-3, 4, (S, D)).astype(np.float64)
    Q, K1, K2 = enc(q[None, None], F16), enc(k[None, None], F16), enc((k + c)[None, None], F16)
    V = rand((1, 1, S, D), 16, F16)
    assert np.allclose(oatt.attention(Q, K1, V, F16), oatt.attention(Q, K2, V, F16), rtol=1e-13, atol=1e-13)


def test_heads_of_a_group_share_keys_and_values():
    Q1 = rand((1, 1, 10, 16), 17, F16)
    Q = np.concatenate([Q1] * 4, axis=1)            # 4 query heads, identical
    K = rand((1, 1, 10, 16), 18, F16)
    V = rand((1, 1, 10, 16), 19, F16)
    O = oatt.attention(Q, K, V, F16, causal=True)
    assert all(np.array_equal(O[:, h], O[:, 0]) for h in range(4))


def test_rows_agree_with_whole_and_flops():
    Q = rand((2, 2, 40, 16), 20, F16)
    K = rand((2, 1, 40, 16), 21, F16)
    V = rand((2, 1, 40, 16), 22, F16)
    whole = oatt.attention(Q, K, V, F16, causal=True, chunk=7)
    rows = [0, 5, 39]
    assert np.array_equal(oatt.attention_rows(Q, K, V, F16, 1, 1, rows, causal=True), whole[1, 1, rows])
    assert oatt.attention_flops(1, 1, 4, 4, 2) == 4 * 2 * 16
    assert oatt.attention_flops(1, 1, 4, 4, 2, causal=True) == 4 * 2 * 10


def test_rejects_bad_shapes():
    Q = rand((1, 3, 4, 8), 23, F16)
    K = rand((1, 2, 4, 8), 24, F16)
    with pytest.raises(ValueError):
        oatt.attention(Q, K, K, F16)
    with pytest.raises(ValueError):
        oatt.attention(Q[:, :2], K[:, :, :3], K[:, :, :3], F16, causal=True)
