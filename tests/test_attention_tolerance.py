"""The attention parity bound (tests/attn_error_model.py) checked on the CPU:
it admits the kernel's arithmetic emulated in numpy (key tiles of 128, fp32
scores, a reference max per 32-query block that moves only when some query's
max has grown by more than 2^8, fp32 exp2, P rounded to the input dtype for
both the second product and the row sum, fp32 sums, output rounded), and it
rejects the two plausible mistakes the GPU comparison must catch: one 64-key
tile left out of the softmax, and the causal diagonal shifted by one key."""
import numpy as np
import pytest

from oracle import attention as oatt
from oracle import gemm as og
from software_pipelined_tiled_03_amd import inputs

import attn_error_model as em

F16, BF16 = inputs.F16, inputs.BF16
NP16 = {F16: np.float16}


def emulate_kernel(Q, K, V, dtype, causal, bn=128, block=32):
    """fp32 emulation of the kernel's numerics for head (0, 0), all rows."""
    q = og.decode(Q[0, 0], dtype).astype(np.float32)
    k = og.decode(K[0, 0], dtype).astype(np.float32)
    v = og.decode(V[0, 0], dtype).astype(np.float32)
    sq, skv = q.shape[0], k.shape[0]
    sl2 = np.float32(1.0 / np.sqrt(q.shape[1]) * 1.4426950408889634)
    m = np.full((sq, 1), -np.inf, np.float32)
    l = np.zeros((sq, 1), np.float32)
    acc = np.zeros((sq, v.shape[1]), np.float32)
    with np.errstate(invalid="ignore"):
        for k0 in range(0, skv, bn):
            s = q @ k[k0:k0 + bn].T
            if causal:
                keys = np.arange(k0, min(k0 + bn, skv))
                s = np.where(keys[None, :] <= np.arange(sq)[:, None], s, -np.inf).astype(np.float32)
            mx = s.max(axis=1, keepdims=True)
            for r0 in range(0, sq, block):
                rr = slice(r0, r0 + block)
                if ((mx[rr] - m[rr]) * sl2 > 8).any():
                    m_new = np.maximum(m[rr], mx[rr])
                    alpha = np.exp2((m[rr] - m_new) * sl2).astype(np.float32)
                    l[rr] *= alpha
                    acc[rr] *= alpha
                    m[rr] = m_new
            e = np.exp2(s * sl2 - m * sl2).astype(np.float32)
            p = og.decode(og.encode(e, dtype), dtype).astype(np.float32)     # P rounded to the input dtype
            l += p.sum(axis=1, dtype=np.float32, keepdims=True)
            acc += p @ v[k0:k0 + bn]
    o = acc / l
    return og.decode(og.encode(o.astype(np.float32), dtype), dtype).astype(np.float64)


def problem(dtype, causal, S=1024, nrows=None, grow=False):
    w = inputs.attention_custom(dtype, 1, 1, 1, S, S, 128, causal, seed=4242 + dtype + 2 * causal)
    Q, K, V = w.make()
    if grow:
        # key j scaled by 2^e_j, e_j rising from 0 to 6: the reference max moves on many tiles
        e = (7 * np.arange(S)) // S
        K = og.encode(og.decode(K, dtype).astype(np.float32) * np.exp2(e.astype(np.float32))[None, None, :, None],
                      dtype)
    rows = np.arange(S if nrows is None else nrows)
    want = oatt.attention_rows(Q, K, V, dtype, 0, 0, rows, causal=causal)
    R, A = oatt.attention_rows_weights(Q, K, V, dtype, 0, 0, rows, causal=causal)
    return Q, K, V, want, R, A


def rounded(x, dtype):
    return og.decode(og.encode(x.astype(np.float32), dtype), dtype).astype(np.float64)


@pytest.mark.parametrize("grow", [False, True], ids=["normal", "growing_keys"])
@pytest.mark.parametrize("dtype,causal", [(F16, False), (F16, True), (BF16, True)])
def test_bound_admits_the_kernels_arithmetic(dtype, causal, grow):
    Q, K, V, want, R, A = problem(dtype, causal, grow=grow)
    got = emulate_kernel(Q, K, V, dtype, causal)
    bad = em.violations(got, want, R, A, dtype, K.shape[2], 128)
    assert not bad.any(), "%d elements outside the bound" % int(bad.sum())


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_bound_rejects_a_dropped_key_tile(dtype):
    # 4096 keys, one of their 64 tiles of 64 left out: a 1.6 % change of the
    # softmax support (first 512 queries)
    Q, K, V, want, R, A = problem(dtype, False, S=4096, nrows=512)
    keep = np.r_[0:64, 128:K.shape[2]]                 # keys 64..127 (one 64-key tile) left out
    bad_ref = oatt.attention_rows(Q, K[:, :, keep], V[:, :, keep], dtype, 0, 0, np.arange(512))
    bad = em.violations(rounded(bad_ref, dtype), want, R, A, dtype, K.shape[2], 128)
    assert bad.sum() > 100
    # the GEMM tolerance (1e-2 + 1e-2 |ref|) lets most of this mistake through
    loose = np.abs(rounded(bad_ref, dtype) - want) > 1e-2 + 1e-2 * np.abs(want)
    assert loose.mean() < 0.1


def test_bound_rejects_a_shifted_causal_diagonal():
    dtype = F16
    Q, K, V, want, R, A = problem(dtype, True)
    S = Q.shape[2]
    # query i also sees key i + 1
    rows = np.arange(S - 1)
    q = og.decode(Q[0, 0, rows], dtype).astype(np.float64)
    k = og.decode(K[0, 0], dtype).astype(np.float64)
    v = og.decode(V[0, 0], dtype).astype(np.float64)
    s = (q @ k.T) / np.sqrt(128)
    s = np.where(np.arange(S)[None, :] <= rows[:, None] + 1, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    shifted = (p / p.sum(axis=1, keepdims=True)) @ v
    bad = em.violations(rounded(shifted, dtype), want[rows], R[rows], A[rows], dtype, S, 128)
    assert bad[:64].any(axis=1).all()       # every early row, where one key more is a large change
    assert bad.sum() > 1000
