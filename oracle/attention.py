"""Plain attention: the KV-length reduction loop the pages pipeline like GEMM's
K loop.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes, in float64 from the exactly widened fp16/bf16 inputs:

    S[i, j] = scale * sum_d Q[b, h, i, d] * K[b, h // groups, j, d]
    P[i, :] = softmax over the visible keys j of S[i, :]     (j <= i if causal)
    O[b, h, i, :] = sum_j P[i, j] * V[b, h // groups, j, :]

Sources:
  * TileLang tutorial, chapter 11, section 1.4: the attention KV-length loop
    is one of the long reduction loops where pipelining pays, like the GEMM K
    loop; section 3.8: the flashattn(batch, heads, seq_len, dim, is_causal,
    groups, block_M, block_N, num_stages, threads) example of a tuned kernel.
  * Tilelang-Learning notes "Stage 04 - GEMM": QK^T and P@V are the GEMMs of
    attention.
Readings where the pages are silent: the scale is 1/sqrt(dim) unless given;
`groups` query heads share one KV head (head h reads KV head h // groups, with
heads = groups * kv_heads); causal means key j is visible to query i iff
j <= i, for seq_q == seq_kv; the softmax is the exact one (max-subtracted
exponentials normalised by their sum).

The result is returned in float64 (not rounded to the input format): the GPU
path is compared with it by tolerance.
"""
import numpy as np

from . import gemm as _gemm


def _widen(bits, dtype):
    return _gemm.decode(np.ascontiguousarray(bits), dtype).astype(np.float64)


def attention_rows(Q, K, V, dtype, b, h, rows, causal=False, scale=None):
    """O[b, h, rows, :] as float64 [len(rows), D].  Q: uint16 [B, H, Sq, D];
    K, V: uint16 [B, Hkv, Skv, D]."""
    B, H, Sq, D = Q.shape
    Hkv, Skv = K.shape[1], K.shape[2]
    if H % Hkv or K.shape != V.shape or K.shape[0] != B or K.shape[3] != D:
        raise ValueError("shapes do not match (heads must be a multiple of kv_heads)")
    if causal and Sq != Skv:
        raise ValueError("causal attention needs seq_q == seq_kv")
    g = H // Hkv
    s = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    q = _widen(Q[b, h, rows], dtype)                      # [R, D]
    k = _widen(K[b, h // g], dtype)                       # [Skv, D]
    v = _widen(V[b, h // g], dtype)                       # [Skv, D]
    S = s * (q @ k.T)                                     # [R, Skv]
    if causal:
        S = np.where(np.arange(Skv)[None, :] <= rows[:, None], S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    P = E / E.sum(axis=1, keepdims=True)
    return P @ v


def attention_rows_weights(Q, K, V, dtype, b, h, rows, causal=False, scale=None):
    """The magnitudes an error bound for O[b, h, rows, :] is built from, in
    float64: R[r, d] = sum_j P[r, j] |V[j, d]| (P as in attention_rows) and
    A[r] = scale * max_j sum_d |Q[r, d] K[j, d]| over the visible keys."""
    B, H, Sq, D = Q.shape
    Hkv, Skv = K.shape[1], K.shape[2]
    g = H // Hkv
    s = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    q = _widen(Q[b, h, rows], dtype)
    k = _widen(K[b, h // g], dtype)
    v = _widen(V[b, h // g], dtype)
    S = s * (q @ k.T)
    Aqk = s * (np.abs(q) @ np.abs(k).T)
    if causal:
        vis = np.arange(Skv)[None, :] <= rows[:, None]
        S = np.where(vis, S, -np.inf)
        Aqk = np.where(vis, Aqk, 0.0)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    P = E / E.sum(axis=1, keepdims=True)
    return P @ np.abs(v), Aqk.max(axis=1)


def attention(Q, K, V, dtype, causal=False, scale=None, chunk=512):
    """The whole O [B, H, Sq, D] in float64 (row chunks of `chunk` queries)."""
    B, H, Sq, D = Q.shape
    O = np.empty((B, H, Sq, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, chunk):
                rows = np.arange(r0, min(Sq, r0 + chunk))
                O[b, h, r0:r0 + len(rows)] = attention_rows(Q, K, V, dtype, b, h, rows, causal, scale)
    return O


def attention_flops(B, H, Sq, Skv, D, causal=False):
    """2 * (QK^T) + 2 * (PV) multiply-adds over the visible (query, key) pairs:
    4 * B * H * D * pairs, pairs = Sq * Skv, or Sq * (Sq + 1) / 2 when causal."""
    pairs = Sq * (Sq + 1) // 2 if causal else Sq * Skv
    return 4 * B * H * D * pairs
