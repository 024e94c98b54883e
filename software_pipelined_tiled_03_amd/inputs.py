"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random numbers and stores them as 16-bit encodings; it
holds none of the GEMM's arithmetic.  The GPU path and the CPU oracle both take
their operands from here, byte for byte.

Recipe (the pages publish no dataset; every input is synthetic):
  * generator: numpy.random.default_rng(seed);
  * fp16 operands: uniform(-1, 1) drawn as float32, rounded to binary16 by
    numpy's float32 -> float16 cast (round to nearest, ties to even);
  * bf16 operands: standard normal drawn as float32, rounded to bfloat16 by
    torch's CPU float32 -> bfloat16 cast (round to nearest, ties to even);
  * A is [M, K]; B is [N, K] for the NT form and [K, N] for the NN form; all
    contiguous row-major; returned as numpy uint16 arrays of encodings;
  * seeds: A uses 1000 * workload_id, B uses 1000 * workload_id + 1; the
    ragged workload uses 5000/5001 and the long-K workload 5100/5101.
"""
from dataclasses import dataclass
from typing import Tuple

import numpy as np

F16 = 0
BF16 = 1


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def random_matrix(shape: Tuple[int, int], seed: int, dtype: int, dist: str = None) -> np.ndarray:
    """A seeded random matrix of 16-bit encodings.

    dist defaults to "uniform" (in [-1, 1)) for fp16 and "normal" for bf16.
    """
    rng = np.random.default_rng(seed)
    if dist is None:
        dist = "uniform" if dtype == F16 else "normal"
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    elif dist == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
    else:
        raise ValueError("unknown distribution %r" % dist)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return _to_bf16_bits(x)
    raise ValueError("unknown dtype %r" % dtype)


@dataclass(frozen=True)
class Workload:
    name: str
    layout: str  # "nt" (B [N,K]) or "nn" (B [K,N])
    dtype: int
    M: int
    N: int
    K: int
    seed_a: int
    seed_b: int

    def b_shape(self):
        return (self.N, self.K) if self.layout == "nt" else (self.K, self.N)

    def make(self):
        """(A, B) as uint16 encodings."""
        A = random_matrix((self.M, self.K), self.seed_a, self.dtype)
        B = random_matrix(self.b_shape(), self.seed_b, self.dtype)
        return A, B

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


#: The five measured workloads (the fifth in two shapes), and one GPU's share of the third.
WORKLOADS = {
    "nt_f16_128": Workload("nt_f16_128", "nt", F16, 128, 128, 128, 1000, 1001),
    "nt_f16_1024": Workload("nt_f16_1024", "nt", F16, 1024, 1024, 1024, 2000, 2001),
    "nt_f16_4096": Workload("nt_f16_4096", "nt", F16, 4096, 4096, 4096, 3000, 3001),
    "nn_bf16_4096": Workload("nn_bf16_4096", "nn", BF16, 4096, 4096, 4096, 4000, 4001),
    "nt_f16_ragged_4000x5000x3000": Workload("nt_f16_ragged_4000x5000x3000", "nt", F16, 4000, 5000, 3000,
                                             5000, 5001),
    "nt_f16_longk_512x512x65536": Workload("nt_f16_longk_512x512x65536", "nt", F16, 512, 512, 65536,
                                           5100, 5101),
    # one GPU's share of the 4096^3 problem split over 8 GPUs along M: the
    # same seeds draw A row by row, so A here is rows 0..511 of that A
    "nt_f16_shard8_512x4096x4096": Workload("nt_f16_shard8_512x4096x4096", "nt", F16, 512, 4096, 4096,
                                            3000, 3001),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def custom(layout: str, dtype: int, M: int, N: int, K: int, seed: int) -> Workload:
    """An ad-hoc workload (tests of edge shapes): seeds seed and seed + 1."""
    return Workload("custom", layout, dtype, M, N, K, seed, seed + 1)


# ---------------------------------------------------------------------------
# Attention (the KV-length loop): Q [B, H, Sq, D], K and V [B, Hkv, Skv, D],
# each drawn as standard normal float32 and rounded to the dtype (so scores
# q.k / sqrt(D) are of order one); seeds seed, seed + 1, seed + 2.

@dataclass(frozen=True)
class AttentionWorkload:
    name: str
    dtype: int
    batch: int
    heads: int
    kv_heads: int
    seq_q: int
    seq_kv: int
    dim: int
    causal: bool
    seed: int

    def make(self):
        """(Q, K, V) as uint16 encodings."""
        q = random_matrix((self.batch * self.heads * self.seq_q, self.dim), self.seed, self.dtype, "normal")
        k = random_matrix((self.batch * self.kv_heads * self.seq_kv, self.dim), self.seed + 1, self.dtype, "normal")
        v = random_matrix((self.batch * self.kv_heads * self.seq_kv, self.dim), self.seed + 2, self.dtype, "normal")
        return (q.reshape(self.batch, self.heads, self.seq_q, self.dim),
                k.reshape(self.batch, self.kv_heads, self.seq_kv, self.dim),
                v.reshape(self.batch, self.kv_heads, self.seq_kv, self.dim))

    @property
    def flops(self) -> int:
        pairs = self.seq_q * (self.seq_q + 1) // 2 if self.causal else self.seq_q * self.seq_kv
        return 4 * self.batch * self.heads * self.dim * pairs


ATTENTION_WORKLOADS = {
    "attn_f16_b4_h32_s4096_d128": AttentionWorkload("attn_f16_b4_h32_s4096_d128", F16, 4, 32, 32, 4096, 4096,
                                                    128, False, 6000),
    "attn_f16_b4_h32_s4096_d128_causal": AttentionWorkload("attn_f16_b4_h32_s4096_d128_causal", F16, 4, 32, 32,
                                                           4096, 4096, 128, True, 6100),
    "attn_bf16_b2_h32_kv8_s2048_d128_causal": AttentionWorkload("attn_bf16_b2_h32_kv8_s2048_d128_causal", BF16,
                                                                2, 32, 8, 2048, 2048, 128, True, 6200),
    "attn_f16_b4_h32_s4096_d64": AttentionWorkload("attn_f16_b4_h32_s4096_d64", F16, 4, 32, 32, 4096, 4096, 64,
                                                   False, 6300),
    "attn_f16_b4_h32_s4096_d64_causal": AttentionWorkload("attn_f16_b4_h32_s4096_d64_causal", F16, 4, 32, 32,
                                                          4096, 4096, 64, True, 6400),
}


def attention_workload(name: str) -> AttentionWorkload:
    return ATTENTION_WORKLOADS[name]


def attention_custom(dtype, batch, heads, kv_heads, seq_q, seq_kv, dim, causal, seed) -> AttentionWorkload:
    return AttentionWorkload("custom", dtype, batch, heads, kv_heads, seq_q, seq_kv, dim, causal, seed)
