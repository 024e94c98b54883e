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


#: The five measured workloads (the fifth in two shapes).
WORKLOADS = {
    "nt_f16_128": Workload("nt_f16_128", "nt", F16, 128, 128, 128, 1000, 1001),
    "nt_f16_1024": Workload("nt_f16_1024", "nt", F16, 1024, 1024, 1024, 2000, 2001),
    "nt_f16_4096": Workload("nt_f16_4096", "nt", F16, 4096, 4096, 4096, 3000, 3001),
    "nn_bf16_4096": Workload("nn_bf16_4096", "nn", BF16, 4096, 4096, 4096, 4000, 4001),
    "nt_f16_ragged_4000x5000x3000": Workload("nt_f16_ragged_4000x5000x3000", "nt", F16, 4000, 5000, 3000,
                                             5000, 5001),
    "nt_f16_longk_512x512x65536": Workload("nt_f16_longk_512x512x65536", "nt", F16, 512, 512, 65536,
                                           5100, 5101),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def custom(layout: str, dtype: int, M: int, N: int, K: int, seed: int) -> Workload:
    """An ad-hoc workload (tests of edge shapes): seeds seed and seed + 1."""
    return Workload("custom", layout, dtype, M, N, K, seed, seed + 1)
