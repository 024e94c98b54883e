"""On-chip memory budget of a multi-buffered GEMM tile, and the pruned
configuration space it implies.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: TileLang tutorial, chapter 11 "pipeline and autotuning":
  * section 2.3 -- multi-buffering turns each copied tile buffer of shape
    (block_M, block_K) into num_stages copies, so the footprint grows linearly
    with depth;
  * section 4.4 -- only buffers written inside the pipelined loop are
    versioned; read-only inputs are not copied;
  * section 4.5 -- bytes per A tile = block_M * block_K * sizeof(dtype), per B
    tile = block_K * block_N * sizeof(dtype), pipeline footprint =
    num_stages * (A + B); exceeding the budget is a hard compile/launch failure;
    the worked examples (128x128x32 and 256x256x64 in fp16 against a 228 KiB
    budget) are the values this module must reproduce;
  * section 3.7 / 5.1 -- the tuning grid (64,128,256)^2 x (16,32,64) x
    (1,2,3,4) x (128,256) threads for a 4096^3 problem, pruned first of tiles
    that do not divide the problem and then of over-budget combinations,
    keeps 214 of 216 candidates.

The accumulator fragment lives in registers and is not counted (section 4.5).
"""
from dataclasses import dataclass
from itertools import product
from typing import Iterable, List, Tuple

#: The 228 KiB per-block shared-memory budget the pages use (an H100 figure).
H100_BUDGET = 228 * 1024
#: Largest LDS allocation per workgroup on gfx950 (MI355X): 160 KiB.
MI355X_BUDGET = 160 * 1024


def stage_bytes(block_M: int, block_N: int, block_K: int, elem_bytes: int = 2) -> int:
    """Bytes of one A tile plus one B tile."""
    return (block_M * block_K + block_K * block_N) * elem_bytes


def lds_bytes(block_M: int, block_N: int, block_K: int, num_stages: int, elem_bytes: int = 2) -> int:
    """Upper-bound pipeline footprint: num_stages copies of (A tile + B tile)."""
    return num_stages * stage_bytes(block_M, block_N, block_K, elem_bytes)


def fits(block_M, block_N, block_K, num_stages, budget, elem_bytes=2) -> bool:
    return lds_bytes(block_M, block_N, block_K, num_stages, elem_bytes) <= budget


def max_stages(block_M: int, block_N: int, block_K: int, budget: int, elem_bytes: int = 2) -> int:
    """Largest stage count whose footprint is within the budget."""
    return budget // stage_bytes(block_M, block_N, block_K, elem_bytes)


@dataclass
class FootprintRow:
    num_stages: int
    bytes: int
    kib: float
    fits: bool
    percent: float  # of the budget


def footprint_table(block_M, block_N, block_K, stages: Iterable[int], budget, elem_bytes=2) -> List[FootprintRow]:
    rows = []
    for s in stages:
        b = lds_bytes(block_M, block_N, block_K, s, elem_bytes)
        rows.append(FootprintRow(s, b, b / 1024.0, b <= budget, 100.0 * b / budget))
    return rows


def grid_configs(M: int, N: int, K: int, budget: int, block_Ms=(64, 128, 256), block_Ns=(64, 128, 256),
                 block_Ks=(16, 32, 64), stages=(1, 2, 3, 4), threads=(128, 256), elem_bytes=2):
    """Enumerate the tuning grid and split it into (legal, rejected).

    A candidate is dropped first if its tile does not divide the problem, then
    if its pipeline footprint exceeds the budget.
    """
    requested, legal, rejected = [], [], []
    for bm, bn, bk, s, th in product(block_Ms, block_Ns, block_Ks, stages, threads):
        cfg = dict(block_M=bm, block_N=bn, block_K=bk, num_stages=s, threads=th)
        requested.append(cfg)
        if M % bm or N % bn or K % bk:
            continue
        if fits(bm, bn, bk, s, budget, elem_bytes):
            legal.append(cfg)
        else:
            rejected.append(cfg)
    return requested, legal, rejected


def count_grid(M, N, K, budget, **kw) -> Tuple[int, int, int]:
    """(requested, legal, rejected-over-budget) counts of grid_configs()."""
    req, legal, rej = grid_configs(M, N, K, budget, **kw)
    return len(req), len(legal), len(rej)
