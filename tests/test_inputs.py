"""The seeded input generators shared by the tests, smoke() and bench.py: the
recipe (seeds, distributions, layouts) and the one-GPU-share workload."""
import numpy as np

from software_pipelined_tiled_03_amd import inputs


def test_generators_are_deterministic_and_shaped():
    for name, w in inputs.WORKLOADS.items():
        if w.M * w.K > 4096 * 4096:
            continue
        A, B = w.make()
        assert A.shape == (w.M, w.K) and A.dtype == np.uint16, name
        assert B.shape == w.b_shape() and B.dtype == np.uint16, name
        A2, _ = w.make()
        assert np.array_equal(A, A2), name


def test_distributions_follow_the_recipe():
    # fp16 workloads draw uniform[-1, 1]; the bf16 one draws normal(0, 1)
    a = inputs.random_matrix((256, 256), 7, inputs.F16).view(np.float16).astype(np.float64)
    assert a.min() >= -1.0 and a.max() <= 1.0 and abs(a.mean()) < 0.02 and abs(a.std() - 1 / np.sqrt(3)) < 0.01
    b = inputs.random_matrix((256, 256), 7, inputs.BF16).astype(np.uint32) << 16
    b = b.view(np.float32).astype(np.float64)
    assert abs(b.mean()) < 0.02 and abs(b.std() - 1.0) < 0.02 and np.abs(b).max() > 3.0


def test_shard_is_the_first_rows_of_the_4096_problem():
    # one GPU's share of 4096^3 split over 8 GPUs along M is rows 0..511 of
    # the same A with the whole of the same B
    full = inputs.workload("nt_f16_4096")
    shard = inputs.workload("nt_f16_shard8_512x4096x4096")
    assert (shard.M * 8, shard.N, shard.K) == (full.M, full.N, full.K)
    As, Bs = shard.make()
    Af, Bf = full.make()
    assert np.array_equal(As, Af[:512]) and np.array_equal(Bs, Bf)
