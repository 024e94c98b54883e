"""Pins for the oracle GEMM against facts that do not depend on it.

Each test is chosen so that a plausible slip in the oracle fails it:
  * exact integer results (small integers make every fp32 partial sum exact)
    catch a dropped or repeated k term, a wrong sign, a transposed operand;
  * exact rational brute force + Higham's bound on recursive summation catch
    a wrong accumulation precision or order-independent blunders on real data;
  * identity / permutation B, the K=1 outer product and the M=N=1 dot product
    are closed forms;
  * the fp32-accumulation discriminator separates fp32 from fp16 accumulation;
  * the executed multiply-add count must equal M*N*K (flops = 2MNK, the
    TFLOP/s formula of the "Stage 04 - GEMM" notes, "exercises").
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

F16, BF16 = 0, 1


def _enc(values, dtype):
    """Library rounding of exactly-representable or to-be-rounded values."""
    v = np.asarray(values, dtype=np.float32)
    if dtype == F16:
        return v.astype(np.float16).view(np.uint16)
    return torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _small_int_operands(rng, M, N, K, dtype, layout):
    a = rng.integers(-4, 5, size=(M, K))
    b = rng.integers(-4, 5, size=(K, N))  # logical B[k, n]
    A = _enc(a, dtype)
    B = _enc(b.T if layout == "nt" else b, dtype)
    return a, b, A, B


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", ["nt", "nn"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (8, 8, 64), (17, 9, 33), (2, 40, 16)])
def test_small_integers_exact(oracle_gemm, dtype, layout, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    a, b, A, B = _small_int_operands(rng, M, N, K, dtype, layout)
    exact = a @ b  # int64; |entries| <= 16 * K <= 1024, every fp32 partial sum is exact
    fn = oracle_gemm.gemm_nt if layout == "nt" else oracle_gemm.gemm_nn
    C, S = fn(A, B, dtype, return_sums=True)
    assert np.array_equal(S, exact.astype(np.float32))
    assert np.array_equal(C, _enc(exact, dtype))


def _fp16_uniform(rng, shape):
    return rng.uniform(-1, 1, size=shape).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("shape", [(2, 3, 5), (4, 4, 31), (3, 2, 128)])
def test_rational_brute_force_within_higham_bound(oracle_gemm, shape):
    M, N, K = shape
    rng = np.random.default_rng(sum(shape))
    A = _fp16_uniform(rng, (M, K))
    B = _fp16_uniform(rng, (N, K))
    C, S = oracle_gemm.gemm_nt(A, B, F16, return_sums=True)
    a = A.view(np.float16).astype(np.float64)
    b = B.view(np.float16).astype(np.float64)
    u = Fraction(1, 2 ** 24)
    gamma = K * u / (1 - K * u)
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(a[m, k])) * Fraction(float(b[n, k])) for k in range(K)]
            exact = sum(terms, Fraction(0))
            absum = sum((abs(t) for t in terms), Fraction(0))
            err = abs(Fraction(float(S[m, n])) - exact)
            assert err <= gamma * absum, (m, n)
    # the output is the binary32 sum rounded to binary16 (numpy's cast as reference)
    assert np.array_equal(C, S.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("layout", ["nt", "nn"])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_identity_b_returns_a(oracle_gemm, layout, dtype):
    K = 48
    rng = np.random.default_rng(7)
    A = _enc(rng.uniform(-1, 1, size=(13, K)), dtype)
    I = _enc(np.eye(K), dtype)
    fn = oracle_gemm.gemm_nt if layout == "nt" else oracle_gemm.gemm_nn
    assert np.array_equal(fn(A, I, dtype), A)


@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_permutation_b_permutes_columns(oracle_gemm, layout):
    K = 40
    rng = np.random.default_rng(8)
    A = _enc(rng.uniform(-1, 1, size=(9, K)), F16)
    perm = rng.permutation(K)
    P = np.zeros((K, K))          # logical B[k, n] = 1 iff k == perm[n]
    P[perm, np.arange(K)] = 1.0
    B = _enc(P.T if layout == "nt" else P, F16)
    fn = oracle_gemm.gemm_nt if layout == "nt" else oracle_gemm.gemm_nn
    assert np.array_equal(fn(A, B, F16), A[:, perm])


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_k1_outer_product(oracle_gemm, dtype):
    rng = np.random.default_rng(9)
    A = _enc(rng.uniform(-2, 2, size=(11, 1)), dtype)
    B = _enc(rng.uniform(-2, 2, size=(7, 1)), dtype)
    a = oracle_gemm.decode(A, dtype)[:, 0].astype(np.float64)
    b = oracle_gemm.decode(B, dtype)[:, 0].astype(np.float64)
    exact = np.outer(a, b)  # products of two 16-bit values are exact in binary64
    assert np.array_equal(oracle_gemm.gemm_nt(A, B, dtype), _enc(exact, dtype))


def test_m1_n1_dot_product(oracle_gemm):
    rng = np.random.default_rng(10)
    K = 257
    A = _enc(rng.integers(-3, 4, size=(1, K)), F16)
    B = _enc(rng.integers(-3, 4, size=(1, K)), F16)
    dot = int(np.dot(A.view(np.float16).astype(np.int64)[0], B.view(np.float16).astype(np.int64)[0]))
    C, S = oracle_gemm.gemm_nt(A, B, F16, return_sums=True)
    assert S[0, 0] == dot and C[0, 0] == _enc([dot], F16)[0]


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_nt_equals_nn_of_transpose(oracle_gemm, dtype):
    rng = np.random.default_rng(11)
    A = _enc(rng.uniform(-1, 1, size=(21, 70)), dtype)
    B = _enc(rng.uniform(-1, 1, size=(19, 70)), dtype)  # [N, K]
    assert np.array_equal(oracle_gemm.gemm_nt(A, B, dtype),
                          oracle_gemm.gemm_nn(A, np.ascontiguousarray(B.T), dtype))


def test_fp32_accumulation_discriminator(oracle_gemm):
    # 4096 products of 1 * 2^-12 sum to exactly 1.0 in fp32; an fp16 accumulator
    # stalls at 0.5, where adding 2^-12 is a tie that rounds back to 0.5.
    K = 4096
    A = _enc(np.ones((1, K)), F16)
    B = _enc(np.full((1, K), 2.0 ** -12), F16)
    C = oracle_gemm.gemm_nt(A, B, F16)
    assert int(C[0, 0]) == 0x3C00


@pytest.mark.parametrize("shape", [(1, 1, 1), (5, 3, 17), (33, 65, 7), (128, 64, 96)])
def test_multiply_add_count_is_mnk(oracle_gemm, shape):
    M, N, K = shape
    rng = np.random.default_rng(12)
    A = _fp16_uniform(rng, (M, K))
    B = _fp16_uniform(rng, (N, K))
    _, cnt = oracle_gemm.gemm_nt(A, B, F16, return_count=True)
    assert cnt == M * N * K
    if M > 2:
        _, cnt = oracle_gemm.gemm_nt(A, B, F16, rows=(1, M - 1), return_count=True)
        assert cnt == (M - 2) * N * K


def test_row_ranges_and_points_agree_with_whole(oracle_gemm):
    rng = np.random.default_rng(13)
    M, N, K = 37, 29, 83
    A = _fp16_uniform(rng, (M, K))
    B = _fp16_uniform(rng, (K, N))
    whole = oracle_gemm.gemm_nn(A, B, F16)
    assert np.array_equal(oracle_gemm.gemm_nn(A, B, F16, rows=(5, 20)), whole[5:20])
    r = rng.integers(0, M, 50)
    c = rng.integers(0, N, 50)
    assert np.array_equal(oracle_gemm.gemm_points(A, B, "nn", F16, r, c), whole[r, c])


def test_empty_k_gives_zero(oracle_gemm):
    A = np.zeros((3, 0), np.uint16)
    B = np.zeros((4, 0), np.uint16)
    assert np.array_equal(oracle_gemm.gemm_nt(A, B, F16), np.zeros((3, 4), np.uint16))


def test_rejects_mismatched_shapes(oracle_gemm):
    with pytest.raises(ValueError):
        oracle_gemm.gemm_nt(np.zeros((2, 3), np.uint16), np.zeros((2, 4), np.uint16), F16)


# --------------------------------------------------------------------------
# The ReLU epilogue (TileLang tutorial, chapter 11, section 4.6: GEMM+ReLU)

@pytest.mark.parametrize("layout", ["nt", "nn"])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_relu_of_identity_b_is_elementwise_max_with_zero(oracle_gemm, layout, dtype):
    # with B = I every sum is one input value, so the epilogue is numpy's
    # elementwise maximum with zero of A (negative values and zeros become +0)
    K = 48
    rng = np.random.default_rng(17)
    a = rng.uniform(-1, 1, size=(13, K)).astype(np.float32)
    a[0, :5] = [0.0, -0.0, -1.0, 1.0, -2.0 ** -20]
    A = _enc(a, dtype)
    I = _enc(np.eye(K), dtype)
    fn = oracle_gemm.gemm_nt if layout == "nt" else oracle_gemm.gemm_nn
    want = _enc(np.maximum(oracle_gemm.decode(A, dtype), np.float32(0)) + np.float32(0), dtype)
    got = fn(A, I, dtype, relu=True)
    assert np.array_equal(got, want)
    assert not (got == (0x8000 if dtype == F16 else 0x8000)).any(), "a negative zero survived the epilogue"


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_relu_commutes_with_the_final_rounding(oracle_gemm, dtype):
    # rounding to nearest is monotone and maps 0 to 0, so for finite sums
    # relu-then-round equals round-then-relu (with -0 mapped to +0)
    rng = np.random.default_rng(18)
    A = _enc(rng.uniform(-1, 1, size=(37, 70)), dtype)
    B = _enc(rng.uniform(-1, 1, size=(29, 70)), dtype)
    plain, sums = oracle_gemm.gemm_nt(A, B, dtype, return_sums=True)
    fused = oracle_gemm.gemm_nt(A, B, dtype, relu=True)
    assert np.isfinite(sums).all() and (sums < 0).any() and (sums > 0).any()
    want = np.where(oracle_gemm.decode(plain, dtype) > 0, plain, np.uint16(0))
    assert np.array_equal(fused, want)


def test_relu_of_a_nan_sum_is_positive_zero(oracle_gemm):
    A = _enc(np.ones((2, 8)), F16)
    A[1, 3] = 0x7E00  # a quiet NaN in row 1
    B = _enc(np.ones((3, 8)), F16)
    plain = oracle_gemm.gemm_nt(A, B, F16)
    assert (plain[0] == _enc([8.0], F16)[0]).all() and np.isnan(oracle_gemm.decode(plain[1], F16)).all()
    fused = oracle_gemm.gemm_nt(A, B, F16, relu=True)
    assert (fused[0] == plain[0]).all() and (fused[1] == 0).all()


def test_relu_points_agree_with_rows(oracle_gemm):
    rng = np.random.default_rng(19)
    A = _enc(rng.uniform(-1, 1, size=(20, 40)), BF16)
    B = _enc(rng.uniform(-1, 1, size=(40, 24)), BF16)
    whole = oracle_gemm.gemm_nn(A, B, BF16, relu=True)
    rows = rng.integers(0, 20, 30)
    cols = rng.integers(0, 24, 30)
    assert np.array_equal(oracle_gemm.gemm_points(A, B, "nn", BF16, rows, cols, relu=True), whole[rows, cols])
