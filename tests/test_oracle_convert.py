"""Pins for the oracle's binary16 / bfloat16 conversions.

The oracle writes both conversions from the IEEE 754 bit layouts; here they are
checked against independent library routines (numpy's float16 casts, torch's
bfloat16 casts) over every encoding and many random binary32 values, and
against hand-derived encodings of boundary cases.
"""
import numpy as np
import pytest
import torch

F16, BF16 = 0, 1


def test_decode_every_f16_encoding_matches_numpy(oracle_gemm):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_gemm.decode(bits, F16)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_decode_every_bf16_encoding_matches_torch(oracle_gemm):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_gemm.decode(bits, BF16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _random_f32(seed, n=400000):
    rng = np.random.default_rng(seed)
    # every binary32 exponent, random significands, both signs
    raw = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    x = raw.view(np.float32)
    return x[np.isfinite(x)]


def _tie_values(mbits, lo_exp, hi_exp):
    """Values exactly halfway between neighbours of a format with mbits bits."""
    out = []
    for e in range(lo_exp, hi_exp):
        for m in (0, 1, 2, 3, 2**mbits - 2, 2**mbits - 1):
            base = (2**mbits + m) * 2.0 ** (e - mbits)
            out.append(base + 2.0 ** (e - mbits - 1))
    v = np.array(out, dtype=np.float64)
    v = v[(v < 3e38)].astype(np.float32)
    return np.concatenate([v, -v])


def test_encode_f16_matches_numpy_on_random_and_ties(oracle_gemm):
    x = np.concatenate([_random_f32(1),
                        np.random.default_rng(2).uniform(-70000, 70000, 100000).astype(np.float32),
                        np.random.default_rng(3).uniform(-1e-4, 1e-4, 100000).astype(np.float32),
                        _tie_values(10, -24, 16)])
    ours = oracle_gemm.encode(x, F16)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_encode_bf16_matches_torch_on_random_and_ties(oracle_gemm):
    x = np.concatenate([_random_f32(4), _tie_values(7, -133, 127),
                        np.random.default_rng(5).standard_normal(100000).astype(np.float32)])
    ours = oracle_gemm.encode(x, BF16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3C00),
    (-2.0, 0xC000),
    (65504.0, 0x7BFF),             # largest finite binary16
    (65519.0, 0x7BFF),             # below the midpoint to 2^16: stays finite
    (65520.0, 0x7C00),             # the midpoint rounds to even = overflow to +inf
    (2.0 ** -24, 0x0001),          # smallest subnormal
    (2.0 ** -25, 0x0000),          # half the smallest subnormal: tie to even (0)
    (3 * 2.0 ** -25, 0x0002),      # 1.5 quanta: tie to even (2)
    (2.0 ** -14, 0x0400),          # smallest normal
    (1.0 + 2.0 ** -11, 0x3C00),    # tie between 1 and 1+2^-10: even is 1
    (1.0 + 3 * 2.0 ** -11, 0x3C02),  # tie between 1+2^-10 and 1+2^-9: even is 1+2^-9
    (float("inf"), 0x7C00),
    (-0.0, 0x8000),
])
def test_encode_f16_boundaries(oracle_gemm, value, bits):
    assert int(oracle_gemm.encode(np.array([value], np.float32), F16)[0]) == bits


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),      # tie: even significand (1.0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),  # tie: rounds up to the even neighbour
    (3.3895313892515355e38, 0x7F7F),  # largest finite bfloat16
    (float("inf"), 0x7F80),
])
def test_encode_bf16_boundaries(oracle_gemm, value, bits):
    assert int(oracle_gemm.encode(np.array([value], np.float32), BF16)[0]) == bits


def test_encode_nan_stays_nan(oracle_gemm):
    for dt in (F16, BF16):
        e = int(oracle_gemm.encode(np.array([np.nan], np.float32), dt)[0])
        assert np.isnan(oracle_gemm.decode(np.array([e], np.uint16), dt)[0])
