"""The attention part of the C-ABI on the CPU: pipeattn.h's functions are
exported, the LDS rule is the pages' (num_stages versioned K and V tiles),
and validation runs in the documented order without a device."""
import ctypes
import os
import re

import pytest

from software_pipelined_tiled_03_amd import binding as pg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MI355X = 160 * 1024
F16, BF16 = pg.GEMM_F16, pg.GEMM_BF16


def declared():
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "pipeattn.h")).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_and_exports():
    assert declared() == ["attn_check", "attn_default_config", "attn_fwd", "attn_lds_bytes"]
    lib = ctypes.CDLL(pg.LIB_PATH)
    for name in declared():
        assert hasattr(lib, name), name


def check(B=4, H=32, Hkv=32, Sq=4096, Skv=4096, D=128, dtype=F16, causal=0, bm=128, bn=64, s=2, th=256,
          budget=MI355X):
    return pg.attn_check(B, H, Hkv, Sq, Skv, D, dtype, causal, bm, bn, s, th, budget)


def test_lds_rule_is_stages_times_k_and_v_tiles():
    for bn, d, s in [(64, 128, 1), (64, 128, 2), (128, 128, 2), (128, 64, 3)]:
        assert pg.attn_lds_bytes(bn, d, s) == s * 2 * bn * d * 2
    assert pg.attn_lds_bytes(64, 128, 0) == pg.attn_lds_bytes(64, 128, 1)
    assert pg.attn_lds_bytes(-1, 128, 1) == -1


def test_budget_checked_before_everything_but_arguments():
    assert check(bn=128, s=3) == pg.GEMM_ERR_LDS_BUDGET        # 192 KiB
    assert "LDS budget" in pg.last_error()
    assert check(bn=128, s=3, D=120) == pg.GEMM_ERR_LDS_BUDGET  # also misaligned and unbuilt
    assert check(bn=64, s=6) == pg.GEMM_ERR_LDS_BUDGET          # 192 KiB
    assert check(bn=64, s=5) == pg.GEMM_ERR_UNSUPPORTED         # exactly 160 KiB: fits, not built
    assert check(bn=64, s=4) == pg.GEMM_OK                      # 128 KiB
    assert check(bn=128, s=2) == pg.GEMM_OK                     # 128 KiB


def test_argument_errors():
    assert check(Hkv=5) == pg.GEMM_ERR_ARG
    assert check(causal=1, Skv=2048) == pg.GEMM_ERR_ARG
    assert check(Sq=0) == pg.GEMM_ERR_ARG
    assert check(dtype=7) == pg.GEMM_ERR_ARG
    assert check(th=100) == pg.GEMM_ERR_ARG
    assert check(s=-1) == pg.GEMM_ERR_ARG


def test_alignment_and_unsupported():
    assert check(D=60) == pg.GEMM_ERR_ALIGN
    assert check(D=64) == pg.GEMM_OK                            # head dimensions 64 and 128 are built
    assert check(D=64, bm=256, th=256) == pg.GEMM_OK            # two blocks per wave at 64 too
    assert check(D=96) == pg.GEMM_ERR_UNSUPPORTED
    assert check(D=256, bn=64, s=1) == pg.GEMM_ERR_UNSUPPORTED  # fits the budget, not built
    assert check(bm=128, th=512) == pg.GEMM_ERR_UNSUPPORTED     # threads must be 2 x block_M
    assert check(bm=256, th=256, bn=128) == pg.GEMM_ERR_UNSUPPORTED   # not built (two blocks per wave, 128 keys)
    assert check(bm=256, th=512, bn=128) == pg.GEMM_OK
    assert check(bm=256, th=512, bn=64) == pg.GEMM_OK
    assert check(bm=256, th=0, bn=64) == pg.GEMM_OK             # default threads = 2 x block_M
    assert check(bn=32) == pg.GEMM_ERR_UNSUPPORTED
    assert check(s=5, bn=64, budget=1 << 20) == pg.GEMM_ERR_UNSUPPORTED   # fits a bigger budget, not built


def test_grouped_and_causal_configurations_are_valid():
    assert check(B=2, H=32, Hkv=8, Sq=2048, Skv=2048, dtype=BF16, causal=1) == pg.GEMM_OK
    assert check(Sq=1, Skv=1) == pg.GEMM_OK
    assert check(Sq=300, Skv=777) == pg.GEMM_OK


def test_sizes_past_the_limits_are_rejected_without_overflow():
    # products of these sizes overflow 64 bits: the limits are checked by division
    big = 1 << 61
    assert check(Sq=big, Skv=big, causal=1) == pg.GEMM_ERR_UNSUPPORTED
    assert "2 GiB" in pg.last_error()
    assert check(B=1 << 40, H=1 << 40, Hkv=1) == pg.GEMM_ERR_UNSUPPORTED
    assert "workgroups" in pg.last_error()
    # just inside and just past one head's 2 GiB of Q at dim 128 (256-byte rows)
    assert check(Sq=(1 << 23) - 1, Skv=64) == pg.GEMM_OK
    assert check(Sq=1 << 23, Skv=64) == pg.GEMM_ERR_UNSUPPORTED
    # workgroups: B H ceil(Sq / block_M) must stay below 2^31
    assert check(B=1 << 16, H=1 << 15, Hkv=1 << 15, Sq=128, Skv=64, bm=128) == pg.GEMM_ERR_UNSUPPORTED
    assert check(B=1 << 15, H=(1 << 16) - 1, Hkv=(1 << 16) - 1, Sq=128, Skv=64, bm=128) == pg.GEMM_OK


def test_default_configuration_table():
    D128, D64 = 128, 64
    # the measured winners at 4096 keys over 4 x 32 heads
    assert pg.attn_default_config(4, 32, 4096, D128, False) == (256, 128, 2, 512)
    assert pg.attn_default_config(4, 32, 4096, D128, True) == (256, 128, 2, 512)
    assert pg.attn_default_config(4, 32, 4096, D64, False) == (512, 128, 2, 512)
    assert pg.attn_default_config(4, 32, 4096, D64, True) == (128, 64, 2, 256)
    # a grid of fewer 8-wave workgroups than compute units takes the 4-wave tile
    assert pg.attn_default_config(1, 16, 2048, D128, False) == (128, 64, 2, 256)   # 128 workgroups
    assert pg.attn_default_config(1, 16, 4096, D128, False) == (256, 128, 2, 512)  # 256
    assert pg.attn_default_config(2, 32, 2048, D64, False) == (512, 128, 2, 512)   # 256
    assert pg.attn_default_config(1, 32, 2048, D64, False) == (128, 64, 2, 256)    # 128
    # no overflow with huge sizes: plenty of workgroups
    assert pg.attn_default_config(1 << 40, 1 << 40, 1 << 40, D128, False) == (256, 128, 2, 512)
    # errors
    with pytest.raises(pg.GemmArgumentError):
        pg.attn_default_config(0, 1, 1, D128, False)
    with pytest.raises(pg.UnsupportedConfigError):
        pg.attn_default_config(1, 1, 1, 96, False)


@pytest.mark.parametrize("B,H,Hkv,S,D,causal", [(4, 32, 32, 4096, 128, 0), (4, 32, 32, 4096, 64, 1),
                                                 (1, 16, 16, 2048, 128, 1), (2, 32, 8, 300, 64, 0),
                                                 (1, 1, 1, 1, 128, 1), (1, 4, 2, 8388600, 128, 0)])
def test_default_configuration_passes_validation(B, H, Hkv, S, D, causal):
    bm, bn, s, th = pg.attn_default_config(B, H, S, D, causal)
    for dtype in (F16, BF16):
        assert check(B=B, H=H, Hkv=Hkv, Sq=S, Skv=S, D=D, dtype=dtype, causal=causal, bm=bm, bn=bn, s=s,
                     th=th) == pg.GEMM_OK, (bm, bn, s, th, pg.last_error())


def test_scale_must_be_zero_or_positive_and_finite():
    # rejected as an argument error before any device is touched: the
    # pointers below are aligned placeholders that are never dereferenced
    fake = [0x100000, 0x200000, 0x300000, 0x400000]
    for scale in (-1.0, -1e-30, float("nan"), float("inf"), float("-inf")):
        st = pg.attn_fwd_raw(*fake, 1, 1, 1, 128, 128, 128, F16, 0, scale, 128, 64, 2, 256, None)
        assert st == pg.GEMM_ERR_ARG, scale
        assert "scale" in pg.last_error()
