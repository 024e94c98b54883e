"""The C-ABI boundary on the CPU: the library loads, exports every function the
header declares, and validates requests (argument, LDS budget, alignment and
configuration checks, in that order) without a device."""
import ctypes
import os
import re

import pytest

from oracle import budget as obudget
from software_pipelined_tiled_03_amd import binding as pg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pipegemm.h")
MI355X = 160 * 1024
NT, NN, F16, BF16 = pg.GEMM_NT, pg.GEMM_NN, pg.GEMM_F16, pg.GEMM_BF16


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["gemm_nt", "gemm_nn", "gemm_nt_relu", "gemm_nn_relu", "gemm_lds_bytes", "gemm_lds_budget", "gemm_check",
         "gemm_last_error", "gemm_configs", "gemm_prune", "gemm_rank", "gemm_tune", "gemm_default_config",
         "gemm_stamped"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def check(layout=NT, M=4096, N=4096, K=4096, dtype=F16, bm=128, bn=128, bk=32, s=3, th=256, budget=MI355X):
    return pg.gemm_check(layout, M, N, K, dtype, bm, bn, bk, s, th, budget)


def test_lds_bytes_matches_the_oracle_formula():
    for bm, bn, bk in [(128, 128, 32), (256, 256, 64), (128, 256, 64), (64, 128, 16)]:
        for s in range(0, 8):
            assert pg.gemm_lds_bytes(bm, bn, bk, s) == obudget.lds_bytes(bm, bn, bk, max(s, 1))
    assert pg.gemm_lds_bytes(-1, 128, 32, 1) == -1
    assert pg.gemm_lds_bytes(128, 128, 32, 1, 7) == -1


def test_over_budget_is_rejected_before_anything_else():
    # 256x256x64 at 4 stages needs 256 KiB; at 3 stages 192 KiB: both over 160 KiB
    for s in (3, 4):
        assert check(layout=NN, dtype=BF16, bm=256, bn=256, bk=64, s=s) == pg.GEMM_ERR_LDS_BUDGET
        assert "LDS budget" in pg.last_error()
    # still a budget error when the shape is also misaligned or the tile unbuilt
    assert check(K=4090, bm=256, bn=256, bk=64, s=4) == pg.GEMM_ERR_LDS_BUDGET
    assert check(bm=512, bn=512, bk=64, s=2) == pg.GEMM_ERR_LDS_BUDGET   # unbuilt tile, 256 KiB
    assert check(bm=512, bn=512, bk=64, s=1) == pg.GEMM_ERR_UNSUPPORTED  # fits (128 KiB), not built


def test_budget_boundary_is_inclusive():
    # 128x128x32 is 16 KiB per stage: 10 stages fill 160 KiB exactly, 11 exceed it
    assert check(s=10, th=256) == pg.GEMM_OK
    assert check(s=11) == pg.GEMM_ERR_LDS_BUDGET
    assert check(bm=128, bn=256, bk=64, s=3) == pg.GEMM_OK        # 144 KiB
    assert check(bm=128, bn=256, bk=64, s=4) == pg.GEMM_ERR_LDS_BUDGET
    assert check(bm=256, bn=256, bk=64, s=2) == pg.GEMM_OK        # 128 KiB


def test_same_rule_against_the_pages_budget():
    # against 228 KiB, 256x256x64 fits at 3 stages and fails at 4 (as the pages' table)
    h = obudget.H100_BUDGET
    assert check(bm=256, bn=256, bk=64, s=3, budget=h) != pg.GEMM_ERR_LDS_BUDGET
    assert check(bm=256, bn=256, bk=64, s=4, budget=h) == pg.GEMM_ERR_LDS_BUDGET


def test_config_grid_rejections_agree_with_the_oracle():
    _, legal, rejected = obudget.grid_configs(4096, 4096, 4096, MI355X)
    for c in rejected:
        st = check(bm=c["block_M"], bn=c["block_N"], bk=c["block_K"], s=c["num_stages"], th=c["threads"])
        assert st == pg.GEMM_ERR_LDS_BUDGET, c
    for c in legal:
        st = check(bm=c["block_M"], bn=c["block_N"], bk=c["block_K"], s=c["num_stages"], th=c["threads"])
        assert st != pg.GEMM_ERR_LDS_BUDGET, c


def test_argument_errors():
    assert check(M=-1) == pg.GEMM_ERR_ARG
    assert check(dtype=5) == pg.GEMM_ERR_ARG
    assert check(layout=3) == pg.GEMM_ERR_ARG
    assert check(s=-1) == pg.GEMM_ERR_ARG
    assert check(th=96) == pg.GEMM_ERR_ARG
    assert check(bm=0) == pg.GEMM_ERR_ARG
    assert check(budget=-5) == pg.GEMM_ERR_ARG


def test_alignment_errors():
    assert check(K=4092) == pg.GEMM_ERR_ALIGN
    assert check(layout=NN, N=4092) == pg.GEMM_ERR_ALIGN
    assert check(layout=NT, N=4092) == pg.GEMM_OK       # NT only needs K % 8
    assert check(layout=NT, M=4001, N=5001, K=3000) == pg.GEMM_OK


def test_unsupported_configurations():
    assert check(bm=64, bn=64, bk=32) == pg.GEMM_ERR_UNSUPPORTED
    assert check(th=1024) == pg.GEMM_ERR_UNSUPPORTED
    assert "no kernel built" in pg.last_error()
    # 2 waves of 128x128x32 each issue 8 1-KiB copies per tile; with S slots up
    # to S-1 tiles are in flight behind the one waited for: 8 stages keep 56
    # loads in flight, 9 stages would need 64, one more than a wave can count
    assert check(th=128, s=8) == pg.GEMM_OK
    assert check(th=128, s=9) == pg.GEMM_ERR_UNSUPPORTED


def test_leading_a_ring_budget_and_errors():
    # S=2 plus one leading A tile: 256x256x64 fills 160 KiB exactly
    assert pg.gemm_lds_bytes(256, 256, 64, 2, F16, a_lead=1) == 3 * 256 * 64 * 2 + 2 * 256 * 64 * 2 == MI355X
    assert pg.gemm_lds_bytes(128, 256, 64, 2, F16, a_lead=1) == 3 * 128 * 64 * 2 + 2 * 256 * 64 * 2
    assert pg.gemm_lds_bytes(128, 128, 32, 2, F16, a_lead=2) == -1
    assert pg.gemm_check(NT, 4096, 4096, 4096, F16, 256, 256, 64, 2, 256, MI355X, a_lead=1) == pg.GEMM_OK
    assert pg.gemm_check(NT, 4096, 4096, 4096, F16, 256, 256, 64, 2, 512, MI355X, a_lead=1) == pg.GEMM_OK
    # 128x256x64: three stages are 144 KiB, plus a 16 KiB A tile = 160 KiB
    assert pg.gemm_check(NT, 4096, 4096, 4096, F16, 128, 256, 64, 3, 256, MI355X, a_lead=1) == pg.GEMM_OK
    # 256x128x64: three stages are 144 KiB, plus a 32 KiB A tile is over
    assert pg.gemm_check(NT, 4096, 4096, 4096, F16, 256, 128, 64, 3, 256, MI355X, a_lead=1) == \
        pg.GEMM_ERR_LDS_BUDGET
    assert "leading" in pg.last_error()
    assert pg.gemm_check(NT, 64, 64, 64, F16, 128, 128, 32, 1, 256, MI355X, a_lead=1) == pg.GEMM_ERR_ARG
    assert pg.gemm_check(NT, 64, 64, 64, F16, 128, 128, 32, 0, 256, MI355X, a_lead=1) == pg.GEMM_ERR_ARG
    assert pg.gemm_check(NT, 64, 64, 64, F16, 128, 128, 32, 3, 256, MI355X, a_lead=-1) == pg.GEMM_ERR_ARG
    assert pg.gemm_check(NT, 64, 64, 64, F16, 128, 128, 32, 5, 256, MI355X, a_lead=1) == pg.GEMM_ERR_UNSUPPORTED
    # against a larger budget a ring above 160 KiB passes the budget rule but has no kernel
    assert pg.gemm_check(NT, 64, 64, 64, F16, 256, 256, 64, 3, 256, 228 * 1024) == pg.GEMM_ERR_UNSUPPORTED


def test_zero_stages_is_the_single_buffer():
    assert check(s=0) == pg.GEMM_OK
    assert pg.gemm_lds_bytes(128, 128, 32, 0) == pg.gemm_lds_bytes(128, 128, 32, 1)


def test_empty_sizes_are_valid():
    assert check(M=0) == pg.GEMM_OK
    assert check(N=0) == pg.GEMM_OK
    assert check(K=0) == pg.GEMM_OK


def test_default_threads():
    assert check(th=0) == pg.GEMM_OK


def test_ok_clears_the_message():
    check(M=-1)
    assert pg.last_error()
    assert check() == pg.GEMM_OK
    assert pg.last_error() == ""


def test_no_device_reported_as_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert pg.load().gemm_lds_budget() == -1
    assert check(budget=0) == pg.GEMM_ERR_HIP
    # launching entry points: bad arguments are still reported as such
    assert pg.gemm_nt_raw(None, None, None, -1, 4, 8, F16, 128, 128, 32, 2, 0, 256, None) == pg.GEMM_ERR_ARG
    assert pg.gemm_nt_raw(16, 16, 16, 4, 4, 8, F16, 128, 128, 32, 2, 0, 256, None) == pg.GEMM_ERR_HIP
    assert pg.gemm_nt_raw(16, 16, 16, 4, 4, 8, F16, 128, 128, 32, 1, 1, 256, None) == pg.GEMM_ERR_ARG


def test_stamped_entry_point_arguments():
    # a null or misaligned stamp array is an argument error, reported before
    # the budget (validation order), and without touching a device
    st = pg.gemm_stamped_raw(pg.GEMM_NT, 16, 16, 16, 4096, 4096, 4096, F16, 256, 256, 64, 4, 0, 512, None, None)
    assert st == pg.GEMM_ERR_ARG and "stamps" in pg.last_error()
    st = pg.gemm_stamped_raw(pg.GEMM_NT, 16, 16, 16, 4096, 4096, 4096, F16, 256, 256, 64, 2, 1, 512, None, 0x1004)
    assert st == pg.GEMM_ERR_ARG
    # otherwise it validates exactly as gemm_nt (the launch budget comes from
    # the device, so on a host without one a valid call ends in GEMM_ERR_HIP)
    import torch
    if not torch.cuda.is_available():
        st = pg.gemm_stamped_raw(pg.GEMM_NT, 16, 16, 16, 4096, 4096, 4096, F16, 256, 256, 64, 2, 1, 512, None, 0x1000)
        assert st == pg.GEMM_ERR_HIP


def test_size_limits_of_the_32_bit_offsets():
    # a workgroup addresses its A and B panels and its rows of C through buffer
    # resources with 32-bit offsets below 2 GiB
    lim = 1 << 31
    assert check(K=lim // (2 * 128) - 8) == pg.GEMM_OK
    assert check(K=lim // (2 * 128)) == pg.GEMM_ERR_UNSUPPORTED
    assert "operand panel" in pg.last_error()
    assert check(N=lim // (2 * 128) - 8, K=64) == pg.GEMM_OK
    assert check(N=lim // (2 * 128), K=64) == pg.GEMM_ERR_UNSUPPORTED
    assert "panel of C rows" in pg.last_error()
    assert check(N=lim // (2 * 256), K=64, bm=256, bn=256, bk=64, s=2, th=512) == pg.GEMM_ERR_UNSUPPORTED
    assert check(M=lim, K=64) == pg.GEMM_ERR_UNSUPPORTED
