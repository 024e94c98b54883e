"""Assembly checks of the built kernels (the gfx950 analogue of the pages'
look at the generated code, chapter 11 sections 2.1 and 4.3: the pipelined
loop keeps one wait and one barrier per round, the non-pipelined one two
barriers, and the wait count grows with the number of stages).

Compiles one kernel translation unit of this repository to gfx950 assembly on
the CPU (hipcc cross-compiles; no device) and inspects every K loop of one
instantiation: the dispatch on num_stages gives one loop per built ring."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "software_pipelined_tiled_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Tile<128,128,32,2,2> (32x32x16 MFMA): 4 waves, 2 + 2 one-KiB copies per wave per K tile
KERNEL = "_ZN8pipegemm11gemm_kernelIDF16_Lb0ENS_4TileILi128ELi128ELi32ELi2ELi2ELi32EEELb0EEEvNS_10KernelArgsE"
LA = LB = 2


@pytest.fixture(scope="module")
def loops(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "k.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-DPG_ELEM=_Float16",
                    "-DPG_NN=0", "-DPG_KCHECK=0", "--cuda-device-only", "-S",
                    os.path.join(CSRC, "pipegemm_kernels.hip"), "-o", str(out)], check=True, capture_output=True)
    text = out.read_text()
    start = text.index(KERNEL + ":")
    end = text.index(".Lfunc_end", start)
    body = text[start:end].splitlines()
    labels = {m.group(1): k for k, l in enumerate(body) for m in [re.match(r"^(\.LBB\d+_\d+):", l)] if m}
    found = []
    for k, l in enumerate(body):
        m = re.search(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < k and "Loop Header" in body[labels[m.group(1)]]:
            seg = body[labels[m.group(1)]:k + 1]
            found.append(dict(
                barriers=sum(1 for x in seg if re.match(r"\s*s_barrier\b", x)),
                vmcnt=[int(x) for y in seg for x in re.findall(r"s_waitcnt vmcnt\((\d+)\)", y)],
                mfma=sum(1 for x in seg if "v_mfma_f32_32x32x16_f16" in x),
                lds_loads=sum(1 for x in seg if re.search(r"buffer_load_dwordx4\b.*\blds\b", x)),
                lds_reads=sum(1 for x in seg if "ds_read_b128" in x),
                valu=sum(1 for x in seg if re.match(r"\s*v_(?!mfma|accvgpr)", x)),
                text="\n".join(seg)))
    return found


def expected_rings():
    """(S, a_lead) -> the steady-state wait count (copies allowed in flight)."""
    rings = {(1, 0): 0, (2, 0): 0}
    for s in range(3, 11):
        rings[(s, 0)] = (s - 2) * (LA + LB)
    for s in range(2, 5):
        rings[(s, 1)] = (s - 2) * (LA + LB) + LA
    return rings


def test_one_loop_per_built_ring(loops):
    assert len(loops) == len(expected_rings())


def test_barriers_per_round(loops):
    # one barrier per steady round when pipelined, two (copy | compute) when S = 1
    assert sorted(l["barriers"] for l in loops) == [1] * (len(loops) - 1) + [2]


def test_waits_grow_with_the_ring_depth(loops):
    single = [l for l in loops if l["barriers"] == 2]
    assert single[0]["vmcnt"] == [0]
    waits = sorted(l["vmcnt"][0] for l in loops if l["barriers"] == 1 and len(l["vmcnt"]) == 1)
    want = sorted(v for (s, lead), v in expected_rings().items() if s >= 2)
    assert waits == want
    assert all(len(l["vmcnt"]) == 1 for l in loops), "exactly one copy wait per round"


def test_every_round_copies_and_multiplies(loops):
    for l in loops:
        # 32x32x16 MFMAs: each of the 4 waves owns 2x2 blocks of 32x32, 2 k-steps of 16 per K tile
        assert l["mfma"] == 4 * 2
        assert l["lds_loads"] == LA + LB              # one tile's copies per round
        assert l["lds_reads"] == 4 * 2                # A and B fragments, 2 k-steps


def test_no_vector_alu_per_copy_in_the_steady_state(loops):
    # copy offsets are loop-invariant (per-tile scalar buffer resources): the
    # pipelined rounds carry only a few vector ALU instructions (LDS read
    # addresses), not the 4-5 per copy of a per-lane bound check
    for l in loops:
        if l["barriers"] == 1:
            assert l["valu"] <= 8, l["text"]
