"""Assembly checks of the built kernels (the gfx950 analogue of the pages'
look at the generated code, chapter 11 sections 2.1 and 4.3, and the
"expected output" of the num_stages IR-diff and T.Pipelined examples: the
pipelined loop keeps one wait and one barrier per round, the non-pipelined one
two barriers, and the wait count grows with the number of stages).

Compiles kernel translation units of this repository to gfx950 assembly on the
CPU (hipcc cross-compiles; no device) and inspects every K loop of an
instantiation: the dispatch on num_stages gives one loop per built ring.
Checked instantiations:
  - Tile<128,128,32,2,2> (32x32x16 MFMA, 4 waves), every ring it builds;
  - the headline Tile<256,256,64,2,4> (16x16x32 MFMA, 8 waves): S = 1, 2 and
    2 + a_lead with early B copies and paired wave-priority changes.
And for the NN form, whose transposed LDS reads are inline assembly the
compiler does not track: on every control-flow path, no instruction touches a
transposed read's destination registers before the next s_waitcnt
lgkmcnt(0)."""
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
# the headline Tile<256,256,64,2,4> (16x16x32 MFMA): 8 waves, 4 + 4 copies per wave per K tile
HEADLINE = "_ZN8pipegemm11gemm_kernelIDF16_Lb0ENS_4TileILi256ELi256ELi64ELi2ELi4ELi16EEELb0EEEvNS_10KernelArgsE"
HLA = HLB = 4


def _compile(tmp_path_factory, elem, nn):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / ("k_%s_%d.s" % (elem.strip("_"), nn))
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-DPG_ELEM=" + elem,
                    "-DPG_NN=%d" % nn, "-DPG_KCHECK=0", "--cuda-device-only", "-S",
                    os.path.join(CSRC, "pipegemm_kernels.hip"), "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


@pytest.fixture(scope="module")
def nt_f16_asm(tmp_path_factory):
    return _compile(tmp_path_factory, "_Float16", 0)


@pytest.fixture(scope="module")
def nn_bf16_asm(tmp_path_factory):
    return _compile(tmp_path_factory, "__bf16", 1)


def k_loops(text, kernel, mfma):
    """Every loop (back edge to a 'Loop Header' label) of one kernel, with its
    counts and its instructions in order."""
    start = text.index(kernel + ":")
    end = text.index(".Lfunc_end", start)
    body = text[start:end].splitlines()
    labels = {m.group(1): k for k, l in enumerate(body) for m in [re.match(r"^(\.LBB\d+_\d+):", l)] if m}
    found = []
    for k, l in enumerate(body):
        m = re.search(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < k and "Loop Header" in body[labels[m.group(1)]]:
            seg = body[labels[m.group(1)]:k + 1]
            ins = [x.strip() for x in seg if x.strip() and not x.strip().startswith(";") and not x.strip().endswith(":")]
            found.append(dict(
                barriers=sum(1 for x in ins if re.match(r"s_barrier\b", x)),
                vmcnt=[int(x) for y in ins for x in re.findall(r"s_waitcnt vmcnt\((\d+)\)", y)],
                mfma=sum(1 for x in ins if mfma in x),
                lds_loads=sum(1 for x in ins if re.search(r"buffer_load_dwordx4\b.*\blds\b", x)),
                lds_reads=sum(1 for x in ins if "ds_read_b128" in x),
                valu=sum(1 for x in ins if re.match(r"v_(?!mfma|accvgpr)", x)),
                ins=ins, text="\n".join(seg)))
    return found


@pytest.fixture(scope="module")
def loops(nt_f16_asm):
    return k_loops(nt_f16_asm, KERNEL, "v_mfma_f32_32x32x16_f16")


@pytest.fixture(scope="module")
def headline_loops(nt_f16_asm):
    return k_loops(nt_f16_asm, HEADLINE, "v_mfma_f32_16x16x32_f16")


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


# --- the headline instantiation ---------------------------------------------

def test_headline_rings(headline_loops):
    # 256 x 256 x 64 stages are 64 KiB: S = 1 (64 KiB), S = 2 (128 KiB) and
    # S = 2 + a_lead (160 KiB) fit the 160 KiB LDS, nothing deeper
    assert len(headline_loops) == 3
    by_wait = sorted((l["barriers"], tuple(l["vmcnt"])) for l in headline_loops)
    # S = 1: two barriers and a full wait; S = 2: one barrier, wait for
    # everything (ring_wait_steady(2, 0) = 0); S = 2 + a_lead: one barrier,
    # the leading A tile's 4 copies stay in flight (ring_wait_steady(2, 1, 4, 4))
    assert by_wait == [(1, (0,)), (1, (HLA,)), (2, (0,))]


def test_headline_rounds_copy_read_and_multiply(headline_loops):
    for l in headline_loops:
        # each of the 8 waves owns 128 x 64 = 8 x 4 blocks of 16 x 16, 2 k-steps of 32 per K tile
        assert l["mfma"] == 8 * 4 * 2
        assert l["lds_loads"] == HLA + HLB                 # one K tile's copies per round
        assert l["lds_reads"] == (8 + 4) * 2               # A and B fragments of both k-steps


def test_headline_early_b_and_priority(headline_loops):
    lead = [l for l in headline_loops if l["vmcnt"] == [HLA]]
    assert len(lead) == 1
    ins = lead[0]["ins"]
    bar = next(i for i, x in enumerate(ins) if x.startswith("s_barrier"))
    wait = next(i for i, x in enumerate(ins) if x.startswith("s_waitcnt") and "vmcnt" in x)
    copies = [i for i, x in enumerate(ins) if re.search(r"buffer_load_dwordx4\b.*\blds\b", x)]
    # A copies of tile j+2 before the wait, B copies of tile j+2 after the barrier (early B)
    assert sum(1 for i in copies if i < wait) == HLA
    assert sum(1 for i in copies if i > bar) == HLB
    # wave priority: raised and dropped in pairs, and low while waiting
    prio = [(i, int(x.split()[1])) for i, x in enumerate(ins) if x.startswith("s_setprio")]
    assert [p for _, p in prio].count(1) == [p for _, p in prio].count(0) >= 1
    before_wait = [p for i, p in prio if i < wait]
    assert before_wait and before_wait[-1] == 0, "the wave waits for its copies at priority 0"
    after_bar = [p for i, p in prio if i > bar]
    assert after_bar and after_bar[0] == 1, "priority is raised again after the barrier"
    # 8-wave tiles keep their accumulators in VGPRs: no accumulator copies in the loop
    assert not any(x.startswith("v_accvgpr") for x in ins)


# --- NN form: untracked transposed reads --------------------------------------

def _regs(tok):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", tok):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def tr_read_hazards(text):
    """(reads, hazards): for each ds_read_b64_tr_b16, follow every control-flow
    path (fall-through and branch targets) until an s_waitcnt with
    lgkmcnt(0); a hazard is any instruction on the way that reads or writes
    one of the read's destination VGPRs.  Paths the dispatch on num_stages
    makes impossible are followed too, so the check is conservative."""
    lines = text.splitlines()
    labels = {m.group(1): i for i, l in enumerate(lines) for m in [re.match(r"^(\.LBB\d+_\d+):", l)] if m}
    reads = hazards = 0
    for i, l in enumerate(lines):
        t = l.strip()
        if not t.startswith("ds_read_b64_tr_b16"):
            continue
        reads += 1
        dst = _regs(t.split(None, 1)[1].split(",")[0])
        stack, seen, hit = [i + 1], set(), False
        while stack and not hit:
            j = stack.pop()
            while j < len(lines) and j not in seen:
                seen.add(j)
                u = lines[j].strip()
                j += 1
                if not u or u.startswith((";", ".")) or u.endswith(":"):
                    continue
                if u.startswith("s_waitcnt") and "lgkmcnt(0)" in u:
                    break
                if u.startswith("s_endpgm"):
                    break
                op = u.split(None, 1)
                if op[0] == "s_branch":
                    stack.append(labels[op[1].strip()])
                    break
                if op[0].startswith("s_cbranch"):
                    stack.append(labels[op[1].strip()])
                    continue
                if len(op) > 1 and _regs(op[1]) & dst:
                    hit = True
                    break
        hazards += hit
    return reads, hazards


def test_nn_transposed_reads_are_waited_for(nn_bf16_asm):
    reads, hazards = tr_read_hazards(nn_bf16_asm)
    assert reads > 1000  # every NN tile and ring issues them
    assert hazards == 0


# --- the register table the knee analysis uses ---------------------------------

def _reg_counts(text):
    out = {}
    for m in re.finditer(r"\.agpr_count:\s+\d+.*?\.name:\s+(\S+).*?\.vgpr_count:\s+(\d+)", text, re.S):
        t = re.search(r"TileILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi\d+", m.group(1))
        bm, bn, bk, wm, wn = (int(x) for x in t.groups())
        out[(bm, bn, bk, 64 * wm * wn)] = int(m.group(2))
    return out


def test_knee_register_table_matches_the_builds(nt_f16_asm, nn_bf16_asm):
    from oracle import knee

    nt, nn = _reg_counts(nt_f16_asm), _reg_counts(nn_bf16_asm)
    assert set(nt) == set(nn) == set(knee.REG_COUNT)
    for key, v in knee.REG_COUNT.items():
        assert v == max(nt[key], nn[key]), key
        # the occupancy the table implies is the same for every build of the tile
        for regs in (nt[key], nn[key]):
            assert 512 // (-(-regs // 8) * 8) == knee.reg_waves_per_simd(*key), key


@pytest.fixture(scope="module")
def attn_f16_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "attn_f16.s"
    from software_pipelined_tiled_03_amd import build

    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", *build.ATTN_FLAGS, "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                    "-DPG_ELEM=_Float16",
                    "--cuda-device-only", "-S", os.path.join(CSRC, "attn_kernels.hip"), "-o", str(out)], check=True,
                   capture_output=True)
    return out.read_text()


def _scratch_in_loops(text):
    """(kernel, line) of every scratch (spill) access inside a loop: the
    compiler marks each basic block of a loop with 'Loop Header' or 'in
    Loop' on its label line."""
    found = []
    kernel, in_loop = None, False
    for line in text.splitlines():
        if re.match(r"^_ZN8pipegemm\w+:", line):
            kernel, in_loop = line.split(":")[0], False
        elif re.match(r"^(\.LBB\w+:|; %bb\.\d+:)", line):
            in_loop = "Loop Header" in line or "in Loop" in line
        elif in_loop and "scratch_" in line and kernel:
            found.append((kernel, line.strip()))
    return found


def test_no_spill_traffic_inside_any_loop(nt_f16_asm, nn_bf16_asm, attn_f16_asm):
    # register spills, where the compiler needs them at all (the 4-wave
    # 256x256 tiles hold 512 registers), stay outside the K and KV loops
    for text in (nt_f16_asm, nn_bf16_asm, attn_f16_asm):
        assert text.count("Loop Header") > 0
        bad = _scratch_in_loops(text)
        assert not bad, bad[:3]


def test_attention_and_headline_kernels_do_not_spill(nt_f16_asm, attn_f16_asm):
    for m in re.finditer(r"\.name:\s+(\S+)\s.*?\.vgpr_spill_count:\s+(\d+)", attn_f16_asm, re.S):
        assert int(m.group(2)) == 0, m.group(1)
    for m in re.finditer(r"\.name:\s+(\S+)\s.*?\.vgpr_spill_count:\s+(\d+)", nt_f16_asm, re.S):
        if m.group(1) == HEADLINE:
            assert int(m.group(2)) == 0


def test_one_wave_per_simd_attention_tiles_move_no_accumulators(attn_f16_asm):
    # built with the VGPR form of the MFMAs (build.ATTN_FLAGS), the attention
    # tiles keep their accumulators in VGPRs: no v_accvgpr copies between the
    # register files (by default the 4-wave tiles made 1000-3400 per kernel),
    # except the two-block D = 128 tile, whose 300-odd registers exceed 256
    seen = 0
    for m in re.finditer(r"^(_ZN8pipegemm11attn_kernel\w+):[^\n]*\n(.*?)\.Lfunc_end", attn_f16_asm, re.S | re.M):
        name, body = m.group(1), m.group(2)
        tile = re.search(r"AttnTileILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", name).groups()
        moves = body.count("v_accvgpr_read") + body.count("v_accvgpr_write")
        seen += 1
        if tile == ("64", "4", "2", "128"):
            assert moves < 500, (tile, moves)
        else:
            assert moves == 0, (tile, moves)
    assert seen == 12
