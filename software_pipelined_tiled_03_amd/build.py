"""Build the HIP library (software_pipelined_tiled_03_amd/_lib/libpipegemm.so) for gfx950.

The library is plain C-ABI (include/pipegemm.h); it is built in-tree with hipcc
so that it travels with the source tree.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libpipegemm.so")
KERNEL_SRC = os.path.join(CSRC, "pipegemm_kernels.hip")
ATTN_SRC = os.path.join(CSRC, "attn_kernels.hip")
HOST_SRC = os.path.join(CSRC, "pipegemm.hip")
DEPS = [KERNEL_SRC, ATTN_SRC, HOST_SRC] + [os.path.join(CSRC, f) for f in (
    "pipegemm_kernel.hpp", "pipegemm_launch.hpp", "pipegemm_layout.hpp", "attn_kernel.hpp", "attn_launch.hpp",
    "attn_map.hpp", "launch_util.hpp")] + [
    os.path.join(ROOT, "include", f) for f in ("pipegemm.h", "pipeattn.h")]
# one kernel translation unit per (element type, B layout, K bound), compiled in parallel
VARIANTS = [("%s_%s_k%d" % (n, l, kc), e, nn, kc)
            for n, e in (("f16", "_Float16"), ("bf16", "__bf16")) for l, nn in (("nt", 0), ("nn", 1)) for kc in (0, 1)]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]

# Attention units only: MFMA accumulators in VGPRs.  By default the compiler
# gives the accumulators of the one-wave-per-SIMD attention tiles AGPRs and
# then copies them (and other loop values) between the two register files
# every key tile, 1000-3400 v_accvgpr moves per kernel; with the VGPR form
# those tiles need none (the two-block D = 128 tile, which needs more than 256
# registers, keeps a few hundred) and run 4-23 % faster, bit-identical.  The
# 8-wave tiles already use VGPRs only and compile to the same code.  The GEMM
# units keep the default: their 4-wave tiles hold 256 accumulators per lane.
ATTN_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _compile_cmds(objdir, extra):
    cmds = []
    for name, elem, nn, kcheck in VARIANTS:
        obj = os.path.join(objdir, "kernels_%s.o" % name)
        cmds.append((obj, [HIPCC, *FLAGS, *extra, "-DPG_ELEM=" + elem, "-DPG_NN=%d" % nn,
                           "-DPG_KCHECK=%d" % kcheck, "-c", KERNEL_SRC, "-o", obj]))
    for name, elem in (("f16", "_Float16"), ("bf16", "__bf16")):
        obj = os.path.join(objdir, "attn_%s.o" % name)
        cmds.append((obj, [HIPCC, *FLAGS, *ATTN_FLAGS, *extra, "-DPG_ELEM=" + elem, "-c", ATTN_SRC, "-o", obj]))
    obj = os.path.join(objdir, "host.o")
    cmds.append((obj, [HIPCC, *FLAGS, *extra, "-c", HOST_SRC, "-o", obj]))
    return cmds


def build(verbose: bool = False, extra=()) -> str:
    """Compile the library (always) and return its path."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(LIBDIR, exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="pipegemm_build_") as objdir:
        cmds = _compile_cmds(objdir, list(extra))
        workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))

        def run(c):
            if verbose:
                print(" ".join(c[1]), flush=True)
            return subprocess.run(c[1], capture_output=True, text=True)

        with ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(run, cmds))
        for (obj, cmd), r in zip(cmds, results):
            err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
            if r.returncode != 0:
                raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), err))
            if verbose and err.strip():
                print(err, file=sys.stderr)
        tmp = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in cmds], "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


if __name__ == "__main__":
    build(verbose=True)
