"""The boundary from C: tests/c_consumer.c is compiled as C99 against
include/pipegemm.h and include/pipeattn.h (warnings as errors), linked with
the library and run on the CPU (its calls are the pure-host entry points)."""
import os
import shutil
import subprocess

import pytest

from software_pipelined_tiled_03_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_headers_compile_as_c_and_host_entry_points_answer(tmp_path):
    libdir = os.path.dirname(binding.LIB_PATH)
    assert os.path.exists(binding.LIB_PATH), "library not built"
    exe = tmp_path / "c_consumer"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I" + os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_consumer.c"), "-L" + libdir, "-lpipegemm",
                    "-Wl,-rpath," + libdir, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c consumer: OK" in r.stdout
