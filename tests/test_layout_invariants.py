"""Host-side invariants of the kernel's LDS layouts and ring schedule.

tests/layout_check.cpp includes the same header the kernel uses
(software_pipelined_tiled_03_amd/csrc/pipegemm_layout.hpp) and enumerates
every copy destination, operand read and ring step; it is compiled with g++
here, no GPU needed."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_layouts_and_schedule(tmp_path):
    exe = tmp_path / "layout_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", os.path.join(ROOT, "software_pipelined_tiled_03_amd",
                                                                            "csrc"),
                    os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK" in r.stdout
