"""The C ABI from plain C: tests/c/abi_host_check.c is compiled with gcc
against include/zero.h, linked to libzero_mi355x.so and run (host-only
entry points; no GPU needed)."""
import os
import subprocess

from zero_sharded_optimizer_step_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_plain_c_caller(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    libdir = os.path.dirname(_abi.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-o", exe,
                    "-L" + libdir, "-lzero_mi355x", "-Wl,-rpath," + libdir], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_launch_grids_are_xcd_bijections(tmp_path):
    """tests/c/grid_check.cpp, built with g++ against the library's internal
    header: for the workloads' shard sizes and the edges of the grid
    rounding, every launch covers its work, the XCD remap is a bijection
    onto the grid, each XCD gets runs of consecutive logical blocks, and the
    padding stays under one round."""
    exe = str(tmp_path / "grid_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "zero_sharded_optimizer_step_amd", "csrc"),
                    os.path.join(ROOT, "tests", "c", "grid_check.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
