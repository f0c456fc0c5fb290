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
