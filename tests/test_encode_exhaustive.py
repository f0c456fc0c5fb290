"""All 2^32 fp32 bit patterns through three fp32 -> fp16 / bf16 encoders
that share no code: a reference written from the IEEE-754 definition with
integer arithmetic (tests/c/encode_exhaustive.c), the oracle's encoders,
and the library's host cast (zero_host_adamw with lr = 0, where the update
leaves every master unchanged).  CPU only; about a minute on 8 cores."""
import os
import subprocess

import oracle
from zero_sharded_optimizer_step_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_fp32_pattern_encodes_alike(tmp_path):
    exe = str(tmp_path / "encode_exhaustive")
    odir = os.path.dirname(oracle.build(force=False))
    zdir = os.path.dirname(_abi.LIB_PATH)
    subprocess.run(["gcc", "-std=gnu99", "-O2", "-Wall", "-Werror", "-pthread",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "c", "encode_exhaustive.c"), "-o", exe,
                    "-L" + odir, "-loracle", "-L" + zdir, "-lzero_mi355x",
                    "-Wl,-rpath," + odir, "-Wl,-rpath," + zdir], check=True)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    r = subprocess.run([exe, str(threads)], capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all 4294967296 patterns agree" in r.stdout
