"""The library's host-only code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

zero_host.cpp (partition, bucket plan, loss scaler, checkpoint headers,
re-partition plan, argument checks) is compiled with g++ and both
sanitizers, together with tests/c/host_edges.cpp, which drives every
host-only entry point at the edges of its argument ranges (counts near
INT64_MAX, world sizes up to INT32_MAX, alignments up to 2^30) and on
random inputs: random bucket tables, random partitions for the
re-partition plan, hand-built partitions with random shard sizes, 20,000
checkpoint headers of random or bit-flipped bytes, and a long random
loss-scaler run.  Any out-of-bounds access, signed overflow or other
undefined behaviour aborts the run; the driver also checks that every
accepted result is consistent.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_entry_points_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_edges")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "zero_sharded_optimizer_step_amd", "csrc"),
                    os.path.join(ROOT, "zero_sharded_optimizer_step_amd", "csrc", "zero_host.cpp"),
                    os.path.join(ROOT, "tests", "c", "host_edges.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "all checks passed" in r.stdout
