"""Build the HIP library libzero_mi355x.so in place, for gfx950 only.

    python -m zero_sharded_optimizer_step_amd.build

Flags: -O3; no floating-point contraction (the kernels write their fused
multiply-adds explicitly, so every other operation is rounded as written);
no errno from math calls (lets the host update's square roots vectorize;
results are unchanged);
packed fp32 instructions disabled; IEEE division and square root (hipcc's
default) and denormals kept (no flush-to-zero, no fast-math).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libzero_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["zero_host.cpp", "zero_offload.cpp", "zero_kernels.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def compile_flags() -> list[str]:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-fno-math-errno",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def build(out: str = LIB_PATH, verbose: bool = False) -> str:
    """Compile every source into one shared library (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + compile_flags() + ["-shared"] + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that note is harmless and is dropped here.
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("HIP build failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
