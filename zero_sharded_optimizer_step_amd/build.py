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

import hashlib
import os
import shutil
import struct
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


def _elf_sections(d: bytes) -> dict:
    """Section name -> bytes of a little-endian ELF64 image."""
    if d[:4] != b"\x7fELF" or d[4] != 2 or d[5] != 1:
        raise ValueError("not a little-endian ELF64 image")
    shoff, = struct.unpack_from("<Q", d, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", d, 0x3A)
    table = []
    for i in range(shnum):
        name, _typ, _flags, _addr, off, size = struct.unpack_from("<IIQQQQ", d, shoff + i * shentsize)
        table.append((name, off, size))
    strtab = table[shstrndx][1]
    out = {}
    for name, off, size in table:
        end = d.index(b"\0", strtab + name)
        out[d[strtab + name:end].decode()] = d[off:off + size]
    return out


def code_hash(path: str = LIB_PATH) -> str:
    """First 16 hex digits of a SHA-256 over the code a built library runs:
    the host .text and .rodata (entry points, checks and the launch
    geometry they compute) and, from the clang offload bundle in
    .hip_fatbin, the gfx950 code object's .text, .rodata (kernel
    descriptors) and .note (kernel metadata).  These are byte-identical
    across builds of the same sources, whereas the symbol tables carry a
    per-build unique name; edits to comments leave the hash unchanged."""
    secs = _elf_sections(open(path, "rb").read())
    h = hashlib.sha256()
    for name in (".text", ".rodata"):
        h.update(secs[name])
    fb = secs[".hip_fatbin"]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    if not fb.startswith(magic):
        raise ValueError("%s: .hip_fatbin is not an offload bundle" % path)
    count, = struct.unpack_from("<Q", fb, len(magic))
    pos = len(magic) + 8
    found = False
    for _ in range(count):
        off, size, id_len = struct.unpack_from("<QQQ", fb, pos)
        pos += 24
        ident = fb[pos:pos + id_len].decode()
        pos += id_len
        if ident.endswith("-" + ARCH):
            dev = _elf_sections(fb[off:off + size])
            for name in (".text", ".rodata", ".note"):
                h.update(dev[name])
            found = True
    if not found:
        raise ValueError("%s holds no %s code object" % (path, ARCH))
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
