"""The device entry points from plain C: tests/c/abi_gpu_check (built by
__graft_entry__.build() with gcc against include/zero.h and the HIP runtime)
allocates with hipMalloc, runs every rank's reduce, the combine and every
rank's apply for two steps on one stream (or, for a world of one rank,
zero_shard_step_noalloc with no workspace at all), and writes the results to
a file.
No Python or torch takes part in those calls.  The results are compared
with the oracle's world step on the same inputs."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import parity

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "abi_gpu_check")
GLOBAL = np.dtype([("sumsq", "<f8"), ("norm", "<f8"), ("coef", "<f4"), ("overflow", "<i4"),
                   ("clipped", "<i4"), ("reserved", "<i4")])


@pytest.mark.parametrize("P,N,A,R,dtype,scale,clip,mode", [
    (100_003, 4, 128, 4, oracle.BF16, 1.0, 1.0, None),
    (30_011, 3, 8, 5, oracle.FP16, 2.0**12, 1.0, None),
    (5, 4, 8, 2, oracle.BF16, 1.0, 0.0, None),      # three empty ranks, clipping off
    # one rank's whole step through zero_shard_step_noalloc, no workspace
    (50_021, 1, 128, 3, oracle.FP16, 2.0**10, 1.0, "noalloc"),
    (5, 1, 8, 2, oracle.BF16, 1.0, 0.0, "noalloc"),
])
def test_plain_c_world_step_matches_oracle(tmp_path, P, N, A, R, dtype, scale, clip, mode):
    if not os.path.exists(EXE):
        pytest.fail("tests/c/abi_gpu_check is not built: run __graft_entry__.build()")
    print("plain C caller: P=%d N=%d R=%d dtype=%d %s" % (P, N, R, dtype, mode or ""),
          flush=True)
    s, padded, valid = oracle.partition(P, N, A)
    rng = np.random.default_rng(P)
    enc = oracle.f32_to_f16 if dtype == oracle.FP16 else oracle.f32_to_bf16
    reps = []
    for _ in range(R):
        f = np.zeros(padded, np.uint16)
        f[:P] = enc((rng.standard_normal(P) * 1e-2 * scale).astype(np.float32))
        reps.append(f)
    masters = np.zeros(padded, np.float32)
    masters[:P] = (rng.standard_normal(P) * 0.02).astype(np.float32)
    steps = 2
    src, dst = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(src, "wb") as f:
        np.array([P, N, A, R, dtype, steps], np.int64).tofile(f)
        np.array([scale, clip], np.float64).tofile(f)
        for x in reps:
            x.tofile(f)
        masters.tofile(f)
    r = subprocess.run([EXE, src, dst] + ([mode] if mode else []), capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = np.fromfile(dst, np.uint8)
    per_step = GLOBAL.itemsize + 3 * 4 * padded + 2 * padded
    assert raw.size == steps * per_step

    ps = [masters[k * s:(k + 1) * s].copy() for k in range(N)]
    ms = [np.zeros(s, np.float32) for _ in range(N)]
    vs = [np.zeros(s, np.float32) for _ in range(N)]
    full = np.zeros(padded, np.uint16)
    hp = oracle.Hyper(max_grad_norm=clip, loss_scale=scale)
    real = np.zeros(padded, bool)
    for k in range(N):
        real[k * s:k * s + valid[k]] = True
    for t in range(1, steps + 1):
        info = oracle.step(reps, dtype, P, N, A, ps, ms, vs, full, hp, t)
        o = (t - 1) * per_step
        g = raw[o:o + GLOBAL.itemsize].view(GLOBAL)[0]
        o += GLOBAL.itemsize
        got = [raw[o + f * 4 * padded:o + (f + 1) * 4 * padded].view(np.float32)
               for f in range(3)]
        got_full = raw[o + 12 * padded:o + 14 * padded].view(np.uint16)
        assert bool(g["overflow"]) == info.overflow and bool(g["clipped"]) == info.clipped
        assert abs(g["norm"] - info.norm) <= parity.RTOL_NORM * max(info.norm, 1e-300)
        for f, ref in enumerate((ps, ms, vs)):
            for k in range(N):
                n = valid[k]
                mine = got[f][k * s:(k + 1) * s]
                parity.assert_rel("step %d field %d rank %d" % (t, f, k), mine[:n], ref[k][:n],
                                  parity.RTOL_STATE)
                parity.assert_bitwise("step %d field %d rank %d padding" % (t, f, k), mine[n:],
                                      ref[k][n:])
        parity.assert_cast("step %d cast" % t, got_full[real], full[real])
        parity.assert_bitwise("step %d outside the real elements" % t, got_full[~real],
                              full[~real])
