"""GPU tests of the sharded checkpoint and elastic resume, through the C ABI.

zero_repartition is compared bit for bit with the oracle's re-partition.  A
resumed run must reproduce the uninterrupted one: a world of 4 ranks runs
6 fp16 steps with a dynamic loss scale; after step 3 it is saved to shard
files and also re-partitioned on the device.  A world of 3 ranks resumed
from the files and a world of 6 ranks resumed from the device copy then run
steps 4-6 on the same gradients.  With clipping off every update is
elementwise, so all three end bit-identical; with clipping on, the norm's
summation order follows the partition, so they agree within the stated
tolerance, and each matches the oracle's unsharded run.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import zero_sharded_optimizer_step_amd as Z
from zero_sharded_optimizer_step_amd import workloads as W
from zero_sharded_optimizer_step_amd.world import Hyper, SimulatedWorld

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("old,new", [((1000, 4, 8), (3, 8)), ((100_003, 8, 128), (3, 128)),
                                     ((5, 4, 8), (2, 1)), ((1_048_579, 2, 128), (7, 1)),
                                     ((300_001, 3, 128), (3, 128))])
def test_device_repartition_matches_oracle(old, new):
    P, N, A = old
    M, B = new
    say("repartition %s -> %s" % (old, new))
    src = SimulatedWorld(P, N, n_replicas=1, alignment=A, grad_dtype=torch.bfloat16)
    dst = SimulatedWorld(P, M, n_replicas=1, alignment=B, grad_dtype=torch.bfloat16)
    for k in range(N):
        for f, t in enumerate(src.state(k)):
            W.flat_normal(t, k * src.s, P, 1.0, ("repart", f))
    for k in range(M):
        for t in dst.state(k):
            t.fill_(7.0)                                   # padding must come back zero
    dst.repartition_from(src)
    for f in range(3):
        ref = oracle.repartition([parity.f32(src.state(k)[f]) for k in range(N)], P, N, A, M, B)
        for k in range(M):
            parity.assert_bitwise("field %d rank %d" % (f, k), parity.f32(dst.state(k)[f]), ref[k])


def _advance(world, steps, hp, scaler, t, poison_step=None, log=None):
    """Run `steps` (global step indices) on `world`; gradients depend only on
    the step and replica.  Returns the next t."""
    for step in steps:
        hp.loss_scale = scaler.scale
        for i in range(world.n_replicas):
            W.flat_normal(world.grads[i], world.lo, world.numel, 1e-3, ("ckpt", step, i),
                          scale=scaler.scale)
        if step == poison_step:
            W.plant(world.grads[1], W.Poison(step, 1, world.numel // 3, 0))
        world.step(hp, t)
        res = world.result()
        if not Z.zero_loss_scaler_update(scaler, bool(res.overflow)):
            t += 1
        if log:
            log("  step %d: overflow %d norm %.6g scale %g" % (step, res.overflow, res.norm,
                                                              scaler.scale))
    return t


def _flat_state(world):
    return [np.concatenate([parity.f32(world.state(k)[f][:world.valid[k]])
                            for k in range(world.world_size)]) for f in range(3)]


def _real_params(world):
    full = parity.u16(world.full_params)
    return np.concatenate([full[r * world.s:r * world.s + world.valid[r]]
                           for r in range(world.world_size)])


def _copy_scaler(sc):
    return Z.zero_loss_scaler_t.from_buffer_copy(bytes(sc))


@pytest.mark.parametrize("clip", [0.0, 1.0])
def test_resume_reproduces_the_uninterrupted_run(tmp_path, clip):
    P, R = 200_003, 4
    say("resume, clip %g" % clip)
    hp = Hyper(max_grad_norm=clip)
    a = SimulatedWorld(P, 4, n_replicas=R, alignment=128, grad_dtype=torch.float16)
    for k in range(4):
        W.flat_normal(a.master[k], k * a.s, P, 0.02, ("ckpt-master",))
    sc = Z.zero_loss_scaler_init(14, 2, 2, 1.0)
    t = _advance(a, range(3), hp, sc, 1, poison_step=1, log=say)
    a.save_checkpoint(str(tmp_path), t - 1, sc)
    c = SimulatedWorld(P, 6, n_replicas=R, alignment=8, grad_dtype=torch.float16)
    c.repartition_from(a)
    t_c, sc_c = t, _copy_scaler(sc)
    t_a = _advance(a, range(3, 6), hp, sc, t, log=say)

    b = SimulatedWorld(P, 3, n_replicas=R, alignment=128, grad_dtype=torch.float16)
    step, sc_b = b.load_checkpoint(str(tmp_path))
    assert step == t - 1 and bytes(sc_b) == bytes(sc_c)
    t_b = _advance(b, range(3, 6), hp, sc_b, step + 1)
    t_c = _advance(c, range(3, 6), hp, sc_c, t_c)
    assert t_a == t_b == t_c and sc.scale == sc_b.scale == sc_c.scale

    # the oracle's unsharded run of the same six steps
    ref = SimulatedWorld(P, 1, n_replicas=R, alignment=1, grad_dtype=torch.float16)
    W.flat_normal(ref.master[0], 0, P, 0.02, ("ckpt-master",))
    o_p = parity.f32(ref.master[0])
    o_m, o_v = np.zeros(P, np.float32), np.zeros(P, np.float32)
    o_full = np.zeros(P, np.uint16)
    o_sc = oracle.LossScaler(14, 2, 2, 1.0)
    o_t = 1
    for step in range(6):
        for i in range(R):
            W.flat_normal(ref.grads[i], 0, P, 1e-3, ("ckpt", step, i), scale=o_sc.scale)
        if step == 1:
            W.plant(ref.grads[1], W.Poison(step, 1, P // 3, 0))
        reps = [parity.u16(g) for g in ref.grads]
        info = oracle.step(reps, oracle.FP16, P, 1, 1, [o_p], [o_m], [o_v], o_full,
                           oracle.Hyper(max_grad_norm=clip, loss_scale=o_sc.scale), o_t)
        if not o_sc.update(info.overflow):
            o_t += 1
    assert o_t == t_a and o_sc.scale == sc.scale

    states = [_flat_state(w) for w in (a, b, c)]
    params = [_real_params(w) for w in (a, b, c)]
    for name, f in (("master", 0), ("exp_avg", 1), ("exp_avg_sq", 2)):
        for w, st in zip("abc", states):
            parity.assert_rel("%s world %s vs oracle" % (name, w), st[f],
                              (o_p, o_m, o_v)[f], parity.RTOL_STATE)
        if clip == 0.0:
            parity.assert_bitwise("%s resumed from files" % name, states[1][f], states[0][f])
            parity.assert_bitwise("%s resumed on device" % name, states[2][f], states[0][f])
    for w, p in zip("abc", params):
        parity.assert_cast("params world %s vs oracle" % w, p, o_full)
    if clip == 0.0:
        parity.assert_bitwise("params resumed", params[1], params[0])
        parity.assert_bitwise("params resumed on device", params[2], params[0])
