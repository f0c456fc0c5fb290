"""GPU parity against the CPU oracle over seeded random worlds.

The hand-picked cases of test_gpu_parity.py fix one axis at a time.  Here
every case draws all of them at once from a fixed seed: the flat size
(log-uniform, or placed just around a block, XCD-run or tile boundary of
the kernels' grids), the world and replica counts, the alignment, both
gradient and parameter formats, a static or dynamic loss scale, the
predivide factor, the AdamW hyper-parameters, clipping, an accumulation
window in either order, the state layout, and sometimes a poisoned step.
Each case runs two or three steps through parity.run, which compares every
element with the oracle at the stated tolerances.  The list is the same on
every run; each case prints its draw before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import parity
import zero_sharded_optimizer_step_amd as Z
from zero_sharded_optimizer_step_amd import workloads as W
from zero_sharded_optimizer_step_amd.world import Hyper

BF16, FP16 = torch.bfloat16, torch.float16

# Element counts at which the kernels' geometry changes: a reduce block
# covers 1024 elements and an apply block 256 (one state tile); XCD runs
# are 256 blocks of either.
BOUNDARIES = [256, 1024, 256 * 256, 256 * 1024]


def _numel_and_shape(rng):
    world = int(rng.integers(1, 9))
    alignment = int(rng.choice([8, 16, 64, 128, 256]))
    if rng.random() < 0.5:
        numel = int(math.exp(rng.uniform(0.0, math.log(4e6))))
    else:
        # a shard of k boundaries plus a small offset, the last rank short
        # of a full shard by a few elements
        unit = int(rng.choice(BOUNDARIES))
        k = int(rng.integers(1, max(2, 4_000_000 // (unit * world))))
        shard = k * unit + int(rng.choice([0, 8, 16, 64])) * int(rng.choice([-1, 1]))
        shard = max(alignment, -(-shard // alignment) * alignment)
        numel = max(1, world * shard - int(rng.integers(0, 3 * alignment)))
    return max(1, numel), world, alignment


def _draw(i, rng):
    numel, world, alignment = _numel_and_shape(rng)
    gdt = BF16 if rng.random() < 0.5 else FP16
    pdt = gdt if rng.random() < 0.8 else (FP16 if gdt == BF16 else BF16)
    n_rep = world if rng.random() < 0.7 else int(rng.integers(1, 13))
    micro = int(rng.choice([1, 1, 1, 2, 3]))
    local = micro > 1 and rng.random() < 0.5
    dynamic = gdt == FP16 and rng.random() < 0.4
    scale = 1.0 if gdt == BF16 else float(2.0 ** int(rng.integers(0, 15)))
    hp = Hyper(lr=float(10 ** rng.uniform(-5, -2)),
               beta1=float(rng.choice([0.0, 0.5, 0.9])),
               beta2=float(rng.choice([0.95, 0.999])),
               eps=float(rng.choice([1e-8, 1e-6])),
               weight_decay=float(rng.choice([0.0, 0.01, 0.1])),
               max_grad_norm=float(rng.choice([0.0, 0.5, 1.0, 100.0])),
               loss_scale=scale,
               grad_predivide=float(rng.choice([1.0, float(n_rep), 0.5])))
    steps = int(rng.integers(2, 4))
    poison = None
    poison_micro = 0
    if rng.random() < 0.25:
        at = int(rng.integers(0, steps))
        poison = [None] * steps
        poison[at] = W.Poison(at, int(rng.integers(0, n_rep)), int(rng.integers(0, numel)),
                              int(rng.integers(0, 3)))
        poison_micro = int(rng.integers(0, micro))
    layout = Z.ZERO_STATE_TILED if rng.random() < 0.25 else Z.ZERO_STATE_SEPARATE
    return parity.Spec(numel=numel, world_size=world, alignment=alignment, grad_dtype=gdt,
                       param_dtype=pdt, grad_sigma=float(rng.choice([1e-3, 1e-2])),
                       n_replicas=n_rep, steps=steps, hp=hp, dynamic_scale=dynamic,
                       scaler_args=(12, 2, 1, 1.0), poison=poison, poison_micro=poison_micro,
                       micro_batches=micro, local_accumulation=local, state_layout=layout,
                       name="random-%d" % i, seed=i)


def _cases(n=48, seed=20240611):
    rng = np.random.default_rng(seed)
    return [_draw(i, rng) for i in range(n)]


CASES = _cases()


def _describe(s):
    return ("P%d N%d R%d A%d %s/%s K%d%s%s %s steps%d lr%.1e b1 %g b2 %g eps %g wd %g "
            "clip %g scale %g%s D %g" % (
                s.numel, s.world_size, s.n_replicas, s.alignment, str(s.grad_dtype)[6:],
                str(s.param_dtype)[6:], s.micro_batches, " local" if s.local_accumulation else "",
                " poison@%d" % next(i for i, p in enumerate(s.poison) if p) if s.poison else "",
                "tiled" if s.state_layout == Z.ZERO_STATE_TILED else "separate", s.steps,
                s.hp.lr, s.hp.beta1, s.hp.beta2, s.hp.eps, s.hp.weight_decay,
                s.hp.max_grad_norm, s.hp.loss_scale, " dynamic" if s.dynamic_scale else "",
                s.hp.grad_predivide))


def test_draws_cover_every_axis():
    """The fixed draw reaches each option it is meant to exercise (CPU)."""
    assert {s.grad_dtype for s in CASES} == {BF16, FP16}
    assert any(s.param_dtype != s.grad_dtype for s in CASES)
    assert any(s.local_accumulation for s in CASES)
    assert any(s.micro_batches > 1 and not s.local_accumulation for s in CASES)
    assert any(s.state_layout == Z.ZERO_STATE_TILED for s in CASES)
    assert any(s.poison for s in CASES)
    assert any(s.dynamic_scale for s in CASES)
    assert any(s.n_replicas != s.world_size for s in CASES)
    assert any(s.world_size == 1 for s in CASES)
    assert any(s.hp.max_grad_norm == 0.0 for s in CASES)
    assert any(s.numel < 1024 for s in CASES) and any(s.numel > 1_000_000 for s in CASES)


@pytest.mark.gpu
@pytest.mark.parametrize("spec", CASES, ids=[s.name for s in CASES])
def test_random_world_matches_oracle(spec):
    print("case %s: %s" % (spec.name, _describe(spec)), flush=True)
    rep = parity.run(spec)
    if spec.poison:
        assert rep.skipped >= 1
    print("  norm rel err %.2e, bitwise state fraction %.6f, cast max ulp %d, skipped %d"
          % (rep.norm_rel_err, rep.state_bitwise, rep.cast_max_ulp, rep.skipped), flush=True)
