"""The allocation-free step (zero_shard_step_noalloc) against zero_shard_step
with a caller-owned workspace, on identical inputs, through the C ABI.

Two calls in a row share the library's scratch array: the encoder layer's
rank 2 (8,390,656 elements, bf16, 8 replicas), then a smaller fp16 shard
with padding (rank 3 of 100,003 parameters over 4 ranks, loss scale 2^12,
predivide 4).  Each result must equal the existing entry point's bit for
bit: the combine's result, master, both moments and the full buffer, whose
elements outside the rank's slice must keep their canary.
"""
import pytest
import torch

import parity
import zero_sharded_optimizer_step_amd as Z
from zero_sharded_optimizer_step_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


class Rank:
    """One rank's inputs, with two copies of the state and full buffer."""

    def __init__(self, numel, world, rank, nrep, dtype, sigma, scale, key):
        self.part = Z.zero_partition(numel, world, 128)
        self.rank, self.world, self.dtype = rank, world, dtype
        s = self.s = self.part.shard_numel
        self.n = Z.zero_partition_valid_numel(self.part, rank)
        dev = "cuda"
        self.grads = []
        for i in range(nrep):
            g = torch.empty(s, dtype=dtype, device=dev)
            W.flat_normal(g, rank * s, numel, sigma, key + ("grad", i), scale=scale)
            self.grads.append(g)
        master = torch.empty(s, dtype=torch.float32, device=dev)
        W.flat_normal(master, rank * s, numel, 0.02, key + ("master",))
        m = torch.empty(s, dtype=torch.float32, device=dev)
        W.flat_normal(m, rank * s, numel, 1e-4, key + ("m",))
        v = torch.empty(s, dtype=torch.float32, device=dev)
        W.flat_normal(v, rank * s, numel, 1e-4, key + ("v",))
        v.mul_(v)
        full = torch.full((self.part.padded_numel,), parity.CANARY, dtype=torch.int16, device=dev)
        self.state = [[t.clone() for t in (master, m, v, full)] for _ in range(2)]

    def args(self, which, workspace, **hp):
        p, m, v, full = self.state[which]
        return Z.StepArgs(world_size=self.world, rank=self.rank, shard_numel=self.s,
                          valid_numel=self.n, replica_grads=self.grads, master=p, exp_avg=m,
                          exp_avg_sq=v, full_params=full.view(self.dtype), workspace=workspace,
                          step=3, grad_dtype=self.dtype, param_dtype=self.dtype, **hp)

    def compare(self, what, ia, ib):
        for f in ("sumsq", "norm", "coef", "overflow", "clipped"):
            assert getattr(ia, f) == getattr(ib, f), (what, f, getattr(ia, f), getattr(ib, f))
        names = ("master", "exp_avg", "exp_avg_sq", "full params")
        for name, a, b in zip(names, self.state[0], self.state[1]):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), \
                "%s: %s differs" % (what, name)
        full = self.state[1][3]
        lo, hi = self.rank * self.s, self.rank * self.s + self.n
        assert bool((full[:lo] == parity.CANARY).all()) and \
            bool((full[hi:] == parity.CANARY).all()), "%s: wrote outside the slice" % what


def test_noalloc_step_equals_step_with_workspace_twice_in_a_row():
    cases = [
        ("encoder layer rank 2 of 8, bf16, 8 replicas",
         dict(numel=W.ENCODER_4096.numel, world=8, rank=2, nrep=8, dtype=torch.bfloat16,
              sigma=1e-2, scale=1.0, key=("noalloc", 0)), dict()),
        ("rank 3 of 100,003 over 4 (padding), fp16, scale 2^12, predivide 4",
         dict(numel=100_003, world=4, rank=3, nrep=4, dtype=torch.float16, sigma=1e-3,
              scale=2.0**12, key=("noalloc", 1)),
         dict(loss_scale=2.0**12, grad_predivide=4.0, max_grad_norm=0.5)),
    ]
    for what, kw, hp in cases:
        say("noalloc: %s" % what)
        r = Rank(**kw)
        assert r.s <= Z.ZERO_NOALLOC_MAX_SHARD
        ws = torch.empty(Z.zero_shard_workspace_bytes(r.s), dtype=torch.uint8, device="cuda")
        ia = Z.zero_shard_step(r.args(0, ws, **hp), want_info=True)
        ib = Z.zero_shard_step_noalloc(r.args(1, None, **hp), want_info=True)
        assert ia.overflow == 0
        r.compare(what, ia, ib)
        say("  equal: norm %.6g, coef %.6g, clipped %d" % (ib.norm, ib.coef, ib.clipped))
        del r, ws
        torch.cuda.empty_cache()
