"""A whole data-parallel world held by one process on one GPU.

With one GPU the reduce-scatter's arithmetic becomes a read of N replica
gradient buffers that sit in the same HBM, the all-reduce of the norm and
overflow flag becomes the combine over every simulated rank's partials, and
the all-gather becomes each rank's cast into its slice of one shared full
parameter buffer.  This class only allocates the buffers (torch) and queues
the library's calls in the step's order; it computes nothing itself.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import (GLOBAL_BYTES, ZERO_STATE_SEPARATE, ZERO_STATE_TILED, StepArgs, checkpoint,
               tiled_state_numel, zero_global_t, zero_partials_bytes, zero_accumulate_local,
               zero_partition, zero_partition_valid_numel, zero_repartition,
               zero_repartition_tiled, zero_shard_accumulate, zero_shard_apply,
               zero_shard_combine, zero_shard_reduce, zero_shard_workspace_bytes,
               zero_state_tile, zero_state_untile)


@dataclass
class Hyper:
    lr: float = 6e-5
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 1.0
    loss_scale: float = 1.0
    grad_predivide: float = 1.0


class SimulatedWorld:
    """Buffers of `ranks` (default: every rank) of a world of `world_size`.

    grads[i] holds replica i's flat gradient over the simulated ranks'
    range [lo, hi) of the padded flat space; full_params spans the whole
    padded space; master/exp_avg/exp_avg_sq[k] are rank ranks[k]'s shard,
    or, with state_layout ZERO_STATE_TILED, tiled[k] is its tiled state
    (and master/exp_avg/exp_avg_sq are None).
    """

    def __init__(self, numel: int, world_size: int, n_replicas: Optional[int] = None,
                 alignment: int = 128, grad_dtype=torch.bfloat16, param_dtype=None,
                 device="cuda", ranks: Optional[Sequence[int]] = None,
                 allocate_grads: bool = True, state_layout: int = ZERO_STATE_SEPARATE):
        self.part = zero_partition(numel, world_size, alignment)
        self.numel = numel
        self.world_size = world_size
        self.n_replicas = n_replicas or world_size
        self.s = self.part.shard_numel
        self.padded = self.part.padded_numel
        self.valid = [zero_partition_valid_numel(self.part, r) for r in range(world_size)]
        self.ranks = list(ranks) if ranks is not None else list(range(world_size))
        self.grad_dtype = grad_dtype
        self.param_dtype = param_dtype or grad_dtype
        self.device = torch.device(device)
        self.lo = min(self.ranks) * self.s
        self.hi = (max(self.ranks) + 1) * self.s
        d = self.device
        self.grads = [torch.zeros(self.hi - self.lo, dtype=grad_dtype, device=d)
                      for _ in range(self.n_replicas)] if allocate_grads else []
        self.state_layout = state_layout
        if state_layout == ZERO_STATE_TILED:
            self.tiled = [torch.zeros(tiled_state_numel(self.s), dtype=torch.float32, device=d)
                          for _ in self.ranks]
            self.master = self.exp_avg = self.exp_avg_sq = None
        else:
            self.tiled = None
            self.master = [torch.zeros(self.s, dtype=torch.float32, device=d) for _ in self.ranks]
            self.exp_avg = [torch.zeros(self.s, dtype=torch.float32, device=d) for _ in self.ranks]
            self.exp_avg_sq = [torch.zeros(self.s, dtype=torch.float32, device=d)
                               for _ in self.ranks]
        self.full_params = torch.zeros(self.padded, dtype=self.param_dtype, device=d)
        ws = zero_shard_workspace_bytes(self.s)
        self.workspace = [torch.empty(ws, dtype=torch.uint8, device=d) for _ in self.ranks]
        self.partials = torch.zeros(zero_partials_bytes(len(self.ranks)), dtype=torch.uint8,
                                    device=d)
        self.global_buf = torch.zeros(256, dtype=torch.uint8, device=d)
        assert GLOBAL_BYTES <= 256

    def grad_slice(self, replica: int, rank: int) -> torch.Tensor:
        off = rank * self.s - self.lo
        return self.grads[replica][off:off + self.s]

    def rank_args(self, k: int, hp: Hyper, t: int, accumulate: bool = False) -> StepArgs:
        r = self.ranks[k]
        tiled = self.state_layout == ZERO_STATE_TILED
        return StepArgs(world_size=self.world_size, rank=r, shard_numel=self.s,
                        valid_numel=self.valid[r],
                        replica_grads=[self.grad_slice(i, r) for i in range(self.n_replicas)],
                        master=self.tiled[k] if tiled else self.master[k],
                        exp_avg=None if tiled else self.exp_avg[k],
                        exp_avg_sq=None if tiled else self.exp_avg_sq[k],
                        full_params=self.full_params,
                        workspace=self.workspace[k], lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2,
                        eps=hp.eps, weight_decay=hp.weight_decay, step=t,
                        loss_scale=hp.loss_scale, grad_predivide=hp.grad_predivide,
                        max_grad_norm=hp.max_grad_norm, grad_dtype=self.grad_dtype,
                        param_dtype=self.param_dtype, accumulate=accumulate,
                        state_layout=self.state_layout)

    def separate_state(self, k: int):
        """Rank ranks[k]'s (master, exp_avg, exp_avg_sq) as three fp32
        tensors of shard length: the arrays themselves, or, for a tiled
        state, new tensors the library untiles it into."""
        if self.state_layout != ZERO_STATE_TILED:
            return (self.master[k], self.exp_avg[k], self.exp_avg_sq[k])
        out = tuple(torch.empty(self.s, dtype=torch.float32, device=self.device)
                    for _ in range(3))
        zero_state_untile(self.tiled[k], *out, first=0, n=self.s)
        return out

    def set_state(self, k: int, master, exp_avg=None, exp_avg_sq=None) -> None:
        """Set rank ranks[k]'s state from fp32 tensors of shard length (the
        moments default to zero), through the library for a tiled state."""
        z = lambda: torch.zeros(self.s, dtype=torch.float32, device=self.device)
        m = exp_avg if exp_avg is not None else z()
        v = exp_avg_sq if exp_avg_sq is not None else z()
        if self.state_layout == ZERO_STATE_TILED:
            zero_state_tile(master, m, v, self.tiled[k], first=0, n=self.s)
        else:
            self.master[k].copy_(master)
            self.exp_avg[k].copy_(m)
            self.exp_avg_sq[k].copy_(v)

    def accumulate(self, hp: Hyper, first: bool, stream=None) -> None:
        """Queue pass 1 only for every simulated rank: a micro-batch before
        the last of an accumulation window (`first` sets the slices, later
        ones add to them)."""
        for k in range(len(self.ranks)):
            zero_shard_accumulate(self.rank_args(k, hp, 1, accumulate=not first), stream)

    def accumulate_local(self, micro_grads, first: bool, stream=None) -> None:
        """Accumulation before the reduce (grads must be fp32): replica i's
        micro-batch gradient micro_grads[i] (16-bit, same range as grads[i])
        is widened into grads[i], which `first` sets and later calls add to.
        The window's step then reduces the fp32 sums."""
        if self.grad_dtype != torch.float32:
            raise ValueError("accumulate_local needs a world with float32 replica buffers")
        for i, g in enumerate(micro_grads):
            zero_accumulate_local(g, self.grads[i], first, stream=stream)

    def step(self, hp: Hyper, t: int, stream=None, accumulate: bool = False) -> None:
        """Queue one optimizer step of every simulated rank (no host wait).
        With accumulate, pass 1 adds this micro-batch to the slices the
        earlier micro-batches of the window left in the workspaces."""
        args = [self.rank_args(k, hp, t, accumulate) for k in range(len(self.ranks))]
        for k, a in enumerate(args):
            zero_shard_reduce(a, k, self.partials, stream)
        zero_shard_combine(self.partials, len(self.ranks), hp.max_grad_norm, self.global_buf,
                           stream)
        for a in args:
            zero_shard_apply(a, self.global_buf, stream)

    def result(self) -> zero_global_t:
        """The last combine's result (waits for the device)."""
        raw = self.global_buf[:GLOBAL_BYTES].cpu().numpy().tobytes()
        return zero_global_t.from_buffer_copy(raw)

    def reduced_grad(self, k: int) -> torch.Tensor:
        """Rank ranks[k]'s fp32 reduced gradient from its last reduce."""
        return self.workspace[k][:self.s * 4].view(torch.float32)

    # ------------------------------------------------- checkpoint and resume
    def _all_ranks(self):
        if self.ranks != list(range(self.world_size)):
            raise ValueError("needs every rank of the world")

    def state(self, k: int):
        """Rank ranks[k]'s state as stored: three arrays, or one tiled one."""
        if self.state_layout == ZERO_STATE_TILED:
            return (self.tiled[k],)
        return (self.master[k], self.exp_avg[k], self.exp_avg_sq[k])

    def save_checkpoint(self, directory: str, step: int, scaler=None) -> None:
        """One shard file per rank: `step` optimizer steps applied so far."""
        self._all_ranks()
        torch.cuda.synchronize(self.device)
        checkpoint.save_world(directory, self.part, [self.state(k) for k in range(self.world_size)],
                              self.param_dtype, step, scaler)

    def load_checkpoint(self, directory: str):
        """Resume every simulated rank from a run saved under any world size;
        returns (step, scaler) of the saved run."""
        out = None
        for k, r in enumerate(self.ranks):
            out = checkpoint.load_rank_resharded(directory, self.part, r, self.state(k))
        return out

    def repartition_from(self, other: "SimulatedWorld", stream=None) -> None:
        """Take over the optimizer state of a resident world of the same
        numel but another partition (and the same state layout), on the
        device."""
        self._all_ranks()
        other._all_ranks()
        if self.state_layout != other.state_layout:
            raise ValueError("both worlds must keep their state in the same layout")
        if self.state_layout == ZERO_STATE_TILED:
            zero_repartition_tiled(other.part, other.tiled, self.part, self.tiled, stream)
            return
        for field in range(3):
            zero_repartition(other.part, [other.state(k)[field] for k in range(other.world_size)],
                             self.part, [self.state(k)[field] for k in range(self.world_size)],
                             stream)
