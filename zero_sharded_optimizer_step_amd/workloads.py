"""Seeded synthetic inputs for the sharded step, shared by tests and bench.

This module synthesizes data only and holds none of the step's arithmetic.
Every tensor is a pure function of its key (workload, seed, step, replica,
...) and of the 64 Mi-element chunk it falls in, so any chunk can be
regenerated on its own.  Values are drawn as fp32 normals by torch's
generator on the requested device and rounded to the storage type by torch.
The pages measure on no public dataset; these shapes and distributions stand
in for a model's gradients and weights.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

CHUNK = 1 << 26


def seed_of(key: Tuple) -> int:
    h = hashlib.blake2b(repr(tuple(key)).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _chunk_values(c: int, total: int, sigma: float, key: Tuple, device,
                  scale: float) -> torch.Tensor:
    """Chunk c (fp32) of a virtual flat tensor of `total` elements."""
    n = min(CHUNK, total - c * CHUNK)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_of(tuple(key) + (c,)))
    x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    return x.mul_(sigma * scale)


def flat_normal(out: torch.Tensor, flat_lo: int, total: int, sigma: float, key: Tuple,
                scale: float = 1.0) -> torch.Tensor:
    """Write elements [flat_lo, flat_lo + out.numel()) of a virtual flat
    tensor of `total` elements, N(0, sigma) * scale drawn chunk by chunk, into
    `out` (rounded to out's dtype by torch).  Indices at or past `total`
    (padding) are written as zeros."""
    n = out.numel()
    hi = min(flat_lo + n, total)
    if hi < flat_lo + n:
        out[max(hi - flat_lo, 0):].zero_()
    if hi <= flat_lo:
        return out
    c = flat_lo // CHUNK
    while c * CHUNK < hi:
        vals = _chunk_values(c, total, sigma, key, out.device, scale)
        a = max(flat_lo, c * CHUNK)
        b = min(hi, c * CHUNK + vals.numel())
        out[a - flat_lo:b - flat_lo].copy_(vals[a - c * CHUNK:b - c * CHUNK])
        c += 1
    return out


INF_CODES = {torch.float16: (0x7C00, 0xFC00, 0x7E00), torch.bfloat16: (0x7F80, 0xFF80, 0x7FC0)}


@dataclass(frozen=True)
class Poison:
    step: int
    replica: int
    index: int
    kind: int            # 0: +inf, 1: -inf, 2: nan


def poison_schedule(steps: int, n_replicas: int, numel: int, p: float = 0.05,
                    seed: int = 0) -> List[Optional[Poison]]:
    """Per step, None or one non-finite value at a uniform (replica, index)."""
    rng = np.random.default_rng(seed)
    out: List[Optional[Poison]] = []
    for t in range(steps):
        if rng.random() < p:
            kind = int(rng.integers(3))
            rep = int(rng.integers(n_replicas))
            idx = int(rng.integers(numel))
            out.append(Poison(t, rep, idx, kind))
        else:
            out.append(None)
    return out


def plant(flat: torch.Tensor, poison: Poison) -> None:
    """Write the poison's non-finite code into a replica's flat buffer."""
    code = INF_CODES[flat.dtype][poison.kind]
    flat.view(torch.int16)[poison.index] = code - 65536 if code >= 32768 else code


def ragged_sizes(n: int = 2000, lo: float = 1e3, hi: float = 1e7, seed: int = 0) -> List[int]:
    """Tensor sizes floor(exp(U(ln lo, ln hi)))."""
    rng = np.random.default_rng(seed)
    return [int(math.floor(math.exp(u))) for u in rng.uniform(math.log(lo), math.log(hi), n)]


@dataclass(frozen=True)
class Workload:
    name: str
    numel: int
    world_size: int
    grad_dtype: torch.dtype
    grad_sigma: float
    alignment: int = 128
    loss_scale: float = 1.0            # fp16: 2^initial_scale_power
    master_sigma: float = 0.02
    steps: int = 1
    tensor_sizes: Tuple[int, ...] = field(default=())
    ranks: Optional[Tuple[int, ...]] = None   # None: every rank is simulated
    lr: float = 6e-5
    weight_decay: float = 0.01
    max_grad_norm: float = 1.0


TINY = Workload(
    name="tiny: tensors 512x512, 512, 512x1024, 1024 (787,968 params), 4 ranks, fp16 grads x 2^16",
    numel=787_968, world_size=4, grad_dtype=torch.float16, grad_sigma=1e-3,
    loss_scale=2.0**16, tensor_sizes=(512 * 512, 512, 512 * 1024, 1024))

ENCODER_4096 = Workload(
    name="encoder layer d_model=4096, q/k/v/out projections + biases (67,125,248 params), "
         "8 ranks, bf16, 10 steps",
    numel=67_125_248, world_size=8, grad_dtype=torch.bfloat16, grad_sigma=1e-2, steps=10,
    tensor_sizes=(4096 * 4096, 4096) * 4)

SHARD_13B_OF_8 = Workload(
    name="13B params over 8 ranks: rank 0's 1,625,000,064-element shard, 8 bf16 replicas",
    numel=13_000_000_000, world_size=8, grad_dtype=torch.bfloat16, grad_sigma=1e-3,
    ranks=(0,))

SCALER_50M = Workload(
    name="fp16 dynamic loss scaling, 50,000,000 params, 4 ranks, 200 steps, 5% poisoned steps",
    numel=50_000_000, world_size=4, grad_dtype=torch.float16, grad_sigma=1e-3,
    loss_scale=2.0**16, steps=200, master_sigma=0.02)

RAGGED_2000 = Workload(
    name="2000 ragged tensors (sizes log-uniform 1e3..1e7), buckets of 2e8, 8 ranks, bf16",
    numel=sum(ragged_sizes()), world_size=8, grad_dtype=torch.bfloat16, grad_sigma=1e-3,
    tensor_sizes=tuple(ragged_sizes()))

ALL = (TINY, ENCODER_4096, SHARD_13B_OF_8, SCALER_50M, RAGGED_2000)


def grad_key(w: Workload, seed: int, step: int, replica: int) -> Tuple:
    return ("grad", w.name, seed, step, replica)


def master_key(w: Workload, seed: int) -> Tuple:
    return ("master", w.name, seed)
