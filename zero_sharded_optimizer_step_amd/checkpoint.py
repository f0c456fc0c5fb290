"""Sharded checkpoint files of the optimizer state, and elastic resume.

"大模型分片训练：ZeRO-3策略在PyTorch中的实现" (practice notes): a sharded run
is saved through the engine, because saving a plain state dict loses the
shard information.  Here every rank writes one file: the 128-byte header
that the library fills and checks (zero_ckpt_header_make,
zero_ckpt_header_check) and then the rank's real elements of master,
exp_avg and exp_avg_sq as little-endian fp32, in that order.  Element e of
the rank's slice is flat parameter rank * shard_numel + e, so a new rank of
a different world reads just the byte ranges it owns from the old files.

This module moves bytes between tensors (device or host) and files through
a pinned staging buffer; it computes nothing.  Resuming the working
low-precision parameters is not needed: they are the cast of the masters,
and the first step after a resume writes them.

A state is either three fp32 tensors (master, exp_avg, exp_avg_sq) or,
for ZERO_STATE_TILED, one tiled device tensor.  The file layout is the
same for both; a tiled state goes through the library's layout conversion
(zero_state_untile on save, zero_state_tile on load) a chunk at a time.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

from . import (dtype_code, tiled_state_numel, zero_ckpt_header_check, zero_ckpt_header_make,
               zero_ckpt_header_t, zero_loss_scaler_t, zero_partition_t,
               zero_partition_valid_numel, zero_repartition_plan, zero_state_tile,
               zero_state_untile)

HEADER_BYTES = ctypes.sizeof(zero_ckpt_header_t)
STAGING_ELEMS = 1 << 26             # 256 MiB of fp32 per transfer
FIELDS = ("master", "exp_avg", "exp_avg_sq")


def rank_path(directory: str, rank: int) -> str:
    return os.path.join(directory, "zero_rank%05d.zsc" % rank)


def _staging(device: torch.device, n: int) -> torch.Tensor:
    pin = device.type == "cuda"
    return torch.empty(min(n, STAGING_ELEMS), dtype=torch.float32, pin_memory=pin)


def _write_fp32(f, t: torch.Tensor, staging: torch.Tensor) -> None:
    n = t.numel()
    for a in range(0, n, staging.numel()):
        b = min(n, a + staging.numel())
        buf = staging[:b - a]
        buf.copy_(t[a:b])
        f.write(memoryview(buf.numpy()).cast("B"))


def _read_fp32(f, t: torch.Tensor, staging: torch.Tensor) -> None:
    n = t.numel()
    for a in range(0, n, staging.numel()):
        b = min(n, a + staging.numel())
        buf = staging[:b - a]
        view = memoryview(buf.numpy()).cast("B")
        if f.readinto(view) != view.nbytes:
            raise IOError("checkpoint file ends early")
        t[a:b].copy_(buf)


def _is_tiled(state: Sequence[torch.Tensor]) -> bool:
    if len(state) == 1:
        if state[0].device.type != "cuda":
            raise ValueError("a tiled state is converted on the device: pass a device tensor")
        return True
    if len(state) != 3:
        raise ValueError("a state is three fp32 tensors or one tiled tensor")
    return False


def _temporaries(device: torch.device, n: int):
    return tuple(torch.empty(n, dtype=torch.float32, device=device) for _ in range(3))


def save_rank(path: str, part: zero_partition_t, rank: int, state: Sequence[torch.Tensor],
              param_dtype, step: int, scaler: Optional[zero_loss_scaler_t] = None
              ) -> zero_ckpt_header_t:
    """Write rank `rank`'s master, exp_avg, exp_avg_sq (three fp32 tensors,
    each at least its valid elements long, or one tiled device tensor) and
    the run's step and scaler state."""
    h = zero_ckpt_header_make(part, rank, dtype_code(param_dtype), step, scaler)
    n = h.valid_numel
    tiled = _is_tiled(state)
    if tiled:
        if state[0].dtype != torch.float32 or state[0].numel() < tiled_state_numel(n):
            raise ValueError("the tiled state holds fewer than valid_numel elements' tiles")
    elif any(t.dtype != torch.float32 or t.numel() < n for t in state):
        raise ValueError("state is three fp32 tensors of at least valid_numel elements")
    tmp = path + ".tmp%d" % os.getpid()
    staging = _staging(state[0].device, max(n, 1))
    with open(tmp, "wb") as f:
        f.write(bytes(h))
        if not tiled:
            for t in state:
                _write_fp32(f, t[:n], staging)
        else:
            # a chunk of elements untiled at a time, each field written at
            # its place in the file
            parts = _temporaries(state[0].device, min(n, STAGING_ELEMS))
            for a in range(0, n, STAGING_ELEMS):
                b = min(n, a + STAGING_ELEMS)
                zero_state_untile(state[0], *[x[:b - a] for x in parts], first=a, n=b - a)
                for field, x in enumerate(parts):
                    f.seek(HEADER_BYTES + 4 * (field * n + a))
                    _write_fp32(f, x[:b - a], staging)
    os.replace(tmp, path)
    return h


def read_header(path: str) -> Tuple[zero_ckpt_header_t, zero_partition_t]:
    with open(path, "rb") as f:
        raw = f.read(HEADER_BYTES)
    if len(raw) != HEADER_BYTES:
        raise IOError("%s: shorter than a checkpoint header" % path)
    h = zero_ckpt_header_t.from_buffer_copy(raw)
    return h, zero_ckpt_header_check(h, os.path.getsize(path))


def _run_info(headers: List[zero_ckpt_header_t]):
    h0 = headers[0]
    for r, h in enumerate(headers):
        if (h.rank != r or h.numel != h0.numel or h.world_size != h0.world_size or
                h.alignment != h0.alignment or h.step != h0.step or
                h.has_scaler != h0.has_scaler or h.param_dtype != h0.param_dtype or
                bytes(h.scaler) != bytes(h0.scaler)):
            raise ValueError("checkpoint shards do not belong to one run (rank %d)" % r)
    return h0.step, (zero_loss_scaler_t.from_buffer_copy(bytes(h0.scaler)) if h0.has_scaler
                     else None)


def save_world(directory: str, part: zero_partition_t, states: Sequence[Sequence[torch.Tensor]],
               param_dtype, step: int, scaler: Optional[zero_loss_scaler_t] = None) -> None:
    """Every rank's file (states[r] = rank r's three state tensors)."""
    os.makedirs(directory, exist_ok=True)
    for r in range(part.world_size):
        save_rank(rank_path(directory, r), part, r, states[r], param_dtype, step, scaler)


def load_rank_resharded(directory: str, new_part: zero_partition_t, new_rank: int,
                        state: Sequence[torch.Tensor]):
    """Fill new rank `new_rank` of partition new_part (same numel, any world
    size and alignment) from a directory of one run's shard files, reading
    only the byte ranges it owns; the padding is zeroed.  Returns the run's
    (step, scaler).  Which old file and which elements each piece comes
    from is the library's read plan (zero_repartition_plan); this function
    only seeks and reads."""
    old_world = read_header(rank_path(directory, 0))[0].world_size
    hp = [read_header(rank_path(directory, r)) for r in range(old_world)]
    headers = [h for h, _ in hp]
    step, scaler = _run_info(headers)
    old = hp[0][1]
    if old.numel != new_part.numel:
        raise ValueError("checkpoint holds %d parameters, the new partition %d"
                         % (old.numel, new_part.numel))
    s_new = new_part.shard_numel
    tiled = _is_tiled(state)
    if tiled:
        if state[0].dtype != torch.float32 or state[0].numel() < tiled_state_numel(s_new):
            raise ValueError("the tiled state holds fewer than shard_numel elements' tiles")
    elif any(t.dtype != torch.float32 or t.numel() < s_new for t in state):
        raise ValueError("state is three fp32 tensors of shard_numel elements")
    n_new = zero_partition_valid_numel(new_part, new_rank)
    pieces = zero_repartition_plan(old, new_part, new_rank)
    if not tiled:
        for t in state:
            t[n_new:s_new].zero_()
        if not pieces:
            return step, scaler
        staging = _staging(state[0].device, max(p.count for p in pieces))
        for p in pieces:
            n_k = headers[p.old_rank].valid_numel
            with open(rank_path(directory, p.old_rank), "rb") as f:
                for field, t in enumerate(state):
                    f.seek(HEADER_BYTES + 4 * (field * n_k + p.old_offset))
                    _read_fp32(f, t[p.new_offset:p.new_offset + p.count], staging)
        return step, scaler
    # tiled: each piece is read a chunk at a time into three temporaries,
    # which the library tiles into place; the padding is tiled from zeros
    longest = max([p.count for p in pieces] + [s_new - n_new, 1])
    parts = _temporaries(state[0].device, min(longest, STAGING_ELEMS))
    if s_new > n_new:
        for x in parts:
            x.zero_()
        for a in range(n_new, s_new, STAGING_ELEMS):
            b = min(s_new, a + STAGING_ELEMS)
            zero_state_tile(*[x[:b - a] for x in parts], state[0], first=a, n=b - a)
    if not pieces:
        return step, scaler
    staging = _staging(state[0].device, min(longest, STAGING_ELEMS))
    for p in pieces:
        n_k = headers[p.old_rank].valid_numel
        with open(rank_path(directory, p.old_rank), "rb") as f:
            for a in range(0, p.count, STAGING_ELEMS):
                b = min(p.count, a + STAGING_ELEMS)
                for field, x in enumerate(parts):
                    f.seek(HEADER_BYTES + 4 * (field * n_k + p.old_offset + a))
                    _read_fp32(f, x[:b - a], staging)
                zero_state_tile(*[x[:b - a] for x in parts], state[0], first=p.new_offset + a,
                                n=b - a)
    return step, scaler
