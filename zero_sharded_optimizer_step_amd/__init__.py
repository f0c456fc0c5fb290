"""MI355X-native ZeRO sharded-optimizer step: Python binding.

Every function here has the name of the C entry point it calls (see
include/zero.h) and only marshals arguments: torch tensors become device
pointers, the current torch stream becomes the hipStream_t, and negative
status codes become ``ZeroError``.  All arithmetic of the step runs in the
HIP kernels of libzero_mi355x.so; nothing here computes on the CPU.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

from . import _abi
from ._abi import (ZERO_BF16, ZERO_CKPT_MAGIC, ZERO_CKPT_VERSION, ZERO_EALIGN, ZERO_EDEVICE,
                   ZERO_EINVAL, ZERO_ESIZE, ZERO_FP16, ZERO_FP32, ZERO_MAX_REPLICAS,
                   ZERO_NOALLOC_MAX_SHARD, ZERO_OK, ZERO_STATE_SEPARATE, ZERO_STATE_TILE,
                   ZERO_STATE_TILED, ZeroError,
                   check, lib, zero_bucket_t, zero_ckpt_header_t, zero_global_t,
                   zero_loss_scaler_t, zero_offload_staging_t, zero_partition_t,
                   zero_repartition_piece_t, zero_step_args, zero_step_info,
                   zero_step_scalars_t, zero_tensor_slot_t)

__all__ = [
    "ZERO_OK", "ZERO_EINVAL", "ZERO_EALIGN", "ZERO_ESIZE", "ZERO_EDEVICE",
    "ZERO_FP16", "ZERO_BF16", "ZERO_FP32", "ZERO_MAX_REPLICAS", "ZERO_NOALLOC_MAX_SHARD",
    "ZERO_STATE_SEPARATE", "ZERO_STATE_TILED", "ZERO_STATE_TILE", "tiled_state_numel",
    "ZeroError", "lib",
    "zero_last_error", "zero_partition", "zero_partition_valid_numel",
    "zero_bucket_plan", "zero_bucket_flatten", "zero_shard_workspace_bytes",
    "zero_partials_bytes", "zero_shard_reduce", "zero_shard_accumulate",
    "zero_accumulate_local", "zero_shard_combine",
    "zero_shard_apply", "zero_shard_step", "zero_shard_step_noalloc", "zero_step_scalars",
    "zero_loss_scaler_init",
    "zero_loss_scaler_update", "zero_ckpt_header_make", "zero_ckpt_header_check",
    "zero_repartition", "zero_repartition_plan", "zero_repartition_tiled", "zero_state_tile",
    "zero_state_untile", "zero_gather_params", "zero_offload_apply",
    "zero_host_adamw", "zero_host_threads",
    "OffloadStaging",
    "StepArgs", "dtype_code", "GLOBAL_BYTES",
]

GLOBAL_BYTES = ctypes.sizeof(zero_global_t)


def _torch():
    import torch
    return torch


def dtype_code(dtype) -> int:
    """ZERO_FP16 / ZERO_BF16 / ZERO_FP32 for a torch dtype (or pass an int
    through).  ZERO_FP32 is accepted only as a replica gradient format."""
    if isinstance(dtype, int):
        return dtype
    torch = _torch()
    if dtype == torch.float16:
        return ZERO_FP16
    if dtype == torch.bfloat16:
        return ZERO_BF16
    if dtype == torch.float32:
        return ZERO_FP32
    raise ValueError("only float16, bfloat16 and float32 are supported, got %s" % dtype)


def tiled_state_numel(shard_numel: int) -> int:
    """fp32 values of a rank's ZERO_STATE_TILED state: whole tiles of
    master, exp_avg and exp_avg_sq."""
    return 3 * ZERO_STATE_TILE * (-(-shard_numel // ZERO_STATE_TILE))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, nbytes: int, what: str) -> None:
    """Refuse a buffer smaller than the bytes a call will touch in it.  The
    C ABI receives only addresses, so this is the one place where a short
    tensor can be caught before a kernel reads or writes past its end."""
    if t is None or nbytes <= 0:
        return
    have = t.nbytes if isinstance(getattr(t, "nbytes", None), int) else t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s holds %d bytes; the call touches %d" % (what, have, nbytes))


# ------------------------------------------------------------------ host only
def zero_last_error() -> str:
    return lib().zero_last_error().decode()


def zero_partition(numel: int, world_size: int, alignment: int) -> zero_partition_t:
    out = zero_partition_t()
    check(lib().zero_partition(numel, world_size, alignment, ctypes.byref(out)),
          "zero_partition")
    return out


def zero_partition_valid_numel(part: zero_partition_t, rank: int) -> int:
    n = lib().zero_partition_valid_numel(ctypes.byref(part), rank)
    if n < 0:
        raise ValueError("rank %d outside the partition's world" % rank)
    return n


def zero_bucket_plan(tensor_numel: Sequence[int], reduce_bucket_size: int):
    """Return (slots, buckets) as ctypes arrays of zero_tensor_slot_t and
    zero_bucket_t."""
    n = len(tensor_numel)
    sizes = (_abi.i64 * max(n, 1))(*tensor_numel)
    slots = (zero_tensor_slot_t * max(n, 1))()
    nb = _abi.i32(0)
    cap = 0
    while True:
        buckets = (zero_bucket_t * max(cap, 1))()
        rc = lib().zero_bucket_plan(sizes, n, reduce_bucket_size, slots, buckets, cap,
                                    ctypes.byref(nb))
        if rc == ZERO_ESIZE and nb.value > cap:
            cap = nb.value
            continue
        check(rc, "zero_bucket_plan")
        break
    return slots[:n], buckets[:nb.value]


def zero_shard_workspace_bytes(shard_numel: int) -> int:
    return lib().zero_shard_workspace_bytes(shard_numel)


def zero_partials_bytes(n_slots: int) -> int:
    return lib().zero_partials_bytes(n_slots)


def zero_loss_scaler_init(initial_scale_power: int = 16, loss_scale_window: int = 100,
                          hysteresis: int = 2, min_loss_scale: float = 1.0) -> zero_loss_scaler_t:
    st = zero_loss_scaler_t()
    check(lib().zero_loss_scaler_init(initial_scale_power, loss_scale_window, hysteresis,
                                      min_loss_scale, ctypes.byref(st)),
          "zero_loss_scaler_init")
    return st


def zero_loss_scaler_update(st: zero_loss_scaler_t, overflow: bool) -> bool:
    """Advance the scaler by one step's overflow flag; True if skipped."""
    skip = _abi.i32(0)
    check(lib().zero_loss_scaler_update(ctypes.byref(st), 1 if overflow else 0,
                                        ctypes.byref(skip)), "zero_loss_scaler_update")
    return bool(skip.value)


# --------------------------------------------------------------- device calls
def zero_bucket_flatten(slots, srcs, dtype, flat, flat_numel: Optional[int] = None,
                        stream=None) -> None:
    """Copy tensors `srcs` (device) into `flat` at their slots' offsets,
    zero the gaps between consecutive slots and [end of the last slot,
    flat_numel)."""
    n = len(slots)
    if len(srcs) != n:
        raise ValueError("one source tensor per slot")
    arr = (zero_tensor_slot_t * max(n, 1))(*slots)
    ptrs = (_abi.vp * max(n, 1))(*[_dptr(s) for s in srcs])
    if flat_numel is None:
        flat_numel = flat.numel()
    _need(flat, 2 * flat_numel, "flat")
    for t, (sl, src) in enumerate(zip(slots, srcs)):
        _need(src, 2 * sl.numel, "srcs[%d]" % t)
    check(lib().zero_bucket_flatten(arr, n, ptrs, dtype_code(dtype), _dptr(flat), flat_numel,
                                    _stream(stream)), "zero_bucket_flatten")


@dataclass
class StepArgs:
    """Builds a zero_step_args from torch tensors and keeps the pointer
    array it refers to alive.  `replica_grads` are the per-replica slices
    that start at this rank's shard."""
    world_size: int
    rank: int
    shard_numel: int
    valid_numel: int
    replica_grads: Sequence
    master: object
    exp_avg: object
    exp_avg_sq: object
    full_params: object
    workspace: object
    lr: float = 6e-5
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1
    loss_scale: float = 1.0
    grad_predivide: float = 1.0
    max_grad_norm: float = 1.0
    grad_dtype: Optional[int] = None
    param_dtype: Optional[int] = None
    accumulate: bool = False
    param_shard: object = None          # ZeRO-3: the rank's own parameter shard
    master_out: object = None           # optional second state set (ping-pong)
    exp_avg_out: object = None
    exp_avg_sq_out: object = None
    # ZERO_STATE_TILED: `master` (and `master_out`) hold the tiled state and
    # exp_avg, exp_avg_sq (and their outputs) are None
    state_layout: int = ZERO_STATE_SEPARATE
    # device buffer (>= 64 bytes) holding a zero_step_scalars_t the kernels
    # read at run time instead of taking the scalars as launch arguments
    scalars: object = None

    def check_sizes(self, gsize: int) -> None:
        """Every buffer must hold what the step touches in it: valid_numel
        elements of each replica slice and state array, and the rank's
        slice of the full buffer (or its own parameter shard)."""
        n = self.valid_numel
        if n <= 0 or not 0 <= self.rank < self.world_size:
            return            # nothing is touched, or the library rejects the call
        for i, r in enumerate(self.replica_grads):
            _need(r, gsize * n, "replica_grads[%d]" % i)
        if self.state_layout == ZERO_STATE_TILED:
            for name in ("master", "master_out"):
                _need(getattr(self, name), 4 * tiled_state_numel(n), name)
        else:
            for name in ("master", "exp_avg", "exp_avg_sq", "master_out", "exp_avg_out",
                         "exp_avg_sq_out"):
                _need(getattr(self, name), 4 * n, name)
        if self.param_shard is not None:
            _need(self.param_shard, 2 * n, "param_shard")
        else:
            _need(self.full_params, 2 * (self.rank * self.shard_numel + n), "full_params")

    def c_args(self) -> zero_step_args:
        reps = list(self.replica_grads)
        self._ptrs = (_abi.vp * max(len(reps), 1))(*[_dptr(r) for r in reps])
        a = zero_step_args()
        a.world_size = self.world_size
        a.rank = self.rank
        a.shard_numel = self.shard_numel
        a.valid_numel = self.valid_numel
        a.grad_dtype = dtype_code(self.grad_dtype if self.grad_dtype is not None else reps[0].dtype)
        a.param_dtype = dtype_code(self.param_dtype if self.param_dtype is not None
                                   else (self.full_params if self.full_params is not None
                                         else self.param_shard).dtype)
        a.n_replicas = len(reps)
        a.accumulate = 1 if self.accumulate else 0
        a.replica_grad = ctypes.cast(self._ptrs, ctypes.POINTER(_abi.vp))
        a.master = _dptr(self.master)
        a.exp_avg = _dptr(self.exp_avg)
        a.exp_avg_sq = _dptr(self.exp_avg_sq)
        a.full_params = _dptr(self.full_params)
        a.param_shard = _dptr(self.param_shard)
        a.master_out = _dptr(self.master_out)
        a.exp_avg_out = _dptr(self.exp_avg_out)
        a.exp_avg_sq_out = _dptr(self.exp_avg_sq_out)
        a.workspace = _dptr(self.workspace)
        a.workspace_bytes = 0 if self.workspace is None else \
            self.workspace.numel() * self.workspace.element_size()
        a.lr, a.beta1, a.beta2, a.eps = self.lr, self.beta1, self.beta2, self.eps
        a.weight_decay = self.weight_decay
        a.step = self.step
        a.loss_scale = self.loss_scale
        a.grad_predivide = self.grad_predivide
        a.max_grad_norm = self.max_grad_norm
        a.state_layout = self.state_layout
        a.scalars = _dptr(self.scalars)
        _need(self.scalars, ctypes.sizeof(zero_step_scalars_t), "scalars")
        self.check_sizes(4 if a.grad_dtype == ZERO_FP32 else 2)
        self._c = a
        return a


def _args(a) -> zero_step_args:
    return a.c_args() if isinstance(a, StepArgs) else a


def zero_shard_reduce(args, slot: int, partials, stream=None) -> None:
    _need(partials, (slot + 1) * zero_partials_bytes(1), "partials")
    check(lib().zero_shard_reduce(ctypes.byref(_args(args)), slot, _dptr(partials),
                                  _stream(stream)), "zero_shard_reduce")


def zero_shard_accumulate(args, stream=None) -> None:
    """Pass 1 only, into the rank's workspace (micro-batches before the last
    of an accumulation window; args.accumulate selects set or add)."""
    check(lib().zero_shard_accumulate(ctypes.byref(_args(args)), _stream(stream)),
          "zero_shard_accumulate")


def zero_accumulate_local(grad, acc, first: bool, n: Optional[int] = None,
                          stream=None) -> None:
    """Gradient accumulation before the reduce: acc[:n] (fp32) is set to
    (first) or incremented by grad[:n] widened to fp32.  n defaults to
    grad.numel()."""
    n = grad.numel() if n is None else n
    _need(grad, grad.element_size() * n, "grad")
    _need(acc, 4 * n, "acc")
    check(lib().zero_accumulate_local(_dptr(grad), dtype_code(grad.dtype), _dptr(acc), n,
                                      1 if first else 0, _stream(stream)),
          "zero_accumulate_local")


def zero_shard_combine(partials, n_slots: int, max_grad_norm: float, global_buf,
                       stream=None) -> None:
    _need(partials, n_slots * zero_partials_bytes(1), "partials")
    _need(global_buf, GLOBAL_BYTES, "global_buf")
    check(lib().zero_shard_combine(_dptr(partials), n_slots, max_grad_norm, _dptr(global_buf),
                                   _stream(stream)), "zero_shard_combine")


def zero_shard_apply(args, global_buf, stream=None) -> None:
    _need(global_buf, GLOBAL_BYTES, "global_buf")
    check(lib().zero_shard_apply(ctypes.byref(_args(args)), _dptr(global_buf), _stream(stream)),
          "zero_shard_apply")


def zero_shard_step(args, peer_sumsq: float = 0.0, peer_overflow: bool = False,
                    want_info: bool = False, stream=None) -> Optional[zero_step_info]:
    """One rank's whole step.  With want_info the call waits for the stream
    and returns the combine's result; otherwise it returns None at once."""
    info = zero_step_info() if want_info else None
    check(lib().zero_shard_step(ctypes.byref(_args(args)), peer_sumsq, 1 if peer_overflow else 0,
                                ctypes.byref(info) if info is not None else None,
                                _stream(stream)), "zero_shard_step")
    return info


def zero_step_scalars(args, peer_sumsq: float = 0.0, peer_overflow: bool = False
                      ) -> zero_step_scalars_t:
    """The step's scalars, computed on the host, for a device copy that
    args.scalars points at (see zero.h)."""
    out = zero_step_scalars_t()
    check(lib().zero_step_scalars(ctypes.byref(_args(args)), peer_sumsq, 1 if peer_overflow else 0,
                                  ctypes.byref(out)), "zero_step_scalars")
    return out


def zero_shard_step_noalloc(args, peer_sumsq: float = 0.0, peer_overflow: bool = False,
                            want_info: bool = False, stream=None) -> Optional[zero_step_info]:
    """zero_shard_step with the library's own scratch memory as workspace
    (args.workspace must be None); allocates nothing."""
    info = zero_step_info() if want_info else None
    check(lib().zero_shard_step_noalloc(ctypes.byref(_args(args)), peer_sumsq,
                                        1 if peer_overflow else 0,
                                        ctypes.byref(info) if info is not None else None,
                                        _stream(stream)), "zero_shard_step_noalloc")
    return info


# ------------------------------------------------------- sharded checkpoint
def zero_ckpt_header_make(part: zero_partition_t, rank: int, param_dtype, step: int,
                          scaler: Optional[zero_loss_scaler_t] = None) -> zero_ckpt_header_t:
    h = zero_ckpt_header_t()
    check(lib().zero_ckpt_header_make(ctypes.byref(part), rank, dtype_code(param_dtype), step,
                                      ctypes.byref(scaler) if scaler is not None else None,
                                      ctypes.byref(h)), "zero_ckpt_header_make")
    return h


def zero_ckpt_header_check(header: zero_ckpt_header_t, file_bytes: int) -> zero_partition_t:
    """Validate a header read from a file of file_bytes bytes; return the
    partition it was saved under."""
    part = zero_partition_t()
    check(lib().zero_ckpt_header_check(ctypes.byref(header), file_bytes, ctypes.byref(part)),
          "zero_ckpt_header_check")
    return part


def zero_repartition(from_part: zero_partition_t, srcs: Sequence, to_part: zero_partition_t,
                     dsts: Sequence, stream=None) -> None:
    """Move one fp32 state array from partition from_part (one device tensor
    per old rank) to to_part (one device tensor per new rank)."""
    sp = (_abi.vp * max(len(srcs), 1))(*[_dptr(t) for t in srcs])
    dp = (_abi.vp * max(len(dsts), 1))(*[_dptr(t) for t in dsts])
    if len(srcs) != from_part.world_size or len(dsts) != to_part.world_size:
        raise ValueError("one tensor per rank of each partition")
    if from_part.numel == to_part.numel and from_part.world_size >= 1 and to_part.world_size >= 1:
        for k, t in enumerate(srcs):
            _need(t, 4 * max(0, min(from_part.shard_numel,
                                    from_part.numel - k * from_part.shard_numel)), "srcs[%d]" % k)
        for j, t in enumerate(dsts):
            _need(t, 4 * to_part.shard_numel, "dsts[%d]" % j)
    check(lib().zero_repartition(ctypes.byref(from_part), sp, ctypes.byref(to_part), dp,
                                 _stream(stream)), "zero_repartition")


def zero_repartition_tiled(from_part: zero_partition_t, srcs: Sequence, to_part: zero_partition_t,
                           dsts: Sequence, stream=None) -> None:
    """Move a ZERO_STATE_TILED state (one tiled tensor per rank) from
    partition from_part to to_part."""
    if len(srcs) != from_part.world_size or len(dsts) != to_part.world_size:
        raise ValueError("one tensor per rank of each partition")
    if from_part.numel == to_part.numel and from_part.world_size >= 1 and to_part.world_size >= 1:
        for k, t in enumerate(srcs):
            n_k = max(0, min(from_part.shard_numel, from_part.numel - k * from_part.shard_numel))
            _need(t, 4 * tiled_state_numel(n_k), "srcs[%d]" % k)
        for j, t in enumerate(dsts):
            _need(t, 4 * tiled_state_numel(to_part.shard_numel), "dsts[%d]" % j)
    sp = (_abi.vp * max(len(srcs), 1))(*[_dptr(t) for t in srcs])
    dp = (_abi.vp * max(len(dsts), 1))(*[_dptr(t) for t in dsts])
    check(lib().zero_repartition_tiled(ctypes.byref(from_part), sp, ctypes.byref(to_part), dp,
                                       _stream(stream)), "zero_repartition_tiled")


def zero_state_tile(master, exp_avg, exp_avg_sq, tiled, first: int = 0, n: Optional[int] = None,
                    stream=None) -> None:
    """Elements [0, n) of the three separate arrays into elements
    [first, first + n) of the tiled state (n defaults to master.numel())."""
    n = master.numel() if n is None else n
    for t, name in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        _need(t, 4 * n, name)
    _need(tiled, 4 * tiled_state_numel(first + n), "tiled")
    check(lib().zero_state_tile(_dptr(master), _dptr(exp_avg), _dptr(exp_avg_sq), n, _dptr(tiled),
                                first, _stream(stream)), "zero_state_tile")


def zero_state_untile(tiled, master, exp_avg, exp_avg_sq, first: int = 0,
                      n: Optional[int] = None, stream=None) -> None:
    """Elements [first, first + n) of the tiled state into elements [0, n)
    of the three separate arrays (n defaults to master.numel())."""
    n = master.numel() if n is None else n
    for t, name in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        _need(t, 4 * n, name)
    _need(tiled, 4 * tiled_state_numel(first + n), "tiled")
    check(lib().zero_state_untile(_dptr(tiled), first, n, _dptr(master), _dptr(exp_avg),
                                  _dptr(exp_avg_sq), _stream(stream)), "zero_state_untile")


def zero_repartition_plan(from_part: zero_partition_t, to_part: zero_partition_t,
                          new_rank: int) -> list:
    """The pieces (zero_repartition_piece_t) new rank `new_rank` of to_part
    reads from the old ranks of from_part, in ascending new_offset."""
    n = _abi.i32(0)
    cap = 0
    while True:
        pieces = (zero_repartition_piece_t * max(cap, 1))()
        rc = lib().zero_repartition_plan(ctypes.byref(from_part), ctypes.byref(to_part), new_rank,
                                         pieces, cap, ctypes.byref(n))
        if rc == ZERO_ESIZE and n.value > cap:
            cap = n.value
            continue
        check(rc, "zero_repartition_plan")
        return pieces[:n.value]


# ------------------------------------------------------- optimizer offload
class OffloadStaging:
    """Two pinned host buffers per direction for zero_offload_apply."""

    def __init__(self, chunk_elems: int = 1 << 25, n_threads: int = 0):
        torch = _torch()
        self.grad = [torch.empty(chunk_elems, dtype=torch.float32, pin_memory=True)
                     for _ in range(2)]
        self.param = [torch.empty(chunk_elems, dtype=torch.int16, pin_memory=True)
                      for _ in range(2)]
        self.c = zero_offload_staging_t()
        for i in range(2):
            self.c.grad_stage[i] = self.grad[i].data_ptr()
            self.c.param_stage[i] = self.param[i].data_ptr()
        self.c.chunk_elems = chunk_elems
        self.c.n_threads = n_threads


def zero_offload_apply(args, global_buf, staging: OffloadStaging, want_info: bool = False,
                       stream=None) -> Optional[zero_step_info]:
    """Pass 2 on the host: args.master / exp_avg / exp_avg_sq are host (pinned)
    tensors; waits for the stream."""
    info = zero_step_info() if want_info else None
    _need(global_buf, GLOBAL_BYTES, "global_buf")
    check(lib().zero_offload_apply(ctypes.byref(_args(args)), _dptr(global_buf),
                                   ctypes.byref(staging.c),
                                   ctypes.byref(info) if info is not None else None,
                                   _stream(stream)), "zero_offload_apply")
    return info


def zero_host_threads() -> int:
    """Host threads the offloaded update uses when n_threads is 0."""
    return int(lib().zero_host_threads())


def zero_host_adamw(g, coef: float, master, exp_avg, exp_avg_sq, params_out=None,
                    param_dtype=ZERO_BF16, lr: float = 6e-5, beta1: float = 0.9,
                    beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.01,
                    step: int = 1, n_threads: int = 0) -> None:
    """The offloaded update on host arrays (anything with data_ptr(), or
    numpy arrays via their ctypes data pointer)."""
    def ptr(x):
        if x is None:
            return None
        return x.data_ptr() if hasattr(x, "data_ptr") else x.ctypes.data
    n = g.numel() if hasattr(g, "numel") and callable(g.numel) else g.size
    for x, name in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        _need(x, 4 * n, name)
    _need(params_out, 2 * n, "params_out")
    check(lib().zero_host_adamw(n, ptr(g), coef, ptr(master), ptr(exp_avg), ptr(exp_avg_sq),
                                ptr(params_out), dtype_code(param_dtype), lr, beta1, beta2, eps,
                                weight_decay, step, n_threads), "zero_host_adamw")


# ------------------------------------------------------ ZeRO-3 gathering
def zero_gather_params(part: zero_partition_t, shards: Sequence, dtype, lo: int, hi: int, dst,
                       stream=None) -> None:
    """Copy flat parameters [lo, hi) into dst from the ranks' shards (one
    device tensor per rank)."""
    if len(shards) != part.world_size:
        raise ValueError("one shard per rank")
    s = part.shard_numel
    if s > 0 and 0 <= lo < hi <= part.numel:
        _need(dst, 2 * (hi - lo), "dst")
        for k in range(lo // s, (hi - 1) // s + 1):
            _need(shards[k], 2 * (min(hi, (k + 1) * s) - k * s), "shards[%d]" % k)
    sp = (_abi.vp * len(shards))(*[_dptr(t) for t in shards])
    check(lib().zero_gather_params(ctypes.byref(part), sp, dtype_code(dtype), lo, hi, _dptr(dst),
                                   _stream(stream)), "zero_gather_params")
