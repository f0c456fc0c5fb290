"""CPU oracle for the per-rank ZeRO sharded-optimizer step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It never imports the
HIP library and the HIP library never imports it.

The arithmetic lives in ``zero_oracle.c`` (plain scalar C, single thread);
this module only marshals numpy arrays into it and strings the primitives
together in the order the pages describe one optimizer step:

  * each rank owns one of N equal parts of the flat parameter space
    ("ZeRO技术解析：大模型分布式训练的革命性突破" §2.1, §4.1);
  * gradients are reduce-scattered, so a rank sums the replicas' values of
    its own slice only (same page §2.1; "ZeRO 和分片优化器", technical
    insight);
  * fp16 loss scaling with a dynamic scaler, or bf16 (first page §3.3, §5.1);
  * global-norm clipping at 1.0 (first page §6 configuration);
  * AdamW with lr 6e-5 and weight decay 0.01 (first page §3.1) on fp32
    master weights and moments ("ZeRO 和分片优化器" FAQ);
  * the updated part is all-gathered in the working precision (first page
    §2.1 and the §1.2.1 configuration).

Parity of the loss-scaler rule is unpinned by the pages (they give only the
knobs); every other function is pinned by the CPU tests.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

FP16 = 1
BF16 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zero_oracle.c")
# ZERO_ORACLE_LIB lets the mutation test load a deliberately broken copy.
_LIB_PATH = os.environ.get("ZERO_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def compile_oracle(src: str, out: str, strict: bool = True) -> None:
    """gcc -O2 with no contraction and no fast-math: every fp operation in
    the source is one IEEE-754 operation in the order written."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-fPIC", "-shared", "-Wall"]
    cmd += ["-Werror"] if strict else ["-w"]
    cmd += ["-I", _HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(force: bool = True) -> str:
    """Compile the oracle library in place (always, when force is set)."""
    if force or not os.path.exists(_LIB_PATH):
        compile_oracle(_SRC, _LIB_PATH)
    return _LIB_PATH


class _Scaler(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("good", ctypes.c_int32),
                ("hyst", ctypes.c_int32), ("window", ctypes.c_int32),
                ("hysteresis", ctypes.c_int32), ("min_scale", ctypes.c_double)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, f32, f64 = (ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                              ctypes.c_double)
        vp = ctypes.c_void_p
        L.oracle_partition.argtypes = [i64, i32, i32, vp, vp, vp]
        L.oracle_partition.restype = ctypes.c_int
        L.oracle_bucket_plan.argtypes = [vp, i32, i64, vp, vp]
        L.oracle_bucket_plan.restype = i32
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = f32
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = f32
        L.oracle_f32_to_f16.argtypes = [f32]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [f32]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        for name in ("oracle_f32_to_f16_array", "oracle_f32_to_bf16_array",
                     "oracle_f16_to_f32_array", "oracle_bf16_to_f32_array"):
            getattr(L, name).argtypes = [i64, vp, vp]
            getattr(L, name).restype = None
        L.oracle_reduce.argtypes = [i32, vp, i32, i64, f32, vp, vp, vp]
        L.oracle_reduce.restype = None
        L.oracle_reduce_accumulate.argtypes = [i32, vp, i32, i64, f32, vp, vp, vp]
        L.oracle_reduce_accumulate.restype = None
        L.oracle_accumulate_local.argtypes = [i32, i64, vp, vp, i32]
        L.oracle_accumulate_local.restype = None
        L.oracle_reduce_f32.argtypes = [i32, vp, i64, f32, vp, vp, vp]
        L.oracle_reduce_f32.restype = None
        L.oracle_clip.argtypes = [f64, f64, vp, vp]
        L.oracle_clip.restype = i32
        L.oracle_adamw.argtypes = [i64, vp, vp, vp, vp, f64, f64, f64, f64,
                                   f64, f64, i64]
        L.oracle_adamw.restype = None
        L.oracle_scaler_init.argtypes = [ctypes.POINTER(_Scaler), i32, i32,
                                         i32, f64]
        L.oracle_scaler_init.restype = None
        L.oracle_scaler_update.argtypes = [ctypes.POINTER(_Scaler), i32]
        L.oracle_scaler_update.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


# ---------------------------------------------------------------- partition
def partition(numel: int, world_size: int, alignment: int):
    """Return (shard_numel, padded_numel, valid_per_rank) or raise."""
    s = ctypes.c_int64()
    padded = ctypes.c_int64()
    valid = np.zeros(max(world_size, 1), dtype=np.int64)
    rc = lib().oracle_partition(numel, world_size, alignment,
                                ctypes.addressof(s), ctypes.addressof(padded),
                                _ptr(valid))
    if rc != 0:
        raise ValueError("invalid partition arguments")
    return s.value, padded.value, [int(x) for x in valid[:world_size]]


def bucket_plan(sizes, bucket_size: int):
    """Return (offsets, bucket_of, n_buckets) for tensors laid end to end."""
    n = np.ascontiguousarray(np.asarray(sizes, dtype=np.int64))
    off = np.zeros(max(len(n), 1), dtype=np.int64)
    bof = np.zeros(max(len(n), 1), dtype=np.int32)
    nb = lib().oracle_bucket_plan(_ptr(n) if len(n) else None, len(n),
                                  bucket_size, _ptr(off), _ptr(bof))
    if nb < 0:
        raise ValueError("invalid bucket arguments")
    return off[:len(n)].copy(), bof[:len(n)].copy(), nb


def flatten(tensors, bucket_size: int, padded_numel: int) -> np.ndarray:
    """contiguous_gradients ("ZeRO技术解析" §5.2): one replica's per-tensor
    16-bit gradients laid end to end, in order and with no gaps, at the
    offsets of the bucket plan, then zeros up to the padded length.  The
    buckets only group the copies; they do not move anything."""
    tensors = [np.ascontiguousarray(t, dtype=np.uint16) for t in tensors]
    offsets, _, _ = bucket_plan([t.size for t in tensors], bucket_size)
    end = int(offsets[-1]) + tensors[-1].size if tensors else 0
    if end > padded_numel:
        raise ValueError("the tensors hold more than padded_numel elements")
    flat = np.zeros(padded_numel, dtype=np.uint16)
    for t, off in zip(tensors, offsets):
        flat[int(off):int(off) + t.size] = t
    return flat


# ------------------------------------------------------------ number formats
def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_f16_array(x.size, _ptr(x), _ptr(out))
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(x.size, _ptr(x), _ptr(out))
    return out


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().oracle_f16_to_f32_array(h.size, _ptr(h), _ptr(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib().oracle_bf16_to_f32_array(b.size, _ptr(b), _ptr(out))
    return out


def to_low_precision(p: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_f16(p) if dtype == FP16 else f32_to_bf16(p)


# ------------------------------------------------------------------ reduce
def inv_scale(loss_scale: float, predivide: float = 1.0) -> np.float32:
    """fp32 of 1 / (loss_scale * predivide), the unscale multiplier."""
    return np.float32(1.0 / (float(loss_scale) * float(predivide)))


def reduce(replicas, dtype: int, inv: float, sumsq: float = 0.0,
           overflow: int = 0):
    """Sum the replicas' slices; return (g, sumsq, overflow) accumulated."""
    reps = [np.ascontiguousarray(r, dtype=np.uint16) for r in replicas]
    n = reps[0].size
    assert all(r.size == n for r in reps)
    arr = (ctypes.c_void_p * len(reps))(*[_ptr(r) for r in reps])
    g = np.empty(n, dtype=np.float32)
    ss = ctypes.c_double(sumsq)
    of = ctypes.c_int32(overflow)
    lib().oracle_reduce(len(reps), ctypes.addressof(arr), dtype, n,
                        np.float32(inv), _ptr(g), ctypes.addressof(ss),
                        ctypes.addressof(of))
    return g, ss.value, of.value


def reduce_accumulate(replicas, dtype: int, inv: float, g: np.ndarray, sumsq: float = 0.0,
                      overflow: int = 0):
    """Add one more micro-batch's reduced, unscaled slice into g (fp32, in
    place); return (sumsq, overflow) of the updated g, accumulated."""
    reps = [np.ascontiguousarray(r, dtype=np.uint16) for r in replicas]
    n = reps[0].size
    assert all(r.size == n for r in reps) and g.size == n
    assert g.dtype == np.float32 and g.flags["C_CONTIGUOUS"]
    arr = (ctypes.c_void_p * len(reps))(*[_ptr(r) for r in reps])
    ss = ctypes.c_double(sumsq)
    of = ctypes.c_int32(overflow)
    lib().oracle_reduce_accumulate(len(reps), ctypes.addressof(arr), dtype, n, np.float32(inv),
                                   _ptr(g), ctypes.addressof(ss), ctypes.addressof(of))
    return ss.value, of.value


def accumulate_local(micro_grads, dtype: int) -> np.ndarray:
    """One replica's micro-batch gradients (16-bit codes, equal lengths)
    summed into a new fp32 buffer in micro-batch order: the first sets it,
    each later one adds."""
    grads = [np.ascontiguousarray(x, dtype=np.uint16) for x in micro_grads]
    n = grads[0].size
    assert all(x.size == n for x in grads)
    acc = np.empty(n, dtype=np.float32)
    for j, x in enumerate(grads):
        lib().oracle_accumulate_local(dtype, n, _ptr(x), _ptr(acc), 1 if j == 0 else 0)
    return acc


def reduce_f32(replicas, inv: float, sumsq: float = 0.0, overflow: int = 0):
    """`reduce` over fp32 replica slices; return (g, sumsq, overflow)."""
    reps = [np.ascontiguousarray(r, dtype=np.float32) for r in replicas]
    n = reps[0].size
    assert all(r.size == n for r in reps)
    arr = (ctypes.c_void_p * len(reps))(*[_ptr(r) for r in reps])
    g = np.empty(n, dtype=np.float32)
    ss = ctypes.c_double(sumsq)
    of = ctypes.c_int32(overflow)
    lib().oracle_reduce_f32(len(reps), ctypes.addressof(arr), n, np.float32(inv), _ptr(g),
                            ctypes.addressof(ss), ctypes.addressof(of))
    return g, ss.value, of.value


def clip(sumsq: float, max_norm: float):
    """Return (applies, norm, coef)."""
    norm = ctypes.c_double()
    coef = ctypes.c_double()
    applies = lib().oracle_clip(sumsq, max_norm, ctypes.addressof(norm),
                                ctypes.addressof(coef))
    return bool(applies), norm.value, coef.value


def adamw(g, p, m, v, coef, lr, beta1, beta2, eps, weight_decay, t):
    """Update fp32 arrays p, m, v in place."""
    for a in (g, p, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    n = g.size
    assert p.size == n and m.size == n and v.size == n
    lib().oracle_adamw(n, _ptr(g), _ptr(p), _ptr(m), _ptr(v), float(coef),
                       float(lr), float(beta1), float(beta2), float(eps),
                       float(weight_decay), int(t))


# ------------------------------------------------- sharded checkpoint layout
def repartition(slices, numel: int, from_world: int, from_align: int, to_world: int,
                to_align: int):
    """Re-cut a sharded state array ("大模型分片训练" practice notes: a
    sharded checkpoint keeps the shard information).  The old ranks' real
    elements, concatenated in rank order, are the flat vector; it is cut by
    the new partition, each new slice padded with zeros to the shard size."""
    s_old, _, valid_old = partition(numel, from_world, from_align)
    s_new, _, valid_new = partition(numel, to_world, to_align)
    flat = np.concatenate([np.asarray(slices[r][:valid_old[r]]) for r in range(from_world)] +
                          [np.zeros(0, np.float32)])
    assert flat.size == numel
    out = []
    for r in range(to_world):
        x = np.zeros(s_new, np.float32)
        x[:valid_new[r]] = flat[r * s_new:r * s_new + valid_new[r]]
        out.append(x)
    return out


def gather(slices, numel: int, world: int, align: int, lo: int, hi: int):
    """ZeRO-3 all-gather of flat parameters [lo, hi) ("ZeRO 和分片优化器",
    technical insight): the ranks' real elements concatenated in rank order,
    sliced."""
    _, _, valid = partition(numel, world, align)
    flat = np.concatenate([np.asarray(slices[r][:valid[r]]) for r in range(world)] +
                          [np.zeros(0, np.asarray(slices[0]).dtype)])
    return flat[lo:hi].copy()


# ------------------------------------------------------------------ scaler
class LossScaler:
    """Dynamic loss scaler (reading; parity unpinned by the pages)."""

    def __init__(self, initial_scale_power=16, window=100, hysteresis=2,
                 min_scale=1.0):
        self._s = _Scaler()
        lib().oracle_scaler_init(ctypes.byref(self._s), initial_scale_power,
                                 window, hysteresis, min_scale)

    @property
    def scale(self) -> float:
        return self._s.scale

    @property
    def good(self) -> int:
        return self._s.good

    @property
    def hyst(self) -> int:
        return self._s.hyst

    def update(self, overflow: bool) -> bool:
        """Record one step's overflow flag; return True when it is skipped."""
        return bool(lib().oracle_scaler_update(ctypes.byref(self._s),
                                               1 if overflow else 0))


# ---------------------------------------------------------- one full step
@dataclass
class Hyper:
    lr: float = 6e-5
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 1.0
    loss_scale: float = 1.0
    predivide: float = 1.0


@dataclass
class StepInfo:
    sumsq: float
    norm: float
    coef: float
    clipped: bool
    overflow: bool
    skipped: bool
    grads: list = field(default_factory=list)   # reduced fp32 grad per rank


def step(replica_flats, dtype: int, numel: int, world_size: int,
         alignment: int, masters, exp_avgs, exp_avg_sqs, full_params,
         hp: Hyper, t: int, keep_grads: bool = False, cast: bool = True,
         param_dtype: Optional[int] = None) -> StepInfo:
    """One sharded step for every rank of the world, in rank order.

    replica_flats: N flat uint16 gradient buffers (one per data-parallel
        replica), each at least `numel` long (padding beyond is ignored).
    masters, exp_avgs, exp_avg_sqs: world_size fp32 arrays of shard length,
        updated in place (their padding tail is never touched).
    full_params: uint16 array of the padded full length; each rank's real
        elements are overwritten with its cast masters.
    A step whose reduced gradient holds inf or nan anywhere is skipped: no
    state changes, and the caller must not advance t.  With cast=False the
    full buffer is left alone (for steps whose cast nobody reads).
    param_dtype is the format of the full buffer, by default the gradients'.
    """
    return step_accumulated([replica_flats], dtype, numel, world_size, alignment, masters,
                            exp_avgs, exp_avg_sqs, full_params, hp, t, keep_grads, cast,
                            param_dtype)


def step_accumulated(micro_batches, dtype: int, numel: int, world_size: int,
                     alignment: int, masters, exp_avgs, exp_avg_sqs, full_params,
                     hp: Hyper, t: int, keep_grads: bool = False,
                     cast: bool = True, param_dtype: Optional[int] = None) -> StepInfo:
    """One sharded step over an accumulation window of K micro-batches.

    micro_batches: K lists of N replica flats (as `step` takes one).  For
    each rank, micro-batch 1 sets the rank's fp32 reduced slice and each
    later one adds to it; the norm, the overflow flag, clipping and AdamW
    then act on the accumulated slice, as in `step`.
    """
    s, padded, valid = partition(numel, world_size, alignment)
    inv = inv_scale(hp.loss_scale, hp.predivide)
    sumsq, overflow = 0.0, 0
    grads = []
    for r in range(world_size):
        lo, n = r * s, valid[r]
        g = None
        for k, flats in enumerate(micro_batches):
            reps = [f[lo:lo + n] for f in flats]
            last = k == len(micro_batches) - 1
            if k == 0:
                g, ss, of = reduce(reps, dtype, inv, sumsq if last else 0.0,
                                   overflow if last else 0)
            else:
                ss, of = reduce_accumulate(reps, dtype, inv, g, sumsq if last else 0.0,
                                           overflow if last else 0)
            if last:
                sumsq, overflow = ss, of
        grads.append(g)
    overflow = overflow or not math.isfinite(sumsq)
    applies, norm, coef = clip(sumsq, hp.max_grad_norm)
    info = StepInfo(sumsq, norm, coef, applies, bool(overflow),
                    bool(overflow), grads if keep_grads else [])
    if overflow:
        return info
    for r in range(world_size):
        lo, n = r * s, valid[r]
        p, m, v = masters[r][:n], exp_avgs[r][:n], exp_avg_sqs[r][:n]
        adamw(grads[r], p, m, v, coef, hp.lr, hp.beta1, hp.beta2, hp.eps,
              hp.weight_decay, t)
        if cast:
            full_params[lo:lo + n] = to_low_precision(p, param_dtype or dtype)
    return info


def step_local_accumulated(micro_batches, dtype: int, numel: int, world_size: int,
                           alignment: int, masters, exp_avgs, exp_avg_sqs, full_params,
                           hp: Hyper, t: int, keep_grads: bool = False,
                           cast: bool = True, param_dtype: Optional[int] = None) -> StepInfo:
    """One sharded step over an accumulation window of K micro-batches, with
    the window summed before the reduce (the no_sync pattern).

    micro_batches: K lists of N replica flats (as `step_accumulated` takes).
    Each replica first sums its K micro-batch gradients into an fp32 flat
    buffer of its own; each rank then reduces its slice of the N fp32
    buffers, and the norm, the overflow flag, clipping, AdamW and the cast
    follow as in `step`.
    """
    s, padded, valid = partition(numel, world_size, alignment)
    inv = inv_scale(hp.loss_scale, hp.predivide)
    n_rep = len(micro_batches[0])
    local = [accumulate_local([flats[i][:numel] for flats in micro_batches], dtype)
             for i in range(n_rep)]
    sumsq, overflow = 0.0, 0
    grads = []
    for r in range(world_size):
        lo, n = r * s, valid[r]
        g, sumsq, overflow = reduce_f32([a[lo:lo + n] for a in local], inv, sumsq, overflow)
        grads.append(g)
    overflow = overflow or not math.isfinite(sumsq)
    applies, norm, coef = clip(sumsq, hp.max_grad_norm)
    info = StepInfo(sumsq, norm, coef, applies, bool(overflow),
                    bool(overflow), grads if keep_grads else [])
    if overflow:
        return info
    for r in range(world_size):
        lo, n = r * s, valid[r]
        p, m, v = masters[r][:n], exp_avgs[r][:n], exp_avg_sqs[r][:n]
        adamw(grads[r], p, m, v, coef, hp.lr, hp.beta1, hp.beta2, hp.eps,
              hp.weight_decay, t)
        if cast:
            full_params[lo:lo + n] = to_low_precision(p, param_dtype or dtype)
    return info
