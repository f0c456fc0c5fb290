"""ctypes mirror of include/zero.h and the loader of libzero_mi355x.so.

Marshalling only: structures, argument types and the library handle.  The
library is loaded from this package's directory; if it is not there the
import of any entry point fails loudly (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libzero_mi355x.so")

ZERO_OK = 0
ZERO_EINVAL = -1
ZERO_EALIGN = -2
ZERO_ESIZE = -3
ZERO_EDEVICE = -4
ZERO_FP16 = 1
ZERO_BF16 = 2
ZERO_FP32 = 3
ZERO_MAX_REPLICAS = 64
ZERO_STATE_SEPARATE = 0
ZERO_STATE_TILED = 1
ZERO_STATE_TILE = 256
ZERO_NOALLOC_MAX_SHARD = 16777216

i32, i64, f32, f64, vp, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t)


class zero_partition_t(ctypes.Structure):
    _fields_ = [("numel", i64), ("shard_numel", i64), ("padded_numel", i64),
                ("world_size", i32), ("alignment", i32)]


class zero_tensor_slot_t(ctypes.Structure):
    _fields_ = [("offset", i64), ("numel", i64), ("bucket", i32), ("reserved", i32)]


class zero_bucket_t(ctypes.Structure):
    _fields_ = [("begin", i64), ("end", i64), ("first_tensor", i32), ("n_tensors", i32)]


class zero_step_args(ctypes.Structure):
    _fields_ = [("world_size", i32), ("rank", i32), ("shard_numel", i64),
                ("valid_numel", i64), ("grad_dtype", i32), ("param_dtype", i32),
                ("n_replicas", i32), ("accumulate", i32),
                ("replica_grad", ctypes.POINTER(vp)),
                ("master", vp), ("exp_avg", vp), ("exp_avg_sq", vp),
                ("full_params", vp), ("workspace", vp), ("workspace_bytes", sz),
                ("lr", f64), ("beta1", f64), ("beta2", f64), ("eps", f64),
                ("weight_decay", f64), ("step", i64), ("loss_scale", f64),
                ("grad_predivide", f64), ("max_grad_norm", f64), ("param_shard", vp),
                ("master_out", vp), ("exp_avg_out", vp), ("exp_avg_sq_out", vp),
                ("state_layout", i32), ("reserved", i32), ("scalars", vp)]


class zero_step_scalars_t(ctypes.Structure):
    _fields_ = [("inv_scale", f32), ("decay", f32), ("beta1", f32), ("one_minus_beta1", f32),
                ("beta2", f32), ("one_minus_beta2", f32), ("step_size", f32),
                ("inv_sqrt_bc2", f32), ("eps", f32), ("peer_overflow", i32),
                ("reserved", i32 * 2), ("max_grad_norm", f64), ("peer_sumsq", f64)]


assert ctypes.sizeof(zero_step_scalars_t) == 64


class zero_global_t(ctypes.Structure):
    _fields_ = [("sumsq", f64), ("norm", f64), ("coef", f32), ("overflow", i32),
                ("clipped", i32), ("reserved", i32)]


zero_step_info = zero_global_t


class zero_loss_scaler_t(ctypes.Structure):
    _fields_ = [("scale", f64), ("min_scale", f64), ("good_steps", i32),
                ("hysteresis_left", i32), ("window", i32), ("hysteresis", i32)]


ZERO_CKPT_MAGIC = 0x3143535A
ZERO_CKPT_VERSION = 1


class zero_ckpt_header_t(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("numel", i64),
                ("shard_numel", i64), ("valid_numel", i64), ("world_size", i32), ("rank", i32),
                ("alignment", i32), ("param_dtype", i32), ("step", i64), ("has_scaler", i32),
                ("reserved0", i32), ("scaler", zero_loss_scaler_t),
                ("payload_bytes", ctypes.c_uint64), ("pad", ctypes.c_uint8 * 24)]


assert ctypes.sizeof(zero_ckpt_header_t) == 128

class zero_repartition_piece_t(ctypes.Structure):
    _fields_ = [("old_offset", i64), ("new_offset", i64), ("count", i64), ("old_rank", i32),
                ("reserved", i32)]


class zero_offload_staging_t(ctypes.Structure):
    _fields_ = [("grad_stage", vp * 2), ("param_stage", vp * 2), ("chunk_elems", i64),
                ("n_threads", i32), ("reserved", i32)]


_PROTOTYPES = {
    "zero_last_error": (ctypes.c_char_p, []),
    "zero_partition": (ctypes.c_int, [i64, i32, i32, ctypes.POINTER(zero_partition_t)]),
    "zero_partition_valid_numel": (i64, [ctypes.POINTER(zero_partition_t), i32]),
    "zero_bucket_plan": (ctypes.c_int, [ctypes.POINTER(i64), i32, i64,
                                        ctypes.POINTER(zero_tensor_slot_t),
                                        ctypes.POINTER(zero_bucket_t), i32,
                                        ctypes.POINTER(i32)]),
    "zero_bucket_flatten": (ctypes.c_int, [ctypes.POINTER(zero_tensor_slot_t), i32,
                                           ctypes.POINTER(vp), i32, vp, i64, vp]),
    "zero_shard_workspace_bytes": (sz, [i64]),
    "zero_partials_bytes": (sz, [i32]),
    "zero_shard_reduce": (ctypes.c_int, [ctypes.POINTER(zero_step_args), i32, vp, vp]),
    "zero_shard_accumulate": (ctypes.c_int, [ctypes.POINTER(zero_step_args), vp]),
    "zero_shard_combine": (ctypes.c_int, [vp, i32, f64, vp, vp]),
    "zero_shard_apply": (ctypes.c_int, [ctypes.POINTER(zero_step_args), vp, vp]),
    "zero_shard_step": (ctypes.c_int, [ctypes.POINTER(zero_step_args), f64, i32,
                                       ctypes.POINTER(zero_step_info), vp]),
    "zero_step_scalars": (ctypes.c_int, [ctypes.POINTER(zero_step_args), f64, i32,
                                         ctypes.POINTER(zero_step_scalars_t)]),
    "zero_shard_step_noalloc": (ctypes.c_int, [ctypes.POINTER(zero_step_args), f64, i32,
                                               ctypes.POINTER(zero_step_info), vp]),
    "zero_loss_scaler_init": (ctypes.c_int, [i32, i32, i32, f64,
                                             ctypes.POINTER(zero_loss_scaler_t)]),
    "zero_loss_scaler_update": (ctypes.c_int, [ctypes.POINTER(zero_loss_scaler_t), i32,
                                               ctypes.POINTER(i32)]),
    "zero_ckpt_header_make": (ctypes.c_int, [ctypes.POINTER(zero_partition_t), i32, i32, i64,
                                             ctypes.POINTER(zero_loss_scaler_t),
                                             ctypes.POINTER(zero_ckpt_header_t)]),
    "zero_ckpt_header_check": (ctypes.c_int, [ctypes.POINTER(zero_ckpt_header_t), ctypes.c_uint64,
                                              ctypes.POINTER(zero_partition_t)]),
    "zero_repartition": (ctypes.c_int, [ctypes.POINTER(zero_partition_t), ctypes.POINTER(vp),
                                        ctypes.POINTER(zero_partition_t), ctypes.POINTER(vp), vp]),
    "zero_repartition_plan": (ctypes.c_int, [ctypes.POINTER(zero_partition_t),
                                             ctypes.POINTER(zero_partition_t), i32,
                                             ctypes.POINTER(zero_repartition_piece_t), i32,
                                             ctypes.POINTER(i32)]),
    "zero_state_tile": (ctypes.c_int, [vp, vp, vp, i64, vp, i64, vp]),
    "zero_state_untile": (ctypes.c_int, [vp, i64, i64, vp, vp, vp, vp]),
    "zero_repartition_tiled": (ctypes.c_int, [ctypes.POINTER(zero_partition_t), ctypes.POINTER(vp),
                                              ctypes.POINTER(zero_partition_t), ctypes.POINTER(vp),
                                              vp]),
    "zero_gather_params": (ctypes.c_int, [ctypes.POINTER(zero_partition_t), ctypes.POINTER(vp),
                                          i32, i64, i64, vp, vp]),
    "zero_offload_apply": (ctypes.c_int, [ctypes.POINTER(zero_step_args), vp,
                                          ctypes.POINTER(zero_offload_staging_t),
                                          ctypes.POINTER(zero_step_info), vp]),
    "zero_host_adamw": (ctypes.c_int, [i64, vp, f32, vp, vp, vp, vp, i32, f64, f64, f64, f64,
                                       f64, i64, i32]),
    "zero_host_threads": (i32, []),
    "zero_accumulate_local": (ctypes.c_int, [vp, i32, vp, i64, i32, vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libzero_mi355x.so is not built (expected at %s); run "
                "`python -m zero_sharded_optimizer_step_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOTYPES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class ZeroError(RuntimeError):
    """A library call returned a negative ZERO_E* status."""

    def __init__(self, code: int, where: str, message: str):
        super().__init__("%s failed with %d: %s" % (where, code, message))
        self.code = code


def check(code: int, where: str) -> None:
    if code != ZERO_OK:
        raise ZeroError(code, where, lib().zero_last_error().decode())
