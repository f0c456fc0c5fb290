"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
and its host-only logic (partition, bucket plan, loss scaler, argument
checks) matches the oracle.  No call here reaches the HIP runtime: device
entry points are only called with arguments they reject before any work.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import zero_sharded_optimizer_step_amd as Z
from zero_sharded_optimizer_step_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 13
    L = ctypes.CDLL(_abi.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert set(names) == set(_abi._PROTOTYPES), "binding and header disagree"


def test_code_hash_covers_host_and_device_code(tmp_path):
    # The key of the committed counter record: the built library's host
    # code and its gfx950 code object, read from the file.
    from zero_sharded_optimizer_step_amd import build
    h = build.code_hash(_abi.LIB_PATH)
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    assert build.code_hash(_abi.LIB_PATH) == h
    data = bytearray(open(_abi.LIB_PATH, "rb").read())
    secs = build._elf_sections(bytes(data))
    assert ".hip_fatbin" in secs and ".text" in secs
    # a flipped byte in the host code changes the hash
    text = secs[".text"]
    at = bytes(data).index(text[:4096]) + 100
    data[at] ^= 0xFF
    bad = tmp_path / "lib_flipped.so"
    bad.write_bytes(bytes(data))
    assert build.code_hash(str(bad)) != h
    # and so does one in the gfx950 kernels' code
    data[at] ^= 0xFF
    fb = secs[".hip_fatbin"]
    elf = fb.index(b"\x7fELF")
    dev_text = build._elf_sections(fb[elf:])[".text"]
    at = bytes(data).index(dev_text[:4096]) + 100
    data[at] ^= 0xFF
    bad.write_bytes(bytes(data))
    assert build.code_hash(str(bad)) != h
    junk = tmp_path / "junk.so"
    junk.write_bytes(b"not an ELF file")
    with pytest.raises(ValueError):
        build.code_hash(str(junk))


def test_binding_names_match_the_abi():
    for n in declared_symbols():
        assert callable(getattr(Z, n)), n


# ---------------------------------------------------------------- partition
def test_partition_matches_oracle():
    rng = np.random.default_rng(0)
    cases = [(P, N, A) for P in (0, 1, 7, 8, 127, 128, 129, 1000, 4096)
             for N in (1, 2, 3, 4, 7, 8, 16) for A in (1, 2, 8, 128)]
    cases += [(int(rng.integers(0, 2**40)), int(rng.integers(1, 1025)), int(2 ** rng.integers(0, 12)))
              for _ in range(500)]
    cases += [(13_000_000_000, 8, 128), (50_000_000, 4, 128), (67_125_248, 8, 128)]
    for P, N, A in cases:
        part = Z.zero_partition(P, N, A)
        s, padded, valid = oracle.partition(P, N, A)
        assert (part.shard_numel, part.padded_numel) == (s, padded), (P, N, A)
        assert [Z.zero_partition_valid_numel(part, r) for r in range(N)] == valid


@pytest.mark.parametrize("args", [(-1, 4, 8), (10, 0, 8), (10, 4, 0), (10, 4, 3), (10, 4, 96)])
def test_partition_rejects(args):
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_partition(*args)
    assert e.value.code == Z.ZERO_EINVAL
    assert Z.zero_last_error()


def test_partition_rejects_padded_counts_beyond_int64():
    big = 2**63 - 1
    part = Z.zero_partition(big, 1, 1)               # no padding needed: representable
    assert part.padded_numel == big
    for N, A in ((3, 1024), (8, 128), (2, 2)):
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_partition(big, N, A)
        assert e.value.code == Z.ZERO_EINVAL and "overflows" in Z.zero_last_error()
    # the largest count that still pads into int64 is accepted
    unit = 8 * 128
    top = (big // unit) * unit
    part = Z.zero_partition(top, 8, 128)
    assert part.padded_numel == top and part.shard_numel == top // 8


def test_partition_valid_numel_out_of_range():
    part = Z.zero_partition(100, 4, 8)
    with pytest.raises(ValueError):
        Z.zero_partition_valid_numel(part, 4)


# -------------------------------------------------------------- bucket plan
def test_bucket_plan_matches_oracle():
    rng = np.random.default_rng(1)
    for _ in range(300):
        T = int(rng.integers(0, 80))
        sizes = [int(x) for x in rng.integers(0, 3000, size=T)]
        if T and rng.random() < 0.3:
            sizes[int(rng.integers(T))] = 0
        cap = int(rng.integers(1, 6000))
        slots, buckets = Z.zero_bucket_plan(sizes, cap)
        off, bof, nb = oracle.bucket_plan(sizes, cap)
        assert [s.offset for s in slots] == list(off)
        assert [s.numel for s in slots] == sizes
        assert [s.bucket for s in slots] == list(bof)
        assert len(buckets) == nb
        for b, bk in enumerate(buckets):
            members = [t for t in range(T) if bof[t] == b]
            assert bk.first_tensor == members[0] and bk.n_tensors == len(members)
            assert bk.begin == off[members[0]]
            assert bk.end == off[members[-1]] + sizes[members[-1]]


def test_bucket_plan_ragged_workload():
    from zero_sharded_optimizer_step_amd.workloads import RAGGED_2000
    sizes = list(RAGGED_2000.tensor_sizes)
    slots, buckets = Z.zero_bucket_plan(sizes, int(2e8))
    off, bof, nb = oracle.bucket_plan(sizes, int(2e8))
    assert len(buckets) == nb and [s.bucket for s in slots] == list(bof)
    assert buckets[-1].end == sum(sizes) == RAGGED_2000.numel
    assert all(b.end - b.begin <= 2e8 for b in buckets)


def test_bucket_plan_rejects_sizes_summing_past_int64():
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_bucket_plan([2**62, 2**62, 2**62], int(2e8))
    assert e.value.code == Z.ZERO_EINVAL and "sum past int64" in Z.zero_last_error()
    slots, buckets = Z.zero_bucket_plan([2**62, 2**62 - 1], int(2e8))   # sums to 2^63 - 1
    assert [b.n_tensors for b in buckets] == [1, 1] and buckets[-1].end == 2**63 - 1


def test_bucket_plan_reports_needed_capacity():
    sizes = (_abi.i64 * 3)(5, 5, 5)
    slots = (_abi.zero_tensor_slot_t * 3)()
    buckets = (_abi.zero_bucket_t * 1)()
    nb = _abi.i32()
    rc = Z.lib().zero_bucket_plan(sizes, 3, 5, slots, buckets, 1, ctypes.byref(nb))
    assert rc == Z.ZERO_ESIZE and nb.value == 3
    rc = Z.lib().zero_bucket_plan(sizes, 3, 0, slots, buckets, 1, ctypes.byref(nb))
    assert rc == Z.ZERO_EINVAL


# ---------------------------------------------------------------- scaler
@pytest.mark.parametrize("seed", range(12))
def test_loss_scaler_matches_oracle(seed):
    # random knobs, floors that are and are not powers of two, and overflow
    # rates from rare to most steps, so runs sit at the floor for a while
    rng = np.random.default_rng(seed)
    window = int(rng.integers(1, 8))
    hyst = int(rng.integers(1, 4))
    power = int(rng.integers(-4, 20))
    floor = [1.0, 0.25, 3.0, 256.0][seed % 4]
    rate = [0.05, 0.2, 0.6][seed % 3]
    mine = Z.zero_loss_scaler_init(power, window, hyst, floor)
    ref = oracle.LossScaler(power, window, hyst, floor)
    for _ in range(400):
        of = bool(rng.random() < rate)
        assert Z.zero_loss_scaler_update(mine, of) == ref.update(of)
        assert mine.scale == ref.scale
        assert mine.good_steps == ref.good and mine.hysteresis_left == ref.hyst


def test_loss_scaler_rejects():
    for args in ((16, 0, 2, 1.0), (16, 100, 0, 1.0), (16, 100, 2, 0.0), (200, 100, 2, 1.0)):
        with pytest.raises(Z.ZeroError):
            Z.zero_loss_scaler_init(*args)
    st = _abi.zero_loss_scaler_t()        # never initialised
    with pytest.raises(Z.ZeroError):
        Z.zero_loss_scaler_update(st, False)


# ------------------------------------------------ argument checks, no device
class FakeTensor:
    """Stands in for a device tensor: only an address and a size."""

    def __init__(self, addr, nbytes=1 << 20, dtype=None):
        self.addr, self.nbytes, self.dtype = addr, nbytes, dtype

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def good_args(**kw):
    import torch
    s = 1024
    d = dict(world_size=4, rank=1, shard_numel=s, valid_numel=s,
             replica_grads=[FakeTensor(0x10000 * (i + 1), dtype=torch.bfloat16) for i in range(4)],
             master=FakeTensor(0x100000), exp_avg=FakeTensor(0x200000),
             exp_avg_sq=FakeTensor(0x300000),
             full_params=FakeTensor(0x400000, dtype=torch.bfloat16),
             workspace=FakeTensor(0x500000, Z.zero_shard_workspace_bytes(s)),
             grad_dtype=Z.ZERO_BF16, param_dtype=Z.ZERO_BF16)
    d.update(kw)
    return Z.StepArgs(**d)


BAD = [
    (dict(world_size=0), Z.ZERO_EINVAL), (dict(rank=4), Z.ZERO_EINVAL),
    (dict(rank=-1), Z.ZERO_EINVAL), (dict(shard_numel=1001, valid_numel=10), Z.ZERO_EINVAL),
    (dict(valid_numel=1025), Z.ZERO_EINVAL), (dict(step=0), Z.ZERO_EINVAL),
    (dict(loss_scale=0.0), Z.ZERO_EINVAL), (dict(grad_predivide=-1.0), Z.ZERO_EINVAL),
    (dict(beta1=1.0), Z.ZERO_EINVAL), (dict(beta2=-0.1), Z.ZERO_EINVAL),
    (dict(eps=0.0), Z.ZERO_EINVAL), (dict(lr=float("nan")), Z.ZERO_EINVAL),
    (dict(max_grad_norm=float("nan")), Z.ZERO_EINVAL), (dict(grad_dtype=4), Z.ZERO_EINVAL),
    (dict(param_dtype=0), Z.ZERO_EINVAL), (dict(replica_grads=[]), Z.ZERO_EINVAL),
    (dict(replica_grads=[FakeTensor(0x10000 * (i + 1)) for i in range(Z.ZERO_MAX_REPLICAS + 1)]),
     Z.ZERO_EINVAL),
    (dict(master=FakeTensor(0)), Z.ZERO_EINVAL),
    (dict(master=FakeTensor(0x100004)), Z.ZERO_EALIGN),
    (dict(full_params=FakeTensor(0x400002)), Z.ZERO_EALIGN),
    (dict(workspace=FakeTensor(0x500000, 64)), Z.ZERO_ESIZE),
]


@pytest.mark.parametrize("kw,code", BAD)
def test_step_rejects_bad_arguments_before_any_work(kw, code):
    import torch
    if kw.get("replica_grads") == []:
        a = good_args()
        c = a.c_args()
        c.n_replicas = 0
        rc = Z.lib().zero_shard_step(ctypes.byref(c), 0.0, 0, None, None)
        assert rc == code
        return
    a = good_args(**kw)
    for call in (lambda: Z.zero_shard_step(a, stream=0),
                 lambda: Z.zero_shard_reduce(a, 0, FakeTensor(0x600000), stream=0),
                 lambda: Z.zero_shard_apply(a, FakeTensor(0x700000), stream=0)):
        with pytest.raises(Z.ZeroError) as e:
            call()
        assert e.value.code == code, Z.zero_last_error()


def test_misaligned_replica_pointer():
    import torch
    reps = [FakeTensor(0x10000, dtype=torch.bfloat16), FakeTensor(0x20008, dtype=torch.bfloat16)]
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_shard_step(good_args(replica_grads=reps), stream=0)
    assert e.value.code == Z.ZERO_EALIGN and "replica_grad[1]" in Z.zero_last_error()


def test_combine_and_flatten_reject():
    L = Z.lib()
    assert L.zero_shard_combine(None, 1, 1.0, 0x1000, None) == Z.ZERO_EINVAL
    assert L.zero_shard_combine(0x1000, 0, 1.0, 0x2000, None) == Z.ZERO_EINVAL
    assert L.zero_shard_combine(0x1008, 1, 1.0, 0x2000, None) == Z.ZERO_EALIGN
    assert L.zero_shard_combine(0x1000, 1, float("nan"), 0x2000, None) == Z.ZERO_EINVAL
    slots = (_abi.zero_tensor_slot_t * 2)()
    slots[0].offset, slots[0].numel = 0, 10
    slots[1].offset, slots[1].numel = 5, 10          # overlaps slot 0
    ptrs = (_abi.vp * 2)(0x1000, 0x2000)
    assert L.zero_bucket_flatten(slots, 2, ptrs, Z.ZERO_BF16, 0x4000, 100, None) == Z.ZERO_EINVAL
    slots[1].offset = 10
    assert L.zero_bucket_flatten(slots, 2, ptrs, Z.ZERO_BF16, 0x4000, 15, None) == Z.ZERO_EINVAL
    assert L.zero_bucket_flatten(slots, 2, ptrs, 7, 0x4000, 100, None) == Z.ZERO_EINVAL
    # an offset near the top of int64 is out of range, not an overflow
    slots[1].offset, slots[1].numel = 2**63 - 5, 10
    assert L.zero_bucket_flatten(slots, 2, ptrs, Z.ZERO_BF16, 0x4000, 100, None) == Z.ZERO_EINVAL
    assert "out of order or outside" in Z.zero_last_error()
    slots[1].offset, slots[1].numel = 10, 10
    assert L.zero_bucket_flatten(slots, 2, ptrs, Z.ZERO_BF16, 0x4002, 100, None) == Z.ZERO_EALIGN
    ptrs[1] = 0x2001
    assert L.zero_bucket_flatten(slots, 2, ptrs, Z.ZERO_BF16, 0x4000, 100, None) == Z.ZERO_EALIGN


def test_binding_refuses_buffers_shorter_than_the_call_touches():
    # The C ABI sees addresses only; the binding compares each buffer's size
    # with the extent the kernels touch and raises before any call.
    import torch
    s = 1024
    with pytest.raises(ValueError, match="master"):
        Z.zero_shard_step(good_args(master=FakeTensor(0x100000, 4 * s - 4)), stream=0)
    with pytest.raises(ValueError, match="replica_grads\\[2\\]"):
        reps = [FakeTensor(0x10000 * (i + 1), 2 * s, dtype=torch.bfloat16) for i in range(4)]
        reps[2] = FakeTensor(0x30000, 2 * s - 2, dtype=torch.bfloat16)
        Z.zero_shard_step(good_args(replica_grads=reps), stream=0)
    # rank 1 writes full-buffer elements [s, 2s)
    with pytest.raises(ValueError, match="full_params"):
        Z.zero_shard_step(good_args(full_params=FakeTensor(0x400000, 2 * 2 * s - 2,
                                                           dtype=torch.bfloat16)), stream=0)
    # exactly enough passes the size check and reaches the library's own checks
    ok = good_args(master=FakeTensor(0x100000, 4 * s), valid_numel=s, step=0)
    with pytest.raises(Z.ZeroError):
        Z.zero_shard_step(ok, stream=0)
    with pytest.raises(ValueError, match="acc"):
        Z.zero_accumulate_local(FakeTensor(0x10000, 200, dtype=torch.bfloat16),
                                FakeTensor(0x20000, 399), True, n=100, stream=0)
    with pytest.raises(ValueError, match="global_buf"):
        Z.zero_shard_combine(FakeTensor(0x10000, Z.zero_partials_bytes(2)), 2, 1.0,
                             FakeTensor(0x20000, Z.GLOBAL_BYTES - 1), stream=0)
    with pytest.raises(ValueError, match="partials"):
        Z.zero_shard_combine(FakeTensor(0x10000, Z.zero_partials_bytes(2) - 1), 2, 1.0,
                             FakeTensor(0x20000, Z.GLOBAL_BYTES), stream=0)
    slots, _ = Z.zero_bucket_plan([10, 7], 100)
    with pytest.raises(ValueError, match="srcs\\[1\\]"):
        Z.zero_bucket_flatten(slots, [FakeTensor(0x1000, 20), FakeTensor(0x2000, 13)],
                              torch.bfloat16, FakeTensor(0x4000, 64), 32, stream=0)
    with pytest.raises(ValueError, match="flat"):
        Z.zero_bucket_flatten(slots, [FakeTensor(0x1000, 20), FakeTensor(0x2000, 14)],
                              torch.bfloat16, FakeTensor(0x4000, 63), 32, stream=0)
    part = Z.zero_partition(100, 4, 8)               # shards of 32; rank 3 holds 4 real
    shards = [FakeTensor(0x1000 * (k + 1), 64) for k in range(4)]
    shards[3] = FakeTensor(0x4000, 7)
    with pytest.raises(ValueError, match="shards\\[3\\]"):
        Z.zero_gather_params(part, shards, torch.bfloat16, 90, 100, FakeTensor(0x9000, 64),
                             stream=0)
    with pytest.raises(ValueError, match="dst"):
        Z.zero_gather_params(part, [FakeTensor(0x1000 * (k + 1), 64) for k in range(4)],
                             torch.bfloat16, 10, 50, FakeTensor(0x9000, 79), stream=0)
    to = Z.zero_partition(100, 2, 8)                 # new shards of 56 fp32
    with pytest.raises(ValueError, match="dsts\\[1\\]"):
        Z.zero_repartition(part, [FakeTensor(0x1000 * (k + 1), 128) for k in range(4)], to,
                           [FakeTensor(0x8000, 224), FakeTensor(0x9000, 223)], stream=0)
    with pytest.raises(ValueError, match="srcs\\[3\\]"):
        Z.zero_repartition(part, [FakeTensor(0x1000 * (k + 1), 128) for k in range(3)] +
                           [FakeTensor(0x4000, 15)], to,
                           [FakeTensor(0x8000, 224), FakeTensor(0x9000, 224)], stream=0)
    g = np.zeros(100, np.float32)
    with pytest.raises(ValueError, match="exp_avg_sq"):
        Z.zero_host_adamw(g, 1.0, np.zeros(100, np.float32), np.zeros(100, np.float32),
                          np.zeros(99, np.float32))
    with pytest.raises(ValueError, match="params_out"):
        Z.zero_host_adamw(g, 1.0, np.zeros(100, np.float32), np.zeros(100, np.float32),
                          np.zeros(100, np.float32), params_out=np.zeros(99, np.uint16))


def test_workspace_and_partials_sizes():
    slot = Z.zero_partials_bytes(1)
    assert slot >= 16 + 256 * 16
    assert Z.zero_partials_bytes(8) == 8 * slot
    for s in (0, 8, 1024, 1_625_000_064):
        ws = Z.zero_shard_workspace_bytes(s)
        # reduced gradient, one 16-byte partial per 1024 elements, a slot, the result
        assert ws >= 4 * s + 16 * -(-s // 1024) + slot + 32 and ws % 256 == 0
    assert Z.zero_shard_workspace_bytes(1_625_000_064) < 4 * 1_625_000_064 * 1.01


def test_accumulate_flag_must_be_zero_or_one():
    a = good_args()
    c = a.c_args()
    c.accumulate = 2
    for rc in (Z.lib().zero_shard_step(ctypes.byref(c), 0.0, 0, None, None),
               Z.lib().zero_shard_accumulate(ctypes.byref(c), None)):
        assert rc == Z.ZERO_EINVAL and "accumulate" in Z.zero_last_error()


def test_output_state_pointers_are_checked():
    c = good_args().c_args()
    c.master_out = 0x800000
    rc = Z.lib().zero_shard_step(ctypes.byref(c), 0.0, 0, None, None)
    assert rc == Z.ZERO_EINVAL and "together" in Z.zero_last_error()
    c.exp_avg_out, c.exp_avg_sq_out = 0x900000, 0xA00008
    assert Z.lib().zero_shard_step(ctypes.byref(c), 0.0, 0, None, None) == Z.ZERO_EALIGN
    c.exp_avg_sq_out = c.exp_avg_sq
    assert Z.lib().zero_shard_step(ctypes.byref(c), 0.0, 0, None, None) == Z.ZERO_EINVAL
    c.exp_avg_sq_out = 0xA00000
    st = Z.zero_offload_staging_t()
    assert Z.lib().zero_offload_apply(ctypes.byref(c), 0x1000, ctypes.byref(st), None,
                                      None) == Z.ZERO_EINVAL
    assert "in place" in Z.zero_last_error()


def test_accumulate_local_rejects_bad_arguments_before_any_work():
    # Fake device addresses: every call must fail in the host checks.
    L = Z.lib()
    g, acc = 0x100000, 0x200000
    cases = [
        ((g, Z.ZERO_BF16, acc, -1, 1), Z.ZERO_EINVAL),          # n < 0
        ((g, Z.ZERO_FP32, acc, 64, 1), Z.ZERO_EINVAL),          # fp32 is not a micro-batch format
        ((g, 0, acc, 64, 1), Z.ZERO_EINVAL),
        ((g, Z.ZERO_BF16, acc, 64, 2), Z.ZERO_EINVAL),          # first not 0 or 1
        ((None, Z.ZERO_BF16, acc, 64, 1), Z.ZERO_EINVAL),
        ((g, Z.ZERO_BF16, None, 64, 0), Z.ZERO_EINVAL),
        ((g + 2, Z.ZERO_BF16, acc, 64, 1), Z.ZERO_EALIGN),
        ((g, Z.ZERO_BF16, acc + 4, 64, 1), Z.ZERO_EALIGN),
        ((acc + 64, Z.ZERO_FP16, acc, 64, 1), Z.ZERO_EINVAL),   # overlapping
    ]
    for args, code in cases:
        assert L.zero_accumulate_local(*args, None) == code, args
        assert Z.zero_last_error()
    assert L.zero_accumulate_local(None, Z.ZERO_BF16, None, 0, 1, None) == Z.ZERO_OK   # empty


def test_step_accepts_fp32_replicas_only_as_gradients():
    import torch
    a = good_args(replica_grads=[FakeTensor(0x10000 * (i + 1), dtype=torch.float32)
                                 for i in range(4)], grad_dtype=None)
    assert a.c_args().grad_dtype == Z.ZERO_FP32
    bad = good_args(param_dtype=Z.ZERO_FP32)
    with pytest.raises(Z.ZeroError):
        Z.zero_shard_step(bad, stream=0)


# ------------------------------------------- partitions are re-derived, not trusted
def _hand_built(numel, world, align, shard, padded=None):
    p = _abi.zero_partition_t()
    p.numel, p.world_size, p.alignment = numel, world, align
    p.shard_numel = shard
    p.padded_numel = shard * world if padded is None else padded
    return p


@pytest.mark.parametrize("part", [
    _hand_built(1000, 4, 8, 264),                      # covers numel but is not minimal
    _hand_built(1000, 4, 8, 256, padded=1000),          # padded_numel inconsistent
    _hand_built(1000, 4, 8, 2**62),                     # shard * world overflows int64
    _hand_built(1000, 4, 3, 252),                       # alignment not a power of two
    _hand_built(1000, 0, 8, 256),                       # no ranks
    _hand_built(-1, 4, 8, 0),                           # negative numel
])
def test_gather_and_repartition_refuse_inconsistent_partitions(part):
    # Both checks run before any device work, so no GPU is needed.
    L = Z.lib()
    shards = (_abi.vp * 4)(0x1000, 0x2000, 0x3000, 0x4000)
    assert L.zero_gather_params(ctypes.byref(part), shards, Z.ZERO_BF16, 0, 10, 0x8000,
                                None) == Z.ZERO_EINVAL
    good = Z.zero_partition(1000, 4, 8)
    ptrs = (_abi.vp * 4)(0x1000, 0x2000, 0x3000, 0x4000)
    assert L.zero_repartition(ctypes.byref(part), ptrs, ctypes.byref(good), ptrs,
                              None) == Z.ZERO_EINVAL
    assert L.zero_repartition(ctypes.byref(good), ptrs, ctypes.byref(part), ptrs,
                              None) == Z.ZERO_EINVAL


_EMPTY_RANK_CALLS = r"""
import ctypes, sys
sys.path.insert(0, %r)
import zero_sharded_optimizer_step_amd as Z
from zero_sharded_optimizer_step_amd import _abi
L = Z.lib()
a = _abi.zero_step_args()
a.world_size, a.rank, a.shard_numel, a.valid_numel = 8, 7, 1024, 0
a.grad_dtype = a.param_dtype = Z.ZERO_BF16
a.n_replicas, a.step, a.loss_scale, a.grad_predivide = 8, 1, 1.0, 1.0
a.lr, a.beta1, a.beta2, a.eps = 1e-3, 0.9, 0.999, 1e-8
a.workspace = 0x100000
a.workspace_bytes = 1 << 30
a.replica_grad = None           # an empty rank passes no replica array
codes = [L.zero_shard_accumulate(ctypes.byref(a), None),
         L.zero_shard_reduce(ctypes.byref(a), 0, 0x200000, None),
         L.zero_shard_step(ctypes.byref(a), 0.0, 0, None, None)]
print(codes)
"""


def test_empty_rank_may_pass_no_replica_array():
    # valid_numel 0 accepts replica_grad == NULL.  The calls pass their
    # checks and reach the launch, which on a machine without a GPU fails
    # with ZERO_EDEVICE; the process must not crash on the NULL array.  Run
    # in a child so that a crash fails this test only.
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "-c", _EMPTY_RANK_CALLS % ROOT], capture_output=True,
                       text=True, timeout=120, env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode == 0, r.stderr[-2000:]
    codes = eval(r.stdout.strip().splitlines()[-1])
    assert all(c in (Z.ZERO_OK, Z.ZERO_EDEVICE) for c in codes), codes


# ------------------------------------------------- the allocation-free step
@pytest.mark.parametrize("kw,code", [kc for kc in BAD if "workspace" not in kc[0]])
def test_noalloc_step_rejects_bad_arguments_before_any_work(kw, code):
    if kw.get("replica_grads") == []:
        return                                  # the binding cannot build that struct
    a = good_args(workspace=None, **kw)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_shard_step_noalloc(a, stream=0)
    assert e.value.code == code, Z.zero_last_error()


def test_noalloc_step_own_limits():
    # A caller's workspace, an accumulation window and shards beyond the
    # scratch array are refused before the scratch address is even looked up.
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_shard_step_noalloc(good_args(), stream=0)
    assert e.value.code == Z.ZERO_EINVAL and "workspace must be NULL" in Z.zero_last_error()
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_shard_step_noalloc(good_args(workspace=None, accumulate=True), stream=0)
    assert e.value.code == Z.ZERO_EINVAL and "accumulate" in Z.zero_last_error()
    big = Z.ZERO_NOALLOC_MAX_SHARD + 8
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_shard_step_noalloc(good_args(workspace=None, shard_numel=big, valid_numel=0),
                                  stream=0)
    assert e.value.code == Z.ZERO_ESIZE
    # the largest accepted shard's workspace is what the scratch array holds
    assert Z.zero_shard_workspace_bytes(Z.ZERO_NOALLOC_MAX_SHARD) == 67_375_616
    assert Z.zero_shard_workspace_bytes(Z.ZERO_NOALLOC_MAX_SHARD - 8) <= 67_375_616


# ------------------------------------------------------ the tiled state layout
def tiled_args(**kw):
    d = dict(exp_avg=None, exp_avg_sq=None, state_layout=Z.ZERO_STATE_TILED,
             master=FakeTensor(0x1000000, 4 * Z.tiled_state_numel(1024)))
    d.update(kw)
    return good_args(**d)


@pytest.mark.parametrize("kw,code,what", [
    (dict(exp_avg=FakeTensor(0x200000)), Z.ZERO_EINVAL, "must be NULL"),
    (dict(exp_avg_sq=FakeTensor(0x300000)), Z.ZERO_EINVAL, "must be NULL"),
    (dict(master=FakeTensor(0)), Z.ZERO_EINVAL, "NULL"),
    (dict(master=FakeTensor(0x1000008, 1 << 20)), Z.ZERO_EALIGN, "aligned"),
    (dict(master_out=FakeTensor(0x1000000, 1 << 20)), Z.ZERO_EINVAL, "output state"),
    (dict(master_out=FakeTensor(0x2000004, 1 << 20)), Z.ZERO_EALIGN, "master_out"),
    (dict(state_layout=2), Z.ZERO_EINVAL, "state_layout"),
])
def test_tiled_state_arguments_are_checked(kw, code, what):
    a = tiled_args(**kw)
    for call in (lambda: Z.zero_shard_step(a, stream=0),
                 lambda: Z.zero_shard_apply(a, FakeTensor(0x700000), stream=0)):
        with pytest.raises(Z.ZeroError) as e:
            call()
        assert e.value.code == code and what in Z.zero_last_error(), Z.zero_last_error()


def test_tiled_state_sizes_and_binding_checks():
    assert Z.tiled_state_numel(0) == 0
    assert Z.tiled_state_numel(1) == 768 and Z.tiled_state_numel(256) == 768
    assert Z.tiled_state_numel(257) == 1536
    assert Z.tiled_state_numel(1_625_000_064) == 3 * 256 * 6_347_657
    # the binding refuses a tiled state shorter than its whole tiles
    with pytest.raises(ValueError):
        tiled_args(master=FakeTensor(0x1000000, 4 * Z.tiled_state_numel(1024) - 4)).c_args()
    # a separate-layout call still needs all three arrays
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_shard_step(good_args(exp_avg=None), stream=0)
    assert e.value.code == Z.ZERO_EINVAL


def test_layout_conversions_reject_bad_arguments_before_any_work():
    L = Z.lib()
    a, b, c, t = 0x10000, 0x20000, 0x30000, 0x40000
    assert L.zero_state_tile(a, b, c, 0, None, 0, None) == Z.ZERO_OK         # nothing to do
    assert L.zero_state_tile(a, b, c, -1, t, 0, None) == Z.ZERO_EINVAL
    assert L.zero_state_tile(a, b, c, 10, t, -1, None) == Z.ZERO_EINVAL
    assert L.zero_state_tile(a, None, c, 10, t, 0, None) == Z.ZERO_EINVAL
    assert L.zero_state_tile(a, b, c + 4, 10, t, 0, None) == Z.ZERO_EALIGN
    assert L.zero_state_untile(t, 0, 10, a, b, None, None) == Z.ZERO_EINVAL
    assert L.zero_state_untile(t + 8, 0, 10, a, b, c, None) == Z.ZERO_EALIGN
    assert L.zero_state_untile(t, 2**62, 2**62, a, b, c, None) == Z.ZERO_EINVAL
    good = Z.zero_partition(1000, 4, 8)
    bad = Z.zero_partition(1000, 4, 8)
    bad.shard_numel = 512
    ptrs = (_abi.vp * 4)(0x100000, 0x200000, 0x300000, 0x400000)
    assert L.zero_repartition_tiled(ctypes.byref(bad), ptrs, ctypes.byref(good), ptrs,
                                    None) == Z.ZERO_EINVAL
    other = Z.zero_partition(999, 4, 8)
    assert L.zero_repartition_tiled(ctypes.byref(good), ptrs, ctypes.byref(other), ptrs,
                                    None) == Z.ZERO_EINVAL
    mis = (_abi.vp * 4)(0x100000, 0x200004, 0x300000, 0x400000)
    assert L.zero_repartition_tiled(ctypes.byref(good), mis, ctypes.byref(good), ptrs,
                                    None) == Z.ZERO_EALIGN


# ------------------------------------------------------ step scalars on the device
@pytest.mark.parametrize("hp", [dict(), dict(lr=1e-3, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1,
                                          step=7, loss_scale=2.0**12, grad_predivide=3.0),
                                dict(lr=0.0, beta1=0.0, step=123456, loss_scale=0.5,
                                     max_grad_norm=0.0)])
def test_step_scalars_are_the_step_constants(hp):
    # Each field is the hyper-parameter expression evaluated in fp64 and
    # rounded once to fp32, as the kernels' launch arguments are.
    a = good_args(**hp)
    sc = Z.zero_step_scalars(a, peer_sumsq=2.5, peer_overflow=True)
    f = np.float32
    t = a.step
    assert sc.inv_scale == f(1.0 / (a.loss_scale * a.grad_predivide))
    assert sc.decay == f(1.0 - a.lr * a.weight_decay)
    assert (sc.beta1, sc.one_minus_beta1) == (f(a.beta1), f(1.0 - a.beta1))
    assert (sc.beta2, sc.one_minus_beta2) == (f(a.beta2), f(1.0 - a.beta2))
    assert sc.step_size == f(a.lr / (1.0 - a.beta1 ** t))
    assert sc.inv_sqrt_bc2 == f(1.0 / np.sqrt(1.0 - a.beta2 ** t))
    assert sc.eps == f(a.eps)
    assert (sc.max_grad_norm, sc.peer_sumsq, sc.peer_overflow) == (a.max_grad_norm, 2.5, 1)
    assert list(sc.reserved) == [0, 0]


def test_step_scalars_checks():
    with pytest.raises(Z.ZeroError):
        Z.zero_step_scalars(good_args(step=0))
    with pytest.raises(Z.ZeroError):
        Z.zero_step_scalars(good_args(), peer_sumsq=float("nan"))
    with pytest.raises(Z.ZeroError) as e:       # a misaligned device copy is refused by the step
        Z.zero_shard_step(good_args(scalars=FakeTensor(0x900008, 64)), stream=0)
    assert e.value.code == Z.ZERO_EALIGN and "scalars" in Z.zero_last_error()
    with pytest.raises(ValueError):             # and a short one by the binding
        good_args(scalars=FakeTensor(0x900000, 32)).c_args()
