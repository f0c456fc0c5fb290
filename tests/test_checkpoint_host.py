"""CPU tests of the sharded checkpoint: the oracle's re-partition, the
library's header checks, and the checkpoint files (host tensors only)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_step_amd as Z
from zero_sharded_optimizer_step_amd import checkpoint as C


# ------------------------------------------------------- oracle re-partition
def test_repartition_hand_example():
    # 10 params over 3 ranks at alignment 2: shards of 4 -> [0..4) [4..8) [8..10)+2 pad;
    # over 2 ranks at alignment 1: shards of 5 -> [0..5) [5..10).
    old = [np.array([0, 1, 2, 3], np.float32), np.array([4, 5, 6, 7], np.float32),
           np.array([8, 9, -1, -1], np.float32)]
    new = oracle.repartition(old, 10, 3, 2, 2, 1)
    assert [x.tolist() for x in new] == [[0, 1, 2, 3, 4], [5, 6, 7, 8, 9]]
    back = oracle.repartition(new, 10, 2, 1, 3, 2)
    assert [x.tolist() for x in back] == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 0, 0]]


def test_repartition_round_trip_and_empty_ranks():
    rng = np.random.default_rng(0)
    for P, N, A, M, B in ((1000, 4, 8, 3, 128), (5, 4, 8, 7, 1), (4097, 1, 1, 16, 8)):
        s, _, valid = oracle.partition(P, N, A)
        old = [np.where(np.arange(s) < valid[r], rng.standard_normal(s), 0).astype(np.float32)
               for r in range(N)]
        new = oracle.repartition(old, P, N, A, M, B)
        assert len(new) == M and all(x.size == oracle.partition(P, M, B)[0] for x in new)
        back = oracle.repartition(new, P, M, B, N, A)
        for x, y in zip(old, back):
            assert np.array_equal(x, y)


# -------------------------------------------------------------- headers
def make_header(P=1000, N=4, A=8, rank=3, step=7, scaler=True):
    part = Z.zero_partition(P, N, A)
    sc = Z.zero_loss_scaler_init(12, 50, 2, 1.0) if scaler else None
    return part, Z.zero_ckpt_header_make(part, rank, Z.ZERO_FP16, step, sc)


def test_header_round_trip():
    part, h = make_header()
    assert ctypes.sizeof(h) == 128 and h.magic == Z.ZERO_CKPT_MAGIC
    assert h.valid_numel == Z.zero_partition_valid_numel(part, 3)
    assert h.payload_bytes == 12 * h.valid_numel and h.scaler.scale == 4096.0
    q = Z.zero_ckpt_header_check(h, 128 + h.payload_bytes)
    assert (q.numel, q.shard_numel, q.world_size, q.alignment) == (1000, 256, 4, 8)


@pytest.mark.parametrize("field,value,code", [
    ("magic", 0x12345678, Z.ZERO_EINVAL), ("version", 2, Z.ZERO_EINVAL),
    ("shard_numel", 264, Z.ZERO_EINVAL), ("valid_numel", 5, Z.ZERO_EINVAL),
    ("rank", 4, Z.ZERO_EINVAL), ("param_dtype", 9, Z.ZERO_EINVAL),
    ("payload_bytes", 12, Z.ZERO_EINVAL), ("step", -1, Z.ZERO_EINVAL),
    ("alignment", 3, Z.ZERO_EINVAL), ("has_scaler", 2, Z.ZERO_EINVAL)])
def test_header_check_rejects(field, value, code):
    _, h = make_header()
    setattr(h, field, value)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_ckpt_header_check(h, 1 << 20)
    assert e.value.code == code


def test_header_check_rejects_short_file_and_bad_scaler():
    _, h = make_header()
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_ckpt_header_check(h, 128 + h.payload_bytes - 1)
    assert e.value.code == Z.ZERO_ESIZE
    h.scaler.window = 0
    with pytest.raises(Z.ZeroError):
        Z.zero_ckpt_header_check(h, 1 << 20)


# ------------------------------------------------------ files, host tensors
def world_state(rng, P, N, A):
    s, _, valid = oracle.partition(P, N, A)
    return [[torch.from_numpy(np.where(np.arange(s) < valid[r], rng.standard_normal(s), 0)
                              .astype(np.float32)) for _ in range(3)] for r in range(N)]


@pytest.mark.parametrize("old,new", [((1000, 4, 8), (3, 128)), ((50_001, 8, 128), (3, 8)),
                                     ((77, 4, 8), (4, 8)), ((5, 4, 8), (2, 1))])
def test_files_resume_under_any_partition(tmp_path, old, new, monkeypatch):
    monkeypatch.setattr(C, "STAGING_ELEMS", 64)         # many staging round trips
    rng = np.random.default_rng(1)
    P, N, A = old
    M, B = new
    part = Z.zero_partition(P, N, A)
    states = world_state(rng, P, N, A)
    sc = Z.zero_loss_scaler_init(10, 20, 2, 1.0)
    Z.zero_loss_scaler_update(sc, True)
    C.save_world(str(tmp_path), part, states, torch.float16, 11, sc)
    assert sorted(os.listdir(tmp_path)) == ["zero_rank%05d.zsc" % r for r in range(N)]
    new_part = Z.zero_partition(P, M, B)
    got = []
    for r in range(M):
        st = [torch.full((new_part.shard_numel,), 5.0) for _ in range(3)]
        step, scaler = C.load_rank_resharded(str(tmp_path), new_part, r, st)
        assert step == 11 and scaler.hysteresis_left == 1 and scaler.scale == 1024.0
        got.append(st)
    for field in range(3):
        ref = oracle.repartition([states[r][field].numpy() for r in range(N)], P, N, A, M, B)
        for r in range(M):
            assert np.array_equal(got[r][field].numpy(), ref[r]), (field, r)


def test_files_from_different_runs_are_rejected(tmp_path):
    rng = np.random.default_rng(2)
    part = Z.zero_partition(1000, 2, 8)
    states = world_state(rng, 1000, 2, 8)
    C.save_world(str(tmp_path), part, states, torch.bfloat16, 3)
    C.save_rank(C.rank_path(str(tmp_path), 1), part, 1, states[1], torch.bfloat16, 4)
    st = [torch.zeros(part.shard_numel) for _ in range(3)]
    with pytest.raises(ValueError):
        C.load_rank_resharded(str(tmp_path), part, 0, st)
    with open(C.rank_path(str(tmp_path), 0), "r+b") as f:       # truncate rank 0
        f.truncate(200)
    with pytest.raises(Z.ZeroError):
        C.read_header(C.rank_path(str(tmp_path), 0))


# ------------------------------------------------------------ ZeRO-3 gather
def test_oracle_gather_hand_example():
    shards = [np.array([0, 1, 2, 3], np.uint16), np.array([4, 5, 6, 7], np.uint16),
              np.array([8, 9, 0xAAAA, 0xAAAA], np.uint16)]     # 10 params, N=3, A=2
    assert oracle.gather(shards, 10, 3, 2, 3, 9).tolist() == [3, 4, 5, 6, 7, 8]
    assert oracle.gather(shards, 10, 3, 2, 0, 10).tolist() == list(range(10))
    assert oracle.gather(shards, 10, 3, 2, 5, 5).size == 0


# ----------------------------------------------------- the library's read plan
def _apply_plan(old_slices, old_part, new_part, new_rank):
    """New rank new_rank's slice, built only from the library's read plan."""
    x = np.zeros(new_part.shard_numel, np.float32)
    covered = np.zeros(new_part.shard_numel, np.int32)
    pieces = Z.zero_repartition_plan(old_part, new_part, new_rank)
    n_new = Z.zero_partition_valid_numel(new_part, new_rank)
    last_new, last_old = -1, -1
    for p in pieces:
        assert p.count > 0 and p.reserved == 0
        assert p.new_offset > last_new and p.old_rank > last_old     # ascending
        last_new, last_old = p.new_offset, p.old_rank
        n_k = Z.zero_partition_valid_numel(old_part, p.old_rank)
        assert 0 <= p.old_offset and p.old_offset + p.count <= n_k   # inside real elements
        x[p.new_offset:p.new_offset + p.count] = \
            old_slices[p.old_rank][p.old_offset:p.old_offset + p.count]
        covered[p.new_offset:p.new_offset + p.count] += 1
    assert np.all(covered[:n_new] == 1) and np.all(covered[n_new:] == 0)
    assert len(pieces) <= old_part.world_size
    return x


def test_repartition_plan_matches_oracle_by_brute_force():
    # Every (numel, old world, old alignment, new world, new alignment) of a
    # small grid: the slices the plan builds equal the oracle's re-cut, and
    # each real element is read exactly once from inside an old rank's
    # real elements.
    cases = 0
    for P in (0, 1, 5, 7, 8, 63, 64, 65, 200, 257, 1000):
        for N, A in ((1, 1), (2, 8), (3, 2), (4, 8), (7, 1), (8, 128)):
            s_old, _, valid_old = oracle.partition(P, N, A)
            old = [np.where(np.arange(s_old) < valid_old[r],
                            r * s_old + np.arange(s_old) + 1, 0).astype(np.float32)
                   for r in range(N)]
            old_part = Z.zero_partition(P, N, A)
            for M, B in ((1, 1), (2, 1), (3, 8), (5, 2), (8, 8), (16, 1)):
                new_part = Z.zero_partition(P, M, B)
                ref = oracle.repartition(old, P, N, A, M, B)
                for j in range(M):
                    got = _apply_plan(old, old_part, new_part, j)
                    assert np.array_equal(got, ref[j]), (P, N, A, M, B, j)
                    cases += 1
    assert cases > 1000


def test_repartition_plan_capacity_and_errors():
    L = Z.lib()
    old = Z.zero_partition(1000, 8, 8)          # shards of 128
    new = Z.zero_partition(1000, 2, 8)          # shards of 504: rank 0 reads old ranks 0..3
    n = Z._abi.i32(-1)
    pieces = (Z.zero_repartition_piece_t * 8)()
    assert L.zero_repartition_plan(ctypes.byref(old), ctypes.byref(new), 0, pieces, 2,
                                   ctypes.byref(n)) == Z.ZERO_ESIZE and n.value == 4
    assert L.zero_repartition_plan(ctypes.byref(old), ctypes.byref(new), 0, pieces, 4,
                                   ctypes.byref(n)) == Z.ZERO_OK and n.value == 4
    assert [(p.old_rank, p.old_offset, p.new_offset, p.count) for p in pieces[:4]] == \
        [(0, 0, 0, 128), (1, 0, 128, 128), (2, 0, 256, 128), (3, 0, 384, 120)]
    assert L.zero_repartition_plan(ctypes.byref(old), ctypes.byref(new), 2, pieces, 8,
                                   ctypes.byref(n)) == Z.ZERO_EINVAL          # rank out of range
    other = Z.zero_partition(999, 2, 8)
    assert L.zero_repartition_plan(ctypes.byref(old), ctypes.byref(other), 0, pieces, 8,
                                   ctypes.byref(n)) == Z.ZERO_EINVAL          # numel differs
    bad = Z.zero_partition(1000, 2, 8)
    bad.shard_numel = 512                                                    # not minimal
    bad.padded_numel = 1024
    assert L.zero_repartition_plan(ctypes.byref(old), ctypes.byref(bad), 0, pieces, 8,
                                   ctypes.byref(n)) == Z.ZERO_EINVAL
    assert "zero_partition gives" in Z.zero_last_error()
    assert L.zero_repartition_plan(ctypes.byref(old), ctypes.byref(new), 0, None, 8,
                                   ctypes.byref(n)) == Z.ZERO_EINVAL
    # a rank with no real elements reads nothing
    tail = Z.zero_partition(10, 8, 8)            # shards of 8: ranks 2..7 are empty
    assert Z.zero_repartition_plan(Z.zero_partition(10, 1, 1), tail, 5) == []
