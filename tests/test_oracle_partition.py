"""Pins for the oracle's partition and bucket plan (CPU only).

The partition is checked by brute force on small sizes and against the
memory figures the pages print (golden/page_figures.json).  The bucket plan
is checked by its defining properties.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "page_figures.json")))


def brute_partition(P, N, A):
    s = 0
    while N * s < P:
        s += A
    valid = [len([i for i in range(r * s, (r + 1) * s) if i < P]) for r in range(N)]
    return s, N * s, valid


@pytest.mark.parametrize("A", [1, 8, 128])
def test_partition_brute_force(A):
    for N in range(1, 17):
        for P in list(range(0, 300)) + [1023, 1024, 1025, 4095, 4096, 4097]:
            got = oracle.partition(P, N, A)
            assert got == brute_partition(P, N, A), (P, N, A)


def test_partition_tiles_and_counts():
    rng = np.random.default_rng(0)
    for _ in range(300):
        P = int(rng.integers(0, 10**7))
        N = int(rng.integers(1, 65))
        A = int(2 ** rng.integers(0, 9))
        s, padded, valid = oracle.partition(P, N, A)
        assert s % A == 0 and padded == N * s and padded >= P
        assert s == 0 or N * (s - A) < P          # minimal
        assert sum(valid) == P
        # ranks are filled in order: full shards, one partial, then empty
        full = P // s if s else 0
        assert all(v == s for v in valid[:full])
        assert all(v == 0 for v in valid[full + 1:])


@pytest.mark.parametrize("args", [(-1, 4, 8), (10, 0, 8), (10, 4, 0)])
def test_partition_rejects_invalid(args):
    with pytest.raises(ValueError):
        oracle.partition(*args)


def test_workload_partitions():
    # The five workloads' shard sizes (alignment 128).
    assert oracle.partition(787_968, 4, 128)[0] == 196_992
    assert oracle.partition(67_125_248, 8, 128)[0] == 8_390_656
    s, padded, valid = oracle.partition(13_000_000_000, 8, 128)
    assert s == 1_625_000_064 and padded == 13_000_000_512
    assert valid[0] == s and valid[7] == s - 512
    s, padded, valid = oracle.partition(50_000_000, 4, 128)
    assert s == 12_500_096 and valid[3] == s - 384


# ----------------------------------------------- memory figures of the pages
def model_state_bytes(P, N, stage, A=1):
    """Per-rank bytes of model state under mixed-precision Adam: 2-byte
    working params and grads, 12 bytes of fp32 master, m and v per param;
    each stage shards one more of them (the shard size from the oracle)."""
    s = oracle.partition(P, N, A)[0]
    if stage == 0:
        return 16 * P
    if stage == 1:
        return 2 * P + 2 * P + 12 * s
    if stage == 2:
        return 2 * P + 2 * s + 12 * s
    return 16 * s


def test_zero1_saves_87_5_percent_at_8():
    fig = GOLDEN["optimizer_state_saved_at_8_gpus"]
    for P in (8 * 128 * 1000, 67_125_248, 13_000_000_000 - 512):
        s = oracle.partition(P, 8, 128)[0]
        saved = 1.0 - (12 * s) / (12 * P)
        assert saved == pytest.approx(fig["value"], abs=1e-12)
    # Not divisible: padding makes the saving slightly smaller, never larger.
    s = oracle.partition(1001, 8, 128)[0]
    assert 1.0 - s / 1001 < 0.875


def test_zero3_is_one_over_n():
    fig = GOLDEN["zero3_320GB_on_4_cards"]
    P = int(fig["model_bytes"] / 16)       # 16 bytes of model state per param
    per_card = model_state_bytes(P, fig["n_gpus"], 3)
    assert per_card == pytest.approx(fig["per_card_bytes"], rel=1e-6)
    for N in (2, 8, 64):
        assert model_state_bytes(N * 128 * 977, N, 3, 128) * N == \
            model_state_bytes(N * 128 * 977, N, 0)


def test_stage_savings_limits():
    fig = GOLDEN["stage_savings"]
    P = 2**40
    r1 = [model_state_bytes(P, N, 0) / model_state_bytes(P, N, 1) for N in (8, 64, 4096)]
    r2 = [model_state_bytes(P, N, 0) / model_state_bytes(P, N, 2) for N in (8, 64, 4096)]
    assert r1 == sorted(r1) and r2 == sorted(r2)
    assert r1[-1] == pytest.approx(fig["zero1"], rel=1e-2) and r1[-1] < fig["zero1"]
    assert r2[-1] == pytest.approx(fig["zero2"], rel=1e-2) and r2[-1] < fig["zero2"]
    r3 = model_state_bytes(P, 64, 0) / model_state_bytes(P, 64, 3)
    assert 10 <= r3 <= 99                              # "tens of times"


def test_d_model_4096_layer_figures():
    fig = GOLDEN["d_model_4096_layer"]
    d = fig["d_model"]
    weights = 4 * d * d                                # q, k, v, out projections
    assert weights == pytest.approx(fig["params_approx"], rel=0.05)
    assert 4 * weights == pytest.approx(fig["fp32_bytes_approx"], rel=0.002)
    assert 4 * (4 * weights) > fig["total_bytes_at_least"]
    # With biases the flat count is the encoder-layer workload's P.
    assert weights + 4 * d == 67_125_248


# ------------------------------------------------------------ bucket plan
def brute_buckets(sizes, cap):
    buckets, cur, fill = [], [], 0
    for t, n in enumerate(sizes):
        if cur and fill + n > cap:
            buckets.append(cur)
            cur, fill = [], 0
        cur.append(t)
        fill += n
    if cur:
        buckets.append(cur)
    return buckets


def test_bucket_plan_properties():
    rng = np.random.default_rng(1)
    for trial in range(200):
        T = int(rng.integers(0, 60))
        sizes = [int(x) for x in rng.integers(0, 5000, size=T)]
        cap = int(rng.integers(1, 8000))
        off, bof, nb = oracle.bucket_plan(sizes, cap)
        assert list(off) == [sum(sizes[:t]) for t in range(T)]
        groups = brute_buckets(sizes, cap)
        assert nb == len(groups)
        for b, members in enumerate(groups):
            assert all(bof[t] == b for t in members)
        for b in range(nb):
            members = [t for t in range(T) if bof[t] == b]
            total = sum(sizes[t] for t in members)
            assert total <= cap or len([t for t in members if sizes[t] > 0]) == 1
            assert members == list(range(members[0], members[-1] + 1))


def test_bucket_plan_hand_example():
    # 2e8 buckets over sizes in units of 1e7.
    sizes = [int(x * 1e7) for x in (5, 9, 6, 25, 1, 19, 1)]
    off, bof, nb = oracle.bucket_plan(sizes, int(2e8))
    assert list(bof) == [0, 0, 0, 1, 2, 2, 3]
    assert nb == 4
    with pytest.raises(ValueError):
        oracle.bucket_plan([1, 2], 0)


def test_flatten_hand_example():
    # three tensors of 2, 0 and 3 codes, padded to 8: end to end, then zeros
    t = [np.array([7, 8], np.uint16), np.zeros(0, np.uint16), np.array([1, 2, 3], np.uint16)]
    assert oracle.flatten(t, 4, 8).tolist() == [7, 8, 1, 2, 3, 0, 0, 0]
    assert oracle.flatten([], 4, 3).tolist() == [0, 0, 0]
    with pytest.raises(ValueError):
        oracle.flatten(t, 4, 4)


def test_flatten_places_every_tensor_at_its_running_offset():
    # each tensor's codes sit at the sum of the sizes before it, whatever the
    # bucket size; everything after the last tensor is zero
    rng = np.random.default_rng(4)
    for trial in range(50):
        sizes = [int(x) for x in rng.integers(0, 300, size=int(rng.integers(1, 40)))]
        t = [rng.integers(1, 65536, n).astype(np.uint16) for n in sizes]
        padded = sum(sizes) + int(rng.integers(0, 50))
        flats = [oracle.flatten(t, cap, padded) for cap in (1, 97, 10**6)]
        for f in flats[1:]:
            assert np.array_equal(f, flats[0])
        pos = 0
        for x in t:
            assert np.array_equal(flats[0][pos:pos + x.size], x)
            pos += x.size
        assert not flats[0][pos:].any()
