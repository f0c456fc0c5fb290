"""Seeded random sweeps of the entry points that only move 16-bit or fp32
values, compared bit for bit with the oracle's plain definitions.

- Flatten: random tensor counts and size mixes (empty, a few elements,
  log-uniform up to 2e6), sources at odd element offsets, random bucket
  sizes, flattened at once or bucket by bucket, against `oracle.flatten`;
  and random slot tables with gaps and empty slots, against the
  definition (slot data, zeros in every gap and up to flat_numel, nothing
  touched before the first slot or past flat_numel).
- Re-partition: random flat sizes and random old and new world sizes and
  alignments, all three state fields, against `oracle.repartition`.
- ZeRO-3 gather: random partitions and random ranges, against
  `oracle.gather`.

The draws are fixed by their seeds; each case prints its draw first.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
import zero_sharded_optimizer_step_amd as Z
from zero_sharded_optimizer_step_amd import workloads as W
from zero_sharded_optimizer_step_amd.world import SimulatedWorld

pytestmark = pytest.mark.gpu

CANARY = 0x1357


def say(msg):
    print(msg, flush=True)


def _codes(rng, n):
    return rng.integers(0, 65536, n, dtype=np.uint64).astype(np.uint16)


def _sizes(rng, k):
    out = []
    for _ in range(k):
        u = rng.random()
        if u < 0.05:
            out.append(0)
        elif u < 0.35:
            out.append(int(rng.integers(1, 17)))
        else:
            out.append(int(math.exp(rng.uniform(math.log(17), math.log(2e6)))))
    return out


def _sources(rng, sizes, dtype):
    """Device tensors holding random codes, each a view at an element
    offset 0-7 of its own allocation."""
    srcs = []
    for n in sizes:
        off = int(rng.integers(0, 8))
        base = torch.from_numpy(_codes(rng, n + off).view(np.int16)).cuda()
        srcs.append(base[off:off + n].view(dtype))
    return srcs


@pytest.mark.parametrize("case", range(24))
def test_random_flatten_matches_oracle(case):
    rng = np.random.default_rng(1000 + case)
    sizes = _sizes(rng, int(rng.integers(0, 400)))
    dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float16
    bucket = int(rng.choice([1, 1000, 100_000, 1 << 20, 1 << 24]))
    per_bucket = bool(rng.random() < 0.5)
    total = sum(sizes)
    flat_numel = total + int(rng.integers(0, 300))
    say("flatten case %d: %d tensors, %d elements, bucket %d, %s, flat %d, %s"
        % (case, len(sizes), total, bucket, "per bucket" if per_bucket else "at once", flat_numel,
           str(dtype)[6:]))
    srcs = _sources(rng, sizes, dtype)
    slots, buckets = Z.zero_bucket_plan(sizes, bucket)
    flat = torch.full((flat_numel + 64,), CANARY, dtype=torch.int16, device="cuda")
    if per_bucket and buckets:
        for j, b in enumerate(buckets):
            end = flat_numel if j == len(buckets) - 1 else b.end
            Z.zero_bucket_flatten(slots[b.first_tensor:b.first_tensor + b.n_tensors],
                                  srcs[b.first_tensor:b.first_tensor + b.n_tensors], dtype,
                                  flat.view(dtype), end)
    else:
        Z.zero_bucket_flatten(slots, srcs, dtype, flat.view(dtype), flat_numel)
    got = parity.u16(flat)
    ref = oracle.flatten([parity.u16(s) for s in srcs], bucket, flat_numel)
    parity.assert_bitwise("flat", got[:flat_numel], ref)
    assert (got[flat_numel:] == CANARY).all(), "wrote past flat_numel"


@pytest.mark.parametrize("case", range(16))
def test_random_gapped_slot_tables(case):
    rng = np.random.default_rng(2000 + case)
    sizes = _sizes(rng, int(rng.integers(1, 300)))
    dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float16
    offsets = []
    at = int(rng.integers(0, 50))
    for n in sizes:
        offsets.append(at)
        at += n + (int(rng.integers(0, 40)) if rng.random() < 0.5 else 0)
    flat_numel = at + int(rng.integers(0, 100))
    say("gapped flatten case %d: %d slots, first at %d, flat %d" % (case, len(sizes), offsets[0],
                                                                     flat_numel))
    srcs = _sources(rng, sizes, dtype)
    slots = [Z.zero_tensor_slot_t(o, n, 0, 0) for o, n in zip(offsets, sizes)]
    flat = torch.full((flat_numel + 64,), CANARY, dtype=torch.int16, device="cuda")
    Z.zero_bucket_flatten(slots, srcs, dtype, flat.view(dtype), flat_numel)
    # the definition: [first offset, flat_numel) holds the slots' data and
    # zeros elsewhere; the rest keeps the canary
    ref = np.full(flat_numel + 64, CANARY, np.uint16)
    ref[offsets[0]:flat_numel] = 0
    for o, n, s in zip(offsets, sizes, srcs):
        ref[o:o + n] = parity.u16(s)
    parity.assert_bitwise("flat", parity.u16(flat), ref)


def _partition(rng):
    return int(rng.integers(1, 10)), int(rng.choice([1, 8, 64, 128, 256]))


@pytest.mark.parametrize("case", range(16))
def test_random_repartition_matches_oracle(case):
    rng = np.random.default_rng(3000 + case)
    P = int(math.exp(rng.uniform(0.0, math.log(3e6))))
    (N, A), (M, B) = _partition(rng), _partition(rng)
    say("repartition case %d: P %d, %d ranks (A %d) -> %d ranks (A %d)" % (case, P, N, A, M, B))
    src = SimulatedWorld(P, N, n_replicas=1, alignment=A, grad_dtype=torch.bfloat16)
    dst = SimulatedWorld(P, M, n_replicas=1, alignment=B, grad_dtype=torch.bfloat16)
    for k in range(N):
        for f, t in enumerate(src.state(k)):
            W.flat_normal(t, k * src.s, P, 1.0, ("random-repart", case, f))
    for k in range(M):
        for t in dst.state(k):
            t.fill_(7.0)
    dst.repartition_from(src)
    for f in range(3):
        ref = oracle.repartition([parity.f32(src.state(k)[f]) for k in range(N)], P, N, A, M, B)
        for k in range(M):
            parity.assert_bitwise("field %d rank %d" % (f, k), parity.f32(dst.state(k)[f]), ref[k])


@pytest.mark.parametrize("case", range(16))
def test_random_gather_ranges_match_oracle(case):
    rng = np.random.default_rng(4000 + case)
    P = int(math.exp(rng.uniform(0.0, math.log(3e6))))
    N, A = int(rng.integers(1, 10)), int(rng.choice([1, 8, 16, 128, 256]))
    part = Z.zero_partition(P, N, A)
    s = part.shard_numel
    dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float16
    say("gather case %d: P %d, %d ranks, A %d, %s" % (case, P, N, A, str(dtype)[6:]))
    shards = [torch.from_numpy(_codes(rng, s).view(np.int16)).cuda() for _ in range(N)]
    host = [parity.u16(x) for x in shards]
    ranges = [tuple(sorted(int(x) for x in rng.integers(0, P + 1, 2))) for _ in range(12)]
    # ranges that start or end at shard edges
    for _ in range(6):
        e = min(P, s * int(rng.integers(0, N + 1)))
        d = int(rng.integers(0, 9))
        ranges.append((max(0, e - d), min(P, e + int(rng.integers(0, 9)))))
    for lo, hi in ranges:
        dst = torch.full((hi - lo + 16,), CANARY, dtype=torch.int16, device="cuda")
        Z.zero_gather_params(part, [x.view(dtype) for x in shards], dtype, lo, hi, dst.view(dtype))
        got = parity.u16(dst)
        parity.assert_bitwise("gather [%d, %d)" % (lo, hi), got[:hi - lo],
                              oracle.gather(host, P, N, A, lo, hi))
        assert (got[hi - lo:] == CANARY).all(), "wrote past the range"
