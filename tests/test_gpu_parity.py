"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Small and mid sizes that the oracle finishes in seconds but that span many
blocks of the kernels' grid and end in ragged tails; empty ranks, poisoned
gradients, both formats, clipping on and off, several steps.  Each case
prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import zero_sharded_optimizer_step_amd as Z
from zero_sharded_optimizer_step_amd import workloads as W
from zero_sharded_optimizer_step_amd.world import Hyper, SimulatedWorld

pytestmark = pytest.mark.gpu

BF16, FP16 = torch.bfloat16, torch.float16


def say(msg):
    print(msg, flush=True)


CASES = [
    # (numel, world, alignment, dtype, sigma, loss_scale, clip, steps)
    (5, 4, 8, BF16, 1e-2, 1.0, 1.0, 2),             # three empty ranks, tail only
    (1000, 3, 8, BF16, 1e-2, 1.0, 1.0, 3),
    (4097, 4, 8, FP16, 1e-3, 2.0**16, 1.0, 3),
    (100_003, 8, 128, BF16, 1e-3, 1.0, 1.0, 3),
    (100_003, 8, 128, BF16, 1e-3, 1.0, 0.0, 3),     # clipping off
    (1_048_583, 4, 128, FP16, 1e-3, 2.0**12, 1e9, 2),  # clip threshold never reached
    (3_000_001, 2, 128, BF16, 3e-2, 1.0, 1.0, 2),   # 1.5M-element shards, 2 ranks
]


@pytest.mark.parametrize("case", CASES, ids=[f"P{c[0]}-N{c[1]}-A{c[2]}-{str(c[3])[6:]}-clip{c[6]}"
                                             for c in CASES])
def test_world_matches_oracle(case):
    numel, world, align, dt, sigma, scale, clip, steps = case
    say("case %s" % (case,))
    spec = parity.Spec(numel=numel, world_size=world, alignment=align, grad_dtype=dt,
                       grad_sigma=sigma, steps=steps, name="small-%d-%d" % (numel, world),
                       hp=Hyper(loss_scale=scale, max_grad_norm=clip))
    rep = parity.run(spec)
    say("norm rel err %.2e, bitwise state fraction %.6f, cast max ulp %d"
        % (rep.norm_rel_err, rep.state_bitwise, rep.cast_max_ulp))


PREDIVIDE_CASES = [
    # (numel, world, alignment, dtype, sigma, loss_scale, predivide, clip, steps):
    # DDP-style averaging over a world that is not a power of two, and a
    # static loss scale that is not one, so the unscale multiplier
    # fp32(1/(S·D)) is rounded on both sides
    (100_003, 3, 128, BF16, 1e-3, 1.0, 3.0, 1.0, 2),
    (300_007, 6, 8, FP16, 1e-3, 1000.0, 6.0, 1.0, 2),
    (65_537, 5, 8, FP16, 1e-2, 2.0**12, 0.7, 1e9, 2),
]


@pytest.mark.parametrize("case", PREDIVIDE_CASES,
                         ids=[f"P{c[0]}-N{c[1]}-S{c[5]:g}-D{c[6]:g}" for c in PREDIVIDE_CASES])
def test_world_with_predivide_matches_oracle(case):
    numel, world, align, dt, sigma, scale, pre, clip, steps = case
    say("predivide case %s" % (case,))
    spec = parity.Spec(numel=numel, world_size=world, alignment=align, grad_dtype=dt,
                       grad_sigma=sigma, steps=steps, name="predivide-%d-%d" % (numel, world),
                       hp=Hyper(loss_scale=scale, grad_predivide=pre, max_grad_norm=clip))
    rep = parity.run(spec)
    say("norm rel err %.2e, bitwise state fraction %.6f, cast max ulp %d"
        % (rep.norm_rel_err, rep.state_bitwise, rep.cast_max_ulp))


HYPER_CASES = [
    # AdamW settings other than the workloads' defaults, over enough steps
    # for the bias corrections to move: a common large-model setting, no
    # first moment and no decay, and a large step with a strong decay
    dict(lr=1e-3, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1),
    dict(lr=3e-4, beta1=0.0, beta2=0.99, eps=1e-8, weight_decay=0.0),
    dict(lr=0.1, beta1=0.5, beta2=0.5, eps=1e-3, weight_decay=1.0),
]


@pytest.mark.parametrize("hyper", HYPER_CASES,
                         ids=["lr%g-b%g-%g-eps%g-wd%g" % tuple(h.values()) for h in HYPER_CASES])
def test_hyper_parameters_match_oracle(hyper):
    say("hyper-parameters %s" % hyper)
    spec = parity.Spec(numel=200_003, world_size=4, alignment=128, grad_dtype=BF16,
                       grad_sigma=1e-2, steps=5, name="hyper",
                       hp=Hyper(max_grad_norm=1.0, **hyper))
    rep = parity.run(spec)
    say("norm rel err %.2e, bitwise state fraction %.6f, cast max ulp %d"
        % (rep.norm_rel_err, rep.state_bitwise, rep.cast_max_ulp))


@pytest.mark.parametrize("gdt,pdt,scale", [(BF16, FP16, 1.0), (FP16, BF16, 2.0**14)],
                         ids=["bf16-grads-fp16-params", "fp16-grads-bf16-params"])
def test_crossed_gradient_and_parameter_formats(gdt, pdt, scale):
    """The decode follows grad_dtype and the cast follows param_dtype, each
    on its own."""
    say("crossed formats %s -> %s" % (gdt, pdt))
    spec = parity.Spec(numel=150_001, world_size=4, alignment=8, grad_dtype=gdt,
                       param_dtype=pdt, grad_sigma=1e-3, steps=2, name="crossed",
                       hp=Hyper(loss_scale=scale))
    rep = parity.run(spec)
    say("norm rel err %.2e, bitwise state fraction %.6f, cast max ulp %d"
        % (rep.norm_rel_err, rep.state_bitwise, rep.cast_max_ulp))


def test_tiny_workload_matches_oracle():
    w = W.TINY
    say("tiny workload")
    spec = parity.Spec(numel=w.numel, world_size=w.world_size, grad_dtype=w.grad_dtype,
                       grad_sigma=w.grad_sigma, hp=Hyper(loss_scale=w.loss_scale), steps=2,
                       name="tiny")
    rep = parity.run(spec)
    assert rep.norms[0] > 1.0          # the clip is active on this workload


def test_more_replicas_than_ranks_and_generic_replica_count():
    # 11 replicas (the kernel's generic replica loop) over 3 ranks.
    say("11 replicas, 3 ranks")
    spec = parity.Spec(numel=50_001, world_size=3, n_replicas=11, alignment=8, grad_dtype=BF16,
                       grad_sigma=1e-2, steps=2, name="generic-replicas")
    parity.run(spec)


@pytest.mark.parametrize("nrep,dt", [(1, BF16), (5, FP16), (6, BF16), (7, FP16), (64, BF16)])
def test_each_replica_count(nrep, dt):
    # The reduce is compiled for 1..8 replicas and has a generic loop above;
    # these cover the counts no other case reaches, up to the maximum.
    say("%d replicas, 3 ranks, %s" % (nrep, str(dt)[6:]))
    scale = 2.0**12 if dt == FP16 else 1.0
    spec = parity.Spec(numel=30_011, world_size=3, n_replicas=nrep, alignment=8, grad_dtype=dt,
                       grad_sigma=1e-3, steps=2, name="replicas-%d" % nrep,
                       hp=Hyper(loss_scale=scale))
    parity.run(spec)


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("where", ["first", "last_rank_tail", "middle"])
def test_poisoned_step_is_skipped_everywhere(kind, where):
    numel, world = 20_011, 4
    say("poison kind %d at %s" % (kind, where))
    s = Z.zero_partition(numel, world, 8).shard_numel
    idx = {"first": 0, "last_rank_tail": numel - 1, "middle": s + s // 2}[where]
    sched = [None, W.Poison(1, 2, idx, kind), None]
    spec = parity.Spec(numel=numel, world_size=world, alignment=8, grad_dtype=FP16,
                       grad_sigma=1e-3, steps=3, poison=sched, dynamic_scale=True,
                       scaler_args=(10, 2, 1, 1.0), name="poison")
    rep = parity.run(spec)
    assert rep.skipped == 1


@pytest.mark.parametrize("dt", [FP16, BF16])
@pytest.mark.parametrize("kind", [0, 1, 2])
def test_nonfinite_code_in_padding_is_no_overflow(kind, dt):
    # Reading: the overflow flag covers the ranks' real elements.  A replica
    # whose padding (past the last real element, on the last rank) holds
    # +inf, -inf or nan still takes the step, on both sides, and the state
    # matches the oracle.
    numel, world = 20_011, 4
    part = Z.zero_partition(numel, world, 128)
    assert part.padded_numel - numel == 469
    idx = numel + 200                                   # inside rank 3's padding
    say("non-finite code %d in the padding at %d, %s" % (kind, idx, str(dt)[6:]))
    sched = [W.Poison(0, 1, idx, kind), W.Poison(1, 3, part.padded_numel - 1, kind)]
    scale = 2.0**12 if dt == FP16 else 1.0
    spec = parity.Spec(numel=numel, world_size=world, alignment=128, grad_dtype=dt,
                       grad_sigma=1e-3, steps=2, poison=sched, name="padding-poison",
                       hp=Hyper(loss_scale=scale))
    rep = parity.run(spec)
    assert rep.skipped == 0 and rep.steps == 2


def test_dynamic_scale_trajectory_small():
    # The scaled workload's schedule, at a size the oracle runs every step of.
    steps = 200
    numel, world = 65_543, 4
    sched = W.poison_schedule(steps, world, numel, p=0.05, seed=0)
    say("scaler trajectory, %d poisoned steps" % sum(x is not None for x in sched))
    spec = parity.Spec(numel=numel, world_size=world, grad_dtype=FP16, grad_sigma=1e-3,
                       steps=steps, poison=sched, dynamic_scale=True,
                       scaler_args=(16, 100, 2, 1.0), name="scaler-small")
    rep = parity.run(spec, check_every_step=False)
    assert rep.skipped == sum(x is not None for x in sched)
    assert min(rep.scales) < 2.0**16          # overflows halved the scale


def test_dynamic_scale_grows_and_shrinks():
    # A short window so the scale also grows; same poison rate.
    steps = 120
    numel, world = 10_007, 2
    sched = W.poison_schedule(steps, world, numel, p=0.05, seed=1)
    say("scaler window 5, %d poisoned steps" % sum(x is not None for x in sched))
    spec = parity.Spec(numel=numel, world_size=world, alignment=8, grad_dtype=FP16,
                       grad_sigma=1e-3, steps=steps, poison=sched, dynamic_scale=True,
                       scaler_args=(10, 5, 2, 1.0), name="scaler-grow")
    rep = parity.run(spec, check_every_step=False)
    ups = sum(b > a for a, b in zip(rep.scales, rep.scales[1:]))
    downs = sum(b < a for a, b in zip(rep.scales, rep.scales[1:]))
    assert ups > 0 and downs > 0


def _fill(world, seed):
    for i in range(world.n_replicas):
        W.flat_normal(world.grads[i], world.lo, world.numel, 1e-2, ("det", seed, i))
    for k, r in enumerate(world.ranks):
        W.flat_normal(world.master[k], r * world.s, world.numel, 0.02, ("detm", seed))


def test_run_to_run_bitwise_determinism():
    say("determinism")
    outs = []
    for _ in range(2):
        world = SimulatedWorld(777_777, 8, alignment=128, grad_dtype=BF16)
        _fill(world, 1)
        for t in (1, 2):
            world.step(Hyper(), t)
        res = world.result()
        outs.append((res.sumsq, res.norm, res.coef,
                     [parity.f32(m) for m in world.master + world.exp_avg + world.exp_avg_sq],
                     parity.u16(world.full_params)))
    a, b = outs
    assert a[:3] == b[:3]
    for x, y in zip(a[3], b[3]):
        parity.assert_bitwise("rerun", x, y)
    parity.assert_bitwise("rerun params", a[4], b[4])


def test_concurrent_threads_and_streams_equal_one_stream():
    # The library keeps no state between calls: four host threads, each
    # queueing one rank's reduce and apply on its own stream at the same
    # time, give the bits of the same step queued on one stream.
    import threading
    say("4 ranks on 4 threads and 4 streams")
    worlds = [SimulatedWorld(2_000_003, 4, alignment=128, grad_dtype=BF16) for _ in range(2)]
    for w in worlds:
        _fill(w, 3)
    hp = Hyper()
    worlds[0].step(hp, 1)
    w = worlds[1]
    args = [w.rank_args(k, hp, 1) for k in range(4)]
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in range(4)]
    errors = []

    def on_threads(fn):
        def body(k):
            try:
                with torch.cuda.stream(streams[k]):
                    fn(k)
            except Exception as e:          # reported after the join
                errors.append(e)
        ts = [threading.Thread(target=body, args=(k,)) for k in range(4)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        assert not errors, errors

    for st in streams:
        st.wait_stream(main)
    on_threads(lambda k: Z.zero_shard_reduce(args[k], k, w.partials, streams[k]))
    for st in streams:
        main.wait_stream(st)
    Z.zero_shard_combine(w.partials, 4, hp.max_grad_norm, w.global_buf, main)
    for st in streams:
        st.wait_stream(main)
    on_threads(lambda k: Z.zero_shard_apply(args[k], w.global_buf, streams[k]))
    for st in streams:
        main.wait_stream(st)
    torch.cuda.synchronize()
    a, b = worlds[0].result(), w.result()
    assert (a.sumsq, a.norm, a.coef, a.overflow) == (b.sumsq, b.norm, b.coef, b.overflow)
    for x, y in zip(worlds[0].master + worlds[0].exp_avg + worlds[0].exp_avg_sq,
                    w.master + w.exp_avg + w.exp_avg_sq):
        parity.assert_bitwise("state", parity.f32(y), parity.f32(x))
    parity.assert_bitwise("params", parity.u16(w.full_params), parity.u16(worlds[0].full_params))


def test_sharded_concatenation_equals_unsharded_on_gpu():
    say("sharded == unsharded")
    numel = 300_007
    sharded = SimulatedWorld(numel, 4, alignment=8, grad_dtype=BF16)
    whole = SimulatedWorld(numel, 1, n_replicas=4, alignment=8, grad_dtype=BF16)
    _fill(sharded, 2)
    for i in range(4):
        W.flat_normal(whole.grads[i], 0, numel, 1e-2, ("det", 2, i))
    W.flat_normal(whole.master[0], 0, numel, 0.02, ("detm", 2))
    for w in (sharded, whole):
        w.step(Hyper(), 1)
    assert sharded.result().clipped and whole.result().clipped
    assert abs(sharded.result().norm - whole.result().norm) <= 1e-12 * whole.result().norm
    cat = torch.cat([m[:v] for m, v in zip(sharded.master, sharded.valid)])
    parity.assert_rel("masters", parity.f32(cat), parity.f32(whole.master[0][:numel]), 1e-6)


def test_fused_step_equals_split_calls_and_peer_sum():
    say("zero_shard_step vs reduce/combine/apply")
    numel, world = 123_457, 1
    w1 = SimulatedWorld(numel, world, n_replicas=8, alignment=128, grad_dtype=BF16)
    w2 = SimulatedWorld(numel, world, n_replicas=8, alignment=128, grad_dtype=BF16)
    for w in (w1, w2):
        for i in range(8):
            W.flat_normal(w.grads[i], 0, numel, 1e-2, ("fused", i))
        W.flat_normal(w.master[0], 0, numel, 0.02, ("fusedm",))
    hp = Hyper()
    w1.step(hp, 1)
    info = Z.zero_shard_step(w2.rank_args(0, hp, 1), want_info=True)
    r1 = w1.result()
    assert (info.sumsq, info.coef, info.overflow) == (r1.sumsq, r1.coef, r1.overflow)
    parity.assert_bitwise("master", parity.f32(w1.master[0]), parity.f32(w2.master[0]))
    # peers' sum of squares enters the norm: with a large peer sum the clip
    # factor follows the combined norm
    w3 = SimulatedWorld(numel, world, n_replicas=8, alignment=128, grad_dtype=BF16)
    for i in range(8):
        W.flat_normal(w3.grads[i], 0, numel, 1e-2, ("fused", i))
    info3 = Z.zero_shard_step(w3.rank_args(0, hp, 1), peer_sumsq=3 * r1.sumsq,
                              want_info=True)
    assert abs(info3.norm - 2 * r1.norm) <= 1e-12 * r1.norm
    assert abs(info3.coef - np.float32(1.0 / (2 * r1.norm + 1e-6))) <= 1e-7 * info3.coef
    info4 = Z.zero_shard_step(w3.rank_args(0, hp, 1), peer_overflow=True, want_info=True)
    assert info4.overflow == 1


# ---------------------------------------------------------------- flatten
def _flatten_case(sizes, odd_views, flat_numel=None, seed=0):
    rng = np.random.default_rng(seed)
    srcs = []
    for k, n in enumerate(sizes):
        off = int(rng.integers(1, 8)) if odd_views and k % 2 else 0
        base = torch.from_numpy(rng.integers(0, 65536, n + off, dtype=np.uint64)
                                .astype(np.uint16).view(np.int16)).cuda()
        srcs.append(base[off:off + n].view(torch.bfloat16))
    slots, buckets = Z.zero_bucket_plan(sizes, 1 << 14)
    total = sum(sizes)
    flat_numel = flat_numel if flat_numel is not None else total + 77
    flat = torch.full((flat_numel + 64,), 0x1357, dtype=torch.int16, device="cuda")
    Z.zero_bucket_flatten(slots, srcs, torch.bfloat16, flat.view(torch.bfloat16), flat_numel)
    got = parity.u16(flat.view(torch.bfloat16))
    ref = oracle.flatten([parity.u16(s) for s in srcs], 1 << 14, flat_numel)
    parity.assert_bitwise("flat", got[:flat_numel], ref)
    assert (got[flat_numel:] == 0x1357).all(), "wrote past flat_numel"
    return slots, buckets, srcs


@pytest.mark.parametrize("odd", [False, True])
def test_flatten_ragged_tensors(odd):
    rng = np.random.default_rng(3)
    sizes = [int(x) for x in rng.integers(0, 40_000, 300)]
    sizes[5] = 0
    sizes[6] = 1
    sizes[7] = 7
    sizes[8] = 9
    say("flatten %d tensors, odd views %s" % (len(sizes), odd))
    _flatten_case(sizes, odd)


def test_flatten_edge_cases():
    say("flatten edges")
    _flatten_case([], False, flat_numel=100)
    _flatten_case([3], True, flat_numel=3)
    _flatten_case([1, 1, 1, 1, 1, 1, 1, 1, 1], True)
    _flatten_case([5_000_001], True)
    _flatten_case([8] * 130 + [13] * 131, True)             # more than one launch batch


def test_flatten_large_tables_with_crowded_slots():
    # Tables of more than 16 entries use the coarse index of the launch's
    # blocks; here big tensors sit between runs of one-block tensors, so
    # single slots hold many entries, and tables of 17, 128 and 129 entries
    # cross the switch and the launch batch.
    say("flatten: crowded coarse-index slots")
    crowd = []
    for k in range(6):
        crowd += [2_000_003 + 97 * k] + [1 + (j % 9) for j in range(20)]
    _flatten_case(crowd, True, seed=1)
    _flatten_case([300] * 17, True, seed=2)
    _flatten_case([1] * 100 + [3_000_001] + [5] * 27, True, seed=3)
    _flatten_case([7] * 64 + [1_000_000] + [7] * 64, False, seed=4)


def test_flatten_destinations_beyond_2_pow_32_elements():
    # Slots whose destinations cross 2^32 elements, with gaps between them
    # (zeroed, like the padding) and untouched elements before the first.
    # A launch's table counts destinations from its first one in 32 bits,
    # so the launcher must start a new batch before that would overflow.
    say("flatten: destinations beyond 2^32 elements")
    n32 = 1 << 32
    specs = [(16, 984), (1000, 5), (n32 - 3, 100), (n32 + 1000, 7), (n32 + 1007, 33)]
    flat_numel = n32 + 4096
    flat = torch.full((flat_numel + 64,), 0x1357, dtype=torch.int16, device="cuda")
    rng = np.random.default_rng(12)
    srcs = [torch.from_numpy(rng.integers(0, 65536, n + 3, dtype=np.uint64).astype(np.uint16)
                             .view(np.int16)).cuda()[k % 3:k % 3 + n].view(torch.bfloat16)
            for k, (_, n) in enumerate(specs)]
    slots = [Z.zero_tensor_slot_t(off, n, 0, 0) for off, n in specs]
    Z.zero_bucket_flatten(slots, srcs, torch.bfloat16, flat.view(torch.bfloat16), flat_numel)
    torch.cuda.synchronize()
    for (off, n), src in zip(specs, srcs):
        assert torch.equal(flat[off:off + n], src.view(torch.int16)), "slot at %d" % off
    assert bool((flat[:16] == 0x1357).all()), "wrote before the first slot"
    for lo, hi in ((1005, n32 - 3), (n32 + 97, n32 + 1000)):
        assert bool((flat[lo:hi] == 0).all()), "gap [%d, %d) not zeroed" % (lo, hi)
    end = specs[-1][0] + specs[-1][1]
    assert bool((flat[end:flat_numel] == 0).all()), "padding not zeroed"
    assert bool((flat[flat_numel:] == 0x1357).all()), "wrote past flat_numel"
    del flat
    torch.cuda.empty_cache()


def test_flatten_zeroes_gaps_between_slots():
    # Gaps between consecutive slots are zeroed like the padding, so no
    # stale value between two tensors can reach the reduce; elements before
    # the first slot belong to someone else and are left alone.
    say("flatten: gaps between slots")
    specs = [(5, 100), (120, 33), (153, 0), (160, 9), (300, 1)]
    flat_numel = 333
    flat = torch.full((flat_numel + 64,), 0x7F80, dtype=torch.int16, device="cuda")   # +inf
    rng = np.random.default_rng(13)
    srcs = [torch.from_numpy(rng.integers(0, 65536, max(n, 1), dtype=np.uint64)
                             .astype(np.uint16).view(np.int16)).cuda()[:n].view(torch.bfloat16)
            for _, n in specs]
    slots = [Z.zero_tensor_slot_t(off, n, 0, 0) for off, n in specs]
    Z.zero_bucket_flatten(slots, srcs, torch.bfloat16, flat.view(torch.bfloat16), flat_numel)
    got = parity.u16(flat.view(torch.bfloat16))
    ref = np.zeros(flat_numel + 64, np.uint16)
    ref[:5] = 0x7F80
    ref[flat_numel:] = 0x7F80
    for (off, n), src in zip(specs, srcs):
        ref[off:off + n] = parity.u16(src)
    parity.assert_bitwise("flat", got, ref)


def test_flatten_per_bucket():
    say("flatten bucket by bucket")
    rng = np.random.default_rng(4)
    sizes = [int(x) for x in rng.integers(1, 9000, 60)]
    slots, buckets = Z.zero_bucket_plan(sizes, 20_000)
    srcs = [torch.randint(-32768, 32767, (n,), dtype=torch.int16, device="cuda")
            .view(torch.bfloat16) for n in sizes]
    total = sum(sizes)
    flat = torch.full((total,), 0x1111, dtype=torch.int16, device="cuda")
    for b in buckets:
        sl = slots[b.first_tensor:b.first_tensor + b.n_tensors]
        Z.zero_bucket_flatten(sl, srcs[b.first_tensor:b.first_tensor + b.n_tensors],
                              torch.bfloat16, flat.view(torch.bfloat16), b.end)
    ref = np.concatenate([parity.u16(s) for s in srcs])
    parity.assert_bitwise("flat", parity.u16(flat.view(torch.bfloat16)), ref)


def test_flatten_pieces_beyond_one_table_entry():
    # A tensor and a padding run longer than one table entry (2^30
    # elements), the tensor at an odd source offset.
    n = (1 << 30) + 12_345
    pad = (1 << 30) + 77
    say("flatten one tensor of %d elements and %d padding" % (n, pad))
    base = torch.randint(-32768, 32767, (n + 3,), dtype=torch.int16, device="cuda")
    src = base[3:].view(torch.bfloat16)
    slots, _ = Z.zero_bucket_plan([n], 1 << 40)
    flat = torch.full((n + pad + 64,), 0x1357, dtype=torch.int16, device="cuda")
    # destination offset 5: shift the slot so the copy is misaligned on both sides
    slots[0].offset = 5
    Z.zero_bucket_flatten(slots, [src], torch.bfloat16, flat.view(torch.bfloat16), n + pad)
    assert torch.equal(flat[5:5 + n], base[3:]), "body differs"
    assert bool((flat[:5] == 0x1357).all()), "wrote before the slot"
    assert bool((flat[5 + n:n + pad] == 0).all()), "padding not zeroed"
    assert bool((flat[n + pad:] == 0x1357).all()), "wrote past flat_numel"


# ---------------------------------------------------- gradient accumulation
ACC_CASES = [
    # (numel, world, alignment, dtype, sigma, loss_scale, micro_batches, steps)
    (5, 4, 8, BF16, 1e-2, 1.0, 2, 2),              # empty ranks, tail only
    (4097, 4, 8, FP16, 1e-3, 2.0**12, 3, 2),
    (100_003, 8, 128, BF16, 1e-3, 1.0, 4, 2),
    (1_000_003, 2, 128, BF16, 3e-2, 1.0, 2, 3),
]


@pytest.mark.parametrize("case", ACC_CASES, ids=["P%d-N%d-%s-K%d" % (c[0], c[1], str(c[3])[6:], c[6])
                                                 for c in ACC_CASES])
def test_accumulation_window_matches_oracle(case):
    numel, world, align, dt, sigma, scale, K, steps = case
    say("accumulation %s" % (case,))
    spec = parity.Spec(numel=numel, world_size=world, alignment=align, grad_dtype=dt,
                       grad_sigma=sigma, steps=steps, micro_batches=K,
                       name="acc-%d-%d-%d" % (numel, world, K), hp=Hyper(loss_scale=scale))
    rep = parity.run(spec)
    say("norm rel err %.2e, bitwise state %.6f" % (rep.norm_rel_err, rep.state_bitwise))


@pytest.mark.parametrize("micro", [0, 1, 2])
def test_accumulation_poison_in_any_micro_batch_skips(micro):
    numel, world = 20_011, 4
    say("accumulation, poison in micro-batch %d" % micro)
    sched = [None, W.Poison(1, 1, 777, 2), None]
    spec = parity.Spec(numel=numel, world_size=world, alignment=8, grad_dtype=FP16,
                       grad_sigma=1e-3, steps=3, poison=sched, poison_micro=micro,
                       micro_batches=3, dynamic_scale=True, scaler_args=(10, 2, 1, 1.0),
                       name="acc-poison")
    rep = parity.run(spec)
    assert rep.skipped == 1


LOCAL_CASES = [
    # (numel, world, alignment, dtype, sigma, loss_scale, micro_batches, replicas)
    (5, 4, 8, BF16, 1e-2, 1.0, 2, 4),              # empty ranks, tail only
    (40_001, 3, 8, FP16, 1e-3, 2.0**12, 4, 3),
    (100_003, 4, 128, BF16, 1e-3, 1.0, 3, 4),
    (1_000_003, 8, 128, BF16, 3e-2, 1.0, 2, 8),
    (77_777, 2, 128, FP16, 1e-3, 2.0**10, 3, 11),  # generic replica loop
]


@pytest.mark.parametrize("case", LOCAL_CASES,
                         ids=["P%d-N%d-%s-K%d-R%d" % (c[0], c[1], str(c[3])[6:], c[6], c[7])
                              for c in LOCAL_CASES])
def test_local_accumulation_matches_oracle(case):
    # Each replica sums its window in fp32 (zero_accumulate_local), then one
    # reduce of the fp32 sums (grad_dtype ZERO_FP32); the window sums, the
    # reduced slices, the state and the cast are compared with the oracle.
    numel, world, align, dt, sigma, scale, K, R = case
    say("local accumulation %s" % (case,))
    spec = parity.Spec(numel=numel, world_size=world, n_replicas=R, alignment=align,
                       grad_dtype=dt, grad_sigma=sigma, steps=2, micro_batches=K,
                       local_accumulation=True, name="local-%d-%d-%d" % (numel, world, K),
                       hp=Hyper(loss_scale=scale))
    rep = parity.run(spec)
    say("norm rel err %.2e, bitwise state %.6f" % (rep.norm_rel_err, rep.state_bitwise))


@pytest.mark.parametrize("micro", [0, 2])
def test_local_accumulation_poison_in_any_micro_batch_skips(micro):
    say("local accumulation, poison in micro-batch %d" % micro)
    sched = [None, W.Poison(1, 1, 777, 1), None]
    spec = parity.Spec(numel=20_011, world_size=4, alignment=8, grad_dtype=FP16,
                       grad_sigma=1e-3, steps=3, poison=sched, poison_micro=micro,
                       micro_batches=3, local_accumulation=True, dynamic_scale=True,
                       scaler_args=(10, 2, 1, 1.0), name="local-poison")
    rep = parity.run(spec)
    assert rep.skipped == 1


def test_accumulate_local_edges():
    # Ragged lengths end in a scalar tail; nothing past n is written.
    say("zero_accumulate_local edges")
    import oracle
    for n in (1, 3, 4, 5, 1023, 4099):
        g1 = torch.randn(n + 8, device="cuda").to(BF16)
        g2 = torch.randn(n + 8, device="cuda").to(BF16)
        acc = torch.full((n + 8,), 5.0, device="cuda")
        Z.zero_accumulate_local(g1, acc, True, n=n)
        Z.zero_accumulate_local(g2, acc, False, n=n)
        ref = oracle.accumulate_local([parity.u16(g1[:n]), parity.u16(g2[:n])], oracle.BF16)
        parity.assert_bitwise("n=%d" % n, parity.f32(acc[:n]), ref)
        assert bool((acc[n:] == 5.0).all()), "wrote past n"


def test_accumulate_then_fused_step_equals_split_calls():
    say("zero_shard_accumulate + zero_shard_step vs the split world")
    numel, K = 123_457, 3
    w1 = SimulatedWorld(numel, 1, n_replicas=8, alignment=128, grad_dtype=BF16)
    w2 = SimulatedWorld(numel, 1, n_replicas=8, alignment=128, grad_dtype=BF16)
    for w in (w1, w2):
        W.flat_normal(w.master[0], 0, numel, 0.02, ("accm",))
    hp = Hyper()
    for j in range(K):
        for w in (w1, w2):
            for i in range(8):
                W.flat_normal(w.grads[i], 0, numel, 1e-2, ("acc", i, j))
        if j < K - 1:
            w1.accumulate(hp, first=j == 0)
            Z.zero_shard_accumulate(w2.rank_args(0, hp, 1, accumulate=j > 0))
        else:
            w1.step(hp, 1, accumulate=True)
            info = Z.zero_shard_step(w2.rank_args(0, hp, 1, accumulate=True), want_info=True)
    r1 = w1.result()
    assert (info.sumsq, info.coef, info.overflow) == (r1.sumsq, r1.coef, r1.overflow)
    # real elements only: the workspace's padding tail is never written
    for a, b in ((w1.master[0], w2.master[0]), (w1.exp_avg[0], w2.exp_avg[0]),
                 (w1.reduced_grad(0), w2.reduced_grad(0))):
        parity.assert_bitwise("fused vs split", parity.f32(a[:numel]), parity.f32(b[:numel]))


def test_ping_pong_state_equals_in_place():
    # Two state sets alternated step by step give the same bits as one set
    # updated in place.
    say("ping-pong state")
    numel, K = 250_007, 4
    hp = Hyper()
    w1 = SimulatedWorld(numel, 1, n_replicas=8, alignment=128, grad_dtype=BF16)
    w2 = SimulatedWorld(numel, 1, n_replicas=8, alignment=128, grad_dtype=BF16)
    second = [torch.full((w2.s,), 9.0, device="cuda") for _ in range(3)]
    for w in (w1, w2):
        W.flat_normal(w.master[0], 0, numel, 0.02, ("ppm",))
    sets = [list(w2.state(0)), second]
    for t in range(1, K + 1):
        for w in (w1, w2):
            for i in range(8):
                W.flat_normal(w.grads[i], 0, numel, 1e-2, ("pp", t, i))
        w1.step(hp, t)
        a = w2.rank_args(0, hp, t)
        src, dst = sets[(t - 1) % 2], sets[t % 2]
        a.master, a.exp_avg, a.exp_avg_sq = src
        a.master_out, a.exp_avg_out, a.exp_avg_sq_out = dst
        Z.zero_shard_step(a)
    final = sets[K % 2]
    for got, ref in zip(final, w1.state(0)):
        parity.assert_bitwise("ping-pong state", parity.f32(got[:numel]), parity.f32(ref[:numel]))
    parity.assert_bitwise("ping-pong params", parity.u16(w2.full_params), parity.u16(w1.full_params))


def test_adamw_on_ieee_edge_values_matches_oracle():
    # Every combination of master, m and v drawn from signed zeros,
    # subnormals, the smallest normal, ordinary values, the largest finite
    # value, infinities and NaN, under finite gradients from tiny to near the
    # bf16 maximum (clipping off, so nothing rescales them).  The device's
    # division, square root and subnormal handling must give the oracle's
    # bits; a NaN must be a NaN on both sides.
    import itertools
    import oracle
    say("AdamW on IEEE edge values")
    S = np.array([0.0, -0.0, 1.4e-45, -1.4e-45, 1e-40, 1.17549435e-38, 1e-20, 0.02, -0.5, 3.0,
                  1e20, 3.4028235e38, -3.4028235e38, np.inf, -np.inf, np.nan], np.float32)
    G = np.array([0.0, -0.0, 1e-40, 0.5, -3.0, 1e30, 3.38e38, -1e-3], np.float32)
    combos = np.array(list(itertools.product(range(S.size), repeat=3)), np.int64)
    n = combos.shape[0] * G.size
    p0 = np.tile(S[combos[:, 0]], G.size)
    m0 = np.tile(S[combos[:, 1]], G.size)
    v0 = np.tile(S[combos[:, 2]], G.size)
    gcodes = np.repeat(oracle.f32_to_bf16(G), combos.shape[0])
    g = oracle.bf16_to_f32(gcodes)
    hp = Hyper(max_grad_norm=0.0)
    world = SimulatedWorld(n, 1, n_replicas=1, alignment=8, grad_dtype=BF16)
    world.grads[0].view(torch.int16)[:n].copy_(torch.from_numpy(gcodes.view(np.int16)))
    for dev, host in ((world.master[0], p0), (world.exp_avg[0], m0), (world.exp_avg_sq[0], v0)):
        dev[:n].copy_(torch.from_numpy(host))
    p, m, v = p0.copy(), m0.copy(), v0.copy()
    for t in (1, 3):
        world.step(hp, t)
        res = world.result()
        assert not res.overflow and not res.clipped
        oracle.adamw(g, p, m, v, 1.0, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t)
        for name, dev, ref in (("master", world.master[0], p), ("exp_avg", world.exp_avg[0], m),
                               ("exp_avg_sq", world.exp_avg_sq[0], v)):
            got = parity.f32(dev)[:n]
            nan = np.isnan(ref)
            assert np.array_equal(np.isnan(got), nan), "%s: NaN positions differ (t=%d)" % (name, t)
            parity.assert_bitwise("t=%d %s" % (t, name), got[~nan], ref[~nan])
        cast = parity.u16(world.full_params)[:n]
        want = oracle.f32_to_bf16(p)
        cnan = np.isnan(oracle.bf16_to_f32(want))
        assert np.array_equal(np.isnan(oracle.bf16_to_f32(cast)), cnan)
        parity.assert_bitwise("t=%d cast" % t, cast[~cnan], want[~cnan])
