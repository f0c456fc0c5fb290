"""GPU parity at the five workloads' own sizes, through the C ABI.

The encoder layer (67M params, 10 steps) and the fp16 scaler run (50M
params, 200 steps) are compared with the oracle element by element over
their whole state.  The 13B/8 shard runs in the launch configuration the
bench times, and the ragged 2000-tensor workload runs bucketed and flattened
over a world of 8 ranks (2.18e9 params).  For those, and for a shard beyond
2^31 elements, the oracle regenerates the inputs chunk by chunk and takes
its reduce over every element (its norm, overflow flag and fp32 reduced
gradient), then its AdamW and cast over every element, a chunk at a time,
split over host threads; every element of the reduced gradient, master,
both moments and the cast is compared with the device's.  A structural
sample (block and XCD-range edges plus random elements) is checked first,
as a quick pre-check, and the full buffer outside the ranks' slices must
keep its canary.  Each case prints its progress before and while it
touches the GPU.
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


def say(msg):
    print(msg, flush=True)


def test_encoder_layer_workload_10_steps():
    w = W.ENCODER_4096
    say("encoder layer: %d params, %d ranks, %d steps" % (w.numel, w.world_size, w.steps))
    spec = parity.Spec(numel=w.numel, world_size=w.world_size, grad_dtype=w.grad_dtype,
                       grad_sigma=w.grad_sigma, master_sigma=w.master_sigma, steps=w.steps,
                       name="encoder-4096")
    rep = parity.run(spec, check_every_step=False, log=say)
    assert rep.steps == 10 and rep.skipped == 0
    assert all(n > 1.0 for n in rep.norms)            # clipping active every step
    say("norm rel err %.2e, bitwise state %.6f, cast max ulp %d"
        % (rep.norm_rel_err, rep.state_bitwise, rep.cast_max_ulp))


def test_scaler_workload_200_steps():
    w = W.SCALER_50M
    sched = W.poison_schedule(w.steps, w.world_size, w.numel, p=0.05, seed=0)
    n_poison = sum(x is not None for x in sched)
    say("fp16 scaler: %d params, %d ranks, %d steps, %d poisoned" % (w.numel, w.world_size,
                                                                      w.steps, n_poison))
    spec = parity.Spec(numel=w.numel, world_size=w.world_size, grad_dtype=w.grad_dtype,
                       grad_sigma=w.grad_sigma, master_sigma=w.master_sigma, steps=w.steps,
                       poison=sched, dynamic_scale=True, scaler_args=(16, 100, 2, 1.0),
                       name="scaler-50m")
    rep = parity.run(spec, check_every_step=False,
                     log=lambda m: say(m) if m.startswith("step") and
                     int(m.split()[1].rstrip(":")) % 20 == 0 else None)
    assert rep.skipped == n_poison
    assert len(rep.scales) == w.steps
    say("scales: start %g, min %g, max %g, final %g"
        % (2.0**16, min(rep.scales), max(rep.scales), rep.scales[-1]))


# ------------------------------------------------------------ 13B/8 shard
def _chunked(n, step=1 << 28):
    for a in range(0, n, step):
        yield a, min(n, a + step)


def test_13b_shard_in_bench_configuration():
    """Rank 0 of 8 over 13e9 params: the bench's buffers and calls."""
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s = part.shard_numel
    n = Z.zero_partition_valid_numel(part, 0)
    nrep = w.world_size
    say("13B/8 shard: s=%d, %d replicas; allocating ~78 GB" % (s, nrep))
    dev = "cuda"
    gkey = lambda i: W.grad_key(w, 0, 0, i)
    grads = []
    for i in range(nrep):
        g = torch.empty(s, dtype=torch.bfloat16, device=dev)
        W.flat_normal(g, 0, w.numel, w.grad_sigma, gkey(i))
        grads.append(g)
    master = torch.empty(s, dtype=torch.float32, device=dev)
    W.flat_normal(master, 0, w.numel, w.master_sigma, W.master_key(w, 0))
    m = torch.zeros(s, dtype=torch.float32, device=dev)
    v = torch.zeros(s, dtype=torch.float32, device=dev)
    full = torch.full((part.padded_numel,), parity.CANARY, dtype=torch.int16, device=dev)
    ws = torch.empty(Z.zero_shard_workspace_bytes(s), dtype=torch.uint8, device=dev)
    hp = Hyper(lr=w.lr, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm)

    def args(t):
        return Z.StepArgs(world_size=w.world_size, rank=0, shard_numel=s, valid_numel=n,
                          replica_grads=grads, master=master, exp_avg=m, exp_avg_sq=v,
                          full_params=full.view(torch.bfloat16), workspace=ws, lr=hp.lr,
                          weight_decay=hp.weight_decay, step=t, max_grad_norm=hp.max_grad_norm,
                          grad_dtype=torch.bfloat16, param_dtype=torch.bfloat16)

    # the oracle's norm over every element, from regenerated inputs, and
    # its AdamW on a sample as a quick pre-check (every element follows)
    oref = parity.shard13b_reference(log=say)
    sample, inv = oref["sample"], oref["inv"]
    assert oref["overflow"] == 0
    applies, onorm, o_g = oref["applies"], oref["norm"], oref["g"]

    # step 1, the fused entry point (the bench's kernels and grids)
    say("step 1")
    info = Z.zero_shard_step(args(1), want_info=True)
    assert info.overflow == 0 and bool(info.clipped) == applies
    assert abs(info.norm - onorm) <= parity.RTOL_NORM * onorm, (info.norm, onorm)
    gdev = ws[:4 * s].view(torch.float32)
    parity.assert_bitwise("reduced grad (sample)", parity.take(gdev, sample).numpy(), o_g)

    for t in (1, 2):
        if t == 2:
            say("step 2 (same gradients, as the bench repeats)")
            info2 = Z.zero_shard_step(args(2), want_info=True)
            assert info2.overflow == 0 and info2.norm == info.norm
        o_p, o_m, o_v = oref["states"][t - 1]
        for name, dev_t, ref in (("master", master, o_p), ("exp_avg", m, o_m),
                                 ("exp_avg_sq", v, o_v)):
            parity.assert_rel("step %d %s (sample)" % (t, name), parity.take(dev_t, sample).numpy(),
                              ref, parity.RTOL_STATE)
        got = parity.take(full, sample).numpy().view(np.uint16)
        parity.assert_cast("step %d cast (sample)" % t, got, oracle.f32_to_bf16(o_p))
        # every element: the oracle's AdamW steps 1..t and its cast
        say("step %d: the oracle's update over all %d elements" % (t, n))
        st = parity.check_every_element("step %d" % t, oref["g_full"], (master, m, v),
                                        oref["init_master"], oref["coef"], hp, range(1, t + 1),
                                        oracle.BF16, full=full, full_off=0,
                                        grad=gdev if t == 1 else None, log=say)
        assert st["elements"] == n == 1_625_000_064
        say("step %d: %d elements equal the oracle (%d state values and %d casts not bit-equal)"
            % (t, st["elements"], st["state_bits_differ"], st["cast_differ"]))
    # nothing written outside rank 0's real elements
    for a, b in _chunked(part.padded_numel - s, 1 << 30):
        assert bool((full[s + a:s + b] == parity.CANARY).all()), "write outside the slice"
    say("13B/8 shard matches: norm %.6f (oracle %.6f), coef %.9g" % (info.norm, onorm, info.coef))
    del grads, master, m, v, full, ws
    torch.cuda.empty_cache()


# -------------------------------------------------------- ragged, bucketed
def test_ragged_bucketed_workload():
    """2000 tensors, flattened bucket by bucket, then one step of 8 ranks."""
    w = W.RAGGED_2000
    sizes = list(w.tensor_sizes)
    P, N = w.numel, w.world_size
    slots, buckets = Z.zero_bucket_plan(sizes, int(2e8))
    off, bof, nb = oracle.bucket_plan(sizes, int(2e8))
    assert [x.offset for x in slots] == list(off) and len(buckets) == nb
    say("ragged: %d tensors, %d params, %d buckets, %d ranks" % (len(sizes), P, nb, N))
    world = SimulatedWorld(P, N, alignment=w.alignment, grad_dtype=torch.bfloat16)
    s, padded = world.s, world.padded
    gkey = lambda i: W.grad_key(w, 0, 0, i)
    # per-tensor gradients live at odd offsets of one pool, one element apart
    pool = torch.empty(P + len(sizes) + 8, dtype=torch.bfloat16, device="cuda")
    ref = torch.empty(padded, dtype=torch.bfloat16, device="cuda")
    for i in range(N):
        W.flat_normal(ref, 0, P, w.grad_sigma, gkey(i))      # generator, zero padding
        srcs = []
        for k, x in enumerate(slots):
            src = pool[x.offset + k + 1:x.offset + k + 1 + x.numel]
            src.copy_(ref[x.offset:x.offset + x.numel])
            srcs.append(src)
        world.grads[i].fill_(-1.0)
        for bi, b in enumerate(buckets):
            last = bi == len(buckets) - 1
            Z.zero_bucket_flatten(slots[b.first_tensor:b.first_tensor + b.n_tensors],
                                  srcs[b.first_tensor:b.first_tensor + b.n_tensors],
                                  torch.bfloat16, world.grads[i], padded if last else b.end)
        assert torch.equal(world.grads[i].view(torch.int16), ref.view(torch.int16)), \
            "replica %d: flattened buffer differs from the generator" % i
        say("  replica %d flattened and checked" % i)
    del pool, ref
    for k, r in enumerate(world.ranks):
        W.flat_normal(world.master[k], r * s, P, 0.02, W.master_key(w, 0))
    world.full_params.view(torch.int16).fill_(parity.CANARY)

    rng = np.random.default_rng(6)
    # each rank's own block and XCD-range edges, both ends, random elements
    sample = np.unique(np.concatenate(
        [r * s + parity.structural_sample(world.valid[r], rng, n_random=8192) for r in range(N)]))
    say("oracle: reduce over %d elements x %d replicas" % (P, N))
    inv = oracle.inv_scale(1.0)
    fr = parity.oracle_reduce_full(N, 0, P, P, w.grad_sigma, gkey, torch.bfloat16, inv, log=say)
    assert fr.overflow == 0
    applies, onorm, ocoef = oracle.clip(fr.sumsq, w.max_grad_norm)
    # the sample first, as a quick check
    real = sample < P
    sample = sample[real]
    o_g = fr.g[sample].copy()
    o_p = parity.gather_generated(sample, 0, P, 0.02, W.master_key(w, 0), torch.float32, P).copy()
    o_m = np.zeros(sample.size, np.float32)
    o_v = np.zeros(sample.size, np.float32)
    oracle.adamw(o_g, o_p, o_m, o_v, ocoef, w.lr, 0.9, 0.999, 1e-8, w.weight_decay, 1)

    say("step over %d ranks" % N)
    hp = Hyper(lr=w.lr, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm)
    world.step(hp, 1)
    res = world.result()
    assert res.overflow == 0 and bool(res.clipped) == applies
    assert abs(res.norm - onorm) <= parity.RTOL_NORM * onorm, (res.norm, onorm)
    rank_of = sample // s
    loc = sample - rank_of * s
    got = {k: np.empty(sample.size, np.float32) for k in ("g", "p", "m", "v")}
    for r in range(N):
        sel = np.flatnonzero(rank_of == r)
        if not sel.size:
            continue
        got["g"][sel] = parity.take(world.reduced_grad(r), loc[sel]).numpy()
        got["p"][sel] = parity.take(world.master[r], loc[sel]).numpy()
        got["m"][sel] = parity.take(world.exp_avg[r], loc[sel]).numpy()
        got["v"][sel] = parity.take(world.exp_avg_sq[r], loc[sel]).numpy()
    parity.assert_bitwise("reduced grad (sample)", got["g"], o_g)
    parity.assert_rel("master (sample)", got["p"], o_p, parity.RTOL_STATE)
    parity.assert_rel("exp_avg (sample)", got["m"], o_m, parity.RTOL_STATE)
    parity.assert_rel("exp_avg_sq (sample)", got["v"], o_v, parity.RTOL_STATE)
    full = world.full_params.view(torch.int16)
    parity.assert_cast("cast (sample)", parity.take(full, sample).numpy().view(np.uint16),
                       oracle.f32_to_bf16(o_p))
    # every element of every rank: the oracle's reduced gradient, AdamW and cast
    total = 0
    for r in range(N):
        lo, n = r * s, world.valid[r]
        say("rank %d: the oracle's update over all %d elements" % (r, n))
        st = parity.check_every_element(
            "rank %d" % r, fr.g[lo:lo + n], (world.master[r], world.exp_avg[r], world.exp_avg_sq[r]),
            lambda a, b, lo=lo: parity.gen_host(lo + a, lo + b, P, 0.02, W.master_key(w, 0)),
            ocoef, hp, (1,), oracle.BF16, full=full, full_off=lo, grad=world.reduced_grad(r))
        total += st["elements"]
        assert bool((full[lo + n:lo + s] == parity.CANARY).all()), "padding written, rank %d" % r
    assert total == P == 2_184_105_843
    say("ragged workload matches over all %d elements: norm %.6f (oracle %.6f)"
        % (total, res.norm, onorm))


def test_shard_beyond_2_pow_31_elements():
    """One rank whose shard holds more than 2^31 elements (64-bit indexing in
    every kernel), 2 bf16 replicas, a ragged tail."""
    P = (1 << 31) + (1 << 20) + 5
    R = 2
    say("shard of %d elements, %d replicas" % (P, R))
    world = SimulatedWorld(P, 1, n_replicas=R, alignment=8, grad_dtype=torch.bfloat16)
    s = world.s
    gkey = lambda i: ("big", i)
    for i in range(R):
        W.flat_normal(world.grads[i], 0, P, 1e-3, gkey(i))
    W.flat_normal(world.master[0], 0, P, 0.02, ("big-master",))
    world.full_params.view(torch.int16).fill_(parity.CANARY)
    rng = np.random.default_rng(8)
    sample = np.unique(np.concatenate([
        parity.structural_sample(P, rng, n_random=1 << 15),
        (1 << 31) + np.arange(-4, 5, dtype=np.int64), np.arange(P - 7, P, dtype=np.int64)]))
    inv = oracle.inv_scale(1.0)
    fr = parity.oracle_reduce_full(R, 0, P, P, 1e-3, gkey, torch.bfloat16, inv, log=say)
    assert fr.overflow == 0
    applies, onorm, ocoef = oracle.clip(fr.sumsq, 1.0)
    o_g = fr.g[sample].copy()
    o_p = parity.gather_generated(sample, 0, P, 0.02, ("big-master",), torch.float32, P).copy()
    o_m = np.zeros(sample.size, np.float32)
    o_v = np.zeros(sample.size, np.float32)
    oracle.adamw(o_g, o_p, o_m, o_v, ocoef, 6e-5, 0.9, 0.999, 1e-8, 0.01, 1)
    say("step")
    world.step(Hyper(), 1)
    res = world.result()
    assert res.overflow == 0 and bool(res.clipped) == applies
    assert abs(res.norm - onorm) <= parity.RTOL_NORM * onorm, (res.norm, onorm)
    parity.assert_bitwise("reduced grad (sample)", parity.take(world.reduced_grad(0), sample)
                          .numpy(), o_g)
    parity.assert_rel("master (sample)", parity.take(world.master[0], sample).numpy(), o_p,
                      parity.RTOL_STATE)
    parity.assert_rel("exp_avg (sample)", parity.take(world.exp_avg[0], sample).numpy(), o_m,
                      parity.RTOL_STATE)
    parity.assert_rel("exp_avg_sq (sample)", parity.take(world.exp_avg_sq[0], sample).numpy(),
                      o_v, parity.RTOL_STATE)
    full = world.full_params.view(torch.int16)
    parity.assert_cast("cast (sample)", parity.take(full, sample).numpy().view(np.uint16),
                       oracle.f32_to_bf16(o_p))
    say("the oracle's update over all %d elements" % P)
    st = parity.check_every_element(
        "beyond 2^31", fr.g, (world.master[0], world.exp_avg[0], world.exp_avg_sq[0]),
        lambda a, b: parity.gen_host(a, b, P, 0.02, ("big-master",)), ocoef, Hyper(), (1,),
        oracle.BF16, full=full, full_off=0, grad=world.reduced_grad(0), log=say)
    assert st["elements"] == P
    assert bool((full[P:s] == parity.CANARY).all())
    say("shard beyond 2^31 matches over all %d elements: norm %.6f" % (P, res.norm))
