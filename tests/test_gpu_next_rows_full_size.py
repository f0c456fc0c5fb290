"""GPU parity of the next rows at the sizes, and in the launch
configurations, the benchmark times them.

- Offload (`bench.py --workload offload`): rank 0 of the 13B/8 workload with
  its fp32 state in pinned host memory.  Pass 1 and the combine run on the
  GPU, zero_offload_apply does the rest; two steps on the same gradients.
  The oracle's reduce, AdamW and cast over every element decide (a
  structural sample is checked first), and nothing outside the rank's
  slice is written.
- ZeRO-3 gather (`--workload zero3`): the 13B model's bf16 parameters as 8
  rank shards, walked as 40 layers with prefetch.  Every layer equals its
  flat range of the parameter buffer (the definition: the shards laid end
  to end), and sampled elements equal the generator's values.
- Re-partition (`--workload repartition`): the ragged model's optimizer
  state (2.18e9 params, 3 arrays) moved from 8 ranks to 3.  Sampled
  elements equal the generator's values at their flat index, every new
  rank's real elements equal the old slices laid end to end, and the
  padding is zero.
- Two state sets (`--state-buffers 2`): the 13B/8 step read from one set
  and written to the other equals the same step in place, bit for bit over
  every element of the state and of the cast slice, and both equal the
  oracle's two steps over every element.
- Accumulation per micro-batch (`--micro-batches 4`): rank 0 of the 13B/8
  workload reduces the 8 replicas 4 times into its fp32 slice (the first
  sets it, the others add), over the same gradients each time as the
  bench repeats them, then combines and applies.  The oracle's window over
  every element of the shard (its norm, its reduced gradient, AdamW and the
  cast) decides, after a quick check at a structural sample; the canary
  outside the slice holds.
- Accumulation before the reduce (`--micro-batches 4 --accumulation
  local`): the rank's own 13e9-element gradient summed 4 times in fp32,
  then one reduce of its shard over 8 fp32 replicas.  The oracle's window
  sums at a sample of the whole gradient, and its reduce, AdamW and cast
  over every element of the shard decide.
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


def _chunked(n, step=1 << 28):
    for a in range(0, n, step):
        yield a, min(n, a + step)


def _free(*_):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ offload
def test_offload_13b_in_bench_configuration():
    oref = parity.shard13b_reference(log=say)
    w, part, s, n, sample = oref["w"], oref["part"], oref["s"], oref["n"], oref["sample"]
    assert oref["overflow"] == 0
    say("offload 13B/8: 8 replicas on the GPU, 3 x %d fp32 pinned on the host" % s)
    grads = []
    for i in range(w.world_size):
        g = torch.empty(s, dtype=torch.bfloat16, device="cuda")
        W.flat_normal(g, 0, w.numel, w.grad_sigma, oref["gkey"](i))
        grads.append(g)
    master = torch.empty(s, dtype=torch.float32, pin_memory=True)
    tmp = torch.empty(W.CHUNK, dtype=torch.float32, device="cuda")
    for a in range(0, s, W.CHUNK):
        b = min(s, a + W.CHUNK)
        W.flat_normal(tmp[:b - a], a, w.numel, w.master_sigma, W.master_key(w, 0))
        master[a:b].copy_(tmp[:b - a])
    m = torch.zeros(s, dtype=torch.float32, pin_memory=True)
    v = torch.zeros(s, dtype=torch.float32, pin_memory=True)
    full = torch.full((part.padded_numel,), parity.CANARY, dtype=torch.int16, device="cuda")
    ws = torch.empty(Z.zero_shard_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    partials = torch.zeros(Z.zero_partials_bytes(1), dtype=torch.uint8, device="cuda")
    glob = torch.zeros(256, dtype=torch.uint8, device="cuda")
    staging = Z.OffloadStaging(1 << 25, 0)
    hp = oref["hp"]
    idx = torch.from_numpy(sample)
    for t in (1, 2):
        say("offloaded step %d" % t)
        a = Z.StepArgs(world_size=w.world_size, rank=0, shard_numel=s, valid_numel=n,
                       replica_grads=grads, master=master, exp_avg=m, exp_avg_sq=v,
                       full_params=full.view(torch.bfloat16), workspace=ws, lr=hp.lr,
                       weight_decay=hp.weight_decay, step=t, max_grad_norm=hp.max_grad_norm)
        Z.zero_shard_reduce(a, 0, partials)
        Z.zero_shard_combine(partials, 1, hp.max_grad_norm, glob)
        info = Z.zero_offload_apply(a, glob, staging, want_info=True)
        assert info.overflow == 0 and bool(info.clipped) == oref["applies"]
        assert abs(info.norm - oref["norm"]) <= parity.RTOL_NORM * oref["norm"]
        o_p, o_m, o_v = oref["states"][t - 1]
        for name, host, ref in (("master", master, o_p), ("exp_avg", m, o_m),
                                ("exp_avg_sq", v, o_v)):
            parity.assert_rel("step %d %s (sample)" % (t, name), host[idx].numpy(), ref,
                              parity.RTOL_STATE)
        parity.assert_cast("step %d cast (sample)" % t,
                           parity.take(full, sample).numpy().view(np.uint16),
                           oracle.f32_to_bf16(o_p))
        say("step %d: the oracle's update over all %d elements" % (t, n))
        st = parity.check_every_element("offloaded step %d" % t, oref["g_full"], (master, m, v),
                                        oref["init_master"], oref["coef"], hp, range(1, t + 1),
                                        oracle.BF16, full=full, full_off=0, log=say)
        assert st["elements"] == n
    for a0, b0 in _chunked(part.padded_numel - s, 1 << 30):
        assert bool((full[s + a0:s + b0] == parity.CANARY).all()), "write outside the slice"
    say("offload matches: norm %.6f" % info.norm)
    del grads, full, ws, tmp
    _free()


# ------------------------------------------------------------ ZeRO-3 gather
def test_zero3_gather_13b_in_bench_configuration():
    from zero_sharded_optimizer_step_amd.zero3 import LayerGatherer
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s = part.shard_numel
    key = ("bench-zero3",)
    say("ZeRO-3 gather: 13B bf16 parameters, 8 shards, 40 layers")
    full = torch.empty(part.padded_numel, dtype=torch.bfloat16, device="cuda")
    W.flat_normal(full, 0, w.numel, 0.02, key)
    shards = [full[r * s:(r + 1) * s] for r in range(w.world_size)]
    L = 40
    sizes = [w.numel // L] * L
    sizes[-1] += w.numel - sum(sizes)
    g = LayerGatherer(part, shards, sizes, int(2e8), int(1e9))    # the bench's live bound
    rng = np.random.default_rng(9)
    edges = np.concatenate([np.cumsum(sizes)[:-1], np.arange(1, w.world_size) * s])
    sample = np.unique(np.concatenate([rng.integers(0, w.numel, 1 << 16, dtype=np.int64),
                                       edges - 1, edges, [0, w.numel - 1]]))
    expected = parity.gather_generated(sample, 0, w.numel, 0.02, key, torch.bfloat16, w.numel)
    got = np.zeros(sample.size, np.uint16)
    seen = 0
    for k, params in g.forward():
        lo, n = g.layers[k]
        assert k == seen and params.numel() == n
        seen += 1
        assert torch.equal(params.view(torch.int16), full[lo:lo + n].view(torch.int16)), \
            "layer %d differs from its flat range" % k
        sel = np.flatnonzero((sample >= lo) & (sample < lo + n))
        got[sel] = parity.take(params.view(torch.int16), sample[sel] - lo).numpy().view(np.uint16)
    assert seen == L
    parity.assert_bitwise("gathered parameters (sample)", got, expected)
    say("all %d layers gathered bit-exact" % L)
    del g, shards, full
    _free()


# -------------------------------------------------------------- re-partition
def test_repartition_ragged_state_in_bench_configuration():
    P = W.RAGGED_2000.numel
    say("re-partition: %d params, 3 fp32 arrays, 8 ranks -> 3" % P)
    src = SimulatedWorld(P, 8, n_replicas=1, alignment=128, grad_dtype=torch.bfloat16)
    dst = SimulatedWorld(P, 3, n_replicas=1, alignment=128, grad_dtype=torch.bfloat16)
    for wld in (src, dst):
        wld.grads = []
        wld.workspace = []
    _free()
    for k in range(8):
        for f, t in enumerate(src.state(k)):
            W.flat_normal(t, k * src.s, P, 1.0, ("bench-repart", f))
    for j in range(3):
        for t in dst.state(j):
            t.fill_(7.0)
    dst.repartition_from(src)
    rng = np.random.default_rng(10)
    edges = np.concatenate([np.arange(1, 8) * src.s, np.arange(1, 3) * dst.s])
    sample = np.unique(np.concatenate([rng.integers(0, P, 1 << 16, dtype=np.int64),
                                       edges - 1, edges, [0, P - 1]]))
    sample = sample[sample < P]
    for f in range(3):
        expected = parity.gather_generated(sample, 0, P, 1.0, ("bench-repart", f), torch.float32, P)
        got = np.zeros(sample.size, np.float32)
        for j in range(3):
            sel = np.flatnonzero((sample >= j * dst.s) & (sample < (j + 1) * dst.s))
            got[sel] = parity.take(dst.state(j)[f], sample[sel] - j * dst.s).numpy()
        parity.assert_bitwise("field %d (sample)" % f, got, expected)
        for j in range(3):
            lo, hi = j * dst.s, j * dst.s + dst.valid[j]
            new = dst.state(j)[f]
            for k in range(lo // src.s, (hi - 1) // src.s + 1):
                a, b = max(lo, k * src.s), min(hi, (k + 1) * src.s)
                assert torch.equal(new[a - lo:b - lo], src.state(k)[f][a - k * src.s:b - k * src.s]), \
                    "field %d rank %d differs in [%d, %d)" % (f, j, a, b)
            assert bool((new[hi - lo:] == 0).all()), "padding of rank %d not zero" % j
    say("re-partition matches")
    del src, dst
    _free()


# ---------------------------------------------- accumulation before the reduce
def test_local_accumulation_13b_in_bench_configuration():
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s, P, K = part.shard_numel, part.padded_numel, 4
    n = Z.zero_partition_valid_numel(part, 0)
    gkey = lambda i: W.grad_key(w, 0, 0, i)
    say("local accumulation 13B/8: %d-element gradient x %d, 7 fp32 peer slices" % (P, K))
    own = torch.empty(P, dtype=torch.bfloat16, device="cuda")
    W.flat_normal(own, 0, w.numel, w.grad_sigma, gkey(0))
    acc = torch.full((P,), 3.0, dtype=torch.float32, device="cuda")
    peers = []
    for i in range(1, w.world_size):
        x = torch.empty(s, dtype=torch.float32, device="cuda")
        W.flat_normal(x, 0, w.numel, w.grad_sigma * K, gkey(i))
        peers.append(x)
    master = torch.empty(s, dtype=torch.float32, device="cuda")
    W.flat_normal(master, 0, w.numel, w.master_sigma, W.master_key(w, 0))
    m = torch.zeros(s, dtype=torch.float32, device="cuda")
    v = torch.zeros(s, dtype=torch.float32, device="cuda")
    full = torch.full((P,), parity.CANARY, dtype=torch.int16, device="cuda")
    ws = torch.empty(Z.zero_shard_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    hp = Hyper(lr=w.lr, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm)
    for j in range(K):
        Z.zero_accumulate_local(own, acc, j == 0)
    info = Z.zero_shard_step(Z.StepArgs(
        world_size=w.world_size, rank=0, shard_numel=s, valid_numel=n,
        replica_grads=[acc[:s]] + peers, master=master, exp_avg=m, exp_avg_sq=v,
        full_params=full.view(torch.bfloat16), workspace=ws, lr=hp.lr,
        weight_decay=hp.weight_decay, step=1, max_grad_norm=hp.max_grad_norm), want_info=True)

    # window sums over the whole gradient, at a sample
    rng = np.random.default_rng(11)
    wsample = np.unique(np.concatenate([rng.integers(0, w.numel, 1 << 16, dtype=np.int64),
                                        np.arange(w.numel - 5, P, dtype=np.int64)]))
    codes = parity.gather_generated(wsample, 0, w.numel, w.grad_sigma, gkey(0), torch.bfloat16, P)
    parity.assert_bitwise("window sums (sample)", parity.take(acc, wsample).numpy(),
                          oracle.accumulate_local([codes] * K, oracle.BF16))

    # the oracle's reduce of the shard over every element, chunk by chunk
    say("oracle: window sums and fp32 reduce over %d elements" % n)
    sample = parity.structural_sample(n, rng)
    inv = oracle.inv_scale(1.0)
    ss, of = 0.0, 0
    o_g_full = np.empty(n, np.float32)
    vals = [np.zeros(sample.size, np.float32) for _ in range(w.world_size)]
    buf16 = torch.empty(W.CHUNK, dtype=torch.bfloat16, device="cuda")
    buf32 = torch.empty(W.CHUNK, dtype=torch.float32, device="cuda")
    for a in range(0, n, W.CHUNK):
        b = min(n, (a // W.CHUNK + 1) * W.CHUNK)
        W.flat_normal(buf16[:b - a], a, w.numel, w.grad_sigma, gkey(0))
        own_codes = buf16[:b - a].view(torch.int16).cpu().numpy().view(np.uint16)
        reps = [oracle.accumulate_local([own_codes] * K, oracle.BF16)]
        for i in range(1, w.world_size):
            W.flat_normal(buf32[:b - a], a, w.numel, w.grad_sigma * K, gkey(i))
            reps.append(buf32[:b - a].cpu().numpy())
        o_g_full[a:b], ss, of = oracle.reduce_f32(reps, inv, ss, of)
        sel = (sample >= a) & (sample < b)
        for i in range(w.world_size):
            vals[i][sel] = reps[i][sample[sel] - a]
        if (a // W.CHUNK) % 8 == 0:
            say("  [%d, %d) done" % (a, b))
    assert of == 0 and info.overflow == 0
    applies, onorm, ocoef = oracle.clip(ss, hp.max_grad_norm)
    assert bool(info.clipped) == applies
    assert abs(info.norm - onorm) <= parity.RTOL_NORM * onorm, (info.norm, onorm)
    o_g, _, _ = oracle.reduce_f32(vals, inv)
    gdev = ws[:4 * s].view(torch.float32)
    parity.assert_bitwise("reduced grad (sample)", parity.take(gdev, sample).numpy(), o_g)
    o_p = parity.gather_generated(sample, 0, w.numel, w.master_sigma, W.master_key(w, 0),
                                  torch.float32, n).copy()
    o_m = np.zeros(sample.size, np.float32)
    o_v = np.zeros(sample.size, np.float32)
    oracle.adamw(o_g, o_p, o_m, o_v, ocoef, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, 1)
    for name, dev_t, ref in (("master", master, o_p), ("exp_avg", m, o_m), ("exp_avg_sq", v, o_v)):
        parity.assert_rel("%s (sample)" % name, parity.take(dev_t, sample).numpy(), ref,
                          parity.RTOL_STATE)
    parity.assert_cast("cast (sample)", parity.take(full, sample).numpy().view(np.uint16),
                       oracle.f32_to_bf16(o_p))
    # every element: the oracle's reduced gradient, AdamW and cast
    say("the oracle's update over all %d elements" % n)
    st = parity.check_every_element(
        "local accumulation", o_g_full, (master, m, v),
        lambda a, b: parity.gen_host(a, b, w.numel, w.master_sigma, W.master_key(w, 0)), ocoef,
        hp, (1,), oracle.BF16, full=full, full_off=0, grad=gdev, log=say)
    assert st["elements"] == n
    del o_g_full
    for a, b in _chunked(P - s, 1 << 30):
        assert bool((full[s + a:s + b] == parity.CANARY).all()), "write outside the slice"
    say("local accumulation matches: norm %.6f (oracle %.6f)" % (info.norm, onorm))
    del own, acc, peers, master, m, v, full, ws, buf16, buf32
    _free()


# ---------------------------------------------- accumulation per micro-batch
def test_reduced_accumulation_13b_in_bench_configuration():
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s, K = part.shard_numel, 4
    n = Z.zero_partition_valid_numel(part, 0)
    nrep = w.world_size
    gkey = lambda i: W.grad_key(w, 0, 0, i)
    say("accumulation per micro-batch 13B/8: s=%d, %d replicas, window of %d" % (s, nrep, K))
    grads = []
    for i in range(nrep):
        g = torch.empty(s, dtype=torch.bfloat16, device="cuda")
        W.flat_normal(g, 0, w.numel, w.grad_sigma, gkey(i))
        grads.append(g)
    master = torch.empty(s, dtype=torch.float32, device="cuda")
    W.flat_normal(master, 0, w.numel, w.master_sigma, W.master_key(w, 0))
    m = torch.zeros(s, dtype=torch.float32, device="cuda")
    v = torch.zeros(s, dtype=torch.float32, device="cuda")
    full = torch.full((part.padded_numel,), parity.CANARY, dtype=torch.int16, device="cuda")
    ws = torch.empty(Z.zero_shard_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    hp = Hyper(lr=w.lr, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm)

    def args(accumulate):
        return Z.StepArgs(world_size=w.world_size, rank=0, shard_numel=s, valid_numel=n,
                          replica_grads=grads, master=master, exp_avg=m, exp_avg_sq=v,
                          full_params=full.view(torch.bfloat16), workspace=ws, lr=hp.lr,
                          weight_decay=hp.weight_decay, step=1, max_grad_norm=hp.max_grad_norm,
                          accumulate=accumulate)

    # the bench's calls: K - 1 passes into the slice, then the step that adds the last
    for j in range(K - 1):
        Z.zero_shard_accumulate(args(j > 0))
    info = Z.zero_shard_step(args(True), want_info=True)

    # the oracle's window over every element of the shard, chunk by chunk in
    # index order; each chunk's last micro-batch carries the running norm
    say("oracle: %d reduces over %d elements" % (K, n))
    rng = np.random.default_rng(12)
    sample = parity.structural_sample(n, rng)
    inv = oracle.inv_scale(1.0)
    ss, of = 0.0, 0
    o_g_full = np.empty(n, np.float32)
    codes = [np.empty(sample.size, np.uint16) for _ in range(nrep)]
    gens = [parity.gen_chunks(0, n, w.numel, w.grad_sigma, gkey(i), torch.bfloat16)
            for i in range(nrep)]
    for k, parts in enumerate(zip(*gens)):
        a, b = parts[0][0], parts[0][1]
        reps = [x[2] for x in parts]
        g_chunk, _, _ = oracle.reduce(reps, oracle.BF16, inv)
        for j in range(1, K):
            last = j == K - 1
            r_ss, r_of = oracle.reduce_accumulate(reps, oracle.BF16, inv, g_chunk,
                                                  ss if last else 0.0, of if last else 0)
            if last:
                ss, of = r_ss, r_of
        o_g_full[a:b] = g_chunk
        sel = (sample >= a) & (sample < b)
        for i in range(nrep):
            codes[i][sel] = reps[i][sample[sel] - a]
        if k % 8 == 0:
            say("  [%d, %d) done" % (a, b))
    assert of == 0 and info.overflow == 0
    applies, onorm, ocoef = oracle.clip(ss, hp.max_grad_norm)
    assert bool(info.clipped) == applies
    assert abs(info.norm - onorm) <= parity.RTOL_NORM * onorm, (info.norm, onorm)

    # at the sample: the window's reduced gradient, AdamW and the cast
    o_g, _, _ = oracle.reduce(codes, oracle.BF16, inv)
    for j in range(1, K):
        oracle.reduce_accumulate(codes, oracle.BF16, inv, o_g)
    gdev = ws[:4 * s].view(torch.float32)
    parity.assert_bitwise("window's reduced grad (sample)", parity.take(gdev, sample).numpy(), o_g)
    o_p = parity.gather_generated(sample, 0, w.numel, w.master_sigma, W.master_key(w, 0),
                                  torch.float32, n).copy()
    o_m = np.zeros(sample.size, np.float32)
    o_v = np.zeros(sample.size, np.float32)
    oracle.adamw(o_g, o_p, o_m, o_v, ocoef, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, 1)
    for name, dev_t, ref in (("master", master, o_p), ("exp_avg", m, o_m), ("exp_avg_sq", v, o_v)):
        parity.assert_rel("%s (sample)" % name, parity.take(dev_t, sample).numpy(), ref,
                          parity.RTOL_STATE)
    parity.assert_cast("cast (sample)", parity.take(full, sample).numpy().view(np.uint16),
                       oracle.f32_to_bf16(o_p))

    # every element: the oracle's window, AdamW and cast; nothing written
    # outside the rank's slice
    say("the oracle's update over all %d elements" % n)
    st = parity.check_every_element(
        "accumulation per micro-batch", o_g_full, (master, m, v),
        lambda a, b: parity.gen_host(a, b, w.numel, w.master_sigma, W.master_key(w, 0)), ocoef,
        hp, (1,), oracle.BF16, full=full, full_off=0, grad=gdev, log=say)
    assert st["elements"] == n
    del o_g_full
    for a, b in _chunked(part.padded_numel - s, 1 << 30):
        assert bool((full[s + a:s + b] == parity.CANARY).all()), "write outside the slice"
    say("accumulation per micro-batch matches: norm %.6f (oracle %.6f)" % (info.norm, onorm))
    del grads, master, m, v, full, ws
    _free()


# --------------------------------------------------------- two state sets
def test_two_state_sets_13b_equal_in_place():
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s = part.shard_numel
    n = Z.zero_partition_valid_numel(part, 0)
    say("two state sets 13B/8: s=%d" % s)
    grads = []
    for i in range(w.world_size):
        g = torch.empty(s, dtype=torch.bfloat16, device="cuda")
        W.flat_normal(g, 0, w.numel, w.grad_sigma, W.grad_key(w, 0, 0, i))
        grads.append(g)
    a_p = torch.empty(s, dtype=torch.float32, device="cuda")
    W.flat_normal(a_p, 0, w.numel, w.master_sigma, W.master_key(w, 0))
    # a state with nonzero moments: one step in place first
    a_m = torch.zeros(s, dtype=torch.float32, device="cuda")
    a_v = torch.zeros(s, dtype=torch.float32, device="cuda")
    full = torch.zeros(part.padded_numel, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(Z.zero_shard_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    hp = Hyper(lr=w.lr, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm)

    def args(t, p, m, v, out=None):
        a = Z.StepArgs(world_size=w.world_size, rank=0, shard_numel=s, valid_numel=n,
                       replica_grads=grads, master=p, exp_avg=m, exp_avg_sq=v,
                       full_params=full, workspace=ws, lr=hp.lr, weight_decay=hp.weight_decay,
                       step=t, max_grad_norm=hp.max_grad_norm)
        if out is not None:
            a.master_out, a.exp_avg_out, a.exp_avg_sq_out = out
        return a

    Z.zero_shard_step(args(1, a_p, a_m, a_v))
    # step 2 from set A into set B, then the same step in place on A
    b = tuple(torch.full((s,), 7.0, dtype=torch.float32, device="cuda") for _ in range(3))
    i1 = Z.zero_shard_step(args(2, a_p, a_m, a_v, b), want_info=True)
    cast_b = full[:s].clone()
    full[:s].zero_()
    i2 = Z.zero_shard_step(args(2, a_p, a_m, a_v), want_info=True)
    assert i1.overflow == 0 and (i1.norm, i1.coef) == (i2.norm, i2.coef)
    for name, x, y in zip(("master", "exp_avg", "exp_avg_sq"), b, (a_p, a_m, a_v)):
        for lo, hi in _chunked(n):
            assert torch.equal(x[lo:hi].view(torch.int32), y[lo:hi].view(torch.int32)), \
                "%s differs in [%d, %d)" % (name, lo, hi)
        assert bool((x[n:] == 7.0).all()), "%s: the other set's padding was written" % name
    for lo, hi in _chunked(s):
        assert torch.equal(cast_b[lo:hi].view(torch.int16), full[lo:hi].view(torch.int16))
    # and both equal the oracle's two steps, every element
    oref = parity.shard13b_reference(log=say)
    assert (bool(i1.clipped), i1.overflow) == (oref["applies"], 0)
    assert abs(i1.norm - oref["norm"]) <= parity.RTOL_NORM * oref["norm"]
    say("the oracle's two steps over all %d elements" % n)
    st = parity.check_every_element("second state set after step 2", oref["g_full"], b,
                                    oref["init_master"], oref["coef"], hp, (1, 2), oracle.BF16,
                                    full=full.view(torch.int16), full_off=0, log=say)
    assert st["elements"] == n
    say("two state sets equal in place and the oracle: norm %.6f" % i1.norm)
    del grads, a_p, a_m, a_v, b, full, ws, cast_b
    _free()
