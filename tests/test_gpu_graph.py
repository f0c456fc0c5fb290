"""The step inside a HIP graph, through the C ABI.

zero_shard_step without a result read-back queues four kernels and
nothing else (no allocation, no host wait, no memset), and the skip
decision is taken on the device, so the whole step can be captured once
and replayed.  A captured step is replayed 4 times, each time on new
gradients copied into the captured input buffers and with eager work and
synchronisations between replays (one replay is poisoned and must skip);
every replay must equal an eager world's step bit for bit.  The step's
scalars (t, lr, loss scale, ...) are kernel arguments fixed at capture, so
every replay here is a step at t = 1 and is compared with an eager step at
t = 1; a caller whose t or scale changes re-captures.
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


def test_captured_step_replays_equal_eager_steps():
    numel, R = 400_009, 4
    print("graph capture of zero_shard_step", flush=True)
    hp = Hyper(loss_scale=2.0**12)
    eager = SimulatedWorld(numel, 1, n_replicas=R, alignment=128, grad_dtype=torch.float16)
    graph_w = SimulatedWorld(numel, 1, n_replicas=R, alignment=128, grad_dtype=torch.float16)
    for w in (eager, graph_w):
        W.flat_normal(w.master[0], 0, numel, 0.02, ("graph-m",))
    # the step number is baked into the captured launch: every replay is t = 1
    args = graph_w.rank_args(0, hp, 1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                   # warm the library on the side stream
        Z.zero_shard_step(args, stream=s)
    torch.cuda.synchronize()
    for w in (eager, graph_w):                   # restart both from the same state
        W.flat_normal(w.master[0], 0, numel, 0.02, ("graph-m",))
        w.exp_avg[0].zero_()
        w.exp_avg_sq[0].zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Z.zero_shard_step(args)
    for rep in range(4):
        for i in range(R):
            W.flat_normal(eager.grads[i], 0, numel, 1e-3, ("graph", rep, i), scale=hp.loss_scale)
            graph_w.grads[i].copy_(eager.grads[i])
        if rep == 2:
            for w in (eager, graph_w):
                W.plant(w.grads[3], W.Poison(rep, 3, numel // 2, 1))
        eager.step(hp, 1)
        g.replay()
        _ = torch.ones(1000, device="cuda").sum().item()      # eager work and a sync between
        res = eager.result()
        assert bool(res.overflow) == (rep == 2)
        for f, name in enumerate(("master", "exp_avg", "exp_avg_sq")):
            parity.assert_bitwise("replay %d %s" % (rep, name),
                                  parity.f32(graph_w.state(0)[f][:numel]),
                                  parity.f32(eager.state(0)[f][:numel]))
        parity.assert_bitwise("replay %d params" % rep, parity.u16(graph_w.full_params),
                              parity.u16(eager.full_params))


@pytest.mark.parametrize("mode", ["reduced", "local"])
def test_captured_accumulation_window_replays_equal_eager(mode):
    # A whole window of K = 3 micro-batches captured once: either pass 1 per
    # micro-batch into the rank's slice (zero_shard_accumulate, then the
    # step with accumulate = 1), or the fp32 window sums of every replica
    # (zero_accumulate_local) and a step over them.  Each replay runs on new
    # micro-batch gradients and must equal the eager window bit for bit.
    numel, R, K = 300_007, 4, 3
    print("graph capture of an accumulation window (%s)" % mode, flush=True)
    hp = Hyper()
    local = mode == "local"
    gdt = torch.float32 if local else torch.bfloat16
    eager = SimulatedWorld(numel, 1, n_replicas=R, alignment=128, grad_dtype=gdt,
                           param_dtype=torch.bfloat16)
    graph_w = SimulatedWorld(numel, 1, n_replicas=R, alignment=128, grad_dtype=gdt,
                             param_dtype=torch.bfloat16)
    # the captured window reads its micro-batches from fixed buffers
    micro = [[torch.zeros(graph_w.padded, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
             for _ in range(K)]
    emicro = [[torch.zeros_like(x) for x in mb] for mb in micro]

    def window(w, mbufs, stream=None):
        for j in range(K):
            if local:
                w.accumulate_local(mbufs[j], first=j == 0, stream=stream)
            else:
                for i in range(R):
                    w.grads[i].copy_(mbufs[j][i])
                if j < K - 1:
                    w.accumulate(hp, first=j == 0, stream=stream)
        if local:
            Z.zero_shard_step(w.rank_args(0, hp, 1), stream=stream)
        else:
            Z.zero_shard_step(w.rank_args(0, hp, 1, accumulate=True), stream=stream)

    def reset():
        for w in (eager, graph_w):
            W.flat_normal(w.master[0], 0, numel, 0.02, ("graph-acc-m",))
            w.exp_avg[0].zero_()
            w.exp_avg_sq[0].zero_()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                   # warm up on a side stream
        window(graph_w, micro, stream=s)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        window(graph_w, micro)
    for rep in range(3):
        for j in range(K):
            for i in range(R):
                W.flat_normal(emicro[j][i], 0, numel, 1e-3, ("graph-acc", rep, j, i))
                micro[j][i].copy_(emicro[j][i])
        window(eager, emicro)
        g.replay()
        _ = torch.ones(1000, device="cuda").sum().item()      # eager work and a sync between
        for f, name in enumerate(("master", "exp_avg", "exp_avg_sq")):
            parity.assert_bitwise("%s replay %d %s" % (mode, rep, name),
                                  parity.f32(graph_w.state(0)[f][:numel]),
                                  parity.f32(eager.state(0)[f][:numel]))
        parity.assert_bitwise("%s replay %d params" % (mode, rep), parity.u16(graph_w.full_params),
                              parity.u16(eager.full_params))


def _scalars_bytes(sc):
    return torch.frombuffer(bytearray(bytes(sc)), dtype=torch.uint8)


@pytest.mark.parametrize("entry,layout", [("step", Z.ZERO_STATE_SEPARATE),
                                          ("noalloc", Z.ZERO_STATE_SEPARATE),
                                          ("step", Z.ZERO_STATE_TILED)])
def test_captured_step_with_device_scalars_serves_every_step(entry, layout):
    # One capture of a step whose scalars live in a device buffer
    # (zero_step_args.scalars), replayed for 6 consecutive training steps:
    # before each replay the host refills the buffer with zero_step_scalars
    # for that step's t (advanced only after applied steps), learning rate
    # (a decaying schedule) and fp16 loss scale (driven by the dynamic
    # scaler; one replay is poisoned and must skip and halve it).  Every
    # replay must equal an eager step with the same scalars as launch
    # arguments, bit for bit, and the eager run must match the oracle.
    numel, R = 400_009, 4
    print("graph capture with device scalars (%s, layout %d)" % (entry, layout), flush=True)
    eager = SimulatedWorld(numel, 1, n_replicas=R, alignment=128, grad_dtype=torch.float16,
                           state_layout=layout)
    graph_w = SimulatedWorld(numel, 1, n_replicas=R, alignment=128, grad_dtype=torch.float16,
                             state_layout=layout)
    scal_dev = torch.zeros(64, dtype=torch.uint8, device="cuda")
    sc_lib = Z.zero_loss_scaler_init(12, 2, 1, 1.0)
    o_sc = oracle.LossScaler(12, 2, 1, 1.0)

    def hyper(t, scale):
        return Hyper(lr=1e-3 * 0.8 ** (t - 1), loss_scale=scale)

    def graph_args(t, scale):
        a = graph_w.rank_args(0, hyper(t, scale), t)
        a.scalars = scal_dev
        if entry == "noalloc":
            a.workspace = None
        return a

    def call(a, stream=None):
        if entry == "noalloc":
            Z.zero_shard_step_noalloc(a, stream=stream)
        else:
            Z.zero_shard_step(a, stream=stream)

    def reset():
        for w in (eager, graph_w):
            m0 = torch.empty(w.s, dtype=torch.float32, device="cuda")
            W.flat_normal(m0, 0, numel, 0.02, ("graph-sc-m",))
            w.set_state(0, m0)                   # zero moments
            w.full_params.zero_()

    scal_dev.copy_(_scalars_bytes(Z.zero_step_scalars(graph_args(1, sc_lib.scale))))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                   # warm the library on the side stream
        call(graph_args(1, sc_lib.scale), stream=s)
    torch.cuda.synchronize()
    reset()
    o_p = parity.f32(eager.separate_state(0)[0])[:numel].copy()
    o_m = np.zeros(numel, np.float32)
    o_v = np.zeros(numel, np.float32)
    o_full = np.zeros(numel, np.uint16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):                    # captured once, with t = 1's launch arguments
        call(graph_args(1, sc_lib.scale))
    t = 1
    skipped = 0
    for rep in range(6):
        scale = sc_lib.scale
        for i in range(R):
            W.flat_normal(eager.grads[i], 0, numel, 1e-3, ("graph-sc", rep, i), scale=scale)
        if rep == 3:
            W.plant(eager.grads[2], W.Poison(rep, 2, numel // 5, 2))
        for i in range(R):
            graph_w.grads[i].copy_(eager.grads[i])
        reps = [parity.u16(x)[:numel] for x in eager.grads]
        # this step's scalars into the captured buffer, then the replay
        scal_dev.copy_(_scalars_bytes(Z.zero_step_scalars(graph_args(t, scale))))
        g.replay()
        eager.step(hyper(t, scale), t)
        res = eager.result()
        _ = torch.ones(1000, device="cuda").sum().item()      # eager work and a sync between
        info = oracle.step(reps, oracle.FP16, numel, 1, 1, [o_p], [o_m], [o_v], o_full,
                           oracle.Hyper(lr=hyper(t, scale).lr, loss_scale=scale), t)
        assert bool(res.overflow) == info.overflow == (rep == 3)
        for f, name in enumerate(("master", "exp_avg", "exp_avg_sq")):
            got = parity.f32(graph_w.separate_state(0)[f][:numel])
            parity.assert_bitwise("replay %d %s vs eager" % (rep, name), got,
                                  parity.f32(eager.separate_state(0)[f][:numel]))
            parity.assert_rel("replay %d %s vs oracle" % (rep, name), got, (o_p, o_m, o_v)[f],
                              parity.RTOL_STATE)
        parity.assert_bitwise("replay %d params" % rep, parity.u16(graph_w.full_params),
                              parity.u16(eager.full_params))
        skip = Z.zero_loss_scaler_update(sc_lib, bool(res.overflow))
        assert skip == o_sc.update(info.overflow) and sc_lib.scale == o_sc.scale
        if skip:
            skipped += 1
        else:
            t += 1
    assert skipped == 1 and t == 6 and sc_lib.scale != 2.0**12   # the scale moved
