"""Benchmark of the ZeRO sharded-optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload shard13b]

Default workload: a 13B-parameter flat model over 8 data-parallel ranks;
this GPU is rank 0 and owns a 1,625,000,064-element shard.  Eight bf16
replica gradient slices, fp32 master weights and Adam moments (one set,
updated in place; --state-buffers 2 alternates two), and the
13,000,000,512-element bf16 full parameter buffer sit in HBM before timing
starts.  One step = replica reduce (+ unscale, inf/nan flag, partial norm,
then the fold of the block partials), combine (norm, clip factor), AdamW +
cast into the rank's slice of the full buffer: the kernels zero_shard_step
queues, here queued by the split calls so that HIP events between them
time each kernel.

Prints one JSON line.  `value` is params updated per second (the shard's
real elements / step time); `roofline` is for the dominant kernel (the
AdamW + cast pass; in an accumulation window, the adding pass 1) against
the 8 TB/s HBM peak, with `traffic` from the committed counter record of
the same library code; `copy_ceiling` is a plain one-read, one-write copy
of one gradient slice through the library's flatten kernel, timed in the
same process, for reading `roofline.frac` against what the part streams in
practice; `cpu_baseline` is the CPU oracle timed on a bounded sample of the
same inputs on one host core.
"""
from __future__ import annotations

import argparse
import contextlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "ZeRO shard step: params updated/s + achieved HBM GB/s (% of 8 TB/s peak)"
# stage3_max_live_parameters of the pages' ZeRO-3 configuration
# ("ZeRO技术解析：大模型分布式训练的革命性突破" §3.1)
MAX_LIVE_PARAMETERS = int(1e9)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="shard13b",
                    choices=["shard13b", "ragged", "repartition", "offload", "zero3"],
                    help="shard13b: rank 0 of the 13B/8 flat model (the headline); "
                         "ragged: 2000 tensors flattened bucket by bucket, then the step of "
                         "all 8 ranks; repartition: the ragged model's optimizer state moved "
                         "from 8 ranks to 3 on the device, and one rank's checkpoint file "
                         "written and read back; offload: the 13B/8 shard with its optimizer "
                         "state in pinned host memory (pass 1 on the GPU, AdamW on the host); "
                         "zero3: the 13B model's bf16 parameters gathered layer by layer "
                         "(40 layers) from 8 rank shards with prefetch")
    ap.add_argument("--host-threads", type=int, default=0,
                    help="offload: host threads for the update (0: the library's default, "
                         "OMP_NUM_THREADS or the process's CPU affinity)")
    ap.add_argument("--chunk", type=int, default=1 << 25,
                    help="offload: elements per transfer chunk")
    ap.add_argument("--micro-batches", type=int, default=1,
                    help="shard13b: gradient-accumulation window K; each step reduces K "
                         "micro-batches (the first sets the fp32 slice, the others add to it) "
                         "before the combine and AdamW")
    ap.add_argument("--accumulation", default="reduced", choices=["reduced", "local"],
                    help="shard13b with --micro-batches K > 1: 'reduced' reduces every "
                         "micro-batch into the rank's fp32 slice (the default); 'local' "
                         "sums the rank's own full gradient over the window in fp32 first "
                         "(zero_accumulate_local) and reduces the replicas' fp32 sums once")
    ap.add_argument("--state-buffers", type=int, default=1, choices=[1, 2],
                    help="shard13b: 1 updates one fp32 state set in place (the default); "
                         "2 keeps two sets and alternates them, so pass 2 reads one and "
                         "writes the other")
    ap.add_argument("--state-layout", default="separate", choices=["separate", "tiled"],
                    help="shard13b: 'separate' keeps master, exp_avg and exp_avg_sq in three "
                         "arrays; 'tiled' keeps them in one array of 256-element tiles "
                         "(ZERO_STATE_TILED), so the update pass moves two state streams "
                         "instead of six")
    ap.add_argument("--flatten-streams", type=int, default=2,
                    help="ragged: HIP streams the 8 replicas' flatten calls are spread over "
                         "(replica i on stream i mod S, so one launch's tail overlaps the "
                         "next one's start); the step waits for all of them")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=1 << 29,
                    help="elements of the shard the CPU oracle is timed on")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="only run N torch copies of 4 GiB (counter calibration)")
    return ap.parse_args()


def kernel_hash() -> str:
    """Hash of the host and gfx950 code of the library the bench loads."""
    from zero_sharded_optimizer_step_amd import _abi, build
    return build.code_hash(_abi.LIB_PATH)


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)


def measured_traffic(workload: str):
    """Calibrated HBM bytes (FETCH_SIZE + WRITE_SIZE) of the roofline's
    kernel, over the same unit as its `achieved` figure, from the committed
    counter runs; None when absent or taken on a library whose code
    differs from the one loaded."""
    try:
        rec = json.load(open(traffic_file(workload)))
    except (OSError, ValueError):
        return None
    here = kernel_hash()
    if rec.get("library_code_sha256_16") != here or rec.get("workload") != workload:
        log("traffic: the %s counter record was taken on library code %s, this library is %s; "
            "roofline.traffic is null" % (workload, rec.get("library_code_sha256_16"), here))
        return None
    return rec.get("roofline_traffic")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workloads
def setup_shard13b(torch, Z, W, state_buffers=1, state_layout="separate"):
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s = part.shard_numel
    valid = Z.zero_partition_valid_numel(part, 0)
    dev = "cuda"
    log("allocating: 8 x %d bf16 grads, 3 x fp32 state, %d bf16 full params" % (s, part.padded_numel))
    grads = []
    for i in range(w.world_size):
        g = torch.empty(s, dtype=torch.bfloat16, device=dev)
        W.flat_normal(g, 0, w.numel, w.grad_sigma, W.grad_key(w, 0, 0, i))
        grads.append(g)
        log("  replica %d generated" % i)
    master = torch.empty(s, dtype=torch.float32, device=dev)
    W.flat_normal(master, 0, w.numel, w.master_sigma, W.master_key(w, 0))
    m = torch.zeros(s, dtype=torch.float32, device=dev)
    v = torch.zeros(s, dtype=torch.float32, device=dev)
    alt = None
    if state_layout == "tiled":
        # one tiled array holds all three; the library tiles the initial state
        tiled = torch.empty(Z.tiled_state_numel(s), dtype=torch.float32, device=dev)
        Z.zero_state_tile(master, m, v, tiled)
        torch.cuda.synchronize()
        del master, v
        master, m, v = tiled, None, None
        if state_buffers == 2:
            alt = (torch.zeros(Z.tiled_state_numel(s), dtype=torch.float32, device=dev), None, None)
    elif state_buffers == 2:
        # the second state set of the ping-pong layout
        alt = tuple(torch.zeros(s, dtype=torch.float32, device=dev) for _ in range(3))
    full = torch.zeros(part.padded_numel, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(Z.zero_shard_workspace_bytes(s), dtype=torch.uint8, device=dev)
    partials = torch.zeros(Z.zero_partials_bytes(1), dtype=torch.uint8, device=dev)
    glob = torch.zeros(256, dtype=torch.uint8, device=dev)
    return dict(w=w, s=s, valid=valid, grads=grads, master=master, m=m, v=v, alt=alt, full=full,
                ws=ws, partials=partials, glob=glob, nrep=w.world_size)


def run_shard13b(args, torch, Z, W):
    st = setup_shard13b(torch, Z, W, args.state_buffers, args.state_layout)
    layout = Z.ZERO_STATE_TILED if args.state_layout == "tiled" else Z.ZERO_STATE_SEPARATE
    w, s, valid = st["w"], st["s"], st["valid"]
    torch.cuda.synchronize()

    MB = args.micro_batches
    sets = [(st["master"], st["m"], st["v"])] + ([st["alt"]] if st["alt"] else [])

    def step_args(t, accumulate=False):
        # ping-pong: step t reads set (t - 1) % 2 and writes the other one
        src = sets[(t - 1) % len(sets)]
        a = Z.StepArgs(world_size=w.world_size, rank=0, shard_numel=s, valid_numel=valid,
                       replica_grads=st["grads"], master=src[0], exp_avg=src[1],
                       exp_avg_sq=src[2], full_params=st["full"], workspace=st["ws"],
                       lr=w.lr, weight_decay=w.weight_decay, step=t,
                       max_grad_norm=w.max_grad_norm, accumulate=accumulate,
                       state_layout=layout)
        if len(sets) == 2:
            a.master_out, a.exp_avg_out, a.exp_avg_sq_out = sets[t % 2]
        return a

    def fused_step(t):
        for j in range(MB - 1):
            Z.zero_shard_accumulate(step_args(t, accumulate=j > 0), stream)
        return Z.zero_shard_step(step_args(t, accumulate=MB > 1), stream=stream)

    stream = torch.cuda.current_stream()
    t = 1
    for _ in range(args.warmup):
        fused_step(t)
        t += 1
    torch.cuda.synchronize()
    K = args.steps
    # events: e[0] at the start, e[1 + j] after pass 1 of micro-batch j < MB - 1,
    # e[MB] after the last pass 1 and its fold, e[MB + 1] after the combine,
    # e[MB + 2] after AdamW
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(MB + 3)] for _ in range(K)]
    wall0 = time.perf_counter()
    for k in range(K):
        a = step_args(t, accumulate=MB > 1)
        e = ev[k]
        e[0].record(stream)
        for j in range(MB - 1):
            Z.zero_shard_accumulate(step_args(t, accumulate=j > 0), stream)
            e[1 + j].record(stream)
        Z.zero_shard_reduce(a, 0, st["partials"], stream)
        e[MB].record(stream)
        Z.zero_shard_combine(st["partials"], 1, w.max_grad_norm, st["glob"], stream)
        e[MB + 1].record(stream)
        Z.zero_shard_apply(a, st["glob"], stream)
        e[MB + 2].record(stream)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev[0][0].elapsed_time(ev[-1][MB + 2])
    red = sum(e[0].elapsed_time(e[MB]) for e in ev) / K
    comb = sum(e[MB].elapsed_time(e[MB + 1]) for e in ev) / K
    app = sum(e[MB + 1].elapsed_time(e[MB + 2]) for e in ev) / K
    # one adding pass 1 (micro-batches 2..MB): the accumulate calls alone when
    # there are any, else the last pass 1 with its fold
    if MB >= 3:
        add_ms = sum(e[j].elapsed_time(e[j + 1]) for e in ev for j in range(1, MB - 1)) / (K * (MB - 2))
    elif MB == 2:
        add_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    else:
        add_ms = None
    ms = total_ms / K
    per_step = sorted(e[0].elapsed_time(e[MB + 2]) for e in ev)
    log("per-step ms: " + " ".join("%.3f" % e[0].elapsed_time(e[MB + 2]) for e in ev))
    # the fused entry point over the same inputs, as a cross-check
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        fused_step(t)
        t += 1
    e1.record(stream)
    torch.cuda.synchronize()
    fused_ms = e0.elapsed_time(e1) / K
    for j in range(MB - 1):
        Z.zero_shard_accumulate(step_args(t, accumulate=j > 0), stream)
    info = Z.zero_shard_step(step_args(t, accumulate=MB > 1), want_info=True)
    nrep = st["nrep"]
    # pass 1 of the first micro-batch writes the fp32 slice; later ones also read it
    bytes_reduce = valid * (MB * 2 * nrep + 4 + (MB - 1) * 8)
    bytes_apply = valid * (16 + 14)
    bytes_step = bytes_reduce + bytes_apply
    res = dict(ms=ms, wall_ms=wall * 1e3 / K, step_ms_min=per_step[0],
               step_ms_median=per_step[len(per_step) // 2], step_ms_max=per_step[-1], fused_ms=fused_ms, reduce_ms=red, combine_ms=comb,
               apply_ms=app, add_ms=add_ms, valid=valid, bytes_step=bytes_step, bytes_reduce=bytes_reduce,
               bytes_apply=bytes_apply, norm=info.norm, clipped=info.clipped,
               overflow=info.overflow, grads=st["grads"], master0=None, st=st)
    return res


def run_shard13b_local(args, torch, Z, W):
    """The 13B/8 rank with gradient accumulation before the reduce.  Per
    step: K passes of zero_accumulate_local over the rank's own full flat
    gradient (13e9 elements, bf16 into an fp32 sum), then one reduce of its
    shard over the 8 replicas' fp32 sums (its own, plus 7 resident fp32
    slices standing in for the peers'), combine and AdamW."""
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s, P, K = part.shard_numel, part.padded_numel, args.micro_batches
    valid = Z.zero_partition_valid_numel(part, 0)
    dev = "cuda"
    log("local accumulation: %d bf16 gradient + fp32 sum, 7 fp32 peer slices" % P)
    own = torch.empty(P, dtype=torch.bfloat16, device=dev)
    W.flat_normal(own, 0, w.numel, w.grad_sigma, W.grad_key(w, 0, 0, 0))
    acc = torch.empty(P, dtype=torch.float32, device=dev)
    peers = []
    for i in range(1, w.world_size):
        x = torch.empty(s, dtype=torch.float32, device=dev)
        W.flat_normal(x, 0, w.numel, w.grad_sigma * K, W.grad_key(w, 0, 0, i))
        peers.append(x)
    master = torch.empty(s, dtype=torch.float32, device=dev)
    W.flat_normal(master, 0, w.numel, w.master_sigma, W.master_key(w, 0))
    m = torch.zeros(s, dtype=torch.float32, device=dev)
    v = torch.zeros(s, dtype=torch.float32, device=dev)
    full = torch.zeros(P, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(Z.zero_shard_workspace_bytes(s), dtype=torch.uint8, device=dev)
    partials = torch.zeros(Z.zero_partials_bytes(1), dtype=torch.uint8, device=dev)
    glob = torch.zeros(256, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step_args(t):
        return Z.StepArgs(world_size=w.world_size, rank=0, shard_numel=s, valid_numel=valid,
                          replica_grads=[acc[:s]] + peers, master=master, exp_avg=m,
                          exp_avg_sq=v, full_params=full, workspace=ws, lr=w.lr,
                          weight_decay=w.weight_decay, step=t, max_grad_norm=w.max_grad_norm)

    t = 1
    for _ in range(args.warmup):
        for j in range(K):
            Z.zero_accumulate_local(own, acc, j == 0, stream=stream)
        Z.zero_shard_step(step_args(t), stream=stream)
        t += 1
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(K + 3)] for _ in range(args.steps)]
    for k in range(args.steps):
        e = ev[k]
        e[0].record(stream)
        for j in range(K):
            Z.zero_accumulate_local(own, acc, j == 0, stream=stream)
            e[1 + j].record(stream)
        a = step_args(t)
        Z.zero_shard_reduce(a, 0, partials, stream)
        Z.zero_shard_combine(partials, 1, w.max_grad_norm, glob, stream)
        e[K + 1].record(stream)
        Z.zero_shard_apply(a, glob, stream)
        e[K + 2].record(stream)
        t += 1
    torch.cuda.synchronize()
    n = args.steps
    ms = ev[0][0].elapsed_time(ev[-1][K + 2]) / n
    first_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / n
    add_ms = (sum(e[1].elapsed_time(e[K]) for e in ev) / n / (K - 1)) if K > 1 else None
    red_ms = sum(e[K].elapsed_time(e[K + 1]) for e in ev) / n
    app_ms = sum(e[K + 1].elapsed_time(e[K + 2]) for e in ev) / n
    info = Z.zero_shard_step(step_args(t), want_info=True)
    b_first, b_add = P * 6, P * 10
    b_acc = b_first + (K - 1) * b_add
    b_red, b_app = valid * (w.world_size * 4 + 4), valid * 30
    b_step = b_acc + b_red + b_app
    dom_ms, dom_b, dom_name = (add_ms, b_add, "accumulate_local_kernel (add)") if K > 1 else \
        (first_ms, b_first, "accumulate_local_kernel (set)")
    achieved = dom_b / (dom_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": valid / (ms * 1e-3), "unit": "params/s", "n_gpus": 1,
        "steps": n, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name + ", gradient accumulation before the reduce",
                   "micro_batches": K, "shard_numel": s, "full_gradient_numel": P,
                   "world_size": 8, "replicas": 8, "grad_dtype": "bf16 (fp32 window sums)",
                   "param_dtype": "bf16"},
        "hbm_gbps": b_step / (ms * 1e-3) / 1e9, "hbm_frac": b_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "bytes_per_step": b_step,
        "kernels_ms": {"accumulate_set": first_ms, "accumulate_add": add_ms,
                       "reduce_fp32_and_fold_and_combine": red_ms, "apply": app_ms},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic("shard13b_local") if K > 1 else None},
        "reduce_gbps": b_red / (red_ms * 1e-3) / 1e9, "apply_gbps": b_app / (app_ms * 1e-3) / 1e9,
        "step_check": {"norm": info.norm, "clipped": info.clipped, "overflow": info.overflow},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        with one_host_core():
            out["cpu_baseline"] = cpu_baseline_local(args, torch, W, own, peers, K)
    print(json.dumps(out), flush=True)


@contextlib.contextmanager
def one_host_core():
    """Run the block with the calling thread pinned to one CPU of the
    process's set (the oracle is single-threaded; pinning keeps the timing
    off thread migrations), and restore the thread's CPUs after."""
    global _HOST_CPUS
    tid = threading.get_native_id()
    before = os.sched_getaffinity(tid)
    _HOST_CPUS = len(before)
    try:
        os.sched_setaffinity(tid, {min(before)})
        pinned = True
    except OSError:
        pinned = False
    try:
        yield
    finally:
        if pinned:
            os.sched_setaffinity(tid, before)


_HOST_CPUS = None      # the CPUs the thread could use before one_host_core pinned it


def cpu_record(n, dt, sample, total):
    """A `cpu_baseline` entry: the oracle's rate over a sample of n of the
    workload's `total` params (the timed region covers those n only)."""
    mine = os.sched_getaffinity(threading.get_native_id())
    where = "pinned to CPU %d" % min(mine) if len(mine) == 1 else "unpinned"
    return dict(value=n / dt, unit="params/s", cores=1, kind="oracle",
                sample="%s; one host thread of %s (%d CPUs available, %s), %.1f s"
                       % (sample, host_cpu(), _HOST_CPUS or len(mine), where, dt),
                sample_elements=int(n), workload_elements=int(total),
                sample_fraction=float(n) / float(total) if total else 1.0, seconds=dt)


def host_u16(torch, t):
    import numpy as np
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def initial_masters(torch, W, w, n):
    """The 13B/8 rank's first n initial masters, regenerated on the device
    (the timed steps changed the device copy)."""
    mdev = torch.empty(n, dtype=torch.float32, device="cuda")
    W.flat_normal(mdev, 0, w.numel, w.master_sigma, W.master_key(w, 0))
    return mdev.cpu().numpy()


def cpu_baseline_shard13b(args, torch, W, grads, micro_batches=1):
    """The oracle on the first n elements of the same inputs: the 8-replica
    reduce (once per micro-batch of the window: the first sets the fp32
    slice, the others add to it, over the same gradients as the GPU run),
    clip (norm of the sample), AdamW and bf16 cast."""
    import numpy as np
    import oracle
    w = W.SHARD_13B_OF_8
    n = min(args.cpu_sample // (2 if micro_batches > 1 else 1), grads[0].numel())
    reps = [host_u16(torch, g[:n]) for g in grads]
    p, m, v = [initial_masters(torch, W, w, n)], [np.zeros(n, np.float32)], [np.zeros(n, np.float32)]
    full = np.zeros(n, np.uint16)
    hp = oracle.Hyper(lr=w.lr, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm)
    t0 = time.perf_counter()
    oracle.step_accumulated([reps] * micro_batches, oracle.BF16, n, 1, 8, p, m, v, full, hp, 1)
    dt = time.perf_counter() - t0
    what = "reduce" if micro_batches == 1 else "%d reduces (set, then add)" % micro_batches
    return cpu_record(n, dt, "first %d of the %d elements of rank 0's shard (8 bf16 replicas): "
                             "%s, clip, AdamW, bf16 cast" % (n, grads[0].numel(), what),
                      grads[0].numel())


def cpu_baseline_local(args, torch, W, own, peers, K):
    """The oracle on a proportional sample of the accumulation-before-the-
    reduce leg: for n shard elements, the window sum of 8n elements of the
    rank's own gradient (K micro-batches, the same gradient each time as on
    the GPU), the 8-way fp32 reduce of its first n sums and the peers'
    slices, clip, AdamW and bf16 cast."""
    import numpy as np
    import oracle
    w = W.SHARD_13B_OF_8
    n = min(args.cpu_sample // 2, peers[0].numel())
    g_own = host_u16(torch, own[:8 * n])
    peer = [x[:n].cpu().numpy() for x in peers]
    p, m, v = initial_masters(torch, W, w, n), np.zeros(n, np.float32), np.zeros(n, np.float32)
    t0 = time.perf_counter()
    acc = oracle.accumulate_local([g_own] * K, oracle.BF16)
    g, ss, of = oracle.reduce_f32([acc[:n]] + peer, oracle.inv_scale(1.0))
    _, _, coef = oracle.clip(ss, w.max_grad_norm)
    if not of:
        oracle.adamw(g, p, m, v, coef, w.lr, 0.9, 0.999, 1e-8, w.weight_decay, 1)
    oracle.to_low_precision(p, oracle.BF16)
    dt = time.perf_counter() - t0
    return cpu_record(n, dt, "%d of the %d shard elements: the fp32 window sum of %d elements "
                             "of the rank's own bf16 gradient over %d micro-batches, the 8-way "
                             "fp32 reduce, clip, AdamW, bf16 cast"
                      % (n, peers[0].numel(), 8 * n, K), peers[0].numel())


def cpu_baseline_ragged(args, torch, W, r):
    """The oracle on the first tensors of the ragged workload, up to about
    `cpu_sample` / 2 params: each of the 8 replicas' tensors flattened into
    its flat buffer (contiguous gradients), then the step of all 8 ranks of
    that smaller flat model (reduce, clip, AdamW, bf16 cast)."""
    import numpy as np
    import oracle
    w = W.RAGGED_2000
    slots, pools = r["slots"], r["pools"]
    T, n = 0, 0
    while T < len(slots) and (T == 0 or n + slots[T].numel <= args.cpu_sample // 2):
        n += slots[T].numel
        T += 1
    s, padded, _ = oracle.partition(n, w.world_size, w.alignment)
    tensors = [[host_u16(torch, pool[x.offset + k + 1:x.offset + k + 1 + x.numel])
                for k, x in enumerate(slots[:T])] for pool in pools]
    rng = np.random.default_rng(0)
    p = [(rng.standard_normal(s) * w.master_sigma).astype(np.float32) for _ in range(w.world_size)]
    m = [np.zeros(s, np.float32) for _ in range(w.world_size)]
    v = [np.zeros(s, np.float32) for _ in range(w.world_size)]
    full = np.zeros(padded, np.uint16)
    hp = oracle.Hyper(lr=w.lr, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm)
    t0 = time.perf_counter()
    flats = [oracle.flatten(tt, int(2e8), padded) for tt in tensors]
    oracle.step(flats, oracle.BF16, n, w.world_size, w.alignment, p, m, v, full, hp, 1)
    dt = time.perf_counter() - t0
    return cpu_record(n, dt, "the first %d of the %d tensors (%d params): 8 replicas flattened, "
                             "then the step of 8 ranks (reduce, clip, AdamW, bf16 cast)"
                      % (T, len(slots), n), w.numel)


def cpu_baseline_repartition(args, torch, src_world):
    """The oracle re-cutting three fp32 state arrays of a 4 x `cpu_sample`-
    param model (about the whole ragged model) from 8 ranks to 3, the slices
    taken from the device state."""
    import oracle
    n = min(4 * args.cpu_sample, src_world.s * 8)
    s, _, valid = oracle.partition(n, 8, 128)
    arrays = [[src_world.state(k)[f][:s].cpu().numpy() for k in range(8)] for f in range(3)]
    t0 = time.perf_counter()
    for sl in arrays:
        oracle.repartition(sl, n, 8, 128, 3, 128)
    dt = time.perf_counter() - t0
    return cpu_record(n, dt, "master, exp_avg and exp_avg_sq of a %d-param model re-partitioned "
                             "from 8 ranks to 3" % n, src_world.numel)


def cpu_baseline_zero3(args, torch, shards):
    """The oracle gathering the first 8 x `cpu_sample` params of a model
    sharded over 8 ranks from their shards (slices of the device shards)."""
    import oracle
    n = min(8 * args.cpu_sample, shards[0].numel() * 8)
    s, _, _ = oracle.partition(n, 8, 128)
    host = [host_u16(torch, x[:s]) for x in shards]
    t0 = time.perf_counter()
    oracle.gather(host, n, 8, 128, 0, n)
    dt = time.perf_counter() - t0
    return cpu_record(n, dt, "%d bf16 params gathered from 8 rank shards" % n,
                      shards[0].numel() * len(shards))


def host_cpu() -> str:
    """The host's CPU model, from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "an unknown CPU"


def run_ragged(args, torch, Z, W):
    """The ragged workload: every replica's 2000 per-tensor gradients (at odd
    offsets of one pool) flattened bucket by bucket into its flat buffer,
    then the step of all 8 ranks (reduce per rank, one combine, AdamW +
    cast per rank).  One step = both; HIP events split them."""
    from zero_sharded_optimizer_step_amd import _abi
    from zero_sharded_optimizer_step_amd.world import Hyper, SimulatedWorld
    w = W.RAGGED_2000
    sizes = list(w.tensor_sizes)
    P, N = w.numel, w.world_size
    slots, buckets = Z.zero_bucket_plan(sizes, int(2e8))
    world = SimulatedWorld(P, N, alignment=w.alignment, grad_dtype=torch.bfloat16)
    padded = world.padded
    log("ragged: %d tensors, %d params, %d buckets; generating 8 replicas" % (len(sizes), P,
                                                                           len(buckets)))
    pools, calls = [], []
    ref = torch.empty(padded, dtype=torch.bfloat16, device="cuda")
    # tensor k sits at pool offset (its flat offset) + k + 1, so sources
    # start at odd element offsets; the pool is filled a generator chunk at
    # a time, each flat element j going to j + k(j) + 1
    starts = torch.tensor([x.offset for x in slots], dtype=torch.int64, device="cuda")
    for i in range(N):
        W.flat_normal(ref, 0, P, w.grad_sigma, W.grad_key(w, 0, 0, i))
        pool = torch.empty(P + len(sizes) + 8, dtype=torch.bfloat16, device="cuda")
        for a in range(0, P, W.CHUNK):
            j = torch.arange(a, min(P, a + W.CHUNK), dtype=torch.int64, device="cuda")
            pool[j + torch.searchsorted(starts, j, right=True)] = ref[a:a + j.numel()]
            del j
        ptrs = [pool[x.offset + k + 1:].data_ptr() for k, x in enumerate(slots)]
        pools.append(pool)
        for bi, b in enumerate(buckets):
            sl = slots[b.first_tensor:b.first_tensor + b.n_tensors]
            arr = (_abi.zero_tensor_slot_t * len(sl))(*sl)
            parr = (_abi.vp * len(sl))(*ptrs[b.first_tensor:b.first_tensor + b.n_tensors])
            flat_numel = padded if bi == len(buckets) - 1 else b.end
            calls.append((i, arr, len(sl), parr, world.grads[i].data_ptr(), flat_numel))
    del ref
    for k, r in enumerate(world.ranks):
        W.flat_normal(world.master[k], r * world.s, P, w.master_sigma, W.master_key(w, 0))
    hp = Hyper(lr=w.lr, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm)
    L = Z.lib()
    stream = torch.cuda.current_stream()
    # replica i's calls go to stream i mod S; side streams start after the
    # main stream's earlier work and the main stream waits for them
    S = max(1, args.flatten_streams)
    streams = [stream] + [torch.cuda.Stream() for _ in range(S - 1)]

    def flatten_all():
        if S > 1:
            start = torch.cuda.Event()
            start.record(stream)
            for st in streams[1:]:
                st.wait_event(start)
        for i, arr, n, parr, dst, fn in calls:
            Z.check(L.zero_bucket_flatten(arr, n, parr, Z.ZERO_BF16, dst, fn,
                                          streams[i % S].cuda_stream), "zero_bucket_flatten")
        for st in streams[1:]:
            done = torch.cuda.Event()
            done.record(st)
            stream.wait_event(done)

    t = 1
    for _ in range(args.warmup):
        flatten_all()
        world.step(hp, t, stream)
        t += 1
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for k in range(K):
        ev[k][0].record(stream)
        flatten_all()
        ev[k][1].record(stream)
        world.step(hp, t, stream)
        ev[k][2].record(stream)
        t += 1
    torch.cuda.synchronize()
    flat_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    step_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    res = world.result()
    return dict(P=P, N=N, s=world.s, flat_ms=flat_ms, step_ms=step_ms,
                ms=ev[0][0].elapsed_time(ev[-1][2]) / K, n_buckets=len(buckets),
                norm=res.norm, clipped=res.clipped, overflow=res.overflow,
                slots=slots, pools=pools)


def report_ragged(args, r, W, torch):
    P, N = r["P"], r["N"]
    flat_bytes = N * P * 4                   # each replica: 2 B read + 2 B written per element
    step_bytes = P * (2 * N + 34)
    flat_gbps = flat_bytes / (r["flat_ms"] * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": P / (r["ms"] * 1e-3),
        "unit": "params/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": W.RAGGED_2000.name, "params": P, "tensors": 2000,
                   "buckets": r["n_buckets"], "world_size": N, "replicas": N,
                   "flatten_streams": max(1, args.flatten_streams),
                   "shard_numel": r["s"], "grad_dtype": "bf16", "param_dtype": "bf16"},
        "hbm_gbps": (flat_bytes + step_bytes) / (r["ms"] * 1e-3) / 1e9,
        "hbm_frac": (flat_bytes + step_bytes) / (r["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "bytes_per_step": flat_bytes + step_bytes,
        "phases_ms": {"flatten_8_replicas": r["flat_ms"], "step_8_ranks": r["step_ms"]},
        "step_gbps": step_bytes / (r["step_ms"] * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "kernel": "flatten_kernel (all launches of one step)",
                     "achieved": flat_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": flat_gbps / HBM_PEAK_GBPS, "traffic": measured_traffic("ragged")},
        "step_check": {"norm": r["norm"], "clipped": r["clipped"], "overflow": r["overflow"]},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        with one_host_core():
            out["cpu_baseline"] = cpu_baseline_ragged(args, torch, W, r)
    print(json.dumps(out), flush=True)


def run_repartition(args, torch, Z, W):
    """Elastic resume of the ragged model's optimizer state (2.18e9 params):
    all three fp32 arrays moved from 8 ranks to 3 on the device (one step =
    three zero_repartition calls), and rank 0's checkpoint file written and
    read back through pinned staging (host-bound; reported, not the roofline)."""
    import tempfile
    from zero_sharded_optimizer_step_amd import checkpoint as C
    from zero_sharded_optimizer_step_amd.world import SimulatedWorld
    P = W.RAGGED_2000.numel
    src = SimulatedWorld(P, 8, n_replicas=1, alignment=128, grad_dtype=torch.bfloat16)
    dst = SimulatedWorld(P, 3, n_replicas=1, alignment=128, grad_dtype=torch.bfloat16)
    for w in (src, dst):
        w.grads = []
        w.workspace = []
    for k in range(8):
        for f, t in enumerate(src.state(k)):
            W.flat_normal(t, k * src.s, P, 1.0, ("bench-repart", f))
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        dst.repartition_from(src, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        dst.repartition_from(src, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # 3 arrays: every real element read once and written once, the new padding zeroed
    nbytes = 3 * (4 * P + 4 * dst.padded)
    # one rank's file: 3 x 273M fp32 written, then read back into a new rank
    d = tempfile.mkdtemp(prefix="zero_ckpt_")
    path = C.rank_path(d, 0)
    t0 = time.perf_counter()
    C.save_rank(path, src.part, 0, src.state(0), torch.bfloat16, 1)
    t_save = time.perf_counter() - t0
    fbytes = os.path.getsize(path)
    t0 = time.perf_counter()
    with open(path, "rb") as f:
        f.seek(C.HEADER_BYTES)
        for t in src.state(0):
            C._read_fp32(f, t[:src.valid[0]], C._staging(t.device, src.valid[0]))
    torch.cuda.synchronize()
    t_load = time.perf_counter() - t0
    os.remove(path)
    os.rmdir(d)
    gbps = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": P / (ms * 1e-3), "unit": "params/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "optimizer state of %d params re-partitioned from 8 ranks to 3 "
                               "(master, exp_avg, exp_avg_sq)" % P, "params": P},
        "hbm_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS, "bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "kernel": "flatten_kernel (range copies of zero_repartition, "
                                                "all launches of one step)",
                     "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": measured_traffic("repartition")},
        "checkpoint_file": {"bytes": fbytes, "save_s": t_save, "save_gbps": fbytes / t_save / 1e9,
                            "load_s": t_load, "load_gbps": fbytes / t_load / 1e9,
                            "where": "temporary directory on the host"},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        with one_host_core():
            out["cpu_baseline"] = cpu_baseline_repartition(args, torch, src)
    print(json.dumps(out), flush=True)


def run_offload(args, torch, Z, W):
    """The 13B/8 shard with its fp32 master and moments in pinned host memory:
    pass 1 and the combine on the GPU, then zero_offload_apply (gradient
    down, host AdamW, parameters up, pipelined by chunk)."""
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s = part.shard_numel
    valid = Z.zero_partition_valid_numel(part, 0)
    log("offload: generating 8 replicas and pinning 3 x %d fp32 of host state" % s)
    grads = []
    for i in range(w.world_size):
        g = torch.empty(s, dtype=torch.bfloat16, device="cuda")
        W.flat_normal(g, 0, w.numel, w.grad_sigma, W.grad_key(w, 0, 0, i))
        grads.append(g)
    master = torch.empty(s, dtype=torch.float32, pin_memory=True)
    tmp = torch.empty(min(s, W.CHUNK), dtype=torch.float32, device="cuda")
    for a in range(0, s, tmp.numel()):
        b = min(s, a + tmp.numel())
        W.flat_normal(tmp[:b - a], a, w.numel, w.master_sigma, W.master_key(w, 0))
        master[a:b].copy_(tmp[:b - a])
    del tmp
    m = torch.zeros(s, dtype=torch.float32, pin_memory=True)
    v = torch.zeros(s, dtype=torch.float32, pin_memory=True)
    full = torch.zeros(part.padded_numel, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(Z.zero_shard_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    partials = torch.zeros(Z.zero_partials_bytes(1), dtype=torch.uint8, device="cuda")
    glob = torch.zeros(256, dtype=torch.uint8, device="cuda")
    staging = Z.OffloadStaging(args.chunk, args.host_threads)
    stream = torch.cuda.current_stream()

    def step(t):
        a = Z.StepArgs(world_size=w.world_size, rank=0, shard_numel=s, valid_numel=valid,
                       replica_grads=grads, master=master, exp_avg=m, exp_avg_sq=v,
                       full_params=full, workspace=ws, lr=w.lr, weight_decay=w.weight_decay,
                       step=t, max_grad_norm=w.max_grad_norm)
        Z.zero_shard_reduce(a, 0, partials, stream)
        Z.zero_shard_combine(partials, 1, w.max_grad_norm, glob, stream)
        return Z.zero_offload_apply(a, glob, staging, want_info=True, stream=stream)

    t = 1
    for _ in range(args.warmup):
        step(t)
        t += 1
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        info = step(t)
        t += 1
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / K
    pcie = valid * (4 + 2)
    host_bytes = valid * (12 + 12 + 4 + 2)     # state read + written, staged gradient, cast
    threads = args.host_threads or Z.zero_host_threads()
    out = {
        "metric": METRIC, "value": valid / sec, "unit": "params/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": sec * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name + ", optimizer state offloaded to pinned host memory",
                   "shard_numel": s, "chunk_elems": args.chunk, "host_threads": threads},
        "pcie_gbps": pcie / sec / 1e9, "host_memory_gbps": host_bytes / sec / 1e9,
        "bytes_over_link_per_step": pcie,
        "roofline": None,
        "step_check": {"norm": info.norm, "clipped": info.clipped, "overflow": info.overflow},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        with one_host_core():
            out["cpu_baseline"] = cpu_baseline_shard13b(args, torch, W, grads)
    print(json.dumps(out), flush=True)


def run_zero3(args, torch, Z, W):
    """ZeRO-3 forward-pass gathering on the 13B/8 model: its bf16 parameters
    sit as 8 rank shards (one 26 GB buffer); one step walks 40 equal layers
    in order, each gathered from the shards on a side stream, prefetched
    within the live bound of the pages' configuration
    (stage3_max_live_parameters = 1e9 elements, three layers).  Bytes: every
    parameter read from its shard and written to its layer buffer, 4 B."""
    from zero_sharded_optimizer_step_amd.zero3 import LayerGatherer
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s = part.shard_numel
    full = torch.empty(part.padded_numel, dtype=torch.bfloat16, device="cuda")
    W.flat_normal(full, 0, w.numel, 0.02, ("bench-zero3",))
    shards = [full[r * s:(r + 1) * s] for r in range(w.world_size)]
    L = 40
    sizes = [w.numel // L] * L
    sizes[-1] += w.numel - sum(sizes)
    g = LayerGatherer(part, shards, sizes, int(2e8), MAX_LIVE_PARAMETERS)
    stream = torch.cuda.current_stream()

    def walk():
        n = 0
        for _, params in g.forward(stream):
            n += params.numel()
        return n

    for _ in range(args.warmup):
        walk()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        assert walk() == w.numel
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = 4 * w.numel
    gbps = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": w.numel / (ms * 1e-3), "unit": "params/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "13B bf16 parameters as 8 rank shards, gathered as 40 layers with "
                               "prefetch (live bound: 1e9 parameters)", "params": w.numel,
                   "layers": L, "max_live_parameters": MAX_LIVE_PARAMETERS},
        "hbm_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS, "bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "kernel": "flatten_kernel (range copies of zero_gather_params, "
                                                "all launches of one walk)",
                     "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": measured_traffic("zero3")},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        with one_host_core():
            out["cpu_baseline"] = cpu_baseline_zero3(args, torch, shards)
    print(json.dumps(out), flush=True)


def copy_ceiling(torch, Z, st, reps=10):
    """A plain copy through the library's flatten kernel, timed in the same
    process: rank 0's bf16 gradient slice of replica 0 (one table entry:
    one read and one write stream) into rank 1's slice of the full buffer,
    which rank 0's step never touches; the slice is zeroed again after.
    Its bandwidth is what a one-read, one-write stream reaches on this
    part, the practical ceiling for the streaming passes (the AdamW pass
    keeps four read and four write streams in flight)."""
    s = st["s"]
    src, dst = st["grads"][0], st["full"][s:2 * s]
    slot = Z.zero_tensor_slot_t(offset=0, numel=s, bucket=0, reserved=0)
    stream = torch.cuda.current_stream()
    Z.zero_bucket_flatten([slot], [src], src.dtype, dst, s, stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        Z.zero_bucket_flatten([slot], [src], src.dtype, dst, s, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
    dst.zero_()
    torch.cuda.synchronize()
    return {"kernel": "flatten_kernel copying one %d-element bf16 tensor" % s,
            "bytes": 4 * s, "median_ms": ms, "gbps": 4 * s / (ms * 1e-3) / 1e9}


def calibrate_copy(torch, n):
    """Plain copies of a known size, for scaling the HBM byte counters."""
    nbytes = 4 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for i in range(n):
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy %d of %d bytes done" % (i, nbytes))
    print(json.dumps({"calibration_copy_bytes_read": nbytes, "bytes_written": nbytes}))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: it times one rank's step on its own device and "
              "has no multi-GPU launcher. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import __graft_entry__
    __graft_entry__.ensure_built()             # only a fresh checkout is built here
    import zero_sharded_optimizer_step_amd as Z
    from zero_sharded_optimizer_step_amd import workloads as W
    Z.lib()
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy)
        return
    if args.workload == "ragged":
        report_ragged(args, run_ragged(args, torch, Z, W), W, torch)
        return
    if args.workload == "repartition":
        run_repartition(args, torch, Z, W)
        return
    if args.workload == "offload":
        run_offload(args, torch, Z, W)
        return
    if args.workload == "zero3":
        run_zero3(args, torch, Z, W)
        return
    if args.accumulation == "local":
        if args.micro_batches < 1:
            raise SystemExit("--accumulation local needs --micro-batches >= 1")
        run_shard13b_local(args, torch, Z, W)
        return
    r = run_shard13b(args, torch, Z, W)
    app_gbps = r["bytes_apply"] / (r["apply_ms"] * 1e-3) / 1e9
    step_gbps = r["bytes_step"] / (r["ms"] * 1e-3) / 1e9
    if args.micro_batches > 1:
        # the adding pass 1 dominates an accumulation window
        add_bytes = r["valid"] * (2 * r["st"]["nrep"] + 8)
        add_gbps = add_bytes / (r["add_ms"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": "reduce_kernel (adding pass 1 of a micro-batch)",
                    "achieved": add_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": add_gbps / HBM_PEAK_GBPS, "traffic": measured_traffic("shard13b_accum")}
    else:
        # each state layout and state-set count runs its own instantiation
        # of the kernel, counted under its own record
        variant = "shard13b" + ("_tiled" if args.state_layout == "tiled" else "") + \
            ("_pingpong" if args.state_buffers == 2 else "")
        roofline = {"bound": "hbm", "kernel": "apply_kernel (AdamW + cast)",
                    "achieved": app_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": app_gbps / HBM_PEAK_GBPS, "traffic": measured_traffic(variant)}
    out = {
        "metric": METRIC,
        "value": r["valid"] / (r["ms"] * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": W.SHARD_13B_OF_8.name, "shard_numel": r["st"]["s"],
                   "world_size": 8, "replicas": 8, "micro_batches": args.micro_batches,
                   "state_buffers": args.state_buffers, "state_layout": args.state_layout,
                   "grad_dtype": "bf16", "param_dtype": "bf16",
                   "lr": 6e-5, "weight_decay": 0.01, "max_grad_norm": 1.0},
        "hbm_gbps": step_gbps,
        "hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "bytes_per_step": r["bytes_step"],
        "kernels_ms": {"reduce_and_fold": r["reduce_ms"], "combine": r["combine_ms"],
                       "apply": r["apply_ms"], "adding_pass1": r["add_ms"]},
        "fused_call_ms_per_step": r["fused_ms"],
        "step_ms": {"min": r["step_ms_min"], "median": r["step_ms_median"], "max": r["step_ms_max"]},
        "wall_ms_per_step": r["wall_ms"],
        "roofline": roofline,
        "apply_gbps": app_gbps,
        "reduce_gbps": r["bytes_reduce"] / (r["reduce_ms"] * 1e-3) / 1e9,
        "step_check": {"norm": r["norm"], "clipped": r["clipped"], "overflow": r["overflow"]},
    }
    cc = copy_ceiling(torch, Z, r["st"])
    cc["frac_of_peak"] = cc["gbps"] / HBM_PEAK_GBPS
    cc["roofline_kernel_frac_of_copy"] = roofline["achieved"] / cc["gbps"]
    out["copy_ceiling"] = cc
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        with one_host_core():
            out["cpu_baseline"] = cpu_baseline_shard13b(args, torch, W, r["st"]["grads"],
                                                        args.micro_batches)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
