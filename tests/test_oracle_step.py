"""Pins for the oracle's reduce, clip, AdamW, scaler and full step (CPU only).

Each arithmetic piece is pinned to something other than itself: special
cases with exact answers (one replica, N equal replicas, constant
gradients, the first Adam step), library routines on the CPU
(torch.optim.AdamW and torch.nn.utils.clip_grad_norm_ in float64,
numpy sums), and the invariants the pages fix: a rank updates only its own
part, and the concatenated parts equal the unsharded step.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def f32_bits_to_code(x, dtype):
    return oracle.f32_to_f16(x) if dtype == oracle.FP16 else oracle.f32_to_bf16(x)


def decode(c, dtype):
    return oracle.f16_to_f32(c) if dtype == oracle.FP16 else oracle.bf16_to_f32(c)


def rand_codes(rng, n, dtype, sigma=1.0):
    return f32_bits_to_code((rng.standard_normal(n) * sigma).astype(np.float32), dtype)


# ------------------------------------------------------------------ reduce
@pytest.mark.parametrize("dtype", [oracle.FP16, oracle.BF16])
def test_reduce_one_replica_is_identity(dtype):
    rng = np.random.default_rng(0)
    x = rand_codes(rng, 4097, dtype)
    for scale in (1.0, 2.0**16, 2.0**-3):
        g, ss, of = oracle.reduce([x], dtype, oracle.inv_scale(scale))
        ref = decode(x, dtype).astype(np.float64) / scale
        assert np.array_equal(g.astype(np.float64), ref)
        assert of == 0
        assert ss == pytest.approx(float(np.sum(ref * ref)), rel=1e-13)


@pytest.mark.parametrize("dtype", [oracle.FP16, oracle.BF16])
@pytest.mark.parametrize("N", [2, 4, 8])
def test_reduce_equal_replicas_is_exact_multiple(dtype, N):
    rng = np.random.default_rng(N)
    x = rand_codes(rng, 1000, dtype)
    g, _, of = oracle.reduce([x] * N, dtype, oracle.inv_scale(1.0))
    assert np.array_equal(g, decode(x, dtype) * np.float32(N))
    assert of == 0


@pytest.mark.parametrize("dtype", [oracle.FP16, oracle.BF16])
@pytest.mark.parametrize("N", [2, 3, 4, 6, 8])
def test_reduce_mean_of_equal_replicas_is_the_replica(dtype, N):
    """A predivide factor D = N turns the sum into the DDP mean, so N equal
    replicas give back the replica, bit for bit.  The sum N·x is exact in
    fp32 (a 16-bit code's significand times N <= 8 fits in 24 bits).  For
    a power of two N the multiplier 1/N is exact too.  For N = 3 and 6,
    fp32(1/N)·N = 1 + 2^-25 exactly, so the product is x·(1 + 2^-25), which
    lies less than half an ulp from x and rounds to x."""
    if N & (N - 1):
        assert float(oracle.inv_scale(1.0, float(N))) * N == 1.0 + 2.0**-25
    rng = np.random.default_rng(100 + N)
    x = rand_codes(rng, 4001, dtype, sigma=1e-2)
    xf = decode(x, dtype)
    for S in (1.0, 2.0**10):
        xs = f32_bits_to_code(xf * np.float32(S), dtype)     # the scaled code each replica holds
        g, _, of = oracle.reduce([xs] * N, dtype, oracle.inv_scale(S, float(N)))
        assert of == 0
        assert np.array_equal(g.astype(np.float64), decode(xs, dtype).astype(np.float64) / S)


def test_reduce_predivide_enters_with_the_loss_scale_as_one_product():
    """Unscale and predivide are one multiply by fp32(1/(S·D)); with S·D a
    power of two it is exact, so halving S and doubling D changes nothing,
    and the result is the plain sum divided by S·D."""
    rng = np.random.default_rng(7)
    reps = [rand_codes(rng, 2001, oracle.FP16, sigma=50.0) for _ in range(5)]
    ref = None
    for S, D in ((1024.0, 4.0), (512.0, 8.0), (4096.0, 1.0)):
        g, _, _ = oracle.reduce(reps, oracle.FP16, oracle.inv_scale(S, D))
        if ref is None:
            ref = g
            acc = decode(reps[0], oracle.FP16).copy()
            for r in reps[1:]:
                acc = np.add(acc, decode(r, oracle.FP16), dtype=np.float32)
            assert np.array_equal(g.astype(np.float64), acc.astype(np.float64) / 4096.0)
        assert np.array_equal(g, ref)


@pytest.mark.parametrize("dtype", [oracle.FP16, oracle.BF16])
def test_reduce_matches_numpy_fp32_running_sum(dtype):
    rng = np.random.default_rng(11)
    N, n = 7, 3001
    reps = [rand_codes(rng, n, dtype, sigma=10.0 ** rng.uniform(-3, 3)) for _ in range(N)]
    acc = decode(reps[0], dtype).copy()
    for r in reps[1:]:
        acc = np.add(acc, decode(r, dtype), dtype=np.float32)
    inv = oracle.inv_scale(8.0)
    g, ss, of = oracle.reduce(reps, dtype, inv)
    assert np.array_equal(g, np.multiply(acc, inv, dtype=np.float32))
    assert of == 0
    exact = math.fsum(float(v) * float(v) for v in g)
    assert ss == pytest.approx(exact, rel=1e-12)


def test_reduce_sum_of_squares_accumulates_across_calls():
    rng = np.random.default_rng(2)
    a = rand_codes(rng, 500, oracle.BF16)
    b = rand_codes(rng, 700, oracle.BF16)
    inv = oracle.inv_scale(1.0)
    _, s1, _ = oracle.reduce([a], oracle.BF16, inv)
    _, s2, _ = oracle.reduce([b], oracle.BF16, inv, s1, 0)
    _, s12, _ = oracle.reduce([np.concatenate([a, b])], oracle.BF16, inv)
    assert s2 == s12


@pytest.mark.parametrize("dtype", [oracle.FP16, oracle.BF16])
@pytest.mark.parametrize("poison", [np.inf, -np.inf, np.nan])
def test_reduce_flags_any_nonfinite(dtype, poison):
    rng = np.random.default_rng(5)
    reps = [rand_codes(rng, 300, dtype) for _ in range(4)]
    for r in range(4):
        for i in (0, 150, 299):
            bad = [x.copy() for x in reps]
            bad[r][i] = f32_bits_to_code(np.array([poison], np.float32), dtype)[0]
            g, _, of = oracle.reduce(bad, dtype, oracle.inv_scale(2.0**16))
            assert of == 1 and not np.isfinite(g[i])
            assert np.isfinite(np.delete(g, i)).all()


def test_reduce_flags_fp32_overflow_of_the_sum():
    big = oracle.f32_to_bf16(np.array([3.0e38], np.float32))
    g, _, of = oracle.reduce([big, big], oracle.BF16, oracle.inv_scale(1.0))
    assert of == 1 and np.isinf(g[0])
    g, _, of = oracle.reduce([big], oracle.BF16, oracle.inv_scale(1.0))
    assert of == 0


# -------------------------------------------------------------------- clip
def test_clip_constant_gradient_closed_form():
    for n, c in ((100, 0.5), (10_000, 1e-3), (1, 3.0)):
        g = np.full(n, c, np.float32)
        _, ss, _ = oracle.reduce([oracle.f32_to_bf16(g)], oracle.BF16, 1.0)
        cval = float(oracle.bf16_to_f32(oracle.f32_to_bf16(np.float32([c])))[0])
        applies, norm, coef = oracle.clip(ss, 1.0)
        assert norm == pytest.approx(abs(cval) * math.sqrt(n), rel=1e-15)
        assert applies == (norm + 1e-6 > 1.0)
        assert coef == (1.0 / (norm + 1e-6) if applies else 1.0)


def test_clip_matches_torch_clip_grad_norm():
    rng = np.random.default_rng(9)
    for sigma in (1e-4, 1e-2, 1.0):
        g = (rng.standard_normal(5000) * sigma).astype(np.float32)
        t = torch.nn.Parameter(torch.zeros(5000, dtype=torch.float64))
        t.grad = torch.from_numpy(g.astype(np.float64))
        total = torch.nn.utils.clip_grad_norm_([t], 1.0)
        ss = float(np.sum(g.astype(np.float64) ** 2))
        applies, norm, coef = oracle.clip(ss, 1.0)
        assert norm == pytest.approx(float(total), rel=1e-12)
        assert np.allclose(g.astype(np.float64) * coef, t.grad.numpy(), rtol=1e-14, atol=0)
    assert oracle.clip(4.0, 0.0) == (False, 2.0, 1.0)      # max_norm <= 0: off
    assert oracle.clip(4.0, -1.0)[0] is False


# ------------------------------------------------------------------- AdamW
U = 2.0**-24          # unit roundoff of fp32


def adam_bounds(g, m, v, p, coef, lr, b1, b2, eps, wd, t):
    """Per-element bounds on |fp32 evaluation - exact| for one AdamW step
    from the same fp32 state, derived from the operation count: each fp32
    operation and each fp32 constant adds at most U relative to the term it
    rounds, so m' is off by <= 4U (b1|m| + (1-b1)|g'|), v' by <= 6U v', and
    p' by <= 10U (|p decay| + step |m'|/d + step S_m/d) + U|p'|."""
    g = g.astype(np.float64) * coef
    m, v, p = (x.astype(np.float64) for x in (m, v, p))
    m1 = b1 * m + (1 - b1) * g
    v1 = b2 * v + (1 - b2) * g * g
    sm = b1 * np.abs(m) + (1 - b1) * np.abs(g)
    step = lr / (1 - b1**t)
    d = np.sqrt(v1) / math.sqrt(1 - b2**t) + eps
    p1 = p * (1 - lr * wd) - step * m1 / d
    bm = 4 * U * sm
    bv = 6 * U * v1
    bp = 10 * U * (np.abs(p * (1 - lr * wd)) + step * (np.abs(m1) + sm) / d) + U * np.abs(p1)
    return (m1, v1, p1), (bm, bv, bp)


def test_adamw_first_step_closed_form():
    # t = 1, m = v = 0: m' = (1-b1) g, v' = (1-b2) g^2 and the bias-corrected
    # ratio is g / (|g| + eps), so p' = p (1 - lr wd) - lr g / (|g| + eps).
    rng = np.random.default_rng(4)
    g = (rng.standard_normal(2000) * 10.0 ** rng.uniform(-6, 1, 2000)).astype(np.float32)
    p0 = (rng.standard_normal(2000) * 0.02).astype(np.float32)
    p, m, v = p0.copy(), np.zeros_like(g), np.zeros_like(g)
    lr, wd, eps = 6e-5, 0.01, 1e-8
    oracle.adamw(g, p, m, v, 1.0, lr, 0.9, 0.999, eps, wd, 1)
    gd, pd = g.astype(np.float64), p0.astype(np.float64)
    assert np.all(np.abs(m - 0.1 * gd) <= 2 * U * np.abs(0.1 * gd))
    assert np.all(np.abs(v - 0.001 * gd * gd) <= 4 * U * 0.001 * gd * gd)
    upd = lr * gd / (np.abs(gd) + eps)
    expect = pd * (1 - lr * wd) - upd
    assert np.all(np.abs(p - expect) <= 10 * U * (np.abs(pd) + 2 * np.abs(upd)) + U * np.abs(expect))
    # relative to the size of the two terms the update combines
    assert np.max(np.abs(p - expect) / (np.abs(pd) + np.abs(upd))) < 4e-7


def test_adamw_clip_coefficient_scales_gradient():
    rng = np.random.default_rng(6)
    g = rng.standard_normal(100).astype(np.float32)
    p = rng.standard_normal(100).astype(np.float32)
    a = [p.copy(), np.zeros(100, np.float32), np.zeros(100, np.float32)]
    b = [p.copy(), np.zeros(100, np.float32), np.zeros(100, np.float32)]
    oracle.adamw(g, *a, 0.25, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    oracle.adamw((g * np.float32(0.25)).astype(np.float32), *b, 1.0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("coef", [1.0, 0.37])
@pytest.mark.parametrize("hyper", [(6e-5, 0.9, 0.999, 1e-8, 0.01), (1e-3, 0.8, 0.95, 1e-6, 0.1),
                                   (3e-4, 0.0, 0.99, 1e-8, 0.0), (0.1, 0.5, 0.5, 1e-3, 1.0)],
                         ids=["default", "large-model", "no-first-moment", "strong-decay"])
def test_adamw_matches_torch_adamw_float64(coef, hyper):
    # From the same fp32 state, one step of torch.optim.AdamW in float64 (a
    # library evaluation of the textbook update) and the oracle's fp32 step
    # agree within the derived bounds, at every t.
    rng = np.random.default_rng(8)
    n = 4000
    lr, b1, b2, eps, wd = hyper
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 12):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0)).astype(np.float32)
        tp = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
        opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                                foreach=False, fused=False)
        opt.state[tp] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                         "exp_avg": torch.from_numpy(m.astype(np.float64)),
                         "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
        # torch clips by scaling the gradient in place; same factor here
        gc = g.astype(np.float64) * float(np.float32(coef))
        tp.grad = torch.from_numpy(gc)
        _, (bm, bv, bp) = adam_bounds(g, m, v, p, float(np.float32(coef)), lr, b1, b2, eps, wd, t)
        opt.step()
        oracle.adamw(g, p, m, v, coef, lr, b1, b2, eps, wd, t)
        st = opt.state[tp]
        for mine, ref, bound in ((m, st["exp_avg"], bm), (v, st["exp_avg_sq"], bv),
                                 (p, tp.detach(), bp)):
            err = np.abs(mine.astype(np.float64) - ref.numpy())
            assert np.all(err <= bound), (t, float(np.max(err / np.maximum(bound, 1e-300))))


# ------------------------------------------------------------------ scaler
def run_scaler(flags, power=4, window=3, hysteresis=2, min_scale=1.0):
    s = oracle.LossScaler(power, window, hysteresis, min_scale)
    out = []
    for f in flags:
        skip = s.update(f)
        out.append((skip, s.scale, s.good, s.hyst))
    return out


def test_scaler_grows_every_window_without_overflow():
    out = run_scaler([False] * 10, power=16, window=3)
    assert [o[1] for o in out] == [2.0 ** (16 + (k + 1) // 3) for k in range(10)]
    assert not any(o[0] for o in out)


def test_scaler_hand_traced_sequence():
    F, T = False, True
    # window 3, hysteresis 2, start 16:
    flags = [F, T, F, F, F, T, T, T, F, F, F, F]
    expect = [
        (False, 16, 1, 2),   # good step
        (True, 16, 0, 1),    # first overflow spends the hysteresis
        (False, 16, 1, 1),
        (False, 16, 2, 1),
        (False, 32, 0, 2),   # third good step: grow, refill hysteresis
        (True, 32, 0, 1),    # overflow: hysteresis 2 -> 1, scale kept
        (True, 16, 0, 1),    # overflow with hysteresis 1: halve
        (True, 8, 0, 1),     # and again
        (False, 8, 1, 1),
        (False, 8, 2, 1),
        (False, 16, 0, 2),
        (False, 16, 1, 2),
    ]
    assert run_scaler(flags) == expect


def test_scaler_floor_at_min_scale():
    out = run_scaler([True] * 10, power=3, window=5, hysteresis=1, min_scale=1.0)
    assert [o[1] for o in out] == [4, 2, 1, 1, 1, 1, 1, 1, 1, 1]
    assert all(o[0] for o in out)
    # a floor that is not a power of two: halving stops at it, and growth
    # doubles from it
    out = run_scaler([True, True, True, False, False, True, False, False, False, False],
                     power=3, window=2, hysteresis=1, min_scale=3.0)
    assert [o[1] for o in out] == [4, 3, 3, 3, 6, 3, 3, 6, 6, 12]


def test_scaler_page_defaults():
    s = oracle.LossScaler(16, 100, 2, 1.0)
    assert s.scale == 65536.0 and s.hyst == 2
    for _ in range(99):
        s.update(False)
    assert s.scale == 65536.0
    s.update(False)
    assert s.scale == 131072.0


# --------------------------------------------------------------- full step
def make_world(rng, P, N, world, A, dtype, sigma, scale=1.0):
    s, padded, valid = oracle.partition(P, world, A)
    reps = []
    for _ in range(N):
        f = np.zeros(padded, np.uint16)
        f[:P] = f32_bits_to_code((rng.standard_normal(P) * sigma * scale).astype(np.float32), dtype)
        reps.append(f)
    master = (rng.standard_normal(padded) * 0.02).astype(np.float32)
    master[P:] = 0
    return s, padded, valid, reps, master


def split(arr, world, s):
    return [arr[r * s:(r + 1) * s].copy() for r in range(world)]


@pytest.mark.parametrize("dtype,sigma,clip", [(oracle.BF16, 1e-2, 1.0),
                                              (oracle.FP16, 1e-3, 1e9),
                                              (oracle.BF16, 1e-5, 1.0)])
def test_sharded_concatenation_equals_unsharded_step(dtype, sigma, clip):
    rng = np.random.default_rng(12)
    P, N, A = 10_007, 8, 8
    scale = 2.0**10 if dtype == oracle.FP16 else 1.0
    s, padded, valid, reps, master = make_world(rng, P, N, N, A, dtype, sigma, scale)
    hp = oracle.Hyper(max_grad_norm=clip, loss_scale=scale)
    ms, ps_, vs = split(np.zeros(padded, np.float32), N, s), split(master, N, s), \
        split(np.zeros(padded, np.float32), N, s)
    full = np.zeros(padded, np.uint16)
    info = oracle.step(reps, dtype, P, N, A, ps_, ms, vs, full, hp, t=1)
    # unsharded: the same N replicas, a world of one rank
    p1 = [master[:P].copy()]
    m1 = [np.zeros(P, np.float32)]
    v1 = [np.zeros(P, np.float32)]
    full1 = np.zeros(P, np.uint16)
    info1 = oracle.step(reps, dtype, P, 1, 1, p1, m1, v1, full1, hp, t=1)
    assert info.sumsq == info1.sumsq and info.clipped == info1.clipped
    assert np.array_equal(np.concatenate(ps_)[:P], p1[0])
    assert np.array_equal(np.concatenate(ms)[:P], m1[0])
    assert np.array_equal(np.concatenate(vs)[:P], v1[0])
    assert np.array_equal(full[:P], full1)
    # padding is never touched
    assert not np.concatenate(ms)[P:].any() and not full[P:].any()


def test_each_rank_updates_only_its_part():
    rng = np.random.default_rng(13)
    P, N, A = 5000, 4, 8
    s, padded, valid, reps, master = make_world(rng, P, N, N, A, oracle.BF16, 1e-2)
    ps_ = split(master, N, s)
    ms = split(np.zeros(padded, np.float32), N, s)
    vs = split(np.zeros(padded, np.float32), N, s)
    full = np.full(padded, 0xABCD, np.uint16)
    oracle.step(reps, oracle.BF16, P, N, A, ps_, ms, vs, full, oracle.Hyper(), t=1)
    assert np.array_equal(full[:P], oracle.f32_to_bf16(np.concatenate(ps_)[:P]))
    assert (full[P:] == 0xABCD).all()


def test_parameter_format_changes_only_the_cast():
    """The full buffer's format is independent of the gradients': the state
    after a step is the same, and the buffer holds each format's
    round-to-nearest-even of the same new masters."""
    rng = np.random.default_rng(15)
    P, N, A = 3000, 3, 8
    s, padded, valid, reps, master = make_world(rng, P, N, N, A, oracle.BF16, 1e-2)
    out = {}
    for pdt in (oracle.BF16, oracle.FP16):
        ps_ = split(master.copy(), N, s)
        ms = split(np.zeros(padded, np.float32), N, s)
        vs = split(np.zeros(padded, np.float32), N, s)
        full = np.full(padded, 0xABCD, np.uint16)
        oracle.step(reps, oracle.BF16, P, N, A, ps_, ms, vs, full, oracle.Hyper(), t=1,
                    param_dtype=pdt)
        out[pdt] = (np.concatenate(ps_), np.concatenate(ms), np.concatenate(vs), full)
    for a, b in zip(out[oracle.BF16][:3], out[oracle.FP16][:3]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    p1 = out[oracle.BF16][0][:P]
    assert np.array_equal(out[oracle.BF16][3][:P], oracle.f32_to_bf16(p1))
    assert np.array_equal(out[oracle.FP16][3][:P], oracle.f32_to_f16(p1))
    assert not np.array_equal(out[oracle.BF16][3][:P], out[oracle.FP16][3][:P])


@pytest.mark.parametrize("where", [(0, 0), (3, 4999), (2, 2600)])
def test_overflow_anywhere_skips_every_rank(where):
    rng = np.random.default_rng(14)
    P, N, A = 5000, 4, 8
    s, padded, valid, reps, master = make_world(rng, P, N, N, A, oracle.FP16, 1e-3, 2.0**16)
    reps[where[0]][where[1]] = 0x7C00                      # +inf
    ps_ = split(master, N, s)
    ms = split(np.full(padded, 0.5, np.float32), N, s)
    vs = split(np.full(padded, 0.25, np.float32), N, s)
    full = np.full(padded, 0x1234, np.uint16)
    before = [x.copy() for x in ps_ + ms + vs] + [full.copy()]
    info = oracle.step(reps, oracle.FP16, P, N, A, ps_, ms, vs, full,
                       oracle.Hyper(loss_scale=2.0**16), t=3)
    assert info.overflow and info.skipped
    for a, b in zip(before, ps_ + ms + vs + [full]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", [oracle.FP16, oracle.BF16])
@pytest.mark.parametrize("kind", [0, 1, 2])
def test_nonfinite_code_in_padding_is_no_overflow(dtype, kind):
    # Reading: the overflow flag covers the real elements only.  Padding
    # holds no parameter, so the unsharded step (a world of one rank with
    # alignment 1, which has no padding at all) never sees it; the sharded
    # step's concatenated parts equal that step whatever the replicas'
    # padding holds, and it is not skipped.
    rng = np.random.default_rng(21)
    P, N, A = 5000, 4, 128                      # s = 1280, padding 120 on rank 3
    scale = 2.0**16 if dtype == oracle.FP16 else 1.0
    s, padded, valid, reps, master = make_world(rng, P, N, N, A, dtype, 1e-3, scale)
    assert padded - P == 120
    codes = (0x7C00, 0xFC00, 0x7E00) if dtype == oracle.FP16 else (0x7F80, 0xFF80, 0x7FC0)
    for i, r in enumerate(reps):
        r[P + 7 * i] = codes[kind]
    hp = oracle.Hyper(loss_scale=scale)
    ps_, ms, vs = split(master, N, s), split(np.zeros(padded, np.float32), N, s), \
        split(np.zeros(padded, np.float32), N, s)
    full = np.zeros(padded, np.uint16)
    info = oracle.step(reps, dtype, P, N, A, ps_, ms, vs, full, hp, t=1)
    assert not info.overflow and not info.skipped and math.isfinite(info.sumsq)
    p1 = [master[:P].copy()]
    m1, v1 = [np.zeros(P, np.float32)], [np.zeros(P, np.float32)]
    full1 = np.zeros(P, np.uint16)
    info1 = oracle.step([r[:P].copy() for r in reps], dtype, P, 1, 1, p1, m1, v1, full1, hp, t=1)
    # both sum the squares over the same elements in the same order
    assert info1.sumsq == info.sumsq and info1.coef == info.coef
    assert np.array_equal(np.concatenate([x[:n] for x, n in zip(ps_, valid)]), p1[0])
    assert np.array_equal(full[:P], full1)
    # the state's padding (zero here) is never written
    for x, n in zip(ps_ + ms + vs, valid * 3):
        assert not np.any(x[n:])


# ----------------------------------------------------- gradient accumulation
@pytest.mark.parametrize("dtype", [oracle.FP16, oracle.BF16])
def test_accumulate_adds_the_reduced_micro_batch(dtype):
    # The accumulated slice equals the first micro-batch's reduced slice
    # plus the second's, added in fp32 by numpy; the sum of squares is that
    # of the updated slice.
    rng = np.random.default_rng(21)
    n, N = 3001, 4
    mb1 = [rand_codes(rng, n, dtype, sigma=10.0 ** rng.uniform(-3, 1)) for _ in range(N)]
    mb2 = [rand_codes(rng, n, dtype, sigma=10.0 ** rng.uniform(-3, 1)) for _ in range(N)]
    inv = oracle.inv_scale(4.0)
    g1, _, _ = oracle.reduce(mb1, dtype, inv)
    g2, _, _ = oracle.reduce(mb2, dtype, inv)
    acc = g1.copy()
    ss, of = oracle.reduce_accumulate(mb2, dtype, inv, acc)
    assert np.array_equal(acc, np.add(g1, g2, dtype=np.float32))
    assert of == 0
    assert ss == pytest.approx(math.fsum(float(v) * float(v) for v in acc), rel=1e-12)


def test_accumulate_exact_closed_form():
    # Dyadic values whose sums are exact: K micro-batches of N equal
    # replicas give exactly K * N * x.
    x = np.array([0.5, -0.25, 3.0, 1.0 / 64, -7.0, 0.0], np.float32)
    codes = oracle.f32_to_bf16(x)
    N, K = 4, 5
    g, _, _ = oracle.reduce([codes] * N, oracle.BF16, oracle.inv_scale(1.0))
    for _ in range(K - 1):
        oracle.reduce_accumulate([codes] * N, oracle.BF16, oracle.inv_scale(1.0), g)
    assert np.array_equal(g, x * np.float32(K * N))


def test_accumulate_sign_of_zero_and_overflow():
    neg0 = oracle.f32_to_f16(np.array([-0.0], np.float32))
    g, _, _ = oracle.reduce([neg0], oracle.FP16, oracle.inv_scale(1.0))
    assert np.signbit(g[0])                     # the first micro-batch sets g
    oracle.reduce_accumulate([oracle.f32_to_f16(np.array([0.0], np.float32))], oracle.FP16,
                             oracle.inv_scale(1.0), g)
    assert g[0] == 0 and not np.signbit(g[0])   # -0 + 0 = +0 in round-to-nearest
    # an inf in an early micro-batch survives later finite ones
    inf = oracle.f32_to_f16(np.array([np.inf, 1.0], np.float32))
    fin = oracle.f32_to_f16(np.array([1.0, 1.0], np.float32))
    g, _, of = oracle.reduce([inf], oracle.FP16, oracle.inv_scale(1.0))
    ss, of = oracle.reduce_accumulate([fin], oracle.FP16, oracle.inv_scale(1.0), g)
    assert of == 1 and np.isinf(g[0]) and g[1] == 2.0


def test_accumulated_step_equals_one_step_over_all_gradients_when_sums_are_exact():
    # With dyadic gradients every sum is exact, so K micro-batches of N
    # replicas give the same step as one reduce over all K * N gradients.
    rng = np.random.default_rng(22)
    P, N, A, K = 5003, 4, 8, 3
    s, padded, valid = oracle.partition(P, N, A)

    def dyadic():
        f = np.zeros(padded, np.uint16)
        f[:P] = oracle.f32_to_bf16((rng.integers(-64, 65, P) / 1024.0).astype(np.float32))
        return f

    micro = [[dyadic() for _ in range(N)] for _ in range(K)]
    master = (rng.standard_normal(padded) * 0.02).astype(np.float32)
    hp = oracle.Hyper(max_grad_norm=1.0)

    def run(fn, batches):
        ps = split(master, N, s)
        ms = split(np.zeros(padded, np.float32), N, s)
        vs = split(np.zeros(padded, np.float32), N, s)
        full = np.zeros(padded, np.uint16)
        info = fn(batches, oracle.BF16, P, N, A, ps, ms, vs, full, hp, 1, keep_grads=True)
        return info, ps, ms, vs, full

    a = run(oracle.step_accumulated, micro)
    b = run(oracle.step, [f for mb in micro for f in mb])
    assert a[0].sumsq == b[0].sumsq and a[0].clipped and b[0].clipped
    for x, y in zip(a[0].grads, b[0].grads):
        assert np.array_equal(x, y)
    for xs, ys in zip(a[1:4], b[1:4]):
        for x, y in zip(xs, ys):
            assert np.array_equal(x, y)
    assert np.array_equal(a[4], b[4])


# ------------------------------------ accumulation before the reduce (no_sync)
@pytest.mark.parametrize("dtype", [oracle.FP16, oracle.BF16])
def test_local_accumulation_matches_numpy_fp32_running_sum(dtype):
    # A replica's window, widened and added in micro-batch order by numpy.
    rng = np.random.default_rng(31)
    K, n = 5, 3001
    micro = [rand_codes(rng, n, dtype, sigma=10.0 ** rng.uniform(-3, 2)) for _ in range(K)]
    acc = oracle.accumulate_local(micro, dtype)
    ref = decode(micro[0], dtype).copy()
    for x in micro[1:]:
        ref = np.add(ref, decode(x, dtype), dtype=np.float32)
    assert np.array_equal(acc, ref)


def test_reduce_f32_matches_numpy_running_sum():
    rng = np.random.default_rng(32)
    N, n = 6, 2999
    reps = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
            for _ in range(N)]
    inv = oracle.inv_scale(8.0)
    g, ss, of = oracle.reduce_f32(reps, inv)
    acc = reps[0].copy()
    for r in reps[1:]:
        acc = np.add(acc, r, dtype=np.float32)
    ref = np.multiply(acc, inv, dtype=np.float32)
    assert np.array_equal(g, ref) and of == 0
    assert ss == np.cumsum(ref.astype(np.float64) ** 2)[-1]     # sequential, index order
    bad = [r.copy() for r in reps]
    bad[3][17] = np.nan
    assert oracle.reduce_f32(bad, inv)[2] == 1


def test_local_accumulation_exact_closed_form():
    # Dyadic values whose sums are exact: N replicas, each summing K equal
    # micro-batches, give exactly N * K * x, unscaled.
    x = np.array([0.5, -0.25, 3.0, 1.0 / 64, -7.0, 0.0], np.float32)
    codes = oracle.f32_to_f16(x)
    N, K = 3, 4
    local = [oracle.accumulate_local([codes] * K, oracle.FP16) for _ in range(N)]
    g, _, _ = oracle.reduce_f32(local, oracle.inv_scale(2.0))
    assert np.array_equal(g, x * np.float32(N * K / 2.0))


def test_local_accumulation_order_differs_from_reduce_per_micro_batch():
    # Worked by hand, bf16 inputs, scale 1, one element, 2 replicas, 2
    # micro-batches: replica 0 sees 1 then 2^-24, replica 1 sees 0 then 2^-24.
    # Summed locally first: replica 0 holds 1 + 2^-24, a tie between 1 and
    # 1 + 2^-23 that rounds to the even 1; replica 1 holds 2^-24; their sum
    # 1 + 2^-24 rounds to 1 again.  Reduced per micro-batch: 1 + 0 = 1, then
    # 2^-24 + 2^-24 = 2^-23, and 1 + 2^-23 is exact.
    one, tiny, zero = 0x3F80, 0x3380, 0x0000          # bf16 codes of 1, 2^-24, 0
    assert oracle.bf16_to_f32(np.array([tiny], np.uint16))[0] == 2.0 ** -24
    micro = [[np.array([one], np.uint16), np.array([zero], np.uint16)],
             [np.array([tiny], np.uint16), np.array([tiny], np.uint16)]]

    def run(fn):
        z = [np.zeros(1, np.float32)]
        info = fn(micro, oracle.BF16, 1, 1, 1, [np.zeros(1, np.float32)], z,
                  [np.zeros(1, np.float32)], np.zeros(1, np.uint16), oracle.Hyper(), 1,
                  keep_grads=True)
        return info.grads[0][0]

    assert run(oracle.step_local_accumulated) == np.float32(1.0)
    assert run(oracle.step_accumulated) == np.float32(1.0 + 2.0 ** -23)


def test_local_accumulation_sign_of_zero_and_skip():
    neg0 = oracle.f32_to_bf16(np.array([-0.0, 1.0], np.float32))
    acc = oracle.accumulate_local([neg0, neg0], oracle.BF16)
    assert np.signbit(acc[0])                   # -0 + -0 = -0; the first sets, not adds
    g, _, _ = oracle.reduce_f32([acc], oracle.inv_scale(1.0))
    assert np.signbit(g[0]) and g[1] == 2.0
    # a NaN in one micro-batch of one replica skips the whole window
    P, N, A, K = 1001, 2, 8, 3
    s, padded, valid = oracle.partition(P, N, A)
    rng = np.random.default_rng(33)
    micro = [[rand_codes(rng, padded, oracle.BF16, 1e-2) for _ in range(N)] for _ in range(K)]
    micro[1][1][700] = 0x7FC0                   # bf16 NaN
    ps = split((rng.standard_normal(padded) * 0.02).astype(np.float32), N, s)
    before = [p.copy() for p in ps]
    info = oracle.step_local_accumulated(micro, oracle.BF16, P, N, A, ps,
                                         split(np.zeros(padded, np.float32), N, s),
                                         split(np.zeros(padded, np.float32), N, s),
                                         np.zeros(padded, np.uint16), oracle.Hyper(), 1)
    assert info.overflow and info.skipped
    assert all(np.array_equal(a, b) for a, b in zip(before, ps))


def test_local_accumulation_of_one_micro_batch_is_the_plain_step():
    # Widening is exact, so a window of one micro-batch reduces the same
    # fp32 values in the same order as the plain step.
    rng = np.random.default_rng(34)
    P, N, A = 4099, 4, 128
    s, padded, valid = oracle.partition(P, N, A)
    flats = [rand_codes(rng, padded, oracle.FP16, 1e-3 * 2**12) for _ in range(N)]
    master = (rng.standard_normal(padded) * 0.02).astype(np.float32)
    hp = oracle.Hyper(loss_scale=2.0**12)
    out = []
    for fn, arg in ((oracle.step_local_accumulated, [flats]), (oracle.step, flats)):
        ps, ms, vs = (split(a, N, s) for a in (master, np.zeros(padded, np.float32),
                                                np.zeros(padded, np.float32)))
        full = np.zeros(padded, np.uint16)
        info = fn(arg, oracle.FP16, P, N, A, ps, ms, vs, full, hp, 1)
        out.append((info.sumsq, ps, ms, vs, full))
    assert out[0][0] == out[1][0]
    for xs, ys in zip(out[0][1:4], out[1][1:4]):
        assert all(np.array_equal(x, y) for x, y in zip(xs, ys))
    assert np.array_equal(out[0][4], out[1][4])
