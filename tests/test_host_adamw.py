"""CPU tests of the library's host AdamW (the update of the offloaded
optimizer step) against the oracle: same fp32 operations in the same order,
so the same bits, on any thread count; and its round-to-nearest-even casts
on midpoints, subnormals, the overflow edge and NaN."""
import os

import numpy as np
import pytest

import oracle
import zero_sharded_optimizer_step_amd as Z


@pytest.mark.parametrize("threads", [1, 3, 0])
@pytest.mark.parametrize("dtype", [Z.ZERO_BF16, Z.ZERO_FP16])
def test_host_adamw_matches_oracle_bitwise(threads, dtype):
    rng = np.random.default_rng(31)
    n = 300_007
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    op, om, ov = p.copy(), m.copy(), v.copy()
    out = np.empty(n, np.uint16)
    for t, coef in ((1, 1.0), (2, 0.37), (3, 1.0), (10, 0.001)):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, 1)).astype(np.float32)
        Z.zero_host_adamw(g, coef, p, m, v, out, dtype, step=t, n_threads=threads)
        oracle.adamw(g, op, om, ov, float(np.float32(coef)), 6e-5, 0.9, 0.999, 1e-8, 0.01, t)
        for name, a, b in (("master", p, op), ("exp_avg", m, om), ("exp_avg_sq", v, ov)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (name, t)
        ref = oracle.f32_to_bf16(op) if dtype == Z.ZERO_BF16 else oracle.f32_to_f16(op)
        assert np.array_equal(out, ref), t


def cast_probes(decode, top):
    codes = np.arange(0, top, dtype=np.uint32).astype(np.uint16)
    vals = decode(codes).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(0)), vals.astype(np.float32)])
    return np.concatenate([x, -x])


@pytest.mark.parametrize("dtype", [Z.ZERO_BF16, Z.ZERO_FP16])
def test_host_casts_round_to_nearest_even(dtype):
    # lr = 0 and no decay leave the masters unchanged, so params_out is the
    # cast of the given values.
    if dtype == Z.ZERO_FP16:
        x = cast_probes(oracle.f16_to_f32, 0x7C00)
        edges = [65504, 65519.996, 65520, 65536, 1e9, 2.0**-24, 2.0**-25, 1.5 * 2.0**-25,
                 2.0**-26, 6.1e-5, np.inf, -np.inf, np.nan, 3.4e38]
    else:
        x = cast_probes(oracle.bf16_to_f32, 0x7F80)
        edges = [3.3961776e38, 3.3961775e38, np.finfo(np.float32).max, 1e-45, 2.0**-133,
                 np.inf, -np.inf, np.nan]
    rng = np.random.default_rng(7)
    rnd = rng.integers(0, 2**32, 1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, np.array(edges, np.float32), rnd[np.isfinite(rnd)]]).astype(np.float32)
    x = x[x != 0]                   # p - 0 * (m / d) turns -0 into +0 on both sides alike
    p = x.copy()
    out = np.empty(x.size, np.uint16)
    Z.zero_host_adamw(np.zeros(x.size, np.float32), 1.0, p, np.zeros(x.size, np.float32),
                      np.zeros(x.size, np.float32), out, dtype, lr=0.0, weight_decay=0.0)
    assert np.array_equal(p.view(np.uint32)[np.isfinite(x)], x.view(np.uint32)[np.isfinite(x)])
    ref = oracle.f32_to_bf16(p) if dtype == Z.ZERO_BF16 else oracle.f32_to_f16(p)
    nan = np.isnan(p)
    assert np.array_equal(out[~nan], ref[~nan])
    nan_code = (out[nan] & 0x7FFF) > (0x7F80 if dtype == Z.ZERO_BF16 else 0x7C00)
    assert nan_code.all()


def test_host_adamw_rejects():
    g = np.zeros(4, np.float32)
    with pytest.raises(Z.ZeroError):
        Z.zero_host_adamw(g, 1.0, g.copy(), g.copy(), g.copy(), None, Z.ZERO_BF16, step=0)
    with pytest.raises(Z.ZeroError):
        Z.zero_host_adamw(g, 1.0, g.copy(), g.copy(), g.copy(), None, 7)
    with pytest.raises(Z.ZeroError):
        Z.zero_host_adamw(g, float("nan"), g.copy(), g.copy(), g.copy(), None, Z.ZERO_BF16)


def test_host_threads_default_follows_omp_and_affinity():
    """n_threads = 0 resolves to OMP_NUM_THREADS, else the affinity mask."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r); import zero_sharded_optimizer_step_amd as Z; "
            "print(Z.zero_host_threads())" % root)
    env = dict(os.environ, OMP_NUM_THREADS="3")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         check=True).stdout
    assert int(out) == 3
    env.pop("OMP_NUM_THREADS")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         check=True).stdout
    assert int(out) == len(os.sched_getaffinity(0))


@pytest.mark.parametrize("dtype", [Z.ZERO_BF16, Z.ZERO_FP16])
def test_host_adamw_on_ieee_edge_values(dtype):
    # The offloaded update on every combination of master, m and v drawn
    # from signed zeros, subnormals, extremes, infinities and NaN, under
    # gradients from 0 to 3e38: the oracle's bits, NaN for NaN.
    import itertools
    S = np.array([0.0, -0.0, 1.4e-45, -1.4e-45, 1e-40, 1.17549435e-38, 1e-20, 0.02, -0.5, 3.0,
                  1e20, 3.4028235e38, -3.4028235e38, np.inf, -np.inf, np.nan], np.float32)
    G = np.array([0.0, -0.0, 1e-40, 0.5, -3.0, 1e30, 3e38, -1e-3], np.float32)
    combos = np.array(list(itertools.product(range(S.size), repeat=3)), np.int64)
    p = np.tile(S[combos[:, 0]], G.size)
    m = np.tile(S[combos[:, 1]], G.size)
    v = np.tile(S[combos[:, 2]], G.size)
    g = np.repeat(G, combos.shape[0])
    op, om, ov = p.copy(), m.copy(), v.copy()
    out = np.empty(p.size, np.uint16)
    for t in (1, 3):
        Z.zero_host_adamw(g, 1.0, p, m, v, out, dtype, step=t, n_threads=3)
        oracle.adamw(g, op, om, ov, 1.0, 6e-5, 0.9, 0.999, 1e-8, 0.01, t)
        for name, a, b in (("master", p, op), ("exp_avg", m, om), ("exp_avg_sq", v, ov)):
            nan = np.isnan(b)
            assert np.array_equal(np.isnan(a), nan), (name, t)
            assert np.array_equal(a[~nan].view(np.uint32), b[~nan].view(np.uint32)), (name, t)
        enc, dec = ((oracle.f32_to_bf16, oracle.bf16_to_f32) if dtype == Z.ZERO_BF16
                    else (oracle.f32_to_f16, oracle.f16_to_f32))
        ref = enc(op)
        cnan = np.isnan(dec(ref))
        assert np.array_equal(np.isnan(dec(out)), cnan)
        assert np.array_equal(out[~cnan], ref[~cnan]), t
