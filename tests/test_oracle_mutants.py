"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutant is a copy of the oracle source with one planted mistake (a
dropped term, a wrong sign or operand, a wrong rounding rule).  A mutant of
the C file is built to a temporary library; a mutant of the Python layer
(the unscale multiplier, the cross-rank norm and skip, re-partition,
gather) is a copy of the oracle package and the pin tests in a temporary
tree.  The pin tests run against it in a subprocess; every mutant must make
them fail.  Nothing here touches the HIP library.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "zero_oracle.c")
PINS = [os.path.join(HERE, f) for f in
        ("test_oracle_partition.py", "test_oracle_formats.py", "test_oracle_step.py")]

MUTANTS = {
    "m_bias_correction_dropped": ("(float)(lr / (1.0 - pow(beta1, (double)t)))", "(float)lr"),
    "v_bias_correction_dropped": ("(float)(1.0 / sqrt(1.0 - pow(beta2, (double)t)))", "1.0f"),
    "decay_sign_flipped": ("(float)(1.0 - lr * weight_decay)", "(float)(1.0 + lr * weight_decay)"),
    "eps_inside_sqrt": ("sqrtf(v1) * inv_sqrt_bc2 + epsf", "sqrtf(v1 + epsf) * inv_sqrt_bc2"),
    "v_uses_g_not_g2": ("c2 * (gi * gi)", "c2 * gi"),
    "betas_swapped_in_m": ("b1 * m[i] + c1 * gi", "b2 * m[i] + c2 * gi"),
    "clip_not_applied_to_g": ("float gi = g[i] * cf;", "float gi = g[i];"),
    "decay_applied_to_update": ("p[i] * decay - step_size * (m1 / d)",
                                "(p[i] - step_size * (m1 / d)) * decay * decay"),
    "ties_away_from_zero": ("nearbyint(units)", "round(units)"),
    "reduce_in_double": ("float acc = 0.0f;", "double acc = 0.0;"),
    "unscale_dropped": ("float gi = acc * inv_scale;\n        g[i] = gi;", "float gi = acc;\n        g[i] = gi;"),
    "accumulate_overwrites": ("float gi = g[i] + acc * inv_scale;", "float gi = acc * inv_scale;"),
    "accumulate_unscale_dropped": ("float gi = g[i] + acc * inv_scale;", "float gi = g[i] + acc;"),
    "local_accumulate_overwrites": ("acc[i] = first ? x : acc[i] + x;", "acc[i] = x;"),
    "local_accumulate_starts_at_zero": ("acc[i] = first ? x : acc[i] + x;",
                                        "acc[i] = (first ? 0.0f : acc[i]) + x;"),
    "reduce_f32_drops_first_replica": ("for (int32_t r = 0; r < n_replicas; ++r) {\n            float x = replicas[r][i];",
                                       "for (int32_t r = 1; r < n_replicas; ++r) {\n            float x = replicas[r][i];"),
    "nan_not_flagged": ("if (!isfinite(gi)) bad = 1;", "if (isinf(gi)) bad = 1;"),
    "clip_eps_dropped": ("max_norm / (*norm + 1e-6)", "max_norm / (*norm)"),
    "partition_floor_not_ceil": ("(numel % world_size != 0 ? 1 : 0)", "0"),
    "bucket_boundary_off_by_one": ("filled + n > bucket_size", "filled + n >= bucket_size"),
    "f16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_bias_off_by_one": ("e - 134", "e - 133"),
    "scaler_no_hysteresis_refill": ("s->good = 0;\n        s->hyst = s->hysteresis;",
                                    "s->good = 0;"),
    "scaler_halves_too_early": ("if (s->hyst > 1) {", "if (s->hyst > 2) {"),
}


def run_c_mutant(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    # a site shared by the plain and the accumulating reduce is mutated in both
    if src.count(before) < 1:
        return None
    mutant_src = tmp_path / "zero_oracle.c"
    mutant_src.write_text(src.replace(before, after))
    lib = str(tmp_path / "liboracle_mutant.so")
    oracle.compile_oracle(str(mutant_src), lib, strict=False)
    env = dict(os.environ, ZERO_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-W", "ignore::RuntimeWarning"] + PINS,
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")
CKPT_PINS = ["test_checkpoint_host.py::test_repartition_hand_example",
             "test_checkpoint_host.py::test_repartition_round_trip_and_empty_ranks",
             "test_checkpoint_host.py::test_oracle_gather_hand_example"]

PY_MUTANTS = {
    "predivide_dropped": ("return np.float32(1.0 / (float(loss_scale) * float(predivide)))",
                          "return np.float32(1.0 / float(loss_scale))"),
    "norm_restarts_every_rank": ("sumsq if last else 0.0", "0.0"),
    "overflow_does_not_skip": ("    if overflow:\n        return info\n", ""),
    "repartition_ranks_reversed": ("for r in range(from_world)] +",
                                   "for r in reversed(range(from_world))] +"),
    "gather_one_past_the_end": ("return flat[lo:hi].copy()", "return flat[lo:hi + 1].copy()"),
    "flatten_one_element_late": ("flat[int(off):int(off) + t.size] = t",
                                 "flat[int(off) + 1:int(off) + 1 + t.size] = t"),
    "cast_format_swapped": ("return f32_to_f16(p) if dtype == FP16 else f32_to_bf16(p)",
                            "return f32_to_bf16(p) if dtype == FP16 else f32_to_f16(p)"),
}


def run_pins_on_copy(tmp_path, py_src):
    """The pin tests, in a temporary tree whose oracle package has `py_src`
    as its Python layer and loads the oracle library as built."""
    root = tmp_path / "root"
    shutil.copytree(os.path.join(ROOT, "oracle"), root / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__", "*.so*"))
    (root / "oracle" / "__init__.py").write_text(py_src)
    shutil.copytree(HERE, root / "tests", ignore=shutil.ignore_patterns("__pycache__", "c"))
    # the copy's own directory comes first on the path (cwd and conftest);
    # the library package, which the checkpoint pins import, comes from ROOT
    env = dict(os.environ, ZERO_ORACLE_LIB=oracle.build(force=False), PYTHONPATH=ROOT)
    pins = [os.path.basename(f) for f in PINS] + CKPT_PINS
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-W", "ignore::RuntimeWarning"] + ["tests/" + f for f in pins],
                          cwd=str(root), env=env, capture_output=True, text=True, timeout=600)


def run_python_mutant(name, tmp_path):
    before, after = PY_MUTANTS[name]
    src = open(PY_SRC).read()
    if src.count(before) < 1:
        return None
    return run_pins_on_copy(tmp_path, src.replace(before, after))


@pytest.fixture(scope="module")
def pin_runs(tmp_path_factory):
    """Every mutant's pin run (and one on an unmutated copy), several at a
    time: each is an independent subprocess in its own directory."""
    jobs = {("c", n): run_c_mutant for n in MUTANTS}
    jobs.update({("py", n): run_python_mutant for n in PY_MUTANTS})
    jobs[("py", None)] = lambda _, tmp: run_pins_on_copy(tmp, open(PY_SRC).read())
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as pool:
        futs = {k: pool.submit(f, k[1], tmp_path_factory.mktemp("%s_%s" % (k[0], k[1])))
                for k, f in jobs.items()}
        return {k: f.result() for k, f in futs.items()}


def test_pins_pass_on_an_unmutated_copy(pin_runs):
    r = pin_runs[("py", None)]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, pin_runs):
    r = pin_runs[("c", name)]
    assert r is not None, "mutation site not found: " + name
    assert r.returncode == 1, "mutant survived the pins: " + name + "\n" + r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_pins_kill_python_mutant(name, pin_runs):
    r = pin_runs[("py", name)]
    assert r is not None, "mutation site not found: " + name
    assert r.returncode == 1, "mutant survived the pins: " + name + "\n" + r.stdout[-2000:]
