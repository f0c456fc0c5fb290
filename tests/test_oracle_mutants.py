"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutant is a copy of the oracle source with one planted mistake (a
dropped term, a wrong sign or operand, a wrong rounding rule).  It is built
to a temporary library and the pin tests run against it in a subprocess;
every mutant must make them fail.  Nothing here touches the HIP library.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "zero_oracle.c")
PINS = [os.path.join(HERE, f) for f in
        ("test_oracle_partition.py", "test_oracle_formats.py", "test_oracle_step.py")]

MUTANTS = {
    "m_bias_correction_dropped": ("double m_hat = m1 / bc1;", "double m_hat = m1;"),
    "v_bias_correction_dropped": ("double v_hat = v1 / bc2;", "double v_hat = v1;"),
    "decay_sign_flipped": ("pi - lr * weight_decay * pi", "pi + lr * weight_decay * pi"),
    "eps_inside_sqrt": ("(sqrt(v_hat) + eps)", "sqrt(v_hat + eps)"),
    "v_uses_g_not_g2": ("(1.0 - beta2) * gi * gi", "(1.0 - beta2) * gi"),
    "betas_swapped_in_m": ("beta1 * (double)m[i] + (1.0 - beta1)",
                           "beta2 * (double)m[i] + (1.0 - beta2)"),
    "clip_not_applied_to_g": ("double gi = (double)g[i] * coef;", "double gi = (double)g[i];"),
    "ties_away_from_zero": ("nearbyint(units)", "round(units)"),
    "reduce_in_double": ("float acc = 0.0f;", "double acc = 0.0;"),
    "unscale_dropped": ("float gi = acc * inv_scale;", "float gi = acc;"),
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


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, "mutation site not found: " + name
    mutant_src = tmp_path / "zero_oracle.c"
    mutant_src.write_text(src.replace(before, after))
    lib = str(tmp_path / "liboracle_mutant.so")
    oracle.compile_oracle(str(mutant_src), lib, strict=False)
    env = dict(os.environ, ZERO_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-W", "ignore::RuntimeWarning"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, "mutant survived the pins: " + name + "\n" + r.stdout[-2000:]
