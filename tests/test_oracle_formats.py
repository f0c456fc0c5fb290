"""Pins for the oracle's fp16 / bf16 conversions (CPU only).

Decoding is checked exhaustively over all 2^16 codes against numpy's
float16 and torch's bfloat16 (library routines).  Encoding (round to
nearest, ties to even) is checked against the same libraries on every
midpoint between neighbouring codes, one fp32 step either side of it, the
overflow edge and 2^22 random fp32 patterns, and against an exact-rational
rounding written from the IEEE-754 definition on a random sample.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def same_bits_or_both_nan_f32(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return nan | (a.view(np.uint32) == b.view(np.uint32))


def same_code_or_both_nan(a, b, dtype):
    a = np.asarray(a, np.uint16)
    b = np.asarray(b, np.uint16)
    if dtype == oracle.FP16:
        isnan = lambda c: ((c & 0x7C00) == 0x7C00) & ((c & 0x03FF) != 0)
    else:
        isnan = lambda c: ((c & 0x7F80) == 0x7F80) & ((c & 0x007F) != 0)
    return (isnan(a) & isnan(b)) | (a == b)


def lib_f16(x):
    # overflow to inf is the expected result for values past the fp16 range
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def lib_bf16(x):
    t = torch.from_numpy(np.asarray(x, np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_decode_f16_exhaustive():
    got = oracle.f16_to_f32(ALL16)
    ref = ALL16.view(np.float16).astype(np.float32)
    assert same_bits_or_both_nan_f32(got, ref).all()


def test_decode_bf16_exhaustive():
    got = oracle.bf16_to_f32(ALL16)
    ref = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert same_bits_or_both_nan_f32(got, ref).all()


def midpoint_probes(decode):
    """All midpoints between neighbouring finite codes of one sign, and the
    fp32 values one step either side (midpoints are exact in fp32)."""
    codes = np.arange(0, 0x7C00 if decode is oracle.f16_to_f32 else 0x7F80,
                      dtype=np.uint32).astype(np.uint16)
    vals = decode(codes).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    x = np.concatenate([mids, up, dn, vals.astype(np.float32)])
    return np.concatenate([x, -x])


def random_patterns(n=1 << 22):
    rng = np.random.default_rng(7)
    return rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


def test_encode_f16_midpoints_and_random():
    edges = np.array([65504, 65519.996, 65520, 65535, 65536, 1e9, np.inf, -np.inf,
                      np.nan, 2.0**-24, 2.0**-25, 1.5 * 2.0**-25, 2.0**-26,
                      np.nextafter(np.float32(2.0**-25), np.float32(1)), 0.0, -0.0],
                     dtype=np.float32)
    for x in (midpoint_probes(oracle.f16_to_f32), random_patterns(), edges):
        assert same_code_or_both_nan(oracle.f32_to_f16(x), lib_f16(x), oracle.FP16).all()


def test_encode_bf16_midpoints_and_random():
    big = np.float32(np.finfo(np.float32).max)
    edges = np.array([big, -big, np.inf, np.nan, 2.0**-133, 2.0**-134,
                      np.float32(1.5 * 2.0**-134), 1e-45, 0.0, -0.0, 3.3961776e38,
                      3.3961775e38], dtype=np.float32)
    for x in (midpoint_probes(oracle.bf16_to_f32), random_patterns(), edges):
        assert same_code_or_both_nan(oracle.f32_to_bf16(x), lib_bf16(x), oracle.BF16).all()


def exact_rne(x: float, frac_bits: int, emin: int, max_finite: Fraction) -> Fraction:
    """Round a finite nonzero value to the format, from the definition: the
    two nearest representable values, ties to the even significand."""
    a = abs(Fraction(x))
    k = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** k > a:
        k -= 1
    while Fraction(2) ** (k + 1) <= a:
        k += 1
    q = Fraction(2) ** (max(k, emin) - frac_bits)
    lo = (a // q) * q
    hi = lo + q
    if a - lo < hi - a:
        r = lo
    elif hi - a < a - lo:
        r = hi
    else:
        r = lo if (lo / q) % 2 == 0 else hi
    if r > max_finite:
        return None                      # overflows to infinity
    return r if x > 0 else -r


def test_encode_against_exact_rational():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, size=3000, dtype=np.uint64).astype(np.uint32)
    xs = bits.view(np.float32)
    xs = xs[np.isfinite(xs) & (xs != 0)]
    # also values inside the fp16 range, where rounding is most exercised
    xs = np.concatenate([xs, (rng.standard_normal(3000) * 100).astype(np.float32)])
    f16max = Fraction(65504)
    bfmax = Fraction(255) * Fraction(2) ** 120
    h = oracle.f16_to_f32(oracle.f32_to_f16(xs))
    b = oracle.bf16_to_f32(oracle.f32_to_bf16(xs))
    for i, x in enumerate(xs.tolist()):
        r = exact_rne(x, 10, -14, f16max)
        assert (np.isinf(h[i]) and r is None) or Fraction(float(h[i])) == r
        r = exact_rne(x, 7, -126, bfmax)
        assert (np.isinf(b[i]) and r is None) or Fraction(float(b[i])) == r


def test_to_low_precision_follows_the_requested_format():
    """The step's cast picks its encoder by the parameter format: fp16 codes
    for FP16 and bfloat16 codes for BF16, each against torch's own
    round-to-nearest-even cast, on values where the two formats differ
    (bfloat16's range and fp16's finer fraction)."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(4096).astype(np.float32) * 100,
                        np.float32([1e5, -3e38, 1.0009765625, 2.0 ** -20, 65520.0])])
    f16 = oracle.to_low_precision(x, oracle.FP16)
    bf16 = oracle.to_low_precision(x, oracle.BF16)
    t = torch.from_numpy(x)
    assert np.array_equal(f16, t.to(torch.float16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(bf16, t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert not np.array_equal(f16, bf16)
