"""Pins for the oracle's RMSNorm (oracle/norm.py) against exact rational arithmetic, a closed form
and an invariance.  The reference values here are computed independently: sums of squares as exact
rationals, the square root to 60 decimal digits, and every fp32 / bf16 rounding by bracketing."""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

from oracle import norm


def _nearest_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (ties to even) fp32 of an exact rational in the normal range."""
    if fr == 0:
        return np.float32(0.0)
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    errs = [abs(Fraction(float(c)) - fr) for c in cands]
    best = min(errs)
    ties = [c for c, e in zip(cands, errs) if e == best]
    if len(ties) == 1:
        return ties[0]
    return [c for c in ties if (np.array(c, np.float32).view(np.uint32) & 1) == 0][0]


def _nearest_bf16(fr: Fraction) -> Fraction:
    """Nearest value with 8 significant bits (ties to even), exact."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    unit = Fraction(2) ** (e - 7)
    n = a / unit
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * unit


def _bf16_values(shape, seed, scale=1.0):
    r = np.random.default_rng(seed)
    v = (r.standard_normal(shape) * scale).astype(np.float32)
    return norm.round_bf16(v)


def _reference(x: np.ndarray, gamma: np.ndarray, eps: float):
    getcontext().prec = 60
    d = x.shape[1]
    e = Fraction(float(np.float32(eps)))
    inv = []
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        ss = sum(Fraction(float(v)) ** 2 for v in x[t])
        m = ss / d + e
        root = (Decimal(m.numerator) / Decimal(m.denominator)).sqrt()
        inv32 = _nearest_f32(Fraction(Decimal(1) / root))
        inv.append(inv32)
        for i in range(d):
            p = _nearest_f32(Fraction(float(x[t, i])) * Fraction(float(inv32)))
            q = _nearest_f32(Fraction(float(p)) * Fraction(float(gamma[i])))
            y[t, i] = float(_nearest_bf16(Fraction(float(q))))
    return np.array(inv, np.float32), y


def test_rmsnorm_matches_exact_rational_reference():
    for d, seed, scale in ((128, 0, 1.0), (256, 1, 37.0), (384, 2, 1e-3)):
        x = _bf16_values((6, d), seed, scale)
        gamma = _bf16_values((d,), seed + 10) + np.float32(1.0)
        gamma = norm.round_bf16(gamma)
        inv_ref, y_ref = _reference(x, gamma, 1e-6)
        assert np.array_equal(norm.inv_rms(x, 1e-6), inv_ref)
        assert np.array_equal(norm.rmsnorm(x, gamma, 1e-6), y_ref)


def test_constant_power_of_two_rows_give_gamma():
    d = 256
    gamma = _bf16_values((d,), 7)
    for c in (1.0, -4.0, 2.0 ** -20, 2.0 ** 30):
        x = np.full((1, d), c, np.float32)
        y = norm.rmsnorm(x, gamma, 0.0)             # inv = 1/|c| exactly, x * inv = +-1
        assert np.array_equal(y[0], np.sign(c) * gamma)


def test_power_of_two_scaling_invariance():
    x = _bf16_values((8, 512), 3)
    gamma = _bf16_values((512,), 4)
    y0 = norm.rmsnorm(x, gamma, 0.0)
    for k in (-12, -1, 3, 40):
        assert np.array_equal(norm.rmsnorm(np.ldexp(x, k).astype(np.float32), gamma, 0.0), y0)


def test_eps_only_matters_for_tiny_rows():
    x = _bf16_values((4, 128), 5, 1e-5)
    gamma = np.ones(128, np.float32)
    big, small = norm.rmsnorm(x, gamma, 1e-2), norm.rmsnorm(x, gamma, 1e-12)
    assert np.max(np.abs(big)) < 1e-2                 # eps dominates: output ~ x / 0.1
    rms = np.sqrt(np.mean(small.astype(np.float64) ** 2, axis=1))
    assert np.all(np.abs(rms - 1) < 1e-2)             # unit RMS up to bf16 rounding
