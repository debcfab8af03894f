"""Pin for the oracle's fp32 fused multiply-add emulation: every result must equal the
exact rational a*b + c rounded once to fp32 (nearest, ties to even), computed here
with Python fractions and integer arithmetic -- an independent route."""
from fractions import Fraction

import numpy as np

from oracle.fparith import fma32


def rn32(q: Fraction) -> float:
    """Round a rational to the nearest fp32 (ties to even), gradual underflow."""
    if q == 0:
        return 0.0
    neg = q < 0
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = q / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    v = lo * quantum
    if v >= Fraction(2) ** 128:
        return -np.inf if neg else np.inf
    return -float(v) if neg else float(v)


def _check(a, b, c):
    got = fma32(a, b, c)
    for x, y, z, g in zip(a, b, c, got):
        want = rn32(Fraction(float(x)) * Fraction(float(y)) + Fraction(float(z)))
        assert np.float32(want).view(np.uint32) == np.float32(g).view(np.uint32) or \
            (want == 0 and g == 0), (x, y, z, g, want)


def test_random_operands_all_exponent_gaps():
    rng = np.random.default_rng(0)
    n = 20000
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    c = np.abs(rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))).astype(np.float32)
    _check(a, a, c)                       # the squared-error accumulation shape
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    _check(a, b, -c)


def test_double_rounding_midpoints_are_resolved():
    # a*b = 2^-24 (1 - 2^-46): c + a*b lands 2^-70 below an fp32 midpoint, which a
    # plain fp64 sum rounds onto the midpoint; the odd c makes ties-to-even go the
    # wrong way unless the TwoSum error is used.
    a = np.float32(2.0 ** -12 * (1 + 2.0 ** -23))
    b = np.float32(2.0 ** -12 * (1 - 2.0 ** -23))
    cs = [np.float32(1 + 2.0 ** -23), np.float32(1 + 3 * 2.0 ** -23), np.float32(1.0)]
    for c in cs:
        _check(np.array([a, b, -a]), np.array([b, a, -b]), np.array([c, c, c]))
    got = fma32(np.array([a]), np.array([b]), np.array([np.float32(1 + 2.0 ** -23)]))[0]
    assert got == np.float32(1 + 2.0 ** -23)
    # and just above a midpoint
    a2 = np.float32(2.0 ** -12 * (1 + 2.0 ** -22))
    b2 = np.float32(2.0 ** -12)
    _check(np.array([a2]), np.array([b2]), np.array([np.float32(1.0)]))


def test_subnormal_and_overflow_results():
    a = np.array([1e-30, 3e-39, 1e20, 2e19], np.float32)
    b = np.array([1e-15, 1.0, 1e20, 2e19], np.float32)
    c = np.array([1e-45, -2e-39, 0.0, 1e38], np.float32)
    _check(a, b, c)
