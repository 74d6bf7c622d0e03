"""Pins, in exact rational arithmetic (no GPU), of the rounding facts the kernels rely on
when they decide scales, zero points and codes from their fp32 values:

1. For an fp32 x and a positive integer d up to 255, rounding the correctly rounded fp32
   quotient x / d to fp16 (nearest even) gives the fp16 rounding of the exact x / d.
2. For an fp32 x and an fp16 s > 0, rounding the fp32 quotient x / s to an integer
   (nearest even) gives the rounding of the exact x / s wherever |x / s| < 4096.
3. A range mx - mn that is itself rounded to fp32 before the division can give the
   other fp16 neighbour; kept as a rounded difference plus its exact error (two-sum),
   the quotient's fp16 rounding is decided exactly by the sign of
   (xh - d m) + xl at the fp16 midpoint m next to the fp32 quotient.

Each is checked on values built to sit next to the rounding boundaries (one to three
fp32 ulps from an fp16 midpoint or a half-integer, and on it), where a mistake would
show."""
from fractions import Fraction

import numpy as np
import pytest

F32 = np.float32


def _f16_exact(q: Fraction) -> np.float16:
    """fp16 nearest (ties to even) of a positive rational, by exact comparison with the
    fp16 neighbours of its fp64 approximation."""
    c = np.float16(float(q))
    cands = {c, np.nextafter(c, np.float16(np.inf)), np.nextafter(c, np.float16(0))}
    best = sorted(cands, key=lambda v: (abs(Fraction(float(v)) - q), int(np.array(v).view(np.uint16)) & 1))
    return best[0]


def _rint_exact(q: Fraction) -> int:
    """Nearest integer, ties to even, of a rational."""
    f = q.numerator // q.denominator
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def _near(v: float, k: int) -> list:
    """fp32 values 0 .. k ulps on either side of v (rounded to fp32)."""
    x = F32(v)
    out = [x]
    up = dn = x
    for _ in range(k):
        up = np.nextafter(up, F32(np.inf))
        dn = np.nextafter(dn, F32(-np.inf))
        out += [up, dn]
    return out


def _midpoints(rng, n):
    """Midpoints between random adjacent positive normal fp16 numbers (fp64, exact)."""
    h = rng.integers(0x0400, 0x7BFF, size=n).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    return (lo + hi) / 2.0


@pytest.mark.parametrize("d", [3, 6, 7, 15, 127, 255])
def test_fp32_quotient_by_small_integer_rounds_to_fp16_exactly(d):
    rng = np.random.default_rng(d)
    n_checked = 0
    for m in _midpoints(rng, 400):
        for x in _near(m * d, 3):
            if not np.isfinite(x) or x <= 0:
                continue
            got = np.float16(F32(x) / F32(d))
            assert got == _f16_exact(Fraction(float(x)) / d), (x, d)
            n_checked += 1
    assert n_checked > 2000


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp32_quotient_by_fp16_scale_rounds_to_integer_exactly(seed):
    rng = np.random.default_rng(seed)
    s16 = rng.integers(0x0400, 0x7800, size=300).astype(np.uint16).view(np.float16)
    half = rng.integers(-4095, 4095, size=300) + 0.5
    for s, h in zip(s16, half):
        s32 = F32(s)
        for x in _near(float(h) * float(s), 3):
            if not np.isfinite(x):
                continue
            t = F32(x) / s32
            assert int(np.rint(t)) == _rint_exact(Fraction(float(x)) / Fraction(float(s))), (x, s, h)


def _two_sum(a, b):
    s = F32(a + b)
    bb = F32(s - a)
    return s, F32(F32(a - F32(s - bb)) + F32(b - bb))


def _f16_of_range(mx, mn, d):
    """fp16 of (mx - mn) / d from the rounded difference and its error, decided at the
    midpoint next to the fp32 quotient (the kernels' rule, restated)."""
    xh, xl = _two_sum(F32(mx), F32(-mn))
    s = F32(xh / F32(d))
    c = np.float16(s)
    if F32(c) == s:
        return c
    n = np.nextafter(c, np.float16(np.inf)) if s > F32(c) else np.nextafter(c, np.float16(0))
    m = F32(F32(F32(c) + F32(n)) * F32(0.5))
    r = F32(F32(xh - F32(F32(d) * m)) + xl)
    if r == 0:
        return c if (int(np.array(c).view(np.uint16)) & 1) == 0 else n
    return n if (r > 0) == (n > c) else c


@pytest.mark.parametrize("d", [3, 7, 15, 255])
def test_rounded_range_needs_its_error_term(d):
    rng = np.random.default_rng(100 + d)
    naive_miss = 0
    n_checked = 0
    for m in _midpoints(rng, 300):
        R = m * d
        for frac in (0.13, 0.5, 0.87):
            mn = F32(-frac * R)
            for mx in _near(float(mn) + R, 3):
                exact = _f16_exact((Fraction(float(mx)) - Fraction(float(mn))) / d)
                assert _f16_of_range(mx, mn, d) == exact, (mx, mn, d)
                naive_miss += np.float16(F32(F32(mx - mn) / F32(d))) != exact
                n_checked += 1
    assert n_checked > 2000
    assert naive_miss > 0
