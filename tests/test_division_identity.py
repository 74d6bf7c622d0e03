"""The sweep decides a code from t = fl32(w / S16).  On the GPU the quotient is formed
from the correctly rounded reciprocal r = RN(1 / S16): q0 = RN(w r), then one
correction with the exact residual w - q0 S16, t = RN(q0 + (w - q0 S16) r) (one fused
multiply-add, a single rounding).  This checks, in exact rational arithmetic, that the
sequence gives the IEEE quotient RN(w / S16) for every positive normal fp16 scale and
a seeded sample of weights (Markstein's correction theorem for a correctly rounded
reciprocal; no library division is involved in the check)."""
from fractions import Fraction

import numpy as np


def rn32(x: Fraction) -> Fraction:
    """Round a rational to the nearest float32 value (ties to even), exactly."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    # x in [2^e, 2^(e+1)): 24 significant bits -> quantum 2^(e-23)
    q = Fraction(2) ** (e - 23)
    m = x / q
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def gpu_quotient(w: Fraction, s: Fraction) -> Fraction:
    r = rn32(1 / s)
    q0 = rn32(w * r)
    res = rn32(w - q0 * s)           # one fused multiply-add (the residual is representable)
    return rn32(q0 + res * r)        # one fused multiply-add


def test_reciprocal_correction_equals_ieee_division():
    h = np.arange(0x0400, 0x7C00, dtype=np.uint16)          # every positive normal fp16
    scales = h.view(np.float16).astype(np.float64)
    rng = np.random.default_rng(20241203)
    n_bad = 0
    n = 0
    for k, s_f in enumerate(scales):
        s = Fraction(float(s_f))
        # weights: random float32 values of the sizes the sweep sees, plus quotients
        # placed just around half-integers (where the code decision flips)
        if k % 7 == 0:
            ws = rng.standard_normal(3).astype(np.float32) * np.float32(0.05)
            half = np.float32((rng.integers(-8, 8) + 0.5) * s_f)
            near = [half, np.nextafter(half, np.float32(np.inf)), np.nextafter(half, np.float32(-np.inf))]
            cands = list(ws) + near
        else:
            cands = list(rng.standard_normal(1).astype(np.float32) * np.float32(0.05))
        for w_f in cands:
            w = Fraction(float(w_f))
            n += 1
            if gpu_quotient(w, s) != rn32(w / s):
                n_bad += 1
    assert n > 35000
    assert n_bad == 0
