"""Pins of the oracle's FP4 E2M1 grid (Quantization concepts guide, "FP4 with block
scales": 1 sign, 2 exponent and 1 mantissa bit; the values 0, 0.5, 1, 1.5, 2, 3, 4, 6
and their negatives; one scale per small block)."""
import numpy as np

from oracle import gptq_oracle as o


def test_e2m1_table_is_the_bit_format_and_the_page_list():
    """Decoding (e, m) as a float with 2 exponent bits (bias 1, e = 0 subnormal) and one
    mantissa bit gives exactly the page's eight magnitudes, in code order."""
    vals = []
    for e in range(4):
        for m in range(2):
            vals.append(m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))
    assert vals == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(o.E2M1_VALUES) == vals


def test_e2m1_rounding_ties_to_even_and_saturates():
    for v in o.E2M1_VALUES:   # every grid value, either sign, maps to itself
        assert o.E2M1_VALUES[o.e2m1_round(np.array([v]))[0]] == v
        assert o.E2M1_VALUES[o.e2m1_round(np.array([-v]))[0]] == v
    mids = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for t, v in mids.items():
        assert o.E2M1_VALUES[o.e2m1_round(np.array([t]))[0]] == v, t
    assert o.E2M1_VALUES[o.e2m1_round(np.array([7.0]))[0]] == 6.0
    assert o.E2M1_VALUES[o.e2m1_round(np.array([2.6]))[0]] == 3.0


def test_e2m1_group_scale_and_codes():
    """The group's largest magnitude lands on +-6; codes carry the sign in bit 3."""
    W = np.array([[0.6, -0.05, 0.3, -0.6, 0.0, 0.12, -0.2, 0.45]])
    p = o.Params(bits=4, group_size=0, fp4=True)
    r = o.rtn(W, p)
    assert abs(float(r.scales16[0, 0]) - 0.1) < 1e-4          # 0.6 / 6
    assert r.codes[0, 0] == 7 and r.codes[0, 3] == 8 + 7        # +6, -6
    assert r.codes[0, 4] == 0
    # S16 = fp16(0.1): -0.05 -> -0.5, 0.3 -> 3, 0.12 -> 1.2 -> 1, -0.2 -> -2, 0.45 -> 4.5 -> 4 (nearer than 6)
    assert list(r.codes[0]) == [7, 8 + 1, 5, 8 + 7, 0, 2, 8 + 4, 6]
    deq = o.dequantize_e2m1(r.codes, r.scales16, 0)
    assert np.array_equal(deq.astype(np.float64), r.what)


def test_e2m1_identity_hessian_and_blocking():
    rng = np.random.default_rng(11)
    W = rng.standard_normal((6, 256)) * 0.02
    for g in (128, 0, -1):
        p = o.Params(bits=4, group_size=g, fp4=True)
        a, b = o.gptq_blocked(W, np.eye(256), p), o.rtn(W, p)
        assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales16, b.scales16)
    X = rng.standard_normal((512, 256))
    U, _ = o.prepare_u(o.hessian([X]), 0.01)
    p = o.Params(bits=4, group_size=128, fp4=True)
    a, b = o.gptq_blocked(W, U, p), o.gptq(W, U, p)
    assert np.array_equal(a.scales16, b.scales16)
    assert np.mean(a.codes == b.codes) >= 0.999


def test_mxfp4_scale_is_the_power_of_two_above_absmax_over_6():
    """MXFP4 ("FP4 with block scales": a power-of-two scale): S = 2^ceil(log2(absmax/6)),
    so absmax / 6 <= S < absmax / 3 and the largest magnitude lands in (3, 6]."""
    rng = np.random.default_rng(12)
    W = rng.standard_normal((40, 128)) * 0.02
    W[0, :] = 0.0
    W[0, 5] = 0.75            # absmax / 6 = 0.125 exactly: S = 0.125, the value lands on 6
    W[1, 7] = -0.6            # absmax / 6 = 0.1 -> S = 0.125, -0.6 / 0.125 = -4.8 -> -4
    p = o.Params(bits=4, group_size=0, fp4=True, mx=True)
    r = o.rtn(W, p)
    S = r.scales16.astype(np.float64)[:, 0]
    a = np.max(np.abs(W), axis=1)
    assert np.all(np.exp2(np.round(np.log2(S))) == S)
    assert np.all(a / 6 <= S) and np.all(S < a / 3)
    assert S[0] == 0.125 and r.codes[0, 5] == 7
    assert S[1] == 0.125 and r.codes[1, 7] == 8 + 6
    # the pre-rounding scale is absmax / 6, before the power of two
    assert r.S[0, 0] == 0.125 and r.S[1, 0] == 0.6 / 6
    a2 = o.gptq_blocked(W, np.eye(128), dataclasses_replace(p, group_size=32))
    b2 = o.rtn(W, dataclasses_replace(p, group_size=32))
    assert np.array_equal(a2.codes, b2.codes) and np.array_equal(a2.scales16, b2.scales16)


def dataclasses_replace(p, **kw):
    import dataclasses
    return dataclasses.replace(p, **kw)
