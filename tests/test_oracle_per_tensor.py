"""Pins of the oracle's per-tensor granularity (one scale and zero point for the whole
matrix; Quantization concepts guide, "Choose granularity"): the guide's affine worked
example spread over two rows, the identity-Hessian invariant and blocked = unblocked."""
import json
import os

import numpy as np

from oracle import gptq_oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _example():
    with open(os.path.join(GOLD, "affine_int8_example.json")) as f:
        return json.load(f)


def test_per_tensor_worked_example_across_rows():
    """The range -1.8 .. 2.4 has its minimum in row 0 and its maximum in row 1: only a
    range taken over the whole matrix gives every row the page's S ~= 0.0165 and
    Z = -19 (109 on the unsigned grid), 0.5 -> 11 (139) and back to ~= 0.494."""
    g = _example()
    W = np.array([[g["vmin"], g["x"], 0.0, 0.3],
                  [0.7, -0.2, g["vmax"], 0.0]])
    p = o.Params(bits=8, group_size=-1, sym=False)
    r = o.rtn(W, p)
    assert r.scales16.shape == (2, 1)
    for row in range(2):
        assert abs(float(r.scales16[row, 0]) - g["S_approx"]) < 5e-5
        assert r.zeros[row, 0] == g["Z"] + 128
    assert r.codes[0, 0] == g["q_at_vmin"] + 128 and r.codes[1, 2] == g["q_at_vmax"] + 128
    assert r.codes[0, 1] == g["q"] + 128
    assert r.codes[0, 2] == g["q_at_zero"] + 128
    assert abs(r.what[0, 1] - g["xhat_approx"]) < 1e-3
    # one group per row gives row 0 the range -1.8 .. 0.5 instead: a different scale
    rr = o.rtn(W, o.Params(bits=8, group_size=0, sym=False))
    assert abs(float(rr.scales16[0, 0]) - g["S_approx"]) > 5e-3


def test_per_tensor_identity_hessian_is_round_to_nearest():
    """With H = I no error is propagated (U = I), so GPTQ at per-tensor granularity is
    round-to-nearest on the one tensor-wide grid, asymmetric and symmetric."""
    rng = np.random.default_rng(7)
    W = rng.standard_normal((12, 256)) * 0.02
    W[3, 17] = 0.2   # a row far wider than the others
    U = np.eye(256)
    for bits, sym in ((4, False), (3, True), (8, False)):
        p = o.Params(bits=bits, group_size=-1, sym=sym)
        a, b = o.gptq_blocked(W, U, p), o.rtn(W, p)
        assert np.array_equal(a.codes, b.codes)
        assert np.array_equal(a.scales16, b.scales16) and np.array_equal(a.zeros, b.zeros)
        assert np.all(a.scales16 == a.scales16[0, 0]) and np.all(a.zeros == a.zeros[0, 0])


def test_per_tensor_blocked_equals_unblocked():
    """Lazy blocking regroups the same updates: with a real H the blocked and unblocked
    sweeps give the same codes and the same tensor-wide parameters."""
    rng = np.random.default_rng(8)
    X = rng.standard_normal((512, 200))
    X[:, 5] *= 20.0
    H = o.hessian([X])
    U, _ = o.prepare_u(H, 0.01)
    W = rng.standard_normal((10, 200)) * 0.02
    p = o.Params(bits=4, group_size=-1, sym=False, block_size=128)
    a, b = o.gptq_blocked(W, U, p), o.gptq(W, U, p)
    assert np.array_equal(a.scales16, b.scales16) and np.array_equal(a.zeros, b.zeros)
    assert np.mean(a.codes == b.codes) >= 0.999
