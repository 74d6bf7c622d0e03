"""Pins of the oracle's OBQ (the per-row greedy method GPTQ is compared with; GPTQ
summary page, OBQ background): the OBS step against a direct least-squares solve and
a direct inverse, the diagonal-Hessian case (round-to-nearest), greedy selection by
the smallest added error, and the exhaustive optimum as a lower bound."""
import numpy as np

from oracle import gptq_oracle as o


def _spd(d, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((4 * d, d))
    X[:, 0] *= 5.0
    return o.damp(o.hessian([X]), 0.01)[0]


def test_obs_step_matches_direct_solve_and_inverse():
    """After quantizing j, the remaining weights minimise (w' - w)^T H (w' - w) with
    w'_j = q(w_j) fixed: delta_F = -H_FF^-1 H_Fj (q(w_j) - w_j); and the updated inverse
    equals the inverse of H restricted to the remaining weights."""
    d = 7
    H = _spd(d, 1)
    w = np.random.default_rng(2).standard_normal(d) * 0.3
    p = o.Params(bits=3, group_size=0, sym=False)
    _, S16, Z, _ = o.group_params(w[None, :], p)
    j, qj, whj, w1, F1, live = o.obq_step(w, np.linalg.inv(H), np.ones(d, bool), S16[0], int(Z[0]), p)
    F = np.flatnonzero(live)
    delta = -np.linalg.solve(H[np.ix_(F, F)], H[F, j] * (whj - w[j]))
    assert np.allclose(w1[F], w[F] + delta, rtol=0, atol=1e-12)
    assert np.allclose(F1[np.ix_(F, F)], np.linalg.inv(H[np.ix_(F, F)]), rtol=1e-10, atol=1e-12)
    assert np.all(F1[j, :] == 0) and np.all(F1[:, j] == 0)


def test_obq_greedy_picks_smallest_added_error():
    d = 6
    H = _spd(d, 3)
    Hinv = np.linalg.inv(H)
    w = np.random.default_rng(4).standard_normal(d) * 0.3
    p = o.Params(bits=4, group_size=0, sym=False)
    _, S16, Z, _ = o.group_params(w[None, :], p)
    wh = S16[0] * (o.decide_codes(w, np.full(d, S16[0]), np.full(d, Z[0]), p) - Z[0])
    added = (w - wh) ** 2 / np.diag(Hinv)
    j = o.obq_step(w, Hinv, np.ones(d, bool), S16[0], int(Z[0]), p)[0]
    assert j == int(np.argmin(added))


def test_obq_diagonal_hessian_is_round_to_nearest():
    """A diagonal H couples no weights: no update moves anything, in any order."""
    rng = np.random.default_rng(5)
    W = rng.standard_normal((9, 40)) * 0.02
    Hd = np.diag(rng.random(40) + 0.5)
    for bits, sym in ((4, False), (3, True)):
        p = o.Params(bits=bits, group_size=0, sym=sym)
        res, order = o.obq(W, Hd, p)
        ref = o.rtn(W, p)
        assert np.array_equal(res.codes, ref.codes)
        assert np.array_equal(res.scales16, ref.scales16) and np.array_equal(res.zeros, ref.zeros)
        assert all(sorted(order[r]) == list(range(40)) for r in range(9))


def test_obq_not_below_exhaustive_optimum():
    """On tiny rows the exhaustive minimum of the layer objective bounds OBQ from below,
    and OBQ does at least as well as round-to-nearest on these correlated inputs."""
    d = 5
    H = _spd(d, 6)
    rng = np.random.default_rng(7)
    p = o.Params(bits=2 + 1, group_size=0, sym=False)
    W = rng.standard_normal((6, d)) * 0.3
    res, _ = o.obq(W, H, p)
    rt = o.rtn(W, p)
    for r in range(6):
        e_obq = (W[r] - res.what[r]) @ H @ (W[r] - res.what[r])
        e_rtn = (W[r] - rt.what[r]) @ H @ (W[r] - rt.what[r])
        best, _ = o.brute_force_row(W[r], H, float(res.scales16[r, 0]), int(res.zeros[r, 0]), p)
        assert best <= e_obq + 1e-12
        assert e_obq <= e_rtn + 1e-12
