"""The GPU-vs-oracle parity rules themselves (tests/gpu_helpers.py), on the CPU: a
result that takes the other side of a rounding tie, and everything that follows from
it, passes; a difference away from a tie fails, also when it comes after a tie in the
same row.  The "other" results here are the oracle's own runs with a decision fixed."""
import numpy as np

import synth
from gpu_helpers import assert_parity, check_recon, tie_consistent_parity, u_residual_ratio
from oracle import gptq_oracle as o


def _layer(p, d_row=24, d_col=256, seed=3):
    L = synth.scaled(synth.config_layers(2)[0], d_row, d_col, 4 * d_col, seed_offset=seed)
    W = synth.w_as_f64(synth.weights(L))
    X = np.concatenate([synth.x_as_f64(c) for c in synth.x_chunks(L)])
    H = o.hessian([X])
    U, _ = o.prepare_u(H, 0.01)
    return W, H, U


def _as_gpu(res, p):
    return res.codes.copy(), res.scales16.copy(), res.zeros.copy()


def _tie_row(W, U, p, r, c):
    """W with row r's column c moved onto an exact rounding tie of the oracle's decision
    (the weight is not its group's extreme, so the group's scale and zero stay)."""
    ref = o.gptq_blocked(W, U, p)
    k = c // p.group(W.shape[1])
    S16, Z = ref.scales16[r, k].astype(np.float64), ref.zeros[r, k] - p.zero_offset
    w_now = ref.w_at_q[r, c]
    t = w_now / S16 + Z
    target = (np.floor(t) + 0.5 - Z) * S16           # the tie nearest below/above
    W2 = W.copy()
    W2[r, c] += target - w_now                         # earlier columns do not move column c's own shift
    return W2


def test_other_side_of_a_tie_and_its_cascade_pass():
    p = o.Params(bits=4, group_size=128)
    W, H, U = _layer(p)
    r, c = 5, 70
    W2 = _tie_row(W, U, p, r, c)
    ref = o.gptq_blocked(W2, U, p)
    assert abs(ref.t_at_q[r, c] - np.floor(ref.t_at_q[r, c]) - 0.5) < 1e-9
    other = o.gptq_blocked(W2, U, p, forced={("q", r, c): int(ref.q[r, c]) + 1})
    assert not np.array_equal(other.codes[r], ref.codes[r])
    rep = tie_consistent_parity(*_as_gpu(other, p), W2, U, p, tie_window=1e-3, ref=ref)
    assert len(rep["ties"]) == 1 and rep["ties"][0][:3] == (r, "code", c)
    assert_parity(rep, min_code_match=0.99)   # one flipped row of 24 moves its later codes
    check_recon(H, W2, other.what, rep)


def test_difference_away_from_a_tie_fails():
    p = o.Params(bits=4, group_size=128)
    W, H, U = _layer(p)
    ref = o.gptq_blocked(W, U, p)
    t = ref.t_at_q
    dist = np.abs(t - np.floor(t) - 0.5)
    r, c = np.unravel_index(np.argmax(dist[:, 10:]), dist[:, 10:].shape)
    c += 10
    q = int(ref.q[r, c])
    bad = o.gptq_blocked(W, U, p, forced={("q", int(r), int(c)): q + 1 if q < p.qmax else q - 1})
    rep = tie_consistent_parity(*_as_gpu(bad, p), W, U, p, tie_window=1e-3, ref=ref)
    assert rep["unjustified"] and rep["unjustified"][0][:3] == (r, "code", c)
    assert not rep["final_equal"]


def test_difference_after_a_tie_in_the_same_row_fails():
    """A mistake later in a row whose first difference is a legitimate tie is caught:
    the row is checked against the oracle run that follows the tie."""
    p = o.Params(bits=4, group_size=128)
    W, H, U = _layer(p)
    r, c = 7, 40
    W2 = _tie_row(W, U, p, r, c)
    ref = o.gptq_blocked(W2, U, p)
    follow = o.gptq_blocked(W2, U, p, forced={("q", r, c): int(ref.q[r, c]) + 1})
    dist = np.abs(follow.t_at_q[r] - np.floor(follow.t_at_q[r]) - 0.5)
    c2 = 150 + int(np.argmax(dist[150:]))
    q2 = int(follow.q[r, c2])
    bad = o.gptq_blocked(W2, U, p, forced={("q", r, c): int(ref.q[r, c]) + 1,
                                           ("q", r, c2): q2 + 1 if q2 < p.qmax else q2 - 1})
    rep = tie_consistent_parity(*_as_gpu(bad, p), W2, U, p, tie_window=1e-3, ref=ref)
    assert [t[:3] for t in rep["ties"]] == [(r, "code", c)]
    assert rep["unjustified"] and rep["unjustified"][0][:3] == (r, "code", c2)


def test_group_scale_tie_passes_and_zero_away_from_tie_fails():
    p = o.Params(bits=4, group_size=64)
    W, H, U = _layer(p, d_col=192)
    ref = o.gptq_blocked(W, U, p)
    # a zero point one off where min / S16 is not near a half-integer is caught
    zd = np.abs(ref.z_t - np.floor(ref.z_t) - 0.5)
    r, k = np.unravel_index(np.argmax(zd), zd.shape)
    s16 = float(ref.scales16[r, k])
    bad = o.gptq_blocked(W, U, p, forced={("g", int(r), int(k)): (s16, int(ref.zeros[r, k]) + 1)})
    rep = tie_consistent_parity(*_as_gpu(bad, p), W, U, p, tie_window=1e-3, ref=ref)
    assert rep["unjustified"] and rep["unjustified"][0][1] == "group"


def test_u_residual_check_passes_rounded_factor_and_catches_a_bad_tile():
    """The property check used where the oracle cannot factor: an exact factor rounded to
    fp32 passes; a 64 x 64 tile 1% off, or one row's tail 0.1% off, fails."""
    L = synth.scaled(synth.config_layers(5)[1], 64, 1024, 4096)
    X = np.concatenate([synth.x_as_f64(c) for c in synth.x_chunks(L)])
    H = o.hessian([X]).astype(np.float32)
    U, _ = o.prepare_u(H.astype(np.float64), 0.01)
    U32 = U.astype(np.float32)
    js = [0, 7, 512, 1023]
    assert u_residual_ratio(U32, H, js, step=256)[0] <= 1.0
    bad = U32.copy(); bad[64:128, 512:576] *= 1.01
    assert u_residual_ratio(bad, H, js, step=256)[0] > 1.0
    bad = U32.copy(); bad[700, 700:] *= 1.001
    assert u_residual_ratio(bad, H, js, step=256)[0] > 1.0
