"""Helpers shared by the GPU parity tests: device placement of the seeded inputs
and the element-by-element parity rules against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import synth
from oracle import gptq_oracle as o


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(arr: np.ndarray, dtype: str):
    """Host array in storage dtype -> device tensor (bf16 from uint16 bits, or f32)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(arr).astype(np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def layer_x(L: synth.Layer) -> np.ndarray:
    return np.concatenate(list(synth.x_chunks(L)))


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """The stored codes of the GPU byte layout: the 3-bit stream (the oracle's pinned
    unpacking), or plain nibble unpacking (column 2k low nibble), or one per byte."""
    packed = np.asarray(packed, dtype=np.uint8)
    if bits == 3:
        return o.unpack(packed, 3)
    if bits == 8:
        return packed.copy()
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def _fp16_boundary_rel(S: np.ndarray) -> np.ndarray:
    """Relative distance of S to the nearest fp16 rounding boundary."""
    S = np.asarray(S, dtype=np.float64)
    s16 = S.astype(np.float16)
    up = np.nextafter(s16, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(s16, np.float16(0)).astype(np.float64)
    s = s16.astype(np.float64)
    return np.minimum(np.abs(S - (s + up) / 2), np.abs(S - (s + dn) / 2)) / S


def _pow2_boundary_rel(S: np.ndarray) -> np.ndarray:
    """Relative distance of S to the nearest power of two (where the smallest power of
    two not below S changes)."""
    S = np.asarray(S, dtype=np.float64)
    return np.abs(S - np.exp2(np.round(np.log2(S)))) / S


# E2M1 rounding midpoints (half-way between neighbouring magnitudes 0, 0.5, 1, 1.5, 2,
# 3, 4, 6), in units of the group scale
E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def tie_distance(t, p) -> np.ndarray:
    """Distance of the oracle's pre-rounding code value to the nearest rounding tie of
    the grid: a half-integer for the integer grids; for E2M1 (t in half units of the
    scale) the nearest midpoint, in units of the scale."""
    t = np.asarray(t, dtype=np.float64)
    if p.fp4:
        a = np.abs(t) / 2.0
        return np.min(np.abs(a[..., None] - E2M1_MIDPOINTS), axis=-1)
    return np.abs(t - np.floor(t) - 0.5)


def stored_to_signed(codes, p) -> np.ndarray:
    """Stored unsigned code -> the oracle's code value q (signed grid; E2M1: 2 x value)."""
    u = np.asarray(codes).astype(np.int64)
    if p.fp4:
        mag = 2.0 * o.E2M1_VALUES[u & 7]
        return np.where(u & 8, -mag, mag).astype(np.int64)
    return u - p.zero_offset


def _gpu_group(s16, z, p):
    """GPU scale and stored zero -> (S16, Z) as the oracle's sweep uses them."""
    s = float(np.float16(s16))
    if p.fp4:
        return s / 2.0, 0
    return s, int(z) - p.zero_offset


def _first_event(r, codes_gpu, s16_gpu, z_gpu, cur, g, d_col):
    """First difference in row r, in column order: ('group', k) at a group's first
    column (scale or zero), else ('code', c); None when the row matches."""
    bad_g = np.nonzero((s16_gpu[r] != cur["s16"][r]) | (z_gpu[r] != cur["z"][r]))[0]
    bad_c = np.nonzero(codes_gpu[r] != cur["codes"][r])[0]
    eg = bad_g[0] * g if bad_g.size else d_col
    ec = bad_c[0] if bad_c.size else d_col
    if eg >= d_col and ec >= d_col:
        return None
    return ("group", int(bad_g[0])) if eg <= ec else ("code", int(ec))


def tie_consistent_parity(codes_gpu, s16_gpu, z_gpu, W, U, p, tie_window, s_window=1e-5, ref=None,
                          max_ties_per_row=8):
    """Compare the GPU's codes, scales and zeros with the oracle, following the GPU's side
    of every rounding tie.

    Row by row (rows are independent given U), in column order: the first difference
    (a code, or a group's scale or zero at the group's first column) must sit on a tie of
    the oracle's own decision: its pre-rounding value within ``tie_window`` of a rounding
    midpoint, the pre-rounding scale within ``s_window`` (relative) of an fp16 rounding
    boundary (of a power of two for MXFP4), or the zero point's pre-rounding value within
    ``tie_window`` of a half-integer.  Both sides of a tie follow the rule, so the oracle
    is then run again on that row with the GPU's decision fixed there, and the rest of the
    row must match that run under the same rule, again and again until the row matches
    (at most ``max_ties_per_row`` ties).  What follows a tie is therefore checked, not
    only counted.

    Returns the plain match rates against the unforced oracle, the number of ties taken,
    the unjustified differences, and the tie-consistent oracle result (codes, scales16,
    zeros, what for every row)."""
    codes_gpu = np.asarray(codes_gpu).astype(np.int64)
    s16_gpu = np.asarray(s16_gpu).astype(np.float16)
    z_gpu = np.asarray(z_gpu).astype(np.int64)
    d_row, d_col = codes_gpu.shape
    g = p.group(d_col)
    if ref is None:
        ref = o.gptq_blocked(W, U, p)
    cur = dict(codes=ref.codes.astype(np.int64).copy(), s16=ref.scales16.astype(np.float16).copy(),
               z=ref.zeros.astype(np.int64).copy(), what=ref.what.copy(), t=ref.t_at_q.copy(), S=ref.S.copy(),
               zt=ref.z_t.copy())
    code_match = float(np.mean(codes_gpu == cur["codes"]))
    group_match = float(np.mean((s16_gpu == cur["s16"]) & (z_gpu == cur["z"])))
    forced = {r: {} for r in range(d_row)}
    unjustified, ties = [], []
    active = [r for r in range(d_row) if _first_event(r, codes_gpu, s16_gpu, z_gpu, cur, g, d_col) is not None]
    rows_with_events = len(active)
    for rnd in range(max_ties_per_row + 1):
        rerun = []
        for r in active:
            ev = _first_event(r, codes_gpu, s16_gpu, z_gpu, cur, g, d_col)
            if ev is None:
                continue
            kind, i = ev
            if rnd == max_ties_per_row:
                unjustified.append((r, "more ties than allowed", kind, i))
                continue
            if kind == "code":
                dist = float(tie_distance(cur["t"][r, i], p))
                if dist >= tie_window:
                    unjustified.append((r, "code", i, float(cur["t"][r, i]), int(codes_gpu[r, i]),
                                        int(cur["codes"][r, i])))
                    continue
                forced[r][("q", i)] = int(stored_to_signed(codes_gpu[r, i], p))
            else:
                S = float(cur["S"][r, i])
                if s16_gpu[r, i] != cur["s16"][r, i]:
                    near = _pow2_boundary_rel(S) if p.mx else _fp16_boundary_rel(np.array([S]))[0]
                    dist = float(near)
                    ok = dist < s_window
                else:
                    dist = float(tie_distance(cur["zt"][r, i], o.Params(bits=8)))
                    ok = dist < tie_window
                if not ok:
                    unjustified.append((r, "group", i, S, float(s16_gpu[r, i]), float(cur["s16"][r, i]),
                                        int(z_gpu[r, i]), int(cur["z"][r, i])))
                    continue
                forced[r][("g", i)] = _gpu_group(s16_gpu[r, i], z_gpu[r, i], p)
            ties.append((r, kind, i, dist))
            rerun.append(r)
        if not rerun:
            break
        rows = np.array(rerun)
        sub = {}
        for j, r in enumerate(rows):
            for (kind, i), v in forced[r].items():
                sub[(kind, j, i)] = v
            if p.group_size < 0 and ("g", 0) not in forced[r]:
                # per tensor: the range spans every row, so a subset keeps the full run's
                sub[("g", j, 0)] = _gpu_group(cur["s16"][r, 0], cur["z"][r, 0], p)
        res = o.gptq_blocked(np.asarray(W)[rows], U, p, forced=sub)
        cur["codes"][rows] = res.codes
        cur["s16"][rows] = res.scales16.astype(np.float16)
        cur["z"][rows] = res.zeros
        cur["what"][rows] = res.what
        cur["t"][rows] = res.t_at_q
        cur["S"][rows] = res.S
        cur["zt"][rows] = res.z_t
        active = list(rows)
    final_equal = bool(np.array_equal(codes_gpu, cur["codes"]) and np.array_equal(s16_gpu, cur["s16"])
                       and np.array_equal(z_gpu, cur["z"]))
    return dict(code_match=code_match, group_match=group_match, rows_with_events=rows_with_events,
                ties=ties, unjustified=unjustified, final_equal=final_equal, codes=cur["codes"],
                scales16=cur["s16"], zeros=cur["z"], what=cur["what"], plain_what=ref.what)


def assert_parity(rep, log_fn=None, min_code_match=0.999):
    """The code bar of the comparison: at least ``min_code_match`` of the codes equal the
    plain oracle's, every difference sits on a tie (first in its row, or after the
    oracle followed the GPU's side of the earlier ties), and after following those ties
    codes, scales and zeros are all equal."""
    if log_fn:
        worst = max((t[3] for t in rep["ties"]), default=0.0)
        log_fn(f"  codes {rep['code_match']:.6f} groups {rep['group_match']:.6f} rows with events "
               f"{rep['rows_with_events']} ties followed {len(rep['ties'])} (largest distance {worst:.2e}) "
               f"unjustified {rep['unjustified'][:3]}")
    assert rep["code_match"] >= min_code_match, rep["code_match"]
    assert not rep["unjustified"], rep["unjustified"][:5]
    assert rep["final_equal"]


def check_recon(H, W, What_gpu, rep, log_fn=None):
    """Layer objective parity against the tie-consistent oracle: every row to 1e-5
    relative and the layer total to 1e-3 relative.  The difference from the plain
    oracle's objective (whose rows may sit on the other side of a tie) is logged."""
    eg = recon_rows(H, W, What_gpu)
    eo = recon_rows(H, W, rep["what"])
    ep = recon_rows(H, W, rep["plain_what"])
    row_rel = np.abs(eg - eo) / np.maximum(eo, 1e-300)
    worst_row = float(row_rel.max()) if row_rel.size else 0.0
    tot_rel = abs(eg.sum() - eo.sum()) / eo.sum()
    plain_rel = abs(eg.sum() - ep.sum()) / ep.sum()
    if log_fn:
        log_fn(f"  recon gpu {eg.sum():.6e} oracle {eo.sum():.6e} rel {tot_rel:.2e}; worst row {worst_row:.2e}; "
               f"plain oracle {ep.sum():.6e} (rel {plain_rel:.2e})")
    assert worst_row <= 1e-5, worst_row
    assert tot_rel <= 1e-3, tot_rel
    return eg.sum(), eo.sum()


def recon_rows(H: np.ndarray, W: np.ndarray, What: np.ndarray) -> np.ndarray:
    D = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    return 0.5 * np.einsum("ij,jk,ik->i", D, H, D)


def u_residual_ratio(U, H, js, percdamp=0.01, step=2048):
    """Property check of an fp32 factor U of (H + lambda I)^-1 = U^T U without factoring:
    r_j = U^T U (H + lambda I) e_j - e_j on the columns js, in fp64, against the
    componentwise bound of rounding an exact factor to fp32,
    |r_j| <= 2 * 2^-24 |U|^T |U| |(H + lambda I) e_j|.  Returns max |r| / (4 x bound) (at
    most 1 passes) and max |r|.  U and H (d x d, fp32) are read in row blocks of ``step``."""
    d = H.shape[0]
    js = np.asarray(js)
    lam = percdamp * float(np.mean(np.diag(H).astype(np.float64)))
    V = H[:, js].astype(np.float64)
    V[js, np.arange(js.size)] += lam
    a, ab = np.zeros((d, js.size)), np.zeros((d, js.size))
    for r0 in range(0, d, step):
        Ub = U[r0:r0 + step].astype(np.float64)
        a[r0:r0 + step] = Ub @ V
        ab[r0:r0 + step] = np.abs(Ub) @ np.abs(V)
    res, bnd = np.zeros((d, js.size)), np.zeros((d, js.size))
    for r0 in range(0, d, step):
        Ub = U[r0:r0 + step].astype(np.float64)
        res += Ub.T @ a[r0:r0 + step]
        bnd += np.abs(Ub).T @ ab[r0:r0 + step]
    res[js, np.arange(js.size)] -= 1.0
    bound = 2.0 * 2.0 ** -24 * bnd
    return float(np.max(np.abs(res) / (4.0 * bound + 1e-300))), float(np.max(np.abs(res)))
