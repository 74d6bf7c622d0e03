"""Helpers shared by the GPU parity tests: device placement of the seeded inputs
and the element-by-element parity rules against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import synth


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
    """Plain nibble unpacking of the GPU byte layout (column 2k low nibble)."""
    packed = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return packed.copy()
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def _fp16_boundary_rel(S: np.ndarray) -> np.ndarray:
    """Relative distance of S to the nearest fp16 rounding boundary."""
    s16 = S.astype(np.float16)
    up = np.nextafter(s16, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(s16, np.float16(0)).astype(np.float64)
    s = s16.astype(np.float64)
    return np.minimum(np.abs(S - (s + up) / 2), np.abs(S - (s + dn) / 2)) / S


def _half_dist(t: np.ndarray) -> np.ndarray:
    """Distance of t to the nearest rounding tie (half-integer)."""
    t = np.asarray(t, dtype=np.float64)
    return np.abs(t - np.floor(t) - 0.5)


def parity_report(codes_gpu, s16_gpu, z_gpu, ref, group: int, tie_window: float, s_window: float = 1e-5):
    """Compare GPU outputs with the oracle, row by row.

    The first event of each row, in column order (a code mismatch, or a scale /
    zero mismatch at a group's first column), must be a near-tie of the oracle's own
    decision: the pre-rounding code value within ``tie_window`` of a half-integer,
    the pre-rounding scale within ``s_window`` (relative) of an fp16 rounding
    boundary, or the zero-point value within ``tie_window`` of a half-integer.
    Everything after it in that row is the cascade of that flip and is only counted.
    """
    codes_gpu = np.asarray(codes_gpu)
    d_row, d_col = codes_gpu.shape
    g = d_col if group == 0 else group
    ng = s16_gpu.shape[1]
    s_eq = np.asarray(s16_gpu, dtype=np.float16) == ref.scales16
    z_eq = np.asarray(z_gpu).astype(np.int64) == ref.zeros
    grp_ok = s_eq & z_eq
    code_eq = codes_gpu == ref.codes
    unjustified = []
    first_event_cols = []
    for r in range(d_row):
        bad_groups = np.nonzero(~grp_ok[r])[0]
        bad_cols = np.nonzero(~code_eq[r])[0]
        ev_g = bad_groups[0] * g if bad_groups.size else d_col
        ev_c = bad_cols[0] if bad_cols.size else d_col
        if ev_g >= d_col and ev_c >= d_col:
            continue
        if ev_g <= ev_c:
            k = bad_groups[0]
            ok = (not s_eq[r, k] and _fp16_boundary_rel(np.array([ref.S[r, k]]))[0] < s_window) or \
                 (s_eq[r, k] and not z_eq[r, k] and _half_dist(ref.z_t[r, k]) < tie_window)
            first_event_cols.append(ev_g)
            if not ok:
                unjustified.append((r, "group", int(k), float(ref.S[r, k]), float(s16_gpu[r, k]),
                                    float(ref.scales16[r, k]), int(z_gpu[r, k]), int(ref.zeros[r, k])))
        else:
            c = ev_c
            first_event_cols.append(c)
            if not (_half_dist(ref.t_at_q[r, c]) < tie_window):
                unjustified.append((r, "code", int(c), float(ref.t_at_q[r, c]), int(codes_gpu[r, c]),
                                    int(ref.codes[r, c])))
    event_rows = np.array(sorted(set(np.nonzero(~code_eq.all(axis=1))[0]) | set(np.nonzero(~grp_ok.all(axis=1))[0])),
                          dtype=np.int64)
    return dict(code_match=float(code_eq.mean()), group_match=float(grp_ok.mean()),
                rows_with_events=len(first_event_cols), unjustified=unjustified, event_rows=event_rows)


def check_recon(H, W, What_gpu, What_ref, event_rows, log_fn=None):
    """Layer objective parity.  Rows without any event must match to 1e-5 relative
    (only fp32-vs-fp64 rounding differs there).  The layer total must match to 1e-3
    relative plus the share of the oracle's total held by rows whose first event is
    a tie flip (a flip changes the rest of its row, and either side of a tie is a
    correct result)."""
    eg = recon_rows(H, W, What_gpu)
    eo = recon_rows(H, W, What_ref)
    clean = np.ones(eg.shape[0], dtype=bool)
    clean[event_rows] = False
    row_rel = np.abs(eg - eo) / np.maximum(eo, 1e-300)
    worst_clean = float(row_rel[clean].max()) if clean.any() else 0.0
    tot_rel = abs(eg.sum() - eo.sum()) / eo.sum()
    allowance = 1e-3 + float(eo[~clean].sum() / eo.sum())
    if log_fn:
        log_fn(f"  recon gpu {eg.sum():.6e} oracle {eo.sum():.6e} rel {tot_rel:.2e} (allowed {allowance:.2e}); "
               f"worst clean row {worst_clean:.2e}")
    assert worst_clean <= 1e-5, worst_clean
    assert tot_rel <= allowance, (tot_rel, allowance)
    return eg.sum(), eo.sum()


def recon_rows(H: np.ndarray, W: np.ndarray, What: np.ndarray) -> np.ndarray:
    D = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    return 0.5 * np.einsum("ij,jk,ik->i", D, H, D)
