"""Plain, slow CPU oracle of the GPTQ layer quantizer (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the GPU
path (no kernels, headers, helpers or constants) and imports nothing from it.

Sources (the pages this restates; every function cites the passage it follows):

* GPTQ paper summary page (azimuth.plus, "GPTQ: accurate post-training
  quantization for generative pre-trained transformers"), sections on the
  layer-wise objective, the OBQ background, the three innovations (fixed
  column order, lazy batched updates, Cholesky of the inverse Hessian with
  dampening) and the statement of the one-layer procedure.
* Hugging Face Transformers "Quantization concepts" guide, sections "Mapping
  values to fewer bits" (affine and symmetric quantization), "Choose
  granularity" (per-tensor / per-channel / per-group) and "Data types - int8
  and int4" (two int4 values per byte, first value in the low nibble).
* The "What is quantization" explainer (taqaniya), section "How does it work,
  with a simple example" (the absmax int8 example with range -127..127).

The page's display formulas for the objective, the OBS update and the algorithm
listing were lost in extraction; the readings used here are:

* objective: ||W X - What X||^2 with X in the (tokens x d_col) layout, i.e.
  ||X (W - What)^T||_F^2, and H = 2 X^T X (unnormalised);
* dampening: lambda = percdamp * mean(diag H), added to the diagonal;
* U is the upper Cholesky factor of (H + lambda I)^-1, i.e. (H + lambda I)^-1 = U^T U;
  row c of U, divided by U[c, c], is the OBS update direction after
  columns 0..c-1 are eliminated;
* the step for column c: quantize, err = (w_c - q(w_c)) / U[c, c],
  w[c+1:] -= err * U[c, c+1:];
* group scale/zero of a group are computed, at the group's first column, from
  the current (already compensated) values of the group's columns;
* asymmetric grid [0, 2^b - 1] with S = (max - min) / (2^b - 1),
  Z = -round(min / S16); symmetric grid +-(2^(b-1) - 1) with S = absmax / (2^(b-1) - 1),
  Z = 0; S16 = fp16(S) is the scale used for quantizing and stored;
* a code is decided as the guide writes it, q = clamp(rne(w / S16 + Z)), with the
  quotient and the sum in fp64 (round half to even; the pages name no precision,
  so the decision is taken as close to exact arithmetic as fp64 allows); the
  zero point likewise, Z = qmin - rne(min / S16) in fp64;
* stored codes are unsigned: u = q (asymmetric) or q + 2^(b-1) (symmetric), stored
  zero z = Z or 2^(b-1); dequantisation is fl32(S16) * fl32(u - z);
* 3-bit codes are stored as a bitstream per row (eight codes in three bytes, lowest bit
  first), the same first-value-lowest order as the guide's two int4 values per byte.
"""
from __future__ import annotations

import dataclasses
import itertools
from typing import Iterable

import numpy as np


class NotPositiveDefinite(ValueError):
    def __init__(self, k: int):
        super().__init__(f"leading minor of order {k} is not positive definite")
        self.k = k


class NonFinite(ValueError):
    pass


# ---------------------------------------------------------------------------
# Scalar quantizers, exactly as the concept guide writes them.

def affine_params(vmin: float, vmax: float, qmin: int, qmax: int) -> tuple[float, int]:
    """S = (vmax - vmin) / (qmax - qmin); Z = qmin - round(vmin / S).

    [Quantization concepts guide, "Mapping values to fewer bits": scale and zero point]
    """
    S = (vmax - vmin) / (qmax - qmin)
    Z = qmin - int(np.rint(vmin / S))
    return S, Z


def affine_quantize(x, S, Z, qmin, qmax):
    """q = round(x / S + Z), clamped to the grid.  [same section: quantize formula]"""
    return np.clip(np.rint(np.asarray(x, dtype=np.float64) / S + Z), qmin, qmax).astype(np.int64)


def affine_dequantize(q, S, Z):
    """x ~= S * (q - Z).  [same section: dequantize formula]"""
    return S * (np.asarray(q, dtype=np.float64) - Z)


def symmetric_quantize(x, absmax: float, qmax: int):
    """Range [-a, a], zero point fixed at 0: q = round(x * qmax / a), clamped to +-qmax.

    [Quantization concepts guide, "Mapping values to fewer bits": symmetric form;
     explainer page, "How does it work": absmax example with int8 range -127..127]
    """
    return np.clip(np.rint(np.asarray(x, dtype=np.float64) * (qmax / absmax)), -qmax, qmax).astype(np.int64)


# ---------------------------------------------------------------------------
# Quantizer settings of the layer quantizer.

@dataclasses.dataclass(frozen=True)
class Params:
    bits: int = 4
    group_size: int = 128      # 0 = one group per row (per-channel); -1 = one range for the whole matrix (per-tensor)
    sym: bool = False
    block_size: int = 128
    percdamp: float = 0.01
    fp4: bool = False          # E2M1 grid with one fp16 scale per group (bits must be 4)
    mx: bool = False           # with fp4: the scale is a power of two (MXFP4)

    @property
    def qmin(self) -> int:
        return -(2 ** (self.bits - 1) - 1) if self.sym else 0

    @property
    def qmax(self) -> int:
        return (2 ** (self.bits - 1) - 1) if self.sym else 2 ** self.bits - 1

    @property
    def zero_offset(self) -> int:
        """Shift from the signed symmetric grid to the stored unsigned code."""
        return 2 ** (self.bits - 1) if self.sym else 0

    def group(self, d_col: int) -> int:
        return d_col if self.group_size <= 0 else self.group_size


# FP4 E2M1: 1 sign, 2 exponent, 1 mantissa bit; magnitudes by code index 0 .. 7.
# [Quantization concepts guide, "FP4 with block scales"]
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_round(t: np.ndarray) -> np.ndarray:
    """Index (0 .. 7) of the E2M1 magnitude nearest |t|; a tie between two neighbours
    goes to the even index (the even mantissa bit); beyond 6 the largest, 6."""
    a = np.abs(np.asarray(t, dtype=np.float64))
    d = np.abs(a[..., None] - E2M1_VALUES)
    i = np.argmin(d, axis=-1)
    nxt = np.minimum(i + 1, 7)
    tie = (np.take_along_axis(d, nxt[..., None], -1)[..., 0] == np.take_along_axis(d, i[..., None], -1)[..., 0]) & (nxt != i)
    return np.where(tie & (i % 2 == 1), nxt, i)


def _fp16_round(S: np.ndarray) -> np.ndarray:
    """Round the (fp64) scale to fp16 (nearest even); returned as fp64 values."""
    with np.errstate(over="ignore"):
        return np.asarray(S, dtype=np.float64).astype(np.float16).astype(np.float64)


def group_params(vals: np.ndarray, p: Params):
    """Scale and zero point of one group for every row at once.

    ``vals`` is (rows, g): the current values of the group's columns.
    Returns (S, S16, Z, zt): pre-rounding scale (fp64), fp16-rounded scale (as fp64),
    the integer zero point on the signed/unsigned grid, and the fp64 value
    min / S16 whose rounding gave Z (0 for the symmetric grid).

    [Quantization concepts guide, "Mapping values to fewer bits" (asymmetric:
     literal min/max; symmetric: [-a, a], Z = 0) and "Choose granularity"
     (one scale per group of consecutive weights of a row)]
    """
    if p.fp4:
        # E2M1: the group's largest magnitude goes to 6; the returned "S16" is the step
        # S16 / 2 of the half-unit codes q = 2 * (+-E2M1 value), so that What = step * q
        # as for the integer grids, with Z = 0  ["FP4 with block scales": one scale per
        # small block]
        if p.group_size < 0:
            S, S16, Z, t = group_params(np.asarray(vals).reshape(1, -1), dataclasses.replace(p, group_size=0))
            n = vals.shape[0]
            return np.repeat(S, n), np.repeat(S16, n), np.repeat(Z, n), np.repeat(t, n)
        a = np.max(np.abs(vals), axis=1)
        S = np.where(a > 0, a / 6.0, 1.0)
        S_pre = S   # returned as the pre-rounding scale
        if p.mx:
            # MXFP4: the smallest power of two not below absmax / 6 (frexp: x = m 2^e,
            # m in [0.5, 1); exactly 2^(e-1) when m = 0.5)  ["FP4 with block scales":
            # MXFP4's scale is a power of two]
            m, e = np.frexp(S)
            S = np.ldexp(1.0, np.where(m == 0.5, e - 1, e)).astype(np.float64)
        S16 = _fp16_round(S)
        if not np.all(np.isfinite(S16)) or np.any(S16 < 2.0 ** -14):
            raise NonFinite("scale is not a normal fp16 number")
        return S_pre, S16 / 2.0, np.zeros(vals.shape[0], dtype=np.int64), np.zeros(vals.shape[0])
    if p.group_size < 0:
        # Per-tensor: one range over the values of every row, the same S and Z for all
        # rows.  Callers pass the whole matrix before any column is quantized.
        # ["Choose granularity": per-tensor, a single scale for the whole tensor]
        S, S16, Z, t = group_params(np.asarray(vals).reshape(1, -1), dataclasses.replace(p, group_size=0))
        n = vals.shape[0]
        return np.repeat(S, n), np.repeat(S16, n), np.repeat(Z, n), np.repeat(t, n)
    qmin, qmax = p.qmin, p.qmax
    if p.sym:
        a = np.max(np.abs(vals), axis=1)
        S = np.where(a > 0, a / qmax, 1.0)
        S16 = _fp16_round(S)
        Z = np.zeros(vals.shape[0], dtype=np.int64)
        t = np.zeros(vals.shape[0])
    else:
        mn = np.min(vals, axis=1)
        mx = np.max(vals, axis=1)
        # A constant group has no range; widen it to include 0 (the constant then
        # sits on the top or bottom grid point, up to the fp16 rounding of S), and
        # use S = 1 when the group is all zero.
        flat = mn == mx
        mn = np.where(flat, np.minimum(mn, 0.0), mn)
        mx = np.where(flat, np.maximum(mx, 0.0), mx)
        S = np.where(mx > mn, (mx - mn) / (qmax - qmin), 1.0)
        S16 = _fp16_round(S)
        # Z = qmin - round(min / S16)  ["Mapping values to fewer bits": zero point]
        t = mn / S16
        Z = (qmin - np.rint(t)).astype(np.int64)
    if not np.all(np.isfinite(S16)) or np.any(S16 < 2.0 ** -14):
        raise NonFinite("scale is not a normal fp16 number")
    return S, S16, Z, t


def decide_codes(w: np.ndarray, S16: np.ndarray, Z: np.ndarray, p: Params) -> np.ndarray:
    """q = clamp(round(w / S16 + Z)) on the signed (or unsigned) grid, round half to
    even, the quotient and the sum in fp64.

    [Quantization concepts guide, "Mapping values to fewer bits": quantize formula;
     the clamp keeps compensated values that left the group's range on the grid]
    """
    if p.fp4:
        # E2M1: S16 here is the half-unit step; the quotient is by the stored scale 2 step
        t = np.asarray(w, dtype=np.float64) / (2.0 * np.asarray(S16, dtype=np.float64))
        return (np.sign(t) * 2.0 * E2M1_VALUES[e2m1_round(t)]).astype(np.int64)
    return np.clip(np.rint(code_value(w, S16, Z)), p.qmin, p.qmax).astype(np.int64)


def code_value(w: np.ndarray, S16: np.ndarray, Z: np.ndarray) -> np.ndarray:
    """The pre-rounding code value w / S16 + Z in fp64 (what ``decide_codes`` rounds)."""
    return np.asarray(w, dtype=np.float64) / np.asarray(S16, dtype=np.float64) + np.asarray(Z, dtype=np.float64)


# ---------------------------------------------------------------------------
# Hessian, dampening, Cholesky factor of the inverse.

def hessian(x_chunks: Iterable[np.ndarray]) -> np.ndarray:
    """H = 2 X^T X over all calibration tokens (X is tokens x d_col), fp64.

    [GPTQ summary page, statement of the one-layer procedure: H = 2 X X^T with the
     page's X of shape d_col x tokens; the same matrix in the tokens-major layout]
    """
    H = None
    for x in x_chunks:
        x = np.asarray(x, dtype=np.float64)
        part = x.T @ x
        H = part if H is None else H + part
    return 2.0 * H


def damp(H: np.ndarray, percdamp: float) -> tuple[np.ndarray, float]:
    """H + lambda I with lambda = percdamp * mean(diag H).

    [GPTQ summary page, "Innovation 3": a small damping term lambda I for near-singular H]
    """
    lam = percdamp * float(np.mean(np.diag(H)))
    return H + lam * np.eye(H.shape[0]), lam


def cholesky_lower(A: np.ndarray) -> np.ndarray:
    """Textbook unblocked Cholesky A = L L^T (lower), with the LAPACK failure rule.

    Raises NotPositiveDefinite(k) when the leading minor of order k is not
    positive definite (k is 1-based).
    """
    n = A.shape[0]
    L = np.zeros_like(A, dtype=np.float64)
    for j in range(n):
        d = A[j, j] - L[j, :j] @ L[j, :j]
        if not (d > 0.0):
            raise NotPositiveDefinite(j + 1)
        L[j, j] = np.sqrt(d)
        L[j + 1:, j] = (A[j + 1:, j] - L[j + 1:, :j] @ L[j, :j]) / L[j, j]
    return L


def prepare_u(H: np.ndarray, percdamp: float) -> tuple[np.ndarray, float]:
    """U = upper Cholesky factor of (H + lambda I)^-1, computed once.

    (H + lambda I)^-1 = U^T U.  Row c of U gives the compensation direction for
    column c after columns 0..c-1 have been quantized.
    [GPTQ summary page, "Innovation 3": Cholesky decomposition of H^-1 computed once
     in advance, entries read row by row, plus dampening]
    """
    Hd, lam = damp(H, percdamp)
    try:
        L = np.linalg.cholesky(Hd)
    except np.linalg.LinAlgError:
        # locate the failing leading minor with the textbook factorization
        cholesky_lower(Hd)
        raise NotPositiveDefinite(-1)
    Linv = np.linalg.inv(L)
    Hinv = Linv.T @ Linv
    Hinv = 0.5 * (Hinv + Hinv.T)
    U = np.linalg.cholesky(Hinv).T
    return U, lam


def trailing_not_pd_order(H: np.ndarray, percdamp: float) -> int:
    """Order k of the smallest trailing principal submatrix of H + lambda I that is not
    positive definite (0 if it is positive definite).  This is the failure index of a
    Cholesky factorization that starts from the last column (reverse order)."""
    Hd, _ = damp(H, percdamp)
    R = Hd[::-1, ::-1]
    try:
        cholesky_lower(R)
    except NotPositiveDefinite as e:
        return e.k
    return 0


# ---------------------------------------------------------------------------
# The column sweep.

@dataclasses.dataclass
class Result:
    q: np.ndarray          # signed (sym) or unsigned (asym) integer codes, d_row x d_col
    codes: np.ndarray      # stored unsigned codes u, uint8, d_row x d_col
    S: np.ndarray          # pre-rounding scales, d_row x n_groups (fp64)
    scales16: np.ndarray   # fp16 scales, d_row x n_groups (np.float16)
    zeros: np.ndarray      # stored zero points z, d_row x n_groups (int64)
    z_t: np.ndarray        # min / S16, the value rounded to get Z (fp64), d_row x n_groups
    what: np.ndarray       # dequantized weights S16 * (q - Z), fp64
    w_at_q: np.ndarray     # the value each weight had when it was quantized (fp64)
    t_at_q: np.ndarray     # w / S16 + Z, the pre-rounding code value (fp64)


def _n_groups(d_col: int, p: Params) -> int:
    g = p.group(d_col)
    return (d_col + g - 1) // g


def e2m1_codes(Q: np.ndarray) -> np.ndarray:
    """Stored FP4 code of half-unit values Q = 2 * (+-E2M1 value): sign bit 8 (for a
    nonzero negative value) | magnitude index."""
    idx = np.searchsorted(E2M1_VALUES, np.abs(Q) / 2.0)
    return (idx + np.where(Q < 0, 8, 0)).astype(np.uint8)


def _finish(Q, S, S16, Z, ZT, what, w_at_q, t_at_q, p) -> Result:
    if p.fp4:
        return Result(q=Q, codes=e2m1_codes(Q), S=S, scales16=(2.0 * S16).astype(np.float16),
                      zeros=np.zeros_like(Z), z_t=ZT, what=what, w_at_q=w_at_q, t_at_q=t_at_q)
    codes = (Q + p.zero_offset).astype(np.uint8)
    zeros = (Z + p.zero_offset).astype(np.int64) if not p.sym else np.full_like(Z, p.zero_offset)
    return Result(q=Q, codes=codes, S=S, scales16=S16.astype(np.float16), zeros=zeros, z_t=ZT,
                  what=what, w_at_q=w_at_q, t_at_q=t_at_q)


def gptq(W: np.ndarray, U: np.ndarray, p: Params) -> Result:
    """Unblocked GPTQ on one layer, columns in natural order, all rows at once.

    For c = 0 .. d_col-1: (at a group's first column) group scale/zero from the
    current values; quantize column c; err = (w_c - what_c) / U[c, c];
    w[:, c+1:] -= err * U[c, c+1:].
    [GPTQ summary page: OBQ background (quantize one weight, update the remaining
     full-precision weights to compensate, direction given by H^-1); "Innovation 1"
     (one fixed column order shared by all rows, so H_F^-1 is shared); "Innovation 3"
     (rows of the Cholesky factor of H^-1 give the updates)]
    """
    W = np.array(W, dtype=np.float64, copy=True)
    d_row, d_col = W.shape
    g = p.group(d_col)
    ng = _n_groups(d_col, p)
    Q = np.zeros((d_row, d_col), dtype=np.int64)
    S = np.zeros((d_row, ng)); S16 = np.zeros((d_row, ng)); Z = np.zeros((d_row, ng), dtype=np.int64)
    ZT = np.zeros((d_row, ng))
    what = np.zeros_like(W); w_at_q = np.zeros_like(W); t_at_q = np.zeros((d_row, d_col), dtype=np.float64)
    for c in range(d_col):
        k = c // g
        if c % g == 0:
            S[:, k], S16[:, k], Z[:, k], ZT[:, k] = group_params(W[:, c:c + g], p)
        w = W[:, c].copy()
        w_at_q[:, c] = w
        t_at_q[:, c] = code_value(w, S16[:, k], Z[:, k])
        q = decide_codes(w, S16[:, k], Z[:, k], p)
        Q[:, c] = q
        what[:, c] = S16[:, k] * (q - Z[:, k])
        err = (w - what[:, c]) / U[c, c]
        W[:, c + 1:] -= np.outer(err, U[c, c + 1:])
    return _finish(Q, S, S16, Z, ZT, what, w_at_q, t_at_q, p)


def _forced_index(forced):
    """{("q", r, c): q} and {("g", r, k): (S16, Z)} -> per column / per group lists."""
    by_col, by_grp = {}, {}
    for key, val in (forced or {}).items():
        kind, r, i = key
        if kind == "q":
            by_col.setdefault(i, []).append((r, val))
        elif kind == "g":
            by_grp.setdefault(i, []).append((r, val))
        else:
            raise ValueError(key)
    return by_col, by_grp


def gptq_blocked(W: np.ndarray, U: np.ndarray, p: Params, forced: dict | None = None) -> Result:
    """GPTQ with lazy batched updates in blocks of B columns.

    Inside a block the updates stay local to the block; the error block E
    (err of every column of the block) is then applied to all later columns in one
    matrix product W[:, b1:] -= E @ U[b0:b1, b1:].
    [GPTQ summary page, "Innovation 2": process B = 128 columns together, keep the
     intermediate updates inside the block, then one large matrix update]
    Needs the group to lie inside one block (block_size % group_size == 0) or one
    group per row; otherwise a group's first column would see values that lack
    this block's pending updates.

    ``forced`` optionally fixes decisions that another computation took on the other
    side of a rounding tie (both sides of a tie follow the rule): ("q", r, c) -> q sets
    row r's code at column c (signed grid, or half-units for E2M1), and
    ("g", r, k) -> (S16, Z) sets row r's scale and zero point of group k.  Everything
    else, including the compensation that follows a fixed decision, is computed as
    without it.
    """
    f_col, f_grp = _forced_index(forced)
    W = np.array(W, dtype=np.float64, copy=True)
    d_row, d_col = W.shape
    g = p.group(d_col)
    B = p.block_size
    if not (p.group_size <= 0 or B % g == 0):
        raise ValueError("group must not straddle a block")
    ng = _n_groups(d_col, p)
    Q = np.zeros((d_row, d_col), dtype=np.int64)
    S = np.zeros((d_row, ng)); S16 = np.zeros((d_row, ng)); Z = np.zeros((d_row, ng), dtype=np.int64)
    ZT = np.zeros((d_row, ng))
    what = np.zeros_like(W); w_at_q = np.zeros_like(W); t_at_q = np.zeros((d_row, d_col), dtype=np.float64)
    for b0 in range(0, d_col, B):
        b1 = min(b0 + B, d_col)
        Wb = W[:, b0:b1].copy()
        Eb = np.zeros((d_row, b1 - b0))
        for j in range(b1 - b0):
            c = b0 + j
            k = c // g
            if c % g == 0:
                src = Wb[:, j:j + g] if g <= B else W[:, c:c + g]
                S[:, k], S16[:, k], Z[:, k], ZT[:, k] = group_params(src, p)
                for r, (s16, z) in f_grp.get(k, ()):
                    S16[r, k], Z[r, k] = s16, z
            w = Wb[:, j].copy()
            w_at_q[:, c] = w
            t_at_q[:, c] = code_value(w, S16[:, k], Z[:, k])
            q = decide_codes(w, S16[:, k], Z[:, k], p)
            for r, qf in f_col.get(c, ()):
                q[r] = qf
            Q[:, c] = q
            what[:, c] = S16[:, k] * (q - Z[:, k])
            err = (w - what[:, c]) / U[c, c]
            Eb[:, j] = err
            Wb[:, j + 1:] -= np.outer(err, U[c, c + 1:b1])
        W[:, b1:] -= Eb @ U[b0:b1, b1:]
    return _finish(Q, S, S16, Z, ZT, what, w_at_q, t_at_q, p)


def gptq_obs(W: np.ndarray, Hd: np.ndarray, p: Params) -> Result:
    """GPTQ through explicit OBS elimination (no Cholesky factor).

    Before quantizing column c the inverse of the remaining block Hd[c:, c:] is formed
    directly; the update of the remaining weights is
    -(w_c - q(w_c)) / [H_F^-1]_cc * [H_F^-1]_{c, :}.
    [GPTQ summary page, OBQ background: update all remaining weights after each
     quantization, direction given by the inverse Hessian of the remaining weights;
     "Innovation 1": one order shared by all rows]
    O(d_col^4); tiny layers only.
    """
    W = np.array(W, dtype=np.float64, copy=True)
    d_row, d_col = W.shape
    g = p.group(d_col)
    ng = _n_groups(d_col, p)
    Q = np.zeros((d_row, d_col), dtype=np.int64)
    S = np.zeros((d_row, ng)); S16 = np.zeros((d_row, ng)); Z = np.zeros((d_row, ng), dtype=np.int64)
    ZT = np.zeros((d_row, ng))
    what = np.zeros_like(W); w_at_q = np.zeros_like(W); t_at_q = np.zeros((d_row, d_col), dtype=np.float64)
    for c in range(d_col):
        k = c // g
        if c % g == 0:
            S[:, k], S16[:, k], Z[:, k], ZT[:, k] = group_params(W[:, c:c + g], p)
        Finv = np.linalg.inv(Hd[c:, c:])
        w = W[:, c].copy()
        w_at_q[:, c] = w
        q = decide_codes(w, S16[:, k], Z[:, k], p)
        Q[:, c] = q
        what[:, c] = S16[:, k] * (q - Z[:, k])
        W[:, c + 1:] -= np.outer((w - what[:, c]) / Finv[0, 0], Finv[0, 1:])
    return _finish(Q, S, S16, Z, ZT, what, w_at_q, t_at_q, p)


def obq_step(w: np.ndarray, Finv: np.ndarray, live: np.ndarray, S16: float, Z: int, p: Params):
    """One OBQ step on one row: of the remaining weights (mask ``live``), quantize the
    one whose quantization adds the least error, (w_j - q(w_j))^2 / [Finv]_jj (ties to
    the lowest index); move the other remaining weights by the OBS update
    -(w_j - q(w_j)) / [Finv]_jj * Finv[:, j]; remove j from the inverse Hessian of the
    remaining weights, Finv - Finv[:, j] Finv[j, :] / [Finv]_jj.  Returns
    (j, q_j, what_j, w, Finv, live), the arrays updated copies.

    [GPTQ summary page, OBQ background: greedy order by the smallest added error, the
     update of the remaining weights through the inverse Hessian, and the removal of
     the quantized weight from that inverse]
    """
    w = w.copy(); Finv = Finv.copy(); live = live.copy()
    q = decide_codes(w, np.full(w.shape, S16), np.full(w.shape, Z, dtype=np.int64), p)
    wh = S16 * (q - Z)
    score = np.where(live, (w - wh) ** 2 / np.where(live, np.diag(Finv), 1.0), np.inf)
    j = int(np.argmin(score))
    err = (w[j] - wh[j]) / Finv[j, j]
    col = Finv[:, j].copy()
    upd = live.copy(); upd[j] = False
    w[upd] -= err * col[upd]
    Finv -= np.outer(col, col) / col[j]
    live[j] = False
    Finv[j, :] = 0.0; Finv[:, j] = 0.0
    return j, int(q[j]), float(wh[j]), w, Finv, live


def obq(W: np.ndarray, Hd: np.ndarray, p: Params) -> tuple[Result, np.ndarray]:
    """OBQ: every row on its own, its weights quantized in a greedy order (``obq_step``
    until none remain), starting from the inverse of the damped Hessian.  The row's grid
    (one group per row) is fixed first from its original values.  O(d_row d_col^3).
    Returns the result and each row's order of quantization.

    [GPTQ summary page, OBQ background (the method GPTQ is compared with: per-row
     greedy order, inverse Hessian updated after every weight)]
    """
    if p.group_size != 0:
        raise ValueError("OBQ here uses one group per row")
    W = np.array(W, dtype=np.float64, copy=True)
    d_row, d_col = W.shape
    Hinv = np.linalg.inv(Hd)
    S, S16, Z, ZT = group_params(W, p)
    Q = np.zeros((d_row, d_col), dtype=np.int64)
    what = np.zeros_like(W)
    order = np.zeros((d_row, d_col), dtype=np.int64)
    for r in range(d_row):
        w, Finv, live = W[r].copy(), Hinv.copy(), np.ones(d_col, dtype=bool)
        for k in range(d_col):
            j, qj, whj, w, Finv, live = obq_step(w, Finv, live, S16[r], int(Z[r]), p)
            Q[r, j], what[r, j], order[r, k] = qj, whj, j
    res = _finish(Q, S[:, None], S16[:, None], Z[:, None], ZT[:, None], what, np.zeros_like(W),
                  np.zeros_like(W), p)
    return res, order


def rtn(W: np.ndarray, p: Params) -> Result:
    """Round-to-nearest: every weight quantized on its own group grid, no compensation.

    [GPTQ summary page, results: the RTN baseline]
    """
    W = np.asarray(W, dtype=np.float64)
    d_row, d_col = W.shape
    g = p.group(d_col)
    ng = _n_groups(d_col, p)
    Q = np.zeros((d_row, d_col), dtype=np.int64)
    S = np.zeros((d_row, ng)); S16 = np.zeros((d_row, ng)); Z = np.zeros((d_row, ng), dtype=np.int64)
    ZT = np.zeros((d_row, ng))
    what = np.zeros_like(W); t_at_q = np.zeros((d_row, d_col), dtype=np.float64)
    for k in range(ng):
        c0, c1 = k * g, min((k + 1) * g, d_col)
        S[:, k], S16[:, k], Z[:, k], ZT[:, k] = group_params(W[:, c0:c1], p)
        for c in range(c0, c1):
            Q[:, c] = decide_codes(W[:, c], S16[:, k], Z[:, k], p)
            what[:, c] = S16[:, k] * (Q[:, c] - Z[:, k])
    return _finish(Q, S, S16, Z, ZT, what, W.copy(), t_at_q, p)


# ---------------------------------------------------------------------------
# Storage format and dequantisation.

def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Codes of a row into bytes.  bits == 4: two codes per byte, byte k = u[2k] | u[2k+1] << 4
    (first value in the low nibble); bits == 3: a bitstream of the row, code c in stream
    bits 3c .. 3c + 2 (lowest bit first) and stream bit i in bit i % 8 of byte i // 8, so
    eight codes fill three bytes; bits == 8: one code per byte.

    [Quantization concepts guide, "Data types - int8 and int4": sub-byte values are packed
     into bytes, two int4 values per byte with the first in the low 4 bits and the second
     in the high 4 bits; the 3-bit stream continues the same first-value-lowest order]
    """
    codes = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        return codes.copy()
    if bits == 3:
        d = codes.shape[-1]
        if d % 8:
            raise ValueError("3-bit rows hold a multiple of 8 codes")
        out = np.zeros(codes.shape[:-1] + (3 * d // 8,), dtype=np.uint8)
        for c in range(d):
            for b in range(3):
                i = 3 * c + b
                out[..., i // 8] |= (((codes[..., c] >> b) & 1) << (i % 8)).astype(np.uint8)
        return out
    if codes.shape[-1] % 2:
        raise ValueError("odd number of columns")
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of ``pack``: the row's codes from its bytes."""
    packed = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return packed.copy()
    if bits == 3:
        d = packed.shape[-1] * 8 // 3
        out = np.zeros(packed.shape[:-1] + (d,), dtype=np.uint8)
        for c in range(d):
            for b in range(3):
                i = 3 * c + b
                out[..., c] |= (((packed[..., i // 8] >> (i % 8)) & 1) << b).astype(np.uint8)
        return out
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def dequantize_e2m1(codes: np.ndarray, scales16: np.ndarray, group_size: int) -> np.ndarray:
    """What = S16 * (+-E2M1 value of the code), in float32 (exact).
    [Quantization concepts guide, "FP4 with block scales"]"""
    codes = np.asarray(codes).astype(np.int64)
    d_col = codes.shape[1]
    g = d_col if group_size <= 0 else group_size
    idx = np.arange(d_col) // g
    s = np.asarray(scales16, dtype=np.float16).astype(np.float32)[:, idx]
    v = np.where(codes >= 8, -1.0, 1.0) * E2M1_VALUES[codes & 7]
    return (s * v.astype(np.float32)).astype(np.float32)


def dequantize(codes: np.ndarray, scales16: np.ndarray, zeros: np.ndarray, group_size: int) -> np.ndarray:
    """What = S16 * (u - z), evaluated in float32 (exact: an fp16 times a small integer).

    [Quantization concepts guide, "Mapping values to fewer bits": x ~= S (q - Z)]
    """
    codes = np.asarray(codes)
    d_col = codes.shape[1]
    g = d_col if group_size <= 0 else group_size
    idx = np.arange(d_col) // g
    s = np.asarray(scales16, dtype=np.float16).astype(np.float32)[:, idx]
    z = np.asarray(zeros).astype(np.float32)[:, idx]
    return (s * (codes.astype(np.float32) - z)).astype(np.float32)


def linear(x: np.ndarray, codes: np.ndarray, scales16: np.ndarray, zeros: np.ndarray,
           group_size: int) -> np.ndarray:
    """y = x What^T in fp64, What = dequantize(codes, scales16, zeros, group_size): the
    layer's output on its quantized weights, for activations stored tokens x d_col.

    [GPTQ summary page, layer-wise objective (the layer computes W X; here X is tokens
     x d_col, so the output is X W^T) and its results on inference with the packed
     weights]
    """
    What = dequantize(codes, scales16, zeros, group_size).astype(np.float64)
    return np.asarray(x, dtype=np.float64) @ What.T


# ---------------------------------------------------------------------------
# The layer objective.

def recon_error_x(x_chunks: Iterable[np.ndarray], W: np.ndarray, What: np.ndarray) -> float:
    """||X (W - What)^T||_F^2 summed over calibration tokens.

    [GPTQ summary page, layer-wise objective: make the layer output with What as
     close as possible to the output with W]
    """
    D = (np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)).T
    tot = 0.0
    for x in x_chunks:
        y = np.asarray(x, dtype=np.float64) @ D
        tot += float(np.sum(y * y))
    return tot


def recon_error_h(H: np.ndarray, W: np.ndarray, What: np.ndarray, per_row: bool = False):
    """The same objective from H: 1/2 * sum_r (W_r - What_r) H (W_r - What_r)^T."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    rows = 0.5 * np.einsum("ij,jk,ik->i", D, H, D)
    return rows if per_row else float(np.sum(rows))


def brute_force_row(w: np.ndarray, H: np.ndarray, S16: float, Z: int, p: Params):
    """Exhaustive minimum of (w - what) H (w - what)^T over every code vector on the
    grid {S16 * (q - Z) : qmin <= q <= qmax}^d.  Tiny d only."""
    d = w.shape[0]
    levels = np.arange(p.qmin, p.qmax + 1)
    vals = S16 * (levels - Z)
    best, best_q = np.inf, None
    # enumerate in slabs over the first coordinate to bound memory
    rest = np.array(list(itertools.product(range(len(levels)), repeat=d - 1)), dtype=np.int64) if d > 1 else np.zeros((1, 0), dtype=np.int64)
    for i0 in range(len(levels)):
        cand = np.empty((rest.shape[0], d))
        cand[:, 0] = vals[i0]
        cand[:, 1:] = vals[rest]
        D = w[None, :] - cand
        e = np.einsum("ij,jk,ik->i", D, H, D)
        j = int(np.argmin(e))
        if e[j] < best:
            best = float(e[j])
            best_q = np.concatenate([[levels[i0]], levels[rest[j]]])
    return best, best_q
