"""Parity at the largest width the library takes: one layer of 64 x 65535 (int8,
asymmetric, one group per row) from 2048 bf16 tokens of the fc recipe (N(0, 1), outlier
channels x 30), through the C ABI: the Hessian (its 256 x 256 tiles reach 65535 only in
part; H holds 4.3e9 entries, past 32-bit indexing), the factorization at d_col = 65535,
and the sweep with a ragged last block (65535 = 511 x 128 + 127) and odd code rows.

X is stored with a row pitch of 65536 elements (a view of 65535 columns), so the Hessian
takes its matrix-core path.  Checked as at the other wide layers: sampled entries of H
against fp64 sums, U through U^T U (H + lambda I) e_j = e_j on sampled columns and its
trailing 2048 x 2048 block against the oracle's factor, every row's codes, scales and
zeros through the tie-consistent oracle with the GPU's U, the dequantized rows bit for
bit and the rows' objective."""
import dataclasses

import numpy as np
import pytest

import synth
from gpu_helpers import assert_parity, log, tie_consistent_parity, u_residual_ratio, unpack_codes
from oracle import gptq_oracle as o

pytestmark = pytest.mark.gpu

D = 65535


@pytest.fixture(scope="module")
def big():
    import torch
    import post_weight_quantization_25_amd as g
    L = synth.scaled(synth.config_layers(5)[1], 64, D, 2048, seed_offset=700)
    L = dataclasses.replace(L, bits=8, group_size=0, sym=False)
    rng = np.random.default_rng([91, D])
    cols = {0, 1, 255, 256, 511, 512, D // 2, D - 257, D - 256, D - 128, D - 2, D - 1}
    cols = np.array(sorted(cols | set(rng.choice(D, 28, replace=False).tolist())))
    log(f"max width: {L.d_row}x{D}, {L.n_tokens} tokens, int8 per row: generating inputs")
    dev = torch.device("cuda:0")
    Xp = torch.zeros((L.n_tokens, D + 1), dtype=torch.bfloat16, device=dev)
    Xs = np.empty((L.n_tokens, cols.size))
    for c, arr in enumerate(synth.x_chunks(L)):
        lo = c * synth.CHUNK
        Xp[lo:lo + arr.shape[0], :D].copy_(torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16))
        Xs[lo:lo + arr.shape[0]] = synth.bf16_bits_to_f32(arr[:, cols])
    X = Xp[:, :D]
    assert X.stride(0) == D + 1 and X.stride(1) == 1
    W = synth.weights(L)
    Wd = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).to(dev)
    log("  Hessian")
    H = torch.zeros((D, D), dtype=torch.float32, device=dev)
    g.hessian_accumulate(H, X)
    torch.cuda.synchronize()
    del X, Xp
    torch.cuda.empty_cache()
    sym_ok = all(torch.equal(H[r], H[:, r]) for r in (0, 1, 300, D // 2, D - 1))
    log("  factorization")
    with g.Context(1) as ctx:
        U, info = g.prepare_hinv(H, 0.01, ctx=ctx)
        torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("  quantization")
    q = g.quantize_layer(Wd, U, 8, 0, False)
    What = g.dequantize(q)
    torch.cuda.synchronize()
    assert int(info.item()) == 0 and int(q.info.item()) == 0
    out = dict(L=L, cols=cols, Xs=Xs, W=W, sym_ok=sym_ok,
               codes=unpack_codes(q.codes.cpu().numpy(), 8), s16=q.scales.cpu().numpy(),
               z=q.zeros.cpu().numpy().astype(np.int64), What=What.cpu().numpy())
    del q, What, Wd
    log("  H and U to the host")
    out["H"] = H.cpu().numpy()
    del H
    out["U"] = U.cpu().numpy()
    del U
    torch.cuda.empty_cache()
    yield out
    out.clear()


def test_maxsize_hessian(big):
    assert big["sym_ok"]                      # H[r, :] == H[:, r] bit for bit
    cols, H, Xs = big["cols"], big["H"], big["Xs"]
    Hs = H[np.ix_(cols, cols)]
    assert np.array_equal(Hs, Hs.T)
    Ho = 2.0 * (Xs.T @ Xs)
    dg = np.sqrt(np.diag(Ho))
    err = float(np.max(np.abs(Hs.astype(np.float64) - Ho) / np.outer(dg, dg)))
    tol = 2.0 * (big["L"].n_tokens / 16 + 64) * 2.0 ** -24      # as at the other widths
    log(f"  H sampled {cols.size}x{cols.size}: max err {err:.3e} (bound {tol:.3e})")
    assert err <= tol


def test_maxsize_prep(big):
    H, U = big["H"], big["U"]
    js = np.array([0, 1, D // 3, D - 130, D - 1])
    ratio, rmax = u_residual_ratio(U, H, js)
    log(f"  U {D}x{D}: residual on {js.size} columns, max |r| {rmax:.3e}, fraction of 4x the bound {ratio:.3f}")
    assert ratio <= 1.0
    c0 = D - 2048
    lam = 0.01 * float(np.mean(np.diag(H).astype(np.float64)))
    Uo, _ = o.prepare_u(H[c0:, c0:].astype(np.float64) + lam * np.eye(D - c0), 0.0)
    err = float(np.max(np.abs(U[c0:, c0:].astype(np.float64) - Uo) / np.max(np.abs(Uo), axis=1, keepdims=True)))
    log(f"  U trailing block against the oracle: max err / row max {err:.3e}")
    assert err <= 1e-6
    for r0 in range(0, D, 4096):
        Ub = U[r0:r0 + 4096, :r0 + 4096]
        ii = np.arange(Ub.shape[0])[:, None] + r0
        assert not np.any(Ub[np.arange(Ub.shape[1])[None, :] < ii])


def test_maxsize_quant_rows(big):
    L, U, H = big["L"], big["U"], big["H"]
    Wf = synth.w_as_f64(big["W"])
    p = o.Params(bits=8, group_size=0, sym=False)
    ref = o.gptq_blocked(Wf, U, p)
    rep = tie_consistent_parity(big["codes"], big["s16"], big["z"], Wf, U, p, tie_window=1e-3, ref=ref)
    log(f"  all {L.d_row} rows: plain code match {rep['code_match']:.6f}")
    assert_parity(rep, log, min_code_match=0.0)
    deq = big["s16"].astype(np.float32) * (big["codes"].astype(np.float32) - big["z"].astype(np.float32))
    assert np.array_equal(big["What"], deq)
    # objective of every row, GPU and tie-consistent oracle in one pass over H
    Dg = Wf - big["What"].astype(np.float64)
    Do = Wf - rep["what"]
    Dd = np.concatenate([Dg, Do])
    e = np.zeros(Dd.shape[0])
    for c0 in range(0, D, 2048):
        e += np.sum((Dd @ H[:, c0:c0 + 2048].astype(np.float64)) * Dd[:, c0:c0 + 2048], axis=1)
    eg, eo = 0.5 * e[:L.d_row], 0.5 * e[L.d_row:]
    worst = float(np.max(np.abs(eg - eo) / eo))
    tot = abs(eg.sum() - eo.sum()) / eo.sum()
    log(f"  objective: gpu {eg.sum():.6e} oracle {eo.sum():.6e} rel {tot:.2e}, worst row {worst:.2e}")
    assert worst <= 1e-5 and tot <= 1e-3
