"""gptq_quantize_layers (a block's linears in one call, phases overlapped on the streams
of a caller-owned context, or on one stream without it) against one call per phase and
layer, bit for bit, for 1, 2 and 3 slots and twice in a row; the group that shares one
input (q, k, v) also against the oracle."""
import numpy as np
import pytest

import synth
from gpu_helpers import assert_parity, dev_tensor, layer_x, log, tie_consistent_parity, unpack_codes
from oracle import gptq_oracle as o

pytestmark = pytest.mark.gpu

CHAIN_TIE = 1e-3   # as in the end-to-end chain test


def _mini_block():
    """A decoder block's shapes scaled down, recipe of the 7-linear block workload: q, k, v
    share one input, o has its own, gate and up share one, down has its own (width 1408:
    an edge super-block).  Returns [(X layer, W layer)] with equal X layers for sharers."""
    c4 = synth.config_layers(4)
    sc = lambda i, r, c: synth.scaled(c4[i], r, c, 4096)
    xq, xo, xg, xd = sc(0, 256, 512), sc(3, 384, 512), sc(4, 640, 512), sc(6, 256, 1408)
    return [(xq, xq), (xq, sc(1, 320, 512)), (xq, sc(2, 256, 512)), (xo, xo),
            (xg, xg), (xg, sc(5, 640, 512)), (xd, xd)]


SETTINGS = [(3, 0, True), (4, 128, False)]   # the block workload's int3 per-channel sym; int4 g128 asym


@pytest.mark.parametrize("bits,group,sym", SETTINGS)
def test_layers_match_per_phase_calls(bits, group, sym):
    import torch
    import post_weight_quantization_25_amd as g
    spec = _mini_block()
    xs, pairs = {}, []
    for LX, LW in spec:
        if LX.name not in xs:
            xs[LX.name] = (dev_tensor(layer_x(LX), LX.x_dtype), layer_x(LX))
        pairs.append((xs[LX.name][0], dev_tensor(synth.weights(LW), LW.w_dtype)))
    log(f"layers int{bits} g{group} sym={sym}: {[tuple(W.shape) for _, W in pairs]}")
    # one call per phase and layer
    ref = []
    for X, W in pairs:
        H = torch.zeros((X.shape[1], X.shape[1]), dtype=torch.float32, device="cuda")
        g.hessian_accumulate(H, X)
        U, info = g.prepare_hinv(H, 0.01)
        q = g.quantize_layer(W, U, bits=bits, group_size=group, sym=sym)
        torch.cuda.synchronize()
        assert int(info.item()) == 0 and int(q.info.item()) == 0
        ref.append((q.codes.cpu(), q.scales.cpu(), q.zeros.cpu(), U))
    ctx = g.Context(3)
    for slots, c_ in ((1, ctx), (2, ctx), (3, ctx), (2, ctx), (1, None)):
        outs, info = g.quantize_layers(pairs, bits=bits, group_size=group, sym=sym, n_slots=slots, ctx=c_)
        torch.cuda.synchronize()
        assert not info.cpu().any(), info.cpu()
        for k, (q, (c, s, z, _)) in enumerate(zip(outs, ref)):
            assert torch.equal(q.codes.cpu(), c), (slots, k)
            assert torch.equal(q.scales.cpu(), s), (slots, k)
            assert torch.equal(q.zeros.cpu(), z), (slots, k)
        log(f"  {slots} slot(s){' (no context: one stream)' if c_ is None else ''}: all {len(pairs)} layers bit-identical")
    with pytest.raises(g.GptqError):      # more slots than the context holds
        g.quantize_layers(pairs, bits=bits, group_size=group, sym=sym, n_slots=4, ctx=ctx)

    # the shared-input group (q, k, v) against the oracle: one H, one U, three sweeps
    Xh = xs[spec[0][0].name][1]
    Ho = o.hessian([synth.x_as_f64(Xh)])
    Uo, _ = o.prepare_u(Ho, 0.01)
    p = o.Params(bits=bits, group_size=group, sym=sym)
    outs, _ = g.quantize_layers(pairs[:3], bits=bits, group_size=group, sym=sym, n_slots=2, ctx=ctx)
    torch.cuda.synchronize()
    for (LX, LW), q in zip(spec[:3], outs):
        Wf = synth.w_as_f64(synth.weights(LW))
        r = o.gptq_blocked(Wf, Uo, p)
        rep = tie_consistent_parity(unpack_codes(q.codes.cpu().numpy(), bits), q.scales.cpu().numpy(),
                                    q.zeros.cpu().numpy().astype(np.int64), Wf, Uo, p, tie_window=CHAIN_TIE, ref=r)
        log(f"  {LW.name}:")
        assert_parity(rep, log)


def test_layers_wait_bound_reports_minus_two():
    """The context's wait bound reaches the factorizations of gptq_quantize_layers: with
    0 polls every layer's prep reports info = -2 (its kernels all end), and the same
    context with the default bound then gives the per-phase results bit for bit."""
    import torch
    import post_weight_quantization_25_amd as g
    spec = _mini_block()[:4]           # q, k, v share one input (one factorization), o its own
    xs, pairs = {}, []
    for LX, LW in spec:
        if LX.name not in xs:
            xs[LX.name] = dev_tensor(layer_x(LX), LX.x_dtype)
        pairs.append((xs[LX.name], dev_tensor(synth.weights(LW), LW.w_dtype)))
    with g.Context(2) as ctx:
        ctx.set_wait_limit(0)
        _, info = g.quantize_layers(pairs, bits=4, group_size=128, n_slots=2, ctx=ctx)
        torch.cuda.synchronize()
        inf = info.cpu().numpy().reshape(-1, 2)
        log(f"wait bound 0: infos {inf.tolist()}")
        # the factorization's status sits on each group's first layer (q and o)
        assert inf[0, 0] == -2 and inf[3, 0] == -2, inf
        assert inf[1, 0] == 0 and inf[2, 0] == 0, inf
        ctx.set_wait_limit(1 << 25)
        outs, info = g.quantize_layers(pairs, bits=4, group_size=128, n_slots=2, ctx=ctx)
        torch.cuda.synchronize()
    assert not info.cpu().any(), info.cpu()
    for (X, W), q in zip(pairs, outs):
        H = torch.zeros((X.shape[1], X.shape[1]), dtype=torch.float32, device="cuda")
        g.hessian_accumulate(H, X)
        U, i1 = g.prepare_hinv(H, 0.01)
        r = g.quantize_layer(W, U, bits=4, group_size=128)
        torch.cuda.synchronize()
        assert torch.equal(q.codes, r.codes) and torch.equal(q.scales, r.scales) and torch.equal(q.zeros, r.zeros)


def test_layers_deferred_widths_match_per_phase_calls():
    """Widths where the factorization defers its trailing update (outer blocks of 256
    columns from 4200, of 512 from 7168; 4736 and 7424 end in partial outer blocks), two
    and three groups in flight on the context's slot streams, each with its own auxiliary
    stream: bit-identical to one call per phase and layer."""
    import torch
    import post_weight_quantization_25_amd as g
    c4 = synth.config_layers(4)
    xa, xb, xc = synth.scaled(c4[6], 192, 4736, 8192), synth.scaled(c4[0], 128, 7424, 8192), \
        synth.scaled(c4[3], 160, 4736, 8192, seed_offset=600)
    spec = [(xa, xa), (xa, synth.scaled(c4[1], 96, 4736, 8192)), (xb, xb), (xc, xc)]
    xs, pairs = {}, []
    for LX, LW in spec:
        if LX.name not in xs:
            xs[LX.name] = dev_tensor(layer_x(LX), LX.x_dtype)
        pairs.append((xs[LX.name], dev_tensor(synth.weights(LW), LW.w_dtype)))
    log(f"layers at deferred widths: {[tuple(W.shape) for _, W in pairs]}")
    ref = []
    for X, W in pairs:
        H = torch.zeros((X.shape[1], X.shape[1]), dtype=torch.float32, device="cuda")
        g.hessian_accumulate(H, X)
        U, info = g.prepare_hinv(H, 0.01)
        q = g.quantize_layer(W, U, bits=4, group_size=128)
        torch.cuda.synchronize()
        assert int(info.item()) == 0 and int(q.info.item()) == 0
        ref.append((q.codes.cpu(), q.scales.cpu(), q.zeros.cpu()))
    with g.Context(3) as ctx:
        for slots in (2, 3):
            outs, info = g.quantize_layers(pairs, bits=4, group_size=128, n_slots=slots, ctx=ctx)
            torch.cuda.synchronize()
            assert not info.cpu().any(), info.cpu()
            for k, (q, (c, s, z)) in enumerate(zip(outs, ref)):
                assert torch.equal(q.codes.cpu(), c), (slots, k)
                assert torch.equal(q.scales.cpu(), s), (slots, k)
                assert torch.equal(q.zeros.cpu(), z), (slots, k)
            log(f"  {slots} slots: all {len(pairs)} layers bit-identical")
