"""GPTQ layer quantizer for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libgptq.so`` (C ABI declared in ``include/gptq.h``).
Every step of the computation runs in the library's HIP kernels; this module only
checks tensor placement/dtypes, allocates caller-owned buffers with PyTorch and
passes raw device pointers and the current HIP stream.  If the library is missing
the import fails: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgptq.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_NOT_PD, ERR_NONFINITE = range(7)
F32, BF16, F16 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class GptqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("sym", ctypes.c_int32), ("block_size", ctypes.c_int32)]


class LayerDesc(ctypes.Structure):
    """gptq_layer: one layer's inputs, weights and outputs (device pointers)."""
    _fields_ = [("X", ctypes.c_void_p), ("x_dtype", ctypes.c_int), ("n_tokens", ctypes.c_int64),
                ("ldx", ctypes.c_int64), ("W", ctypes.c_void_p), ("w_dtype", ctypes.c_int),
                ("d_row", ctypes.c_int64), ("d_col", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("scales_f16", ctypes.c_void_p), ("zeros_f16", ctypes.c_void_p)]


LAYERS_MAX_SLOTS = 4


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python -m post_weight_quantization_25_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "gptq_hessian_workspace_size": (sz, [i64, i64]),
        "gptq_hessian_accumulate": (ctypes.c_int, [vp, vp, ctypes.c_int, i64, i64, i64, vp, sz, vp]),
        "gptq_prepare_hinv_workspace_size": (sz, [i64]),
        "gptq_context_create": (ctypes.c_int, [i32, ctypes.POINTER(vp)]),
        "gptq_context_destroy": (ctypes.c_int, [vp]),
        "gptq_context_set_wait_limit": (ctypes.c_int, [vp, ctypes.c_int32]),
        "gptq_prepare_hinv": (ctypes.c_int, [vp, vp, i64, ctypes.c_float, vp, sz, vp, vp, vp]),
        "gptq_quantize_workspace_size": (sz, [i64, i64, ctypes.POINTER(Params)]),
        "gptq_quantize_layer": (ctypes.c_int, [vp, ctypes.c_int, i64, i64, vp, ctypes.POINTER(Params),
                                               vp, vp, vp, vp, sz, vp, vp]),
        "gptq_quantize_layer_noalloc": (ctypes.c_int, [vp, ctypes.c_int, i64, i64, vp, ctypes.POINTER(Params),
                                                       vp, vp, vp, vp, vp]),
        "gptq_quantize_layers_workspace_size": (sz, [ctypes.POINTER(LayerDesc), i32, i32]),
        "gptq_quantize_layers": (ctypes.c_int, [ctypes.POINTER(LayerDesc), i32, ctypes.c_float,
                                                ctypes.POINTER(Params), i32, vp, sz, vp, vp, vp]),
        "gptq_obq_workspace_size": (sz, [i64, i64]),
        "gptq_obq_layer": (ctypes.c_int, [vp, ctypes.c_int, i64, i64, vp, ctypes.POINTER(Params),
                                          vp, vp, vp, vp, sz, vp, vp]),
        "gptq_dequantize": (ctypes.c_int, [vp, vp, vp, i64, i64, i32, i32, vp, ctypes.c_int, vp]),
        "gptq_dequantize_e2m1": (ctypes.c_int, [vp, vp, i64, i64, i32, vp, ctypes.c_int, vp]),
        "gptq_quantized_linear": (ctypes.c_int, [vp, vp, vp, i64, i64, i32, i32, vp, ctypes.c_int, i64, i64,
                                                 vp, ctypes.c_int, vp]),
        "gptq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


lib = _load()


def status_string(s: int) -> str:
    return lib.gptq_status_string(s).decode()


def _check(s: int, what: str):
    if s != OK:
        raise GptqError(s, f"{what}: {status_string(s)}")


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _tensor(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    """A contiguous device tensor of ``dtype`` (or one of a tuple of dtypes), ``shape`` and
    ``device`` where given: what the kernels assume of every buffer they are handed."""
    _dev(t, name)
    if dtype is not None and not (t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype):
        raise ValueError(f"{name} must have dtype {dtype}, not {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")


def _info(t: torch.Tensor, name: str, n: int, device):
    _tensor(t, name, torch.int32, None, device)
    if t.numel() < n:
        raise ValueError(f"{name} must hold at least {n} int32")


def _workspace(nbytes: int, device, ws):
    """The caller's workspace (a uint8 device tensor) if it is large enough, else a new one."""
    if nbytes == 0:
        return None
    if ws is not None:
        _tensor(ws, "ws", torch.uint8, None, device)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


# ---------------------------------------------------------------- context

class Context:
    """A gptq_context: HIP streams and events, owned by this object, with which
    ``prepare_hinv`` and ``quantize_layers`` overlap their own phases.  Made on the
    current device (or ``device``); ``close()`` (or garbage collection) waits for the
    work queued on them and releases them.  One context serves one call at a time."""

    def __init__(self, n_slots: int = LAYERS_MAX_SLOTS, device=None):
        self.device = torch.cuda.current_device() if device is None else torch.device(device).index
        self.n_slots = n_slots
        ptr = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(lib.gptq_context_create(n_slots, ctypes.byref(ptr)), "gptq_context_create")
        self._ptr = ptr.value

    @property
    def ptr(self):
        if not self._ptr:
            raise ValueError("context is closed")
        return self._ptr

    def set_wait_limit(self, polls: int):
        """Bound of the factorization's wait in calls with this context, in polls of
        about 128 clocks (0: give up at once, so that the call reports info = -2)."""
        _check(lib.gptq_context_set_wait_limit(self.ptr, int(polls)), "gptq_context_set_wait_limit")

    def close(self):
        if self._ptr:
            p, self._ptr = self._ptr, None
            _check(lib.gptq_context_destroy(p), "gptq_context_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ctx_ptr(ctx):
    return None if ctx is None else ctx.ptr


# ---------------------------------------------------------------- Hessian

def hessian_workspace_size(n_tokens: int, d_col: int) -> int:
    return lib.gptq_hessian_workspace_size(n_tokens, d_col)


def hessian_accumulate(H: torch.Tensor, X: torch.Tensor, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """H += 2 X^T X (X: tokens x d_col, rows may be strided). Returns H."""
    _dev(H, "H")
    if H.dtype != torch.float32 or H.dim() != 2 or H.shape[0] != H.shape[1]:
        raise ValueError("H must be a square float32 matrix")
    if not X.is_cuda or X.dim() != 2 or X.stride(1) != 1 or X.dtype not in _DT:
        raise ValueError("X must be a 2-D device tensor with unit column stride (f32/bf16/f16)")
    n, d = X.shape
    if d != H.shape[0]:
        raise ValueError("X width must match H")
    if X.device != H.device:
        raise ValueError("X and H must be on the same device")
    ws = _workspace(hessian_workspace_size(n, d), X.device, ws)
    _check(lib.gptq_hessian_accumulate(H.data_ptr(), X.data_ptr(), _DT[X.dtype], n, d, X.stride(0),
                                       ws.data_ptr() if ws is not None else None,
                                       ws.numel() if ws is not None else 0, _stream(stream)),
           "gptq_hessian_accumulate")
    return H


# ---------------------------------------------------------------- preparation

def prepare_hinv_workspace_size(d_col: int) -> int:
    return lib.gptq_prepare_hinv_workspace_size(d_col)


def prepare_hinv(H: torch.Tensor, percdamp: float = 0.01, U: torch.Tensor | None = None,
                 ws: torch.Tensor | None = None, info: torch.Tensor | None = None, stream=None,
                 ctx: Context | None = None):
    """Upper Cholesky factor U of (H + percdamp*mean(diag H) I)^-1.  Returns (U, info).
    With a Context the triangular inverse overlaps the factorization on its auxiliary
    stream; without one every kernel runs on ``stream`` (the same U either way)."""
    _dev(H, "H")
    if H.dim() != 2 or H.shape[0] != H.shape[1]:
        raise ValueError("H must be a square matrix")
    d = H.shape[0]
    _tensor(H, "H", torch.float32)
    if U is None:
        U = torch.empty((d, d), dtype=torch.float32, device=H.device)
    _tensor(U, "U", torch.float32, (d, d), H.device)
    if info is None:
        info = torch.zeros(1, dtype=torch.int32, device=H.device)
    _info(info, "info", 1, H.device)
    ws = _workspace(prepare_hinv_workspace_size(d), H.device, ws)
    _check(lib.gptq_prepare_hinv(H.data_ptr(), U.data_ptr(), d, float(percdamp),
                                 ws.data_ptr() if ws is not None else None,
                                 ws.numel() if ws is not None else 0, info.data_ptr(), _ctx_ptr(ctx),
                                 _stream(stream)),
           "gptq_prepare_hinv")
    return U, info


# ---------------------------------------------------------------- quantization

@dataclass
class Quantized:
    codes: torch.Tensor      # uint8, d_row x code_bytes(bits, d_col)
    scales: torch.Tensor     # float16, d_row x n_groups
    zeros: torch.Tensor      # float16, d_row x n_groups (integer values)
    info: torch.Tensor       # int32 device scalar
    bits: int
    group_size: int
    d_col: int
    fp4: bool = False        # codes on the E2M1 grid (sign bit 8 | magnitude index)


def code_bytes(bits: int, d_col: int) -> int:
    """Bytes of one row of stored codes: the 3-bit stream (eight codes in three bytes),
    two 4-bit codes per byte, or one byte per code."""
    return d_col // 8 * 3 if bits == 3 else d_col // 2 if bits == 4 else d_col


def _n_groups(group_size: int, d_col: int) -> int:
    return 1 if group_size <= 0 else max(1, d_col // group_size)


def _check_quantized(q: Quantized, name: str, d_row: int, device, zeros: bool = True):
    """q's arrays have the shapes and dtypes its bits, group size and width imply."""
    ng = _n_groups(q.group_size, q.d_col)
    _tensor(q.codes, f"{name}.codes", torch.uint8, (d_row, code_bytes(q.bits, q.d_col)), device)
    _tensor(q.scales, f"{name}.scales", torch.float16, (d_row, ng), device)
    if zeros:
        _tensor(q.zeros, f"{name}.zeros", torch.float16, (d_row, ng), device)


def _check_out(q: Quantized, d_row: int, d_col: int, bits: int, group_size: int, fp4: bool, device):
    if (q.bits, q.group_size, q.d_col, bool(q.fp4)) != (bits, group_size, d_col, bool(fp4)):
        raise ValueError(f"out was made for bits {q.bits}, group {q.group_size}, width {q.d_col}, fp4 {q.fp4}; "
                         f"this call has {bits}, {group_size}, {d_col}, {fp4}")
    _check_quantized(q, "out", d_row, device)
    _info(q.info, "out.info", 1, device)


def _check_wu(W: torch.Tensor, U: torch.Tensor):
    _dev(W, "W"); _dev(U, "U")
    if W.dim() != 2 or W.dtype not in _DT:
        raise ValueError("W must be a 2-D f32/bf16/f16 matrix")
    _tensor(U, "U", torch.float32, (W.shape[1], W.shape[1]), W.device)


def make_params(bits=4, group_size=128, sym=False, block_size=128, fp4=False, mx=False) -> Params:
    """sym: symmetric integer grid; fp4: the E2M1 grid (bits 4); mx: with fp4, power-of-two
    group scales (MXFP4)."""
    return Params(bits, group_size, (3 if mx else 2) if fp4 else int(bool(sym)), block_size)


def quantize_workspace_size(d_row: int, d_col: int, p: Params) -> int:
    return lib.gptq_quantize_workspace_size(d_row, d_col, ctypes.byref(p))


def quantize_layer(W: torch.Tensor, U: torch.Tensor, bits: int = 4, group_size: int = 128, sym: bool = False,
                   block_size: int = 128, ws: torch.Tensor | None = None, out: Quantized | None = None,
                   stream=None, fp4: bool = False, mx: bool = False) -> Quantized:
    _check_wu(W, U)
    d_row, d_col = W.shape
    p = make_params(bits, group_size, sym, block_size, fp4, mx)
    n_groups = _n_groups(group_size, d_col)
    if out is None:
        cb = code_bytes(bits, d_col)
        out = Quantized(torch.empty((d_row, cb), dtype=torch.uint8, device=W.device),
                        torch.empty((d_row, n_groups), dtype=torch.float16, device=W.device),
                        torch.empty((d_row, n_groups), dtype=torch.float16, device=W.device),
                        torch.zeros(1, dtype=torch.int32, device=W.device), bits, group_size, d_col, fp4)
    _check_out(out, d_row, d_col, bits, group_size, fp4, W.device)
    ws = _workspace(quantize_workspace_size(d_row, d_col, p), W.device, ws)
    _check(lib.gptq_quantize_layer(W.data_ptr(), _DT[W.dtype], d_row, d_col, U.data_ptr(), ctypes.byref(p),
                                   out.codes.data_ptr(), out.scales.data_ptr(), out.zeros.data_ptr(),
                                   ws.data_ptr() if ws is not None else None,
                                   ws.numel() if ws is not None else 0, out.info.data_ptr(), _stream(stream)),
           "gptq_quantize_layer")
    return out


NOALLOC_SCRATCH_BYTES = 256 << 20   # GPTQ_NOALLOC_SCRATCH_BYTES


def quantize_layer_noalloc(W: torch.Tensor, U: torch.Tensor, out: Quantized, bits: int = 4, group_size: int = 128,
                           sym: bool = False, stream=None, fp4: bool = False, mx: bool = False) -> Quantized:
    """gptq_quantize_layer_noalloc: as quantize_layer, with the library's per-device scratch
    in place of a workspace, into caller-allocated outputs (nothing is allocated here, so
    it can be captured in a graph).  Calls that overlap on one GPU race on the scratch."""
    _check_wu(W, U)
    d_row, d_col = W.shape
    p = make_params(bits, group_size, sym, 128, fp4, mx)
    _check_out(out, d_row, d_col, bits, group_size, fp4, W.device)
    _check(lib.gptq_quantize_layer_noalloc(W.data_ptr(), _DT[W.dtype], d_row, d_col, U.data_ptr(), ctypes.byref(p),
                                           out.codes.data_ptr(), out.scales.data_ptr(), out.zeros.data_ptr(),
                                           out.info.data_ptr(), _stream(stream)),
           "gptq_quantize_layer_noalloc")
    return out


def obq_layer(W: torch.Tensor, U: torch.Tensor, bits: int = 4, sym: bool = False, ws: torch.Tensor | None = None,
              out: Quantized | None = None, stream=None) -> Quantized:
    """OBQ (gptq_obq_layer): per-row greedy order, one group per row; a timing baseline."""
    _check_wu(W, U)
    d_row, d_col = W.shape
    p = make_params(bits, 0, sym)
    if out is None:
        out = Quantized(torch.empty((d_row, code_bytes(bits, d_col)), dtype=torch.uint8, device=W.device),
                        torch.empty((d_row, 1), dtype=torch.float16, device=W.device),
                        torch.empty((d_row, 1), dtype=torch.float16, device=W.device),
                        torch.zeros(1, dtype=torch.int32, device=W.device), bits, 0, d_col)
    _check_out(out, d_row, d_col, bits, 0, False, W.device)
    ws = _workspace(int(lib.gptq_obq_workspace_size(d_row, d_col)), W.device, ws)
    _check(lib.gptq_obq_layer(W.data_ptr(), _DT[W.dtype], d_row, d_col, U.data_ptr(), ctypes.byref(p),
                              out.codes.data_ptr(), out.scales.data_ptr(), out.zeros.data_ptr(),
                              ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
                              out.info.data_ptr(), _stream(stream)),
           "gptq_obq_layer")
    return out


def _layer_descs(pairs, outs):
    arr = (LayerDesc * len(pairs))()
    for k, ((X, W), q) in enumerate(zip(pairs, outs)):
        arr[k] = LayerDesc(X.data_ptr(), _DT[X.dtype], X.shape[0], max(X.stride(0), X.shape[1]), W.data_ptr(),
                           _DT[W.dtype], W.shape[0], W.shape[1], q.codes.data_ptr(), q.scales.data_ptr(),
                           q.zeros.data_ptr())
    return arr


def _layer_descs_shapes(pairs):
    """Descriptors with shapes only (the workspace size reads no pointer)."""
    arr = (LayerDesc * len(pairs))()
    for k, (X, W) in enumerate(pairs):
        arr[k] = LayerDesc(X.data_ptr(), _DT[X.dtype], X.shape[0], max(X.stride(0), X.shape[1]), None,
                           _DT[W.dtype], W.shape[0], W.shape[1], None, None, None)
    return arr


def quantize_layers_workspace_size(pairs, n_slots: int = 2) -> int:
    """Bytes of workspace for ``quantize_layers`` on these (X, W) pairs."""
    return int(lib.gptq_quantize_layers_workspace_size(_layer_descs_shapes(pairs), len(pairs), n_slots))


def quantize_layers(pairs, bits: int = 4, group_size: int = 128, sym: bool = False, percdamp: float = 0.01,
                    n_slots: int = 2, ws: torch.Tensor | None = None, outs: list | None = None,
                    info: torch.Tensor | None = None, stream=None, ctx: Context | None = None):
    """Quantize several layers in one call (gptq_quantize_layers): ``pairs`` is a list of
    (X, W) device tensors, X tokens x d_col (rows may be strided), W d_row x d_col.
    Consecutive pairs with the same X tensor share one H and one U.  With a Context the
    groups' phases overlap on its streams (``n_slots`` groups in flight); without one
    they run on ``stream`` one after another.  Returns (outs, info): one Quantized per
    layer and the device int32[2 n] status array."""
    if not pairs:
        return [], info
    dev = pairs[0][1].device
    for X, W in pairs:
        _dev(W, "W")
        if not X.is_cuda or X.dim() != 2 or X.stride(1) != 1 or X.dtype not in _DT or W.dtype not in _DT:
            raise ValueError("X must be 2-D with unit column stride and f32/bf16/f16, W f32/bf16/f16")
        if W.dim() != 2 or X.shape[1] != W.shape[1]:
            raise ValueError("X and W must have the same d_col")
        if X.device != dev or W.device != dev:
            raise ValueError("every X and W must be on one device")
    p = make_params(bits, group_size, sym)
    if outs is None:
        outs = []
        for _, W in pairs:
            d_row, d_col = W.shape
            n_groups = 1 if group_size <= 0 else max(1, d_col // group_size)
            outs.append(Quantized(torch.empty((d_row, code_bytes(bits, d_col)), dtype=torch.uint8, device=dev),
                                  torch.empty((d_row, n_groups), dtype=torch.float16, device=dev),
                                  torch.empty((d_row, n_groups), dtype=torch.float16, device=dev),
                                  torch.zeros(1, dtype=torch.int32, device=dev), bits, group_size, d_col))
    if len(outs) != len(pairs):
        raise ValueError("outs must hold one Quantized per (X, W) pair")
    for (_, W), q in zip(pairs, outs):
        _check_out(q, W.shape[0], W.shape[1], bits, group_size, False, dev)
    if info is None:
        info = torch.empty(2 * len(pairs), dtype=torch.int32, device=dev)
    _info(info, "info", 2 * len(pairs), dev)
    need = int(lib.gptq_quantize_layers_workspace_size(_layer_descs_shapes(pairs), len(pairs), n_slots))
    ws = _workspace(need, dev, ws)
    descs = _layer_descs(pairs, outs)
    _check(lib.gptq_quantize_layers(descs, len(pairs), percdamp, ctypes.byref(p), n_slots,
                                    ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
                                    info.data_ptr(), _ctx_ptr(ctx), _stream(stream)),
           "gptq_quantize_layers")
    return outs, info


def dequantize(q: Quantized, out_dtype=torch.float32, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _dev(q.codes, "q.codes")
    d_row = q.codes.shape[0]
    _check_quantized(q, "q", d_row, q.codes.device, zeros=not q.fp4)
    if out is None:
        out = torch.empty((d_row, q.d_col), dtype=out_dtype, device=q.codes.device)
    _tensor(out, "out", tuple(_DT), (d_row, q.d_col), q.codes.device)
    if q.fp4:
        _check(lib.gptq_dequantize_e2m1(q.codes.data_ptr(), q.scales.data_ptr(), d_row, q.d_col, q.group_size,
                                        out.data_ptr(), _DT[out.dtype], _stream(stream)), "gptq_dequantize_e2m1")
        return out
    _check(lib.gptq_dequantize(q.codes.data_ptr(), q.scales.data_ptr(), q.zeros.data_ptr(), d_row, q.d_col,
                               q.bits, q.group_size, out.data_ptr(), _DT[out.dtype], _stream(stream)),
           "gptq_dequantize")
    return out


def linear(q: Quantized, x: torch.Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """y = x What^T on the stored format (What as ``dequantize`` defines it), fp32 accumulation.
    x may be a row-strided view (its row pitch is passed as ldx)."""
    if q.fp4:
        raise ValueError("linear reads integer-grid codes; a layer on the E2M1 grid is dequantized with dequantize")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if x.dtype not in _DT or x.dim() != 2 or x.shape[1] != q.d_col or (x.shape[0] > 0 and x.stride(1) != 1):
        raise ValueError("x must be a (n_tokens, d_col) f32/bf16/f16 tensor with unit column stride")
    _dev(q.codes, "q.codes")
    d_row, n = q.codes.shape[0], x.shape[0]
    _check_quantized(q, "q", d_row, x.device)
    if out is None:
        out = torch.empty((n, d_row), dtype=out_dtype, device=x.device)
    if not out.is_contiguous() or tuple(out.shape) != (n, d_row):
        raise ValueError("out must be a contiguous (n_tokens, d_row) tensor")
    _tensor(out, "out", tuple(_DT), (n, d_row), x.device)
    _check(lib.gptq_quantized_linear(q.codes.data_ptr(), q.scales.data_ptr(), q.zeros.data_ptr(), d_row, q.d_col,
                                     q.bits, q.group_size, x.data_ptr(), _DT[x.dtype], n, max(x.stride(0), q.d_col),
                                     out.data_ptr(), _DT[out.dtype], _stream(stream)),
           "gptq_quantized_linear")
    return out


def check_info(info: torch.Tensor, what: str = "gptq"):
    """Synchronize on ``info`` and raise on a device-detected failure."""
    v = int(info.item())
    if v > 0:
        raise GptqError(ERR_NOT_PD, f"{what}: trailing principal submatrix of order {v} of the damped "
                                    "Hessian is not positive definite")
    if v == -2:
        raise GptqError(ERR_HIP, f"{what}: a bounded wait between workgroups of the factorization "
                                 "expired (device overloaded or preempted); results are undefined")
    if v < 0:
        raise GptqError(ERR_NONFINITE, f"{what}: {status_string(ERR_NONFINITE)}")
