"""Seeded synthetic workloads for the GPTQ layer quantizer.

This module only draws random numbers and rounds them to storage dtypes; it
holds none of the quantizer's arithmetic.  Both the CPU oracle (through the
tests and the benchmark) and the GPU path consume what it produces.

Every stream is a NumPy ``default_rng([seed, role, chunk])`` with
``seed = 1000 * config + layer``, role 0 = weights, 1 = activations,
2 = channel scales and outlier choice.  Activations are produced in chunks
of ``CHUNK`` tokens so that a consumer never needs more than one chunk in
host memory and any chunk can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterator

import numpy as np

CHUNK = 8192
ROLE_W, ROLE_X, ROLE_CH = 0, 1, 2


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Layer:
    """One linear layer workload: W is d_row x d_col, X is n_tokens x d_col."""
    name: str
    d_row: int
    d_col: int
    n_tokens: int
    w_std: float
    w_dtype: str            # "f32" or "bf16"
    x_dtype: str            # "f32" or "bf16"
    x_dist: str             # "normal" or "student_t4"
    chan_scale: str         # "none" or "lognormal"
    n_outliers: int         # channels multiplied by outlier_mult
    outlier_mult: float
    bits: int
    group_size: int         # 0 = one group per row
    sym: bool
    seed: int


def _x_chunk_f32(layer: Layer, chunk: int, scales: np.ndarray) -> np.ndarray:
    lo = chunk * CHUNK
    rows = min(CHUNK, layer.n_tokens - lo)
    rng = np.random.default_rng([layer.seed, ROLE_X, chunk])
    if layer.x_dist == "normal":
        z = rng.standard_normal((rows, layer.d_col), dtype=np.float32)
    elif layer.x_dist == "student_t4":
        z = rng.standard_t(4.0, size=(rows, layer.d_col)).astype(np.float32)
    else:
        raise ValueError(layer.x_dist)
    z *= scales[None, :]
    return z


def channel_scales(layer: Layer) -> np.ndarray:
    """Per-input-channel multipliers (log-normal spread and outlier channels)."""
    rng = np.random.default_rng([layer.seed, ROLE_CH, 0])
    s = np.ones(layer.d_col, dtype=np.float64)
    if layer.chan_scale == "lognormal":
        s = rng.lognormal(0.0, 1.0, size=layer.d_col)
    if layer.n_outliers > 0:
        idx = rng.choice(layer.d_col, size=layer.n_outliers, replace=False)
        s[idx] *= layer.outlier_mult
    return s.astype(np.float32)


def n_chunks(layer: Layer) -> int:
    return (layer.n_tokens + CHUNK - 1) // CHUNK


def x_chunk(layer: Layer, chunk: int, scales: np.ndarray | None = None) -> np.ndarray:
    """Chunk ``chunk`` of X in its storage dtype: float32 array, or uint16 bf16 bits."""
    if scales is None:
        scales = channel_scales(layer)
    z = _x_chunk_f32(layer, chunk, scales)
    return f32_to_bf16_bits(z) if layer.x_dtype == "bf16" else z


def x_chunks(layer: Layer, threads: int | None = None) -> Iterator[np.ndarray]:
    """All chunks of X in order (storage dtype), generated a few at a time on host threads."""
    scales = channel_scales(layer)
    threads = threads or min(8, len(os.sched_getaffinity(0)))
    nc = n_chunks(layer)
    with ThreadPoolExecutor(threads) as ex:
        for base in range(0, nc, threads):
            ids = range(base, min(nc, base + threads))
            for a in ex.map(lambda c: x_chunk(layer, c, scales), ids):
                yield a


def x_as_f64(chunk: np.ndarray) -> np.ndarray:
    """Storage-dtype chunk -> float64 values (exact)."""
    if chunk.dtype == np.uint16:
        return bf16_bits_to_f32(chunk).astype(np.float64)
    return chunk.astype(np.float64)


def weights(layer: Layer) -> np.ndarray:
    """W in its storage dtype: float32 array, or uint16 bf16 bits."""
    rng = np.random.default_rng([layer.seed, ROLE_W, 0])
    w = (rng.standard_normal((layer.d_row, layer.d_col), dtype=np.float32) * np.float32(layer.w_std))
    return f32_to_bf16_bits(w) if layer.w_dtype == "bf16" else w


def w_as_f64(w: np.ndarray) -> np.ndarray:
    if w.dtype == np.uint16:
        return bf16_bits_to_f32(w).astype(np.float64)
    return w.astype(np.float64)


# ---------------------------------------------------------------------------
# The five workloads (sizes, distributions and quantizer settings of the
# GPTQ layer-quantization configurations) and scaled-down variants of the same
# recipes for element-by-element parity.

def _layer(cfg, idx, name, d_row, d_col, n, **kw):
    return Layer(name=name, d_row=d_row, d_col=d_col, n_tokens=n, seed=1000 * cfg + idx, **kw)


def config_layers(cfg: int) -> list[Layer]:
    if cfg == 1:
        return [_layer(1, 0, "c1", 256, 512, 2048, w_std=0.02, w_dtype="f32", x_dtype="f32",
                       x_dist="normal", chan_scale="none", n_outliers=4, outlier_mult=20.0,
                       bits=4, group_size=128, sym=False)]
    if cfg == 2:
        return [_layer(2, 0, "c2", 4096, 4096, 262144, w_std=0.02, w_dtype="bf16", x_dtype="bf16",
                       x_dist="normal", chan_scale="lognormal", n_outliers=4, outlier_mult=50.0,
                       bits=4, group_size=128, sym=False)]
    if cfg == 3:
        out = []
        for bits in (4, 3):
            base = 0 if bits == 4 else 2
            kw = dict(w_std=0.02, w_dtype="bf16", x_dtype="bf16", x_dist="student_t4",
                      chan_scale="none", n_outliers=0, outlier_mult=1.0, bits=bits,
                      group_size=128, sym=False)
            out.append(_layer(3, base + 0, f"c3_up_int{bits}", 11008, 4096, 131072, **kw))
            out.append(_layer(3, base + 1, f"c3_down_int{bits}", 4096, 11008, 131072, **kw))
        return out
    if cfg == 4:
        shapes = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                  ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
        return [_layer(4, i, f"c4_{n}", r, c, 65536, w_std=0.02, w_dtype="bf16", x_dtype="bf16",
                       x_dist="normal", chan_scale="none", n_outliers=0, outlier_mult=1.0,
                       bits=3, group_size=0, sym=True)
                for i, (n, r, c) in enumerate(shapes)]
    if cfg == 5:
        kw = dict(w_std=0.01, w_dtype="bf16", x_dtype="bf16", x_dist="normal", chan_scale="none",
                  outlier_mult=30.0, bits=4, group_size=128, sym=False)
        return [_layer(5, 0, "c5_fc1", 49152, 12288, 262144, n_outliers=12, **kw),
                _layer(5, 1, "c5_fc2", 12288, 49152, 262144, n_outliers=49, **kw)]
    raise ValueError(cfg)


def scaled(layer: Layer, d_row: int, d_col: int, n_tokens: int, seed_offset: int = 500) -> Layer:
    """Same recipe at a smaller shape (outlier count scaled to the new width, at least 1)."""
    n_out = 0
    if layer.n_outliers:
        n_out = max(1, round(layer.n_outliers * d_col / layer.d_col))
    return dataclasses.replace(layer, name=f"{layer.name}_{d_row}x{d_col}x{n_tokens}",
                               d_row=d_row, d_col=d_col, n_tokens=n_tokens,
                               n_outliers=n_out, seed=layer.seed + seed_offset)
