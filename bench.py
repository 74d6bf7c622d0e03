"""Benchmark: one GPTQ layer quantization (int4, group 128) of a 4096 x 4096 layer on
one MI355X.

A step is one pass of the whole path on inputs already resident in HBM:
zero H, H += 2 X^T X over 262144 calibration tokens (bf16), damping + Cholesky
factor of the inverse (fp64), the blocked column sweep with trailing updates
(int4 asymmetric, group 128, B = 128), and dequantization of the result.
Prints one JSON line.  ``value`` = quantized weights per second.

Options: --steps K --warmup W --gpus N (only 1 is supported: the path runs on one
GPU) --no-cpu-baseline --calibrate-copy (adds, after the timed region, one plain
elementwise kernel that reads 1 GiB and writes 1 GiB (fp32 multiply by 1), used to
scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes).

--config N (1..5; default 2, the line above) instead times every layer of workload N
(1: 256x512; 3: MLP up/down pair at int4 and int3; 4: a decoder block of 7 linears;
5: the 49152/12288 fc pair) with the same step, and prints one JSON line with
ms/layer and the phase breakdown per layer.

--obq times GPTQ against OBQ (gptq_obq_layer, the per-row greedy method) on the same
layers from the same U and prints their runtime ratio.

--linear measures, instead of the layer step, the product of the quantized layer with
activations read from the stored format (gptq_quantized_linear) for 1, 4, 16, 32, 64, 128 and 256
tokens, beside torch's bf16 product with the unquantized weights, and prints its own
JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GPTQ quantized weights/sec + ms/layer (int4 g128) at 4096x4096, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0
HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hess_bf16_c2_traffic.json")
LINEAR_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "linear_int4_g128_1tok_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--linear", action="store_true")
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--obq", action="store_true")
    ap.add_argument("--no-kernel-split", action="store_true",
                    help="skip the profiled step that splits the quantize phase by kernel")
    return ap.parse_args()


def source_hash(name: str) -> str:
    with open(os.path.join(ROOT, "post_weight_quantization_25_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(launch_bytes_alg: float = 0.0, path: str | None = None, source: str = "hessian.hip"):
    """HBM bytes per launch from a committed rocprofv3 counter summary (the Hessian's by
    default), or None when the kernel source changed since the counters were taken."""
    try:
        with open(path or TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_hash(source):
        return None
    return t.get("bytes_per_launch")


MFMA_BUSY_FILE = os.path.join(ROOT, "profiles", "mfma_busy_c2.json")


SWEEP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sweep_trail_c2_traffic.json")


def _committed(path):
    """A committed rocprofv3 counter summary, or None when a kernel source it names
    changed since the counters were taken."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    for src, h in t.get("source_sha256_16", {}).items():
        if source_hash(src) != h:
            return None
    return t


def measured_mfma_busy():
    """MFMA-busy fraction per kernel (Hessian, trailing update, sweep) of the 4096 x 4096
    layer from the committed counter summary; a kernel's entry is None once a file it is
    built from changed since the counters were taken."""
    try:
        with open(MFMA_BUSY_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    hashes, deps = t.get("source_sha256_16", {}), t.get("kernel_sources", {})
    out = {}
    for k, v in t.get("mfma_busy", {}).items():
        files = deps.get(k, list(hashes))
        out[k] = v if files and all(f in hashes and source_hash(f) == hashes[f] for f in files) else None
    return out


def phase_rooflines(split, r, d, bits: int = 4, group: int = 128):
    """Algorithmic rates of the sweep (HBM) and the trailing update (16-bit MFMA) from the
    per-phase kernel times.  Sweep bytes per layer: the fp32 working copy read once (4 B),
    the scaled fp16 error pair written (4 B), bits / 8 bytes of codes per weight, a scale
    and a zero per group, the diagonal blocks of U (d x 128 fp32).  Trailing-kernel flops: the
    products after each 512-column super-block, 2 r sum_s 512 (d - s1) (the updates
    inside a super-block run in the sweep kernel)."""
    out = {}
    sweep_ms, trail_ms = split.get("sweep"), split.get("trail")
    traffic = _committed(SWEEP_TRAFFIC_FILE) if (r, d) == (4096, 4096) else None
    busy = measured_mfma_busy() if (r, d) == (4096, 4096) else None
    if sweep_ms:
        ng = 1 if group <= 0 else d // group
        byt = r * d * (4 + 4 + bits / 8) + r * ng * 4 + d * 128 * 4
        gbs = byt / (sweep_ms * 1e-3) / 1e9
        out["sweep"] = {"bound": "hbm", "algorithmic_bytes": byt, "ms": sweep_ms, "achieved": gbs,
                        "unit": "GB/s", "peak": HBM_GBS, "frac": gbs / HBM_GBS,
                        "traffic": traffic["sweep_kernel"]["bytes_per_layer"] if traffic else None}
        if traffic:
            out["sweep"]["traffic_frac"] = traffic["sweep_kernel"]["bytes_per_layer"] / (sweep_ms * 1e-3) / 1e9 / HBM_GBS
    if trail_ms:
        fl = 2.0 * r * sum(min(512, d - s0) * (d - min(s0 + 512, d)) for s0 in range(0, d, 512))
        tf = fl / (trail_ms * 1e-3) / 1e12
        out["trail"] = {"bound": "mfma", "algorithmic_flops": fl, "ms": trail_ms, "achieved": tf,
                        "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS,
                        "mfma_busy": busy.get("trail_dma_kernel") if busy else None,
                        "traffic": traffic["trail_bytes_per_layer"] if traffic else None,
                        "note": "products after each super-block (the updates inside a super-block run in "
                                "the sweep kernel); three fp16 products are issued per algorithmic one"}
    return out


def calibrate_copy(dev):
    """One plain elementwise kernel that reads 1 GiB and writes 1 GiB (fp32 times 1): the
    known-size reference for scaling FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()


# kernel name -> phase of the step (kernels of the library; torch's own fills go to "other")
KERNEL_PHASES = [("hess_", "hess"), ("prep_", "prep"), ("gemm_f64", "prep"), ("sweep_kernel", "sweep"),
                 ("trail_", "trail"), ("convert_kernel", "quant_setup"), ("split_u_kernel", "quant_setup"),
                 ("udt_kernel", "quant_setup"), ("row_params", "quant_setup"), ("tensor_", "quant_setup"),
                 ("dequant_kernel", "deq")]


def kernel_split(step, steps: int = 2):
    """Per-phase kernel time of ``steps`` steps (mean per step, ms), from torch's profiler,
    which records every kernel the process launches (the library's included), by kernel
    name.  The quantize phase splits into the sweep, the trailing update and its set-up
    kernels; kernels on two streams (the factorization's inverse) may overlap, so the
    prep sum can exceed its wall time."""
    import torch
    from torch.profiler import ProfilerActivity, profile
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
    out, per_kernel = {}, {}
    for e in prof.events():
        dt = getattr(e, "device_time", None)
        if dt is None:
            dt = getattr(e, "cuda_time", 0.0)
        if not dt or str(getattr(e, "device_type", "")).find("CUDA") < 0:
            continue
        ph = next((v for k, v in KERNEL_PHASES if k in e.name), "other")
        out[ph] = out.get(ph, 0.0) + dt / 1000.0 / steps
        per_kernel[e.name] = per_kernel.get(e.name, 0.0) + dt / 1000.0 / steps
    return out, per_kernel


def cpu_baseline(layer, sample_tokens: int, sample_rows: int):
    """The fp64 oracle on a bounded sample of the same workload, scaled to one layer."""
    import numpy as np

    import synth
    from oracle import gptq_oracle as o

    t0 = time.perf_counter()
    scales = synth.channel_scales(layer)
    chunks = [synth.x_as_f64(synth.x_chunk(layer, c, scales)) for c in range(sample_tokens // synth.CHUNK)]
    t_gen = time.perf_counter() - t0
    t0 = time.perf_counter()
    Hs = o.hessian(chunks)
    t_hess = time.perf_counter() - t0
    H = Hs * (layer.n_tokens / sample_tokens)
    t0 = time.perf_counter()
    U, _ = o.prepare_u(H, 0.01)
    t_prep = time.perf_counter() - t0
    W = synth.w_as_f64(synth.weights(layer))[:sample_rows]
    t0 = time.perf_counter()
    o.gptq_blocked(W, U, o.Params(bits=4, group_size=128))
    t_sweep = time.perf_counter() - t0
    hess_full = t_hess * layer.n_tokens / sample_tokens
    sweep_full = t_sweep * layer.d_row / sample_rows
    total = hess_full + t_prep + sweep_full
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {
        "value": layer.d_row * layer.d_col / total,
        "unit": "weights/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle: H on {sample_tokens} of {layer.n_tokens} tokens "
                   f"({t_hess:.2f} s, scaled x{layer.n_tokens // sample_tokens}), full prep at d=4096 "
                   f"({t_prep:.2f} s), blocked sweep on {sample_rows} of {layer.d_row} rows "
                   f"({t_sweep:.2f} s, scaled x{layer.d_row // sample_rows}); "
                   f"extrapolated {total:.1f} s per layer; input generation {t_gen:.1f} s not counted"),
        "seconds_per_layer": total,
    }


def config_cpu_baseline(layers):
    """The fp64 oracle, unmodified, on a bounded sample of every layer of a workload, each
    scaled to the whole layer (the sample is stated per layer):
    * H on a token subset (8192 tokens), scaled linearly in the token count; at d_col
      49152 on the leading 12288 channels of 1024 tokens, scaled by (49152 / 12288)^2 as
      well (NumPy's X^T X of a 1024 x 49152 fp64 matrix ends in a segmentation fault
      inside its BLAS call, on this image);
    * prep (the oracle's Cholesky route) in full at each distinct d_col up to 12288, timed
      once per workload and width; at d_col 49152 the leading 12288 block is factored and
      the time scaled by (49152 / 12288)^3;
    * the blocked sweep on 32 and on 128 rows, extrapolated linearly in the row count (a
      sweep's per-column cost has a part independent of the rows); at d_col 49152 with the
      12288-wide factor and scaled by (49152 / 12288)^2 (the trailing products dominate).
    Input generation is not counted."""
    import numpy as np

    import synth
    from oracle import gptq_oracle as o
    out, prep_cache, t_all = [], {}, 0.0
    for L in layers:
        d = L.d_col
        tok = min(L.n_tokens, 8192 if d <= 12288 else 1024)
        dh = min(d, 12288)
        scales = synth.channel_scales(L)
        chunk = synth.x_as_f64(synth.x_chunk(L, 0, scales))[:tok]
        t0 = time.perf_counter()
        Hs = o.hessian([chunk[:, :dh]])
        t_h = (time.perf_counter() - t0) * L.n_tokens / tok * (d / dh) ** 2
        H = Hs * (L.n_tokens / tok)
        if dh not in prep_cache:
            t0 = time.perf_counter()
            U, _ = o.prepare_u(H, 0.01)
            prep_cache[dh] = (time.perf_counter() - t0, U)
        t_p, U = prep_cache[dh]
        t_p *= (d / dh) ** 3
        Wf = synth.w_as_f64(synth.weights(L))
        p = o.Params(bits=L.bits, group_size=L.group_size, sym=L.sym)
        ts = []
        for nr in (32, 128):
            t0 = time.perf_counter()
            o.gptq_blocked(Wf[:nr, :dh], U, p)
            ts.append(time.perf_counter() - t0)
        per_row = (ts[1] - ts[0]) / 96.0
        t_s = (ts[0] + per_row * (L.d_row - 32)) * (d / dh) ** 2
        tot = t_h + t_p + t_s
        t_all += tot
        print(f"[oracle] {L.name}: {tot:.1f} s per layer (hess {t_h:.1f}, prep {t_p:.1f}, sweep {t_s:.1f})",
              file=sys.stderr, flush=True)
        out.append({"name": L.name, "seconds_per_layer": tot, "hess_s": t_h, "prep_s": t_p, "sweep_s": t_s,
                    "sample": f"H on {tok} of {L.n_tokens} tokens"
                              f"{' and 12288 channels, scaled by (d/12288)^2' if d > dh else ''}; prep at d={dh}"
                              f"{' scaled by (d/12288)^3' if d > dh else ''}; sweep on 32 and 128 rows"
                              f"{' of a 12288-wide slice, scaled by (d/12288)^2' if d > dh else ''}, extrapolated "
                              f"to {L.d_row} rows"})
        del H, Hs
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    w_tot = sum(L.d_row * L.d_col for L in layers)
    return {"value": w_tot / t_all, "unit": "weights/s", "cores": cores, "kind": "oracle",
            "sample": "per layer, see layers (fp64 NumPy oracle; prep timed once per distinct width)",
            "seconds_all_layers": t_all, "layers": out}


def linear_bench(args, g, q, W, r, d):
    """Time gptq_quantized_linear on the quantized metric layer for 1, 4, 16, 32, 64, 128 and 256 bf16
    tokens, and torch's bf16 product with the unquantized weights on the same
    activations.  Each is captured as a graph of 100 back-to-back calls (so that host
    launch overhead does not hide the kernel time) and replayed: HIP events around 5
    replays after 2 warm-up replays, mean per call."""
    import torch
    reps = 100

    def timed(f):
        f()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(reps):
                f()
        for _ in range(2):
            gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / (5 * reps)

    gen = torch.Generator(device="cuda").manual_seed(5)
    per = {}
    for nt in (1, 4, 16, 32, 64, 128, 256):
        x = torch.randn((nt, d), generator=gen, device="cuda").to(torch.bfloat16)
        y = torch.empty((nt, r), dtype=torch.bfloat16, device="cuda")
        yb = torch.empty((nt, r), dtype=torch.bfloat16, device="cuda")
        us_q = timed(lambda: g.linear(q, x, out=y))
        us_b = timed(lambda: torch.matmul(x, W.t(), out=yb))
        # algorithmic bytes: codes, scales and zeros once, activations in, outputs out
        byt = r * d // 2 + 2 * 2 * r * (d // 128) + 2 * nt * d + 2 * nt * r
        per[str(nt)] = {"us": us_q, "bf16_matmul_us": us_b, "speedup": us_b / us_q,
                        "algorithmic_bytes": byt, "GBps": byt / (us_q * 1e-6) / 1e9}
    one = per["1"]
    rec = {
        "metric": "quantized linear (int4 g128 codes read directly) time per call, 1 token, 4096x4096",
        "value": one["us"], "unit": "us", "n_gpus": 1, "steps": 5 * reps, "warmup": 2 * reps,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "the quantized attention projection of the layer step (4096x4096, int4 asym g128), "
                               "bf16 activations of 1, 4, 16, 32, 64, 128 and 256 tokens, bf16 output", "d_row": r, "d_col": d},
        "per_tokens": per,
        "roofline": {"kernel": "linear_kernel (1 token)", "bound": "hbm", "achieved": one["GBps"],
                     "peak": HBM_GBS, "unit": "GB/s", "frac": one["GBps"] / HBM_GBS,
                     "traffic": measured_traffic(path=LINEAR_TRAFFIC_FILE, source="linear.hip")},
    }
    print(json.dumps(rec), flush=True)


CONFIG_WORKLOADS = {
    1: "single linear layer 256x512: W fp32 ~N(0,0.02^2), X 2048x512 fp32 N(0,1) with 4 channels x20; int4 asym g128",
    2: "attention projection 4096x4096: W bf16 ~N(0,0.02^2), X 262144x4096 bf16 (log-normal channel scales, "
       "4 channels x50); int4 asym g128",
    3: "MLP pair: up 11008x4096 and down 4096x11008, bf16 ~N(0,0.02^2), X 131072 tokens Student-t(4); "
       "int4 g128 and int3 g128 asym",
    4: "decoder block of 7 linears (q, k, v, o 4096x4096; gate, up 11008x4096; down 4096x11008), bf16 "
       "~N(0,0.02^2), each its own X of 65536 bf16 N(0,1) tokens; int3 per-channel symmetric",
    5: "large layers: fc1 49152x12288 and fc2 12288x49152, bf16 ~N(0,0.01^2), X 262144 bf16 N(0,1) tokens "
       "with 0.1% channels x30; int4 asym g128",
}


def _upload(L, dev):
    """The layer's synthetic X and W (the seeded generator's chunks) resident on the device."""
    import numpy as np
    import torch

    import synth
    dt = torch.bfloat16 if L.x_dtype == "bf16" else torch.float32
    X = torch.empty((L.n_tokens, L.d_col), dtype=dt, device=dev)
    for c, arr in enumerate(synth.x_chunks(L)):
        lo = c * synth.CHUNK
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16) if arr.dtype == np.uint16 else torch.from_numpy(arr)
        X[lo:lo + arr.shape[0]].copy_(t)
    w = synth.weights(L)
    W = (torch.from_numpy(w.view(np.int16)).view(torch.bfloat16) if w.dtype == np.uint16 else torch.from_numpy(w)).to(dev)
    return X, W


def layer_bench(g, L, dev, steps: int, warmup: int, damp: float = 0.01, split: bool = True):
    """One layer's step (zero H, Hessian, prep, quantize, dequantize) with inputs resident:
    warm-up steps, then the mean per phase over timed steps (HIP events on the stream);
    with ``split``, one more profiled step splits the quantize phase into the sweep, the
    trailing update and their set-up kernels."""
    import numpy as np
    import torch
    t0 = time.perf_counter()
    X, W = _upload(L, dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t0
    n, d, r = L.n_tokens, L.d_col, L.d_row
    H = torch.empty((d, d), dtype=torch.float32, device=dev)
    ws_h = torch.empty(g.hessian_workspace_size(n, d), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(g.prepare_hinv_workspace_size(d), dtype=torch.uint8, device=dev)
    U = torch.empty((d, d), dtype=torch.float32, device=dev)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    p = g.make_params(L.bits, L.group_size, L.sym)
    ws_q = torch.empty(g.quantize_workspace_size(r, d, p), dtype=torch.uint8, device=dev)
    ng = 1 if L.group_size == 0 else d // L.group_size
    q = g.Quantized(torch.empty((r, g.code_bytes(L.bits, d)), dtype=torch.uint8, device=dev),
                    torch.empty((r, ng), dtype=torch.float16, device=dev),
                    torch.empty((r, ng), dtype=torch.float16, device=dev),
                    torch.zeros(1, dtype=torch.int32, device=dev), L.bits, L.group_size, d)
    What = torch.empty((r, d), dtype=torch.bfloat16, device=dev)
    ctx = g.Context(1)

    def step(ev=None):
        if ev: ev[0].record()
        H.zero_()
        g.hessian_accumulate(H, X, ws=ws_h)
        if ev: ev[1].record()
        g.prepare_hinv(H, damp, U=U, ws=ws_p, info=info, ctx=ctx)
        if ev: ev[2].record()
        g.quantize_layer(W, U, L.bits, L.group_size, L.sym, ws=ws_q, out=q)
        if ev: ev[3].record()
        g.dequantize(q, out=What)
        if ev: ev[4].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g.check_info(info, "prepare_hinv")
    g.check_info(q.info, "quantize_layer")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    ph = {nm: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
          for i, nm in enumerate(["hess", "prep", "quant", "deq"])}
    ms_layer = ph["hess"] + ph["prep"] + ph["quant"]
    rec = {"name": L.name, "d_row": r, "d_col": d, "n_tokens": n, "bits": L.bits, "group_size": L.group_size,
           "sym": bool(L.sym), "phases_ms": ph, "ms_per_layer": ms_layer,
           "ms_per_layer_quantize_only": ph["prep"] + ph["quant"],
           "weights_per_s": r * d / (ms_layer * 1e-3), "input_generation_s": t_gen}
    if split:
        ks, _ = kernel_split(step, steps=1)
        rec["kernel_ms"] = ks
        hfl = float(n) * d * (d + 1)
        rec["hess_frac_bf16"] = hfl / (ph["hess"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
        rec["phase_rooflines"] = phase_rooflines(ks, r, d, L.bits, L.group_size)
    return rec


def block_bench(g, layers, dev, steps: int, warmup: int, shared: bool):
    """The whole decoder block through gptq_quantize_layers (Hessians, factorizations and
    sweeps of different layers overlapped) for 1, 2 and 3 slots: HIP events around the
    call on the caller's stream, mean over the timed calls.  shared: q, k, v read q's
    inputs and gate, up read gate's (one H and one U per group), else every layer its own."""
    import torch
    data = [_upload(L, dev) for L in layers]
    if shared:
        src = {"c4_k": 0, "c4_v": 0, "c4_up": 4}
        data = [(data[src[L.name]][0] if L.name in src else X, W) for L, (X, W) in zip(layers, data)]
    L0 = layers[0]
    out = {}
    ctx = g.Context(3)
    for slots in (1, 2, 3):
        ws = torch.empty(g.quantize_layers_workspace_size(data, slots), dtype=torch.uint8, device=dev)
        res, info = g.quantize_layers(data, L0.bits, L0.group_size, L0.sym, 0.01, slots, ws=ws, ctx=ctx)
        for _ in range(max(0, warmup - 1)):
            g.quantize_layers(data, L0.bits, L0.group_size, L0.sym, 0.01, slots, ws=ws, outs=res, info=info, ctx=ctx)
        torch.cuda.synchronize()
        if info.cpu().any():
            raise RuntimeError(f"gptq_quantize_layers: status {info.cpu().tolist()}")
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for k in range(steps):
            ev[k][0].record()
            g.quantize_layers(data, L0.bits, L0.group_size, L0.sym, 0.01, slots, ws=ws, outs=res, info=info, ctx=ctx)
            ev[k][1].record()
        torch.cuda.synchronize()
        out[str(slots)] = float(sum(e[0].elapsed_time(e[1]) for e in ev) / steps)
        del ws
        torch.cuda.empty_cache()
    return out


def obq_bench(args):
    """GPTQ against OBQ (the per-row greedy method the pages compare with) on the same
    layer from the same U: the 256 x 512 layer of workload 1 and a 1024 x 1024 layer of
    workload 2's recipe (8192 tokens), int4 asymmetric, one group per row (the grid OBQ
    uses here).  HIP events around each call, mean over the timed calls."""
    import torch

    import post_weight_quantization_25_amd as g
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sizes = [synth.config_layers(1)[0], synth.scaled(synth.config_layers(2)[0], 1024, 1024, 8192)]
    rows = []
    for L in sizes:
        X, W = _upload(L, dev)
        d = L.d_col
        H = torch.zeros((d, d), dtype=torch.float32, device=dev)
        g.hessian_accumulate(H, X)
        U, info = g.prepare_hinv(H, 0.01)
        ws_q = torch.empty(g.quantize_workspace_size(L.d_row, d, g.make_params(4, 0)), dtype=torch.uint8, device=dev)
        ws_o = torch.empty(int(g.lib.gptq_obq_workspace_size(L.d_row, d)), dtype=torch.uint8, device=dev)

        def timed(f, n):
            f()
            torch.cuda.synchronize()
            e = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
            for k in range(n):
                e[k][0].record(); f(); e[k][1].record()
            torch.cuda.synchronize()
            return float(sum(a.elapsed_time(b) for a, b in e) / n)

        qg = g.quantize_layer(W, U, 4, 0, False, ws=ws_q)
        qo = g.obq_layer(W, U, 4, False, ws=ws_o)
        ms_g = timed(lambda: g.quantize_layer(W, U, 4, 0, False, ws=ws_q, out=qg), max(args.steps, 3))
        print(f"[obq] {L.d_row}x{d}: GPTQ {ms_g:.3f} ms", file=sys.stderr, flush=True)
        ms_o = timed(lambda: g.obq_layer(W, U, 4, False, ws=ws_o, out=qo), 2)
        print(f"[obq] {L.d_row}x{d}: OBQ {ms_o:.3f} ms", file=sys.stderr, flush=True)
        g.check_info(info, "prepare_hinv"); g.check_info(qg.info, "quantize_layer"); g.check_info(qo.info, "obq")
        rows.append({"d_row": L.d_row, "d_col": d, "gptq_ms": ms_g, "obq_ms": ms_o, "ratio": ms_o / ms_g})
        del X, W, H, U, ws_q, ws_o
        torch.cuda.empty_cache()
    rec = {"metric": "OBQ / GPTQ runtime ratio on the same layer from the same U (int4 asym, one group per row)",
           "value": rows[-1]["ratio"], "unit": "x", "n_gpus": 1, "higher_is_better": True, "vs_baseline": None,
           "dtype": "f32", "data": "synthetic", "config": {"workload": "256x512 (workload 1) and 1024x1024 "
                                                          "(workload 2 recipe, 8192 tokens)"}, "layers": rows}
    print(json.dumps(rec), flush=True)


def config_bench(args, cfg: int):
    """ms/layer and weights/s for every layer of one workload, printed as one JSON line."""
    import torch

    import post_weight_quantization_25_amd as g
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = []
    for L in synth.config_layers(cfg):
        print(f"[config {cfg}] {L.name} {L.d_row}x{L.d_col} n={L.n_tokens}: start", file=sys.stderr, flush=True)
        res = layer_bench(g, L, dev, args.steps, args.warmup, split=not args.no_kernel_split)
        print(f"[config {cfg}] {L.name}: {res['ms_per_layer']:.3f} ms/layer "
              f"(inputs {res['input_generation_s']:.1f} s)", file=sys.stderr, flush=True)
        layers.append(res)
        torch.cuda.empty_cache()
    tot_w = sum(x["d_row"] * x["d_col"] for x in layers)
    tot_ms = sum(x["ms_per_layer"] for x in layers)
    rec = {"metric": METRIC, "value": tot_w / (tot_ms * 1e-3), "unit": "weights/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if cfg != 1 else "f32", "data": "synthetic",
           "config": {"workload": CONFIG_WORKLOADS[cfg], "index": cfg, "damp": 0.01, "block_size": 128},
           "layers": layers, "ms_all_layers": tot_ms}
    if cfg == 4:
        # the block in one call (phases of different layers overlapped), each layer with its
        # own inputs as above, and with q/k/v and gate/up sharing theirs as in a real block
        Ls = synth.config_layers(cfg)
        for shared in (False, True):
            key = "block_shared_inputs_ms" if shared else "block_ms"
            print(f"[config {cfg}] block in one call, shared inputs={shared}", file=sys.stderr, flush=True)
            rec[key] = block_bench(g, Ls, dev, args.steps, args.warmup, shared)
            torch.cuda.empty_cache()
        best = min(rec["block_ms"].values())
        rec["block_weights_per_s"] = tot_w / (best * 1e-3)
        rec["value"] = rec["block_weights_per_s"]
        rec["value_note"] = "block of 7 layers in one gptq_quantize_layers call, best slot count, own inputs per layer"
    if not args.no_cpu_baseline:
        print(f"[config {cfg}] oracle baseline on the host", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = config_cpu_baseline(synth.config_layers(cfg))
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the GPTQ layer quantizer runs on one GPU; only --gpus 1 is supported "
              "(rows shard with no communication and H needs one all-reduce, which this library "
              "does not implement)", file=sys.stderr)
        sys.exit(2)

    if args.obq:
        obq_bench(args)
        return
    if args.config != 2:
        config_bench(args, args.config)
        return

    import numpy as np
    import torch

    import post_weight_quantization_25_amd as g
    import synth

    layer = synth.config_layers(2)[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n, d, r = layer.n_tokens, layer.d_col, layer.d_row

    # synthetic inputs, generated chunk by chunk on the host and kept resident in HBM
    X = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    for c, arr in enumerate(synth.x_chunks(layer)):
        lo = c * synth.CHUNK
        X[lo:lo + arr.shape[0]].copy_(torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16))
    W = torch.from_numpy(synth.weights(layer).view(np.int16)).view(torch.bfloat16).to(dev)
    H = torch.empty((d, d), dtype=torch.float32, device=dev)
    ws_h = torch.empty(g.hessian_workspace_size(n, d), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(g.prepare_hinv_workspace_size(d), dtype=torch.uint8, device=dev)
    U = torch.empty((d, d), dtype=torch.float32, device=dev)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    p = g.make_params(4, 128)
    ws_q = torch.empty(g.quantize_workspace_size(r, d, p), dtype=torch.uint8, device=dev)
    q = g.Quantized(torch.empty((r, d // 2), dtype=torch.uint8, device=dev),
                    torch.empty((r, d // 128), dtype=torch.float16, device=dev),
                    torch.empty((r, d // 128), dtype=torch.float16, device=dev),
                    torch.zeros(1, dtype=torch.int32, device=dev), 4, 128, d)
    What = torch.empty((r, d), dtype=torch.bfloat16, device=dev)
    ctx = g.Context(1)
    torch.cuda.synchronize()

    phases = ["hess", "prep", "quant", "deq"]

    def step(ev=None):
        if ev: ev[0].record()
        H.zero_()
        g.hessian_accumulate(H, X, ws=ws_h)
        if ev: ev[1].record()
        g.prepare_hinv(H, 0.01, U=U, ws=ws_p, info=info, ctx=ctx)
        if ev: ev[2].record()
        g.quantize_layer(W, U, 4, 128, ws=ws_q, out=q)
        if ev: ev[3].record()
        g.dequantize(q, out=What)
        if ev: ev[4].record()

    # the dominant kernel alone (Hessian SYRK), timed with events on the launch stream
    def hess_only(ev):
        ev[0].record()
        g.hessian_accumulate(H, X, ws=ws_h)
        ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    g.check_info(info, "prepare_hinv")
    g.check_info(q.info, "quantize_layer")
    if args.linear:
        linear_bench(args, g, q, W, r, d)
        if args.calibrate_copy:
            calibrate_copy(dev)
        return

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1000.0 / args.steps
    ph = {nm: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
          for i, nm in enumerate(phases)}

    hev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        hess_only(hev[k])
    torch.cuda.synchronize()
    hess_launch_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in hev]))

    if args.calibrate_copy:
        calibrate_copy(dev)
    split = None
    if not args.no_kernel_split:
        split, _ = kernel_split(step)

    flops_hess = float(n) * d * (d + 1)            # symmetric rank-n update, upper triangle incl. diagonal
    achieved = flops_hess / (hess_launch_ms * 1e-3) / 1e12
    ms_layer = ph["hess"] + ph["prep"] + ph["quant"]
    rec = {
        "metric": METRIC,
        "value": r * d / (ms_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attention projection 4096x4096: W bf16 ~N(0,0.02^2), X 262144x4096 bf16 "
                               "(log-normal channel scales, 4 channels x50), int4 asym g128, B=128, damp 0.01",
                   "d_row": r, "d_col": d, "n_tokens": n, "bits": 4, "group_size": 128, "block_size": 128,
                   "arithmetic": "H: bf16 MFMA, fp32 accumulate; prep: fp64 MFMA; sweep: fp32; trailing: fp16 hi/lo split of power-of-two-scaled operands (three products) on fp16 MFMA, fp32 accumulate"},
        "ms_per_layer": ms_layer,
        "ms_per_layer_quantize_only": ph["prep"] + ph["quant"],
        "phases_ms": ph,
        "roofline": {"kernel": "hess_bf16_kernel + hess_reduce_kernel (one gptq_hessian_accumulate call)",
                     "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(flops_hess),
                     "launch_ms": hess_launch_ms,
                     "algorithmic_flops_per_launch": flops_hess},
    }
    mb = measured_mfma_busy()
    rec["roofline"]["mfma_busy"] = mb.get("hess_bf16_kernel") if mb else None
    if split is not None:
        rec["kernel_ms"] = split
        rec["phase_rooflines"] = phase_rooflines(split, r, d)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(layer, sample_tokens=4 * 8192, sample_rows=256)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
