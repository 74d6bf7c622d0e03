"""Parity of gptq_quantized_linear (y = x What^T on the stored format) with the oracle,
element by element, on seeded synthetic codes, scales, zeros and activations.

Tolerance (derived from the arithmetic).  The decode kernel forms, per 32-column piece
of a group, s = sum x (u - z) with fp32 fused multiply-adds, then acc += S16 s; the
batched kernel forms the same sums on the matrix cores per 128-column piece (products
of 16-bit values are exact in fp32) and then acc += S16 s.  Per element at most
d_col + 64 fp32 additions touch the result; they are taken at one unit in the last
place each (2^-23, so the bound does not assume the matrix cores round to nearest).
When a zero is not a small integer the batched kernel splits d = u - z into
hi = 16-bit(d) and lo = 16-bit(d - hi), |hi + lo - d| <= 2^-18 |d|.  So
|y - y_exact| <= ((d_col + 64) 2^-23 + 2^-18) sum_c |x_c What_rc|, plus the final
rounding to a 16-bit output type (2^-8 relative for bf16, 2^-11 for f16)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gptq_oracle as o
from gpu_helpers import log

pytestmark = pytest.mark.gpu


def make_case(d_row, d_col, bits, G, n, seed, frac_zeros=False):
    rng = np.random.default_rng([seed, d_row, d_col, bits, G, n])
    if bits == 8:
        packed = rng.integers(0, 256, size=(d_row, d_col), dtype=np.uint8)
    elif bits == 3:   # every byte pattern is a 3-bit stream (eight codes in three bytes)
        packed = rng.integers(0, 256, size=(d_row, d_col // 8 * 3), dtype=np.uint8)
    else:
        packed = rng.integers(0, 256, size=(d_row, d_col // 2), dtype=np.uint8)
    ng = 1 if G == 0 else d_col // G
    scales = (rng.random((d_row, ng)) * 0.05 + 0.001).astype(np.float16)
    zeros = rng.integers(0, 2 ** bits, size=(d_row, ng)).astype(np.float16)
    if frac_zeros:
        # zeros that are not integers, and a few far outside the code range, so that
        # u - z is not exact in a 16-bit type
        zeros = (rng.random((d_row, ng)) * (2 ** bits)).astype(np.float16)
        far = rng.random((d_row, ng)) < 0.05
        zeros[far] = np.float16(300.0)
    x = rng.standard_normal((n, d_col)).astype(np.float32)
    return packed, scales, zeros, x


def gpu_linear(packed, scales, zeros, x, bits, G, x_dtype, y_dtype, ldx_pad=0, repeat=2):
    import post_weight_quantization_25_amd as g
    d_row = packed.shape[0]
    d_col = x.shape[1]
    q = g.Quantized(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(),
                    torch.zeros(1, dtype=torch.int32, device="cuda"), bits, G, d_col)
    xt = torch.from_numpy(x).cuda().to(x_dtype)
    if ldx_pad:
        buf = torch.zeros((x.shape[0], d_col + ldx_pad), dtype=x_dtype, device="cuda")
        buf[:, :d_col] = xt
        xt = buf[:, :d_col]
    ys = [g.linear(q, xt, out_dtype=y_dtype) for _ in range(repeat)]
    torch.cuda.synchronize()
    y = ys[0]
    for other in ys[1:]:   # the same sums in the same order on every call
        assert torch.equal(other, y)
    x_used = xt.float().cpu().numpy().astype(np.float64)   # the activations as the kernel read them
    return y.float().cpu().numpy().astype(np.float64), x_used


CASES = [
    # d_row, d_col, bits, G, n, x dtype, y dtype, ldx pad
    (4096, 4096, 4, 128, 1, torch.bfloat16, torch.float32, 0),     # the decode shape of the metric layer
    (4096, 4096, 4, 128, 4, torch.bfloat16, torch.bfloat16, 0),
    (300, 512, 4, 128, 3, torch.bfloat16, torch.float32, 0),       # ragged rows, a partial token pass
    (333, 1024, 4, 64, 9, torch.float16, torch.float32, 0),        # three passes, the last partial
    (64, 256, 3, 32, 2, torch.float32, torch.float32, 0),
    (128, 256, 8, 64, 7, torch.float16, torch.bfloat16, 0),        # one code per byte
    (100, 250, 4, 0, 5, torch.bfloat16, torch.float32, 0),         # width not a multiple of 32: general kernel
    (96, 512, 4, 128, 2, torch.bfloat16, torch.float16, 3),        # x rows not 16-byte aligned: general kernel
    (17, 64, 4, 0, 1, torch.bfloat16, torch.float32, 0),           # per-row group, tiny
    # batched kernel (packed codes, 16-bit x, two or more tokens, 128-column chunks)
    (4096, 4096, 4, 128, 16, torch.bfloat16, torch.bfloat16, 0),   # one full token tile, metric layer shape
    (512, 1024, 4, 128, 5, torch.bfloat16, torch.float32, 0),      # a partial token tile
    (272, 512, 4, 256, 20, torch.float16, torch.float32, 0),       # two token tiles, 17 row tiles, two chunks a group
    (200, 384, 3, 128, 70, torch.bfloat16, torch.float32, 0),      # two tile rows of 64 tokens, ragged rows, 3 chunks
    (160, 2048, 4, 0, 2, torch.float16, torch.float16, 0),         # per-row group over 16 chunks
    (64, 1280, 4, 128, 33, torch.bfloat16, torch.float32, 8),      # padded x rows (16-byte aligned)
    (48, 512, 4, 128, 30, torch.bfloat16, torch.float32, 0),       # 32-row workgroups, the second half past the end
    (4096, 4096, 4, 128, 64, torch.bfloat16, torch.bfloat16, 0),   # 64 tokens of the metric layer shape
    (4096, 4096, 4, 128, 256, torch.bfloat16, torch.bfloat16, 0),  # 64-row workgroups (64 x 4 of them)
    (4000, 256, 4, 128, 257, torch.bfloat16, torch.float32, 0),     # 64-row workgroups, ragged rows and tokens
    (2050, 384, 3, 128, 500, torch.float16, torch.float32, 0),      # 64-row workgroups on the 3-bit stream
    # the 3-bit stream (12 bytes per 32 columns): decode, general and batched kernels
    (4096, 4096, 3, 128, 1, torch.bfloat16, torch.float32, 0),
    (300, 512, 3, 0, 3, torch.float16, torch.float32, 0),
    (100, 200, 3, 0, 5, torch.bfloat16, torch.float32, 0),          # width not a multiple of 32: general kernel
    (96, 512, 3, 128, 2, torch.bfloat16, torch.float16, 3),         # x rows not 16-byte aligned: general kernel
    (4096, 4096, 3, 128, 16, torch.bfloat16, torch.bfloat16, 0),    # batched, one full token tile
    (272, 1024, 3, 256, 40, torch.float16, torch.float32, 0),       # batched, three token tiles
]


@pytest.mark.parametrize("d_row,d_col,bits,G,n,xt,yt,pad", CASES)
def test_linear_parity(d_row, d_col, bits, G, n, xt, yt, pad):
    log(f"linear parity {d_row}x{d_col} bits={bits} G={G} n={n} x={xt} y={yt} pad={pad}")
    packed, scales, zeros, x = make_case(d_row, d_col, bits, G, n, 11)
    y, xu = gpu_linear(packed, scales, zeros, x, bits, G, xt, yt, pad)
    codes = o.unpack(packed, bits)
    ref = o.linear(xu, codes, scales, zeros, G)
    What = o.dequantize(codes, scales, zeros, G).astype(np.float64)
    mag = np.abs(xu) @ np.abs(What).T
    bound = ((d_col + 64) * 2.0 ** -23 + 2.0 ** -18) * mag
    if yt == torch.bfloat16:
        bound = bound + 2.0 ** -8 * np.abs(ref) + 1e-30
    elif yt == torch.float16:
        bound = bound + 2.0 ** -11 * np.abs(ref) + 6e-8
    err = np.abs(y - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    log(f"  max |err| / bound = {worst:.3f}")
    assert y.shape == ref.shape
    assert np.all(err <= bound)


@pytest.mark.parametrize("xt", [torch.bfloat16, torch.float16])
def test_linear_batched_inexact_zeros(xt):
    """Zeros that are not small integers take the batched kernel's second product."""
    log(f"linear batched, fractional zeros, x={xt}")
    packed, scales, zeros, x = make_case(256, 1024, 4, 128, 12, 5, frac_zeros=True)
    y, xu = gpu_linear(packed, scales, zeros, x, 4, 128, xt, torch.float32)
    codes = o.unpack(packed, 4)
    ref = o.linear(xu, codes, scales, zeros, 128)
    What = o.dequantize(codes, scales, zeros, 128).astype(np.float64)
    mag = np.abs(xu) @ np.abs(What).T
    bound = ((1024 + 64) * 2.0 ** -23 + 2.0 ** -18) * mag
    err = np.abs(y - ref)
    log(f"  max |err| / bound = {float(np.max(err / np.maximum(bound, 1e-300))):.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("xt", [torch.bfloat16, torch.float16])
def test_linear_batched_inexact_zeros_coherent(xt):
    """Every code 5, every zero 0.3, activations >= 0: u - z = 4.7 is not a 16-bit value
    (bf16 rounds it to 4.6875, f16 to 4.69921875), and the rounding errors all have one
    sign, so a product of the rounded value alone misses by 2.6e-3 (bf16) or 1.6e-4
    (f16) of |y|, above the bound of ((d_col + 64) 2^-23 + 2^-18) |y| = 1.3e-4 |y|."""
    log(f"linear batched, coherent fractional zeros, x={xt}")
    d_row, d_col, n = 64, 1024, 4
    packed = np.full((d_row, d_col // 2), 0x55, dtype=np.uint8)
    scales = np.full((d_row, d_col // 128), 0.01, dtype=np.float16)
    zeros = np.full((d_row, d_col // 128), 0.3, dtype=np.float16)
    x = np.abs(np.random.default_rng(9).standard_normal((n, d_col))).astype(np.float32)
    y, xu = gpu_linear(packed, scales, zeros, x, 4, 128, xt, torch.float32)
    ref = o.linear(xu, o.unpack(packed, 4), scales, zeros, 128)
    bound = ((d_col + 64) * 2.0 ** -23 + 2.0 ** -18) * np.abs(ref)
    err = np.abs(y - ref)
    log(f"  max |err| / bound = {float(np.max(err / bound)):.3f}")
    assert np.all(err <= bound)


def test_linear_no_tokens_is_a_no_op():
    import post_weight_quantization_25_amd as g
    packed, scales, zeros, _ = make_case(32, 64, 4, 32, 1, 3)
    q = g.Quantized(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(),
                    torch.zeros(1, dtype=torch.int32, device="cuda"), 4, 32, 64)
    y = g.linear(q, torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert tuple(y.shape) == (0, 32)


WIDE = [
    # the wide workloads' shapes: fc1, fc2, the MLP up (int4) and down (int3) layers
    (49152, 12288, 4, 128, 1, torch.bfloat16),
    (49152, 12288, 4, 128, 64, torch.float32),
    (12288, 49152, 4, 128, 1, torch.float32),
    (12288, 49152, 4, 128, 16, torch.bfloat16),
    (11008, 4096, 4, 128, 300, torch.float32),
    (4096, 11008, 3, 128, 1, torch.float32),
    (4096, 11008, 3, 128, 40, torch.bfloat16),
]


@pytest.mark.parametrize("d_row,d_col,bits,G,n,yt", WIDE)
def test_linear_wide_sampled(d_row, d_col, bits, G, n, yt):
    """Full-size layers of the wide workloads, bf16 x: every output of 256 sampled rows
    (the first, the last, random) against the oracle, to the bound above."""
    log(f"linear wide {d_row}x{d_col} bits={bits} G={G} n={n} y={yt}")
    packed, scales, zeros, x = make_case(d_row, d_col, bits, G, n, 23)
    y, xu = gpu_linear(packed, scales, zeros, x, bits, G, torch.bfloat16, yt, repeat=1)
    rng = np.random.default_rng([d_row, d_col, n])
    rows = np.array(sorted({0, 1, d_row - 1} | set(rng.choice(d_row, 253, replace=False).tolist())))
    codes = o.unpack(packed[rows], bits)
    ref = o.linear(xu, codes, scales[rows], zeros[rows], G)
    What = o.dequantize(codes, scales[rows], zeros[rows], G).astype(np.float64)
    mag = np.abs(xu) @ np.abs(What).T
    bound = ((d_col + 64) * 2.0 ** -23 + 2.0 ** -18) * mag
    if yt == torch.bfloat16:
        bound = bound + 2.0 ** -8 * np.abs(ref) + 1e-30
    err = np.abs(y[:, rows] - ref)
    log(f"  {rows.size} sampled rows: max |err| / bound = {float(np.max(err / np.maximum(bound, 1e-300))):.3f}")
    assert y.shape == (n, d_row)
    assert np.all(err <= bound)
