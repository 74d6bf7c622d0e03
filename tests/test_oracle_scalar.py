"""Pins of the oracle's scalar quantizers and storage format against the values
the pages print (fixtures under tests/golden/, each naming its source)."""
import json
import os

import numpy as np

from oracle import gptq_oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_affine_worked_example():
    g = _load("affine_int8_example.json")
    S, Z = o.affine_params(g["vmin"], g["vmax"], g["qmin"], g["qmax"])
    assert abs(S - g["S_approx"]) < 5e-5
    assert Z == g["Z"]
    q = int(o.affine_quantize(g["x"], S, Z, g["qmin"], g["qmax"]))
    assert q == g["q"]
    xhat = float(o.affine_dequantize(q, S, Z))
    assert abs(xhat - g["xhat_approx"]) < 5e-4
    assert abs((g["x"] - xhat) - g["error_approx"]) < 5e-4
    assert int(o.affine_quantize(g["vmin"], S, Z, g["qmin"], g["qmax"])) == g["q_at_vmin"]
    assert int(o.affine_quantize(0.0, S, Z, g["qmin"], g["qmax"])) == g["q_at_zero"]
    assert int(o.affine_quantize(g["vmax"], S, Z, g["qmin"], g["qmax"])) == g["q_at_vmax"]


def test_affine_example_through_group_params_unsigned_grid():
    """The layer quantizer works on the unsigned grid [0, 255] with an fp16 scale; the
    page's signed example must come out shifted by 128 with the same dequantized value."""
    g = _load("affine_int8_example.json")
    p = o.Params(bits=8, group_size=0, sym=False)
    vals = np.array([[g["vmin"], g["x"], 0.0, g["vmax"]]])
    S, S16, Z, _ = o.group_params(vals, p)
    assert abs(S[0] - (g["vmax"] - g["vmin"]) / 255) < 1e-15
    assert Z[0] == g["Z"] + 128
    q = o.decide_codes(vals[0], S16, np.repeat(Z, 4), p)
    assert list(q) == [0, g["q"] + 128, g["Z"] + 128, 255]
    xhat = S16[0] * (q[1] - Z[0])
    assert abs(xhat - g["xhat_approx"]) < 1e-3


def test_absmax_worked_example():
    g = _load("absmax_int8_example.json")
    x = np.array(g["x"])
    assert abs(g["qmax"] / g["absmax"] - g["multiplier_approx"]) < 0.05
    q = o.symmetric_quantize(x, g["absmax"], g["qmax"])
    assert list(q) == g["q"]
    # same result through the layer quantizer's symmetric group rule (fp16 scale)
    p = o.Params(bits=8, group_size=0, sym=True)
    S, S16, Z, _ = o.group_params(x[None, :], p)
    assert abs(S[0] - g["absmax"] / g["qmax"]) < 1e-15
    q2 = o.decide_codes(x, np.repeat(S16, x.size), np.repeat(Z, x.size), p)
    assert list(q2) == g["q"]


def test_absmax_example_rejects_full_signed_range():
    """Reading check: the alternative grid [-128, 127] with S = 2a/255 does not print
    the page's values (it maps -2.9 to -60), so the restricted range is the one used."""
    g = _load("absmax_int8_example.json")
    x = np.array(g["x"])
    S = 2 * g["absmax"] / 255
    q = np.clip(np.rint(x / S), -128, 127).astype(int)
    assert list(q) != g["q"]
    assert q[4] == -60


def test_packing_diagram():
    g = _load("int4_packing_example.json")
    b = o.pack(np.array([[g["val1"], g["val2"]]]), 4)
    assert b.shape == (1, 1) and int(b[0, 0]) == g["byte"]
    assert list(o.unpack(b, 4)[0]) == [g["val1"], g["val2"]]


def test_pack_unpack_all_bytes():
    allb = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(o.pack(o.unpack(allb, 4), 4), allb)
    rng = np.random.default_rng(0)
    u = rng.integers(0, 16, size=(7, 64)).astype(np.uint8)
    assert np.array_equal(o.unpack(o.pack(u, 4), 4), u)
    assert o.pack(u, 4).nbytes == u.size // 2      # 0.5 byte per 4-bit weight
    u8 = rng.integers(0, 256, size=(3, 10)).astype(np.uint8)
    assert np.array_equal(o.unpack(o.pack(u8, 8), 8), u8)


def test_dequantize_matches_definition():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, size=(5, 256)).astype(np.uint8)
    s16 = rng.uniform(1e-3, 1e-1, size=(5, 2)).astype(np.float16)
    z = rng.integers(-3, 18, size=(5, 2))
    out = o.dequantize(codes, s16, z, 128)
    for r in range(5):
        for c in range(256):
            k = c // 128
            assert out[r, c] == np.float32(float(s16[r, k]) * (int(codes[r, c]) - int(z[r, k])))


def test_group_params_degenerate_groups():
    p = o.Params(bits=4, group_size=0, sym=False)
    vals = np.array([[0.5, 0.5, 0.5], [0.0, 0.0, 0.0], [-0.25, -0.25, -0.25]])
    S, S16, Z, _ = o.group_params(vals, p)
    for r in range(3):
        q = o.decide_codes(vals[r], np.repeat(S16[r], 3), np.repeat(Z[r], 3), p)
        # the constant lands on an end of the grid: exact up to the fp16 rounding of S
        assert np.all(np.abs(S16[r] * (q - Z[r]) - vals[r]) <= 2.0 ** -11 * np.abs(vals[r]))
    assert S16[1] == 1.0 and Z[1] == 0


def test_group_params_symmetric_int3():
    p = o.Params(bits=3, group_size=0, sym=True)
    assert (p.qmin, p.qmax, p.zero_offset) == (-3, 3, 4)
    vals = np.array([[0.3, -0.9, 0.6, 0.1]])
    S, S16, Z, _ = o.group_params(vals, p)
    assert abs(S[0] - 0.3) < 1e-15 and Z[0] == 0
    q = o.decide_codes(vals[0], np.repeat(S16, 4), np.repeat(Z, 4), p)
    assert list(q) == [1, -3, 2, 0]


# Hand-computed decisions q = clamp(round(w / S16 + Z)) with round half to even, from the
# quotient and sum in exact arithmetic (Quantization concepts guide, "Mapping values to
# fewer bits": quantize formula).  S16 = 0.25 is exact in fp16, so every expected value
# below is worked out by hand.  Near-midpoint cases sit 2^-30 off a tie: closer than half
# a float32 step of w (2^-26 at 0.375), so a float32 quotient would land on the tie itself.
NEAR_MIDPOINTS = [
    # w,                  Z, code value w/S16 + Z,      q
    (0.375,               0, 1.5,                      2),    # exact tie -> even
    (0.625,               0, 2.5,                      2),    # exact tie -> even
    (0.375,               3, 4.5,                      4),    # the tie is decided after adding Z (not rne(1.5) + 3 = 5)
    (0.375 - 2.0 ** -30,  0, 1.5 - 2.0 ** -28,         1),    # just below the tie
    (0.375 + 2.0 ** -30,  0, 1.5 + 2.0 ** -28,         2),    # just above the tie
    (0.625 + 2.0 ** -30,  0, 2.5 + 2.0 ** -28,         3),    # just above an even-down tie
    (-0.125,              5, 4.5,                      4),
    (-0.125 - 2.0 ** -30, 5, 4.5 - 2.0 ** -28,         4),
    (-0.125 + 2.0 ** -30, 5, 4.5 + 2.0 ** -28,         5),
    (4.0,                 3, 19.0,                     15),   # clamped to qmax
    (-2.0,                2, -6.0,                     0),    # clamped to qmin
]


def test_code_value_and_decide_codes_near_midpoints():
    p = o.Params(bits=4, group_size=0, sym=False)
    w = np.array([c[0] for c in NEAR_MIDPOINTS])
    Z = np.array([c[1] for c in NEAR_MIDPOINTS], dtype=np.int64)
    S16 = np.full(w.size, 0.25)
    t = o.code_value(w, S16, Z)
    assert np.array_equal(t, np.array([c[2] for c in NEAR_MIDPOINTS]))
    assert list(o.decide_codes(w, S16, Z, p)) == [c[3] for c in NEAR_MIDPOINTS]
    # the reading is the exact quotient: a float32 quotient would put the case just
    # below the tie on the tie itself (and round it up to 2)
    assert np.float32(NEAR_MIDPOINTS[3][0]) / np.float32(0.25) == np.float32(1.5)


def test_decide_codes_symmetric_near_midpoints():
    """Symmetric grid (Z = 0, codes in +-3 for int3): -1.5 and 2.5 are ties (-> -2, 2);
    2^-30 off them the exact quotient decides."""
    p = o.Params(bits=3, group_size=0, sym=True)
    w = np.array([-0.375, -0.375 + 2.0 ** -30, 0.625, 0.625 - 2.0 ** -30, 1.0])
    q = o.decide_codes(w, np.full(5, 0.25), np.zeros(5, dtype=np.int64), p)
    assert list(q) == [-2, -1, 2, 2, 3]


def test_zero_point_decided_from_the_exact_quotient():
    """Z = qmin - round(min / S16): for a group with range 3.75 at int4 (S = S16 = 0.25)
    and min = -0.625 - 2^-30, min / S16 = -2.5 - 2^-28 rounds to -3, so Z = 3 (a float32
    quotient, -2.5, would round to -2 and give Z = 2)."""
    p = o.Params(bits=4, group_size=0, sym=False)
    mn = -0.625 - 2.0 ** -30
    vals = np.array([[mn, 0.1, mn + 3.75]])
    S, S16, Z, zt = o.group_params(vals, p)
    assert S[0] == 0.25 and S16[0] == 0.25
    assert zt[0] == -2.5 - 2.0 ** -28
    assert Z[0] == 3
    # exactly on the tie, -2.5 goes to the even -2: Z = 2
    S, S16, Z, zt = o.group_params(np.array([[-0.625, 0.0, 3.125]]), p)
    assert zt[0] == -2.5 and Z[0] == 2


def test_int3_bitstream_hand_example():
    g = _load("int3_bitstream_example.json")
    b = o.pack(np.array([g["codes"]]), 3)
    assert b.shape == (1, 3) and list(b[0]) == g["bytes"]
    assert list(o.unpack(b, 3)[0]) == g["codes"]


def test_int3_bitstream_every_position_and_value():
    """Every residue of the eight-codes-in-three-bytes cycle: code value v alone at
    position p of an 8-code group lands in bits 3p .. 3p + 2 of the group's three bytes
    read as one little-endian integer, and the stream round-trips."""
    for p in range(8):
        for v in range(8):
            codes = np.zeros((1, 16), dtype=np.uint8)
            codes[0, 8 + p] = v                     # the second group of the row
            b = o.pack(codes, 3)
            assert b.shape == (1, 6) and not b[0, :3].any()
            assert int.from_bytes(bytes(b[0, 3:]), "little") == v << (3 * p)
            assert np.array_equal(o.unpack(b, 3), codes)
    rng = np.random.default_rng(4)
    u = rng.integers(0, 8, size=(5, 64)).astype(np.uint8)
    assert np.array_equal(o.unpack(o.pack(u, 3), 3), u)
    assert o.pack(u, 3).nbytes == u.size * 3 // 8     # 0.375 byte per 3-bit weight
    # every 3-byte pattern is a valid stream of eight codes
    allb = rng.integers(0, 256, size=(7, 3)).astype(np.uint8)
    assert np.array_equal(o.pack(o.unpack(allb, 3), 3), allb)
