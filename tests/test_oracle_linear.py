"""Pins of the oracle's quantized linear (y = x What^T on the stored format) against
values fixed by hand arithmetic on the pages' printed examples and by special cases
that reduce it to the separately pinned dequantization."""
import json
import os

import numpy as np

from oracle import gptq_oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_example():
    g = json.load(open(os.path.join(GOLD, "linear_hand_example.json")))
    codes = o.unpack(np.array([[g["byte"]]], dtype=np.uint8), 4)
    assert codes.tolist() == [[5, 3]]
    y = o.linear(np.array([g["x"]]), codes, np.array([[g["scale"]]], np.float16), np.array([[g["zero"]]], np.float16), 0)
    assert y.shape == (1, 1) and y[0, 0] == g["y"]


def test_groups_use_their_own_scale_and_zero():
    # row 0: codes [1, 2 | 3, 4], group 2: scales [0.25, 2], zeros [1, 4]
    # What = [0.25*(1-1), 0.25*(2-1), 2*(3-4), 2*(4-4)] = [0, 0.25, -2, 0]; x = [1, 2, 3, 4]
    codes = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    y = o.linear(np.array([[1.0, 2.0, 3.0, 4.0]]), codes, np.array([[0.25, 2.0]], np.float16),
                 np.array([[1.0, 4.0]], np.float16), 2)
    assert y[0, 0] == 0.5 - 6.0


def test_unit_vectors_give_the_dequantized_rows():
    rng = np.random.default_rng(7)
    d_row, d_col, G = 5, 64, 32
    codes = rng.integers(0, 16, size=(d_row, d_col)).astype(np.uint8)
    sc = (rng.random((d_row, d_col // G)) * 0.1 + 0.01).astype(np.float16)
    zr = rng.integers(0, 16, size=(d_row, d_col // G)).astype(np.float16)
    y = o.linear(np.eye(d_col), codes, sc, zr, G)
    np.testing.assert_array_equal(y, o.dequantize(codes, sc, zr, G).astype(np.float64).T)


def test_zero_codes_at_the_zero_point_give_zero():
    codes = np.full((3, 8), 7, dtype=np.uint8)
    y = o.linear(np.ones((2, 8)), codes, np.full((3, 1), 0.5, np.float16), np.full((3, 1), 7, np.float16), 0)
    assert np.all(y == 0)
