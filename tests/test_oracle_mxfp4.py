"""Pins for the oracle's MXFP4 (e2m1 + UE8M0/32) quantizer (CPU only)."""
import numpy as np
import pytest

from oracle import quantize_mxfp4, dequantize_mxfp4, E2M1_GRID
from oracle.mxfp4 import _nearest_grid_index, group_exponent
from tests.conftest import read_golden


def test_e2m1_rounding_golden():
    for tag, x, want in read_golden("mxfp4_rounding.txt"):
        if tag == "R":
            assert _nearest_grid_index(np.array([float(x)]))[0] == int(want), x
        else:
            assert group_exponent(np.array([float(x)]))[0] == int(want), x


def test_e2m1_rounding_matches_bruteforce_midpoints():
    # Every value strictly between two grid points rounds to the nearer one.
    rng = np.random.default_rng(21)
    r = rng.uniform(0, 8, 20000)
    idx = _nearest_grid_index(r)
    d = np.abs(r[:, None] - E2M1_GRID)
    assert np.all(np.abs(E2M1_GRID[idx] - r) == d.min(1))


def test_mxfp4_grid_roundtrip():
    # Inputs +-grid * 2^k with each group's amax in {4, 6} * 2^k come back exactly.
    rng = np.random.default_rng(22)
    for _ in range(300):
        k = rng.integers(-20, 20, 4)
        idx = rng.integers(0, 8, (4, 32))
        idx[:, 0] = rng.choice([6, 7], 4)
        idx = np.minimum(idx, np.where(idx[:, :1] == 6, 6, 7))
        sign = rng.integers(0, 2, (4, 32))
        sign[idx == 0] = 0
        y = (np.where(sign, -1, 1) * E2M1_GRID[idx] * 2.0 ** k[:, None]).reshape(128)
        codes, e, _ = quantize_mxfp4(y[None])
        assert np.array_equal(e[0].astype(np.int64), k + 127)
        assert np.array_equal(codes[0], (sign * 8 + idx).reshape(128))
        assert np.array_equal(dequantize_mxfp4(codes, e)[0], y)


def test_mxfp4_signed_zero_and_zero_group():
    y = np.zeros((1, 128))
    y[0, 40] = 6.0
    y[0, 41] = -0.1          # rounds to zero magnitude, keeps the sign
    codes, e, _ = quantize_mxfp4(y)
    assert e[0, 0] == 0 and e[0, 1] == 127
    assert not codes[0, :32].any()
    assert codes[0, 41] == 8 and codes[0, 40] == 7


def test_mxfp4_error_bound():
    # Per element |y - y^| <= 2 * scale: half the widest grid step (4 -> 6), or the
    # saturation of (6, 8) onto 6.
    rng = np.random.default_rng(23)
    y = rng.standard_normal((500, 128)) * 3
    codes, e, _ = quantize_mxfp4(y)
    yh = dequantize_mxfp4(codes, e)
    scale = np.repeat(2.0 ** (e.astype(np.int64) - 127), 32, axis=1)
    assert np.all(np.abs(y - yh) <= 2.0 * scale)
