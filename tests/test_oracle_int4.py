"""Pins for the oracle's token-wise INT4 quantizer and its paged append (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle import quantize_int4, dequantize_int4, rotation, sylvester
from oracle.paged import encode, FMT_INT4, decode_params_int4
from tests.conftest import read_golden


def _golden_case(tag):
    rows = read_golden("int4_worked.txt")
    vals, deltas, codes = {}, {}, {}
    default = None
    params = None
    for r in rows:
        if r[0] == tag:
            ch = int(r[1])
            vals[ch] = float(r[2])
            if len(r) == 5:
                deltas[ch] = float(r[3])
            codes[ch] = int(r[-1])
        elif r[0] == tag + "_default":
            default = (float(r[1]), int(r[-1]))
        elif r[0] == tag + "_params":
            params = (int(r[1], 16), int(r[2], 16))
    y = np.full(128, default[0])
    want = np.full(128, default[1])
    for ch in vals:
        y[ch] = vals[ch]
        want[ch] = codes[ch]
    return y, want, deltas, params


@pytest.mark.parametrize("tag", ["A", "B", "C"])
def test_int4_golden_worked_example(tag):
    y, want, deltas, (s_bits, z_bits) = _golden_case(tag)
    codes, s16, z16, delta = quantize_int4(y[None])
    assert s16.view(np.uint16)[0] == s_bits
    assert z16.view(np.uint16)[0] == z_bits
    assert np.array_equal(codes[0], want)
    for ch, d in deltas.items():
        assert delta[0, ch] == d
    # The same vector through the byte encoder (no rotation) gives the same params.
    _, pbytes, _ = encode(y[None, None], 1, FMT_INT4)
    s2, z2 = decode_params_int4(pbytes[0, 0])
    assert s2.view(np.uint16) == s_bits and z2.view(np.uint16) == z_bits


def test_int4_grid_roundtrip_no_rotation():
    # Inputs on an exact grid s*c + z with a power-of-two s come back exactly.
    rng = np.random.default_rng(11)
    for _ in range(200):
        c = rng.integers(0, 16, 128)
        c[rng.integers(128)] = 0
        c[rng.integers(128)] = 15
        c[c.argmin()], c[c.argmax()] = 0, 15
        s = 2.0 ** rng.integers(-8, 3)
        z = -float(rng.integers(0, 40)) * s
        y = s * c + z
        codes, s16, z16, _ = quantize_int4(y[None])
        assert np.array_equal(codes[0], c)
        assert float(s16[0]) == s and float(z16[0]) == z
        assert np.array_equal(dequantize_int4(codes, s16, z16)[0], y)


def test_int4_grid_roundtrip_through_rotation_b64():
    # End to end with the b=64 rotation: choose codes, s, z; set y^ = s*c + z and
    # x = R_64 y^ = H_64 y^ / 8 (dyadic, exact in fp16).  Rotating x back gives y^
    # exactly, so the quantizer must return c, s, z unchanged.
    rng = np.random.default_rng(12)
    h = sylvester(64).astype(np.float64)
    for _ in range(100):
        c = rng.integers(0, 16, 128)
        c[0], c[1] = 0, 15
        s = 2.0 ** rng.integers(-6, 0)
        z = -float(rng.integers(0, 10)) * s
        yh = s * c + z
        x = np.concatenate([h @ yh[:64], h @ yh[64:]]) / 8.0
        assert np.array_equal(x.astype(np.float16).astype(np.float64), x)
        rows, params, info = encode(x[None, None], 64, FMT_INT4)
        assert np.array_equal(info["codes"][0, 0], c)
        assert float(info["s16"][0, 0]) == s and float(info["z16"][0, 0]) == z
        assert np.array_equal(oracle.unpack_row(rows[0, 0]), c)


def test_int4_error_bound_random():
    # |y - y^| <= s16/2 + |z16 - lo| + (fp16 rounding slack of s16 times 15).
    rng = np.random.default_rng(13)
    y = rng.standard_normal((2000, 128)) * rng.uniform(0.01, 30, (2000, 1))
    y[:, 3] *= 15
    codes, s16, z16, _ = quantize_int4(y)
    yh = dequantize_int4(codes, s16, z16)
    s = s16.astype(np.float64)
    lo = y.min(1)
    hi = y.max(1)
    slack = np.abs(s * 15 - (hi - lo)) + np.abs(z16.astype(np.float64) - lo)
    bound = s / 2 + slack + 1e-12
    assert np.all(np.abs(y - yh).max(1) <= bound)
    # Both end codes occur in every non-degenerate vector.
    assert np.all(codes.min(1) == 0) and np.all(codes.max(1) == 15)


def test_int4_degenerate_vectors():
    codes, s16, z16, _ = quantize_int4(np.full((1, 128), 3.25))
    assert float(s16[0]) == 0.0 and float(z16[0]) == 3.25 and not codes.any()
    with pytest.raises(ValueError):
        quantize_int4(np.array([[0.0] * 127 + [1e6]]))


def test_rotation_reduces_int4_error_on_outliers():
    # Direction only (the pages: rotation recovers what plain INT4 loses).
    rng = np.random.default_rng(14)
    x = rng.standard_normal((4000, 128))
    x[:, [7, 50, 99]] *= 15
    def mse(b):
        r = rotation(b)
        codes, s16, z16, _ = quantize_int4(x @ r.T)
        return np.mean((dequantize_int4(codes, s16, z16) @ r - x) ** 2)
    assert mse(128) < 0.5 * mse(1) and mse(64) < 0.5 * mse(1)
