"""MXFP4 quantization: e2m1 element codes with one UE8M0 scale per 32 elements, in fp64.

Test infrastructure (see the package docstring).

Source: UltraQuant article (oracore.dev), section on how the method works: the
cache holds FP4 KV tensors with UE8M0 group scales (power-of-two scales stored
as a biased 8-bit exponent), the queries are FP8, and the rotation before it is
a Walsh-Hadamard transform.  The pages give no conversion rule, so the oracle
follows the plain microscaling reading:

    a = max_j |y_j| over a group of 32 consecutive channels
    E = clamp(floor(log2 a) - 2 + 127, 0, 254)          (E = 0 when a == 0)
    r_j = y_j / 2^(E - 127)                              (exact: power of two)
    |r_j| rounds to the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6} (index 0..7),
          ties to the even index, saturating at 6
    code_j = 8 * [y_j < 0] + index

The "- 2" is the largest exponent of e2m1 (6 = 1.5 * 2^2), so a / 2^(E-127)
lands in [4, 8).  A negative value whose magnitude rounds to zero keeps its
sign (code 8) as an IEEE conversion does; exact zeros give code 0.
"""

import numpy as np

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
GROUP = 32


def _nearest_grid_index(mag: np.ndarray) -> np.ndarray:
    """Index of the nearest e2m1 magnitude, ties to the even index (saturating)."""
    dist = np.abs(mag[..., None] - E2M1_GRID)          # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    hit = dist == best                                  # one or two candidates
    even = hit & (np.arange(8) % 2 == 0)
    use_even = even.any(axis=-1, keepdims=True) & (hit.sum(axis=-1, keepdims=True) > 1)
    choose = np.where(use_even, even, hit)
    return np.argmax(choose, axis=-1).astype(np.uint8)


def group_exponent(amax: np.ndarray) -> np.ndarray:
    """Biased UE8M0 exponent for a group whose largest magnitude is ``amax``."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                # amax = m * 2^ex, m in [0.5, 1)
    floor_log2 = ex.astype(np.int64) - 1
    e = np.clip(floor_log2 - 2 + 127, 0, 254)
    return np.where(amax > 0, e, 0).astype(np.uint8)


def quantize_mxfp4(y: np.ndarray):
    """Quantize rotated vectors y[..., D] (D a multiple of 32).

    Returns (codes uint8[..., D] in 0..15, E uint8[..., D/32],
    r float64[..., D]) where ``r`` is the scaled value y / 2^(E-127) used by the
    parity rule to recognise rounding ties.
    """
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    if d % GROUP:
        raise ValueError("MXFP4 needs a multiple of 32 channels")
    g = y.reshape(y.shape[:-1] + (d // GROUP, GROUP))
    amax = np.abs(g).max(axis=-1)
    e = group_exponent(amax)
    scale = np.ldexp(1.0, e.astype(np.int64) - 127)[..., None]
    r = g / scale
    idx = _nearest_grid_index(np.abs(r))
    sign = (g < 0).astype(np.uint8)
    codes = (sign * 8 + idx).astype(np.uint8)
    return codes.reshape(y.shape), e, r.reshape(y.shape)


def dequantize_mxfp4(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """value = (-1)^sign * grid[index] * 2^(E - 127), exact in fp64."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    c = codes.reshape(codes.shape[:-1] + (d // GROUP, GROUP))
    mag = E2M1_GRID[c & 7]
    val = np.where(c >= 8, -mag, mag)
    scale = np.ldexp(1.0, np.asarray(e).astype(np.int64) - 127)[..., None]
    return (val * scale).reshape(codes.shape)
