"""Token-wise asymmetric INT4 quantization with an fp16 scale and zero, in fp64.

Test infrastructure (see the package docstring).

Source: SAW-INT4 summary (aissential.tech), "Summary" / "Method" / "In practice":
token-wise INT4 quantization of each K/V token vector after the block-diagonal
Hadamard rotation.  The tiny workload of the task fixes the parameters as an
fp16 scale and an fp16 zero per token vector.  The pages do not spell out the
quantizer, so the oracle takes the usual min/max asymmetric form:

    lo = min_j y_j,  hi = max_j y_j
    s16 = fp16_rne((hi - lo) / 15),   z16 = fp16_rne(lo)
    c_j = clamp(rne((y_j - z16) / s16), 0, 15)     (all c_j = 0 when s16 == 0)
    y^_j = s16 * c_j + z16

Readings taken where the pages are silent:
* one (scale, zero) pair per (token, kv head, K or V) over all 128 channels,
  whatever the Hadamard block width;
* the codes are chosen against the *stored* fp16 scale and zero, so
  dequantization sees exactly the grid the codes were chosen on; the clamp
  absorbs the fp16 rounding of lo and hi;
* ties round to even;
* vectors whose parameters would overflow fp16 are outside the contract.
"""

import numpy as np

FP16_MAX = 65504.0


def quantize_int4(y: np.ndarray):
    """Quantize rotated vectors y[..., D] (fp64).

    Returns (codes uint8[..., D], s16 float16[...], z16 float16[...],
    delta float64[..., D]) where ``delta`` is the pre-rounding value
    (y - z16) / s16 that the parity rule uses to recognise rounding boundaries
    (it is 0 where s16 == 0).
    """
    y = np.asarray(y, dtype=np.float64)
    lo = y.min(axis=-1)
    hi = y.max(axis=-1)
    span = (hi - lo) / 15.0
    if np.any(np.abs(lo) > FP16_MAX) or np.any(span > FP16_MAX):
        raise ValueError("INT4 parameters overflow fp16: input outside the contract")
    s16 = span.astype(np.float16)
    z16 = lo.astype(np.float16)
    s = s16.astype(np.float64)[..., None]
    z = z16.astype(np.float64)[..., None]
    safe = np.where(s > 0, s, 1.0)
    delta = np.where(s > 0, (y - z) / safe, 0.0)
    codes = np.clip(np.rint(delta), 0, 15).astype(np.uint8)
    return codes, s16, z16, delta


def dequantize_int4(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """y^ = s16 * c + z16, exact in fp64 (an fp16 times a 4-bit integer plus an fp16)."""
    s = np.asarray(s16).astype(np.float64)[..., None]
    z = np.asarray(z16).astype(np.float64)[..., None]
    return s * codes.astype(np.float64) + z
