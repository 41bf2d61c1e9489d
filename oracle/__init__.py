"""Plain fp64 CPU oracle for the rotated 4-bit paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use it.  It shares no code, table or constant generator with
the HIP library; the two meet only through the seeded input generators, which
hold none of the method's arithmetic.

What it computes, and the passages it follows:

* ``hadamard``  -- the block-diagonal Walsh-Hadamard rotation named by the
  SAW-INT4 summary (aissential.tech, "Summary" and "Method") and the
  UltraQuant article (oracore.dev, section on how the method works: a
  Walsh-Hadamard rotation that spreads outliers across channels before
  quantizing).
* ``int4``      -- token-wise asymmetric INT4 with an fp16 scale and zero
  (SAW-INT4 summary, "Summary", "Method", "In practice").
* ``mxfp4``     -- the FP4 (e2m1) variant with one UE8M0 power-of-two scale
  per group of 32 elements and FP8 queries (UltraQuant article, section on how
  the method works).
* ``layout``    -- the page-head byte layout of the paged cache ("paged
  KV-cache layouts", SAW-INT4 summary, "Summary").
* ``paged``     -- append into the page pool through a block table, and
  dequantization of pages.
* ``attention`` -- decode attention over the paged cache with the query rotated
  by the same orthogonal transform (inner products are preserved by an
  orthogonal rotation: IsoQuant abstract, "orthogonal feature decorrelation").
* ``quaternion`` -- the alternative rotation stage: IsoQuant's block-4
  rotation v -> q_L v conj(q_R) of every 4-channel block (IsoQuant abstract),
  accepted wherever a Hadamard block width is.

Every floating-point step runs in fp64 unless the method fixes the precision
(the fp16 scale/zero, the e2m1 grid, the UE8M0 scale).  Functions whose result
no independent pin checks say "parity unpinned" in their docstring; at present
there are none.
"""

from .hadamard import sylvester, rotation, rotation_matrix, rotate
from .quaternion import hamilton, conj, left_matrix, right_matrix, block_matrix, QuatRotation
from .int4 import quantize_int4, dequantize_int4
from .mxfp4 import quantize_mxfp4, dequantize_mxfp4, E2M1_GRID
from .layout import (PAGE_SIZE, HEAD_DIM, PAGE_HEAD_BYTES, K_CODES_OFF, V_CODES_OFF,
                     K_PARAMS_OFF, V_PARAMS_OFF, nibble_position, pack_row, unpack_row)
from .paged import (append, dequant_pages, read_token, FMT_INT4, FMT_MXFP4)
from .attention import decode_attention, decode_attention_one, prefill_attention

__all__ = [
    "prefill_attention", "rotation_matrix", "rotate", "hamilton", "conj", "left_matrix", "right_matrix",
    "block_matrix", "QuatRotation",
    "sylvester", "rotation", "quantize_int4", "dequantize_int4", "quantize_mxfp4",
    "dequantize_mxfp4", "E2M1_GRID", "PAGE_SIZE", "HEAD_DIM", "PAGE_HEAD_BYTES",
    "K_CODES_OFF", "V_CODES_OFF", "K_PARAMS_OFF", "V_PARAMS_OFF", "nibble_position",
    "pack_row", "unpack_row", "append", "dequant_pages", "read_token", "FMT_INT4",
    "FMT_MXFP4", "decode_attention", "decode_attention_one",
]
