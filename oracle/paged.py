"""Append into the paged pool through a block table, and dequantize pages, in fp64.

Test infrastructure (see the package docstring).

Write path (SAW-INT4 summary, "Summary" and "Method"): every new K and V token
vector is rotated with the block-diagonal Hadamard matrix, quantized token-wise
to 4 bits and written into a paged KV-cache layout.  The UltraQuant article
(section on how the method works) rotates the KV vectors, K and V alike, before
quantizing; the oracle therefore rotates V as well as K.

Addressing (the plain reading of a paged cache with a block table): token i of
sequence b, cu_new[b] <= i < cu_new[b+1], goes to position
p = start_pos[b] + (i - cu_new[b]), i.e. page block_table[b][p // 16], slot p % 16.
Only the bytes of the appended slots are written.
"""

import numpy as np

from .hadamard import rotation_matrix, rotate
from .int4 import quantize_int4, dequantize_int4
from .mxfp4 import quantize_mxfp4, dequantize_mxfp4
from .layout import (PAGE_SIZE, HEAD_DIM, K_PARAMS_OFF, V_PARAMS_OFF, pack_row,
                     unpack_row, k_row_offsets, v_row_offsets, param_offsets)

FMT_INT4 = 0
FMT_MXFP4 = 1


def encode(x: np.ndarray, had_block: int, fmt: int):
    """Rotate and quantize vectors x[..., 128] (exact input values, fp64).

    Returns (row_bytes uint8[..., 64], param_bytes uint8[..., 4], info) where
    ``info`` holds the intermediate values the parity rules need.
    """
    y = rotate(x, had_block, HEAD_DIM)
    if fmt == FMT_INT4:
        codes, s16, z16, delta = quantize_int4(y)
        params = np.concatenate(
            [s16.astype("<f2").view(np.uint8).reshape(s16.shape + (2,)),
             z16.astype("<f2").view(np.uint8).reshape(z16.shape + (2,))], axis=-1)
        info = {"y": y, "codes": codes, "s16": s16, "z16": z16, "delta": delta}
    elif fmt == FMT_MXFP4:
        if isinstance(had_block, (int, np.integer)) and had_block not in (1, 128):
            raise ValueError("MXFP4 uses the full 128-wide rotation (or none, for tests)")
        codes, e, rr = quantize_mxfp4(y)
        params = e.astype(np.uint8)
        info = {"y": y, "codes": codes, "e": e, "r": rr}
    else:
        raise ValueError(f"unknown format {fmt}")
    return pack_row(codes), params, info


def token_slots(cu_new, start_pos, block_table):
    """For every appended token i: (sequence, page id, slot)."""
    cu_new = np.asarray(cu_new, dtype=np.int64)
    start_pos = np.asarray(start_pos, dtype=np.int64)
    block_table = np.asarray(block_table, dtype=np.int64)
    seq = np.repeat(np.arange(len(start_pos)), np.diff(cu_new))
    pos = start_pos[seq] + (np.arange(cu_new[-1] - cu_new[0]) + cu_new[0] - cu_new[seq])
    page = block_table[seq, pos // PAGE_SIZE]
    return seq, page, pos % PAGE_SIZE


def append(pool, k, v, cu_new, start_pos, block_table, had_block: int, fmt: int = FMT_INT4):
    """Write tokens cu_new[0]..cu_new[B]-1 of k, v ([T][Hkv][128], exact values) into
    ``pool`` (uint8[num_pages][Hkv][2176], modified in place).  Returns the per-tensor
    ``info`` dicts of :func:`encode` for the appended tokens, shaped [T][Hkv][...].
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    t0, t1 = int(cu_new[0]), int(cu_new[-1])
    _, page, slot = token_slots(cu_new, start_pos, block_table)
    hkv = k.shape[1]
    infos = {}
    for name, x in (("k", k), ("v", v)):
        rows, params, info = encode(x[t0:t1], had_block, fmt)
        infos[name] = info
        row_off = k_row_offsets(slot) if name == "k" else v_row_offsets(slot)
        par_off = param_offsets(slot, name)
        for h in range(hkv):
            pool[page[:, None], h, row_off] = rows[:, h, :]
            pool[page[:, None], h, par_off] = params[:, h, :]
    return infos


def read_token(pool, page: int, head: int, slot: int, which: str):
    """(codes uint8[128], param bytes uint8[4]) of one stored token vector."""
    row_off = k_row_offsets(slot) if which == "k" else v_row_offsets(slot)
    codes = unpack_row(pool[page, head, row_off])
    params = pool[page, head, param_offsets(slot, which)]
    return codes, params


def decode_params_int4(param_bytes):
    """uint8[..., 4] -> (s16, z16) float16 arrays."""
    pb = np.ascontiguousarray(param_bytes, dtype=np.uint8)
    s16 = pb[..., 0:2].copy().view("<f2")[..., 0]
    z16 = pb[..., 2:4].copy().view("<f2")[..., 0]
    return s16, z16


def dequant_block(block: np.ndarray, which: str, fmt: int) -> np.ndarray:
    """One page-head block (uint8[2176]) -> values fp64[16][128] in the rotated basis."""
    slots = np.arange(PAGE_SIZE)
    row_off = k_row_offsets(slots) if which == "k" else v_row_offsets(slots)
    codes = unpack_row(block[row_off])
    pbytes = block[param_offsets(slots, which)]
    if fmt == FMT_INT4:
        s16, z16 = decode_params_int4(pbytes)
        return dequantize_int4(codes, s16, z16)
    return dequantize_mxfp4(codes, pbytes)


def dequant_pages(pool, page_ids, had_block: int, fmt: int = FMT_INT4, unrotate: bool = False):
    """Dequantize whole pages: returns (k, v) fp64[n][Hkv][16][128].

    In the rotated basis by default; with ``unrotate`` the rotation is undone
    (R is orthogonal, so x^ = R^T y^; R_b is also symmetric).
    """
    page_ids = np.asarray(page_ids, dtype=np.int64)
    hkv = pool.shape[1]
    out = {}
    r = rotation_matrix(had_block, HEAD_DIM)
    for which in ("k", "v"):
        vals = np.empty((len(page_ids), hkv, PAGE_SIZE, HEAD_DIM), dtype=np.float64)
        for n, p in enumerate(page_ids):
            for h in range(hkv):
                vals[n, h] = dequant_block(pool[p, h], which, fmt)
        if unrotate:
            vals = vals @ r  # rows: (R^T y)^T = y^T R
        out[which] = vals
    return out["k"], out["v"]
