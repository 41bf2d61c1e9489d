"""Byte layout of one page-head block of the paged 4-bit cache.

Test infrastructure (see the package docstring).

The SAW-INT4 summary ("Summary") requires the quantized cache to live in
*paged* KV-cache layouts with regular memory access; the pages give no byte
format, so this one is the library's own contract, restated here from its
definition (the oracle does not read the library's code or headers).

A page holds PAGE_SIZE = 16 token slots.  The pool is uint8[num_pages][Hkv][2176];
one page-head block (one page, one kv head) is 2176 bytes:

    [0,    1024)  K code rows    slot s, row byte j  at  64*s + j
    [1024, 2048)  V code rows    slot s, row byte j  at  1024 + 256*(s//4) + 4*j + (s%4)
    [2048, 2112)  K parameters   slot s at 2048 + 4*s
    [2112, 2176)  V parameters   slot s at 2112 + 4*s

A code row is 64 bytes = 128 four-bit codes.  Channel ch (0..127, in the
rotated basis) sits at nibble position p(ch) = 8*(ch % 16) + ch // 16 of the
row; nibble p is the low half of row byte p//2 when p is even, the high half
when p is odd.  Equivalently, row byte 4*a + q (a = 0..15, q = 0..3) holds
channel a + 32*q in its low nibble and channel a + 32*q + 16 in its high
nibble.  V rows use the same row bytes, interleaved by groups of four slots
so that the four slots of a group sit in one 32-bit word per row byte.

Parameters: INT4 stores fp16 scale then fp16 zero, little-endian; MXFP4 stores
the four UE8M0 bytes of channel groups [0,32), [32,64), [64,96), [96,128).
"""

import numpy as np

PAGE_SIZE = 16
HEAD_DIM = 128
ROW_BYTES = HEAD_DIM // 2
K_CODES_OFF = 0
V_CODES_OFF = 1024
K_PARAMS_OFF = 2048
V_PARAMS_OFF = 2112
PAGE_HEAD_BYTES = 2176


def nibble_position(ch):
    """Nibble index inside a 64-byte code row that holds channel ``ch``."""
    ch = np.asarray(ch)
    return 8 * (ch % 16) + ch // 16


def pack_row(codes: np.ndarray) -> np.ndarray:
    """codes uint8[..., 128] (each 0..15) -> row bytes uint8[..., 64]."""
    codes = np.asarray(codes, dtype=np.uint8)
    nib = np.zeros(codes.shape, dtype=np.uint8)
    nib[..., nibble_position(np.arange(HEAD_DIM))] = codes
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_row(row: np.ndarray) -> np.ndarray:
    """row bytes uint8[..., 64] -> codes uint8[..., 128] in channel order."""
    row = np.asarray(row, dtype=np.uint8)
    nib = np.empty(row.shape[:-1] + (HEAD_DIM,), dtype=np.uint8)
    nib[..., 0::2] = row & 0x0F
    nib[..., 1::2] = row >> 4
    return nib[..., nibble_position(np.arange(HEAD_DIM))]


def k_row_offsets(slot):
    """Byte offsets (within the page-head block) of the 64 bytes of K row ``slot``."""
    return K_CODES_OFF + 64 * np.asarray(slot)[..., None] + np.arange(ROW_BYTES)


def v_row_offsets(slot):
    """Byte offsets of the 64 bytes of V row ``slot`` (interleaved by slot quads)."""
    s = np.asarray(slot)[..., None]
    return V_CODES_OFF + 256 * (s // 4) + 4 * np.arange(ROW_BYTES) + (s % 4)


def param_offsets(slot, which: str):
    base = K_PARAMS_OFF if which == "k" else V_PARAMS_OFF
    return base + 4 * np.asarray(slot)[..., None] + np.arange(4)
