"""Decode attention over the paged 4-bit cache, in fp64.

Test infrastructure (see the package docstring).

Read path: the SAW-INT4 summary requires the quantized cache to serve fused
attention over paged layouts ("Summary"); the UltraQuant article (section on
how the method works) attends with the queries against the 4-bit KV tensors
and their group scales.  Keys were stored rotated, k' = R k, so the query is
rotated by the same orthogonal transform: (R q) . (R k) = q . k (an orthogonal
map preserves inner products -- the "orthogonal feature decorrelation" of the
IsoQuant abstract).  The values come out in the rotated basis and are rotated
back at the end: o = R (sum_t p_t v'_t), R being its own inverse.

For each sequence b and query head h (kv head g = h // (Hq / Hkv)):

    q'  = R (q_scale * q[b, h])
    s_t = sm_scale * (q' . k^'_t),  t < seq_lens[b]     (no mask: decode sees all)
    p   = softmax(s)                                     (max-subtracted, fp64)
    o   = R (sum_t p_t v^'_t)

k^', v^' are the dequantized cached vectors (rotated basis), read through the
block table: position t lives on page block_table[b][t // 16], slot t % 16.

Chunked prefill over the same cache (``prefill_attention``): the UltraQuant
article (section on what it showed) credits its gains to prefixes that stay
resident in the 4-bit cache, so that a new turn does not re-run the prefill of
the prefix; the new turn's tokens then attend over the resident prefix and,
causally, over each other.  Reading: the chunk of sequence b is its last
n_b = cu_q[b+1] - cu_q[b] positions, already appended to the cache; query token
j of the chunk sits at position p_j = seq_lens[b] - n_b + j and attends
positions 0..p_j -- exactly the decode formula above with seq_len p_j + 1.
"""

import numpy as np

from .hadamard import rotation_matrix
from .layout import PAGE_SIZE, HEAD_DIM
from .paged import dequant_block, FMT_INT4


def gather_sequence(pool, block_table_row, seq_len: int, had_block: int, fmt: int):
    """Dequantized (k', v') fp64[Hkv][L][128] of one sequence, rotated basis."""
    hkv = pool.shape[1]
    n_pages = -(-seq_len // PAGE_SIZE)
    ks = np.empty((hkv, n_pages * PAGE_SIZE, HEAD_DIM))
    vs = np.empty_like(ks)
    # whole pages are dequantized, then cut to seq_len: the slots past the sequence end hold
    # whatever the pool held (possibly inf / NaN parameters), and are never attended
    with np.errstate(invalid="ignore", over="ignore"):
        for j in range(n_pages):
            page = int(block_table_row[j])
            for g in range(hkv):
                ks[g, j * PAGE_SIZE:(j + 1) * PAGE_SIZE] = dequant_block(pool[page, g], "k", fmt)
                vs[g, j * PAGE_SIZE:(j + 1) * PAGE_SIZE] = dequant_block(pool[page, g], "v", fmt)
    return ks[:, :seq_len], vs[:, :seq_len]


def decode_attention_one(q_heads, k_rot, v_rot, had_block: int, q_scale: float = 1.0,
                         sm_scale: float = None, out_rotated: bool = False):
    """Attention of q_heads[Hq][128] over one sequence's k_rot, v_rot [Hkv][L][128]."""
    hq = q_heads.shape[0]
    hkv = k_rot.shape[0]
    group = hq // hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(HEAD_DIM)
    r = rotation_matrix(had_block, HEAD_DIM)
    out = np.empty((hq, HEAD_DIM))
    for h in range(hq):
        g = h // group
        qr = r @ (np.float64(q_scale) * np.asarray(q_heads[h], dtype=np.float64))
        s = np.float64(sm_scale) * (k_rot[g] @ qr)
        p = np.exp(s - s.max())
        p /= p.sum()
        o_rot = p @ v_rot[g]
        out[h] = o_rot if out_rotated else r.T @ o_rot
    return out


def decode_attention(pool, q, seq_lens, block_table, had_block: int, fmt: int = FMT_INT4,
                     q_scale: float = 1.0, sm_scale: float = None, out_rotated: bool = False,
                     seqs=None):
    """o[B][Hq][128] (fp64) for the sequences in ``seqs`` (default: all; other rows NaN)."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, _ = q.shape
    out = np.full((bsz, hq, HEAD_DIM), np.nan)
    for b in (range(bsz) if seqs is None else seqs):
        k_rot, v_rot = gather_sequence(pool, block_table[b], int(seq_lens[b]), had_block, fmt)
        out[b] = decode_attention_one(q[b], k_rot, v_rot, had_block, q_scale, sm_scale,
                                      out_rotated)
    return out


def prefill_attention(pool, q, cu_q, seq_lens, block_table, had_block: int, fmt: int = FMT_INT4,
                      q_scale: float = 1.0, sm_scale: float = None, out_rotated: bool = False,
                      seqs=None):
    """o[T][Hq][128] (fp64) for the chunk tokens of the sequences in ``seqs`` (default: all;
    other rows NaN).  Token i of sequence b (cu_q[b] <= i < cu_q[b+1]) attends positions
    0 .. seq_lens[b] - (cu_q[b+1] - cu_q[b]) + (i - cu_q[b])."""
    q = np.asarray(q, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    out = np.full(q.shape, np.nan)
    for b in (range(len(seq_lens)) if seqs is None else seqs):
        length = int(seq_lens[b])
        n = int(cu_q[b + 1] - cu_q[b])
        if n == 0:
            continue
        k_rot, v_rot = gather_sequence(pool, block_table[b], length, had_block, fmt)
        for j in range(n):
            pos = length - n + j
            i = int(cu_q[b]) + j
            out[i] = decode_attention_one(q[i], k_rot[:, :pos + 1], v_rot[:, :pos + 1], had_block, q_scale,
                                          sm_scale, out_rotated)
    return out
