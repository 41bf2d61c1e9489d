"""Pins for the oracle's decode attention (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import rotation, decode_attention, dequant_pages
from oracle.attention import decode_attention_one, gather_sequence
from oracle.paged import append, FMT_INT4, FMT_MXFP4


def _filled_cache(rng, lens, hkv, hb, fmt=FMT_INT4, permute=True):
    n_pages = [-(-n // 16) for n in lens]
    total = sum(n_pages) + 2
    ids = rng.permutation(total) if permute else np.arange(total)
    table = np.zeros((len(lens), max(n_pages)), np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = ids[off:off + n]
        off += n
    t = sum(lens)
    k = (rng.standard_normal((t, hkv, 128)) * 2).astype(np.float16).astype(np.float64)
    v = rng.standard_normal((t, hkv, 128)).astype(np.float16).astype(np.float64)
    pool = np.full((total, hkv, 2176), 0x3C, np.uint8)
    cu = np.concatenate([[0], np.cumsum(lens)])
    append(pool, k, v, cu, np.zeros(len(lens), np.int64), table, hb, fmt)
    return pool, table


@pytest.mark.parametrize("hb,fmt", [(64, FMT_INT4), (128, FMT_INT4), (1, FMT_INT4), (128, FMT_MXFP4)])
def test_attention_matches_torch_sdpa_fp64(hb, fmt):
    # Against a library routine on the unrotated dequantized cache.
    rng = np.random.default_rng(41)
    lens = [37, 16, 1]
    hkv, hq = 2, 8
    pool, table = _filled_cache(rng, lens, hkv, hb, fmt)
    q = rng.standard_normal((3, hq, 128))
    out = decode_attention(pool, q, lens, table, hb, fmt, q_scale=0.75, sm_scale=0.1)
    r = rotation(hb)
    for b, n in enumerate(lens):
        k_rot, v_rot = gather_sequence(pool, table[b], n, hb, fmt)
        k_un = torch.from_numpy(k_rot @ r.T)       # R is symmetric: R k'
        v_un = torch.from_numpy(v_rot @ r.T)
        qq = torch.from_numpy(0.75 * q[b]).reshape(hkv, hq // hkv, 128)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq[:, :, None, :], k_un[:, None].expand(hkv, hq // hkv, n, 128),
            v_un[:, None].expand(hkv, hq // hkv, n, 128), scale=0.1)
        assert np.allclose(out[b], ref.reshape(hq, 128).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(42)
    hb = 64
    pool, table = _filled_cache(rng, [1, 20], 1, hb)
    kd, vd = dequant_pages(pool, table[0, :1], hb, unrotate=True)
    # L = 1: output is the single unrotated dequantized value vector.
    q = rng.standard_normal((2, 4, 128))
    out = decode_attention(pool, q, [1, 20], table, hb)
    assert np.allclose(out[0], np.broadcast_to(vd[0, 0, 0], (4, 128)), atol=1e-13)
    # q = 0: uniform weights -> mean of the unrotated values.
    out0 = decode_attention(pool, np.zeros((2, 4, 128)), [1, 20], table, hb)
    k_rot, v_rot = gather_sequence(pool, table[1], 20, hb, FMT_INT4)
    assert np.allclose(out0[1], np.broadcast_to((v_rot[0] @ rotation(hb)).mean(0), (4, 128)), atol=1e-13)
    # GQA: query heads that share a kv head and a query give identical rows.
    qs = np.repeat(rng.standard_normal((2, 1, 128)), 4, axis=1)
    o = decode_attention(pool, qs, [1, 20], table, hb)
    assert np.array_equal(o[1, 0], o[1, 3])


def test_attention_identical_keys_uniform():
    k = np.broadcast_to(np.arange(128.0) / 64, (1, 9, 128)).copy()
    v = np.random.default_rng(43).standard_normal((1, 9, 128))
    o = decode_attention_one(np.ones((2, 128)), k, v, 1)
    assert np.allclose(o[0], v[0].mean(0), atol=1e-14)


def test_attention_page_permutation_invariance():
    rng = np.random.default_rng(44)
    pool, table = _filled_cache(rng, [50], 1, 128, permute=False)
    q = rng.standard_normal((1, 4, 128))
    base = decode_attention(pool, q, [50], table, 128)
    perm = rng.permutation(pool.shape[0])
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    out = decode_attention(pool2, q, [50], perm[table], 128)
    assert np.array_equal(base, out)


def test_rotated_output_flag():
    rng = np.random.default_rng(45)
    pool, table = _filled_cache(rng, [33], 1, 64)
    q = rng.standard_normal((1, 4, 128))
    a = decode_attention(pool, q, [33], table, 64)
    b = decode_attention(pool, q, [33], table, 64, out_rotated=True)
    assert np.allclose(a[0], b[0] @ rotation(64), atol=1e-13)


def test_attention_on_lossless_rotated_cache_equals_exact_attention():
    # Inputs x = R_64 y with y on an INT4 grid (dyadic, exact): the rotated cache is
    # lossless, so decode over it (rotate q, attend, rotate back) must equal exact
    # fp64 attention on the raw x -- this pins the rotation wiring of the read path.
    rng = np.random.default_rng(46)
    r = rotation(64)
    n = 24
    def grid_vectors():
        c = rng.integers(0, 16, (n, 128))
        c[:, 0], c[:, 1] = 0, 15
        return c * 0.25 - 2.0
    yk, yv = grid_vectors(), grid_vectors()
    xk, xv = yk @ r.T, yv @ r.T          # exact dyadic values
    q = rng.standard_normal((1, 4, 128))
    table = np.array([[0, 1]], np.int32)
    pool64 = np.zeros((2, 1, 2176), np.uint8)
    append(pool64, xk[:, None], xv[:, None], np.array([0, n]), np.array([0]), table, 64)
    o64 = decode_attention(pool64, q, [n], table, 64)
    s = (xk @ q[0].T) / np.sqrt(128)
    p = np.exp(s - s.max(0))
    p /= p.sum(0)
    assert np.allclose(o64[0], (p.T @ xv), atol=1e-12)


@pytest.mark.parametrize("hb,fmt", [(64, FMT_INT4), (128, FMT_MXFP4)])
def test_prefill_matches_torch_sdpa_causal_fp64(hb, fmt):
    # Chunked prefill against a library routine: SDPA with an explicit causal mask over the
    # unrotated dequantized cache; the chunk is the last n positions of each sequence.
    from oracle import prefill_attention
    rng = np.random.default_rng(43)
    lens = [40, 17, 5]
    chunk = [9, 17, 1]
    hkv, hq = 2, 4
    pool, table = _filled_cache(rng, lens, hkv, hb, fmt)
    cu_q = np.concatenate([[0], np.cumsum(chunk)])
    q = rng.standard_normal((int(cu_q[-1]), hq, 128))
    out = prefill_attention(pool, q, cu_q, lens, table, hb, fmt, q_scale=0.5, sm_scale=0.2)
    r = rotation(hb)
    for b, (length, n) in enumerate(zip(lens, chunk)):
        k_rot, v_rot = gather_sequence(pool, table[b], length, hb, fmt)
        k_un = torch.from_numpy(k_rot @ r.T)
        v_un = torch.from_numpy(v_rot @ r.T)
        qq = torch.from_numpy(0.5 * q[cu_q[b]:cu_q[b + 1]]).permute(1, 0, 2)      # [Hq][n][128]
        qq = qq.reshape(hkv, hq // hkv, n, 128)
        pos = np.arange(length - n, length)
        mask = torch.from_numpy(np.arange(length)[None, :] <= pos[:, None])        # [n][L]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, k_un[:, None].expand(hkv, hq // hkv, length, 128),
            v_un[:, None].expand(hkv, hq // hkv, length, 128), attn_mask=mask, scale=0.2)
        ref = ref.reshape(hq, n, 128).permute(1, 0, 2).numpy()
        assert np.allclose(out[cu_q[b]:cu_q[b + 1]], ref, rtol=1e-12, atol=1e-12)


def test_prefill_is_causal_and_reduces_to_decode():
    from oracle import prefill_attention
    rng = np.random.default_rng(44)
    hb, hkv, hq = 128, 1, 4
    lens = [50]
    pool, table = _filled_cache(rng, lens, hkv, hb, permute=False)
    n = 10
    q = rng.standard_normal((n, hq, 128))
    out = prefill_attention(pool, q, [0, n], lens, table, hb)
    # the last chunk token sees the whole sequence: the decode result
    dec = decode_attention(pool, q[-1:], lens, table, hb)
    assert np.allclose(out[-1], dec[0], rtol=1e-13, atol=1e-13)
    # overwriting positions after token j's position leaves token j's output unchanged
    pool2 = pool.copy()
    rest = np.full((lens[0] - 45, hkv, 128), 3.0)
    append(pool2, rest, -rest, np.array([0, len(rest)]), np.array([45]), table, hb)
    out2 = prefill_attention(pool2, q, [0, n], lens, table, hb)
    p_first_changed = 45 - (lens[0] - n)            # chunk index of position 45
    assert np.array_equal(out2[:p_first_changed], out[:p_first_changed])
    assert not np.allclose(out2[p_first_changed:], out[p_first_changed:])
