"""Pins for the oracle's page layout and paged append (CPU only)."""
import numpy as np

import oracle
from oracle import pack_row, unpack_row, nibble_position
from oracle.layout import v_row_offsets, k_row_offsets
from oracle.paged import append, token_slots, FMT_INT4, FMT_MXFP4, read_token
from tests.conftest import read_golden


def _golden_row(tag):
    for r in read_golden("layout_rows.txt"):
        if r[0] == tag:
            return np.array([int(x, 16) for x in r[1:]], dtype=np.uint8)
    raise KeyError(tag)


def test_row_layout_golden():
    ch = np.arange(128)
    assert np.array_equal(pack_row(ch % 16), _golden_row("P1"))
    assert np.array_equal(pack_row(ch // 16), _golden_row("P2"))


def test_row_pack_unpack_inverse_and_permutation():
    assert sorted(nibble_position(np.arange(128))) == list(range(128))
    rng = np.random.default_rng(31)
    c = rng.integers(0, 16, (20, 128)).astype(np.uint8)
    assert np.array_equal(unpack_row(pack_row(c)), c)


def test_v_quad_interleave_golden():
    block = np.zeros(2176, dtype=np.uint8)
    for s in range(16):
        block[v_row_offsets(s)] = pack_row(np.full(128, s))
    for tq in range(4):
        want = np.tile(_golden_row(f"V{tq}"), 64)
        assert np.array_equal(block[1024 + 256 * tq:1024 + 256 * (tq + 1)], want)


def test_offsets_partition_block():
    used = np.concatenate([k_row_offsets(np.arange(16)).ravel(), v_row_offsets(np.arange(16)).ravel(),
                           2048 + np.arange(128)])
    assert sorted(used) == list(range(2176))


def _rand_kv(rng, t, hkv):
    k = rng.standard_normal((t, hkv, 128)).astype(np.float16).astype(np.float64)
    v = rng.standard_normal((t, hkv, 128)).astype(np.float16).astype(np.float64)
    return k, v


def test_append_only_touches_appended_slots_and_splits_consistently():
    # Appending all tokens at once equals appending them one call per token, and
    # every byte outside the appended slots keeps the sentinel.
    rng = np.random.default_rng(32)
    hkv, n_pages = 2, 12
    lens_new = np.array([5, 21, 1])
    start = np.array([3, 14, 0])
    cu = np.concatenate([[0], np.cumsum(lens_new)])
    table = rng.permutation(n_pages)[:9].reshape(3, 3).astype(np.int32)
    k, v = _rand_kv(rng, int(cu[-1]), hkv)
    for fmt, hb in ((FMT_INT4, 64), (FMT_MXFP4, 128)):
        pool_a = np.full((n_pages, hkv, 2176), 0xA5, dtype=np.uint8)
        append(pool_a, k, v, cu, start, table, hb, fmt)
        pool_b = np.full_like(pool_a, 0xA5)
        for b in range(3):
            for i in range(cu[b], cu[b + 1]):
                append(pool_b, k, v, np.array([i, i + 1]), np.array([start[b] + i - cu[b]]),
                       table[b:b + 1], hb, fmt)
        assert np.array_equal(pool_a, pool_b)
        touched = np.zeros_like(pool_a, dtype=bool)
        _, page, slot = token_slots(cu, start, table)
        for p, s in zip(page, slot):
            touched[p, :, k_row_offsets(s)] = True
            touched[p, :, v_row_offsets(s)] = True
            touched[p, :, 2048 + 4 * s:2048 + 4 * s + 4] = True
            touched[p, :, 2112 + 4 * s:2112 + 4 * s + 4] = True
        assert np.all(pool_a[~touched] == 0xA5)
        assert np.any(pool_a[touched] != 0xA5)


def test_append_addresses_via_block_table():
    # Token at position p of sequence b is found on page table[b][p//16], slot p%16.
    rng = np.random.default_rng(33)
    hkv = 1
    table = np.array([[4, 1, 7]], dtype=np.int32)
    k, v = _rand_kv(rng, 40, hkv)
    pool = np.zeros((8, hkv, 2176), dtype=np.uint8)
    infos = append(pool, k, v, np.array([0, 40]), np.array([5]), table, 128, FMT_INT4)
    for i in range(40):
        p = 5 + i
        codes, params = read_token(pool, table[0, p // 16], 0, p % 16, "k")
        assert np.array_equal(codes, infos["k"]["codes"][i, 0])
        assert params.view("<f2")[0] == infos["k"]["s16"][i, 0]
