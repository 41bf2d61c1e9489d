"""Parity at the sizes the library states as its limits, on wide batches, and on degenerate
inputs (all-zero and constant vectors, whose INT4 scale is zero and MXFP4 groups E = 0)."""
import numpy as np
import pytest
import torch

import oracle
from bit_kv_cache_02_amd import kvq
from tests import parity
from tests.test_gpu_append import run_append, rand_kv, ragged_table
from tests.test_gpu_decode import oracle_cache, run_decode
from tests.test_gpu_prefill import run_prefill

pytestmark = pytest.mark.gpu


def test_decode_longest_context():
    # 131072 positions (8192 pages) next to a one-token sequence: the most splits per unit
    rng = np.random.default_rng(200)
    lens = [131072, 1]
    pool, table = oracle_cache(rng, lens, 1, 128)
    run_decode("limits/decode 131072", pool, table, lens, 8, 128, seed=1)


def test_prefill_at_the_position_limit():
    # chunked prefill attends at most 131072 positions (the staged block table); the last
    # position of the chunk is exactly there
    run_prefill("limits/prefill 131072", [131072, 40], [32, 40], hkv=1, group=8, hb=64, seed=2)


def test_decode_wide_batch_many_heads():
    # 640 sequences x 16 kv heads: 10240 (sequence, kv head) units, the 256-page 4-wave plan
    rng = np.random.default_rng(201)
    lens = [int(x) for x in rng.integers(1, 70, 640)]
    pool, table = oracle_cache(rng, lens, 16, 64)
    run_decode("limits/wide", pool, table, lens, 32, 64, seed=3)


def test_append_many_sequences_and_heads():
    rng = np.random.default_rng(202)
    lens = [int(x) for x in rng.integers(1, 4, 3000)]
    start = [int(x) for x in rng.integers(0, 40, 3000)]
    table, total = ragged_table(rng, lens, start)
    k, v = rand_kv(rng, sum(lens), 16, "bf16")
    run_append("limits/3000 seqs x 16 heads", k, v, lens, start, table, total, 16, 128, oracle.FMT_INT4, "bf16")


@pytest.mark.parametrize("fmt,hb", [(oracle.FMT_INT4, 1), (oracle.FMT_INT4, 128), (oracle.FMT_MXFP4, 128)])
def test_degenerate_vectors_append_and_decode(fmt, hb):
    # zero vectors (zero after any rotation), constant vectors and vectors with all-zero
    # 32-channel groups: the INT4 scale is zero (all codes 0, zero = the constant), an MXFP4
    # group with amax 0 takes E = 0; attention over such keys is uniform
    rng = np.random.default_rng(203 + hb + fmt)
    t = 40
    k = np.zeros((t, 1, 128), np.float32)
    v = np.zeros((t, 1, 128), np.float32)
    k[10:20] = 0.75  # constant vectors (not constant after a Hadamard rotation)
    v[10:20] = -1.5
    k[20:30, :, 32:64] = rng.standard_normal((10, 1, 32))  # one live group, three zero groups
    v[30:40] = rng.standard_normal((10, 1, 128))
    k = torch.from_numpy(k).bfloat16().float().numpy()
    v = torch.from_numpy(v).bfloat16().float().numpy()
    lens = [t]
    table, total = ragged_table(rng, lens, [0])
    cache, pool_o, _ = run_append(f"limits/degenerate fmt{fmt} b{hb}", k, v, lens, [0], table, total, 1, hb,
                                  fmt, "bf16")
    run_decode(f"limits/degenerate decode fmt{fmt} b{hb}", pool_o, table, lens, 4, hb, fmt=fmt, seed=4)
    # page dequantization of the same pages, rotated basis (exact) and rotated back (INT4 b = 64 / 128 on the
    # matrix cores: a zero scale leaves only the zero point's share, z sqrt(b) at each block's first channel)
    ids = np.unique(table[0, :2]).astype(np.int32)  # the two full pages of the 40 tokens
    dcache = kvq.Cache(pool_o.shape[0], 1, hb, "int4" if fmt == oracle.FMT_INT4 else "mxfp4",
                       pool=torch.from_numpy(pool_o).cuda())
    for unrot in (False, True):
        gk, gv = kvq.dequant_pages(dcache, torch.from_numpy(ids).cuda(), unrotate=unrot)
        rk, rv = oracle.dequant_pages(pool_o, ids, hb, fmt, unrotate=unrot)
        for got, ref in ((gk, rk), (gv, rv)):
            got = got.cpu().numpy().astype(np.float64)
            assert np.abs(got - ref).max() <= 1e-6 * max(np.abs(ref).max(), 1e-30), f"dequant unrotate={unrot}"
    # all-zero keys and values: uniform softmax, zero output
    z = np.zeros((16, 1, 128), np.float32)
    table0, total0 = ragged_table(rng, [16], [0])
    _, pool0, _ = run_append(f"limits/zeros fmt{fmt} b{hb}", z, z, [16], [0], table0, total0, 1, hb, fmt, "bf16")
    got = run_decode(f"limits/zeros decode fmt{fmt} b{hb}", pool0, table0, [16], 4, hb, fmt=fmt, seed=5, check=False)
    assert np.array_equal(got, np.zeros_like(got))


@pytest.mark.parametrize("fmt", [oracle.FMT_INT4, oracle.FMT_MXFP4])
@pytest.mark.parametrize("fill", [0xA5, "random"])
def test_unwritten_slots_do_not_leak(fmt, fill):
    # the slots past a sequence's end hold whatever the pool held: a stray MXFP4 scale byte of
    # 0xA5 is 2^38 (fp16 overflow), random fp16 INT4 parameters can be inf or NaN.  Their p is 0,
    # and no such value may reach the result (decode on both MXFP4 q.K paths, and prefill)
    rng = np.random.default_rng(204)
    lens = [40, 17, 300, 1]
    pool, table = oracle_cache(rng, lens, 2, 128, fmt=fmt, fill=fill)
    # 8 and 16 query heads over 2 kv heads: group 4 and 8 (the two INT4 score layouts)
    for hq in (8, 16):
        for scaled in ((False, True) if fmt == oracle.FMT_MXFP4 else (False,)):
            run_decode(f"limits/garbage fmt{fmt} {fill} hq{hq} scaled={scaled}", pool, table, lens, hq, 128,
                       fmt=fmt, seed=6, scaled_mfma=scaled)
    run_prefill(f"limits/garbage prefill fmt{fmt} {fill}", [40, 17, 300], [9, 17, 40], hkv=2, group=4, hb=128,
                fmt=fmt, seed=7, fill=fill)


@pytest.mark.parametrize("group", [4, 8])
def test_step_int4_with_random_bytes_in_the_last_page(group):
    # random fp16 parameters (inf and NaN among them) in the slots past each sequence's end, on
    # both INT4 score layouts (one head per lane group for 4 heads, two for 8)
    from tests.test_gpu_step import run_step
    run_step(f"limits/random step int4 G{group}", [1, 17, 300, 2000], hkv=2, group=group, hb=128, seed=9 + group,
             fill="random")


@pytest.mark.parametrize("scaled", [False, True])
def test_step_mxfp4_with_stray_bytes_in_the_last_page(scaled):
    from tests.test_gpu_step import run_step
    run_step(f"limits/garbage step scaled={scaled}", [1, 17, 300, 2000], hkv=2, group=8, hb=128, fmt="mxfp4",
             q_dtype="e4m3", seed=8, scaled_mfma=scaled, fill=0xA5)

