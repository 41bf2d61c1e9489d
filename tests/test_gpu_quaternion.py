"""Parity of every kernel with the quaternion block-4 rotation (IsoQuant abstract: each 4-channel
block v -> q_L v conj(q_R); IsoQuant-Fast keeps q_L only) against the oracle: append (INT4 and
MXFP4, f16 and bf16 inputs), decode (both MXFP4 q.K paths, rotated and unrotated outputs), the
fused decode step, chunked prefill and page dequantization.  The quaternions are the seeded
fp32 unit quaternions both sides receive."""
import numpy as np
import pytest
import torch

import oracle
from bit_kv_cache_02_amd import kvq, workloads as wl
from tests import parity
from tests.test_gpu_append import run_append, rand_kv, ragged_table
from tests.test_gpu_decode import oracle_cache, run_decode
from tests.test_gpu_prefill import run_prefill
from tests.test_gpu_step import run_step

pytestmark = pytest.mark.gpu


def rot(seed, full):
    return oracle.QuatRotation(wl.unit_quaternions(seed, full))


@pytest.mark.parametrize("fmt", [oracle.FMT_INT4, oracle.FMT_MXFP4])
@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_append_quaternion(fmt, full, dtype):
    rng = np.random.default_rng(100 + 2 * fmt + full)
    lens = [1, 15, 16, 17, 100, 333]
    start = [0, 3, 0, 16, 5, 0]
    table, total = ragged_table(rng, lens, start)
    k, v = rand_kv(rng, sum(lens), 2, dtype)
    run_append(f"quat/fmt{fmt}/full={full}/{dtype}", k, v, lens, start, table, total, 2, rot(fmt + 10, full),
               fmt, dtype)


@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("group", [1, 4, 8])
def test_decode_int4_quaternion(full, group):
    rng = np.random.default_rng(110 + group + full)
    lens = [1, 17, 300, 1000]
    r = rot(20 + group, full)
    pool, table = oracle_cache(rng, lens, 2, r)
    run_decode(f"quat/int4/G{group}/full={full}", pool, table, lens, 2 * group, r, seed=group)


@pytest.mark.parametrize("scaled", [False, True])
def test_decode_mxfp4_quaternion(scaled):
    rng = np.random.default_rng(120 + scaled)
    lens = [5000, 300, 1]
    r = rot(30, True)
    pool, table = oracle_cache(rng, lens, 1, r, fmt=oracle.FMT_MXFP4)
    run_decode(f"quat/mxfp4/scaled={scaled}", pool, table, lens, 8, r, fmt=oracle.FMT_MXFP4, q_dtype="e4m3",
               scaled_mfma=scaled)


def test_decode_quaternion_rotated_output_and_bf16():
    rng = np.random.default_rng(130)
    lens = [90, 31]
    r = rot(40, False)
    pool, table = oracle_cache(rng, lens, 2, r)
    run_decode("quat/rotated", pool, table, lens, 8, r, rotated=True, seed=3)
    f32 = run_decode("quat/f32", pool, table, lens, 8, r, seed=4)
    bf = run_decode("quat/bf16", pool, table, lens, 8, r, seed=4, out_dtype=torch.bfloat16, check=False)
    # a bf16 output is the fp32 output rounded to nearest even
    assert np.array_equal(bf, torch.from_numpy(f32.astype(np.float32)).bfloat16().float().numpy())


@pytest.mark.parametrize("fmt,full", [("int4", False), ("mxfp4", True)])
def test_step_quaternion(fmt, full):
    run_step(f"quat/{fmt}/full={full}", [1, 16, 17, 300, 2000], hkv=2, group=4, hb=rot(50, full), fmt=fmt,
             seed=140 + full)


@pytest.mark.parametrize("fmt,full", [(oracle.FMT_INT4, True), (oracle.FMT_MXFP4, False)])
def test_prefill_quaternion(fmt, full):
    run_prefill(f"quat/fmt{fmt}/full={full}", [40, 17, 300, 1, 33], [9, 17, 40, 1, 16], hkv=2, group=4,
                hb=rot(60, full), fmt=fmt, seed=150 + fmt)


@pytest.mark.parametrize("fmt", [oracle.FMT_INT4, oracle.FMT_MXFP4])
def test_dequant_pages_quaternion(fmt):
    rng = np.random.default_rng(160 + fmt)
    r = rot(70, True)
    pool, table = oracle_cache(rng, [40, 70], 3, r, fmt=fmt)
    print(f"[dequant] quat fmt{fmt}", flush=True)
    khb, quat = parity.kernel_rotation(r)
    cache = kvq.Cache(pool.shape[0], 3, khb, "int4" if fmt == oracle.FMT_INT4 else "mxfp4",
                      pool=torch.from_numpy(pool).cuda(), quat=quat)
    ids = np.array([table[0, 0], table[1, 4], table[1, 0], table[0, 2]], np.int32)
    k, v = kvq.dequant_pages(cache, torch.from_numpy(ids).cuda())
    kr, vr = oracle.dequant_pages(pool, ids, r, fmt)
    assert np.array_equal(k.cpu().numpy(), kr.astype(np.float32))
    assert np.array_equal(v.cpu().numpy(), vr.astype(np.float32))
    ku, vu = kvq.dequant_pages(cache, torch.from_numpy(ids).cuda(), unrotate=True)
    kur, vur = oracle.dequant_pages(pool, ids, r, fmt, unrotate=True)
    for got, ref in ((ku, kur), (vu, vur)):
        got = got.cpu().numpy().astype(np.float64)
        assert np.abs(got - ref).max() <= 1e-6 * np.abs(ref).max()
