"""Seeded random shapes through decode, the fused step and chunked prefill, against the oracle.

Each case draws the batch, kv heads, group size, rotation (Hadamard 64 / 128, none, the
quaternion block rotation), cache format, query dtype and ragged sequence lengths (with page
boundaries among them), so that the planner's choices (one workgroup per unit, fixed splits,
the balanced cut) and the merge of split runs meet shapes the hand-written cases do not."""
import numpy as np
import pytest

import oracle
from bit_kv_cache_02_amd import workloads as wl
from tests.test_gpu_decode import oracle_cache, run_decode
from tests.test_gpu_prefill import run_prefill
from tests.test_gpu_step import run_step

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(9000 + seed)
    fmt = oracle.FMT_MXFP4 if rng.random() < 0.3 else oracle.FMT_INT4
    rot = str(rng.choice(["128", "1", "quat"] if fmt == oracle.FMT_MXFP4 else ["64", "128", "1", "quat"]))
    hb = oracle.QuatRotation(wl.unit_quaternions(seed, bool(rng.integers(2)))) if rot == "quat" else int(rot)
    b = int(rng.integers(1, 13))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.integers(1, 9))
    top = int(rng.choice([40, 700, 3000, 6000]))
    lens = [int(x) for x in rng.integers(1, top + 1, size=b)]
    for i in range(b):
        if rng.random() < 0.25:
            lens[i] = int(rng.choice([1, 15, 16, 17, 32, 33]))
    q_dtype = "e4m3" if fmt == oracle.FMT_MXFP4 and rng.random() < 0.5 else str(rng.choice(["bf16", "f16"]))
    return rng, fmt, rot, hb, b, hkv, group, lens, q_dtype


@pytest.mark.parametrize("seed", range(10))
def test_random_decode(seed):
    rng, fmt, rot, hb, b, hkv, group, lens, q_dtype = draw(seed)
    pool, table = oracle_cache(rng, lens, hkv, hb, fmt=fmt)
    run_decode(f"random/{seed}: fmt{fmt} rot {rot} B{b} Hkv{hkv} G{group} {q_dtype} lens {lens}", pool, table, lens,
               hkv * group, hb, fmt=fmt, q_dtype=q_dtype, seed=seed, scaled_mfma=fmt == oracle.FMT_MXFP4 and seed % 2 == 0)


@pytest.mark.parametrize("seed", range(10, 16))
def test_random_step(seed):
    rng, fmt, rot, hb, b, hkv, group, lens, q_dtype = draw(seed)
    run_step(f"random/{seed}: fmt{fmt} rot {rot} B{b} Hkv{hkv} G{group} lens {lens}", lens, hkv=hkv, group=group,
             hb=hb, fmt="mxfp4" if fmt == oracle.FMT_MXFP4 else "int4", seed=seed,
             q_dtype="bf16" if q_dtype == "e4m3" else q_dtype)


@pytest.mark.parametrize("seed", range(16, 22))
def test_random_prefill(seed):
    rng, fmt, rot, hb, b, hkv, group, lens, q_dtype = draw(seed)
    lens = [min(x, 1500) for x in lens]
    chunks = [int(rng.integers(1, min(x, 80) + 1)) for x in lens]
    run_prefill(f"random/{seed}: fmt{fmt} rot {rot} B{b} Hkv{hkv} G{group} lens {lens} chunks {chunks}", lens,
                chunks, hkv=hkv, group=group, hb=hb, fmt=fmt, q_dtype="bf16" if q_dtype == "e4m3" else q_dtype,
                seed=seed)


PLAN_VARS = ("BALANCED", "SLOTS", "MIN_PIECE", "WAVES", "DEPTH", "PAGES_PER_SPLIT")


@pytest.mark.parametrize("seed", range(22, 30))
def test_random_decode_plans(monkeypatch, seed):
    # the same random shapes under a random plan of the tuning variables (read on every call):
    # fixed splits of 1 to 64 W pages, or the balanced cut with any slot count and minimum run
    rng, fmt, rot, hb, b, hkv, group, lens, q_dtype = draw(seed)
    for k in PLAN_VARS:
        monkeypatch.delenv(f"KVQ_DECODE_{k}", raising=False)
    prng = np.random.default_rng(7000 + seed)
    waves = int(prng.choice([4, 8]))
    plan = {"WAVES": waves, "DEPTH": int(prng.integers(2, 5))}
    if seed % 2:
        plan.update(BALANCED=1, SLOTS=int(prng.integers(1, 600)), MIN_PIECE=int(prng.choice([1, 2, 5, 16])))
    else:
        plan.update(BALANCED=0, PAGES_PER_SPLIT=int(prng.integers(1, 64 * waves + 1)))
    for k, v in plan.items():
        monkeypatch.setenv(f"KVQ_DECODE_{k}", str(v))
    pool, table = oracle_cache(rng, lens, hkv, hb, fmt=fmt)
    run_decode(f"random-plan/{seed}: {plan} fmt{fmt} rot {rot} B{b} Hkv{hkv} G{group} {q_dtype} lens {lens}", pool,
               table, lens, hkv * group, hb, fmt=fmt, q_dtype=q_dtype, seed=seed,
               scaled_mfma=fmt == oracle.FMT_MXFP4 and seed % 4 == 1)
