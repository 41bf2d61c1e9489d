"""Parity of the balanced cut of decode work against the oracle.

In narrow batches of long, uneven sequences, kvq_decode_attn and kvq_decode_step cut every
(sequence, kv head) on the device, from seq_lens, into near-equal runs of pages, one run per
workgroup, and merge the runs' partial softmax states afterwards.  The planner picks the cut for
large work only; these tests force it on small cases through the tuning variables (read on
every call): slot counts from 1 to more than the pages (runs of one page, units of more than 16
runs, so the merge takes several passes), 4- and 8-wave workgroups, every prefetch depth, both
cache formats and both MXFP4 q.K paths, the fused append, and batches of more than 64
sequences (where the cut takes one thread per sequence and block scans instead of one wave)."""
import numpy as np
import pytest

import oracle
from tests.test_gpu_decode import oracle_cache, run_decode
from tests.test_gpu_step import run_step

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 100, 257, 640, 5000]


@pytest.fixture
def balanced(monkeypatch):
    def set_(**kw):
        monkeypatch.setenv("KVQ_DECODE_BALANCED", "1")
        for k in ("SLOTS", "MIN_PIECE", "WAVES", "DEPTH"):
            monkeypatch.delenv(f"KVQ_DECODE_{k}", raising=False)
        for k, v in kw.items():
            monkeypatch.setenv(f"KVQ_DECODE_{k.upper()}", str(v))
    return set_


@pytest.mark.parametrize("slots,min_piece", [(1, 16), (3, 16), (7, 1), (40, 16), (300, 1), (None, 16)])
def test_balanced_int4(balanced, slots, min_piece):
    kw = {"min_piece": min_piece}
    if slots is not None:
        kw["slots"] = slots
    balanced(**kw)
    rng = np.random.default_rng(400 + (slots or 0))
    pool, table = oracle_cache(rng, LENS, 2, 64)
    run_decode(f"balanced/int4/slots={slots}/min={min_piece}", pool, table, LENS, 8, 64, seed=slots or 1)


@pytest.mark.parametrize("waves,depth", [(4, 2), (4, 3), (4, 4), (8, 2), (8, 3)])
def test_balanced_waves_and_depths(balanced, waves, depth):
    balanced(slots=20, waves=waves, depth=depth, min_piece=4)
    rng = np.random.default_rng(410 + waves + depth)
    lens = [3000, 1, 47, 900]
    pool, table = oracle_cache(rng, lens, 3, 128)
    run_decode(f"balanced/W{waves}/D{depth}", pool, table, lens, 3 * 4, 128, seed=depth)


@pytest.mark.parametrize("scaled", [False, True])
def test_balanced_mxfp4(balanced, scaled):
    balanced(slots=33, min_piece=2)
    rng = np.random.default_rng(420 + scaled)
    lens = [4000, 17, 1, 333]
    pool, table = oracle_cache(rng, lens, 2, 128, fmt=oracle.FMT_MXFP4)
    run_decode(f"balanced/mxfp4/scaled={scaled}", pool, table, lens, 16, 128, fmt=oracle.FMT_MXFP4,
               q_dtype="e4m3", seed=5, scaled_mfma=scaled)


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_balanced_fused_step(balanced, fmt):
    # the appended token's page lies in whichever run holds the sequence's last page
    balanced(slots=25, min_piece=3)
    run_step(f"balanced/step/{fmt}", [1, 16, 17, 300, 2001, 4096], hkv=2, group=4, hb=128, fmt=fmt,
             seed=430 + (fmt == "mxfp4"))


def test_balanced_is_the_default_for_large_narrow_batches(monkeypatch):
    # 32 units of up to 750 pages: the planner's own choice (the cut, 2 pages in flight, 512 slots)
    for k in ("BALANCED", "SLOTS", "MIN_PIECE", "WAVES", "DEPTH", "PAGES_PER_SPLIT"):
        monkeypatch.delenv(f"KVQ_DECODE_{k}", raising=False)
    rng = np.random.default_rng(440)
    lens = [12000, 1100, 7000, 3]
    pool, table = oracle_cache(rng, lens, 8, 64)
    run_decode("balanced/default", pool, table, lens, 32, 64, seed=440)


@pytest.mark.parametrize("nseq,slots", [(80, 100), (200, 57)])
def test_balanced_many_sequences(balanced, nseq, slots):
    # more than 64 sequences: the cut runs one thread per sequence with block scans (up to 64,
    # every wave computes it alone); short ragged sequences, some split into several runs
    balanced(slots=slots, min_piece=2)
    rng = np.random.default_rng(450 + nseq)
    lens = [int(x) for x in rng.integers(1, 400, size=nseq)]
    lens[3] = 1500
    pool, table = oracle_cache(rng, lens, 1, 64)
    run_decode(f"balanced/{nseq}-seqs/slots={slots}", pool, table, lens, 4, 64, seed=nseq)
