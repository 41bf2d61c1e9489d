"""Parity of kvq_decode_step (append the step's token, then attend, in one launch).

The cache before the step is written by the oracle (first L-1 tokens of every sequence).  After
the GPU step the pool is read back:
  * the new token's bytes follow the append rules against the oracle's append of the same
    vectors (tests/parity.py), the earlier tokens' bytes are unchanged and nothing else is
    written;
  * the attention output matches the oracle's decode over the pool as the GPU left it, so a
    tolerated code flip cannot leak into the comparison;
  * it also agrees with kvq_append followed by kvq_decode_attn on the same inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from bit_kv_cache_02_amd import kvq
from tests import parity

pytestmark = pytest.mark.gpu
SENT = 0x5A
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
QDT = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}
FMT = {"int4": oracle.FMT_INT4, "mxfp4": oracle.FMT_MXFP4}


def _vectors(rng, t, hkv, kv_dtype):
    k = rng.standard_normal((t, hkv, 128)).astype(np.float32)
    k[:, :, [5, 60, 111]] *= 15
    v = (rng.standard_normal((t, hkv, 128)) * 0.5).astype(np.float32)
    k = torch.from_numpy(k).to(TDT[kv_dtype]).float().numpy()
    v = torch.from_numpy(v).to(TDT[kv_dtype]).float().numpy()
    return k, v


def run_step(label, lens, hkv, group, hb, fmt="int4", kv_dtype="bf16", q_dtype="bf16", seed=0,
             scaled_mfma=False, fill=SENT):
    print(f"[step] {label}", flush=True)
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int64)
    b = len(lens)
    n_pages = [-(-int(n) // 16) for n in lens]
    total = sum(n_pages) + 3
    ids = rng.permutation(total)
    table = np.zeros((b, max(n_pages) + 1), np.int32)
    off = 0
    for i, n in enumerate(n_pages):
        table[i, :n] = ids[off:off + n]
        off += n
    k_all, v_all = [], []
    for n in lens:
        k, v = _vectors(rng, int(n), hkv, kv_dtype)
        k_all.append(k)
        v_all.append(v)
    # cache before the step: tokens 0 .. L-2
    if isinstance(fill, str):  # "random": every byte outside the appended slots random
        pool0 = rng.integers(0, 256, (total, hkv, 2176), dtype=np.uint8)
    else:
        pool0 = np.full((total, hkv, 2176), fill, np.uint8)
    pre = lens - 1
    cu_pre = np.concatenate([[0], np.cumsum(pre)])
    if pre.sum() > 0:
        oracle.append(pool0, np.concatenate([k[:-1] for k in k_all]), np.concatenate([v[:-1] for v in v_all]),
                      cu_pre, np.zeros(b, np.int64), table, hb, FMT[fmt])
    knew = np.stack([k[-1] for k in k_all])
    vnew = np.stack([v[-1] for v in v_all])
    q = rng.standard_normal((b, hkv * group, 128)).astype(np.float32)
    q_t = torch.from_numpy(q).to(QDT[q_dtype])
    dev = torch.device("cuda")
    args = dict(seq_lens=torch.from_numpy(lens.astype(np.int32)).to(dev),
                block_table=torch.from_numpy(table).to(dev), max_seq_len=int(lens.max()))

    khb, quat = parity.kernel_rotation(hb)
    cache = kvq.Cache(total, hkv, khb, fmt, pool=torch.from_numpy(pool0).to(dev), quat=quat)
    out = kvq.decode_step(cache, torch.from_numpy(knew).to(TDT[kv_dtype]).to(dev),
                          torch.from_numpy(vnew).to(TDT[kv_dtype]).to(dev), q_t.to(dev), **args,
                          scaled_mfma=scaled_mfma)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gpu_pool = cache.pool.cpu().numpy()

    # appended bytes: the append rules against the oracle's append of the same vectors
    cu1 = np.arange(b + 1)
    prior = parity.touched_mask(pool0.shape, cu_pre, np.zeros(b, np.int64), table)
    new = parity.touched_mask(pool0.shape, cu1, pre, table)
    pool_ref = pool0.copy()
    infos = oracle.append(pool_ref, knew, vnew, cu1, pre, table, hb, FMT[fmt])
    flips = parity.check_append(gpu_pool, pool_ref, infos, cu1, pre, table, FMT[fmt],
                                pool0 if isinstance(fill, str) else fill, label,
                                prior_mask=prior)
    keep = prior & ~new
    assert np.array_equal(gpu_pool[keep], pool0[keep]), f"{label}: earlier tokens' bytes changed"

    # attention over the pool as the GPU left it
    ref = oracle.decode_attention(gpu_pool, q_t.float().numpy(), lens, table, hb, FMT[fmt])
    err = parity.attn_row_error(got, ref)
    print(f"[step] {label}: {flips} tolerated flips, max row err {err.max():.3e}", flush=True)
    assert err.max() <= parity.ATTN_TOL, f"{label}: row error {err.max():.3e}"

    # the two-call path on the same inputs
    cache2 = kvq.Cache(total, hkv, khb, fmt, pool=torch.from_numpy(pool0).to(dev), quat=quat)
    kvq.append(cache2, torch.from_numpy(knew).to(TDT[kv_dtype]).to(dev),
               torch.from_numpy(vnew).to(TDT[kv_dtype]).to(dev), torch.from_numpy(cu1.astype(np.int32)).to(dev),
               torch.from_numpy(pre.astype(np.int32)).to(dev), args["block_table"], 1)
    out2 = kvq.decode_attn(cache2, q_t.to(dev), **args)
    torch.cuda.synchronize()
    err2 = parity.attn_row_error(got, out2.cpu().numpy())
    assert err2.max() <= parity.ATTN_TOL, f"{label}: fused vs two-call row error {err2.max():.3e}"
    return got


@pytest.mark.parametrize("hb", [1, 64, 128])
def test_step_int4_page_boundaries(hb):
    # L = 1 (first token), slot 15, a new page, and longer sequences
    run_step(f"int4/b{hb}", [1, 2, 15, 16, 17, 33, 300, 1025], hkv=2, group=4, hb=hb, seed=hb)


def test_step_int4_f16_group8():
    run_step("int4/f16/G8", [40, 129, 7], hkv=2, group=8, hb=64, kv_dtype="f16", q_dtype="f16", seed=3)


def test_step_int4_long_splits():
    # several workgroups per (sequence, kv head): the last split appends
    run_step("int4/long", [5000, 3001, 40], hkv=2, group=4, hb=128, seed=4)


def test_step_int4_wide_batch():
    # >= 256 (sequence, kv head) units: the 8-wave plan
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 90, size=64)
    run_step("int4/wide", lens, hkv=4, group=4, hb=128, seed=5)


@pytest.mark.parametrize("fmt,hkv,fill", [("int4", 4, SENT), ("int4", 4, "random"), ("int4", 2, SENT),
                                           ("mxfp4", 4, SENT), ("mxfp4", 2, "random")])
def test_step_every_appending_wave(fmt, hkv, fill):
    # 64 sequences x 4 kv heads = 256 units take the 8-wave plan, x 2 kv heads the 4-wave plan;
    # either way one split per unit, page p streamed by wave p % W.  The wave that streams a
    # sequence's last page also appends its token, so put the last page on every wave, with the
    # new token in slot 0 (a fresh page), 1, 7 and 15 (the page's last slot)
    lens = [16 * (i % 16) + (0, 1, 7, 15)[i // 16] + 1 for i in range(64)]
    group, q_dtype = (4, "bf16") if fmt == "int4" else (8, "e4m3")
    run_step(f"{fmt}/every-wave/hkv{hkv}/{fill}", lens, hkv=hkv, group=group, hb=128, fmt=fmt,
             q_dtype=q_dtype, seed=6, fill=fill)


@pytest.mark.parametrize("scaled", [False, True])
@pytest.mark.parametrize("group,q_dtype", [(8, "e4m3"), (1, "bf16")])
def test_step_mxfp4(group, q_dtype, scaled):
    run_step(f"mxfp4/G{group}/scaled={scaled}", [1, 16, 17, 300, 2000], hkv=2, group=group, hb=128,
             fmt="mxfp4", q_dtype=q_dtype, seed=60 + group, scaled_mfma=scaled)


def test_step_repeated_calls_grow_the_cache():
    # three steps in a row on one cache, each appending one more token
    rng = np.random.default_rng(7)
    hkv, group, hb = 2, 4, 128
    lens = np.array([30, 31, 47], np.int64)
    total = 16
    table = rng.permutation(total)[:12].astype(np.int32).reshape(3, 4)
    k_all, v_all = _vectors(rng, int(lens.sum()) + 9, hkv, "bf16")
    pool = np.full((total, hkv, 2176), SENT, np.uint8)
    cu = np.concatenate([[0], np.cumsum(lens)])
    oracle.append(pool, k_all[:cu[-1]], v_all[:cu[-1]], cu, np.zeros(3, np.int64), table, hb)
    dev = torch.device("cuda")
    cache = kvq.Cache(total, hkv, hb, pool=torch.from_numpy(pool).to(dev))
    ref_pool = pool.copy()
    nxt = cu[-1]
    for step in range(3):
        lens = lens + 1
        kn, vn = k_all[nxt:nxt + 3], v_all[nxt:nxt + 3]
        nxt += 3
        q = rng.standard_normal((3, hkv * group, 128)).astype(np.float32)
        q_t = torch.from_numpy(q).bfloat16()
        out = kvq.decode_step(cache, torch.from_numpy(kn).bfloat16().to(dev), torch.from_numpy(vn).bfloat16().to(dev),
                              q_t.to(dev), torch.from_numpy(lens.astype(np.int32)).to(dev),
                              torch.from_numpy(table).to(dev), int(lens.max()))
        torch.cuda.synchronize()
        gpu_pool = cache.pool.cpu().numpy()
        infos = oracle.append(ref_pool, kn, vn, np.arange(4), lens - 1, table, hb)
        parity.check_append(gpu_pool, ref_pool, infos, np.arange(4), lens - 1, table, oracle.FMT_INT4, SENT,
                            f"repeat/{step}",
                            prior_mask=parity.touched_mask(pool.shape, np.concatenate([[0], np.cumsum(lens - 1)]),
                                                           np.zeros(3, np.int64), table))
        ref = oracle.decode_attention(gpu_pool, q_t.float().numpy(), lens, table, hb)
        assert parity.attn_row_error(out.cpu().numpy(), ref).max() <= parity.ATTN_TOL
        ref_pool = gpu_pool.copy()  # the next step builds on the GPU's bytes


@pytest.mark.parametrize("fmt,rot,scaled,plan", [("int4", "hadamard", False, "fixed"),
                                                 ("mxfp4", "hadamard", True, "fixed"),
                                                 ("int4", "quat", False, "fixed"),
                                                 ("int4", "hadamard", False, "balanced")])
def test_step_graph_replays_match_eager(fmt, rot, scaled, plan, monkeypatch):
    # the step captured in a HIP graph and replayed several times, with eager work and
    # synchronisations in between: every replay gives the eager result bit for bit and leaves
    # the workspace's merge counters at zero (INT4; MXFP4 on the scaled-MFMA path; the
    # quaternion rotation; the balanced cut)
    from bit_kv_cache_02_amd import workloads as wl
    if plan == "balanced":
        monkeypatch.setenv("KVQ_DECODE_BALANCED", "1")
        monkeypatch.setenv("KVQ_DECODE_SLOTS", "37")
    rng = np.random.default_rng(8)
    hkv, group = 2, 4
    hb = 128 if rot == "hadamard" else oracle.QuatRotation(wl.unit_quaternions(9, True))
    lens = np.array([700, 33, 5000], np.int64)
    n_pages = [-(-int(n) // 16) for n in lens]
    total = sum(n_pages)
    table = np.zeros((3, max(n_pages)), np.int32)
    ids = rng.permutation(total)
    off = 0
    for i, n in enumerate(n_pages):
        table[i, :n] = ids[off:off + n]
        off += n
    k, v = _vectors(rng, int(lens.sum()), hkv, "bf16")
    pool = np.full((total, hkv, 2176), SENT, np.uint8)
    cu = np.concatenate([[0], np.cumsum(lens - 1)])
    sel = np.concatenate([np.arange(s, s + n - 1) for s, n in zip(np.concatenate([[0], np.cumsum(lens)])[:-1], lens)])
    oracle.append(pool, k[sel], v[sel], cu, np.zeros(3, np.int64), table, hb, FMT[fmt])
    last = np.cumsum(lens) - 1
    dev = torch.device("cuda")
    kn = torch.from_numpy(k[last]).bfloat16().to(dev)
    vn = torch.from_numpy(v[last]).bfloat16().to(dev)
    q = torch.from_numpy(rng.standard_normal((3, hkv * group, 128)).astype(np.float32)).bfloat16().to(dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    bt = torch.from_numpy(table).to(dev)
    khb, quat = parity.kernel_rotation(hb)
    cache = kvq.Cache(total, hkv, khb, fmt, pool=torch.from_numpy(pool).to(dev), quat=quat)
    ws = kvq.make_workspace(cache, hkv * group, 3, int(lens.max()), dev)
    out = torch.empty((3, hkv * group, 128), dtype=torch.float32, device=dev)
    step = lambda: kvq.decode_step(cache, kn, vn, q, sl, bt, int(lens.max()), out=out, workspace=ws,
                                   scaled_mfma=scaled)
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    eager_pool = cache.pool.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.zero_()
        scratch = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager step"
        assert torch.equal(cache.pool, eager_pool), f"replay {r} wrote different bytes"
        assert int(ws[:65536].count_nonzero()) == 0, f"replay {r} left merge counters set"
        del scratch


@pytest.mark.parametrize("group", [3, 6])
def test_step_odd_group_sizes(group):
    run_step(f"int4/G{group}", [1, 16, 17, 300], hkv=2, group=group, hb=128, seed=90 + group)
