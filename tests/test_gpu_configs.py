"""The five workloads at full size, in the launch configuration the benchmark uses, checked on
sampled sequences against the oracle.

For each decode workload the whole batch goes through the GPU append (prefill, then the step
token) and the GPU decode at its real shape.  The append is checked on the sampled sequences'
slots (parity rules of tests/parity.py) and on the sentinel bytes of the whole pool.  For the
attention check the sampled sequences' pages are overwritten with the oracle's own bytes before
the decode, so both sides attend over the same dequantized cache.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_kv_cache_02_amd import kvq, workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu
SENT = 0xA5
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
QDT = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}
FMT = {"int4": oracle.FMT_INT4, "mxfp4": oracle.FMT_MXFP4}


def _gpu_prefill_and_step(w, lens, table, num_pages, chunk=8):
    """GPU append of the cached tokens (chunks of sequences), then of the step tokens."""
    dev = torch.device("cuda")
    cache = kvq.Cache(num_pages, w.num_kv_heads, w.had_block, w.fmt, fill=SENT)
    bt = torch.from_numpy(table).to(dev)
    pre = lens - 1
    new_k = np.zeros((w.batch, w.num_kv_heads, 128), np.float32)
    new_v = np.zeros_like(new_k)
    for b0 in range(0, w.batch, chunk):
        bs = list(range(b0, min(b0 + chunk, w.batch)))
        ks, vs = [], []
        for b in bs:
            k, v = wl.sequence_kv(w, b, int(lens[b]))
            ks.append(k[:-1])
            vs.append(v[:-1])
            new_k[b], new_v[b] = k[-1], v[-1]
        cu = np.zeros(w.batch + 1, np.int32)
        cnt = np.zeros(w.batch, np.int64)
        cnt[bs] = pre[bs]
        cu[1:] = np.cumsum(cnt)
        kvq.append(cache, torch.from_numpy(np.concatenate(ks)).to(TDT[w.kv_dtype]).to(dev),
                   torch.from_numpy(np.concatenate(vs)).to(TDT[w.kv_dtype]).to(dev),
                   torch.from_numpy(cu).to(dev), torch.zeros(w.batch, dtype=torch.int32, device=dev),
                   bt, int(pre.max()))
    kvq.append(cache, torch.from_numpy(new_k).to(TDT[w.kv_dtype]).to(dev),
               torch.from_numpy(new_v).to(TDT[w.kv_dtype]).to(dev),
               torch.arange(w.batch + 1, dtype=torch.int32, device=dev),
               torch.from_numpy(pre.astype(np.int32)).to(dev), bt, 1)
    torch.cuda.synchronize()
    return cache


def _check_decode_workload(name, sample):
    w = wl.WORKLOADS[name]
    print(f"[config] {name}: building", flush=True)
    lens = wl.seq_lens(w)
    table, num_pages = wl.block_table(w, lens)
    cache = _gpu_prefill_and_step(w, lens, table, num_pages)
    gpu_pool = cache.pool.cpu().numpy()
    cu_all = np.concatenate([[0], np.cumsum(lens)])
    mask = parity.touched_mask(gpu_pool.shape, cu_all, np.zeros(w.batch, np.int64), table)
    assert (gpu_pool[~mask] == SENT).all(), f"{name}: bytes outside appended slots changed"

    # oracle append of the sampled sequences (all their tokens) into an oracle pool
    pool_o = np.full_like(gpu_pool, SENT)
    flips = 0
    for b in sample:
        k, v = wl.sequence_kv(w, b, int(lens[b]))
        infos = oracle.append(pool_o, k, v, np.array([0, lens[b]]), np.array([0]), table[b:b + 1],
                              w.had_block, FMT[w.fmt])
        cu = np.array([0, lens[b]])
        st = np.array([0])
        for which in ("k", "v"):
            codes, params = parity.appended_entries(gpu_pool, cu, st, table[b:b + 1], which)
            if w.fmt == "int4":
                flips += parity.check_int4_entries(codes, params, infos[which], f"{name}/{b}/{which}")
            else:
                flips += parity.check_mxfp4_entries(codes, params, infos[which], f"{name}/{b}/{which}")
    print(f"[config] {name}: append ok on sequences {sample}, {flips} tolerated boundary flips", flush=True)

    # decode over the whole batch; the sampled sequences' pages hold the oracle's bytes
    dev = torch.device("cuda")
    for b in sample:
        pages = table[b, :-(-int(lens[b]) // 16)]
        cache.pool[torch.from_numpy(pages.astype(np.int64)).to(dev)] = \
            torch.from_numpy(pool_o[pages]).to(dev)
    q = wl.queries(w)
    q_t = torch.from_numpy(q).to(QDT[w.q_dtype])
    ref = oracle.decode_attention(pool_o, q_t.float().numpy(), lens, table, w.had_block, FMT[w.fmt],
                                  seqs=sample)
    # MXFP4: also the path with both contractions on the scaled FP8 x FP4 matrix cores
    for scaled in ((False, True) if w.fmt == "mxfp4" else (False,)):
        out = kvq.decode_attn(cache, q_t.to(dev), torch.from_numpy(lens.astype(np.int32)).to(dev),
                              torch.from_numpy(table).to(dev), int(lens.max()), out_dtype=torch.float32,
                              scaled_mfma=scaled)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        err = parity.attn_row_error(got[sample], ref[sample])
        print(f"[config] {name}: decode (scaled={scaled}) max row err {err.max():.3e} on sequences {sample}",
              flush=True)
        assert err.max() <= parity.ATTN_TOL


def test_config_tiny():
    _check_decode_workload("tiny", [0])


def test_config_llama():
    _check_decode_workload("llama", [0, 13, 31])


def test_config_llama_step():
    # the call the benchmark times, at its size: kvq_decode_step over 32 sequences x 4096 tokens,
    # 8 kv heads (the 8-wave plan, 256 pages per (sequence, kv head), the appending waves also
    # streaming the last page).  The GPU appends the 4095 cached tokens of every sequence, then
    # the step appends token 4096 and attends.  Sampled sequences: the step token's bytes follow
    # the append rules, the earlier bytes are unchanged, nothing else is written, and the
    # attention matches the oracle run on the pool as the GPU left it.  A second step call with
    # bf16 output (the benchmark's dtype) gives the round-to-nearest-even of the fp32 result.
    w = wl.WORKLOADS["llama"]
    sample = [0, 13, 31]
    print("[config] llama step: building", flush=True)
    lens = wl.seq_lens(w)
    table, num_pages = wl.block_table(w, lens)
    dev = torch.device("cuda")
    cache = kvq.Cache(num_pages, w.num_kv_heads, w.had_block, w.fmt, fill=SENT)
    bt = torch.from_numpy(table).to(dev)
    pre = lens - 1
    new_k = np.zeros((w.batch, w.num_kv_heads, 128), np.float32)
    new_v = np.zeros_like(new_k)
    for b0 in range(0, w.batch, 8):
        bs = list(range(b0, b0 + 8))
        ks, vs = [], []
        for b in bs:
            k, v = wl.sequence_kv(w, b, int(lens[b]))
            ks.append(k[:-1])
            vs.append(v[:-1])
            new_k[b], new_v[b] = k[-1], v[-1]
        cnt = np.zeros(w.batch, np.int64)
        cnt[bs] = pre[bs]
        cu = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
        kvq.append(cache, torch.from_numpy(np.concatenate(ks)).to(TDT[w.kv_dtype]).to(dev),
                   torch.from_numpy(np.concatenate(vs)).to(TDT[w.kv_dtype]).to(dev),
                   torch.from_numpy(cu).to(dev), torch.zeros(w.batch, dtype=torch.int32, device=dev),
                   bt, int(pre.max()))
    torch.cuda.synchronize()
    pool0 = cache.pool.cpu().numpy()
    q_t = torch.from_numpy(wl.queries(w)).to(QDT[w.q_dtype])
    kn = torch.from_numpy(new_k).to(TDT[w.kv_dtype]).to(dev)
    vn = torch.from_numpy(new_v).to(TDT[w.kv_dtype]).to(dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    out = kvq.decode_step(cache, kn, vn, q_t.to(dev), sl, bt, int(lens.max()), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gpu_pool = cache.pool.cpu().numpy()

    cu_pre = np.concatenate([[0], np.cumsum(pre)])
    prior = parity.touched_mask(pool0.shape, cu_pre, np.zeros(w.batch, np.int64), table)
    step_mask = parity.touched_mask(pool0.shape, np.arange(w.batch + 1), pre, table)
    keep = ~step_mask
    assert np.array_equal(gpu_pool[keep], pool0[keep]), "llama step: bytes outside the step tokens changed"
    assert not (prior & step_mask).any()
    flips = 0
    for b in sample:
        infos = {}
        for which, x in (("k", new_k[b:b + 1]), ("v", new_v[b:b + 1])):
            infos[which] = oracle.paged.encode(x, w.had_block, FMT[w.fmt])[2]
        cu1 = np.array([0, 1])
        st = pre[b:b + 1]
        for which in ("k", "v"):
            codes, params = parity.appended_entries(gpu_pool, cu1, st, table[b:b + 1], which)
            flips += parity.check_int4_entries(codes, params, infos[which], f"llama-step/{b}/{which}")
    ref = oracle.decode_attention(gpu_pool, q_t.float().numpy(), lens, table, w.had_block, FMT[w.fmt],
                                  seqs=sample)
    err = parity.attn_row_error(got[sample], ref[sample])
    print(f"[config] llama step: {flips} tolerated flips, max row err {err.max():.3e} on sequences {sample}",
          flush=True)
    assert err.max() <= parity.ATTN_TOL

    # the benchmark's output dtype: bf16 equals RNE of the fp32 result (the same token appended
    # again at the same slot writes the same bytes)
    out16 = kvq.decode_step(cache, kn, vn, q_t.to(dev), sl, bt, int(lens.max()), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(cache.pool.cpu(), torch.from_numpy(gpu_pool))
    assert torch.equal(out16.cpu(), out.cpu().to(torch.bfloat16))


def test_config_prefill_attention():
    # the chunked-prefill launch the benchmark times, at its size: 32 sequences whose last 512 of
    # 4096 positions are a new turn attending causally over the resident prefix and each other,
    # 32 q / 8 kv heads.  The cache is the GPU's append of the llama workload; sampled chunk tokens
    # (the first, middle and last query tiles) of sequences 0 and 31 are checked against the
    # oracle's attention over that pool, and a bf16 output (the benchmark's dtype) against the
    # round-to-nearest-even of the fp32 one.
    from oracle.attention import decode_attention_one, gather_sequence
    w = wl.WORKLOADS["llama"]
    chunk = 512
    print("[config] prefill attention: building", flush=True)
    lens = wl.seq_lens(w)
    table, num_pages = wl.block_table(w, lens)
    dev = torch.device("cuda")
    cache = kvq.Cache(num_pages, w.num_kv_heads, w.had_block, w.fmt, fill=SENT)
    bt = torch.from_numpy(table).to(dev)
    for b0 in range(0, w.batch, 8):
        bs = list(range(b0, b0 + 8))
        kv = [wl.sequence_kv(w, b, int(lens[b])) for b in bs]
        cnt = np.zeros(w.batch, np.int64)
        cnt[bs] = lens[bs]
        cu = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
        kvq.append(cache, torch.from_numpy(np.concatenate([k for k, _ in kv])).to(TDT[w.kv_dtype]).to(dev),
                   torch.from_numpy(np.concatenate([v for _, v in kv])).to(TDT[w.kv_dtype]).to(dev),
                   torch.from_numpy(cu).to(dev), torch.zeros(w.batch, dtype=torch.int32, device=dev), bt,
                   int(lens.max()))
    rng = np.random.default_rng(77)
    q = rng.standard_normal((w.batch * chunk, w.num_q_heads, 128)).astype(np.float32)
    q_t = torch.from_numpy(q).to(torch.bfloat16)
    cu_q = torch.arange(0, w.batch * chunk + 1, chunk, dtype=torch.int32, device=dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    out = kvq.prefill_attn(cache, q_t.to(dev), cu_q, sl, bt, int(lens.max()), chunk, out_dtype=torch.float32)
    out16 = kvq.prefill_attn(cache, q_t.to(dev), cu_q, sl, bt, int(lens.max()), chunk, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert torch.equal(out16.cpu(), out.cpu().to(torch.bfloat16))
    pool = cache.pool.cpu().numpy()
    qn = q_t.float().numpy()
    worst = 0.0
    for b in (0, 31):
        k_rot, v_rot = gather_sequence(pool, table[b], int(lens[b]), w.had_block, FMT[w.fmt])
        for j in list(range(0, 64)) + list(range(256, 272)) + list(range(448, 512)):
            i = b * chunk + j
            pos = int(lens[b]) - chunk + j
            ref = decode_attention_one(qn[i], k_rot[:, :pos + 1], v_rot[:, :pos + 1], w.had_block)
            worst = max(worst, parity.attn_row_error(got[i], ref).max())
    print(f"[config] prefill attention: max row err {worst:.3e} on sequences 0, 31 (288 tokens)", flush=True)
    assert worst <= parity.ATTN_TOL


def test_config_long_ragged():
    w = wl.WORKLOADS["long"]
    lens = wl.seq_lens(w)
    sample = [int(np.argmax(lens)), int(np.argmin(lens))]
    _check_decode_workload("long", sample)


def test_config_mxfp4():
    _check_decode_workload("mxfp4", [0, 63])


def test_config_prefill_append():
    w = wl.WORKLOADS["prefill"]
    print("[config] prefill: building", flush=True)
    lens = wl.seq_lens(w)
    table, num_pages = wl.block_table(w, lens)
    dev = torch.device("cuda")
    cache = kvq.Cache(num_pages, w.num_kv_heads, w.had_block, fill=SENT)
    ks, vs = zip(*[wl.sequence_kv(w, b, int(lens[b])) for b in range(w.batch)])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kvq.append(cache, torch.from_numpy(np.concatenate(ks)).to(torch.bfloat16).to(dev),
               torch.from_numpy(np.concatenate(vs)).to(torch.bfloat16).to(dev),
               torch.from_numpy(cu).to(dev), torch.zeros(w.batch, dtype=torch.int32, device=dev),
               torch.from_numpy(table).to(dev), int(lens.max()))
    torch.cuda.synchronize()
    gpu_pool = cache.pool.cpu().numpy()
    mask = parity.touched_mask(gpu_pool.shape, cu, np.zeros(w.batch, np.int64), table)
    assert (gpu_pool[~mask] == SENT).all()
    flips = 0
    for b in (0, 37, 63):
        infos = oracle.paged.encode(ks[b], w.had_block, oracle.FMT_INT4)[2], \
            oracle.paged.encode(vs[b], w.had_block, oracle.FMT_INT4)[2]
        for which, info in zip(("k", "v"), infos):
            codes, params = parity.appended_entries(gpu_pool, np.array([0, lens[b]]), np.array([0]),
                                                    table[b:b + 1], which)
            flips += parity.check_int4_entries(codes, params, info, f"prefill/{b}/{which}")
    print(f"[config] prefill: append ok on sequences 0, 37, 63; {flips} tolerated boundary flips", flush=True)
