#!/usr/bin/env python3
"""Benchmark of the rotated 4-bit paged KV-cache hot path on one MI355X.

A step is one decode step of one Llama-3-8B-shaped attention layer: append the new
token of each of 32 sequences into the paged INT4 cache (block-diagonal Hadamard
b = 128, token-wise INT4), then decode attention of 32 query heads over 8 kv heads
and 4096 tokens per sequence (the new one included).  The step runs as one launch of
kvq_decode_step, replayed from a HIP graph; steps cycle over 8 independent layer caches
(8 x 143 MB) so that the 256 MB Infinity Cache cannot serve the pages.

Printed: one JSON line with the whole-step algorithmic throughput (GB/s), the step
kernel's average launch duration from HIP events on its stream and its roofline
fraction against 8 TB/s, the same step as two launches (kvq_append + kvq_decode_attn),
the measured copy and read-only bandwidths, the prefill-append throughput (64 x 2048 tokens, with and
without rotation) and the CPU oracle's rate on a bounded sample.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from bit_kv_cache_02_amd import kvq, profsum, workloads as wl  # noqa: E402

HBM_PEAK_GBPS = 8000.0
PAGE_HEAD = 2176



def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_step_bytes(w, lens, out_bytes=2):
    kv = int(sum(lens)) * w.num_kv_heads * 136
    q = w.batch * w.num_q_heads * 128 * 2
    out = w.batch * w.num_q_heads * 128 * out_bytes
    bt = int(sum(-(-int(n) // 16) for n in lens)) * 4 + w.batch * 4
    return kv + q + out + bt


TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "e4m3": torch.float8_e4m3fn}


def append_bytes(n_tokens, hkv, in_bytes=2):
    return n_tokens * hkv * (2 * 128 * in_bytes + 2 * 68) + n_tokens * 4


def build_layers(w, n_layers, dev):
    """Prefill n_layers caches with the workload's 4095 cached tokens per sequence (on the GPU)."""
    lens = wl.seq_lens(w)
    table, num_pages = wl.block_table(w, lens)
    data = wl.decode_step_inputs(w)
    kdt, qdt = TORCH_DT[w.kv_dtype], TORCH_DT[w.q_dtype]
    k = torch.from_numpy(np.concatenate(data["prefix_k"])).to(kdt).to(dev)
    v = torch.from_numpy(np.concatenate(data["prefix_v"])).to(kdt).to(dev)
    pre = lens - 1
    cu = torch.tensor(np.concatenate([[0], np.cumsum(pre)]), dtype=torch.int32, device=dev)
    start0 = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    bt = torch.from_numpy(table).to(dev)
    caches = []
    for _ in range(n_layers):
        c = kvq.Cache(num_pages, w.num_kv_heads, w.had_block, device=dev)
        kvq.append(c, k, v, cu, start0, bt, int(pre.max()))
        caches.append(c)
    torch.cuda.synchronize()
    del k, v
    step = {
        "k": torch.from_numpy(data["new_k"]).to(kdt).to(dev),
        "v": torch.from_numpy(data["new_v"]).to(kdt).to(dev),
        "cu": torch.arange(w.batch + 1, dtype=torch.int32, device=dev),
        "start": torch.from_numpy(pre.astype(np.int32)).to(dev),
        "q": torch.from_numpy(wl.queries(w)).to(qdt).to(dev),
        "lens": torch.from_numpy(lens.astype(np.int32)).to(dev),
        "bt": bt,
    }
    return caches, step, lens, table


def time_two_call_steps(w, caches, step, lens, steps, warmup):
    """The step as two launches (kvq_append, kvq_decode_attn), eager; per-launch event times."""
    dev = step["q"].device
    max_len = int(lens.max())
    ws = kvq.make_workspace(caches[0], w.num_q_heads, w.batch, max_len, dev)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps + warmup)]
    for i in range(steps + warmup):
        c = caches[i % len(caches)]
        ev[i][0].record()
        kvq.append(c, step["k"], step["v"], step["cu"], step["start"], step["bt"], 1)
        ev[i][1].record()
        kvq.decode_attn(c, step["q"], step["lens"], step["bt"], max_len, out=out, workspace=ws)
        ev[i][2].record()
    torch.cuda.synchronize()
    app = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(warmup, warmup + steps)]) * 1e3
    dec = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(warmup, warmup + steps)]) * 1e3
    # decode launches back to back: average launch duration over the region
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        kvq.decode_attn(caches[i % len(caches)], step["q"], step["lens"], step["bt"], max_len, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    return app, dec, e0.elapsed_time(e1) * 1e3 / steps


def step_graphs(w, caches, step, lens, steps):
    """HIP graphs of kvq_decode_step launches cycling over the layer caches: one of
    chunk = min(steps, 64) launches and, when steps is not a multiple of it, one of the remainder,
    so that a timed run of `steps` launches is whole graph replays with every kernel launched back
    to back inside them."""
    dev = step["q"].device
    max_len = int(lens.max())
    ws = kvq.make_workspace(caches[0], w.num_q_heads, w.batch, max_len, dev)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    n_layers = len(caches)

    def launches(first, count):
        for i in range(first, first + count):
            kvq.decode_step(caches[i % n_layers], step["k"], step["v"], step["q"], step["lens"], step["bt"],
                            max_len, out=out, workspace=ws)

    chunk = max(1, min(steps, 64))
    rem = steps % chunk
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launches(0, n_layers)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    main = torch.cuda.CUDAGraph()
    with torch.cuda.graph(main):
        launches(0, chunk)
    tail = None
    if rem:
        tail = torch.cuda.CUDAGraph()
        with torch.cuda.graph(tail):
            launches(chunk, rem)
    torch.cuda.synchronize()
    return main, chunk, tail, rem


def time_graph_steps(main, chunk, tail, rem, steps, warmup):
    """Exactly `steps` launches: steps // chunk replays of the main graph, then the remainder
    graph.  Every graph is replayed before timing (its first replay uploads it), the clocks settle
    for ~0.3 s, at least `warmup` launches run untimed, and the timed sequence itself (events,
    replays, synchronization) runs once untimed: the first pass through it costs the host ~15 us
    more by the wall clock (measured: 27.3-27.8 us per step at 20 steps against 26.5-27.1 for the
    passes after it, the same by the events).  Returns the wall time and the launch stream's event
    time per launch over the timed region."""
    def run():
        for _ in range(steps // chunk):
            main.replay()
        if tail is not None:
            tail.replay()

    def timed():
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) * 1e3 / steps

    main.replay()
    if tail is not None:
        tail.replay()
    torch.cuda.synchronize()
    settle(main.replay)
    for _ in range(-(-warmup // chunk)):
        main.replay()
    timed()  # untimed pass through the timed sequence
    return timed()


def settle(fn, seconds=0.3):
    """Run fn (GPU work) repeatedly for about `seconds`, so that clocks have settled after the
    host-side input generation that precedes each workload before anything is timed."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()


def time_tiny_step(dev, replays=400):
    """Tiny workload: 1 sequence, 4 q / 1 kv head, fp16, Hadamard block 64; a step appends the
    256th token and attends all 256 (kvq_decode_step), captured in a HIP graph and replayed.
    Latency-bound: the 35 KB cache is far below any bandwidth scale."""
    w = wl.WORKLOADS["tiny"]
    caches, step, lens, _ = build_layers(w, 1, dev)
    max_len = int(lens.max())
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=dev)
    ws = kvq.make_workspace(caches[0], w.num_q_heads, w.batch, max_len, dev)

    def one():
        kvq.decode_step(caches[0], step["k"], step["v"], step["q"], step["lens"], step["bt"], max_len, out=out,
                        out_dtype=torch.float32, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(10):
            one()
    settle(g.replay)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays // 10):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays // 10 * 10)
    nbytes = decode_step_bytes(w, lens, out_bytes=4) + append_bytes(w.batch, w.num_kv_heads)
    del g, caches, step
    return {"workload": "1 sequence, context 256 (255 cached + the appended token), 4 q / 1 kv head, fp16 "
                        "K/V/q, Hadamard block 64, fp32 out; kvq_decode_step in a HIP graph (10 per replay)",
            "us_per_step": round(us, 3), "algorithmic_bytes": nbytes}


def time_long_decode(dev, replays=25):
    """Long/ragged decode: 8 sequences with contexts ~ U{1024..32768}, 32 q / 8 kv heads,
    Hadamard block 64, over a permuted shared page pool; kvq_decode_attn (decode kernel plus the
    merge of split runs) on each of 8 layer caches in turn, captured in one HIP graph and replayed,
    so host launch gaps are not timed."""
    w = wl.WORKLOADS["long"]
    caches, step, lens, _ = build_layers(w, 8, dev)
    max_len = int(lens.max())
    dbytes = decode_step_bytes(w, lens)
    ws = kvq.make_workspace(caches[0], w.num_q_heads, w.batch, max_len, dev)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.bfloat16, device=dev)

    def all_layers():
        for c in caches:
            kvq.decode_attn(c, step["q"], step["lens"], step["bt"], max_len, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        all_layers()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        all_layers()
    settle(g.replay)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays * len(caches))
    gbps = dbytes / us / 1e3
    res = {"workload": "batch 8, contexts U{1024..32768} (seeded), 32 q / 8 kv heads, INT4, Hadamard block 64, "
                       "permuted shared pool, 8 layer caches in one HIP graph",
           "sum_context": int(lens.sum()), "max_context": max_len, "us_per_decode": round(us, 3),
           "algorithmic_bytes": dbytes, "GBps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    del g, caches, step
    torch.cuda.empty_cache()
    return res


def time_mxfp4_decode(dev, repeats=40):
    """MXFP4 decode, 64 x 16K contexts, 64 q / 8 kv heads, fp8 e4m3 queries, over 2 alternating
    pools (2.3 GB, beyond the Infinity Cache): both contractions on f16 tiles vs both on the scaled
    FP8 x FP4 MFMA (FP8 queries, FP8-quantized attention weights)."""
    from concurrent.futures import ThreadPoolExecutor
    w = wl.WORKLOADS["mxfp4"]
    lens = wl.seq_lens(w)
    table, num_pages = wl.block_table(w, lens)
    bt = torch.from_numpy(table).to(dev)
    caches = [kvq.Cache(num_pages, w.num_kv_heads, w.had_block, "mxfp4", device=dev) for _ in range(2)]
    zeros = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    with ThreadPoolExecutor(8) as ex:
        for b0 in range(0, w.batch, 8):
            seqs = list(ex.map(lambda b: wl.sequence_kv(w, b, int(lens[b])), range(b0, b0 + 8)))
            cnt = np.zeros(w.batch, np.int64)
            cnt[b0:b0 + 8] = lens[b0:b0 + 8]
            cu = torch.from_numpy(np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)).to(dev)
            k = torch.from_numpy(np.concatenate([x[0] for x in seqs])).to(torch.bfloat16).to(dev)
            v = torch.from_numpy(np.concatenate([x[1] for x in seqs])).to(torch.bfloat16).to(dev)
            kvq.append(caches[0], k, v, cu, zeros, bt, int(lens.max()))
            del seqs, k, v
    caches[1].pool.copy_(caches[0].pool)
    q = torch.from_numpy(wl.queries(w)).to(torch.float8_e4m3fn).to(dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    max_len = int(lens.max())
    ws = kvq.make_workspace(caches[0], w.num_q_heads, w.batch, max_len, dev)
    # each path as a HIP graph of 8 launches alternating the pools (as a serving loop would replay
    # a step), so that the launch gaps of eager calls stay out of the kernel's time
    def launches(scaled):
        for i in range(8):
            kvq.decode_attn(caches[i % 2], q, sl, bt, max_len, out=out, workspace=ws, scaled_mfma=scaled)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launches(False)
        launches(True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    for scaled in (False, True):
        graphs[scaled] = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graphs[scaled]):
            launches(scaled)
        graphs[scaled].replay()
    torch.cuda.synchronize()
    settle(graphs[False].replay)
    times = {False: [], True: []}
    replays = max(1, repeats // 8)
    for scaled in (False, True, False, True):
        graphs[scaled].replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            graphs[scaled].replay()
        e1.record()
        torch.cuda.synchronize()
        times[scaled].append(e0.elapsed_time(e1) * 1e3 / (8 * replays))
    del graphs
    nbytes = int(lens.sum()) * w.num_kv_heads * 136 + w.batch * w.num_q_heads * 128 * 3 + \
        int(sum(-(-int(n) // 16) for n in lens)) * 4 + w.batch * 4
    f16_us, sc_us = float(np.mean(times[False])), float(np.mean(times[True]))
    # its page stream without the arithmetic, in its plan (4 waves, depth 3, 256-page splits)
    pat_us = time_decode_pattern([c.pool for c in caches], w.num_kv_heads, bt, int(lens[0]) // 16, 4, 3, 256,
                                 launches=8, repeats=repeats)
    del caches
    return {
        "workload": "MXFP4 decode: 64 seqs x context 16384, 64 q / 8 kv heads, fp8 e4m3 queries, e2m1 + "
                    "UE8M0/32 after the Hadamard 128 rotation, bf16 out; 2 pools alternated, HIP graphs of "
                    "8 launches",
        "us_f16_tiles": round(f16_us, 2),
        "us_scaled_mfma": round(sc_us, 2),
        "GBps": round(nbytes / f16_us / 1e3, 1),
        "frac_of_hbm_peak": round(nbytes / f16_us / 1e3 / HBM_PEAK_GBPS, 4),
        "GBps_scaled_mfma": round(nbytes / sc_us / 1e3, 1),
        "algorithmic_bytes": nbytes,
        "us_access_pattern_probe": round(pat_us, 2),
        "frac_of_access_pattern_probe": round(pat_us / f16_us, 4),
    }


def time_prefill_append(dev, repeats=10):
    """64 x 2048 heavy-tailed bf16 tokens into 2 alternating pools; rotation b=128 vs none."""
    w = wl.WORKLOADS["prefill"]
    lens = wl.seq_lens(w)
    table, num_pages = wl.block_table(w, lens)
    ks, vs = [], []
    for b in range(w.batch):
        k, v = wl.sequence_kv(w, b, int(lens[b]))
        ks.append(torch.from_numpy(k).to(torch.bfloat16))
        vs.append(torch.from_numpy(v).to(torch.bfloat16))
    k = torch.cat(ks).to(dev)
    v = torch.cat(vs).to(dev)
    del ks, vs
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    start = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    bt = torch.from_numpy(table).to(dev)
    res = {}
    quats = {"quat_fast": torch.from_numpy(wl.unit_quaternions(w.seed, False)).to(dev),
             "quat_full": torch.from_numpy(wl.unit_quaternions(w.seed, True)).to(dev)}
    for hb in (128, 64, 1, "quat_fast", "quat_full"):
        if isinstance(hb, str):
            pools = [kvq.Cache(num_pages, w.num_kv_heads, kvq.ROT_QUAT4, device=dev, quat=quats[hb])
                     for _ in range(2)]
        else:
            pools = [kvq.Cache(num_pages, w.num_kv_heads, hb, device=dev) for _ in range(2)]
        for c in pools:
            kvq.append(c, k, v, cu, start, bt, int(lens.max()))
        settle(lambda: kvq.append(pools[0], k, v, cu, start, bt, int(lens.max())), 0.1)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(repeats)]
        for i in range(repeats):
            evs[i][0].record()
            kvq.append(pools[i % 2], k, v, cu, start, bt, int(lens.max()))
            evs[i][1].record()
        torch.cuda.synchronize()
        res[hb] = float(np.median([a.elapsed_time(b) for a, b in evs]) * 1e3)
        del pools
    # the same traffic without the arithmetic (kvq_hbm_append_pattern), into the same kind of pools:
    # in the append's order, and one workgroup per page, on this workload's scattered pages and on
    # the same pages in order
    pools = [torch.empty((num_pages, w.num_kv_heads, PAGE_HEAD), dtype=torch.uint8, device=dev) for _ in range(2)]
    new_tokens = int(lens[0])
    bt_inorder = torch.arange(w.batch * table.shape[1], dtype=torch.int32, device=dev).reshape(table.shape)
    bt_inorder = torch.minimum(bt_inorder, torch.tensor(num_pages - 1, dtype=torch.int32, device=dev))
    # and the workload's own scattered pages written in increasing id (order 2: the list of
    # (sequence, page) items sorted by the page each goes to; the rows are then read out of order).
    # The workload's pages are 0 .. num_pages - 1, so page i of that order is the item's own page.
    npg = new_tokens // 16
    touched = table[:, :npg].reshape(-1)
    assert np.array_equal(np.sort(touched), np.arange(num_pages)), "the prefill pages must be 0 .. num_pages - 1"
    by_page = torch.from_numpy(np.argsort(touched, kind="stable").astype(np.int32).reshape(w.batch, npg)).to(dev)
    pattern_us = {}
    for name, order, tbl in (("own", 0, bt), ("page", 1, bt), ("page_in_order", 1, bt_inorder),
                             ("page_by_id", 2, by_page)):
        settle(lambda: kvq.hbm_append_pattern(k, v, tbl, pools[0], new_tokens, order), 0.1)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(repeats)]
        for i in range(repeats):
            evs[i][0].record()
            kvq.hbm_append_pattern(k, v, tbl, pools[i % 2], new_tokens, order)
            evs[i][1].record()
        torch.cuda.synchronize()
        pattern_us[name] = float(np.median([a.elapsed_time(b) for a, b in evs]) * 1e3)
    del pools
    n_tok = int(lens.sum())
    nbytes = append_bytes(n_tok, w.num_kv_heads)
    return {
        "workload": "prefill append: 64 seqs x 2048 new tokens, 8 kv heads, bf16 Student-t(3), page 16",
        "us_rotated_b128": round(res[128], 2),
        "us_rotated_b64": round(res[64], 2),
        "us_plain_int4": round(res[1], 2),
        "us_isoquant_fast": round(res["quat_fast"], 2),
        "us_isoquant_full": round(res["quat_full"], 2),
        "rotation_overhead_pct": round(100.0 * (res[128] / res[1] - 1.0), 2),
        "GBps": round(nbytes / res[128] / 1e3, 1),
        "tokens_per_s": round(n_tok / res[128] * 1e6, 1),
        "frac_of_hbm_peak": round(nbytes / res[128] / 1e3 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": nbytes,
        "us_access_pattern_probe": round(pattern_us["own"], 2),
        "frac_of_access_pattern_probe": round(pattern_us["own"] / res[128], 4),
        "us_access_pattern_probe_page_major": round(pattern_us["page"], 2),
        "us_access_pattern_probe_page_major_pages_in_order": round(pattern_us["page_in_order"], 2),
        "us_access_pattern_probe_page_major_written_by_page_id": round(pattern_us["page_by_id"], 2),
    }


def time_prefill_attention(w, caches, lens, dev, chunk=512, repeats=20):
    """Chunked-prefill attention on the layer caches: every sequence's last `chunk` positions
    (a new turn over the resident prefix) attend causally, 32 q / 8 kv heads."""
    b = w.batch
    gen = torch.Generator().manual_seed(7)
    q = torch.randn((b * chunk, w.num_q_heads, 128), generator=gen).to(torch.bfloat16).to(dev)
    cu_q = torch.arange(0, b * chunk + 1, chunk, dtype=torch.int32, device=dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    table, _ = wl.block_table(w, lens)
    bt = torch.from_numpy(table).to(dev)
    out = torch.empty((b * chunk, w.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    max_len = int(lens.max())
    for i in range(3):
        kvq.prefill_attn(caches[i % len(caches)], q, cu_q, sl, bt, max_len, chunk, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(repeats):
        kvq.prefill_attn(caches[i % len(caches)], q, cu_q, sl, bt, max_len, chunk, out=out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / repeats
    # scores and p.V: 2 x 2 x 128 flop per (query row, attended position)
    attended = sum(int(L) - chunk + j + 1 for L in lens for j in range(chunk))
    flops = 4 * 128 * attended * w.num_q_heads
    kv_bytes = int(sum(lens)) * w.num_kv_heads * 136
    tflops = flops / us / 1e6
    return {
        "workload": f"chunked prefill: {b} seqs x {chunk}-token chunk over a {int(lens[0]) - chunk}-token "
                    f"resident prefix, 32 q / 8 kv heads, INT4, Hadamard 128 (layer caches of the decode bench)",
        "us": round(us, 2),
        "tokens_per_s": round(b * chunk / us * 1e6, 1),
        "TFLOPs": round(tflops, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None},
        "algorithmic_flops": flops,
        "kv_bytes_once": kv_bytes,
    }


def hbm_copy_probe(dev, nbytes=1 << 30, repeats=10):
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    settle(lambda: kvq.hbm_copy(src, dst))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(repeats):
        kvq.hbm_copy(src, dst)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / repeats
    return 2 * nbytes / us / 1e3


def hbm_fold4_probe(dev, out_bytes=1 << 28, repeats=10):
    """The 4:1 read:write probe (kvq_hbm_fold4): 1 GiB read and 256 MiB written per launch;
    GB/s of bytes moved (read + written)."""
    src = torch.empty(4 * out_bytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(out_bytes, dtype=torch.uint8, device=dev)
    settle(lambda: kvq.hbm_fold4(src, dst))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(repeats):
        kvq.hbm_fold4(src, dst)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / repeats
    return 5 * out_bytes / us / 1e3


def time_dequant(cache, dev, n_pages=1024, repeats=20):
    """kvq_dequant_page over n_pages seeded pages of a llama layer cache (all 8 kv heads), plain
    and rotated back: each page-head reads its 2176-byte block and writes K and V as fp32 16 x 128
    (2 x 8 KiB), so the call is bound by its writes."""
    ids = torch.from_numpy(np.random.default_rng(11).permutation(cache.num_pages)[:n_pages].astype(np.int32)).to(dev)
    nbytes = n_pages * cache.num_kv_heads * (PAGE_HEAD + 2 * 16 * 128 * 4) + n_pages * 4
    res = {"workload": f"{n_pages} pages x {cache.num_kv_heads} kv heads of a llama layer cache (INT4, Hadamard "
                       f"{cache.had_block}) to fp32 K and V", "algorithmic_bytes": nbytes}
    for name, unrot in (("plain", False), ("unrotated", True)):
        settle(lambda: kvq.dequant_pages(cache, ids, unrotate=unrot))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(repeats):
            kvq.dequant_pages(cache, ids, unrotate=unrot)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / repeats
        res[f"us_{name}"] = round(us, 2)
        res[f"GBps_{name}"] = round(nbytes / us / 1e3, 1)
        res[f"frac_of_hbm_peak_{name}"] = round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)
    return res


def hbm_read_probe(dev, window=1 << 30, buf_bytes=1 << 30, repeats=20):
    """Read-only probe: GB/s of one launch over `window` bytes; launches cycle over the
    windows of a 1 GiB buffer, so that windows smaller than the 256 MB MALL are not re-read
    from it."""
    window -= window % 16
    src = torch.empty(buf_bytes, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.zeros(kvq.HBM_READ_SINK_WORDS, dtype=torch.int32, device=dev)
    views = [src[k * window:(k + 1) * window] for k in range(buf_bytes // window)]
    for v in views:
        kvq.hbm_read(v, sink)
    torch.cuda.synchronize()
    # one HIP graph holds a launch per window (as the decode step is timed: graph replays)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for v in views:
            kvq.hbm_read(v, sink)
    replays = max(1, -(-repeats // len(views)))
    settle(g.replay)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays * len(views))
    return window / us / 1e3


def time_decode_pattern(pools, hkv, bt, pages_per_seq, waves, depth, pages_per_split, launches=8, repeats=40):
    """The decode's page stream without its arithmetic (kvq_hbm_decode_pattern) on the same pools
    and block table, in the decode's plan: us per launch, launches cycling over the pools in a
    HIP graph of `launches` (as the decode legs are timed)."""
    sink = kvq.hbm_decode_pattern(pools[0], hkv, bt, pages_per_seq, waves, depth, pages_per_split)
    torch.cuda.synchronize()

    def run():
        for i in range(launches):
            kvq.hbm_decode_pattern(pools[i % len(pools)], hkv, bt, pages_per_seq, waves, depth, pages_per_split, sink)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    settle(g.replay)
    replays = max(1, -(-repeats // launches))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (replays * launches)


def cpu_baseline(w, budget_s=12.0, n_seqs=4):
    """The oracle's decode step (append the new token + decode attention) on a sample of
    n_seqs whole sequences of the same workload, repeated until budget_s of CPU time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    seqs = list(range(n_seqs))
    data = wl.decode_step_inputs(w, seqs=seqs)
    lens = data["lens"][:n_seqs]
    sub = wl.small_variant(w, n_seqs, int(lens[0]))
    table, num_pages = wl.block_table(sub, lens)
    pool = np.zeros((num_pages, w.num_kv_heads, PAGE_HEAD), np.uint8)
    pre = lens - 1
    oracle.append(pool, np.concatenate([data["prefix_k"][b] for b in seqs]),
                  np.concatenate([data["prefix_v"][b] for b in seqs]),
                  np.concatenate([[0], np.cumsum(pre)]), np.zeros(n_seqs, np.int64), table, w.had_block)
    q = wl.queries(w)[:n_seqs]
    nk = data["new_k"][:n_seqs]
    nv = data["new_v"][:n_seqs]
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.append(pool, nk, nv, np.arange(n_seqs + 1), pre, table, w.had_block)
        oracle.decode_attention(pool, q, lens, table, w.had_block)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    sub_bytes = decode_step_bytes(sub, lens) + append_bytes(n_seqs, w.num_kv_heads)
    return {
        "value": round(sub_bytes * reps / el / 1e9, 5),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{n_seqs} of {w.batch} sequences (all 32 q / 8 kv heads, context 4096), "
                  f"append of the step token + decode attention, repeated {reps}x in {el:.1f} s; "
                  f"host os.cpu_count()={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}, "
                  f"BLAS threads={blas_threads}",
    }


def cpu_per_workload(budget_s=2.0):
    """The oracle, as it stands, on one sequence of each other workload (the tiny one has only
    one): a decode step (append of the step's token + decode attention) or, for the prefill
    workload, the append of one sequence's new tokens; each repeated for about budget_s.
    Context for the GPU figures, not a target."""
    import oracle

    def run(fn):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        return (time.perf_counter() - t0) / reps, reps

    res = {}
    for name in ("tiny", "long", "mxfp4"):
        w = wl.WORKLOADS[name]
        fmt = oracle.FMT_MXFP4 if w.fmt == "mxfp4" else oracle.FMT_INT4
        data = wl.decode_step_inputs(w, seqs=[0])
        L = int(data["lens"][0])
        lens = np.array([L])
        table, num_pages = wl.block_table(wl.small_variant(w, 1, L), lens)
        pool = np.zeros((num_pages, w.num_kv_heads, PAGE_HEAD), np.uint8)
        oracle.append(pool, data["prefix_k"][0], data["prefix_v"][0], np.array([0, L - 1]), np.zeros(1, np.int64),
                      table, w.had_block, fmt)
        q = wl.queries(w)[:1]
        nk, nv = data["new_k"][:1], data["new_v"][:1]

        def step():
            oracle.append(pool, nk, nv, np.array([0, 1]), np.array([L - 1]), table, w.had_block, fmt)
            oracle.decode_attention(pool, q, lens, table, w.had_block, fmt)

        sec, reps = run(step)
        res[name] = {"sample": f"sequence 0 of {w.batch} (context {L}): append of its step token + decode "
                               f"attention, {reps}x", "s_per_sequence_step": round(sec, 5),
                     "s_per_step_all_sequences_est": round(sec * w.batch, 4) if name != "tiny" else round(sec, 5)}
    w = wl.WORKLOADS["prefill"]
    n = int(wl.seq_lens(w)[0])
    k, v = wl.sequence_kv(w, 0, n)
    table, num_pages = wl.block_table(wl.small_variant(w, 1, n), np.array([n]))
    pool = np.zeros((num_pages, w.num_kv_heads, PAGE_HEAD), np.uint8)
    sec, reps = run(lambda: oracle.append(pool, k, v, np.array([0, n]), np.zeros(1, np.int64), table, w.had_block))
    res["prefill"] = {"sample": f"sequence 0 of {w.batch}: append of its {n} new tokens, {reps}x",
                      "tokens_per_s": round(n / sec, 1)}
    return res


def profile_record(leg):
    """The committed rocprofv3 record of a leg's kernel (profiles/<leg>_traffic.json), if the
    kernel's code has not changed since it was taken (else None)."""
    _, _, src, key, _ = profsum.LEGS[leg]
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", f"{leg}_traffic.json")))
        if rec.get(key) != profsum.code_sha256(src):
            return None
        return rec
    except (OSError, ValueError):
        return None


def traffic_entry(leg):
    """HBM bytes per launch from committed rocprofv3 counter runs (FETCH_SIZE + WRITE_SIZE, each
    scaled by what the counter reads for the bench's 1 GiB copy), if the kernel's code has not
    changed since they were taken."""
    rec = profile_record(leg)
    try:
        return None if rec is None else int(rec["hbm_bytes_per_launch"])
    except (KeyError, TypeError, ValueError):
        return None


def trace_avg_us(leg):
    """The kernel's average duration in the committed rocprofv3 kernel trace of bench.py
    --profile-run, if the kernel's code has not changed since (else None)."""
    rec = profile_record(leg)
    try:
        return None if rec is None else float(rec["kernel_trace_avg_us"])
    except (KeyError, TypeError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=800)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-mxfp4", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--profile-run", action="store_true",
                    help="run for rocprofv3: the fused steps as timed by default, the copy and read "
                         "probes, short page-dequantization legs, three prefill appends, short "
                         "long/ragged, tiny and MXFP4 legs; no two-launch step and no CPU leg")
    args = ap.parse_args()
    if args.profile_run:
        args.no_cpu = True
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    kvq.lib()
    w = wl.WORKLOADS["llama"]
    log("[bench] building 8 layer caches (llama shape)")
    caches, step, lens, _ = build_layers(w, args.layers, dev)
    dbytes = decode_step_bytes(w, lens)
    abytes = append_bytes(w.batch, w.num_kv_heads)
    step_bytes = dbytes + abytes
    res = {}
    # a few milliseconds of the step first, so that clocks have settled before anything is timed
    for i in range(256):
        kvq.decode_step(caches[i % len(caches)], step["k"], step["v"], step["q"], step["lens"], step["bt"],
                        int(lens.max()))
    torch.cuda.synchronize()
    if not args.profile_run:
        log("[bench] two-launch step (kvq_append + kvq_decode_attn)")
        app_us, dec_us, dec_avg_us = time_two_call_steps(w, caches, step, lens, min(args.steps, 200), 20)
        res["two_launch_step"] = {
            "append_us": round(float(app_us.mean()), 3),
            "decode_us": round(float(dec_us.mean()), 3),
            "decode_back_to_back_avg_us": round(dec_avg_us, 3),
            "decode_GBps": round(dbytes / dec_avg_us / 1e3, 1),
            "decode_frac_of_hbm_peak": round(dbytes / dec_avg_us / 1e3 / HBM_PEAK_GBPS, 4),
        }
    log("[bench] capturing the fused step into HIP graphs")
    graphs = step_graphs(w, caches, step, lens, args.steps)
    log("[bench] timing fused steps")
    wall, step_us = time_graph_steps(*graphs, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / step_us / 1e3
    from bit_kv_cache_02_amd.kvq import decode_workspace_bytes
    res = {
        "metric": "INT4-KV append GB/s + paged INT4 decode-attn us/step, % of HBM peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic (seeded; K ~ N(0,1) with 3 outlier channels x15 per kv head, V ~ N(0,0.5), q ~ N(0,1), bf16)",
        "config": {
            "workload": "Llama-3-8B layer decode step: batch 32 x context 4096, 32 q / 8 kv heads, "
                        "head_dim 128, page 16, bf16 K/V/q, token-wise INT4 (fp16 scale+zero), Hadamard "
                        "block 128; append 1 token per sequence + decode attention in one launch "
                        "(kvq_decode_step), HIP graphs of up to 64 launches; 8 layer caches cycled",
            "batch": w.batch, "context": int(lens[0]), "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads, "had_block": w.had_block, "layers_cycled": args.layers,
            "out_dtype": "bf16",
        },
        "step_us": round(step_us, 3),
        "step_GBps": round(achieved, 1),
        "step_frac_of_hbm_peak": round(achieved / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(w.batch / (ms_per_step * 1e-3), 1),
        "algorithmic_bytes": {"decode": dbytes, "append": abytes, "step": step_bytes},
        "decode_workspace_bytes": decode_workspace_bytes(caches[0], w.num_q_heads, w.batch, int(lens.max())),
        "roofline": {
            "bound": "hbm",
            "kernel": "kvq::decode_kernel<0, 8, 3, 1> (kvq_decode_step: append + decode attention, INT4)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_entry("decode_step_llama"),
            "launch_us_events": round(step_us, 3),
            "launch_us_kernel_trace": trace_avg_us("decode_step_llama"),
        },
        **res,
    }
    del graphs
    if not args.no_prefill:
        log("[bench] chunked-prefill attention")
        res["prefill_attention"] = time_prefill_attention(w, caches, lens, dev)
        res["prefill_attention"]["roofline"]["traffic"] = traffic_entry("prefill_attention")
        res["prefill_attention"]["us_kernel_trace"] = trace_avg_us("prefill_attention")
    log("[bench] HBM copy probe")
    res["hbm_copy_GBps"] = round(hbm_copy_probe(dev), 1)
    res["step_frac_of_copy_bw"] = round(achieved / res["hbm_copy_GBps"], 4)
    log("[bench] HBM read probe")
    res["hbm_read_GBps"] = round(hbm_read_probe(dev), 1)
    res["step_frac_of_read_bw"] = round(achieved / res["hbm_read_GBps"], 4)
    # the same probe at one step's byte count per launch (its launch and drain included)
    res["hbm_read_GBps_at_step_bytes"] = round(hbm_read_probe(dev, window=step_bytes, repeats=56), 1)
    res["step_frac_of_read_bw_at_step_bytes"] = round(achieved / res["hbm_read_GBps_at_step_bytes"], 4)
    # the step's page stream without its arithmetic, in the step's plan (8 waves, depth 3, one split)
    log("[bench] decode access-pattern probe")
    pat_us = time_decode_pattern([c.pool for c in caches], w.num_kv_heads, step["bt"], int(lens[0]) // 16, 8, 3, 512,
                                 launches=len(caches), repeats=56)
    page_bytes = int(lens.sum()) * w.num_kv_heads * 136
    res["decode_pattern_probe"] = {"us": round(pat_us, 3), "GBps": round(page_bytes / pat_us / 1e3, 1),
                                   "step_frac_of_probe": round(pat_us / step_us, 4)}
    log("[bench] HBM 4:1 read:write probe")
    res["hbm_fold4_GBps"] = round(hbm_fold4_probe(dev), 1)
    log("[bench] page dequantization")
    res["dequant_pages"] = time_dequant(caches[0], dev, repeats=5 if args.profile_run else 20)
    res["dequant_pages"]["traffic_plain"] = traffic_entry("dequant_plain")
    res["dequant_pages"]["traffic_unrotated"] = traffic_entry("dequant_rotated")
    del caches
    torch.cuda.empty_cache()
    if not args.no_prefill:
        log("[bench] prefill append")
        res["prefill_append"] = time_prefill_append(dev, repeats=3 if args.profile_run else 10)
        res["prefill_append"]["frac_of_fold4_bw"] = round(res["prefill_append"]["GBps"] / res["hbm_fold4_GBps"], 4)
        res["prefill_append"]["traffic"] = traffic_entry("append_prefill")
        res["prefill_append"]["us_kernel_trace"] = trace_avg_us("append_prefill")
        torch.cuda.empty_cache()
    log("[bench] long/ragged decode")
    res["long_ragged_decode"] = time_long_decode(dev, replays=5 if args.profile_run else 25)
    res["long_ragged_decode"]["traffic"] = traffic_entry("decode_long_ragged")
    res["long_ragged_decode"]["us_kernel_trace"] = trace_avg_us("decode_long_ragged")
    log("[bench] tiny decode step")
    res["tiny_step"] = time_tiny_step(dev, replays=100 if args.profile_run else 400)
    if not args.no_mxfp4:
        log("[bench] MXFP4 decode (f16 tiles and scaled FP8 x FP4 MFMA)")
        res["mxfp4_decode"] = time_mxfp4_decode(dev, repeats=3 if args.profile_run else 40)
        res["mxfp4_decode"]["traffic"] = traffic_entry("decode_mxfp4")
        res["mxfp4_decode"]["us_kernel_trace"] = trace_avg_us("decode_mxfp4")
        res["mxfp4_decode"]["traffic_scaled_mfma"] = traffic_entry("decode_mxfp4_scaled")
        res["mxfp4_decode"]["us_kernel_trace_scaled_mfma"] = trace_avg_us("decode_mxfp4_scaled")
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(w, budget_s=args.cpu_budget)
        log("[bench] CPU oracle on the other workloads")
        res["cpu_baseline"]["per_workload"] = cpu_per_workload()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
