"""The bandwidth probes behind the benchmark's measured-ceiling figures: the copy kernel moves
every byte, and the read-only kernel loads every 16-byte vector once (the XOR of its sink words
is the XOR of all 32-bit words of the source), at sizes with ragged tails of its 8-vector steps
and of its grid."""
import numpy as np
import pytest
import torch

from bit_kv_cache_02_amd import kvq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 48, 4096 + 16, 256 * 8 * 16 * 3 + 32, (64 << 20) + 112])
def test_copy_and_read_probes(nbytes):
    print(f"[probes] {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    dst = torch.zeros_like(src)
    kvq.hbm_copy(src, dst)
    sink = torch.zeros(kvq.HBM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    kvq.hbm_read(src, sink)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), host)
    want = np.bitwise_xor.reduce(host)
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want


def test_read_probe_leaves_unused_sink_words():
    src = torch.ones(1024, dtype=torch.int32, device="cuda")  # 4 KiB: one workgroup
    sink = torch.full((kvq.HBM_READ_SINK_WORDS,), 7, dtype=torch.int32, device="cuda")
    kvq.hbm_read(src, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    assert got[0] == 0  # 1024 ones XOR to 0
    assert (got[1:] == 7).all()


@pytest.mark.parametrize("out_bytes", [4096, 3 * 4096, 4096 * 2049, (16 << 20) + 4096 * 5])
def test_fold4_probe(out_bytes):
    # the 4:1 read:write probe: output vector 256 m + t is the XOR of input vectors
    # 1024 m + t + 256 k, with ragged tails of its two-group steps and of its grid
    print(f"[probes] fold4 {out_bytes} bytes out", flush=True)
    rng = np.random.default_rng(out_bytes)
    host = rng.integers(0, 1 << 32, out_bytes, dtype=np.uint32)  # 4 * out_bytes bytes
    src = torch.from_numpy(host.view(np.int32)).cuda()
    dst = torch.full((out_bytes // 4,), 7, dtype=torch.int32, device="cuda")
    kvq.hbm_fold4(src, dst)
    torch.cuda.synchronize()
    v = host.reshape(-1, 4, 256, 4)  # [group m][k][t][4 words]
    want = v[:, 0] ^ v[:, 1] ^ v[:, 2] ^ v[:, 3]
    assert np.array_equal(dst.cpu().numpy().view(np.uint32).reshape(-1, 256, 4), want)


@pytest.mark.parametrize("hkv,num_seqs,new_tokens", [(1, 1, 16), (2, 3, 80), (8, 2, 512), (3, 1, 64)])
def test_append_pattern_probe(hkv, num_seqs, new_tokens):
    # the append's traffic without its arithmetic: for each (sequence, kv head, K|V, page,
    # slot n, g) the XOR of the row words at bytes 16 g + 64 i, written where the append writes
    # that lane's code piece, its first word where the append writes the slot's parameters
    print(f"[probes] append pattern hkv {hkv} seqs {num_seqs} tokens {new_tokens}", flush=True)
    rng = np.random.default_rng(hkv * 100 + num_seqs * 10 + new_tokens)
    t = num_seqs * new_tokens
    kh = rng.integers(0, 1 << 16, (t, hkv, 128), dtype=np.uint16)
    vh = rng.integers(0, 1 << 16, (t, hkv, 128), dtype=np.uint16)
    pages = new_tokens // 16
    total = num_seqs * pages + 3
    table = rng.permutation(total)[:num_seqs * pages].reshape(num_seqs, pages).astype(np.int32)
    table = np.concatenate([table, np.zeros((num_seqs, 1), np.int32)], axis=1)  # one spare entry
    pools = []
    for order in (0, 1):  # the append's order, one workgroup per page: the same bytes
        pool = torch.full((total, hkv, 2176), 0xA5, dtype=torch.uint8, device="cuda")
        kvq.hbm_append_pattern(torch.from_numpy(kh.view(np.int16)).cuda(), torch.from_numpy(vh.view(np.int16)).cuda(),
                               torch.from_numpy(table).cuda(), pool, new_tokens, order)
        pools.append(pool)
    # order 2 (pages written in increasing id): the list item written to page i is the
    # (sequence, page) whose table entry is i; a table of pages 0 .. num_seqs * pages - 1 in a
    # random order, so that order 1 over that table writes the same bytes
    items = rng.permutation(num_seqs * pages).astype(np.int32)
    table_i = np.zeros((num_seqs, pages + 1), np.int32)
    for i, e in enumerate(items):
        table_i[e // pages, e % pages] = i
    pools_i = []
    for order, tbl in ((1, table_i), (2, items.reshape(num_seqs, pages))):
        pool = torch.full((total, hkv, 2176), 0xA5, dtype=torch.uint8, device="cuda")
        kvq.hbm_append_pattern(torch.from_numpy(kh.view(np.int16)).cuda(), torch.from_numpy(vh.view(np.int16)).cuda(),
                               torch.from_numpy(np.ascontiguousarray(tbl)).cuda(), pool, new_tokens, order)
        pools_i.append(pool)
    torch.cuda.synchronize()
    assert np.array_equal(pools_i[0].cpu().numpy(), pools_i[1].cpu().numpy())
    got = pools[0].cpu().numpy()
    assert np.array_equal(pools[1].cpu().numpy(), got)
    assert np.array_equal(pools_i[0].cpu().numpy(), _append_pattern_want(kh, vh, table_i, num_seqs, pages, hkv, total))
    assert np.array_equal(got, _append_pattern_want(kh, vh, table, num_seqs, pages, hkv, total))


def _append_pattern_want(kh, vh, table, num_seqs, pages, hkv, total):
    want = np.full((total, hkv, 2176), 0xA5, np.uint8)
    for which, src in ((0, kh), (1, vh)):
        rows = src.view(np.uint8).reshape(num_seqs, pages, 16, hkv, 256)  # [b][page][slot][h][byte]
        words = rows.reshape(num_seqs, pages, 16, hkv, 4, 4, 16)  # [..][i (64-byte piece)][g][16 bytes]
        x = words[..., 0, :, :] ^ words[..., 1, :, :] ^ words[..., 2, :, :] ^ words[..., 3, :, :]  # [b][p][n][h][g][16]
        for b in range(num_seqs):
            for j in range(pages):
                blk = want[table[b, j]]  # [h][2176]
                for n in range(16):
                    for g in range(4):
                        off = 64 * n + 16 * g if which == 0 else 1024 + 256 * (n // 4) + 64 * g + 16 * (n % 4)
                        blk[:, off:off + 16] = x[b, j, n, :, g]
                    poff = (2048 if which == 0 else 2112) + 4 * n
                    blk[:, poff:poff + 4] = x[b, j, n, :, 0, :4]
    return want



def test_launch_plan_log(capfd, monkeypatch):
    # KVQ_LOG=1: one line per launching call on stderr, with the plan the library chose
    import oracle
    from tests.test_gpu_decode import oracle_cache
    rng = np.random.default_rng(91)
    pool, table = oracle_cache(rng, [40, 1000], 2, 128)
    cache = kvq.Cache(pool.shape[0], 2, 128, pool=torch.from_numpy(pool).cuda())
    q = torch.randn((2, 8, 128), dtype=torch.bfloat16).cuda()
    lens = torch.tensor([40, 1000], dtype=torch.int32).cuda()
    bt = torch.from_numpy(table).cuda()
    kvq.decode_attn(cache, q, lens, bt, 1000)
    torch.cuda.synchronize()
    assert "kvq:" not in capfd.readouterr().err  # silent by default
    monkeypatch.setenv("KVQ_LOG", "1")
    kvq.decode_attn(cache, q, lens, bt, 1000)
    kvq.dequant_pages(cache, torch.from_numpy(table[0, :2].copy()).cuda(), unrotate=True)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert "kvq: kvq_decode_attn launch: 2 seqs, 8 q / 2 kv heads, max_seq_len 1000, variant 0" in err
    assert "kvq: kvq_dequant_page: 2 pages, 2 kv heads, format 0, had_block 128, rotated back on the matrix cores" in err


def _decode_pattern_want(pool, hkv, table, pages_per_seq, waves, pages_per_split):
    """Per wave, the sum mod 2^32 of the words its lanes load (the probe's definition)."""
    num_seqs = table.shape[0]
    blocks = pool.reshape(pool.shape[0], hkv, 2176)
    nsplit = -(-pages_per_seq // pages_per_split)
    units = num_seqs * hkv
    want = np.zeros(units * nsplit * waves, np.uint64)
    for j in range(units * nsplit):
        split, unit = divmod(j, units)
        b, h = divmod(unit, hkv)
        p0, p1 = split * pages_per_split, min((split + 1) * pages_per_split, pages_per_seq)
        for w in range(waves):
            tot = 0
            for p in range(p0 + w, p1, waves):
                blk = blocks[table[b, p], h].view(np.uint32)
                # K rows and V words once each (64 lanes x 16 bytes), the 16 K / V parameter words
                # of each 64-byte run loaded by four lanes each
                tot += int(blk[:512].sum(dtype=np.uint64)) + 4 * int(blk[512:544].sum(dtype=np.uint64))
            want[waves * j + w] = tot
    return (want & 0xFFFFFFFF).astype(np.uint32)


@pytest.mark.parametrize("hkv,num_seqs,pages,waves,depth,pps", [
    (2, 3, 37, 4, 3, 16), (1, 1, 5, 8, 2, 512), (8, 2, 256, 8, 3, 512), (3, 2, 70, 4, 4, 9), (8, 4, 129, 4, 2, 64)])
def test_decode_pattern_probe(hkv, num_seqs, pages, waves, depth, pps):
    # the decode's page stream without its arithmetic: each wave's sink word is the sum of the
    # words its lanes loaded from the page-head blocks of its pages (permuted pool, ragged splits)
    print(f"[probes] decode pattern hkv {hkv} B {num_seqs} pages {pages} W {waves} D {depth} split {pps}", flush=True)
    rng = np.random.default_rng(1000 * hkv + pages)
    n_pool = num_seqs * pages + 3
    pool_h = rng.integers(0, 256, (n_pool, hkv, 2176), dtype=np.uint8)
    max_pages = pages + 2
    table = np.zeros((num_seqs, max_pages), np.int32)
    table[:, :pages] = rng.permutation(n_pool)[:num_seqs * pages].reshape(num_seqs, pages)
    pool = torch.from_numpy(pool_h).cuda()
    bt = torch.from_numpy(table).cuda()
    sink = kvq.hbm_decode_pattern(pool, hkv, bt, pages, waves, depth, pps)
    torch.cuda.synchronize()
    want = _decode_pattern_want(pool_h, hkv, table, pages, waves, pps)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
