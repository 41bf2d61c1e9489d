"""KVQ_DEBUG_CHECKS: with it set, a call whose device-side tables break the contract (sequence
lengths, cumulative counts, start positions, block-table entries, page ids) is refused with
KVQ_ERR_INVALID_ARG (ValueError in the binding) before its kernels run; valid calls give the
same results as without it.

Every invalid case below stays inside allocated memory (page ids past the descriptor's
num_pages but inside the allocated pool, host hints smaller than the data), so a missed check
could not make a kernel read or write outside its buffers."""
import numpy as np
import pytest
import torch

import oracle
from bit_kv_cache_02_amd import kvq
from tests import parity
from tests.test_gpu_decode import oracle_cache

pytestmark = pytest.mark.gpu


@pytest.fixture
def checks(monkeypatch):
    monkeypatch.setenv("KVQ_DEBUG_CHECKS", "1")


def _setup(extra_pages=4):
    rng = np.random.default_rng(300)
    lens = [40, 17, 300]
    pool, table = oracle_cache(rng, lens, 2, 128, permute=False, extra=extra_pages)  # extra pages last
    # the descriptor declares fewer pages than the tensor holds: ids in [num_pages, allocated)
    # are out of contract yet addressable
    num_pages = int(table.max()) + 1
    full = torch.from_numpy(pool).cuda()
    cache = kvq.Cache(num_pages, 2, 128, pool=full[:num_pages])
    return rng, lens, pool, table, cache, full


def _decode(cache, table, lens, max_len=None, q=None):
    q = torch.randn(len(lens), 8, 128, generator=torch.Generator().manual_seed(0)).bfloat16().cuda() if q is None else q
    return kvq.decode_attn(cache, q, torch.tensor(lens, dtype=torch.int32).cuda(), torch.from_numpy(table).cuda(),
                           int(max(lens)) if max_len is None else max_len)


def test_valid_calls_pass_and_agree(checks):
    print("[checks] valid", flush=True)
    rng, lens, pool, table, cache, _ = _setup()
    q = torch.randn(3, 8, 128, generator=torch.Generator().manual_seed(1)).bfloat16().cuda()
    got = _decode(cache, table, lens, q=q).cpu().numpy()
    ref = oracle.decode_attention(pool, q.float().cpu().numpy(), lens, table, 128)
    assert parity.attn_row_error(got, ref).max() <= parity.ATTN_TOL
    k, v = kvq.dequant_pages(cache, torch.from_numpy(table[0, :3].copy()).cuda())
    assert torch.isfinite(k).all()


def test_decode_rejects_bad_tables(checks):
    print("[checks] decode", flush=True)
    rng, lens, pool, table, cache, _ = _setup()
    # a length above the host hint (the table and pool still cover it)
    with pytest.raises(ValueError, match="seq_lens"):
        _decode(cache, table, lens, max_len=299)
    with pytest.raises(ValueError, match="seq_lens"):
        _decode(cache, table, [40, 0, 300])
    bad = table.copy()
    bad[2, 5] = cache.num_pages  # an attended page past num_pages, inside the allocated pool
    with pytest.raises(ValueError, match="page id"):
        _decode(cache, bad, lens)
    # entries past a sequence's last page are not read, so they are not checked
    ok = table.copy()
    ok[1, 2:] = 10 ** 6
    _decode(cache, ok, lens)


def test_step_rejects_bad_tables(checks):
    print("[checks] step", flush=True)
    rng, lens, pool, table, cache, _ = _setup()
    bad = table.copy()
    bad[0, 2] = cache.num_pages
    kn = torch.zeros(3, 2, 128, dtype=torch.bfloat16).cuda()
    q = torch.zeros(3, 8, 128, dtype=torch.bfloat16).cuda()
    with pytest.raises(ValueError, match="page id"):
        kvq.decode_step(cache, kn, kn, q, torch.tensor(lens, dtype=torch.int32).cuda(), torch.from_numpy(bad).cuda(),
                        300)
    assert torch.equal(cache.pool.cpu(), torch.from_numpy(pool[:cache.num_pages])), "a refused step wrote"


def test_append_rejects_bad_tables(checks):
    print("[checks] append", flush=True)
    rng, lens, pool, table, cache, _ = _setup()
    k = torch.zeros(12, 2, 128, dtype=torch.bfloat16).cuda()
    bt = torch.from_numpy(table).cuda()
    start = torch.tensor([40, 17, 0], dtype=torch.int32).cuda()
    with pytest.raises(ValueError, match="cumulative"):
        kvq.append(cache, k, k, torch.tensor([0, 5, 3, 12], dtype=torch.int32).cuda(), start, bt, 12)
    with pytest.raises(ValueError, match="cumulative"):
        kvq.append(cache, k, k, torch.tensor([0, 5, 9, 13], dtype=torch.int32).cuda(), start, bt, 12)
    # appended positions past the table row (row 0 continues into row 1's entries, in bounds)
    far = torch.tensor([table.shape[1] * 16 - 2, 17, 0], dtype=torch.int32).cuda()
    with pytest.raises(ValueError, match="start_pos"):
        kvq.append(cache, k, k, torch.tensor([0, 4, 8, 12], dtype=torch.int32).cuda(), far, bt, 12)
    bad = table.copy()
    bad[1, 1] = cache.num_pages
    with pytest.raises(ValueError, match="page id"):
        kvq.append(cache, k, k, torch.tensor([0, 4, 8, 12], dtype=torch.int32).cuda(), start,
                   torch.from_numpy(bad).cuda(), 12)
    assert torch.equal(cache.pool.cpu(), torch.from_numpy(pool[:cache.num_pages])), "a refused append wrote"


def test_prefill_and_dequant_reject_bad_tables(checks):
    print("[checks] prefill, dequant", flush=True)
    rng, lens, pool, table, cache, _ = _setup()
    q = torch.zeros(12, 8, 128, dtype=torch.bfloat16).cuda()
    cu = torch.tensor([0, 4, 8, 12], dtype=torch.int32).cuda()
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    bt = torch.from_numpy(table).cuda()
    kvq.prefill_attn(cache, q, cu, sl, bt, 300, 4)
    with pytest.raises(ValueError, match="chunk"):
        kvq.prefill_attn(cache, q, cu, sl, bt, 300, 3)  # chunks of 4 tokens, hint 3
    bad = table.copy()
    bad[2, 10] = cache.num_pages
    with pytest.raises(ValueError, match="page id"):
        kvq.prefill_attn(cache, q, cu, sl, torch.from_numpy(bad).cuda(), 300, 4)
    with pytest.raises(ValueError, match="page id"):
        kvq.dequant_pages(cache, torch.tensor([0, cache.num_pages], dtype=torch.int32).cuda())
