"""The C ABI boundary on the CPU: the library loads, exports every declared symbol, and
rejects invalid arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest
import torch

from bit_kv_cache_02_amd import kvq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvq.h")
FAKE = ctypes.c_void_p(4096)   # non-null, aligned; never dereferenced on these paths

pytestmark = pytest.mark.skipif(not os.path.exists(kvq.LIB_PATH), reason="libkvq.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    names = declared_functions()
    assert names == sorted(n for n, _, _ in kvq.SIGNATURES)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(kvq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_sizes():
    assert kvq.abi_version() == 2
    d = kvq.KvqCacheDesc(0, 8, 128, 16, 128, 0, 10, 4096, None)
    assert kvq.lib().kvq_page_bytes(ctypes.byref(d)) == 8 * 2176
    assert kvq.lib().kvq_page_bytes(None) == 0
    for s in (0, -1, -2, -3, -4, 7):
        assert kvq.lib().kvq_strerror(s)


def _desc(**kw):
    base = dict(format=0, num_kv_heads=2, head_dim=128, page_size=16, had_block=64, quat_full=0,
                num_pages=8, pool=4096, quat=None)
    base.update(kw)
    return kvq.KvqCacheDesc(*[base[f] for f, _ in kvq.KvqCacheDesc._fields_])


def _append(desc, **kw):
    args = dict(k=FAKE, v=FAKE, dt=kvq.BF16, T=4, B=1, cu=FAKE, sp=FAKE, bt=FAKE, mp=4, mx=4)
    args.update(kw)
    return kvq.lib().kvq_append(ctypes.byref(desc), args["k"], args["v"], args["dt"], args["T"],
                                args["B"], args["cu"], args["sp"], args["bt"], args["mp"],
                                args["mx"], None)


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, kvq.KVQ_ERR_UNSUPPORTED),
    ("page_size", 32, kvq.KVQ_ERR_UNSUPPORTED),
    ("had_block", 32, kvq.KVQ_ERR_UNSUPPORTED),
    ("format", 5, kvq.KVQ_ERR_UNSUPPORTED),
    ("num_kv_heads", 0, kvq.KVQ_ERR_INVALID_ARG),
    ("num_pages", 0, kvq.KVQ_ERR_INVALID_ARG),
    ("pool", None, kvq.KVQ_ERR_INVALID_ARG),
    ("pool", 4097, kvq.KVQ_ERR_INVALID_ARG),
    ("quat_full", 1, kvq.KVQ_ERR_INVALID_ARG),       # only with the quaternion rotation
    ("quat", 4096, kvq.KVQ_ERR_INVALID_ARG),         # likewise
    ("had_block", 2, kvq.KVQ_ERR_UNSUPPORTED),
])
def test_append_rejects_bad_cache(field, value, status):
    assert _append(_desc(**{field: value})) == status
    assert kvq.lib().kvq_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(quat=None), kvq.KVQ_ERR_INVALID_ARG),      # had_block 4 needs the quaternions
    (dict(quat=4100), kvq.KVQ_ERR_INVALID_ARG),      # 16-byte aligned
    (dict(quat_full=2), kvq.KVQ_ERR_INVALID_ARG),
])
def test_quaternion_rotation_rejects_bad_cache(kw, status):
    base = dict(had_block=kvq.ROT_QUAT4, quat=8192)
    base.update(kw)
    assert _append(_desc(**base)) == status
    assert _decode(_desc(**base)) == status
    # a valid quaternion cache passes the cache checks (then fails on a NULL argument)
    assert _append(_desc(had_block=kvq.ROT_QUAT4, quat=8192, quat_full=1), k=None) == kvq.KVQ_ERR_INVALID_ARG
    assert _append(_desc(format=1, had_block=kvq.ROT_QUAT4, quat=8192), k=None) == kvq.KVQ_ERR_INVALID_ARG


def test_cache_object_checks_quaternions():
    with pytest.raises(ValueError):
        kvq.Cache(4, 1, kvq.ROT_QUAT4, pool=torch.zeros((4, 1, 2176), dtype=torch.uint8))
    with pytest.raises(ValueError):
        kvq.Cache(4, 1, kvq.ROT_QUAT4, pool=torch.zeros((4, 1, 2176), dtype=torch.uint8),
                  quat=torch.zeros((32, 5)))
    with pytest.raises(ValueError):
        kvq.Cache(4, 1, 64, pool=torch.zeros((4, 1, 2176), dtype=torch.uint8), quat=torch.zeros((32, 4)))


def test_mxfp4_needs_full_rotation():
    assert _append(_desc(format=1, had_block=64)) == kvq.KVQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(cu=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(dt=kvq.F32), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(dt=kvq.FP8_E4M3), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(T=-1), kvq.KVQ_ERR_INVALID_ARG),
    (dict(mp=0), kvq.KVQ_ERR_INVALID_ARG),
    (dict(mx=-2), kvq.KVQ_ERR_INVALID_ARG),
    (dict(k=ctypes.c_void_p(4100)), kvq.KVQ_ERR_INVALID_ARG),
])
def test_append_rejects_bad_args(kw, status):
    assert _append(_desc(), **kw) == status


def test_append_empty_is_a_no_op():
    assert _append(_desc(), T=0) == kvq.KVQ_OK
    assert _append(_desc(), B=0) == kvq.KVQ_OK


def _decode(desc, **kw):
    args = dict(q=FAKE, qdt=kvq.BF16, qs=1.0, hq=8, B=2, sl=FAKE, msl=100, bt=FAKE, mp=8, sm=0.1,
                out=FAKE, odt=kvq.F32, flags=0, ws=FAKE, wsb=1 << 30)
    args.update(kw)
    return kvq.lib().kvq_decode_attn(ctypes.byref(desc), args["q"], args["qdt"], args["qs"],
                                     args["hq"], args["B"], args["sl"], args["msl"], args["bt"],
                                     args["mp"], args["sm"], args["out"], args["odt"],
                                     args["flags"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3), kvq.KVQ_ERR_INVALID_ARG),          # not a multiple of Hkv = 2
    (dict(hq=18), kvq.KVQ_ERR_UNSUPPORTED),         # group 9 > 8
    (dict(msl=129), kvq.KVQ_ERR_INVALID_ARG),       # > max_pages * 16
    (dict(msl=0), kvq.KVQ_ERR_INVALID_ARG),
    (dict(q=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(out=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(odt=kvq.FP8_E4M3), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(qdt=9), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(flags=4), kvq.KVQ_ERR_INVALID_ARG),
    (dict(flags=kvq.MX_SCALED_MFMA), kvq.KVQ_ERR_UNSUPPORTED),  # the scaled FP8 x FP4 path on an INT4 cache
    (dict(sm=float("nan")), kvq.KVQ_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_args(kw, status):
    assert _decode(_desc(), **kw) == status


def _step(desc, **kw):
    args = dict(k=FAKE, v=FAKE, kvdt=kvq.BF16, q=FAKE, qdt=kvq.BF16, qs=1.0, hq=8, B=2, sl=FAKE, msl=100,
                bt=FAKE, mp=8, sm=0.1, out=FAKE, odt=kvq.F32, flags=0, ws=FAKE, wsb=1 << 30)
    args.update(kw)
    return kvq.lib().kvq_decode_step(ctypes.byref(desc), args["k"], args["v"], args["kvdt"], args["q"],
                                     args["qdt"], args["qs"], args["hq"], args["B"], args["sl"], args["msl"],
                                     args["bt"], args["mp"], args["sm"], args["out"], args["odt"],
                                     args["flags"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(v=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(kvdt=kvq.F32), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(kvdt=kvq.FP8_E4M3), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(hq=3), kvq.KVQ_ERR_INVALID_ARG),
    (dict(msl=129), kvq.KVQ_ERR_INVALID_ARG),
    (dict(q=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(odt=kvq.FP8_E4M3), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(flags=kvq.MX_SCALED_MFMA), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(flags=kvq.MX_SCALED_MFMA | 4), kvq.KVQ_ERR_INVALID_ARG),
])
def test_decode_step_rejects_bad_args(kw, status):
    assert _step(_desc(), **kw) == status


def test_decode_step_empty_batch_is_a_no_op():
    assert _step(_desc(), B=0) == kvq.KVQ_OK


def _prefill(desc, **kw):
    args = dict(q=FAKE, qdt=kvq.BF16, qs=1.0, hq=8, T=10, B=2, cu=FAKE, sl=FAKE, msl=100, mq=10, bt=FAKE, mp=8,
                sm=0.1, out=FAKE, odt=kvq.F32, flags=0)
    args.update(kw)
    return kvq.lib().kvq_prefill_attn(ctypes.byref(desc), args["q"], args["qdt"], args["qs"], args["hq"], args["T"],
                                      args["B"], args["cu"], args["sl"], args["msl"], args["mq"], args["bt"],
                                      args["mp"], args["sm"], args["out"], args["odt"], args["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=18), kvq.KVQ_ERR_UNSUPPORTED),         # group 9: above 8
    (dict(hq=3), kvq.KVQ_ERR_INVALID_ARG),
    (dict(cu=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(q=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(msl=129), kvq.KVQ_ERR_INVALID_ARG),       # > max_pages * 16
    (dict(msl=140000, mp=9000), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(msl=131073, mp=8193), kvq.KVQ_ERR_UNSUPPORTED),  # one position past the prefill limit
    (dict(mq=101), kvq.KVQ_ERR_INVALID_ARG),        # chunk longer than the sequence bound
    (dict(T=-1), kvq.KVQ_ERR_INVALID_ARG),
    (dict(odt=kvq.FP8_E4M3), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(flags=8), kvq.KVQ_ERR_INVALID_ARG),
])
def test_prefill_rejects_bad_args(kw, status):
    assert _prefill(_desc(), **kw) == status


def test_prefill_empty_is_a_no_op():
    assert _prefill(_desc(), T=0) == kvq.KVQ_OK
    assert _prefill(_desc(), B=0) == kvq.KVQ_OK


def test_decode_workspace_sizing_and_check():
    # a few long sequences are split over several workgroups and need a workspace
    d = _desc(num_kv_heads=8)
    lib = kvq.lib()
    need = lib.kvq_decode_workspace_bytes(ctypes.byref(d), 32, 2, 32768)
    assert need > 0 and need % 4 == 0
    assert lib.kvq_decode_workspace_bytes(ctypes.byref(d), 3, 2, 32768) == ctypes.c_size_t(-1).value
    # one short page: no split, no workspace
    assert lib.kvq_decode_workspace_bytes(ctypes.byref(d), 32, 1, 16) == 0
    big = _desc(num_kv_heads=8, num_pages=1 << 20)
    assert _decode(big, hq=32, B=2, msl=32768, mp=2048, ws=None) == kvq.KVQ_ERR_WORKSPACE
    assert _decode(big, hq=32, B=2, msl=32768, mp=2048, wsb=need - 1) == kvq.KVQ_ERR_WORKSPACE
    assert _decode(big, hq=32, B=2, msl=32768, mp=2048, ws=ctypes.c_void_p(4096 + 16), wsb=need) \
        == kvq.KVQ_ERR_WORKSPACE


def test_dequant_and_copy_reject_bad_args():
    lib = kvq.lib()
    d = _desc()
    assert lib.kvq_dequant_page(ctypes.byref(d), None, 3, FAKE, FAKE, 0, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_dequant_page(ctypes.byref(d), FAKE, -1, FAKE, FAKE, 0, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_dequant_page(ctypes.byref(d), FAKE, 3, FAKE, FAKE, 2, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_dequant_page(ctypes.byref(d), FAKE, 0, FAKE, FAKE, 0, None) == kvq.KVQ_OK
    assert lib.kvq_hbm_copy(FAKE, FAKE, 17, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hbm_copy(None, FAKE, 16, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hbm_copy(FAKE, FAKE, 0, None) == kvq.KVQ_OK
    assert lib.kvq_hbm_read(FAKE, 17, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hbm_read(None, 16, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hbm_read(FAKE, 16, None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hbm_read(ctypes.c_void_p(4096 + 8), 16, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hbm_read(FAKE, 0, FAKE, None) == kvq.KVQ_OK
    assert lib.kvq_hbm_fold4(FAKE, FAKE, 4096 + 16, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hbm_fold4(None, FAKE, 4096, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hbm_fold4(ctypes.c_void_p(4096 + 8), FAKE, 4096, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hbm_fold4(FAKE, FAKE, 0, None) == kvq.KVQ_OK
    # the append-pattern probe: argument checks (no launch)
    ap = lib.kvq_hbm_append_pattern
    assert ap(None, FAKE, 8, 1, 16, FAKE, 1, FAKE, 0, None) == kvq.KVQ_ERR_INVALID_ARG
    assert ap(FAKE, FAKE, 8, 1, 24, FAKE, 2, FAKE, 0, None) == kvq.KVQ_ERR_INVALID_ARG  # not a multiple of 16
    assert ap(FAKE, FAKE, 8, 1, 48, FAKE, 2, FAKE, 0, None) == kvq.KVQ_ERR_INVALID_ARG  # beyond 16 * max_pages
    assert ap(FAKE, FAKE, 0, 1, 16, FAKE, 1, FAKE, 0, None) == kvq.KVQ_ERR_INVALID_ARG
    assert ap(FAKE, FAKE, 1025, 1, 16, FAKE, 1, FAKE, 0, None) == kvq.KVQ_ERR_INVALID_ARG
    assert ap(ctypes.c_void_p(4096 + 8), FAKE, 8, 1, 16, FAKE, 1, FAKE, 0, None) == kvq.KVQ_ERR_INVALID_ARG
    assert ap(FAKE, FAKE, 8, 0, 16, FAKE, 1, FAKE, 0, None) == kvq.KVQ_OK
    assert ap(FAKE, FAKE, 8, 1, 0, FAKE, 1, FAKE, 0, None) == kvq.KVQ_OK
    assert ap(FAKE, FAKE, 8, 1, 16, FAKE, 1, FAKE, 3, None) == kvq.KVQ_ERR_INVALID_ARG
    assert ap(FAKE, FAKE, 9, 1, 16, FAKE, 1, FAKE, 1, None) == kvq.KVQ_ERR_UNSUPPORTED
    assert ap(FAKE, FAKE, 9, 1, 16, FAKE, 1, FAKE, 2, None) == kvq.KVQ_ERR_UNSUPPORTED
    # order 2 reads block_table as a list of exactly num_seqs * new_tokens / 16 items
    assert ap(FAKE, FAKE, 8, 1, 16, FAKE, 2, FAKE, 2, None) == kvq.KVQ_ERR_INVALID_ARG
    # the decode-pattern probe: argument checks (no launch)
    dp = lib.kvq_hbm_decode_pattern
    assert dp(None, 8, 1, 4, FAKE, 4, 4, 3, 16, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG
    assert dp(FAKE, 8, 1, 4, FAKE, 4, 4, 3, 16, None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert dp(ctypes.c_void_p(4096 + 8), 8, 1, 4, FAKE, 4, 4, 3, 16, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG
    assert dp(FAKE, 0, 1, 4, FAKE, 4, 4, 3, 16, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG
    assert dp(FAKE, 8, 1, 5, FAKE, 4, 4, 3, 16, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG  # beyond max_pages
    assert dp(FAKE, 8, 1, 0, FAKE, 4, 4, 3, 16, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG
    assert dp(FAKE, 8, 1, 4, FAKE, 4, 16, 2, 16, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG  # waves
    assert dp(FAKE, 8, 1, 4, FAKE, 4, 4, 5, 16, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG  # depth
    assert dp(FAKE, 8, 1, 4, FAKE, 4, 4, 3, 257, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG  # split > 64 waves
    assert dp(FAKE, 8, 1, 4, FAKE, 4, 4, 3, 0, FAKE, None) == kvq.KVQ_ERR_INVALID_ARG
    assert dp(FAKE, 8, 0, 4, FAKE, 4, 4, 3, 16, FAKE, None) == kvq.KVQ_OK


def test_python_layer_raises_typed_errors():
    with pytest.raises(NotImplementedError):
        kvq._check(kvq.KVQ_ERR_UNSUPPORTED, "x")
    with pytest.raises(ValueError):
        kvq._check(kvq.KVQ_ERR_INVALID_ARG, "x")
    with pytest.raises(kvq.KvqError):
        kvq._check(kvq.KVQ_ERR_HIP, "x")


def _step_noalloc(desc, **kw):
    args = dict(k=FAKE, v=FAKE, kvdt=kvq.BF16, q=FAKE, qdt=kvq.BF16, qs=1.0, hq=8, B=2, sl=FAKE, msl=100,
                bt=FAKE, mp=8, sm=0.1, out=FAKE, odt=kvq.F32, flags=0)
    args.update(kw)
    return kvq.lib().kvq_decode_step_noalloc(ctypes.byref(desc), args["k"], args["v"], args["kvdt"], args["q"],
                                             args["qdt"], args["qs"], args["hq"], args["B"], args["sl"],
                                             args["msl"], args["bt"], args["mp"], args["sm"], args["out"],
                                             args["odt"], args["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(kvdt=kvq.F32), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(hq=3), kvq.KVQ_ERR_INVALID_ARG),
    (dict(msl=129), kvq.KVQ_ERR_INVALID_ARG),
    (dict(q=None), kvq.KVQ_ERR_INVALID_ARG),
    (dict(flags=kvq.MX_SCALED_MFMA), kvq.KVQ_ERR_UNSUPPORTED),
])
def test_decode_step_noalloc_rejects_bad_args(kw, status):
    assert _step_noalloc(_desc(), **kw) == status


def test_decode_step_noalloc_limits():
    # sizes beyond the fixed scratch are refused on the host, before any HIP call
    lib = kvq.lib()
    big = _desc(num_kv_heads=8, num_pages=1 << 22)
    # 512 sequences x 8 kv heads of 128K tokens: the split partials need more than 16 MiB
    need = lib.kvq_decode_workspace_bytes(ctypes.byref(big), 64, 512, 131072)
    assert need > 16 << 20
    assert _step_noalloc(big, hq=64, B=512, msl=131072, mp=8192) == kvq.KVQ_ERR_WORKSPACE
    assert b"16777216" in lib.kvq_last_error()
    # more (sequence, kv head) pairs than the scratch's counters serve, on a plan that splits
    assert lib.kvq_decode_workspace_bytes(ctypes.byref(big), 8, 2049, 9600) > 0
    assert _step_noalloc(big, hq=8, B=2049, msl=9600, mp=600) == kvq.KVQ_ERR_WORKSPACE
    assert b"16384" in lib.kvq_last_error()
    assert _step_noalloc(big, hq=64, B=0) == kvq.KVQ_OK
