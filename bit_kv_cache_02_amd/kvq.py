"""Python binding of libkvq (argument marshalling only).

Every function here forwards to the C ABI declared in ``include/kvq.h``; all the
computation runs in the library's HIP kernels on the caller's current HIP
stream.  PyTorch provides device memory and the stream.  The module raises
if ``libkvq.so`` has not been built: there is no fallback path.
"""

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP = 0, -1, -2, -3, -4
FMT_INT4, FMT_MXFP4 = 0, 1
F16, BF16, F32, FP8_E4M3 = 0, 1, 2, 3
OUT_ROTATED = 1
ROT_QUAT4 = 4
MX_SCALED_MFMA = 2
UNROTATE = 1
HEAD_DIM = 128
PAGE_SIZE = 16
PAGE_HEAD_BYTES = 2176

_DTYPE_CODE = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32,
               torch.float8_e4m3fn: FP8_E4M3}
_FMT_CODE = {"int4": FMT_INT4, "mxfp4": FMT_MXFP4}


class KvqCacheDesc(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("had_block", ctypes.c_int32), ("quat_full", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("pool", ctypes.c_void_p), ("quat", ctypes.c_void_p)]


class KvqError(RuntimeError):
    pass


_lib = None

# (name, restype, argtypes) of every symbol kvq.h declares
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
SIGNATURES = [
    ("kvq_abi_version", ctypes.c_int, []),
    ("kvq_page_bytes", ctypes.c_size_t, [ctypes.POINTER(KvqCacheDesc)]),
    ("kvq_append", ctypes.c_int, [ctypes.POINTER(KvqCacheDesc), _P, _P, _I32, _I32, _I32, _P, _P, _P,
                                  _I32, _I32, _P]),
    ("kvq_decode_workspace_bytes", ctypes.c_size_t, [ctypes.POINTER(KvqCacheDesc), _I32, _I32, _I32]),
    ("kvq_decode_attn", ctypes.c_int, [ctypes.POINTER(KvqCacheDesc), _P, _I32, ctypes.c_float, _I32,
                                       _I32, _P, _I32, _P, _I32, ctypes.c_float, _P, _I32,
                                       ctypes.c_uint32, _P, ctypes.c_size_t, _P]),
    ("kvq_decode_step", ctypes.c_int, [ctypes.POINTER(KvqCacheDesc), _P, _P, _I32, _P, _I32,
                                       ctypes.c_float, _I32, _I32, _P, _I32, _P, _I32, ctypes.c_float,
                                       _P, _I32, ctypes.c_uint32, _P, ctypes.c_size_t, _P]),
    ("kvq_decode_step_noalloc", ctypes.c_int, [ctypes.POINTER(KvqCacheDesc), _P, _P, _I32, _P, _I32,
                                               ctypes.c_float, _I32, _I32, _P, _I32, _P, _I32,
                                               ctypes.c_float, _P, _I32, ctypes.c_uint32, _P]),
    ("kvq_prefill_attn", ctypes.c_int, [ctypes.POINTER(KvqCacheDesc), _P, _I32, ctypes.c_float, _I32, _I32,
                                        _I32, _P, _P, _I32, _I32, _P, _I32, ctypes.c_float, _P, _I32,
                                        ctypes.c_uint32, _P]),
    ("kvq_dequant_page", ctypes.c_int, [ctypes.POINTER(KvqCacheDesc), _P, _I32, _P, _P,
                                        ctypes.c_uint32, _P]),
    ("kvq_strerror", ctypes.c_char_p, [ctypes.c_int]),
    ("kvq_last_error", ctypes.c_char_p, []),
    ("kvq_hbm_copy", ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    ("kvq_hbm_read", ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
    ("kvq_hbm_fold4", ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    ("kvq_hbm_append_pattern", ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P,
                                              ctypes.c_int32, _P, ctypes.c_uint32, _P]),
    ("kvq_hbm_decode_pattern", ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]),
]


def lib():
    """The loaded libkvq (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KvqError(f"{LIB_PATH} is missing: build it with "
                           "`python -m bit_kv_cache_02_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, what: str):
    if status == KVQ_OK:
        return
    msg = f"{what}: {lib().kvq_strerror(status).decode()}: {lib().kvq_last_error().decode()}"
    if status in (KVQ_ERR_INVALID_ARG, KVQ_ERR_WORKSPACE):
        raise ValueError(msg)
    if status == KVQ_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise KvqError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _require(t: torch.Tensor, name: str, dtype=None, device=True):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


class Cache:
    """One layer's paged 4-bit cache: a caller-owned uint8 pool [num_pages][Hkv][2176]."""

    def __init__(self, num_pages: int, num_kv_heads: int, had_block: int, fmt: str = "int4",
                 device="cuda", pool: Optional[torch.Tensor] = None, fill: Optional[int] = None,
                 quat: Optional[torch.Tensor] = None):
        """had_block: Hadamard block width (1, 64, 128) or ROT_QUAT4 with ``quat``, the unit
        quaternions of the block-4 rotation: float32 [32][4] (IsoQuant-Fast) or [32][8]
        (IsoQuant-Full), on the pool's device."""
        if (had_block == ROT_QUAT4) != (quat is not None):
            raise ValueError("quat is given exactly when had_block is 4")
        if quat is not None and (quat.dtype != torch.float32 or tuple(quat.shape) not in ((32, 4), (32, 8))
                                 or not quat.is_contiguous()):
            raise ValueError("quat must be a contiguous float32 [32][4] or [32][8] tensor")
        self.quat = quat
        self.fmt = fmt
        self.num_kv_heads = num_kv_heads
        self.had_block = had_block
        self.num_pages = num_pages
        if pool is None:
            pool = torch.empty((num_pages, num_kv_heads, PAGE_HEAD_BYTES), dtype=torch.uint8,
                               device=device)
            if fill is not None:
                pool.fill_(fill)
        if tuple(pool.shape) != (num_pages, num_kv_heads, PAGE_HEAD_BYTES) or pool.dtype != torch.uint8:
            raise ValueError("pool must be uint8[num_pages][num_kv_heads][2176]")
        self.pool = pool

    def desc(self) -> KvqCacheDesc:
        full = 1 if self.quat is not None and self.quat.shape[1] == 8 else 0
        return KvqCacheDesc(_FMT_CODE[self.fmt], self.num_kv_heads, HEAD_DIM, PAGE_SIZE,
                            self.had_block, full, self.num_pages, self.pool.data_ptr(),
                            None if self.quat is None else self.quat.data_ptr())


def abi_version() -> int:
    return lib().kvq_abi_version()


def append(cache: Cache, k: torch.Tensor, v: torch.Tensor, cu_new: torch.Tensor,
           start_pos: torch.Tensor, block_table: torch.Tensor, max_new_tokens: int):
    """Rotate, quantize and write tokens k, v [T][Hkv][128] into the cache (kvq_append)."""
    for t, n in ((k, "k"), (v, "v")):
        _require(t, n)
    for t, n in ((cu_new, "cu_new"), (start_pos, "start_pos"), (block_table, "block_table")):
        _require(t, n, torch.int32)
    if k.dtype not in (torch.float16, torch.bfloat16) or v.dtype != k.dtype:
        raise ValueError("k and v must both be float16 or bfloat16")
    d = cache.desc()
    st = lib().kvq_append(ctypes.byref(d), _ptr(k), _ptr(v), _DTYPE_CODE[k.dtype], k.shape[0],
                          start_pos.shape[0], _ptr(cu_new), _ptr(start_pos), _ptr(block_table),
                          block_table.shape[1], int(max_new_tokens), _stream())
    _check(st, "kvq_append")


def decode_workspace_bytes(cache: Cache, num_q_heads: int, num_seqs: int, max_seq_len: int) -> int:
    d = cache.desc()
    n = lib().kvq_decode_workspace_bytes(ctypes.byref(d), num_q_heads, num_seqs, max_seq_len)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError(f"kvq_decode_workspace_bytes: {lib().kvq_last_error().decode()}")
    return n


def make_workspace(cache: Cache, num_q_heads: int, num_seqs: int, max_seq_len: int, device="cuda"):
    """Workspace for kvq_decode_attn / kvq_decode_step (None when none is needed), zero-filled as
    the library requires before its first use (the calls leave it zeroed)."""
    n = decode_workspace_bytes(cache, num_q_heads, num_seqs, max_seq_len)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _flags(rotated: bool, scaled_mfma: bool) -> int:
    return (OUT_ROTATED if rotated else 0) | (MX_SCALED_MFMA if scaled_mfma else 0)


def decode_attn(cache: Cache, q: torch.Tensor, seq_lens: torch.Tensor, block_table: torch.Tensor,
                max_seq_len: int, out: Optional[torch.Tensor] = None, q_scale: float = 1.0,
                sm_scale: Optional[float] = None, out_dtype=torch.float32, rotated: bool = False,
                workspace: Optional[torch.Tensor] = None, scaled_mfma: bool = False) -> torch.Tensor:
    """softmax(q'.K'^T) V' over the paged cache, rotated back (kvq_decode_attn).

    scaled_mfma (MXFP4 caches): q.K and p.V on the scaled FP8 x FP4 matrix cores (KVQ_MX_SCALED_MFMA).
    """
    _require(q, "q")
    _require(seq_lens, "seq_lens", torch.int32)
    _require(block_table, "block_table", torch.int32)
    b, hq, dim = q.shape
    if out is None:
        out = torch.empty((b, hq, dim), dtype=out_dtype, device=q.device)
    _require(out, "out")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if workspace is None:
        workspace = make_workspace(cache, hq, b, max_seq_len, q.device)
    d = cache.desc()
    st = lib().kvq_decode_attn(ctypes.byref(d), _ptr(q), _DTYPE_CODE[q.dtype], float(q_scale), hq, b,
                               _ptr(seq_lens), int(max_seq_len), _ptr(block_table),
                               block_table.shape[1], float(sm_scale), _ptr(out),
                               _DTYPE_CODE[out.dtype], _flags(rotated, scaled_mfma),
                               _ptr(workspace), 0 if workspace is None else workspace.numel(),
                               _stream())
    _check(st, "kvq_decode_attn")
    return out


def decode_step(cache: Cache, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, seq_lens: torch.Tensor,
                block_table: torch.Tensor, max_seq_len: int, out: Optional[torch.Tensor] = None,
                q_scale: float = 1.0, sm_scale: Optional[float] = None, out_dtype=torch.float32,
                rotated: bool = False, workspace: Optional[torch.Tensor] = None,
                scaled_mfma: bool = False) -> torch.Tensor:
    """Append k[b], v[b] at position seq_lens[b]-1, then attend [0, seq_lens[b]) (kvq_decode_step)."""
    _require(k, "k")
    _require(v, "v")
    _require(q, "q")
    _require(seq_lens, "seq_lens", torch.int32)
    _require(block_table, "block_table", torch.int32)
    b, hq, dim = q.shape
    if k.shape != (b, cache.num_kv_heads, dim) or v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError(f"k and v must both be [{b}][{cache.num_kv_heads}][{dim}] of one dtype")
    if out is None:
        out = torch.empty((b, hq, dim), dtype=out_dtype, device=q.device)
    _require(out, "out")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if workspace is None:
        workspace = make_workspace(cache, hq, b, max_seq_len, q.device)
    d = cache.desc()
    st = lib().kvq_decode_step(ctypes.byref(d), _ptr(k), _ptr(v), _DTYPE_CODE[k.dtype], _ptr(q),
                               _DTYPE_CODE[q.dtype], float(q_scale), hq, b, _ptr(seq_lens),
                               int(max_seq_len), _ptr(block_table), block_table.shape[1],
                               float(sm_scale), _ptr(out), _DTYPE_CODE[out.dtype],
                               _flags(rotated, scaled_mfma), _ptr(workspace),
                               0 if workspace is None else workspace.numel(), _stream())
    _check(st, "kvq_decode_step")
    return out


def decode_step_noalloc(cache: Cache, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor,
                        seq_lens: torch.Tensor, block_table: torch.Tensor, max_seq_len: int,
                        out: torch.Tensor, q_scale: float = 1.0, sm_scale: Optional[float] = None,
                        rotated: bool = False, scaled_mfma: bool = False) -> torch.Tensor:
    """kvq_decode_step with the library's fixed device scratch instead of a workspace
    (kvq_decode_step_noalloc): the caller passes `out`, and the call allocates nothing."""
    _require(k, "k")
    _require(v, "v")
    _require(q, "q")
    _require(seq_lens, "seq_lens", torch.int32)
    _require(block_table, "block_table", torch.int32)
    _require(out, "out")
    b, hq, dim = q.shape
    if k.shape != (b, cache.num_kv_heads, dim) or v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError(f"k and v must both be [{b}][{cache.num_kv_heads}][{dim}] of one dtype")
    if out.shape != q.shape:
        raise ValueError(f"out must be {tuple(q.shape)}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    d = cache.desc()
    st = lib().kvq_decode_step_noalloc(ctypes.byref(d), _ptr(k), _ptr(v), _DTYPE_CODE[k.dtype], _ptr(q),
                                       _DTYPE_CODE[q.dtype], float(q_scale), hq, b, _ptr(seq_lens),
                                       int(max_seq_len), _ptr(block_table), block_table.shape[1],
                                       float(sm_scale), _ptr(out), _DTYPE_CODE[out.dtype],
                                       _flags(rotated, scaled_mfma), _stream())
    _check(st, "kvq_decode_step_noalloc")
    return out


def prefill_attn(cache: Cache, q: torch.Tensor, cu_q: torch.Tensor, seq_lens: torch.Tensor,
                 block_table: torch.Tensor, max_seq_len: int, max_q_len: int,
                 out: Optional[torch.Tensor] = None, q_scale: float = 1.0, sm_scale: Optional[float] = None,
                 out_dtype=torch.float32, rotated: bool = False) -> torch.Tensor:
    """Causal attention of each sequence's chunk (its last cu_q[b+1]-cu_q[b] positions, already
    appended) over the paged cache (kvq_prefill_attn)."""
    _require(q, "q")
    _require(cu_q, "cu_q", torch.int32)
    _require(seq_lens, "seq_lens", torch.int32)
    _require(block_table, "block_table", torch.int32)
    t, hq, dim = q.shape
    if out is None:
        out = torch.empty((t, hq, dim), dtype=out_dtype, device=q.device)
    _require(out, "out")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    d = cache.desc()
    st = lib().kvq_prefill_attn(ctypes.byref(d), _ptr(q), _DTYPE_CODE[q.dtype], float(q_scale), hq, t,
                                seq_lens.numel(), _ptr(cu_q), _ptr(seq_lens), int(max_seq_len), int(max_q_len),
                                _ptr(block_table), block_table.shape[1], float(sm_scale), _ptr(out),
                                _DTYPE_CODE[out.dtype], OUT_ROTATED if rotated else 0, _stream())
    _check(st, "kvq_prefill_attn")
    return out


def dequant_pages(cache: Cache, page_ids: torch.Tensor, unrotate: bool = False):
    """(k, v) float32 [n][Hkv][16][128] of whole pages (kvq_dequant_page)."""
    _require(page_ids, "page_ids", torch.int32)
    n = page_ids.numel()
    shape = (n, cache.num_kv_heads, PAGE_SIZE, HEAD_DIM)
    out_k = torch.empty(shape, dtype=torch.float32, device=page_ids.device)
    out_v = torch.empty(shape, dtype=torch.float32, device=page_ids.device)
    d = cache.desc()
    st = lib().kvq_dequant_page(ctypes.byref(d), _ptr(page_ids), n, _ptr(out_k), _ptr(out_v),
                                UNROTATE if unrotate else 0, _stream())
    _check(st, "kvq_dequant_page")
    return out_k, out_v


def hbm_copy(src: torch.Tensor, dst: torch.Tensor):
    """Plain copy kernel (bandwidth probe)."""
    st = lib().kvq_hbm_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(), _stream())
    _check(st, "kvq_hbm_copy")


HBM_READ_SINK_WORDS = 4096


def hbm_read(src: torch.Tensor, sink: torch.Tensor):
    """Read-only streaming kernel (bandwidth probe).  sink: int32/uint32 [4096] on the device;
    after a call on a zeroed sink, the XOR of its words is the XOR of src's 32-bit words."""
    if sink.numel() * sink.element_size() < 4 * HBM_READ_SINK_WORDS or not sink.is_contiguous():
        raise ValueError("hbm_read: sink must be a contiguous buffer of 4096 32-bit words")
    st = lib().kvq_hbm_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream())
    _check(st, "kvq_hbm_read")


def hbm_fold4(src: torch.Tensor, dst: torch.Tensor):
    """The 4:1 read:write probe over 16-byte vectors: dst vector 256m + t = XOR of src vectors
    1024m + t + 256k, k = 0..3 (dst: a multiple of 4096 bytes)."""
    _require(src, "src")
    _require(dst, "dst")
    nbytes = dst.numel() * dst.element_size()
    if src.numel() * src.element_size() != 4 * nbytes:
        raise ValueError("src must hold exactly 4 times the bytes of dst")
    _check(lib().kvq_hbm_fold4(_ptr(src), _ptr(dst), nbytes, _stream()), "kvq_hbm_fold4")


def hbm_append_pattern(k: torch.Tensor, v: torch.Tensor, block_table: torch.Tensor, pool: torch.Tensor,
                       new_tokens: int, order: int = 0):
    """The append's memory traffic without its arithmetic (kvq_hbm_append_pattern): k, v
    [num_seqs * new_tokens][Hkv][128] 2-byte elements, block_table int32 [num_seqs][max_pages],
    pool uint8 [pages][Hkv][2176]; order 0 the append's own, 1 one workgroup per page, 2 as 1 with
    the pages written in increasing id: block_table is then the [num_seqs][new_tokens / 16] list
    whose item i names the (sequence, page) b * (new_tokens / 16) + j written to page i."""
    for t, n in ((k, "k"), (v, "v"), (pool, "pool")):
        _require(t, n)
    _require(block_table, "block_table", torch.int32)
    if k.element_size() != 2 or v.shape != k.shape or k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError("k and v must be [T][Hkv][128] with 2-byte elements")
    num_seqs, max_pages = block_table.shape
    if k.shape[0] != num_seqs * new_tokens:
        raise ValueError("k must hold num_seqs * new_tokens rows")
    _check(lib().kvq_hbm_append_pattern(_ptr(k), _ptr(v), k.shape[1], num_seqs, int(new_tokens), _ptr(block_table),
                                        max_pages, _ptr(pool), int(order), _stream()), "kvq_hbm_append_pattern")


def hbm_decode_pattern(pool: torch.Tensor, num_kv_heads: int, block_table: torch.Tensor, pages_per_seq: int,
                       waves: int, depth: int, pages_per_split: int, sink: torch.Tensor = None) -> torch.Tensor:
    """The decode's page stream without its arithmetic (kvq_hbm_decode_pattern): pool uint8,
    block_table int32 [num_seqs][max_pages], every sequence pages_per_seq full pages; returns the
    uint32 sink, one word per wave (the sum of the words its lanes loaded)."""
    _require(pool, "pool")
    _require(block_table, "block_table", torch.int32)
    num_seqs, max_pages = block_table.shape
    nsplit = -(-int(pages_per_seq) // int(pages_per_split))
    words = num_seqs * num_kv_heads * nsplit * waves
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=pool.device)
    _require(sink, "sink", torch.int32)
    if sink.numel() < words:
        raise ValueError(f"sink must hold {words} words")
    _check(lib().kvq_hbm_decode_pattern(_ptr(pool), int(num_kv_heads), num_seqs, int(pages_per_seq),
                                        _ptr(block_table), max_pages, int(waves), int(depth), int(pages_per_split),
                                        _ptr(sink), _stream()), "kvq_hbm_decode_pattern")
    return sink
