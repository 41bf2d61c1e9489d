"""Seeded synthetic workloads (inputs only: no step of the method lives here).

Both the HIP path's tests/bench and the CPU oracle draw their inputs from this
module, so that the two sides see identical values.  It holds random draws,
dtype casts and block-table construction, nothing else.

The pages measure on a multi-turn serving benchmark built from ShareGPT
conversations with 32 concurrent sessions (UltraQuant article, section on what
it showed); no dataset or model weights are used here.  The synthetic inputs
stand in for it with the shapes of the five workloads below: a batch of 32
sequences of 4096 tokens for the concurrent-session decode, ragged 1K-32K
contexts over a shuffled shared page pool for sessions whose prefixes grew
unevenly, and a prefill of 64 x 2048 heavy-tailed tokens for the write path.

Every sequence draws from its own generator, seeded by (workload seed,
sequence index), so any subset of sequences can be regenerated alone.  Values
are drawn in fp32 and rounded to the storage dtype with round-to-nearest-even.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

HEAD_DIM = 128
PAGE_SIZE = 16

_TAG_LENS = 7001
_TAG_PAGES = 7002
_TAG_OUTLIERS = 7003
_TAG_QUERY = 7004
_TAG_QUATERNIONS = 7005


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    kv_dtype: str                 # "f16" | "bf16"
    q_dtype: str                  # "f16" | "bf16" | "f32" | "e4m3"
    had_block: int                # 1, 64 or 128
    fmt: str                      # "int4" | "mxfp4"
    seed: int
    context: Optional[int] = None             # fixed decode context (tokens attended)
    context_range: Optional[Tuple[int, int]] = None   # ragged contexts, inclusive
    new_tokens: Optional[int] = None          # prefill append: tokens per sequence
    pages: str = "contiguous"                 # "contiguous" | "permuted"
    dist: str = "llama"                       # "tiny" | "llama" | "student_t"
    note: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    # 1 sequence, 4 q heads over 1 kv head, 256 cached tokens, fp16, block 64.
    "tiny": Workload("tiny", 1, 4, 1, "f16", "f16", 64, "int4", seed=0, context=256,
                     dist="tiny"),
    # One Llama-3-8B layer: 32 q / 8 kv heads, bf16, batch 32 x 4096, block 128.
    "llama": Workload("llama", 32, 32, 8, "bf16", "bf16", 128, "int4", seed=1, context=4096),
    # Ragged long contexts U[1K, 32K] over a permuted shared pool, block 64.
    "long": Workload("long", 8, 32, 8, "bf16", "bf16", 64, "int4", seed=2,
                     context_range=(1024, 32768), pages="permuted"),
    # Write path: 64 sequences x 2048 new heavy-tailed tokens, block 128.
    "prefill": Workload("prefill", 64, 32, 8, "bf16", "bf16", 128, "int4", seed=3,
                        new_tokens=2048, pages="permuted", dist="student_t"),
    # MXFP4: e2m1 + UE8M0/32 after the full 128 WHT, fp8 e4m3 queries, 64 q / 8 kv, 64 x 16K.
    "mxfp4": Workload("mxfp4", 64, 64, 8, "bf16", "e4m3", 128, "mxfp4", seed=4, context=16384),
}

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32,
                 "e4m3": torch.float8_e4m3fn}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name]


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    """fp32 numpy -> CPU tensor of ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(_TORCH_DTYPES[dtype])


def seq_lens(w: Workload) -> np.ndarray:
    """Tokens attended per sequence (decode) or appended per sequence (prefill)."""
    if w.new_tokens is not None:
        return np.full(w.batch, w.new_tokens, dtype=np.int64)
    if w.context is not None:
        return np.full(w.batch, w.context, dtype=np.int64)
    lo, hi = w.context_range
    return _rng(w.seed, _TAG_LENS).integers(lo, hi + 1, size=w.batch).astype(np.int64)


def block_table(w: Workload, lens: np.ndarray, extra_pages: int = 0):
    """(block_table int32[B][max_pages], num_pages) for sequences of ``lens`` tokens.

    Sequence b owns ceil(lens[b] / 16) pages; ``contiguous`` hands them out in
    order, ``permuted`` draws them from a random permutation of the shared pool.
    ``extra_pages`` leaves that many unused pages at the end of the pool.
    Unused table entries are 0.
    """
    n_pages = [-(-int(n) // PAGE_SIZE) for n in lens]
    total = int(sum(n_pages))
    ids = np.arange(total, dtype=np.int64)
    if w.pages == "permuted":
        ids = _rng(w.seed, _TAG_PAGES).permutation(total)
    width = max(n_pages) if n_pages else 1
    table = np.zeros((len(lens), max(width, 1)), dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = ids[off:off + n]
        off += n
    return table, total + extra_pages


def _outlier_channels(w: Workload):
    """Per kv head, the channels scaled up (and the factor)."""
    rng = _rng(w.seed, _TAG_OUTLIERS)
    if w.dist == "tiny":
        ch = rng.choice(HEAD_DIM, 4, replace=False)
        return [ch for _ in range(w.num_kv_heads)], 20.0
    if w.dist == "llama":
        n = int(round(0.02 * HEAD_DIM))           # 2% of 128 channels -> 3
        return [rng.choice(HEAD_DIM, n, replace=False) for _ in range(w.num_kv_heads)], 15.0
    return None, 1.0


def sequence_kv(w: Workload, b: int, n_tokens: int):
    """K and V of sequence b: fp32 arrays [n_tokens][Hkv][128] (exact in kv dtype)."""
    rng = _rng(w.seed, b)
    shape = (n_tokens, w.num_kv_heads, HEAD_DIM)
    if w.dist == "student_t":
        k = rng.standard_t(3.0, size=shape).astype(np.float32)
        v = rng.standard_t(3.0, size=shape).astype(np.float32)
    else:
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        if w.dist == "llama":
            v *= np.float32(0.5)
        chans, factor = _outlier_channels(w)
        for g in range(w.num_kv_heads):
            k[:, g, chans[g]] *= np.float32(factor)
            if w.dist == "tiny":
                v[:, g, chans[g]] *= np.float32(factor)
    kt = cast(k, w.kv_dtype).to(torch.float32).numpy()
    vt = cast(v, w.kv_dtype).to(torch.float32).numpy()
    return kt, vt


def queries(w: Workload) -> np.ndarray:
    """q fp32 [B][Hq][128], exact in the query dtype."""
    q = _rng(w.seed, _TAG_QUERY).standard_normal((w.batch, w.num_q_heads, HEAD_DIM),
                                                 dtype=np.float32)
    return cast(q, w.q_dtype).to(torch.float32).numpy()


def decode_step_inputs(w: Workload, seqs=None):
    """For a decode workload: per sequence, the L-1 cached tokens and the one new token.

    Returns dict with ``lens`` (tokens attended, L), ``prefix_k``/``prefix_v``
    (lists of fp32 [L-1][Hkv][128]) and ``new_k``/``new_v`` (fp32 [B][Hkv][128]),
    restricted to ``seqs`` when given (other entries None).
    """
    lens = seq_lens(w)
    seqs = range(w.batch) if seqs is None else seqs
    pk, pv = [None] * w.batch, [None] * w.batch
    nk = np.zeros((w.batch, w.num_kv_heads, HEAD_DIM), np.float32)
    nv = np.zeros_like(nk)
    for b in seqs:
        k, v = sequence_kv(w, b, int(lens[b]))
        pk[b], pv[b] = k[:-1], v[:-1]
        nk[b], nv[b] = k[-1], v[-1]
    return {"lens": lens, "prefix_k": pk, "prefix_v": pv, "new_k": nk, "new_v": nv}


def small_variant(w: Workload, batch: int, context: int) -> Workload:
    """Same distributions and heads, fewer/shorter sequences (for quick parity cases)."""
    from dataclasses import replace
    return replace(w, name=f"{w.name}-small", batch=batch, context=context,
                   context_range=None, new_tokens=None if w.new_tokens is None else context)


def unit_quaternions(seed: int, full: bool = False) -> np.ndarray:
    """Random unit quaternions (w, x, y, z) for the quaternion block rotation of a 128-vector:
    fp32[32][4] (one per 4-channel block) or, for ``full``, fp32[32][8] (left then right).

    Uniform on the unit 3-sphere: a 4-vector of independent normals, normalised in fp64, then
    rounded to fp32 -- the values both the kernels and the oracle receive."""
    g = _rng(seed, _TAG_QUATERNIONS, int(full)).standard_normal((32, 2 if full else 1, 4))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    return g.reshape(32, -1).astype(np.float32)

