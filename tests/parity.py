"""Comparison rules between the HIP path and the oracle (used by the GPU tests).

INT4 append
  * fp16 scale and zero: within 1 fp16 ulp of the oracle's;
  * codes: recomputed in fp64 from the oracle's rotated y and the GPU's stored scale and
    zero, delta = (y - z)/s; the GPU code must equal clamp(rne(delta), 0, 15), except
    that +-1 is allowed where delta lies within 1e-5 of a rounding boundary (k + 1/2);
  * every byte outside the appended slots keeps the sentinel.
MXFP4 append
  * UE8M0 bytes exact, except +-1 where log2(amax) lies within 1e-5 of an integer (the
    codes are then checked under the GPU's exponent);
  * codes exact, except an adjacent index where |r| lies within 1e-5 of a tie midpoint, and
    the sign of a zero magnitude where |r| < 1e-5 (a negative r that rounds to zero keeps
    its sign: code 8).
Decode attention
  * per (sequence, query head) row: max_j |o - o_ref| / max_j |o_ref| <= 2e-3.
"""

import numpy as np

import oracle
from oracle.paged import token_slots, decode_params_int4
from oracle.layout import k_row_offsets, v_row_offsets, param_offsets
from oracle.mxfp4 import E2M1_GRID

BOUNDARY_TOL = 1e-5
ATTN_TOL = 2e-3


def f16_ordered(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> integers whose differences count ulps (+0 and -0 coincide)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def appended_entries(gpu_pool, cu_new, start_pos, block_table, which):
    """GPU codes uint8[T][Hkv][128] and param bytes uint8[T][Hkv][4] of the appended slots."""
    _, page, slot = token_slots(cu_new, start_pos, block_table)
    hkv = gpu_pool.shape[1]
    row_off = k_row_offsets(slot) if which == "k" else v_row_offsets(slot)
    par_off = param_offsets(slot, which)
    rows = np.stack([gpu_pool[page[:, None], h, row_off] for h in range(hkv)], axis=1)
    params = np.stack([gpu_pool[page[:, None], h, par_off] for h in range(hkv)], axis=1)
    return oracle.unpack_row(rows), params


def touched_mask(pool_shape, cu_new, start_pos, block_table):
    _, page, slot = token_slots(cu_new, start_pos, block_table)
    mask = np.zeros(pool_shape, dtype=bool)
    for which in ("k", "v"):
        offs = np.concatenate([(k_row_offsets(slot) if which == "k" else v_row_offsets(slot)),
                               param_offsets(slot, which)], axis=1)
        for h in range(pool_shape[1]):
            mask[page[:, None], h, offs] = True
    return mask


def check_int4_entries(codes_gpu, params_gpu, info, label=""):
    """Apply the INT4 rules to one tensor (K or V); returns the number of tolerated flips."""
    s_gpu, z_gpu = decode_params_int4(params_gpu)
    s_ref, z_ref = info["s16"], info["z16"]
    ds = np.abs(f16_ordered(s_gpu.view(np.uint16)) - f16_ordered(s_ref.view(np.uint16)))
    dz = np.abs(f16_ordered(z_gpu.view(np.uint16)) - f16_ordered(z_ref.view(np.uint16)))
    assert ds.max(initial=0) <= 1, f"{label}: scale off by {ds.max()} fp16 ulp"
    assert dz.max(initial=0) <= 1, f"{label}: zero off by {dz.max()} fp16 ulp"
    y = info["y"]
    s = s_gpu.astype(np.float64)[..., None]
    z = z_gpu.astype(np.float64)[..., None]
    delta = np.where(s > 0, (y - z) / np.where(s > 0, s, 1.0), 0.0)
    want = np.clip(np.rint(delta), 0, 15)
    diff = codes_gpu.astype(np.int64) - want.astype(np.int64)
    near = np.abs(delta - (np.floor(delta) + 0.5)) < BOUNDARY_TOL
    bad = (diff != 0) & ~((np.abs(diff) == 1) & near)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{label}: {bad.sum()} code mismatches, e.g. at {idx.tolist()}: "
                             f"gpu {codes_gpu[tuple(idx[0])]}, delta {delta[tuple(idx[0])]}")
    # tolerated deviations: codes off by one at a rounding boundary, and parameters one fp16
    # ulp away (the codes are then judged against the parameters the GPU stored)
    return int((diff != 0).sum()) + int((ds != 0).sum()) + int((dz != 0).sum())


def check_mxfp4_entries(codes_gpu, ebytes_gpu, info, label=""):
    """Apply the MXFP4 rules to one tensor; returns the number of tolerated deviations."""
    e_ref = info["e"].astype(np.int64)
    e_gpu = ebytes_gpu.astype(np.int64)
    y = info["y"]
    groups = y.reshape(y.shape[:-1] + (4, 32))
    amax = np.abs(groups).max(-1)
    with np.errstate(divide="ignore"):
        l2 = np.log2(np.where(amax > 0, amax, 1.0))
    near_int = np.abs(l2 - np.rint(l2)) < BOUNDARY_TOL
    de = e_gpu - e_ref
    bad_e = (de != 0) & ~((np.abs(de) == 1) & near_int)
    assert not bad_e.any(), f"{label}: {bad_e.sum()} UE8M0 exponent mismatches"
    r = groups / np.ldexp(1.0, e_gpu - 127)[..., None]
    mag = np.abs(r)
    dist = np.abs(mag[..., None] - E2M1_GRID)
    best = dist.min(-1, keepdims=True)
    hit = dist == best
    even = hit & (np.arange(8) % 2 == 0)
    choose = np.where(even.any(-1, keepdims=True) & (hit.sum(-1, keepdims=True) > 1), even, hit)
    idx = np.argmax(choose, -1)
    want = (np.where(groups < 0, 8, 0) + idx).reshape(y.shape)
    got = codes_gpu.astype(np.int64)
    mids = (E2M1_GRID[1:] + E2M1_GRID[:-1]) / 2
    near_tie = (np.abs(mag[..., None] - mids) < BOUNDARY_TOL).any(-1).reshape(y.shape)
    adjacent = (np.abs((got & 7) - (want & 7)) == 1) & ((got >> 3) == (want >> 3))
    # a zero magnitude may take either sign only where r itself is within the tolerance of the
    # sign boundary r = 0 (fp32 rounding of the rotation can put it on either side); elsewhere
    # a negative value that rounds to magnitude zero must keep its sign bit (code 8)
    zero_sign = ((got & 7) == 0) & ((want & 7) == 0) & (np.abs(r.reshape(y.shape)) < BOUNDARY_TOL)
    bad = (got != want) & ~(adjacent & near_tie) & ~zero_sign
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{label}: {bad.sum()} e2m1 code mismatches, e.g. {i}: gpu {got[i]} want {want[i]}")
    return int((got != want).sum())


def check_append(gpu_pool, oracle_pool, infos, cu_new, start_pos, block_table, fmt, sentinel, label="",
                 prior_mask=None):
    """All append rules; returns the number of tolerated deviations.  ``prior_mask`` marks
    bytes written by earlier appends into the same pool (excluded from the sentinel check).
    ``sentinel``: the byte every untouched position holds, or the whole pool as it was before
    the append (a pool of random bytes)."""
    mask = touched_mask(gpu_pool.shape, cu_new, start_pos, block_table)
    if prior_mask is not None:
        mask = mask | prior_mask
    untouched_ok = gpu_pool[~mask] == (sentinel[~mask] if isinstance(sentinel, np.ndarray) else sentinel)
    assert untouched_ok.all(), f"{label}: {(~untouched_ok).sum()} bytes outside appended slots changed"
    flips = 0
    for which in ("k", "v"):
        codes, params = appended_entries(gpu_pool, cu_new, start_pos, block_table, which)
        if fmt == oracle.FMT_INT4:
            flips += check_int4_entries(codes, params, infos[which], f"{label}/{which}")
        else:
            flips += check_mxfp4_entries(codes, params, infos[which], f"{label}/{which}")
    return flips


def attn_row_error(out, ref):
    """Row-normwise relative error per (sequence, head) row."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(out - ref).max(-1)
    den = np.abs(ref).max(-1)
    return num / np.where(den > 0, den, 1.0)


def kernel_rotation(rot, device="cuda"):
    """(had_block, quat tensor or None) for kvq.Cache from an oracle rotation: a Hadamard block
    width, or an oracle.QuatRotation (its fp32 quaternions, which are the oracle's values)."""
    if isinstance(rot, (int, np.integer)):
        return int(rot), None
    import torch
    q32 = np.ascontiguousarray(rot.quat, np.float32)
    assert np.array_equal(q32.astype(np.float64), rot.quat), "quaternions must be fp32 values"
    return 4, torch.from_numpy(q32).to(device)

