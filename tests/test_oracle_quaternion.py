"""Pins of the quaternion block rotation (IsoQuant abstract, mlsanity.com: v -> q_L v conj(q_R)
per 4-channel block; IsoQuant-Fast keeps q_L only) against facts fixed outside the oracle:
the quaternion unit table, the 2x2 complex-matrix representation of quaternions, Rodrigues'
rotation formula, the spectrum of an isoclinic rotation, and exact attention on a cache that
the rotation leaves lossless."""
import itertools

import numpy as np
import pytest
import torch

import oracle
from oracle import (QuatRotation, hamilton, conj, left_matrix, block_matrix, append,
                    decode_attention, dequant_pages, FMT_INT4, FMT_MXFP4)
from oracle.attention import gather_sequence
from oracle.paged import encode

ONE, I, J, K = np.eye(4)


def _unit(rng, n):
    q = rng.standard_normal((n, 4))
    return q / np.linalg.norm(q, axis=-1, keepdims=True)


def test_unit_table():
    # i^2 = j^2 = k^2 = ijk = -1, ij = k, jk = i, ki = j and the anticommuted products
    for a, b, c in ((I, J, K), (J, K, I), (K, I, J)):
        assert np.array_equal(hamilton(a, b), c)
        assert np.array_equal(hamilton(b, a), -c)
    for u in (I, J, K):
        assert np.array_equal(hamilton(u, u), -ONE)
    assert np.array_equal(hamilton(hamilton(I, J), K), -ONE)
    q = np.array([0.5, -2.0, 3.0, 0.25])
    assert np.array_equal(hamilton(ONE, q), q) and np.array_equal(hamilton(q, ONE), q)


def _complex_form(q):
    # a + bi + cj + dk  <->  [[a + b i, c + d i], [-c + d i, a - b i]]
    a, b, c, d = q
    return np.array([[a + 1j * b, c + 1j * d], [-c + 1j * d, a - 1j * b]])


def test_product_matches_complex_matrix_representation():
    rng = np.random.default_rng(1)
    for _ in range(50):
        p, q = rng.standard_normal(4), rng.standard_normal(4)
        assert np.allclose(_complex_form(hamilton(p, q)), _complex_form(p) @ _complex_form(q),
                           rtol=0, atol=1e-13)


def test_norm_is_multiplicative_and_conjugate_inverts():
    rng = np.random.default_rng(2)
    p, q = rng.standard_normal((2, 100, 4))
    assert np.allclose(np.linalg.norm(hamilton(p, q), axis=-1),
                       np.linalg.norm(p, axis=-1) * np.linalg.norm(q, axis=-1), rtol=1e-14)
    u = _unit(rng, 20)
    assert np.allclose(hamilton(u, conj(u)), np.tile(ONE, (20, 1)), atol=1e-15)


def test_left_multiplication_is_an_isoclinic_rotation():
    # a unit quaternion a = (cos t, sin t u) acting by left multiplication is a rotation of
    # R^4 whose two rotation angles are equal: eigenvalues cos t +- i sin t, each twice
    rng = np.random.default_rng(3)
    for a in _unit(rng, 30):
        m = left_matrix(a)
        assert np.allclose(m @ m.T, np.eye(4), atol=1e-15)
        assert np.isclose(np.linalg.det(m), 1.0, atol=1e-14)
        ev = np.linalg.eigvals(m)
        s = np.sqrt(1.0 - a[0] ** 2)
        up = np.abs(ev - (a[0] + 1j * s)) < 1e-7
        down = np.abs(ev - (a[0] - 1j * s)) < 1e-7
        assert np.all(up | down) and up.sum() == 2 and down.sum() == 2


def test_sandwich_is_rodrigues_rotation_of_the_pure_part():
    # q = (cos t, sin t u): v -> q v conj(q) fixes the real axis and rotates the pure part by
    # 2t about u (Rodrigues' formula)
    rng = np.random.default_rng(4)
    for _ in range(30):
        u = rng.standard_normal(3)
        u /= np.linalg.norm(u)
        t = rng.uniform(-np.pi, np.pi)
        q = np.concatenate([[np.cos(t)], np.sin(t) * u])
        v = rng.standard_normal(3)
        phi = 2 * t
        rod = v * np.cos(phi) + np.cross(u, v) * np.sin(phi) + u * (u @ v) * (1 - np.cos(phi))
        m = block_matrix(q, q)
        assert np.allclose(m @ np.concatenate([[0.0], v]), np.concatenate([[0.0], rod]), atol=1e-13)
        assert np.allclose(m @ ONE, ONE, atol=1e-15)


def test_fast_is_full_with_identity_right_factor():
    rng = np.random.default_rng(5)
    for a in _unit(rng, 10):
        assert np.allclose(block_matrix(a), block_matrix(a, ONE), atol=0)
        assert np.allclose(block_matrix(a), left_matrix(a), atol=0)


@pytest.mark.parametrize("full", [False, True])
def test_block_rotation_orthogonal_and_preserves_inner_products(full):
    rng = np.random.default_rng(6 + full)
    quat = np.concatenate([_unit(rng, 32), _unit(rng, 32)], axis=1) if full else _unit(rng, 32)
    r = QuatRotation(quat).matrix()
    assert np.allclose(r @ r.T, np.eye(128), atol=1e-14)
    # block-diagonal over contiguous 4-channel blocks
    mask = np.kron(np.eye(32), np.ones((4, 4))).astype(bool)
    assert np.all(r[~mask] == 0)
    q, k = rng.standard_normal((2, 64, 128))
    assert np.allclose(np.einsum("nd,nd->n", q @ r.T, k @ r.T), np.einsum("nd,nd->n", q, k), rtol=1e-12)


def test_identity_quaternions_give_the_plain_encoding():
    rng = np.random.default_rng(8)
    x = torch.from_numpy(rng.standard_normal((40, 128)).astype(np.float32)).bfloat16().double().numpy()
    ident = QuatRotation(np.tile(ONE, (32, 2)))
    for fmt in (FMT_INT4, FMT_MXFP4):
        a = encode(x, ident, fmt)
        b = encode(x, 1, fmt)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _hurwitz_units(rng, n):
    # the 24 unit quaternions with entries in {0, +-1/2, +-1}: products with them are exact
    units = [s * e for e in np.eye(4) for s in (1, -1)]
    units += [0.5 * np.array(sg) for sg in itertools.product((1, -1), repeat=4)]
    return np.array(units)[rng.integers(0, 24, n)]


@pytest.mark.parametrize("full", [False, True])
def test_attention_on_lossless_quaternion_cache_equals_exact_attention(full):
    # x = R^T y with y on an INT4 grid and R built from Hurwitz units (entries 0, +-1/2, +-1):
    # x is exact, the encoder's R x returns y exactly, so the cache is lossless and decode
    # (rotate q, attend, rotate back with R^T) must equal exact attention on the raw x
    rng = np.random.default_rng(9 + full)
    quat = np.concatenate([_hurwitz_units(rng, 32), _hurwitz_units(rng, 32)], axis=1) if full \
        else _hurwitz_units(rng, 32)
    rot = QuatRotation(quat)
    r = rot.matrix()
    n = 24

    def grid_vectors():
        c = rng.integers(0, 16, (n, 128))
        c[:, 0], c[:, 1] = 0, 15
        return c * 0.25 - 2.0
    yk, yv = grid_vectors(), grid_vectors()
    xk, xv = yk @ r, yv @ r  # rows of R^T y
    assert np.allclose(xk @ r.T, yk, atol=0)
    q = rng.standard_normal((1, 4, 128))
    table = np.array([[0, 1]], np.int32)
    pool = np.zeros((2, 1, 2176), np.uint8)
    append(pool, xk[:, None], xv[:, None], np.array([0, n]), np.array([0]), table, rot)
    o = decode_attention(pool, q, [n], table, rot)
    s = (xk @ q[0].T) / np.sqrt(128)
    p = np.exp(s - s.max(0))
    p /= p.sum(0)
    assert np.allclose(o[0], p.T @ xv, atol=1e-12)
    # pages back in the original basis: exactly x
    k, v = dequant_pages(pool, [0, 1], rot, unrotate=True)
    assert np.allclose(k[:, 0].reshape(-1, 128)[:n], xk, atol=1e-12)


@pytest.mark.parametrize("fmt", [FMT_INT4, FMT_MXFP4])
def test_attention_quaternion_matches_torch_sdpa_fp64(fmt):
    # a library routine on the unrotated dequantized cache (k = R^T k', rows k' R)
    rng = np.random.default_rng(11 + fmt)
    rot = QuatRotation(np.concatenate([_unit(rng, 32), _unit(rng, 32)], axis=1))
    r = rot.matrix()
    lens = [37, 5]
    hkv, hq = 2, 8
    table = np.array([[0, 1, 2], [3, 4, 5]], np.int32)
    pool = np.zeros((6, hkv, 2176), np.uint8)
    t = sum(lens)
    k = rng.standard_normal((t, hkv, 128))
    k[:, :, [3, 70]] *= 12
    v = 0.5 * rng.standard_normal((t, hkv, 128))
    append(pool, k, v, np.array([0, lens[0], t]), np.array([0, 0]), table, rot, fmt)
    q = rng.standard_normal((2, hq, 128))
    out = decode_attention(pool, q, lens, table, rot, fmt, q_scale=0.7, sm_scale=0.15)
    for b, length in enumerate(lens):
        k_rot, v_rot = gather_sequence(pool, table[b], length, rot, fmt)
        kk = torch.from_numpy(k_rot @ r).repeat_interleave(hq // hkv, dim=0)
        vv = torch.from_numpy(v_rot @ r).repeat_interleave(hq // hkv, dim=0)
        qq = torch.from_numpy(0.7 * q[b])[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=0.15)[:, 0].numpy()
        assert np.allclose(out[b], ref, rtol=0, atol=1e-12)
