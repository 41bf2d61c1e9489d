"""Pins for the oracle's Hadamard rotation (CPU only)."""
import numpy as np
import pytest

from oracle import sylvester, rotation
from tests.conftest import read_golden


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_orthogonality_exact(n):
    # H H^T = n I, exactly, in integers.
    h = sylvester(n)
    assert h.dtype == np.int64
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("n", [2, 8, 64, 128])
def test_hadamard_closed_form(n):
    # The Kronecker recursion equals the closed form (-1)^popcount(i & j).
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pop = np.vectorize(lambda x: bin(int(x)).count("1"))(i & j)
    assert np.array_equal(sylvester(n), np.where(pop % 2 == 0, 1, -1))


def test_hadamard_golden_h4():
    rows = read_golden("hadamard_h4.txt")
    want = np.array([[int(x) for x in r] for r in rows], dtype=np.int64)
    assert np.array_equal(sylvester(4), want)


@pytest.mark.parametrize("b", [1, 64, 128])
def test_rotation_orthogonal_symmetric(b):
    r = rotation(b)
    assert np.allclose(r @ r.T, np.eye(128), atol=1e-15, rtol=0)
    assert np.array_equal(r, r.T)


@pytest.mark.parametrize("b", [64, 128])
def test_rotation_block_structure(b):
    r = rotation(b)
    blk = sylvester(b) / np.sqrt(b)
    for i0 in range(0, 128, b):
        for j0 in range(0, 128, b):
            sub = r[i0:i0 + b, j0:j0 + b]
            if i0 == j0:
                assert np.array_equal(sub, blk)
            else:
                assert not sub.any()


def test_rotation_identity_block_one():
    assert np.array_equal(rotation(1), np.eye(128))


@pytest.mark.parametrize("b", [64, 128])
def test_inner_product_invariance(b):
    # (R q) . (R k) = q . k  (the query is rotated by the same transform).
    rng = np.random.default_rng(5)
    q = rng.standard_normal((50, 128))
    k = rng.standard_normal((50, 128)) * 10
    r = rotation(b)
    lhs = np.einsum("nd,nd->n", q @ r.T, k @ r.T)
    rhs = np.einsum("nd,nd->n", q, k)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_rotation_spreads_outliers():
    # A single outlier channel is spread evenly over its block (|y_j| = x / sqrt(b)).
    x = np.zeros(128)
    x[5] = 16.0
    y = rotation(64) @ x
    assert np.allclose(np.abs(y[:64]), 2.0) and not y[64:].any()


def test_rotate_constant_vector_closed_form():
    # H_b (c 1) = (c b, 0, ..., 0) per block: the normalised transform of a constant vector is
    # c sqrt(b) in the first channel of each block and exactly zero elsewhere (what the
    # quantizers' zero cases must see)
    from oracle import rotate
    for b in (64, 128):
        y = rotate(np.full((1, 128), 0.75), b)[0]
        first = np.zeros(128, bool)
        first[::b] = True
        assert np.all(y[~first] == 0.0)
        assert np.allclose(y[first], 0.75 * np.sqrt(b), rtol=2.3e-16, atol=0)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, 128))
    for b in (1, 64, 128):
        assert np.allclose(rotate(x, b), x @ rotation(b).T, rtol=0, atol=1e-14)


def test_mxfp4_constant_vector_has_zero_groups():
    from oracle.paged import encode, FMT_MXFP4
    _, params, info = encode(np.full((1, 128), 0.75), 128, FMT_MXFP4)
    assert params[0, 1:].tolist() == [0, 0, 0] and params[0, 0] == 127 + 3 - 2
