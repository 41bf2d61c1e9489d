"""Walsh-Hadamard matrices and the block-diagonal rotation, as explicit fp64 matrices.

Test infrastructure (see the package docstring).

The SAW-INT4 summary ("Summary", "Method") rotates each token vector with a
*block-diagonal Hadamard* matrix before quantizing; the UltraQuant article
(section on how the method works) calls the same step a Walsh-Hadamard rotation
that spreads outlier channels across the block.  Neither page fixes a sign
pattern, a permutation or a normalisation beyond orthogonality, so the oracle
takes the plainest reading: the natural-order Sylvester matrix scaled by
1/sqrt(b), no random signs, repeated along the diagonal over contiguous
channel blocks of width b.  The rotation is applied as a dense matrix product
on purpose (O(d^2)); it is the definition, not a fast transform.
"""

import numpy as np


def sylvester(n: int) -> np.ndarray:
    """Unnormalised Sylvester-Hadamard matrix H_n (entries +-1, int64).

    H_1 = [1];  H_2m = [[H_m, H_m], [H_m, -H_m]], built with a Kronecker product.
    """
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"Hadamard order must be a power of two, got {n}")
    h = np.ones((1, 1), dtype=np.int64)
    two = np.array([[1, 1], [1, -1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.kron(two, h)
    return h


def rotation(had_block: int, dim: int = 128) -> np.ndarray:
    """R_b = blockdiag(H_b / sqrt(b), ..., H_b / sqrt(b)) of size dim x dim, fp64.

    ``had_block`` = 1 gives the identity: the "plain INT4" ablation that the
    SAW-INT4 summary compares against ("matching plain INT4 throughput").
    R_b is symmetric and orthogonal, hence its own inverse.
    """
    if had_block < 1 or dim % had_block != 0:
        raise ValueError(f"had_block {had_block} does not tile dim {dim}")
    blk = sylvester(had_block).astype(np.float64) / np.sqrt(np.float64(had_block))
    r = np.zeros((dim, dim), dtype=np.float64)
    for start in range(0, dim, had_block):
        r[start:start + had_block, start:start + had_block] = blk
    return r


def rotation_matrix(rot, dim: int = 128) -> np.ndarray:
    """The rotation R (y = R x) named by ``rot``: a Hadamard block width (int) or an object
    with a ``matrix()`` method (the quaternion block rotation).  R is orthogonal; only the
    Hadamard one is also symmetric, so the way back is R^T."""
    if isinstance(rot, (int, np.integer)):
        return rotation(int(rot), dim)
    return rot.matrix()

