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


def rotate(x, rot, dim: int = 128) -> np.ndarray:
    """y = R x for the rows of x[..., dim] (fp64).

    For the Hadamard rotation the +-1 product H_b x is formed first and divided by sqrt(b)
    once: the sums of the (fp16/bf16-exact) inputs are exact in fp64, so y carries one
    rounding, and a component whose exact value is zero (a constant vector's, say) comes out
    as exactly zero -- the quantizers' zero cases (an INT4 range of 0, an MXFP4 group amax of
    0) then see what the definition gives.  Other rotations multiply by their matrix.
    """
    x = np.asarray(x, dtype=np.float64)
    if isinstance(rot, (int, np.integer)):
        b = int(rot)
        if b < 1 or dim % b != 0:
            raise ValueError(f"had_block {b} does not tile dim {dim}")
        h = np.zeros((dim, dim))
        blk = sylvester(b).astype(np.float64)
        for start in range(0, dim, b):
            h[start:start + b, start:start + b] = blk
        return (x @ h.T) / np.sqrt(np.float64(b))
    return x @ rot.matrix().T

