"""IsoQuant block-4 rotation as an explicit fp64 matrix.

Test infrastructure (see the package docstring).

The IsoQuant abstract (mlsanity.com) treats every 4-dimensional block of a
vector as a quaternion v and maps it to q_L v conj(q_R), the isoclinic
decomposition of a rotation in SO(4); IsoQuant-Full keeps both unit
quaternions, IsoQuant-Fast only the left one (q_R = 1).  Readings where the
abstract is silent:

* blocks are the contiguous channel groups [4k, 4k+4) and the components of a
  block are (w, x, y, z) = (1, i, j, k) coefficients in that order;
* the quaternions are unit quaternions drawn by the caller (one q_L, and for
  Full one q_R, per block); the oracle takes them as inputs;
* the rotation is applied as a dense 128 x 128 matrix product, like the
  Hadamard rotation: the definition, not a fast form.

Quaternions are arrays whose last axis holds (w, x, y, z).
"""

import numpy as np

HEAD_DIM = 128
BLOCK = 4


def hamilton(p, q):
    """Quaternion product p q, from i^2 = j^2 = k^2 = ijk = -1 (broadcast over leading axes)."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    a1, b1, c1, d1 = np.moveaxis(p, -1, 0)
    a2, b2, c2, d2 = np.moveaxis(q, -1, 0)
    return np.stack([
        a1 * a2 - b1 * b2 - c1 * c2 - d1 * d2,
        a1 * b2 + b1 * a2 + c1 * d2 - d1 * c2,
        a1 * c2 - b1 * d2 + c1 * a2 + d1 * b2,
        a1 * d2 + b1 * c2 - c1 * b2 + d1 * a2,
    ], axis=-1)


def conj(q):
    q = np.asarray(q, dtype=np.float64)
    return q * np.array([1.0, -1.0, -1.0, -1.0])


def left_matrix(q):
    """4 x 4 matrix of v -> q v (its columns are q times the basis quaternions)."""
    return np.stack([hamilton(q, e) for e in np.eye(4)], axis=-1)


def right_matrix(q):
    """4 x 4 matrix of v -> v q."""
    return np.stack([hamilton(e, q) for e in np.eye(4)], axis=-1)


def block_matrix(q_left, q_right=None):
    """4 x 4 matrix of v -> q_left v conj(q_right) (q_right None: IsoQuant-Fast, v -> q_left v)."""
    m = left_matrix(q_left)
    if q_right is not None:
        m = m @ right_matrix(conj(q_right))
    return m


class QuatRotation:
    """The block-diagonal rotation of a 128-vector by 32 quaternion blocks.

    ``quat`` is fp[32][4] (IsoQuant-Fast: q_L per block) or fp[32][8] (IsoQuant-Full:
    q_L then q_R per block).  Used wherever the oracle takes a Hadamard block width.
    """

    def __init__(self, quat):
        quat = np.asarray(quat, dtype=np.float64)
        if quat.shape not in ((HEAD_DIM // BLOCK, 4), (HEAD_DIM // BLOCK, 8)):
            raise ValueError("quat must be [32][4] (Fast) or [32][8] (Full)")
        self.quat = quat
        self.full = quat.shape[1] == 8

    def matrix(self) -> np.ndarray:
        r = np.zeros((HEAD_DIM, HEAD_DIM))
        for k in range(HEAD_DIM // BLOCK):
            ql = self.quat[k, :4]
            qr = self.quat[k, 4:] if self.full else None
            r[BLOCK * k:BLOCK * (k + 1), BLOCK * k:BLOCK * (k + 1)] = block_matrix(ql, qr)
        return r
