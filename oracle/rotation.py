"""Random orthogonal rotations R (d x d), applied as y = R u.

Test infrastructure only (see the package docstring).

* Dense rotation: "TurboQuant 详解", TurboQuant_mse official steps, step 1 -- QR of a Gaussian
  matrix; "TurboQuant first-principles walkthrough", rotation paragraph -- d x d i.i.d.
  Gaussian matrix, keep the orthogonal factor, generated once and shared by all vectors.
  Reading: the Q factor is made unique by flipping column signs so the triangular factor has a
  non-negative diagonal (sign(0) = +1); any correct QR then gives the same R up to rounding.
  Pinned by orthogonality and norm preservation ("TurboQuant 详解", R^T R = I paragraph).
* Randomized Walsh-Hadamard rotation: "TurboQuant 和 RotorQuant 的真相", chapter 3 (the
  O(d log d) Walsh-Hadamard transform used by the llama.cpp ports).  The pages give no
  normalisation or ordering; reading: R = (1/sqrt(d)) H_d diag(sigma) with the Sylvester
  Hadamard matrix and Rademacher signs sigma (signs applied before H).  The sign draw is parity
  unpinned; the matrix form is pinned by orthogonality and by its explicit Sylvester entries.
* Block (group-32) randomized Hadamard rotation: "TurboQuant 和 RotorQuant 的真相", chapter 3
  (splitting the 128 coordinates into 4 groups of 32, each rotated on its own, tried as a faster
  rotation) and chapter 5 (small orthogonal blocks instead of a full-rank d x d transform);
  "Sub-byte KV cache quantization with TurboQuant", engineering path (structured rotations in
  place of the dense matrix).  Reading: R = (1/sqrt(g)) blockdiag(H_g, ..., H_g) diag(sigma)
  with the same Sylvester H and Rademacher sigma as the full WHT, g = 32, for any d that is a
  multiple of g (so also d that are not powers of two).  Pinned by orthogonality, by its block
  structure, by equality with the full WHT when d = g, and by a per-group butterfly transform.
"""

import numpy as np

from .rng import gaussian, rademacher


def dense_rotation(d, seed):
    """Haar-random orthogonal R from the QR of the seeded d x d Gaussian matrix (row-major)."""
    g = gaussian(seed, d * d).reshape(d, d)
    q, r = np.linalg.qr(g)
    sign = np.where(np.diag(r) >= 0.0, 1.0, -1.0)
    return q * sign[None, :]


def sylvester_hadamard(d):
    """Sylvester Hadamard matrix: H[i, j] = (-1)^popcount(i & j); d must be a power of 2."""
    if d < 1 or (d & (d - 1)) != 0:
        raise ValueError("Hadamard order must be a power of two")
    i = np.arange(d)
    pc = np.zeros((d, d), dtype=np.int64)
    a = i[:, None] & i[None, :]
    while np.any(a):
        pc += a & 1
        a = a >> 1
    return np.where(pc % 2 == 0, 1.0, -1.0)


def wht_rotation(d, seed):
    """Explicit matrix of the randomized Hadamard rotation (1/sqrt(d)) H diag(sigma)."""
    sigma = rademacher(seed, d)
    return sylvester_hadamard(d) * sigma[None, :] / np.sqrt(d)


def block_wht_rotation(d, seed, group=32):
    """Explicit matrix of the block randomized Hadamard rotation
    (1/sqrt(g)) blockdiag(H_g, ..., H_g) diag(sigma); d must be a multiple of g."""
    if group < 1 or d % group != 0:
        raise ValueError("d must be a multiple of the group size")
    sigma = rademacher(seed, d)
    h = sylvester_hadamard(group)
    r = np.zeros((d, d))
    for k in range(0, d, group):
        r[k:k + group, k:k + group] = h
    return r * sigma[None, :] / np.sqrt(group)


def rotation_from_matrix(m):
    """Takes a caller's matrix as R (used by the 2-D worked examples, which print R)."""
    m = np.asarray(m, dtype=np.float64)
    if m.ndim != 2 or m.shape[0] != m.shape[1]:
        raise ValueError("rotation must be square")
    return m.copy()
