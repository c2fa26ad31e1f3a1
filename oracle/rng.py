"""Seeded random streams the method draws (rotation R, QJL matrix S, Hadamard signs).

Test infrastructure only (see the package docstring).

The pages say only that the rotation is generated once from a fixed random seed and reused
("TurboQuant first-principles walkthrough", section on deployment parameters: a fixed seed
keeps the rotation consistent across calls; the same section's rotation paragraph: a d x d
i.i.d. Gaussian matrix followed by QR).  Which generator makes the Gaussian matrix is left
open, so each side implements the same published counter-based generator from its
definition:

* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014): element i of stream ``seed`` is mix64(seed + (i + 1) * 0x9E3779B97F4A7C15),
  with mix64 the variant-13 finaliser (shift 30 / multiply 0xBF58476D1CE4E5B9,
  shift 27 / multiply 0x94D049BB133111EB, shift 31).
* uniform on [0, 1): the top 53 bits times 2^-53.
* Gaussian: Box-Muller (Box and Muller 1958), cosine branch only, one pair of uniforms per
  element: sqrt(-2 ln(1 - u1)) * cos(2 pi u2), using stream draws 2e and 2e+1 for element e.
* Rademacher sign: -1 when the top bit of the draw is set, else +1.

Parity unpinned by the pages: no page prints a value of these streams.  They are pinned only
by structural checks (uniformity, Gaussian moments) in the tests.
"""

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed, n, offset=0):
    """Draws ``offset .. offset+n-1`` of the SplitMix64 stream for ``seed`` (uint64 array)."""
    i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform53(z):
    """Top 53 bits of each draw as a float64 in [0, 1)."""
    return (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def gaussian(seed, n):
    """n standard normal float64 values of stream ``seed`` (Box-Muller, cosine branch)."""
    z = splitmix64(seed, 2 * n)
    u1 = uniform53(z[0::2])
    u2 = uniform53(z[1::2])
    return np.sqrt(-2.0 * np.log(1.0 - u1)) * np.cos(2.0 * np.pi * u2)


def rademacher(seed, n):
    """n signs in {-1.0, +1.0}: -1 where the top bit of the draw is set."""
    z = splitmix64(seed, n)
    return np.where((z >> np.uint64(63)) != 0, -1.0, 1.0)
