"""Lloyd-Max scalar codebook for the coordinate density after a random rotation.

Test infrastructure only (see the package docstring).

* Coordinate density: "TurboQuant 详解", section on the key insight (rotate first) --
  f(x) proportional to (1 - x^2)^((d-3)/2) on [-1, 1] for one coordinate of a uniform point
  on the unit sphere; for large d it approaches N(0, 1/d) ("TurboQuant first-principles
  walkthrough", core-insight paragraph).  The normalising Gamma constant cancels in every
  conditional mean, so only the unnormalised weight is used.
* Lloyd-Max iteration: "TurboQuant 详解", pain point 2 (worked example on [1, 2, 8, 9]):
  thresholds are midpoints of adjacent centroids, then each centroid becomes the mean of the
  points in its cell; repeated.
* Recipe: "Sub-byte KV cache quantization with TurboQuant", engineering path, first layer --
  a dense grid of 50000 points over +-6 sigma of the density, 300 Lloyd-Max iterations, done
  once on the CPU and cached per (dimension, bits).

Readings where the pages are silent (each listed in the design notes):
* sigma = 1/sqrt(d); the grid is clipped to [-1, 1] and includes both end points.
* Initial centroids c_k = m * (-1 + (2k + 1) / K) with m = min(3 sigma, 1), K = 2^b.
* A grid point x is in cell #{k : x >= t_k} (ties go to the upper cell); an empty cell keeps
  its centroid.
* After the last iteration the codebook is made exactly antisymmetric,
  c_k <- (c_k - c_{K-1-k}) / 2, so the middle threshold is exactly 0.0.
Pins: the [1, 2, 8, 9] example, the Gaussian-limit centroids printed by the walkthrough page,
the closed form at d = 3 (uniform density), the continuous Lloyd-Max optimum, and the
distortion table of "TurboQuant 详解" (Theorem 1 table).
"""

from dataclasses import dataclass

import numpy as np

GRID_POINTS = 50000
ITERATIONS = 300


@dataclass(frozen=True)
class Codebook:
    """Sorted centroids c (2^b values) and midpoint thresholds t (2^b - 1 values), fp64."""
    d: int
    b: int
    centroids: np.ndarray
    thresholds: np.ndarray

    @property
    def centroids32(self):
        return self.centroids.astype(np.float32)

    @property
    def thresholds32(self):
        return self.thresholds.astype(np.float32)


def lloyd_max_points(x, w, init, iterations):
    """Weighted 1-D Lloyd-Max on fixed points x with weights w, from centroids ``init``.

    Each iteration: midpoints of adjacent centroids are the thresholds; point j goes to cell
    #{k : x_j >= t_k}; a non-empty cell's centroid becomes its weighted mean.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    c = np.array(init, dtype=np.float64)
    k = c.size
    for _ in range(iterations):
        t = 0.5 * (c[:-1] + c[1:])
        cell = np.searchsorted(t, x, side="right")
        mass = np.bincount(cell, weights=w, minlength=k)
        moment = np.bincount(cell, weights=w * x, minlength=k)
        nonempty = mass > 0.0
        c = np.where(nonempty, moment / np.where(nonempty, mass, 1.0), c)
    return c


def coordinate_weights(x, d, density="beta"):
    """Unnormalised density of one rotated coordinate at the points x.

    "beta": (1 - x^2)^((d-3)/2), zero where 1 - x^2 <= 0;  "gauss": exp(-d x^2 / 2).
    """
    x = np.asarray(x, dtype=np.float64)
    if density == "beta":
        one_minus = 1.0 - x * x
        out = np.zeros_like(x)
        ok = one_minus > 0.0
        out[ok] = np.exp(0.5 * (d - 3) * np.log1p(-(x[ok] * x[ok])))
        return out
    if density == "gauss":
        return np.exp(-0.5 * d * x * x)
    raise ValueError("density must be 'beta' or 'gauss'")


def codebook(d, b, density="beta", grid_points=GRID_POINTS, iterations=ITERATIONS):
    """The (d, b) codebook by the grid recipe, in unit-sphere coordinates."""
    if d < 2 or b < 1:
        raise ValueError("need d >= 2 and b >= 1")
    sigma = 1.0 / np.sqrt(d)
    lo = max(-6.0 * sigma, -1.0)
    hi = min(6.0 * sigma, 1.0)
    x = np.linspace(lo, hi, grid_points)
    w = coordinate_weights(x, d, density)
    k = 1 << b
    m = min(3.0 * sigma, 1.0)
    init = m * (-1.0 + (2.0 * np.arange(k) + 1.0) / k)
    c = lloyd_max_points(x, w, init, iterations)
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    return Codebook(d=d, b=b, centroids=c, thresholds=t)


def codebook_from_values(centroids, d=None):
    """A codebook with caller-given sorted centroids (used by the hand examples)."""
    c = np.asarray(centroids, dtype=np.float64)
    if np.any(np.diff(c) <= 0):
        raise ValueError("centroids must be strictly increasing")
    b = int(round(np.log2(c.size)))
    if (1 << b) != c.size:
        raise ValueError("number of centroids must be a power of two")
    t = 0.5 * (c[:-1] + c[1:])
    return Codebook(d=d if d is not None else 0, b=b, centroids=c, thresholds=t)
