"""Pins of the oracle's codebook (density, Lloyd-Max grid recipe) to closed forms, the pages'
printed centroids and distortions, and the continuous Lloyd-Max optimum (scipy)."""

import numpy as np
import pytest
from scipy import integrate, special, stats

import oracle


def test_beta_density_matches_scipy():
    # One coordinate of a uniform point on S^{d-1}: (x + 1) / 2 ~ Beta((d-1)/2, (d-1)/2).
    for d in (3, 8, 128, 1536):
        x = np.linspace(-0.9, 0.9, 101) * min(1.0, 6 / np.sqrt(d))
        w = oracle.coordinate_weights(x, d, "beta")
        a = 0.5 * (d - 1)
        ref = stats.beta.pdf(0.5 * (x + 1.0), a, a)
        ratio = w / ref
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-9)


def test_beta_density_normalisation_constant():
    # Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - x^2)^((d-3)/2) integrates to one.
    for d in (3, 5, 128):
        c = np.exp(special.gammaln(d / 2) - special.gammaln((d - 1) / 2)) / np.sqrt(np.pi)
        val, _ = integrate.quad(lambda t: c * oracle.coordinate_weights(np.array([t]), d)[0], -1, 1)
        assert abs(val - 1.0) < 1e-8


def test_gauss_limit_one_bit_is_sqrt_2_over_pi(golden):
    ex = golden["gaussian_limit_centroids"]
    for d in (128, 1536):
        cb = oracle.codebook(d, 1, "gauss")
        assert abs(cb.centroids[1] * np.sqrt(d) - ex["b1_positive"][0]) < 1e-6
        assert cb.thresholds[0] == 0.0


def test_gauss_limit_two_bit_printed_values(golden):
    ex = golden["gaussian_limit_centroids"]
    cb = oracle.codebook(1536, 2, "gauss")
    pos = cb.centroids[2:] * np.sqrt(1536)
    # printed to 3 decimals; the grid recipe stops ~2e-4 from the continuous optimum
    np.testing.assert_allclose(pos, ex["b2_positive"], atol=1e-3)
    cbb = oracle.codebook(1536, 2, "beta")
    np.testing.assert_allclose(cbb.centroids[2:] * np.sqrt(1536), ex["b2_positive"], atol=1e-3)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_d3_closed_form(b):
    # d = 3: the coordinate is uniform on [-1, 1], so Lloyd-Max is the uniform quantizer.
    cb = oracle.codebook(3, b)
    k = 1 << b
    expect = -1.0 + (2.0 * np.arange(k) + 1.0) / k
    np.testing.assert_allclose(cb.centroids, expect, atol=1e-4)
    # D_mse for unit vectors = 3 * E[(y - Q(y))^2] = 4^-b
    dmse = 3 * _dmse_coordinate(cb, 3)
    assert abs(dmse - 4.0 ** -b) < 1e-4


def test_codebook_antisymmetric_and_sorted():
    for d in (64, 128, 1536):
        for b in (1, 2, 3, 4):
            cb = oracle.codebook(d, b)
            c = cb.centroids
            assert np.all(np.diff(c) > 0)
            np.testing.assert_array_equal(c, -c[::-1])
            assert cb.thresholds[(1 << b) // 2 - 1] == 0.0
            np.testing.assert_array_equal(cb.thresholds, 0.5 * (c[:-1] + c[1:]))


def _beta_cell_mass_moment(lo, hi, d):
    # (x + 1)/2 ~ Beta(a, a), a = (d-1)/2 ; moment integral in closed form:
    # int x (1 - x^2)^p dx = -(1 - x^2)^(p+1) / (2 (p+1)), p = (d-3)/2, times the pdf constant.
    a = 0.5 * (d - 1)
    mass = stats.beta.cdf(0.5 * (hi + 1), a, a) - stats.beta.cdf(0.5 * (lo + 1), a, a)
    const = np.exp(special.gammaln(d / 2) - special.gammaln((d - 1) / 2)) / np.sqrt(np.pi)
    p = 0.5 * (d - 3)
    prim = lambda t: -((1 - t * t) ** (p + 1)) / (2 * (p + 1))
    return mass, const * (prim(hi) - prim(lo))


def _continuous_lloyd(d, b, iters=20000):
    k = 1 << b
    c = (np.arange(k) - (k - 1) / 2) * 1.0 / np.sqrt(d)
    for _ in range(iters):
        t = np.concatenate([[-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]])
        new = np.empty(k)
        for j in range(k):
            m, mom = _beta_cell_mass_moment(t[j], t[j + 1], d)
            new[j] = mom / m
        if np.max(np.abs(new - c)) < 1e-15:
            c = new
            break
        c = new
    return c


@pytest.mark.parametrize("d,b", [(128, 2), (128, 3), (128, 4), (1536, 3)])
def test_grid_recipe_near_continuous_optimum(d, b):
    opt = _continuous_lloyd(d, b)
    cb = oracle.codebook(d, b)
    assert np.max(np.abs(cb.centroids - opt)) * np.sqrt(d) <= 5e-3


def _dmse_coordinate(cb, d):
    # E[(y - Q(y))^2] for one coordinate under the exact Beta density (quadrature per cell).
    c = cb.centroids
    t = np.concatenate([[-1.0], cb.thresholds, [1.0]])
    const = np.exp(special.gammaln(d / 2) - special.gammaln((d - 1) / 2)) / np.sqrt(np.pi)
    tot = 0.0
    for j in range(c.size):
        f = lambda x, cj=c[j]: (x - cj) ** 2 * const * (1 - x * x) ** (0.5 * (d - 3))
        v, _ = integrate.quad(f, t[j], t[j + 1], epsabs=1e-14, epsrel=1e-12, limit=200)
        tot += v
    return tot


def test_distortion_table_and_bound(golden):
    ex = golden["distortion_table"]
    for b, printed in zip(ex["bits"], ex["printed_dmse"]):
        # printed with few significant digits: agree to half a unit of the last printed digit
        digits = len(repr(printed).split(".")[1])
        d = 1536
        dm = d * _dmse_coordinate(oracle.codebook(d, b), d)
        assert abs(dm - printed) <= 0.5 * 10.0 ** -digits + 1e-12, (b, dm, printed)
        for d in (64, 128, 1536):
            dm = d * _dmse_coordinate(oracle.codebook(d, b), d)
            assert dm <= np.sqrt(3) * np.pi / 2 * 4.0 ** -b
            assert dm >= 4.0 ** -b


def test_cosine_quality_synthetic_analogue(golden):
    ex = golden["cosine_quality"]
    d = 128
    rot = oracle.dense_rotation(d, 1)
    x = np.random.default_rng(5).standard_normal((4096, d))
    for b, printed in zip(ex["bits"], ex["printed_cosine"]):
        cb = oracle.codebook(d, b)
        enc = oracle.encode_mse(x, rot, cb)
        xh = oracle.decode_mse(enc.idx, enc.norms, rot, cb)
        cos = np.sum(x * xh, 1) / (np.linalg.norm(x, axis=1) * np.linalg.norm(xh, axis=1))
        assert abs(np.mean(cos) - printed) < 1e-3
