"""Structural and statistical pins of the oracle's generator and rotations.

The generator's exact values are fixed by no page ("parity unpinned"); these checks pin the
published SplitMix64 definition by its reference outputs, the Box-Muller Gaussian by its
moments, and the rotations by orthogonality, norm preservation, explicit Hadamard entries
and the Haar law of a rotated unit vector."""

import numpy as np
import pytest
from scipy import stats

import oracle


def test_splitmix64_reference_outputs():
    # First outputs of the published SplitMix64 reference generator started from state 0.
    z = oracle.splitmix64(0, 3)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_splitmix64_counter_property():
    a = oracle.splitmix64(12345, 100)
    b = oracle.splitmix64(12345, 40, offset=60)
    np.testing.assert_array_equal(a[60:], b)
    assert not np.array_equal(oracle.splitmix64(1, 10), oracle.splitmix64(2, 10))


def test_uniform_is_uniform():
    u = oracle.uniform53(oracle.splitmix64(7, 200000))
    assert u.min() >= 0.0 and u.max() < 1.0
    assert stats.kstest(u, "uniform").pvalue > 1e-4


def test_gaussian_moments():
    n = 400000
    g = oracle.gaussian(3, n)
    se = 1.0 / np.sqrt(n)
    assert abs(g.mean()) < 4 * se
    assert abs(g.var() - 1.0) < 4 * np.sqrt(2.0) * se
    assert abs(stats.skew(g)) < 4 * np.sqrt(6.0) * se
    assert abs(stats.kurtosis(g)) < 4 * np.sqrt(24.0) * se
    assert stats.kstest(g, "norm").pvalue > 1e-4


def test_rademacher_balanced():
    s = oracle.rademacher(9, 100000)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 4 / np.sqrt(s.size)


@pytest.mark.parametrize("d", [2, 3, 64, 128, 256])
def test_dense_rotation_orthogonal(d):
    r = oracle.dense_rotation(d, 1)
    assert np.max(np.abs(r.T @ r - np.eye(d))) <= 1e-13
    x = np.random.default_rng(0).standard_normal((10, d))
    np.testing.assert_allclose(np.linalg.norm(x @ r.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(r, oracle.dense_rotation(d, 1))
    assert not np.allclose(r, oracle.dense_rotation(d, 2))


def test_dense_rotation_is_haar():
    # The first column of a Haar rotation is uniform on the sphere: each coordinate follows
    # the Beta law of the rotated-coordinate density ((x + 1)/2 ~ Beta((d-1)/2, (d-1)/2)).
    d = 16
    vals = np.concatenate([oracle.dense_rotation(d, s)[:, 0] for s in range(1500)])
    a = 0.5 * (d - 1)
    assert stats.kstest(0.5 * (vals + 1.0), stats.beta(a, a).cdf).pvalue > 1e-4
    # triangular factor sign convention: R = Q D makes the QR of G have a positive diagonal
    g = oracle.gaussian(1, d * d).reshape(d, d)
    r = oracle.dense_rotation(d, 1)
    tri = r.T @ g
    assert np.all(np.diag(tri) > 0)
    assert np.max(np.abs(np.tril(tri, -1))) < 1e-12


def test_sylvester_hadamard_entries():
    np.testing.assert_array_equal(oracle.sylvester_hadamard(1), [[1.0]])
    np.testing.assert_array_equal(oracle.sylvester_hadamard(2), [[1, 1], [1, -1]])
    h2 = oracle.sylvester_hadamard(2)
    np.testing.assert_array_equal(oracle.sylvester_hadamard(4), np.block([[h2, h2], [h2, -h2]]))
    h = oracle.sylvester_hadamard(128)
    np.testing.assert_array_equal(h @ h.T, 128 * np.eye(128))
    with pytest.raises(ValueError):
        oracle.sylvester_hadamard(96)


def _fwht(v):
    # in-place butterfly of the Sylvester transform (independent of the matrix form)
    v = v.copy()
    h = 1
    n = v.shape[-1]
    while h < n:
        v = v.reshape(*v.shape[:-1], n // (2 * h), 2, h)
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        v = v.reshape(*v.shape[:-3], n)
        h *= 2
    return v


def test_wht_rotation_matches_butterfly():
    d = 128
    r = oracle.wht_rotation(d, 1)
    assert np.max(np.abs(r.T @ r - np.eye(d))) <= 1e-13
    sigma = oracle.rademacher(1, d)
    u = np.random.default_rng(1).standard_normal((5, d))
    np.testing.assert_allclose(u @ r.T, _fwht(u * sigma) / np.sqrt(d), atol=1e-13)


@pytest.mark.parametrize("d", [128, 96, 1536])
def test_block_wht_rotation_structure(d):
    """Block (group-32) randomized Hadamard: orthogonal, zero outside the diagonal blocks, each
    block the Sylvester H_32 times its slice of the signs, and equal to a per-group butterfly."""
    g = 32
    r = oracle.block_wht_rotation(d, 3, g)
    assert np.max(np.abs(r.T @ r - np.eye(d))) <= 1e-13
    sigma = oracle.rademacher(3, d)
    blocks = np.arange(d) // g
    assert np.all(r[blocks[:, None] != blocks[None, :]] == 0.0)
    h = oracle.sylvester_hadamard(g)
    for k in range(0, d, g):
        np.testing.assert_array_equal(r[k:k + g, k:k + g], h * sigma[None, k:k + g] / np.sqrt(g))
    u = np.random.default_rng(2).standard_normal((4, d))
    ref = _fwht((u * sigma).reshape(4, d // g, g)).reshape(4, d) / np.sqrt(g)
    np.testing.assert_allclose(u @ r.T, ref, atol=1e-13)


def test_block_wht_reduces_to_full_wht():
    np.testing.assert_array_equal(oracle.block_wht_rotation(32, 5, 32), oracle.wht_rotation(32, 5))
    with pytest.raises(ValueError):
        oracle.block_wht_rotation(100, 1, 32)
