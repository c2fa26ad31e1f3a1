"""Pins of the oracle to the worked examples the pages print (fixtures in tests/golden)."""

import numpy as np
import pytest

import oracle


def test_one_bit_example(golden):
    ex = golden["one_bit_example"]
    cb = oracle.codebook_from_values(ex["codebook"])
    idx = oracle.nearest_index(ex["x"], cb.thresholds)
    assert idx.tolist() == ex["expected_idx"]
    assert "".join(str(int(i)) for i in idx) == ex["expected_bitstring"]
    np.testing.assert_allclose(cb.centroids[idx], ex["expected_xhat"], atol=0)
    # The bit string in coordinate order is the LSB-first stream: word 0b0101 once padded.
    padded = np.zeros(32, dtype=np.int64)
    padded[:4] = idx
    assert int(oracle.pack_bits(padded, 1)[0]) == 0b0101
    # 1-bit quantization is scale invariant, so the normalised encode gives the same bits.
    enc = oracle.encode_mse(np.array(ex["x"]), np.eye(4), cb)
    assert enc.idx.tolist() == ex["expected_idx"]


def test_two_bit_uniform_vs_nonuniform(golden):
    ex = golden["two_bit_uniform_vs_lloyd"]
    x = np.array(ex["x"])
    cu = oracle.codebook_from_values(ex["uniform_codebook"])
    cn = oracle.codebook_from_values(ex["nonuniform_codebook"])
    xu = cu.centroids[oracle.nearest_index(x, cu.thresholds)]
    xn = cn.centroids[oracle.nearest_index(x, cn.thresholds)]
    np.testing.assert_allclose(xu, ex["expected_xhat_uniform"], atol=1e-15)
    np.testing.assert_allclose(xn, ex["expected_xhat_nonuniform"], atol=1e-15)
    # The printed "MSE" is the per-coordinate mean of the squared error (5 decimals).
    half = 0.5 * 10.0 ** -ex["mse_print_digits"]
    assert abs(np.mean((x - xu) ** 2) - ex["expected_mse_uniform"]) <= half
    assert abs(np.mean((x - xn) ** 2) - ex["expected_mse_nonuniform"]) <= half
    red = 100.0 * (1.0 - np.mean((x - xn) ** 2) / np.mean((x - xu) ** 2))
    assert round(red) == ex["expected_mse_reduction_percent"]
    y = np.array(ex["query"])
    assert abs(y @ x - ex["expected_ip_true"]) <= 5e-4
    assert abs(y @ xu - ex["expected_ip_uniform"]) <= 5e-4
    assert abs(y @ xn - ex["expected_ip_nonuniform"]) <= 5e-4
    assert abs(abs(y @ x - y @ xu) - ex["expected_ip_abs_err_uniform"]) <= 5e-4
    assert abs(abs(y @ x - y @ xn) - ex["expected_ip_abs_err_nonuniform"]) <= 5e-4


def test_lloyd_max_four_points(golden):
    ex = golden["lloyd_max_four_points"]
    pts = np.array(ex["points"], dtype=float)
    w = np.ones_like(pts)
    init = np.array(ex["init"], dtype=float)
    assert 0.5 * (init[0] + init[1]) == ex["expected_threshold_iter1"]
    c1 = oracle.lloyd_max_points(pts, w, init, 1)
    np.testing.assert_array_equal(c1, ex["expected_after_iter1"])
    assert 0.5 * (c1[0] + c1[1]) == ex["expected_threshold_iter2"]
    c2 = oracle.lloyd_max_points(pts, w, init, 2)
    np.testing.assert_array_equal(c2, ex["expected_after_iter2"])
    # converged: further iterations change nothing
    np.testing.assert_array_equal(oracle.lloyd_max_points(pts, w, init, 50), c2)


def test_rotation_2d_example(golden):
    ex = golden["rotation_2d_example"]
    rot = oracle.rotation_from_matrix(ex["rotation"])
    cb = oracle.codebook_from_values(ex["codebook"])
    enc = oracle.encode_mse(np.array([ex["x"]]), rot, cb)
    np.testing.assert_allclose(enc.y[0], ex["expected_y"], atol=1e-15)
    assert enc.idx[0].tolist() == ex["expected_idx"]
    np.testing.assert_allclose(cb.centroids[enc.idx[0]], ex["expected_yhat"], atol=0)
    xhat = oracle.decode_mse(enc.idx, enc.norms, rot, cb)[0]
    np.testing.assert_allclose(xhat, ex["expected_xhat"], atol=1e-12)


def test_prod_qjl_example(golden):
    ex = golden["prod_qjl_2d_example"]
    x = np.array(ex["x"])
    xm = np.array(ex["xhat_mse_given"])
    smat = np.array(ex["s_matrix"])
    r = x - xm
    np.testing.assert_allclose(r, ex["expected_residual"], atol=1e-15)
    # Feed the printed residual exactly: (S r)_2 is then 0 up to one rounding (a fused
    # multiply-add may leave ~1e-18), and the page's sign rule gives +1 either way.
    r_exact = np.array(ex["expected_residual"])
    z, gamma, proj = oracle.qjl_encode(r_exact, smat)
    assert abs(gamma - ex["expected_gamma"]) <= 5e-5
    np.testing.assert_allclose(proj, ex["expected_sr"], atol=5e-5)
    assert abs(proj[1]) < 1e-15
    assert np.where(z, 1, -1).tolist() == ex["expected_signs"]
    zpm = np.where(z, 1.0, -1.0)
    np.testing.assert_allclose(smat.T @ zpm, ex["expected_st_signs"], atol=1e-12)
    scale = gamma * oracle.QJL_CONST / 2
    assert abs(scale - ex["expected_scale"]) <= 5e-5
    corr = oracle.qjl_correction(z, gamma, smat)
    np.testing.assert_allclose(corr, ex["expected_corr"], atol=5e-4)
    xp = xm + corr
    np.testing.assert_allclose(xp, ex["expected_xhat_prod"], atol=5e-4)
    y = np.array(ex["query"])
    assert abs(y @ xp - ex["expected_ip_prod"]) <= 5e-4
    assert abs(y @ x - ex["expected_ip_true"]) <= 1e-12
    assert abs(y @ xm - ex["expected_ip_mse"]) <= 1e-12


def test_sign_of_zero_is_plus_one():
    # sign(0) = +1, for +0.0 and -0.0 alike (the page's convention in the prod example).
    smat = np.array([[1.0, 0.0], [0.0, -1.0], [0.0, 0.0]])
    z, gamma, proj = oracle.qjl_encode(np.zeros((1, 2)), smat[:2])
    assert z.tolist() == [[True, True]] and gamma[0] == 0.0
    z, _, proj = oracle.qjl_encode(np.array([[0.0, 0.0]]), np.array([[-1.0, 0.0], [0.0, -1.0]]))
    assert z.tolist() == [[True, True]]


def test_prod_example_through_encode():
    """The same example through the full prod encode: with a codebook chosen so that the MSE
    stage returns the printed x_hat_mse, the residual, gamma and the first sign follow."""
    x = np.array([[0.8, 0.5]])
    s = np.linalg.norm(x[0])
    a, b = 0.7 / s, 0.6 / s
    cb = oracle.codebook_from_values([-a, -b, b, a])
    smat = np.array([[0.707, -0.707], [0.707, 0.707]])
    encp = oracle.encode_prod(x, np.eye(2), cb, smat)
    xm = oracle.decode_mse(encp.mse.idx, encp.mse.norms, np.eye(2), cb)
    np.testing.assert_allclose(xm[0], [0.7, 0.6], atol=1e-15)
    assert abs(encp.gamma[0] - np.sqrt(0.02)) <= 1e-12
    assert bool(encp.z[0, 0])
    assert abs(encp.proj[0, 1]) < 1e-15
