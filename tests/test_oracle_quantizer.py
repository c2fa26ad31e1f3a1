"""Pins of the oracle's quantizer, packed format, scores, attention and top-k: brute force on
tiny inputs, invariants, and the statistical properties the pages state (2/pi shrinkage of the
1-bit MSE inner product; unbiasedness of the prod estimator; distortion)."""

import itertools

import numpy as np
import pytest
from scipy import special

import oracle


def _argmin_ties_up(y, c):
    out = []
    for v in y:
        dist = [abs(v - ck) for ck in c]
        m = min(dist)
        out.append(max(k for k, dk in enumerate(dist) if dk == m))
    return out


def test_nearest_index_is_argmin_with_ties_up():
    rng = np.random.default_rng(0)
    for b in (1, 2, 3, 4):
        cb = oracle.codebook(128, b)
        y = rng.standard_normal(2000) / np.sqrt(128)
        assert oracle.nearest_index(y, cb.thresholds).tolist() == _argmin_ties_up(y, cb.centroids)
    # exact midpoints go up
    cb = oracle.codebook_from_values([-1.0, 0.0, 1.0, 3.0])
    assert oracle.nearest_index([-0.5, 0.5, 2.0], cb.thresholds).tolist() == [1, 2, 3]
    assert _argmin_ties_up([-0.5, 0.5, 2.0], cb.centroids) == [1, 2, 3]


def _pack_bruteforce(idx, b):
    bits = []
    for v in idx:
        for j in range(b):
            bits.append((int(v) >> j) & 1)
    words = []
    for w in range(len(bits) // 32):
        words.append(sum(bits[32 * w + i] << i for i in range(32)))
    return words


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_pack_matches_bitwise_definition(b):
    rng = np.random.default_rng(b)
    d = 64
    idx = rng.integers(0, 1 << b, size=(3, d))
    words = oracle.pack_bits(idx, b)
    for row in range(3):
        assert words[row].tolist() == _pack_bruteforce(idx[row], b)
    np.testing.assert_array_equal(oracle.unpack_bits(words, d, b), idx)


def test_pack_three_bit_straddle():
    # coordinate 10 of a 3-bit stream occupies bits 30, 31 of word 0 and bit 0 of word 1
    idx = np.zeros(32, dtype=np.int64)
    idx[10] = 0b101
    w = oracle.pack_bits(idx, 3)
    assert int(w[0]) == (1 << 30) and int(w[1]) == 1 and int(w[2]) == 0
    with pytest.raises(ValueError):
        oracle.pack_bits(np.zeros(10, dtype=np.int64), 3)
    with pytest.raises(ValueError):
        oracle.pack_bits(np.full(32, 8), 3)


def _token_blocked_bruteforce(idx, b):
    n, d = idx.shape
    nblk = (n + 31) // 32
    out = []
    for beta in range(nblk):
        bits = []
        for o in range(4):
            for c in range(d):
                for e in range(8):
                    r = 32 * beta + 8 * o + e
                    v = int(idx[r, c]) if r < n else 0
                    bits.extend((v >> j) & 1 for j in range(b))
        out.append([sum(bits[32 * w + i] << i for i in range(32)) for w in range(len(bits) // 32)])
    return out


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("n", [32, 45, 70])
def test_token_blocked_layout(b, n):
    d = 32
    idx = np.random.default_rng(n * b).integers(0, 1 << b, size=(n, d))
    w = oracle.pack_token_blocked(idx, b)
    assert w.shape == ((n + 31) // 32, d * b)
    assert w.tolist() == _token_blocked_bruteforce(idx, b)
    np.testing.assert_array_equal(oracle.unpack_token_blocked(w, n, d, b), idx)


def test_token_blocked_first_chunk():
    # rows 0..7 at coordinate 0 form the first chunk: 2-bit indices 0,1,2,3,0,1,2,3 -> 0xE4E4
    idx = np.zeros((32, 4), dtype=np.int64)
    idx[:8, 0] = [0, 1, 2, 3, 0, 1, 2, 3]
    w = oracle.pack_token_blocked(idx, 2)
    assert int(w[0, 0]) & 0xFFFF == 0xE4E4


def test_zero_vector():
    d = 128
    cb = oracle.codebook(d, 3)
    rot = oracle.dense_rotation(d, 1)
    enc = oracle.encode_mse(np.zeros((1, d)), rot, cb)
    assert enc.norms[0] == 0.0
    assert np.all(enc.idx == 4)            # y = 0 sits on the middle threshold -> upper index
    np.testing.assert_array_equal(oracle.decode_mse(enc.idx, enc.norms, rot, cb), 0.0)
    smat = oracle.qjl_matrix(d, 2)
    encp = oracle.encode_prod(np.zeros((1, d)), rot, oracle.codebook(d, 2), smat)
    assert encp.gamma[0] == 0.0 and np.all(encp.z)
    q = np.ones((1, d))
    assert oracle.scores_prod(q, encp, rot, oracle.codebook(d, 2), smat)[0, 0] == 0.0


def test_rotation_preserves_error():
    # ||x - x_hat|| = s ||y - y_hat||  (error in the rotated domain equals the original one)
    d = 128
    rot = oracle.dense_rotation(d, 1)
    cb = oracle.codebook(d, 3)
    x = np.random.default_rng(2).standard_normal((50, d)) * 3.0
    enc = oracle.encode_mse(x, rot, cb)
    xh = oracle.decode_mse(enc.idx, enc.norms, rot, cb)
    lhs = np.linalg.norm(x - xh, axis=1)
    rhs = enc.norms * np.linalg.norm(enc.y - cb.centroids[enc.idx], axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12)


def test_scores_equal_inner_product_with_reconstruction():
    d = 128
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, d))
    q = rng.standard_normal((6, d))
    for rot in (oracle.dense_rotation(d, 1), oracle.wht_rotation(d, 1)):
        cb = oracle.codebook(d, 2)
        enc = oracle.encode_mse(x, rot, cb)
        xh = oracle.decode_mse(enc.idx, enc.norms, rot, cb)
        np.testing.assert_allclose(oracle.scores_mse(q, enc.idx, enc.norms, rot, cb), q @ xh.T,
                                   rtol=1e-12, atol=1e-12)
        smat = oracle.qjl_matrix(d, 2)
        encp = oracle.encode_prod(x, rot, cb, smat)
        xp = oracle.decode_prod(encp, rot, cb, smat)
        np.testing.assert_allclose(oracle.scores_prod(q, encp, rot, cb, smat), q @ xp.T,
                                   rtol=1e-12, atol=1e-12)
        # residual in the original scale
        np.testing.assert_allclose(encp.gamma, np.linalg.norm(x - xh, axis=1), rtol=1e-12)


def _mc_dmse(d, b, n=4096, seed=4):
    rot = oracle.dense_rotation(d, 1)
    cb = oracle.codebook(d, b)
    x = np.random.default_rng(seed).standard_normal((n, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    enc = oracle.encode_mse(x, rot, cb)
    err = np.sum((x - oracle.decode_mse(enc.idx, enc.norms, rot, cb)) ** 2, axis=1)
    return err.mean(), err.std() / np.sqrt(n)


def _dmse_quadrature(d, b):
    # d * E[(y - Q(y))^2] under the exact rotated-coordinate density, by quadrature per cell
    from scipy import integrate
    cb = oracle.codebook(d, b)
    t = np.concatenate([[-1.0], cb.thresholds, [1.0]])
    const = np.exp(special.gammaln(d / 2) - special.gammaln((d - 1) / 2)) / np.sqrt(np.pi)
    tot = 0.0
    for j, cj in enumerate(cb.centroids):
        f = lambda x: (x - cj) ** 2 * const * (1 - x * x) ** (0.5 * (d - 3))
        tot += integrate.quad(f, t[j], t[j + 1], epsabs=1e-14, epsrel=1e-12, limit=200)[0]
    return d * tot


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_distortion_monte_carlo(b):
    # The pipeline (rotate, quantize, reconstruct) over random unit vectors must reproduce the
    # distortion the density predicts for the codebook, within 3 standard errors.
    grid_exact = _dmse_quadrature(128, b)
    m, se = _mc_dmse(128, b)
    assert abs(m - grid_exact) < 3 * se + 1e-5
    assert m < np.sqrt(3) * np.pi / 2 * 4.0 ** -b


@pytest.mark.slow
def test_one_bit_shrinkage_two_over_pi():
    # 1-bit MSE: E_R <q, x_hat> = d c_1 E|u_1| <q, x>, E|u_1| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)),
    # a factor that tends to 2/pi (the walkthrough page's shrinkage constant).
    d = 128
    cb = oracle.codebook(d, 1)
    e_abs = np.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / np.sqrt(np.pi)
    factor = d * cb.centroids[1] * e_abs
    assert abs(factor - 0.6391) < 5e-4
    assert abs(d * e_abs * e_abs - 2 / np.pi) < 3e-3
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, d))
    q = x[0] + 0.5 * rng.standard_normal(d)
    ratios = []
    for seed in range(2000):
        rot = oracle.dense_rotation(d, 1000 + seed)
        enc = oracle.encode_mse(x, rot, cb)
        ratios.append(oracle.scores_mse(q[None], enc.idx, enc.norms, rot, cb)[0, 0])
    ratios = np.array(ratios) / (q @ x[0])
    assert abs(ratios.mean() - factor) < 4 * ratios.std() / np.sqrt(ratios.size)


@pytest.mark.slow
def test_prod_unbiased_and_variance():
    d = 128
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, d))
    q = rng.standard_normal(d)
    rot = oracle.dense_rotation(d, 1)
    cb = oracle.codebook(d, 2)
    est = []
    for seed in range(4000):
        smat = oracle.qjl_matrix(d, 10000 + seed)
        encp = oracle.encode_prod(x, rot, cb, smat)
        est.append(oracle.scores_prod(q[None], encp, rot, cb, smat)[0, 0])
    est = np.array(est)
    truth = q @ x[0]
    assert abs(est.mean() - truth) < 4 * est.std() / np.sqrt(est.size)
    # variance (pi / 2d) gamma^2 (||q||^2 - (2/pi) <q, r/gamma>^2); the MSE part is fixed
    enc = oracle.encode_mse(x, rot, cb)
    r = x[0] - oracle.decode_mse(enc.idx, enc.norms, rot, cb)[0]
    g = np.linalg.norm(r)
    pred = np.pi / (2 * d) * g * g * (q @ q - 2 / np.pi * (q @ r / g) ** 2)
    assert abs(est.var() / pred - 1.0) < 0.1
    # MSE-only is biased (shrinks), prod is not
    mse_only = oracle.scores_mse(q[None], enc.idx, enc.norms, rot, cb)[0, 0]
    assert abs(mse_only - (q @ (x[0] - r))) < 1e-9


def test_quantize_rotated_float32_decision():
    cb = oracle.codebook(128, 3)
    t32 = cb.thresholds.astype(np.float32)
    y = np.concatenate([t32, np.nextafter(t32, np.float32(-1)), np.nextafter(t32, np.float32(1))])
    idx = oracle.quantize_rotated(y, cb)
    k = np.arange(7)
    np.testing.assert_array_equal(idx[:7], k + 1)       # on the threshold -> upper cell
    np.testing.assert_array_equal(idx[7:14], k)
    np.testing.assert_array_equal(idx[14:], k + 1)


def test_decode_attention_special_cases():
    d = 32
    rot = oracle.dense_rotation(d, 1)
    cb = oracle.codebook(d, 2)
    rng = np.random.default_rng(8)
    # T = 1: output is v_hat
    k = rng.standard_normal((1, 1, 1, d))
    v = rng.standard_normal((1, 1, 1, d))
    ek, ev = oracle.encode_mse(k, rot, cb), oracle.encode_mse(v, rot, cb)
    q = rng.standard_normal((1, 2, d))
    out = oracle.decode_attention(q, ek.idx, ek.norms, ev.idx, ev.norms, rot, rot, cb, cb, 0.3)
    vh = oracle.decode_mse(ev.idx, ev.norms, rot, cb)[0, 0, 0]
    np.testing.assert_allclose(out[0, 0], vh, atol=1e-14)
    np.testing.assert_allclose(out[0, 1], vh, atol=1e-14)
    # equal logits (identical keys): output is the mean of v_hat
    kk = np.repeat(k, 5, axis=2)
    vv = rng.standard_normal((1, 1, 5, d))
    ek, ev = oracle.encode_mse(kk, rot, cb), oracle.encode_mse(vv, rot, cb)
    out = oracle.decode_attention(q, ek.idx, ek.norms, ev.idx, ev.norms, rot, rot, cb, cb, 0.3)
    vh = oracle.decode_mse(ev.idx, ev.norms, rot, cb)[0, 0]
    np.testing.assert_allclose(out[0, 0], vh.mean(axis=0), atol=1e-13)


def test_decode_attention_bruteforce_and_gqa():
    d, t, hkv, hq = 32, 7, 2, 4
    rot = oracle.dense_rotation(d, 1)
    cbk, cbv = oracle.codebook(d, 3), oracle.codebook(d, 2)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((1, hkv, t, d))
    v = rng.standard_normal((1, hkv, t, d))
    q = rng.standard_normal((1, hq, d))
    ek, ev = oracle.encode_mse(k, rot, cbk), oracle.encode_mse(v, rot, cbv)
    out = oracle.decode_attention(q, ek.idx, ek.norms, ev.idx, ev.norms, rot, rot, cbk, cbv, 0.25)
    for h in range(hq):
        g = h // (hq // hkv)
        kh = [ek.norms[0, g, j] * sum(cbk.centroids[ek.idx[0, g, j, i]] * rot[i] for i in range(d))
              for j in range(t)]
        vh = [ev.norms[0, g, j] * sum(cbv.centroids[ev.idx[0, g, j, i]] * rot[i] for i in range(d))
              for j in range(t)]
        logits = [0.25 * float(np.dot(q[0, h], kj)) for kj in kh]
        mx = max(logits)
        w = [np.exp(l - mx) for l in logits]
        ref = sum(wj * vj for wj, vj in zip(w, vh)) / sum(w)
        np.testing.assert_allclose(out[0, h], ref, atol=1e-12)


def test_topk_bruteforce_with_ties():
    s = np.array([[0.5, 0.9, 0.9, -1.0, 0.9, 0.1]])
    vals, inds = oracle.topk(s, 4)
    assert inds[0].tolist() == [1, 2, 4, 0]
    rng = np.random.default_rng(10)
    s = np.round(rng.standard_normal((20, 50)), 1)
    vals, inds = oracle.topk(s, 10)
    for i in range(20):
        ref = sorted(range(50), key=lambda j: (-s[i, j], j))[:10]
        assert inds[i].tolist() == ref
        np.testing.assert_array_equal(vals[i], s[i, ref])
