"""Pins of the outlier-channel split oracle (oracle/split.py): reduction to two plain encodes,
channel relabelling, the score in the two rotated domains element by element, and each part's
distortion against the exact value of its codebook."""

import numpy as np
import torch
import pytest

import oracle
from test_oracle_quantizer import _dmse_quadrature

D = 128
M = D // 2


def _setup(bo, br):
    return (oracle.dense_rotation(M, 5), oracle.dense_rotation(M, 6),
            oracle.codebook(M, bo), oracle.codebook(M, br))


def _outliers(heads, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(D)[:M] for _ in range(heads)])


def test_channel_order_is_a_permutation_and_validates():
    out = _outliers(3, 1)
    order = oracle.channel_order(out, D)
    for h in range(3):
        assert sorted(order[h].tolist()) == list(range(D))
        assert order[h, :M].tolist() == out[h].tolist()
        assert np.all(np.diff(order[h, M:]) > 0)
    with pytest.raises(ValueError):
        oracle.channel_order(np.zeros((1, M), dtype=np.int64), D)   # repeated channel
    with pytest.raises(ValueError):
        oracle.channel_order(out[:, :M - 1], D)                     # not half of the channels
    bad = out.copy()
    bad[0, 0] = D
    with pytest.raises(ValueError):
        oracle.channel_order(bad, D)


def test_identity_split_is_two_plain_encodes():
    # Outliers = the first half of the channels: the codes are plain TurboQuant_mse codes of the
    # two halves of every vector.
    rot_o, rot_r, cb_o, cb_r = _setup(3, 2)
    x = np.random.default_rng(2).standard_normal((2, 2, 9, D))
    enc = oracle.encode_split(x, np.tile(np.arange(M), (2, 1)), rot_o, rot_r, cb_o, cb_r)
    a = oracle.encode_mse(x[..., :M], rot_o, cb_o)
    b = oracle.encode_mse(x[..., M:], rot_r, cb_r)
    assert np.array_equal(enc.outlier.idx, a.idx) and np.array_equal(enc.rest.idx, b.idx)
    np.testing.assert_allclose(enc.outlier.norms, np.linalg.norm(x[..., :M], axis=-1), rtol=1e-14)
    np.testing.assert_allclose(enc.rest.norms, np.linalg.norm(x[..., M:], axis=-1), rtol=1e-14)
    # budget: 64 b_o + 64 b_r bits per vector, 2.5 bits per channel
    assert enc.outlier.words.shape[-1] + enc.rest.words.shape[-1] == D * 5 // 2 // 32


def test_relabelling_channels_leaves_the_codes_unchanged():
    # Permuting the channels of every vector and mapping the outlier lists through the same
    # permutation must give identical codes and a reconstruction permuted the same way.
    rot_o, rot_r, cb_o, cb_r = _setup(4, 3)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 2, 11, D))
    out = _outliers(2, 4)
    pi = rng.permutation(D)          # new channel c holds old channel pi[c]
    inv = np.argsort(pi)
    xp = x[..., pi]
    # the outlier part keeps its listed order; the rest is ordered by channel, so compare with
    # the rest re-sorted by the new labels
    e1 = oracle.encode_split(x, out, rot_o, rot_r, cb_o, cb_r)
    e2 = oracle.encode_split(xp, inv[out], rot_o, rot_r, cb_o, cb_r)
    assert np.array_equal(e1.outlier.idx, e2.outlier.idx)
    np.testing.assert_allclose(e1.rest.norms, e2.rest.norms, rtol=1e-14)
    x1 = oracle.decode_split(e1, rot_o, rot_r, cb_o, cb_r)
    x2 = oracle.decode_split(e2, rot_o, rot_r, cb_o, cb_r)
    # the rest parts see their channels in another order, hence different codes; the outlier
    # part's reconstruction is the same vector on relabelled channels
    for h in range(2):
        np.testing.assert_allclose(x2[:, h][..., inv[out[h]]], x1[:, h][..., out[h]], rtol=0, atol=1e-12)


def test_scores_match_the_rotated_domain_sum():
    # <q, x_hat> against s_o <R_o q_O, C_o[idx_o]> + s_r <R_r q_R, C_r[idx_r]>, element by
    # element in plain loops, with q_O and q_R gathered by the channel order.
    rot_o, rot_r, cb_o, cb_r = _setup(3, 2)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 2, 5, D))
    q = rng.standard_normal((1, 4, D))
    out = _outliers(2, 6)
    enc = oracle.encode_split(x, out, rot_o, rot_r, cb_o, cb_r)
    sc = oracle.scores_split(q, enc, rot_o, rot_r, cb_o, cb_r)
    order = oracle.channel_order(out, D)
    for hq in range(4):
        h = hq // 2
        for t in range(5):
            tot = 0.0
            for part, rot, cb, off in ((enc.outlier, rot_o, cb_o, 0), (enc.rest, rot_r, cb_r, M)):
                acc = 0.0
                for i in range(M):
                    qi = sum(rot[i][j] * q[0, hq, order[h, off + j]] for j in range(M))
                    acc += qi * cb.centroids[part.idx[0, h, t, i]]
                tot += part.norms[0, h, t] * acc
            assert abs(sc[0, hq, t] - tot) <= 1e-11 * (1 + abs(tot))


@pytest.mark.parametrize("bo,br", [(3, 2), (4, 3)])
def test_part_distortion_matches_the_codebook(bo, br):
    # For isotropic keys (random directions inside each part), E ||x_part - x_hat_part||^2 /
    # ||x_part||^2 is the distortion of that part's codebook (dimension d/2), computed here by
    # quadrature of the exact coordinate density; the mixed budget's distortion lies between
    # the plain b_r and b_o codes'.
    rot_o, rot_r, cb_o, cb_r = _setup(bo, br)
    rng = np.random.default_rng(7)
    n = 4096
    x = rng.standard_normal((1, 1, n, D))
    out = _outliers(1, 8)
    enc = oracle.encode_split(x, out, rot_o, rot_r, cb_o, cb_r)
    xh = oracle.decode_split(enc, rot_o, rot_r, cb_o, cb_r)
    order = enc.order[0]
    for sl, b in ((order[:M], bo), (order[M:], br)):
        rel = np.sum((x[..., sl] - xh[..., sl]) ** 2, axis=-1) / np.sum(x[..., sl] ** 2, axis=-1)
        m, se = rel.mean(), rel.std() / np.sqrt(n)
        assert abs(m - _dmse_quadrature(M, b)) < 4 * se
    tot = np.sum((x - xh) ** 2) / np.sum(x ** 2)
    assert _dmse_quadrature(M, bo) < tot < _dmse_quadrature(M, br)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (2, 2), (8, 1)])
def test_decode_attention_matches_torch_sdpa(hq, hkv):
    # softmax(scale q K_hat^T) V_hat by torch's scaled_dot_product_attention (float64, CPU) on the
    # split reconstruction of the keys and the decoded values
    d, m, B, T, scale = 16, 8, 2, 29, 0.37
    rng = np.random.default_rng(hq + 10 * hkv)
    x = rng.standard_normal((B, hkv, T, d)) * rng.lognormal(0, 0.5, (B, hkv, T, 1))
    outl = np.stack([rng.permutation(d)[:m] for _ in range(hkv)])
    ro, rr, rv = oracle.dense_rotation(m, 3), oracle.dense_rotation(m, 4), oracle.dense_rotation(d, 1)
    co, cr, cv = oracle.codebook(m, 3), oracle.codebook(m, 2), oracle.codebook(d, 2)
    enc = oracle.encode_split(x, outl, ro, rr, co, cr)
    v = rng.standard_normal((B, hkv, T, d))
    ve = oracle.encode_mse(v.reshape(-1, d), rv, cv)
    vi, vn = ve.idx.reshape(B, hkv, T, d), ve.norms.reshape(B, hkv, T)
    q = rng.standard_normal((B, hq, d))
    got = oracle.decode_attention_split(q, enc, vi, vn, ro, rr, rv, co, cr, cv, scale)
    k_hat = oracle.decode_split(enc, ro, rr, co, cr)
    ratio = hq // hkv
    for b in range(B):
        for g in range(hkv):
            v_hat = torch.from_numpy(oracle.decode_mse(vi[b, g], vn[b, g], rv, cv))
            qs = torch.from_numpy(q[b, g * ratio:(g + 1) * ratio]).unsqueeze(1)
            kh = torch.from_numpy(k_hat[b, g]).expand(ratio, -1, -1)
            ref = torch.nn.functional.scaled_dot_product_attention(qs, kh, v_hat.expand(ratio, -1, -1), scale=scale)
            np.testing.assert_allclose(got[b, g * ratio:(g + 1) * ratio], ref[:, 0].numpy(), rtol=0, atol=1e-12)
