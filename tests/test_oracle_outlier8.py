"""Pins of the oracle's outlier-8 keys (outlier channels at 8 bits, the rest TurboQuant_mse):
"TurboQuant 和 RotorQuant 的真相", the different needs of K and V (outlier channels at 8 bits,
the others at 3).  The readings are stated in oracle/outlier8.py; here they are checked against
brute force, the reconstruction's definition channel by channel, the identity of the two score
formulas, and the d = 128 distortion of the rest code."""

import numpy as np
import pytest
import torch

import oracle
from oracle import outlier8 as o8


def _brute_int8(v):
    """Nearest of the 255 levels scale * k, ties to the even k, by exhaustive comparison."""
    v = np.asarray(v, dtype=np.float64)
    amax = np.max(np.abs(v))
    if amax == 0:
        return np.zeros(v.shape, dtype=np.int8), 0.0
    scale = amax / 127.0
    ks = np.arange(-127, 128)
    out = np.empty(v.shape, dtype=np.int8)
    for i, x in enumerate(v):
        dist = np.abs(x / scale - ks)
        best = np.flatnonzero(dist == dist.min())
        out[i] = ks[best[0]] if best.size == 1 else [k for k in ks[best] if k % 2 == 0][0]
    return out, scale


def test_int8_absmax_is_the_nearest_level():
    rng = np.random.default_rng(0)
    rows = [rng.standard_normal(8) * 5, rng.standard_normal(4), np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5]),
            np.zeros(4), np.array([-3.0, 1.0, 0.0, 2.0])]
    for v in rows:
        q, s = o8.int8_absmax(v)
        qb, sb = _brute_int8(v)
        assert s == sb
        np.testing.assert_array_equal(q, qb)
        if s > 0:
            assert np.max(np.abs(q)) == 127 and np.all(np.abs(v - s * q) <= s / 2 + 1e-12)
    # float32 decisions: the same rule in float32 arithmetic (exact inputs, correctly rounded
    # divisions), checked against the brute force on float32 scales
    v = (rng.standard_normal(16) * 3).astype(np.float32)
    q, s = o8.int8_absmax(v, np.float32)
    assert s.dtype == np.float32 and s == np.float32(np.max(np.abs(v))) / np.float32(127)
    levels = np.arange(-127, 128, dtype=np.float32)
    for x, k in zip(v, q):
        r = x / s                                   # float32, as the decision is taken
        dist = np.abs(r.astype(np.float64) - levels)
        best = levels[dist == dist.min()]
        assert k == (best[0] if best.size == 1 else best[best % 2 == 0][0])
    # the printed ties: 2.5 -> 2, 3.5 -> 4, -2.5 -> -2 at scale 1
    q, s = o8.int8_absmax(np.array([127.0, 2.5, 3.5, -2.5]))
    assert s == 1.0 and list(q) == [127, 2, 4, -2]


def _keys(B, H, T, n_o, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, T, 128))
    outl = np.stack([rng.choice(128, size=n_o, replace=False) for _ in range(H)])
    for h in range(H):
        x[:, h][..., outl[h]] *= 8.0
    x *= rng.lognormal(0.0, 0.5, size=(B, H, T, 1))
    return x, outl


@pytest.mark.parametrize("n_o", [4, 8, 16])
def test_reconstruction_by_channel_and_score_identity(n_o):
    d, b, B, H, T = 128, 3, 2, 3, 40
    rot, cb = oracle.dense_rotation(d, 1), oracle.codebook(d, b)
    x, outl = _keys(B, H, T, n_o, seed=n_o)
    enc = o8.encode_outlier8(x, outl, rot, cb)
    mask = o8.rest_mask(outl)
    # the rest code is TurboQuant_mse of the key with its outlier channels zeroed
    xr = x * mask[None, :, None, :]
    np.testing.assert_allclose(enc.rest.norms, np.linalg.norm(xr, axis=-1), rtol=1e-14)
    ref_idx = oracle.encode_mse(xr.reshape(-1, d), rot, cb).idx.reshape(B, H, T, d)
    np.testing.assert_array_equal(enc.rest.idx, ref_idx)
    xh = o8.decode_outlier8(enc, rot, cb)
    full = oracle.decode_mse(enc.rest.idx.reshape(-1, d), enc.rest.norms.reshape(-1), rot, cb).reshape(B, H, T, d)
    for h in range(H):
        rest = mask[h]
        np.testing.assert_array_equal(xh[:, h][..., rest], full[:, h][..., rest])
        xo = x[:, h][..., outl[h]]
        s = enc.scale[:, h][..., None]
        assert np.all(np.abs(xh[:, h][..., outl[h]] - xo) <= s / 2 + 1e-12)
        np.testing.assert_allclose(s[..., 0], np.max(np.abs(xo), axis=-1) / 127.0, rtol=1e-15)
    # the score formula equals the inner product with the reconstruction
    hq = 2 * H
    q = np.random.default_rng(9).standard_normal((B, hq, d))
    sc = o8.scores_outlier8(q, enc, rot, cb)
    for h in range(hq):
        np.testing.assert_allclose(sc[:, h], np.einsum("btd,bd->bt", xh[:, h // 2], q[:, h]), rtol=1e-12, atol=1e-9)


def test_zero_outliers_and_zero_keys():
    d, b = 128, 2
    rot, cb = oracle.dense_rotation(d, 1), oracle.codebook(d, b)
    x, outl = _keys(1, 1, 3, 4, seed=1)
    x[0, 0, 0][outl[0]] = 0.0          # outlier part zero
    x[0, 0, 1] = 0.0                   # whole key zero
    enc = o8.encode_outlier8(x, outl, rot, cb)
    assert enc.scale[0, 0, 0] == 0.0 and np.all(enc.q8[0, 0, 0] == 0)
    assert enc.rest.norms[0, 0, 1] == 0.0 and np.all(enc.rest.idx[0, 0, 1] == 1 << (b - 1))
    xh = o8.decode_outlier8(enc, rot, cb)
    assert np.all(xh[0, 0, 1] == 0.0) and np.all(xh[0, 0, 0][outl[0]] == 0.0)


def test_rest_code_has_the_d128_distortion():
    # The masked keys are coded with the d = 128 rotation and codebook: their normalised error
    # E ||x_rest - x_hat_rest||^2 / ||x_rest||^2 sits at the d = 128, 3-bit value 0.03397 (grid codebook).
    d, b = 128, 3
    rot, cb = oracle.dense_rotation(d, 1), oracle.codebook(d, b)
    x, outl = _keys(1, 4, 1024, 4, seed=5)
    enc = o8.encode_outlier8(x, outl, rot, cb)
    mask = o8.rest_mask(outl)
    xr = (x * mask[None, :, None, :]).reshape(-1, d)
    full = oracle.decode_mse(enc.rest.idx.reshape(-1, d), enc.rest.norms.reshape(-1), rot, cb)
    e = np.sum((xr - full) ** 2, axis=1) / np.sum(xr ** 2, axis=1)
    assert abs(e.mean() - 0.03397) <= 3 * e.std() / np.sqrt(e.size) + 2e-4
    # keeping only the rest channels of the reconstruction never increases the error on them
    restricted = full * np.repeat(mask, 1024, axis=0)
    assert np.all(np.sum((xr - restricted) ** 2, axis=1) <= np.sum((xr - full) ** 2, axis=1) + 1e-12)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (3, 3), (8, 1)])
def test_decode_attention_matches_torch_sdpa(hq, hkv):
    # softmax(scale q K_hat^T) V_hat by torch's scaled_dot_product_attention (float64, CPU) on the
    # outlier-8 reconstruction of the keys and the decoded values
    d, B, T, scale = 128, 2, 37, 1 / np.sqrt(128)
    rot, cbk, cbv = oracle.dense_rotation(d, 1), oracle.codebook(d, 3), oracle.codebook(d, 2)
    x, outl = _keys(B, hkv, T, 8, seed=hq)
    enc = o8.encode_outlier8(x, outl, rot, cbk)
    v = np.random.default_rng(7).standard_normal((B, hkv, T, d))
    ve = oracle.encode_mse(v.reshape(-1, d), rot, cbv)
    vi, vn = ve.idx.reshape(B, hkv, T, d), ve.norms.reshape(B, hkv, T)
    q = np.random.default_rng(8).standard_normal((B, hq, d))
    got = o8.decode_attention_outlier8(q, enc, vi, vn, rot, rot, cbk, cbv, scale)
    k_hat = o8.decode_outlier8(enc, rot, cbk)
    ratio = hq // hkv
    for b in range(B):
        for g in range(hkv):
            v_hat = torch.from_numpy(oracle.decode_mse(vi[b, g], vn[b, g], rot, cbv))
            qs = torch.from_numpy(q[b, g * ratio:(g + 1) * ratio]).unsqueeze(1)             # [ratio, 1, d]
            kh = torch.from_numpy(k_hat[b, g]).expand(ratio, -1, -1)
            ref = torch.nn.functional.scaled_dot_product_attention(qs, kh, v_hat.expand(ratio, -1, -1), scale=scale)
            np.testing.assert_allclose(got[b, g * ratio:(g + 1) * ratio], ref[:, 0].numpy(), rtol=0, atol=1e-12)
