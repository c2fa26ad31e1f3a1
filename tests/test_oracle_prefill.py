"""Pins of the oracle's prefill attention: causal attention of a chunk of new tokens over the
compressed cache after the chunk's own keys and values were appended ("TurboQuant 详解",
KV-cache example, prefill; "TurboQuant 和 RotorQuant 的真相", Flash Attention fusion section).

Pinned against things other than itself: torch's scaled_dot_product_attention (float64, CPU,
an explicit boolean mask) on the same dequantized K_hat and V_hat; decode_attention for chunks
of one token; special cases (the first token sees only itself; equal logits give the mean of
the visible values); chunked prefill against one-shot prefill; causality."""

import numpy as np
import pytest
import torch

import oracle


def _cache(B, hkv, T, d, b, seed):
    rng = np.random.default_rng(seed)
    rot, cb = oracle.dense_rotation(d, 1), oracle.codebook(d, b)
    kx = rng.standard_normal((B, hkv, T, d)) * rng.lognormal(0.0, 0.5, size=(B, hkv, T, 1))
    vx = rng.standard_normal((B, hkv, T, d))
    ke = oracle.encode_mse(kx.reshape(-1, d), rot, cb)
    ve = oracle.encode_mse(vx.reshape(-1, d), rot, cb)
    shape = (B, hkv, T)
    return (rot, cb, ke.idx.reshape(*shape, d), ke.norms.reshape(shape), ve.idx.reshape(*shape, d),
            ve.norms.reshape(shape))


@pytest.mark.parametrize("B,hkv,hq,pos,tn", [(1, 2, 8, 0, 9), (2, 1, 3, 5, 7), (1, 2, 2, 17, 1)])
def test_prefill_matches_torch_sdpa(B, hkv, hq, pos, tn):
    d, b = 16, 2
    T = pos + tn + 3                                   # rows past the chunk are never read
    rot, cb, ki, kn, vi, vn = _cache(B, hkv, T, d, b, seed=pos + 7 * tn)
    q = np.random.default_rng(1).standard_normal((B, hq, tn, d))
    scale = 1.0 / np.sqrt(d)
    got = oracle.prefill_attention(q, ki, kn, vi, vn, pos, rot, rot, cb, cb, scale)
    ratio = hq // hkv
    live = pos + tn
    mask = torch.from_numpy(np.arange(live)[None, :] <= (pos + np.arange(tn))[:, None])   # [tn, live]
    for bi in range(B):
        for g in range(hkv):
            k_hat = torch.from_numpy(oracle.decode_mse(ki[bi, g, :live], kn[bi, g, :live], rot, cb))
            v_hat = torch.from_numpy(oracle.decode_mse(vi[bi, g, :live], vn[bi, g, :live], rot, cb))
            qs = torch.from_numpy(q[bi, g * ratio:(g + 1) * ratio])                       # [ratio, tn, d]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qs, k_hat.expand(ratio, -1, -1), v_hat.expand(ratio, -1, -1), attn_mask=mask, scale=scale)
            np.testing.assert_allclose(got[bi, g * ratio:(g + 1) * ratio], ref.numpy(), rtol=0, atol=1e-12)


def test_single_token_chunk_is_decode_attention():
    d, b, B, hkv, hq, pos = 16, 3, 2, 2, 4, 11
    rot, cb, ki, kn, vi, vn = _cache(B, hkv, pos + 1, d, b, seed=3)
    q = np.random.default_rng(4).standard_normal((B, hq, 1, d))
    got = oracle.prefill_attention(q, ki, kn, vi, vn, pos, rot, rot, cb, cb, 0.25)
    ref = oracle.decode_attention(q[:, :, 0], ki, kn, vi, vn, rot, rot, cb, cb, 0.25)
    np.testing.assert_allclose(got[:, :, 0], ref, rtol=0, atol=1e-13)


def test_first_token_sees_itself_and_equal_logits_give_the_mean():
    d, b, B, hkv, hq, tn = 8, 2, 1, 1, 2, 6
    rot, cb, ki, kn, vi, vn = _cache(B, hkv, tn, d, b, seed=9)
    q = np.random.default_rng(2).standard_normal((B, hq, tn, d))
    got = oracle.prefill_attention(q, ki, kn, vi, vn, 0, rot, rot, cb, cb, 0.5)
    v_hat = oracle.decode_mse(vi[0, 0], vn[0, 0], rot, cb)
    np.testing.assert_allclose(got[0, :, 0], np.broadcast_to(v_hat[0], (hq, d)), rtol=0, atol=1e-14)
    # zero queries: every visible logit is 0, so query i returns the mean of v_hat[0 .. i]
    z = oracle.prefill_attention(np.zeros_like(q), ki, kn, vi, vn, 0, rot, rot, cb, cb, 0.5)
    for i in range(tn):
        np.testing.assert_allclose(z[0, 0, i], v_hat[:i + 1].mean(axis=0), rtol=0, atol=1e-14)


def test_chunked_equals_one_shot_and_causality():
    d, b, B, hkv, hq, T = 16, 2, 1, 2, 4, 23
    rot, cb, ki, kn, vi, vn = _cache(B, hkv, T, d, b, seed=12)
    q = np.random.default_rng(6).standard_normal((B, hq, T, d))
    one = oracle.prefill_attention(q, ki, kn, vi, vn, 0, rot, rot, cb, cb, 0.3)
    first = oracle.prefill_attention(q[:, :, :10], ki, kn, vi, vn, 0, rot, rot, cb, cb, 0.3)
    second = oracle.prefill_attention(q[:, :, 10:], ki, kn, vi, vn, 10, rot, rot, cb, cb, 0.3)
    np.testing.assert_allclose(np.concatenate([first, second], axis=2), one, rtol=0, atol=1e-13)
    # changing the cache after token 9 leaves the outputs of tokens 0 .. 9 unchanged
    ki2, kn2 = ki.copy(), kn.copy()
    ki2[:, :, 10:] = (ki2[:, :, 10:] + 1) % (1 << b)
    kn2[:, :, 10:] *= 3.0
    again = oracle.prefill_attention(q[:, :, :10], ki2, kn2, vi, vn, 0, rot, rot, cb, cb, 0.3)
    np.testing.assert_array_equal(again, first)
    changed = oracle.prefill_attention(q[:, :, 10:], ki2, kn2, vi, vn, 10, rot, rot, cb, cb, 0.3)
    assert np.max(np.abs(changed - second)) > 1e-3
