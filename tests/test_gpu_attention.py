"""GPU parity of the token-blocked value encode and of fused decode attention (C ABI) against
the oracle, on the GPU's own packed data (identical packed inputs), with ragged token counts."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _parity import check_indices, require_gpu, to_np_words

pytestmark = pytest.mark.gpu

R = oracle.dense_rotation(128, 1)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def rot(dev):
    return tq.make_rotation(128, 1)


def _kv(B, hkv, T, which):
    if which == "k":
        bits = wl.kv_tensor_bf16(B, hkv, T, 128, seed=0, outlier_seed=10, scale_seed=11)
    else:
        bits = wl.kv_tensor_bf16(B, hkv, T, 128, seed=20, outlier_seed=21, scale_seed=None)
    x = wl.bf16_bits_to_f32(bits).reshape(-1, 128).astype(np.float64)
    return x, torch.from_numpy(bits.reshape(-1, 128).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("n", [32, 1000, 77])
def test_blocked_encode_parity(dev, rot, b, n):
    x, xt = _kv(1, 1, n, "v")
    cb = tq.codebook(128, b)
    cbo = oracle.codebook(128, b)
    p = tq.encode(xt.to(dev), b, "mse", cb, rot, layout="blocked")
    torch.cuda.synchronize()
    words = to_np_words(p.idx)
    gidx = oracle.unpack_token_blocked(words, n, 128, b)
    enc = oracle.encode_mse(x, R, cbo)
    check_indices(gidx, enc.y, cbo, f"blocked b={b} n={n}")
    # the layout itself is bit-exact (including the zero padding of the last block)
    np.testing.assert_array_equal(words, oracle.pack_token_blocked(gidx, b))
    np.testing.assert_allclose(p.norms.cpu().numpy(), enc.norms, rtol=1e-6)
    # decode understands the layout
    xh = tq.decode(p, cb, rot).cpu().numpy()
    ref = oracle.decode_mse(gidx, p.norms.cpu().numpy().astype(np.float64), R, cbo)
    assert np.all(np.abs(xh - ref) <= 1e-5 * enc.norms[:, None] + 1e-12)


def _attn_case(dev, rot, B, hkv, hq, T, kb, vb):
    xk, kt = _kv(B, hkv, T, "k")
    xv, vt = _kv(B, hkv, T, "v")
    cbk, cbv = tq.codebook(128, kb), tq.codebook(128, vb)
    K = tq.encode(kt.to(dev), kb, "mse", cbk, rot)
    V = tq.encode(vt.to(dev), vb, "mse", cbv, rot, layout="blocked")
    q = wl.gaussian((B, hq, 128), 12)
    out = tq.decode_attn(torch.from_numpy(q).to(dev), K, V, hkv, cbk, cbv, rot, rot)
    torch.cuda.synchronize()
    n = B * hkv * T
    kidx = oracle.unpack_bits(to_np_words(K.idx), 128, kb).reshape(B, hkv, T, 128)
    vidx = oracle.unpack_token_blocked(to_np_words(V.idx), n, 128, vb).reshape(B, hkv, T, 128)
    kn = K.norms.cpu().numpy().astype(np.float64).reshape(B, hkv, T)
    vn = V.norms.cpu().numpy().astype(np.float64).reshape(B, hkv, T)
    ref = oracle.decode_attention(q.astype(np.float64), kidx, kn, vidx, vn, R, R,
                                  oracle.codebook(128, kb), oracle.codebook(128, vb), 1 / np.sqrt(128))
    got = out.cpu().numpy()
    ratio = hq // hkv
    for bi in range(B):
        for h in range(hq):
            g = h // ratio
            vmax = np.max(vn[bi, g]) * 1.0   # ||v_hat_t|| = s_v,t (R orthogonal, unit-norm codebook rows aside)
            vh = oracle.decode_mse(vidx[bi, g], vn[bi, g], R, oracle.codebook(128, vb))
            vmax = np.max(np.linalg.norm(vh, axis=1))
            err = np.max(np.abs(got[bi, h] - ref[bi, h]))
            assert err <= 1e-3 * vmax, (bi, h, err, vmax)


@pytest.mark.parametrize("B,hkv,hq,T,kb,vb", [
    (1, 2, 8, 1000, 2, 2), (2, 2, 8, 333, 4, 4), (1, 1, 4, 1, 2, 2), (1, 2, 2, 31, 3, 3),
    (1, 4, 8, 33, 2, 4), (1, 1, 1, 5000, 2, 2), (2, 1, 4, 4097, 4, 2),
    # sequences that start in the second half of a 32-token block (row offsets 154, 83 and 249):
    # their first block's first 16-token tile lies wholly before the sequence
    (2, 2, 2, 77, 2, 3), (2, 2, 4, 83, 3, 3)])
def test_decode_attention_parity(dev, rot, B, hkv, hq, T, kb, vb):
    _attn_case(dev, rot, B, hkv, hq, T, kb, vb)


def test_decode_attention_errors(dev, rot):
    cb = tq.codebook(128, 2)
    x = torch.zeros((64, 128), dtype=torch.bfloat16, device=dev)
    K = tq.encode(x, 2, "mse", cb, rot)
    V = tq.encode(x, 2, "mse", cb, rot, layout="blocked")
    q = torch.zeros((1, 8, 128), device=dev)
    with pytest.raises(tq.TQError):
        tq.decode_attn(q, V, V, 2, cb, cb, rot, rot)     # K must use the rows layout
    with pytest.raises(tq.TQError):
        tq.decode_attn(q, K, K, 2, cb, cb, rot, rot)     # V must be token-blocked
    with pytest.raises(tq.TQError):
        tq.decode_attn(torch.zeros((1, 6, 128), device=dev), K, V, 2, cb, cb, rot, rot)  # ratio 3
    # zero keys and values: uniform attention over zero vectors gives 0
    out = tq.decode_attn(q, K, V, 2, cb, cb, rot, rot)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0.0)
