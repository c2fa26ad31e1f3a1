"""GPU parity of the block (group-32) randomized Hadamard rotation against the oracle, through the
C ABI and the same kernels as the other rotations: the rotated coordinates at d = 128 and d = 1536,
MSE and prod encode with their scores at d = 128, the value cache and decode attention, and the
general-d encode at d = 1536 (a multiple of 32 that is not a power of two)."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _parity import (check_indices, check_signs, require_gpu, score_tolerance, to_np_words, unpack_z)

pytestmark = pytest.mark.gpu

R_BW = oracle.block_wht_rotation(128, 1, 32)
S_MAT = oracle.qjl_matrix(128, 2)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def rot(dev):
    return tq.make_rotation(128, 1, "block_wht")


def _keys(n_tok, hkv=2, B=1, seed=0):
    bits = wl.kv_tensor_bf16(B, hkv, n_tok, 128, seed=seed, outlier_seed=10, scale_seed=11)
    x = wl.bf16_bits_to_f32(bits).reshape(-1, 128).astype(np.float64)
    return x, torch.from_numpy(bits.reshape(-1, 128).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (128, "f32"), (1536, "f32")])
def test_rotate_block_wht(dev, d, dtype):
    r = tq.make_rotation(d, 1, "block_wht")
    rmat = oracle.block_wht_rotation(d, 1, 32)
    x = wl.gaussian((300 + 7, d), 5) * np.float32(3.0)
    x[4] = 0.0
    if dtype == "bf16":
        bits = wl.f32_to_bf16_bits(x)
        x = wl.bf16_bits_to_f32(bits)
        xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        xt = torch.from_numpy(x)
    y, nr = tq.rotate(xt.to(dev), r)
    torch.cuda.synchronize()
    ref = oracle.encode_mse(x.astype(np.float64), rmat, oracle.codebook(d, 1))
    assert np.max(np.abs(y.cpu().numpy() - ref.y)) <= 1e-5
    np.testing.assert_allclose(nr.cpu().numpy(), ref.norms, rtol=1e-6, atol=0)
    assert np.all(y.cpu().numpy()[4] == 0.0)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_encode_mse_block_wht(dev, rot, b):
    x, xt = _keys(2048 + 37, hkv=4)
    cb_o, cb = oracle.codebook(128, b), tq.codebook(128, b)
    p = tq.encode(xt.to(dev), b, "mse", cb, rot)
    torch.cuda.synchronize()
    enc = oracle.encode_mse(x, R_BW, cb_o)
    gidx = oracle.unpack_bits(to_np_words(p.idx), 128, b)
    bad, _ = check_indices(gidx, enc.y, cb_o, f"block wht mse b={b}")
    np.testing.assert_array_equal(to_np_words(p.idx)[~bad], enc.words[~bad])
    np.testing.assert_allclose(p.norms.cpu().numpy(), enc.norms, rtol=1e-6)


def test_prod_encode_and_scores_block_wht(dev, rot):
    qjl = tq.make_qjl(128, 2, rot)
    hkv, hq, T = 2, 8, 700
    x, xt = _keys(T, hkv=hkv)
    cb_o, cb = oracle.codebook(128, 3), tq.codebook(128, 3)
    p = tq.encode(xt.to(dev), 4, "prod", cb, rot, qjl)
    q = wl.gaussian((1, hq, 128), 12)
    s = tq.scores(torch.from_numpy(q).to(dev), p, hkv, cb, rot, qjl)
    torch.cuda.synchronize()
    encp = oracle.encode_prod(x, R_BW, cb_o, S_MAT)
    gidx = oracle.unpack_bits(to_np_words(p.idx), 128, 3)
    bad, _ = check_indices(gidx, encp.mse.y, cb_o, "block wht prod stage")
    gz = unpack_z(to_np_words(p.qjl), 128)
    check_signs(gz, encp.proj, S_MAT, encp.mse.norms, ~bad, "block wht prod signs")
    g = p.rnorms.cpu().numpy()
    assert np.all(np.abs(g[~bad] - encp.gamma[~bad]) <= 2e-5 * encp.mse.norms[~bad] + 1e-12)
    # scores on the GPU's own packed keys
    norms = p.norms.cpu().numpy().astype(np.float64)
    got = s.cpu().numpy()
    ratio = hq // hkv
    for gi in range(hkv):
        rows = slice(gi * T, (gi + 1) * T)
        sub = oracle.EncodedProd(mse=oracle.EncodedMSE(idx=gidx[rows], words=None, norms=norms[rows], y=None),
                                 z=gz[rows], qjl_words=None, gamma=g[rows].astype(np.float64), proj=None)
        heads = q[0, gi * ratio:(gi + 1) * ratio].astype(np.float64)
        ref = oracle.scores_prod(heads, sub, R_BW, cb_o, S_MAT)
        assert np.all(np.abs(got[0, gi * ratio:(gi + 1) * ratio] - ref) <= score_tolerance(heads, norms[rows]))


def test_attention_block_wht(dev, rot):
    B, hkv, hq, T, b = 1, 2, 8, 1000, 3
    xk, kt = _keys(T, hkv=hkv, B=B)
    xv, vt = _keys(T, hkv=hkv, B=B, seed=20)
    cb, cb_o = tq.codebook(128, b), oracle.codebook(128, b)
    K = tq.encode(kt.to(dev), b, "mse", cb, rot)
    V = tq.encode(vt.to(dev), b, "mse", cb, rot, layout="blocked")
    q = wl.gaussian((B, hq, 128), 12)
    out = tq.decode_attn(torch.from_numpy(q).to(dev), K, V, hkv, cb, cb, rot, rot)
    torch.cuda.synchronize()
    n = B * hkv * T
    vidx = oracle.unpack_token_blocked(to_np_words(V.idx), n, 128, b)
    check_indices(vidx, oracle.encode_mse(xv, R_BW, cb_o).y, cb_o, "block wht values")
    kidx = oracle.unpack_bits(to_np_words(K.idx), 128, b).reshape(B, hkv, T, 128)
    kn = K.norms.cpu().numpy().astype(np.float64).reshape(B, hkv, T)
    vn = V.norms.cpu().numpy().astype(np.float64).reshape(B, hkv, T)
    ref = oracle.decode_attention(q.astype(np.float64), kidx, kn, vidx.reshape(B, hkv, T, 128), vn, R_BW, R_BW,
                                  cb_o, cb_o, 1 / np.sqrt(128))
    got = out.cpu().numpy()
    ratio = hq // hkv
    for gi in range(hkv):
        vh = oracle.decode_mse(vidx.reshape(B, hkv, T, 128)[0, gi], vn[0, gi], R_BW, cb_o)
        vmax = np.max(np.linalg.norm(vh, axis=1))
        err = np.max(np.abs(got[0, gi * ratio:(gi + 1) * ratio] - ref[0, gi * ratio:(gi + 1) * ratio]))
        assert err <= 1e-3 * vmax, (gi, err, vmax)


def test_encode_general_block_wht(dev):
    d, b = 1536, 3
    r = tq.make_rotation(d, 1, "block_wht")
    rmat = oracle.block_wht_rotation(d, 1, 32)
    x = wl.lowrank_unit_vectors(777, d, 64, 24.0, 0, 30, 31)
    cb_o = oracle.codebook(d, b)
    p = tq.encode(torch.from_numpy(x).to(dev), b, "mse", tq.codebook(d, b), r)
    torch.cuda.synchronize()
    ref = oracle.encode_mse(x.astype(np.float64), rmat, cb_o)
    check_indices(oracle.unpack_bits(to_np_words(p.idx), d, b), ref.y, cb_o, "block wht d=1536")
    np.testing.assert_allclose(p.norms.cpu().numpy(), ref.norms, rtol=1e-6, atol=0)


def test_block_wht_needs_multiple_of_32(dev):
    with pytest.raises(tq.TQError):
        tq.make_rotation(100, 1, "block_wht")
