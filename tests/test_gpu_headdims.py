"""GPU parity of the KV side at head dims 64 and 256 (d = 128 has its own kernels and tests),
through the C ABI:

* the d = 64 encode (MSE b = 1..4, prod b = 2..4; bf16 and fp32; the MSE encode also under the
  Hadamard rotations and at vector counts ragged against its 32-vector tiles, rows past n left
  untouched) against the oracle by the band rule (indices and signs), words bit for bit on the
  rows without a flip, norms and gamma;
* scores of MSE (index bits 1..4) and prod (b = 2..4) keys at d = 64 and d = 256 against the
  oracle's formulas on the GPU's own packed keys, within 1e-3 ||q|| ||k||, GQA ratios 1, 3, 4, 8,
  12 and 20 (20: two groups of the kernel's 16 query heads), T ragged against the 16-key tiles
  and 256-key blocks, and a cache whose rows per sequence exceed T;
* decode attention at d = 64 and d = 256 (rows-layout V) against the oracle within
  1e-3 max_t ||v_hat_t||, ratios 1, 3 and 8, K/V bit pairs, T from 1 to 9000 (several 4096-key
  ranges merged);
* error codes for unsupported shapes."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _parity import check_indices, check_signs, require_gpu, score_tolerance, to_np_words, unpack_z

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


_HANDLES = {}


def _handles(d):
    if d not in _HANDLES:
        rot = tq.make_rotation(d, 5, "dense")
        _HANDLES[d] = (rot, tq.make_qjl(d, 6, rot), oracle.dense_rotation(d, 5), oracle.qjl_matrix(d, 6))
    return _HANDLES[d]


def _keys(n, d, seed, dtype="bf16"):
    x = wl.gaussian((n, d), seed) * np.float32(1.7)
    x[::11] *= np.float32(0.01)
    if n > 2:
        x[2] = 0.0
    if dtype == "bf16":
        bits = wl.f32_to_bf16_bits(x)
        return wl.bf16_bits_to_f32(bits).astype(np.float64), torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    return x.astype(np.float64), torch.from_numpy(x)


def _encode(dev, x_t, d, b, mode):
    rot, qjl, _, _ = _handles(d)
    stage = b - 1 if mode == "prod" else b
    cb = tq.codebook(d, stage)
    n = x_t.shape[0]
    ws = None
    nbytes = tq.encode_workspace(n, d, b, mode)
    if nbytes:
        ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    p = tq.encode(x_t.to(dev), b, mode, cb, rot, qjl if mode == "prod" else None, ws=ws)
    return p, cb


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_encode_mse_d64(dev, b, dtype):
    x, xt = _keys(1000 + 5, 64, seed=b, dtype=dtype)
    p, _ = _encode(dev, xt, 64, b, "mse")
    torch.cuda.synchronize()
    _, _, rmat, _ = _handles(64)
    cb_o = oracle.codebook(64, b)
    enc = oracle.encode_mse(x, rmat, cb_o)
    words = to_np_words(p.idx)
    gidx = oracle.unpack_bits(words, 64, b)
    bad, _ = check_indices(gidx, enc.y, cb_o, f"d64 mse b={b} {dtype}")
    np.testing.assert_array_equal(words[~bad], enc.words[~bad])
    np.testing.assert_allclose(p.norms.cpu().numpy(), enc.norms, rtol=1e-6, atol=0)
    assert np.all(gidx[2] == 1 << (b - 1))


@pytest.mark.parametrize("kind", ["wht", "block_wht"])
@pytest.mark.parametrize("b", [2, 3])
def test_encode_mse_d64_hadamard(dev, kind, b):
    # the d = 64 MSE encode takes R as a matrix (two bf16 passes), whatever its kind
    seed = 30 + b
    rot = tq.make_rotation(64, seed, kind)
    rmat = oracle.wht_rotation(64, seed) if kind == "wht" else oracle.block_wht_rotation(64, seed, 32)
    x, xt = _keys(700, 64, seed=40 + b, dtype="bf16")
    cb = tq.codebook(64, b)
    p = tq.encode(xt.to(dev), b, "mse", cb, rot)
    torch.cuda.synchronize()
    cb_o = oracle.codebook(64, b)
    enc = oracle.encode_mse(x, rmat, cb_o)
    words = to_np_words(p.idx)
    bad, _ = check_indices(oracle.unpack_bits(words, 64, b), enc.y, cb_o, f"d64 {kind} b={b}")
    np.testing.assert_array_equal(words[~bad], enc.words[~bad])
    np.testing.assert_allclose(p.norms.cpu().numpy(), enc.norms, rtol=1e-6, atol=0)


@pytest.mark.parametrize("n", [1, 31, 33, 64, 4097])
def test_encode_mse_d64_ragged(dev, n):
    # vector counts against the 32-vector tiles; rows past n keep their contents
    b = 3
    rot, _, rmat, _ = _handles(64)
    x, xt = _keys(n, 64, seed=n, dtype="bf16")
    cb = tq.codebook(64, b)
    full = tq.alloc_packed(n + 40, 64, b, "mse", device=dev)
    full.idx.fill_(-1)
    full.norms.fill_(5.0)
    p = tq.Packed(64, b, "mse", n, full.idx[:n], full.norms[:n])
    tq.encode(xt.to(dev), b, "mse", cb, rot, out=p)
    torch.cuda.synchronize()
    assert torch.all(full.idx[n:] == -1) and torch.all(full.norms[n:] == 5.0)
    cb_o = oracle.codebook(64, b)
    enc = oracle.encode_mse(x, rmat, cb_o)
    words = to_np_words(p.idx)
    bad, _ = check_indices(oracle.unpack_bits(words, 64, b), enc.y, cb_o, f"d64 n={n}")
    np.testing.assert_array_equal(words[~bad], enc.words[~bad])
    np.testing.assert_allclose(p.norms.cpu().numpy(), enc.norms, rtol=1e-6, atol=0)


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("dtype,n", [("f32", 777), ("bf16", 777), ("bf16", 1), ("bf16", 33), ("f32", 4097)])
def test_encode_prod_d64(dev, b, dtype, n):
    x, xt = _keys(n, 64, seed=20 + b + n, dtype=dtype)
    p, _ = _encode(dev, xt, 64, b, "prod")
    torch.cuda.synchronize()
    _, _, rmat, smat = _handles(64)
    cb_o = oracle.codebook(64, b - 1)
    encp = oracle.encode_prod(x, rmat, cb_o, smat)
    gidx = oracle.unpack_bits(to_np_words(p.idx), 64, b - 1)
    bad, _ = check_indices(gidx, encp.mse.y, cb_o, f"d64 prod b={b} {dtype} n={n}")
    gz = unpack_z(to_np_words(p.qjl), 64)
    check_signs(gz, encp.proj, smat, encp.mse.norms, ~bad, f"d64 prod signs b={b} {dtype} n={n}")
    np.testing.assert_allclose(p.norms.cpu().numpy(), encp.mse.norms, rtol=1e-6, atol=0)
    g = p.rnorms.cpu().numpy()
    ok = ~bad
    assert np.all(np.abs(g[ok] - encp.gamma[ok]) <= 2e-5 * encp.mse.norms[ok] + 1e-30)
    if n > 2:
        assert np.all(gz[2]) and g[2] == 0.0              # zero vector: all-ones signs, gamma 0


def _oracle_scores(p, q, d, b, mode):
    _, _, rmat, smat = _handles(d)
    stage = b - 1 if mode == "prod" else b
    cb_o = oracle.codebook(d, stage)
    idx = oracle.unpack_bits(to_np_words(p.idx), d, stage)
    norms = p.norms.cpu().numpy().astype(np.float64)
    if mode == "mse":
        return oracle.scores_mse(q, idx, norms, rmat, cb_o), norms
    mse = oracle.EncodedMSE(idx=idx, words=None, norms=norms, y=None)
    encp = oracle.EncodedProd(mse=mse, z=unpack_z(to_np_words(p.qjl), d), qjl_words=None,
                              gamma=p.rnorms.cpu().numpy().astype(np.float64), proj=None)
    return oracle.scores_prod(q, encp, rmat, cb_o, smat), norms


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("mode,b", [("mse", 1), ("mse", 2), ("mse", 3), ("mse", 4), ("prod", 2), ("prod", 3),
                                    ("prod", 4)])
@pytest.mark.parametrize("B,hkv,hq,T", [(2, 2, 8, 300), (1, 1, 12, 513), (1, 3, 3, 70), (1, 1, 20, 33)])
def test_scores_head_dims(dev, d, mode, b, B, hkv, hq, T):
    rot, qjl, _, _ = _handles(d)
    x, xt = _keys(B * hkv * T, d, seed=d + b + T)
    p, cb = _encode(dev, xt, d, b, mode)
    q = wl.gaussian((B, hq, d), 31 + b)
    s = tq.scores(torch.from_numpy(q).to(dev), p, hkv, cb, rot, qjl if mode == "prod" else None)
    torch.cuda.synchronize()
    got = s.cpu().numpy()
    ratio = hq // hkv
    ref_all, norms = _oracle_scores(p, q.reshape(-1, d).astype(np.float64), d, b, mode)
    ref_all = ref_all.reshape(B, hq, B, hkv, T)
    norms = norms.reshape(B, hkv, T)
    for bb in range(B):
        for h in range(hq):
            g = h // ratio
            tol = score_tolerance(q[bb, h][None, :], norms[bb, g])[0]
            assert np.all(np.abs(got[bb, h] - ref_all[bb, h, bb, g]) <= tol), (d, mode, b, bb, h)


@pytest.mark.parametrize("d", [64, 256])
def test_scores_cache_stride_head_dims(dev, d):
    # keys packed for a capacity of 96 rows per sequence, scored over the first 70
    rot, _, _, _ = _handles(d)
    B, hkv, hq, cap, T = 2, 2, 4, 96, 70
    x, xt = _keys(B * hkv * cap, d, seed=77)
    p, cb = _encode(dev, xt, d, 3, "mse")
    q = wl.gaussian((B, hq, d), 78)
    out = torch.empty((B, hq, T), device=dev)
    ws = torch.empty((tq.scores_workspace(B, hq, d),), dtype=torch.uint8, device=dev)
    tq.check(tq.lib().tq_scores_cache(tq._dptr(torch.from_numpy(q).to(dev)), B, hq, hkv, T, cap,
                                      tq.ctypes.byref(p.descriptor()), cb.ptr, rot.ptr, None, tq._dptr(out),
                                      tq._dptr(ws), ws.numel(), tq._stream()))
    torch.cuda.synchronize()
    ref, norms = _oracle_scores(p, q.reshape(-1, d).astype(np.float64), d, 3, "mse")
    ref = ref.reshape(B, hq, B, hkv, cap)
    norms = norms.reshape(B, hkv, cap)
    got = out.cpu().numpy()
    for bb in range(B):
        for h in range(hq):
            g = h // 2
            tol = score_tolerance(q[bb, h][None, :], norms[bb, g, :T])[0]
            assert np.all(np.abs(got[bb, h] - ref[bb, h, bb, g, :T]) <= tol)


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("B,hkv,hq,T,kb,vb", [(1, 2, 2, 1, 3, 2), (2, 1, 3, 257, 4, 4), (1, 2, 16, 9000, 2, 3),
                                              (1, 1, 8, 4096 + 255, 3, 1), (2, 2, 8, 3000, 4, 2),
                                              (1, 1, 4, 70000, 4, 2)])
def test_decode_attention_head_dims(dev, d, B, hkv, hq, T, kb, vb):
    rot, _, rmat, _ = _handles(d)
    n = B * hkv * T
    xk, xkt = _keys(n, d, seed=T + kb)
    xv, xvt = _keys(n, d, seed=T + 100 + vb)
    K, cbk = _encode(dev, xkt, d, kb, "mse")
    V, cbv = _encode(dev, xvt, d, vb, "mse")
    q = wl.gaussian((B, hq, d), 55)
    out = tq.decode_attn(torch.from_numpy(q).to(dev), K, V, hkv, cbk, cbv, rot, rot)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    cbk_o, cbv_o = oracle.codebook(d, kb), oracle.codebook(d, vb)
    kidx = oracle.unpack_bits(to_np_words(K.idx), d, kb).reshape(B, hkv, T, d)
    vidx = oracle.unpack_bits(to_np_words(V.idx), d, vb).reshape(B, hkv, T, d)
    kn = K.norms.cpu().numpy().astype(np.float64).reshape(B, hkv, T)
    vn = V.norms.cpu().numpy().astype(np.float64).reshape(B, hkv, T)
    ref = oracle.decode_attention(q.astype(np.float64), kidx, kn, vidx, vn, rmat, rmat, cbk_o, cbv_o, 1 / np.sqrt(d))
    ratio = hq // hkv
    for bb in range(B):
        for g in range(hkv):
            vmax = np.max(np.linalg.norm(oracle.decode_mse(vidx[bb, g], vn[bb, g], rmat, cbv_o), axis=1))
            err = np.abs(got[bb, g * ratio:(g + 1) * ratio] - ref[bb, g * ratio:(g + 1) * ratio])
            assert np.all(err <= 1e-3 * vmax), (d, bb, g, float(err.max()), vmax)


def test_head_dim_errors(dev):
    rot, _, _, _ = _handles(256)
    cb = tq.codebook(256, 2)
    x, xt = _keys(64, 256, seed=1)
    K, _ = _encode(dev, xt, 256, 2, "mse")
    q = torch.zeros((1, 16, 256), device=dev)
    with pytest.raises(tq.TQError) as e:                  # GQA ratio 16 at d = 256
        tq.decode_attn(q, K, K, 1, cb, cb, rot, rot)
    assert e.value.status == 3
    Vb = tq.alloc_packed(64, 256, 2, "mse", device=dev, layout="blocked")
    with pytest.raises(tq.TQError) as e:                  # token-blocked V needs d = 128
        tq.decode_attn(torch.zeros((1, 2, 256), device=dev), K, Vb, 1, cb, cb, rot, rot)
    assert e.value.status == 3
    r192 = tq.make_rotation(192, 1, "dense")
    c192 = tq.codebook(192, 2)
    with pytest.raises(tq.TQError) as e:                  # d = 192: no KV kernels
        tq.encode(torch.zeros((4, 192), device=dev), 2, "mse", c192, r192)
    assert e.value.status == 3
    with pytest.raises(tq.TQError) as e:                  # the static-scratch scores take d = 128 only
        tq.scores_noalloc(torch.zeros((1, 2, 256), device=dev), K, 1, cb, rot)
    assert e.value.status == 3


@pytest.mark.parametrize("d", [64, 256])
def test_decode_attention_head_dims_reused_workspace(dev, d):
    # repeated calls on one workspace (and a smaller call in between) give the same result
    rot, _, _, _ = _handles(d)
    B, hkv, hq, T = 2, 2, 8, 5000
    n = B * hkv * T
    _, xkt = _keys(n, d, seed=7)
    _, xvt = _keys(n, d, seed=8)
    K, cbk = _encode(dev, xkt, d, 4, "mse")
    V, cbv = _encode(dev, xvt, d, 2, "mse")
    q = torch.from_numpy(wl.gaussian((B, hq, d), 9)).to(dev)
    ws = torch.empty((tq.decode_attn_workspace(B, hq, hkv, T, d),), dtype=torch.uint8, device=dev)
    first = tq.decode_attn(q, K, V, hkv, cbk, cbv, rot, rot, ws=ws).cpu()
    Ks, cbks = _encode(dev, xkt[: hkv * 300], d, 4, "mse")
    Vs, cbvs = _encode(dev, xvt[: hkv * 300], d, 2, "mse")
    tq.decode_attn(q[:1], Ks, Vs, hkv, cbks, cbvs, rot, rot, ws=ws)
    second = tq.decode_attn(q, K, V, hkv, cbk, cbv, rot, rot, ws=ws).cpu()
    assert torch.equal(first, second)

