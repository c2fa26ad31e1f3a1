"""GPU parity of the HIP path against the fp64 oracle, through the C ABI, on seeded inputs of the
workloads' shapes (several MFMA tiles plus ragged tails) and on the edge cases."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _parity import (BAND, check_indices, check_signs, require_gpu, score_tolerance, to_np_words,
                     unpack_z)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def rot_dense(dev):
    return tq.make_rotation(128, 1, "dense")


@pytest.fixture(scope="module")
def rot_wht(dev):
    return tq.make_rotation(128, 1, "wht")


R_DENSE = oracle.dense_rotation(128, 1)
R_WHT = oracle.wht_rotation(128, 1)
S_MAT = oracle.qjl_matrix(128, 2)


def _keys(n_tok, hkv=2, B=1):
    cfg = wl.CONFIGS["c2"]
    bits = wl.kv_tensor_bf16(B, hkv, n_tok, 128, seed=0, outlier_seed=10, scale_seed=11)
    x = wl.bf16_bits_to_f32(bits).reshape(-1, 128).astype(np.float64)
    t = torch.from_numpy(bits.reshape(-1, 128).view(np.int16)).view(torch.bfloat16)
    return x, t


def test_quantize_rotated_bit_exact(dev):
    rng = np.random.default_rng(0)
    for b in (1, 2, 3, 4):
        cb_o = oracle.codebook(128, b)
        cb = tq.codebook(128, b)
        for n in (1, 7, 1000):
            y = (rng.standard_normal((n, 128)) / np.sqrt(128)).astype(np.float32)
            # plant exact thresholds, their neighbours and signed zeros
            t32 = cb_o.thresholds32
            flat = y.reshape(-1)
            k = min(flat.size, 3 * t32.size + 2)
            plant = np.concatenate([t32, np.nextafter(t32, np.float32(-1)), np.nextafter(t32, np.float32(1)),
                                    np.float32([0.0, -0.0])])[:k]
            flat[:k] = plant
            words = tq.quantize_rotated(torch.from_numpy(y).to(dev), cb)
            torch.cuda.synchronize()
            ref = oracle.pack_bits(oracle.quantize_rotated(y, cb_o), b)
            np.testing.assert_array_equal(to_np_words(words), ref, err_msg=f"b={b} n={n}")


@pytest.mark.parametrize("kind", ["dense", "wht"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rotate_matches_oracle(dev, rot_dense, rot_wht, kind, dtype):
    rot, rmat = (rot_dense, R_DENSE) if kind == "dense" else (rot_wht, R_WHT)
    if dtype == "f32":
        x = wl.gaussian((1000 + 17, 128), 0).astype(np.float64) * 3.0
        xt = torch.from_numpy(x.astype(np.float32))
    else:
        x, xt = _keys(509, hkv=2)
    x[3] = 0.0
    xt = xt.clone()
    xt[3] = 0
    y, nr = tq.rotate(xt.to(dev), rot)
    torch.cuda.synchronize()
    enc = oracle.encode_mse(x, rmat, oracle.codebook(128, 2))
    np.testing.assert_allclose(nr.cpu().numpy(), enc.norms, rtol=1e-6, atol=0)
    err = np.abs(y.cpu().numpy().astype(np.float64) - enc.y)
    assert err.max() <= 1e-5, err.max()
    assert np.all(y.cpu().numpy()[3] == 0.0)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("kind", ["dense", "wht"])
def test_encode_mse_parity_bf16_keys(dev, rot_dense, rot_wht, b, kind):
    rot, rmat = (rot_dense, R_DENSE) if kind == "dense" else (rot_wht, R_WHT)
    x, xt = _keys(2048 + 37, hkv=4)
    cb_o = oracle.codebook(128, b)
    cb = tq.codebook(128, b)
    p = tq.encode(xt.to(dev), b, "mse", cb, rot)
    torch.cuda.synchronize()
    enc = oracle.encode_mse(x, rmat, cb_o)
    gidx = oracle.unpack_bits(to_np_words(p.idx), 128, b)
    bad_rows, nflip = check_indices(gidx, enc.y, cb_o, f"mse b={b} {kind}")
    np.testing.assert_array_equal(to_np_words(p.idx)[~bad_rows], enc.words[~bad_rows])
    np.testing.assert_allclose(p.norms.cpu().numpy(), enc.norms, rtol=1e-6)


@pytest.mark.parametrize("n", [1, 31, 33, 65, 4097])
@pytest.mark.parametrize("dtype,b", [("bf16", 3), ("f32", 2), ("bf16", 4), ("f32", 1)])
def test_encode_mse_dense_ragged(dev, rot_dense, n, dtype, b):
    # vector counts against the 32-vector tiles of the dense-rotation encode, both input types; rows
    # past n keep their contents
    x, xt = _keys(n, hkv=1)
    if dtype == "f32":
        rng = np.random.default_rng(n + b)
        x = x * rng.uniform(0.5, 2.0, size=(n, 1)) + rng.normal(0, 1e-3, size=x.shape)
        x[:: 7] *= 1e-4
        xt = torch.from_numpy(x.astype(np.float32))
        x = xt.numpy().astype(np.float64)
    cb = tq.codebook(128, b)
    full = tq.alloc_packed(n + 40, 128, b, "mse", device=dev)
    full.idx.fill_(-1)
    full.norms.fill_(5.0)
    p = tq.Packed(128, b, "mse", n, full.idx[:n], full.norms[:n])
    tq.encode(xt.to(dev), b, "mse", cb, rot_dense, out=p)
    torch.cuda.synchronize()
    assert torch.all(full.idx[n:] == -1) and torch.all(full.norms[n:] == 5.0)
    cb_o = oracle.codebook(128, b)
    enc = oracle.encode_mse(x, R_DENSE, cb_o)
    words = to_np_words(p.idx)
    bad, _ = check_indices(oracle.unpack_bits(words, 128, b), enc.y, cb_o, f"dense n={n} {dtype} b={b}")
    np.testing.assert_array_equal(words[~bad], enc.words[~bad])
    np.testing.assert_allclose(p.norms.cpu().numpy(), enc.norms, rtol=1e-6, atol=0)


def test_encode_mse_c1_fp32_full(dev, rot_dense):
    x32, _ = wl.c1_inputs()
    x = x32.astype(np.float64)
    cb_o = oracle.codebook(128, 2)
    cb = tq.codebook(128, 2)
    p = tq.encode(torch.from_numpy(x32).to(dev), 2, "mse", cb, rot_dense)
    torch.cuda.synchronize()
    enc = oracle.encode_mse(x, R_DENSE, cb_o)
    gidx = oracle.unpack_bits(to_np_words(p.idx), 128, 2)
    check_indices(gidx, enc.y, cb_o, "c1")
    # reconstruction MSE within 1% of the oracle's
    xh = tq.decode(p, cb, rot_dense).cpu().numpy().astype(np.float64)
    xo = oracle.decode_mse(enc.idx, enc.norms, R_DENSE, cb_o)
    mse_g = np.mean(np.sum((x - xh) ** 2, 1))
    mse_o = np.mean(np.sum((x - xo) ** 2, 1))
    assert abs(mse_g / mse_o - 1) < 0.01


def test_scores_c1_fp32_full(dev, rot_dense):
    # the tiny round trip's own inputs: 4096 fp32 N(0,1) vectors as one KV head of 4096 keys,
    # scored by its 32 fp32 N(0,1) queries (GQA ratio 32, the multi-group path)
    x32, q32 = wl.c1_inputs()
    cb_o, cb = oracle.codebook(128, 2), tq.codebook(128, 2)
    p = tq.encode(torch.from_numpy(x32).to(dev), 2, "mse", cb, rot_dense)
    s = tq.scores(torch.from_numpy(q32.reshape(1, 32, 128)).to(dev), p, 1, cb, rot_dense)
    torch.cuda.synchronize()
    enc = _packed_to_oracle(p, 128, 2, False)
    q = q32.astype(np.float64)
    ref = oracle.scores_mse(q, enc.idx, enc.norms, R_DENSE, cb_o)          # [32, 4096]
    err = np.abs(s.cpu().numpy()[0] - ref)
    tol = score_tolerance(q, enc.norms)
    assert np.all(err <= tol), float((err / tol).max())
    # and the GPU's codes score like the oracle's own encode of the same vectors
    own = oracle.encode_mse(x32.astype(np.float64), R_DENSE, cb_o)
    ref_own = oracle.scores_mse(q, own.idx, own.norms, R_DENSE, cb_o)
    assert np.mean(np.abs(ref - ref_own)) <= 1e-3 * np.mean(np.abs(ref_own))


@pytest.mark.parametrize("kind", ["dense", "wht"])
def test_encode_prod_parity(dev, rot_dense, rot_wht, kind):
    rot, rmat = (rot_dense, R_DENSE) if kind == "dense" else (rot_wht, R_WHT)
    qjl = tq.make_qjl(128, 2, rot)
    x, xt = _keys(1024 + 5, hkv=4)
    cb_o = oracle.codebook(128, 3)
    cb = tq.codebook(128, 3)
    p = tq.encode(xt.to(dev), 4, "prod", cb, rot, qjl)
    torch.cuda.synchronize()
    encp = oracle.encode_prod(x, rmat, cb_o, S_MAT)
    gidx = oracle.unpack_bits(to_np_words(p.idx), 128, 3)
    bad_rows, _ = check_indices(gidx, encp.mse.y, cb_o, f"prod stage {kind}")
    gz = unpack_z(to_np_words(p.qjl), 128)
    check_signs(gz, encp.proj, S_MAT, encp.mse.norms, ~bad_rows, f"prod signs {kind}")
    g = p.rnorms.cpu().numpy()
    ok = ~bad_rows
    assert np.all(np.abs(g[ok] - encp.gamma[ok]) <= 2e-5 * encp.mse.norms[ok] + 1e-12)


@pytest.mark.parametrize("kind,b", [("dense", 4), ("wht", 3), ("dense", 2)])
def test_encode_prod_many_tiles_per_wave(dev, rot_dense, rot_wht, kind, b):
    # 159857 keys: more 32-key tiles than the grid has waves, so every wave runs several
    # tiles in a row (its fragment prefetch wraps from one tile into the next) and a ragged last tile.
    rot, rmat = (rot_dense, R_DENSE) if kind == "dense" else (rot_wht, R_WHT)
    qjl = tq.make_qjl(128, 2, rot)
    x, xt = _keys(40000, hkv=4)
    n = x.shape[0] - 143
    x, xt = x[:n], xt[:n].contiguous()
    cb_o = oracle.codebook(128, b - 1)
    cb = tq.codebook(128, b - 1)
    p = tq.encode(xt.to(dev), b, "prod", cb, rot, qjl)
    torch.cuda.synchronize()
    encp = oracle.encode_prod(x, rmat, cb_o, S_MAT)
    gidx = oracle.unpack_bits(to_np_words(p.idx), 128, b - 1)
    bad_rows, _ = check_indices(gidx, encp.mse.y, cb_o, f"prod stage {kind} b={b}")
    gz = unpack_z(to_np_words(p.qjl), 128)
    check_signs(gz, encp.proj, S_MAT, encp.mse.norms, ~bad_rows, f"prod signs {kind} b={b}")
    g = p.rnorms.cpu().numpy()
    ok = ~bad_rows
    assert np.all(np.abs(g[ok] - encp.gamma[ok]) <= 2e-5 * encp.mse.norms[ok] + 1e-12)
    np.testing.assert_allclose(p.norms.cpu().numpy(), encp.mse.norms, rtol=1e-6)


def _packed_to_oracle(p, d, bits, prod):
    idx = oracle.unpack_bits(to_np_words(p.idx), d, bits)
    norms = p.norms.cpu().numpy().astype(np.float64)
    mse = oracle.EncodedMSE(idx=idx, words=to_np_words(p.idx), norms=norms, y=None)
    if not prod:
        return mse
    z = unpack_z(to_np_words(p.qjl), d)
    return oracle.EncodedProd(mse=mse, z=z, qjl_words=to_np_words(p.qjl),
                              gamma=p.rnorms.cpu().numpy().astype(np.float64), proj=None)


@pytest.mark.parametrize("b,hkv,hq,T,B", [(3, 2, 8, 1000, 2), (2, 1, 32, 4096, 1), (4, 4, 8, 17, 1),
                                         (1, 2, 4, 300, 1), (3, 8, 8, 64, 1), (2, 4, 8, 33, 3),
                                         (3, 2, 6, 257, 1)])
def test_scores_mse_on_gpu_packed(dev, rot_dense, b, hkv, hq, T, B):
    x, xt = _keys(T, hkv=hkv, B=B)
    cb_o = oracle.codebook(128, b)
    cb = tq.codebook(128, b)
    p = tq.encode(xt.to(dev), b, "mse", cb, rot_dense)
    q = wl.gaussian((B, hq, 128), 12)
    s = tq.scores(torch.from_numpy(q).to(dev), p, hkv, cb, rot_dense)
    torch.cuda.synchronize()
    got = s.cpu().numpy()
    enc = _packed_to_oracle(p, 128, b, False)
    ratio = hq // hkv
    for bi in range(B):
        for g in range(hkv):
            rows = slice((bi * hkv + g) * T, (bi * hkv + g + 1) * T)
            heads = q[bi, g * ratio:(g + 1) * ratio].astype(np.float64)
            ref = oracle.scores_mse(heads, enc.idx[rows], enc.norms[rows], R_DENSE, cb_o)
            tol = score_tolerance(heads, enc.norms[rows])
            err = np.abs(got[bi, g * ratio:(g + 1) * ratio] - ref)
            assert np.all(err <= tol), (bi, g, float((err / tol).max()))


@pytest.mark.parametrize("kind", ["dense", "wht"])
@pytest.mark.parametrize("hkv,hq,T,B", [(4, 16, 700, 2), (2, 2, 129, 1)])
def test_scores_prod_on_gpu_packed(dev, rot_dense, rot_wht, kind, hkv, hq, T, B):
    rot, rmat = (rot_dense, R_DENSE) if kind == "dense" else (rot_wht, R_WHT)
    qjl = tq.make_qjl(128, 2, rot)
    x, xt = _keys(T, hkv=hkv, B=B)
    cb_o = oracle.codebook(128, 3)
    cb = tq.codebook(128, 3)
    p = tq.encode(xt.to(dev), 4, "prod", cb, rot, qjl)
    q = wl.gaussian((B, hq, 128), 12)
    s = tq.scores(torch.from_numpy(q).to(dev), p, hkv, cb, rot, qjl)
    torch.cuda.synchronize()
    got = s.cpu().numpy()
    encp = _packed_to_oracle(p, 128, 3, True)
    ratio = hq // hkv
    for bi in range(B):
        for g in range(hkv):
            r0, r1 = (bi * hkv + g) * T, (bi * hkv + g + 1) * T
            sub = oracle.EncodedProd(
                mse=oracle.EncodedMSE(idx=encp.mse.idx[r0:r1], words=None, norms=encp.mse.norms[r0:r1], y=None),
                z=encp.z[r0:r1], qjl_words=None, gamma=encp.gamma[r0:r1], proj=None)
            heads = q[bi, g * ratio:(g + 1) * ratio].astype(np.float64)
            ref = oracle.scores_prod(heads, sub, rmat, cb_o, S_MAT)
            tol = score_tolerance(heads, encp.mse.norms[r0:r1])
            err = np.abs(got[bi, g * ratio:(g + 1) * ratio] - ref)
            assert np.all(err <= tol), (bi, g, float((err / tol).max()))


def test_decode_parity(dev, rot_dense):
    qjl = tq.make_qjl(128, 2, rot_dense)
    x, xt = _keys(300, hkv=1)
    cb_o = oracle.codebook(128, 3)
    cb = tq.codebook(128, 3)
    p = tq.encode(xt.to(dev), 4, "prod", cb, rot_dense, qjl)
    xm = tq.decode(p, cb, rot_dense).cpu().numpy()
    xp = tq.decode(p, cb, rot_dense, qjl).cpu().numpy()
    torch.cuda.synchronize()
    encp = _packed_to_oracle(p, 128, 3, True)
    ref_m = oracle.decode_mse(encp.mse.idx, encp.mse.norms, R_DENSE, cb_o)
    ref_p = oracle.decode_prod(encp, R_DENSE, cb_o, S_MAT)
    s = encp.mse.norms[:, None]
    assert np.all(np.abs(xm - ref_m) <= 1e-5 * s + 1e-12)
    assert np.all(np.abs(xp - ref_p) <= 1e-5 * s + 1e-12)


def test_zero_and_tiny_inputs(dev, rot_dense):
    cb = tq.codebook(128, 3)
    x = torch.zeros((5, 128), dtype=torch.bfloat16, device=dev)
    p = tq.encode(x, 3, "mse", cb, rot_dense)
    torch.cuda.synchronize()
    idx = oracle.unpack_bits(to_np_words(p.idx), 128, 3)
    assert np.all(idx == 4) and np.all(p.norms.cpu().numpy() == 0)
    qjl = tq.make_qjl(128, 2, rot_dense)
    p2 = tq.encode(x, 4, "prod", tq.codebook(128, 3), rot_dense, qjl)
    torch.cuda.synchronize()
    assert np.all(to_np_words(p2.qjl) == 0xFFFFFFFF) and np.all(p2.rnorms.cpu().numpy() == 0)
    # empty batch: nothing launched, nothing written
    e = tq.encode(torch.zeros((0, 128), dtype=torch.bfloat16, device=dev), 3, "mse", cb, rot_dense)
    assert e.n == 0


def test_error_codes_on_device(dev, rot_dense):
    cb3 = tq.codebook(128, 3)
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(tq.TQError) as ei:
        tq.encode(x, 2, "mse", cb3, rot_dense)          # codebook bits != b
    assert ei.value.status == 2
    with pytest.raises(tq.TQError):
        tq.encode(x, 4, "prod", cb3, rot_dense, None)   # prod without qjl
    rot64 = tq.make_rotation(64, 1)
    with pytest.raises(tq.TQError) as ei:
        tq.encode(x, 3, "mse", cb3, rot64)              # d mismatch
    assert ei.value.status == 2
    p = tq.encode(x, 3, "mse", cb3, rot_dense)
    q = torch.zeros((1, 6, 128), dtype=torch.float32, device=dev)
    with pytest.raises(tq.TQError):
        tq.scores(q, p, 4, cb3, rot_dense)              # Hq % Hkv != 0
    ws = torch.empty(8, dtype=torch.uint8, device=dev)
    with pytest.raises(tq.TQError) as ei:
        tq.scores(torch.zeros((1, 4, 128), device=dev), p, 1, cb3, rot_dense, ws=ws)
    assert ei.value.status == 4


@pytest.mark.parametrize("mode,b", [("mse", 3), ("prod", 4)])
def test_scores_prepared_matches_scores(dev, rot_dense, mode, b):
    """The two stages (query prologue on a side stream, then the score kernel) give the very
    scores of tq_scores: same kernels, same inputs."""
    stage = b - 1 if mode == "prod" else b
    qjl = tq.make_qjl(128, 2, rot_dense) if mode == "prod" else None
    cb = tq.codebook(128, stage)
    x, xt = _keys(700, hkv=4, B=2)
    p = tq.encode(xt.to(dev), b, mode, cb, rot_dense, qjl)
    q = torch.from_numpy(wl.gaussian((2, 16, 128), 12)).to(dev)
    ref = tq.scores(q, p, 4, cb, rot_dense, qjl)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ws = tq.prepare_queries(q, 4, rot_dense, qjl)
    torch.cuda.current_stream().wait_stream(side)
    got = tq.scores_prepared(ws, 2, 16, p, 4, cb)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    with pytest.raises(tq.TQError):
        tq.scores_prepared(ws[:16], 2, 16, p, 4, cb)


def test_kernel_timer(dev, rot_dense):
    """The timer attached to a d = 128 encode launch reports a positive duration; ids are reusable
    after a reset."""
    cb = tq.codebook(128, 3)
    x = _keys(4096, hkv=2)[1].to(dev)
    tq.timer_reset()
    t = tq.timer_arm()
    tq.encode(x, 3, "mse", cb, rot_dense)
    ms = tq.timer_read(t)
    assert 0.0 < ms < 1000.0
    tq.timer_reset()
    assert tq.timer_arm() == t      # the first free id again
    tq.encode(x, 3, "mse", cb, rot_dense)
    assert tq.timer_read(t) > 0.0
    tq.timer_reset()
