"""GPU parity of the streaming KV cache (C ABI) against the oracle.

Prefill chunks and single decode tokens are appended into preallocated caches whose storage
starts as seeded garbage: rows-layout key caches (MSE and prod) and token-blocked value caches.
Appended rows must match the oracle's encode within the boundary band, and every other stored
bit must be unchanged: the expected words are the oracle's layout applied to the initial garbage
with the appended rows assigned.  Scores and decode attention over the cached prefix are then
compared with the oracle on the GPU's own packed bytes.  The append plan covers the per-token
kernel (short appends, partial value blocks) and the fused encode path (appends of 64 tokens or
more, with ragged heads and tails around whole blocks)."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _parity import check_indices, check_signs, require_gpu, to_np_words, unpack_z

pytestmark = pytest.mark.gpu

R = oracle.dense_rotation(128, 1)
S_MAT = oracle.qjl_matrix(128, 2)
# (position, tokens): prefill, three decode steps, a long ragged burst, a step, another burst
PLAN = [(0, 37), (37, 1), (38, 1), (39, 1), (40, 100), (140, 1), (141, 70)]
WRITTEN = 211
T_CAP = 224


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def rot(dev):
    return tq.make_rotation(128, 1)


def _tokens(B, H, n, which):
    if which == "k":
        bits = wl.kv_tensor_bf16(B, H, n, 128, seed=40, outlier_seed=10, scale_seed=41)
    else:
        bits = wl.kv_tensor_bf16(B, H, n, 128, seed=42, outlier_seed=21, scale_seed=None)
    x = wl.bf16_bits_to_f32(bits).astype(np.float64)
    return x, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def _garbage(t, seed):
    g = torch.Generator().manual_seed(seed)
    if t.dtype == torch.int32:
        t.copy_(torch.randint(-2**31, 2**31 - 1, t.shape, dtype=torch.int32, generator=g))
    else:
        t.copy_(torch.randn(t.shape, generator=g))


def _fill(cache, seed):
    p = cache.packed
    for i, t in enumerate((p.idx, p.norms, p.qjl, p.rnorms)):
        if t is not None:
            _garbage(t, seed + i)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().clone() for t in (p.idx, p.norms, p.qjl, p.rnorms)]


def _run_plan(cache, xt, dev, cb, rot, qjl=None, dtype=torch.bfloat16):
    for pos, n in PLAN:
        chunk = xt[:, :, pos:pos + n].contiguous().to(dev)
        if dtype == torch.float32:
            chunk = chunk.float()
        tq.cache_append(cache, chunk, pos, cb, rot, qjl)
    torch.cuda.synchronize()


@pytest.mark.parametrize("b", [2, 3, 4])
def test_value_cache_appends(dev, rot, b):
    B, H = 2, 3
    x, xt = _tokens(B, H, WRITTEN, "v")
    cb, cbo = tq.codebook(128, b), oracle.codebook(128, b)
    vc = tq.alloc_cache(B, H, T_CAP, 128, b, "mse", layout="blocked", device=dev)
    init = _fill(vc, 100 + b)
    _run_plan(vc, xt, dev, cb, rot)
    n_rows = B * H * T_CAP
    words = to_np_words(vc.packed.idx)
    words0 = init[0].numpy().view(np.uint32)
    rows = oracle.live_rows(B * H, T_CAP, WRITTEN).reshape(-1)
    gidx = oracle.unpack_token_blocked(words, n_rows, 128, b)
    enc = oracle.encode_mse(x.reshape(-1, 128), R, cbo)
    check_indices(gidx[rows], enc.y, cbo, f"value cache b={b}")
    # every other field untouched, the appended ones where the layout puts them
    np.testing.assert_array_equal(words, oracle.assign_token_blocked(words0, n_rows, 128, b, rows, gidx[rows]))
    norms = vc.packed.norms.cpu().numpy()
    np.testing.assert_allclose(norms[rows], enc.norms, rtol=1e-6)
    keep = np.ones(n_rows, bool)
    keep[rows] = False
    np.testing.assert_array_equal(norms[keep], init[1].numpy()[keep])


@pytest.mark.parametrize("mode,b,dtype", [("mse", 3, torch.bfloat16), ("mse", 2, torch.float32),
                                          ("prod", 4, torch.bfloat16)])
def test_key_cache_appends(dev, rot, mode, b, dtype):
    B, H = 2, 2
    x, xt = _tokens(B, H, WRITTEN, "k")
    stage = b - 1 if mode == "prod" else b
    cb, cbo = tq.codebook(128, stage), oracle.codebook(128, stage)
    qjl = tq.make_qjl(128, 2, rot) if mode == "prod" else None
    kc = tq.alloc_cache(B, H, T_CAP, 128, b, mode, device=dev)
    init = _fill(kc, 200 + b)
    _run_plan(kc, xt, dev, cb, rot, qjl, dtype)
    n_rows = B * H * T_CAP
    rows = oracle.live_rows(B * H, T_CAP, WRITTEN).reshape(-1)
    keep = np.ones(n_rows, bool)
    keep[rows] = False
    words = to_np_words(kc.packed.idx)
    gidx = oracle.unpack_bits(words[rows], 128, stage)
    xf = x.reshape(-1, 128)
    if mode == "prod":
        encp = oracle.encode_prod(xf, R, cbo, S_MAT)
        enc = encp.mse
    else:
        enc = oracle.encode_mse(xf, R, cbo)
    bad, _ = check_indices(gidx, enc.y, cbo, f"key cache {mode} b={b}")
    np.testing.assert_allclose(kc.packed.norms.cpu().numpy()[rows], enc.norms, rtol=1e-6)
    for cur, old in zip((kc.packed.idx, kc.packed.norms, kc.packed.qjl, kc.packed.rnorms), init):
        if cur is not None:
            np.testing.assert_array_equal(cur.cpu().numpy()[keep], old.numpy()[keep])
    if mode == "prod":
        gz = unpack_z(to_np_words(kc.packed.qjl)[rows], 128)
        check_signs(gz, encp.proj, S_MAT, enc.norms, ~bad, "key cache signs")
        g = kc.packed.rnorms.cpu().numpy()[rows]
        ok = ~bad
        assert np.all(np.abs(g[ok] - encp.gamma[ok]) <= 2e-5 * enc.norms[ok] + 1e-12)


def _prefix(words_idx, norms, n_seq, T, stage, blocked):
    rows = oracle.live_rows(n_seq, T_CAP, T).reshape(-1)
    if blocked:
        idx = oracle.unpack_token_blocked(words_idx, n_seq * T_CAP, 128, stage)[rows]
    else:
        idx = oracle.unpack_bits(words_idx[rows], 128, stage)
    return idx, norms[rows].astype(np.float64)


@pytest.mark.parametrize("kb,vb", [(2, 2), (4, 3)])
def test_decode_over_cache(dev, rot, kb, vb):
    """Attention and scores after each stage of the plan, on the prefix written so far."""
    B, Hkv, Hq = 2, 2, 8
    xk, kt = _tokens(B, Hkv, WRITTEN, "k")
    xv, vt = _tokens(B, Hkv, WRITTEN, "v")
    cbk, cbv = tq.codebook(128, kb), tq.codebook(128, vb)
    cbko, cbvo = oracle.codebook(128, kb), oracle.codebook(128, vb)
    kc = tq.alloc_cache(B, Hkv, T_CAP, 128, kb, "mse", device=dev)
    vc = tq.alloc_cache(B, Hkv, T_CAP, 128, vb, "mse", layout="blocked", device=dev)
    _fill(kc, 300)
    _fill(vc, 400)
    q = wl.gaussian((B, Hq, 128), 12)
    qd = torch.from_numpy(q).to(dev)
    ratio = Hq // Hkv
    for pos, n in PLAN:
        tq.cache_append(kc, kt[:, :, pos:pos + n].contiguous().to(dev), pos, cbk, rot)
        tq.cache_append(vc, vt[:, :, pos:pos + n].contiguous().to(dev), pos, cbv, rot)
        T = pos + n
        out = tq.decode_attn_cache(qd, kc, vc, T, cbk, cbv, rot, rot)
        sc = tq.scores_cache(qd, kc, T, cbk, rot)
        torch.cuda.synchronize()
        kidx, kn = _prefix(to_np_words(kc.packed.idx), kc.packed.norms.cpu().numpy(), B * Hkv, T, kb, False)
        vidx, vn = _prefix(to_np_words(vc.packed.idx), vc.packed.norms.cpu().numpy(), B * Hkv, T, vb, True)
        ref = oracle.decode_attention(q.astype(np.float64), kidx.reshape(B, Hkv, T, 128), kn.reshape(B, Hkv, T),
                                      vidx.reshape(B, Hkv, T, 128), vn.reshape(B, Hkv, T), R, R, cbko, cbvo,
                                      1 / np.sqrt(128))
        got = out.cpu().numpy()
        gs = sc.cpu().numpy()
        for bi in range(B):
            for g in range(Hkv):
                sl = slice((bi * Hkv + g) * T, (bi * Hkv + g + 1) * T)
                vh = oracle.decode_mse(vidx[sl], vn[sl], R, cbvo)
                vmax = np.max(np.linalg.norm(vh, axis=1))
                heads = slice(g * ratio, (g + 1) * ratio)
                err = np.max(np.abs(got[bi, heads] - ref[bi, heads]))
                assert err <= 1e-3 * vmax, (T, bi, g, err, vmax)
                sref = oracle.scores_mse(q[bi, heads].astype(np.float64), kidx[sl], kn[sl], R, cbko)
                tol = 1e-3 * np.linalg.norm(q[bi, heads], axis=1)[:, None] * kn[sl][None, :]
                assert np.all(np.abs(gs[bi, heads] - sref) <= tol), (T, bi, g)


def test_prod_scores_over_cache(dev, rot):
    B, Hkv, Hq = 1, 2, 8
    x, kt = _tokens(B, Hkv, WRITTEN, "k")
    cb, cbo = tq.codebook(128, 3), oracle.codebook(128, 3)
    qjl = tq.make_qjl(128, 2, rot)
    kc = tq.alloc_cache(B, Hkv, T_CAP, 128, 4, "prod", device=dev)
    _fill(kc, 500)
    _run_plan(kc, kt, dev, cb, rot, qjl)
    q = wl.gaussian((B, Hq, 128), 13)
    sc = tq.scores_cache(torch.from_numpy(q).to(dev), kc, WRITTEN, cb, rot, qjl)
    torch.cuda.synchronize()
    rows = oracle.live_rows(B * Hkv, T_CAP, WRITTEN).reshape(-1)
    p = kc.packed
    encp = oracle.EncodedProd(
        mse=oracle.EncodedMSE(idx=oracle.unpack_bits(to_np_words(p.idx)[rows], 128, 3), words=None,
                              norms=p.norms.cpu().numpy().astype(np.float64)[rows], y=None),
        z=unpack_z(to_np_words(p.qjl)[rows], 128), qjl_words=None,
        gamma=p.rnorms.cpu().numpy().astype(np.float64)[rows], proj=None)
    gs = sc.cpu().numpy()
    ratio = Hq // Hkv
    for g in range(Hkv):
        sl = slice(g * WRITTEN, (g + 1) * WRITTEN)
        sub = oracle.EncodedProd(mse=oracle.EncodedMSE(idx=encp.mse.idx[sl], words=None, norms=encp.mse.norms[sl],
                                                       y=None),
                                 z=encp.z[sl], qjl_words=None, gamma=encp.gamma[sl], proj=None)
        heads = slice(g * ratio, (g + 1) * ratio)
        ref = oracle.scores_prod(q[0, heads].astype(np.float64), sub, R, cbo, S_MAT)
        tol = 1e-3 * np.linalg.norm(q[0, heads], axis=1)[:, None] * encp.mse.norms[sl][None, :]
        assert np.all(np.abs(gs[0, heads] - ref) <= tol), g


def test_cache_errors(dev, rot):
    cb = tq.codebook(128, 2)
    kc = tq.alloc_cache(1, 2, 64, 128, 2, "mse", device=dev)
    vc = tq.alloc_cache(1, 2, 64, 128, 2, "mse", layout="blocked", device=dev)
    x = torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(tq.TQError):
        tq.cache_append(kc, x, 60, cb, rot)                      # overflows the capacity
    with pytest.raises(tq.TQError):
        tq.cache_append(kc, torch.zeros((1, 3, 8, 128), dtype=torch.bfloat16, device=dev), 0, cb, rot)
    odd = tq.alloc_cache(1, 2, 40, 128, 2, "mse", layout="blocked", device=dev)
    with pytest.raises(tq.TQError):
        tq.cache_append(odd, x, 0, cb, rot)                      # token blocks need T_cap % 32 == 0
    q = torch.zeros((1, 8, 128), device=dev)
    with pytest.raises(tq.TQError):
        tq.decode_attn_cache(q, kc, vc, 65, cb, cb, rot, rot)    # T beyond the capacity
    with pytest.raises(tq.TQError):
        tq.decode_attn_cache(q, kc, vc, 0, cb, cb, rot, rot)     # empty prefix
    with pytest.raises(tq.TQError):
        tq.scores_cache(q, kc, 65, cb, rot)
    # zero tokens appended: nothing to do, no error
    tq.cache_append(kc, torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=dev), 64, cb, rot)
    # zero vectors: norm 0, index of y = 0, and attention over them returns 0
    tq.cache_append(kc, x, 0, cb, rot)
    tq.cache_append(vc, x, 0, cb, rot)
    out = tq.decode_attn_cache(q, kc, vc, 8, cb, cb, rot, rot)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0.0)
    rows = oracle.live_rows(2, 64, 8).reshape(-1)
    assert np.all(kc.packed.norms.cpu().numpy()[rows] == 0.0)
    assert np.all(oracle.unpack_bits(to_np_words(kc.packed.idx)[rows], 128, 2) == 2)


@pytest.mark.parametrize("hkv,hq,mode", [(2, 16, "prod"), (2, 16, "mse"), (4, 4, "mse"), (2, 4, "mse")])
def test_scores_over_cache_gqa(dev, rot, hkv, hq, mode):
    """Scores over a capacity-strided cache at GQA ratios 8 (several head groups per key), 1 and 2."""
    B = 1
    x, kt = _tokens(B, hkv, WRITTEN, "k")
    b = 4 if mode == "prod" else 3
    stage = b - 1 if mode == "prod" else b
    cb, cbo = tq.codebook(128, stage), oracle.codebook(128, stage)
    qjl = tq.make_qjl(128, 2, rot) if mode == "prod" else None
    kc = tq.alloc_cache(B, hkv, T_CAP, 128, b, mode, device=dev)
    _fill(kc, 600)
    _run_plan(kc, kt, dev, cb, rot, qjl)
    q = wl.gaussian((B, hq, 128), 14)
    T = 150
    sc = tq.scores_cache(torch.from_numpy(q).to(dev), kc, T, cb, rot, qjl)
    torch.cuda.synchronize()
    rows = oracle.live_rows(B * hkv, T_CAP, T).reshape(-1)
    p = kc.packed
    idx = oracle.unpack_bits(to_np_words(p.idx)[rows], 128, stage)
    norms = p.norms.cpu().numpy().astype(np.float64)[rows]
    gs = sc.cpu().numpy()
    ratio = hq // hkv
    for g in range(hkv):
        sl = slice(g * T, (g + 1) * T)
        heads = slice(g * ratio, (g + 1) * ratio)
        qh = q[0, heads].astype(np.float64)
        if mode == "prod":
            sub = oracle.EncodedProd(mse=oracle.EncodedMSE(idx=idx[sl], words=None, norms=norms[sl], y=None),
                                     z=unpack_z(to_np_words(p.qjl)[rows][sl], 128), qjl_words=None,
                                     gamma=p.rnorms.cpu().numpy().astype(np.float64)[rows][sl], proj=None)
            ref = oracle.scores_prod(qh, sub, R, cbo, S_MAT)
        else:
            ref = oracle.scores_mse(qh, idx[sl], norms[sl], R, cbo)
        tol = 1e-3 * np.linalg.norm(qh, axis=1)[:, None] * norms[sl][None, :]
        assert np.all(np.abs(gs[0, heads] - ref) <= tol), (g, mode)


@pytest.mark.parametrize("hkv,hq", [(2, 2), (2, 4)])
def test_decode_over_cache_gqa_and_fp32_values(dev, rot, hkv, hq):
    """Attention over the cache at GQA ratios 1 and 2, with the values appended from fp32."""
    B, kb, vb = 1, 3, 2
    xk, kt = _tokens(B, hkv, WRITTEN, "k")
    xv, vt = _tokens(B, hkv, WRITTEN, "v")
    cbk, cbv = tq.codebook(128, kb), tq.codebook(128, vb)
    cbko, cbvo = oracle.codebook(128, kb), oracle.codebook(128, vb)
    kc = tq.alloc_cache(B, hkv, T_CAP, 128, kb, "mse", device=dev)
    vc = tq.alloc_cache(B, hkv, T_CAP, 128, vb, "mse", layout="blocked", device=dev)
    _fill(kc, 700)
    _fill(vc, 800)
    _run_plan(kc, kt, dev, cbk, rot)
    _run_plan(vc, vt, dev, cbv, rot, dtype=torch.float32)
    q = wl.gaussian((B, hq, 128), 15)
    out = tq.decode_attn_cache(torch.from_numpy(q).to(dev), kc, vc, WRITTEN, cbk, cbv, rot, rot)
    torch.cuda.synchronize()
    rows = oracle.live_rows(B * hkv, T_CAP, WRITTEN).reshape(-1)
    vidx_all = oracle.unpack_token_blocked(to_np_words(vc.packed.idx), B * hkv * T_CAP, 128, vb)
    check_indices(vidx_all[rows], oracle.encode_mse(xv.reshape(-1, 128), R, cbvo).y, cbvo, "fp32 values")
    kidx, kn = _prefix(to_np_words(kc.packed.idx), kc.packed.norms.cpu().numpy(), B * hkv, WRITTEN, kb, False)
    vidx, vn = vidx_all[rows], vc.packed.norms.cpu().numpy().astype(np.float64)[rows]
    ref = oracle.decode_attention(q.astype(np.float64), kidx.reshape(B, hkv, WRITTEN, 128),
                                  kn.reshape(B, hkv, WRITTEN), vidx.reshape(B, hkv, WRITTEN, 128),
                                  vn.reshape(B, hkv, WRITTEN), R, R, cbko, cbvo, 1 / np.sqrt(128))
    got = out.cpu().numpy()
    ratio = hq // hkv
    for g in range(hkv):
        sl = slice(g * WRITTEN, (g + 1) * WRITTEN)
        vmax = np.max(np.linalg.norm(oracle.decode_mse(vidx[sl], vn[sl], R, cbvo), axis=1))
        err = np.max(np.abs(got[0, g * ratio:(g + 1) * ratio] - ref[0, g * ratio:(g + 1) * ratio]))
        assert err <= 1e-3 * vmax, (g, err, vmax)


@pytest.mark.parametrize("kb,vb", [(2, 2), (4, 3), (1, 4)])
def test_kv_append_matches_separate_appends(dev, rot, kb, vb):
    """The combined key and value append (one launch for short appends; (1, 4) takes the two-launch
    fallback) leaves both caches bit-identical to two separate appends, over the whole plan."""
    B, H = 2, 2
    _, kt = _tokens(B, H, WRITTEN, "k")
    _, vt = _tokens(B, H, WRITTEN, "v")
    cbk, cbv = tq.codebook(128, kb), tq.codebook(128, vb)
    caches = []
    for seed in (900, 900):
        kc = tq.alloc_cache(B, H, T_CAP, 128, kb, "mse", device=dev)
        vc = tq.alloc_cache(B, H, T_CAP, 128, vb, "mse", layout="blocked", device=dev)
        _fill(kc, seed)
        _fill(vc, seed + 50)
        caches.append((kc, vc))
    for pos, n in PLAN:
        k = kt[:, :, pos:pos + n].contiguous().to(dev)
        v = vt[:, :, pos:pos + n].contiguous().to(dev)
        tq.kv_append(caches[0][0], caches[0][1], k, v, pos, cbk, cbv, rot, rot)
        tq.cache_append(caches[1][0], k, pos, cbk, rot)
        tq.cache_append(caches[1][1], v, pos, cbv, rot)
    torch.cuda.synchronize()
    for a, b_ in zip(caches[0], caches[1]):
        np.testing.assert_array_equal(to_np_words(a.packed.idx), to_np_words(b_.packed.idx))
        np.testing.assert_array_equal(a.packed.norms.cpu().numpy(), b_.packed.norms.cpu().numpy())
    with pytest.raises(tq.TQError):
        tq.kv_append(caches[0][1], caches[0][0], k, v, 0, cbv, cbk, rot, rot)   # layouts swapped
