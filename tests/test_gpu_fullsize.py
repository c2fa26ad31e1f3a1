"""GPU parity at the workloads' full sizes, through the same library calls (and so the same launch
configurations) that bench.py times, checked on seeded samples of the outputs that the oracle
computes one by one, or by properties that hold at any size:

* KV-key compression, 1 x 8 KV heads x 32768 tokens x d = 128 bf16, MSE b = 3, dense R: the
  indices and norms of 4096 sampled keys against the oracle's encode; 4096 sampled (head,
  token) scores of the 32 query heads against the oracle's score of the GPU's own packed keys.
* TurboQuant_prod b = 4, 16 x 8 x 16384 tokens, dense and WHT R: 2048 sampled keys (stage
  indices, QJL signs, residual norms); 4096 sampled scores.
* Decode attention, 4 x 131072 tokens x 8 KV heads, K and V MSE at b = 2 and b = 4: two
  (sequence, KV head) groups, all four query heads of each, against oracle attention over the
  group's 131072 packed keys and values.
* Streaming decode loop on caches of the same shape: a prefill of 131072 - 110 tokens, three
  single-token appends, attention over the prefix: 2048 sampled prefill rows and every appended
  row of both caches against the oracle's encode, and two groups' attention.
* Vector index, 1e6 unit vectors d = 1536, prod b = 4, 1024 queries, top-10: 512 sampled
  database rows against the oracle's encode; for 6 sampled queries the returned scores equal
  the oracle's scores of the returned indices, and the oracle's top-10 over all 1e6 keys (its
  scores of the GPU's packed rows, in chunks on worker processes) is the returned set (up to
  ties within tolerance).

Tolerances are those of the other parity tests (the boundary-band rule for indices and signs,
1e-3 ||q|| ||k|| for scores).
"""

import os

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _oracle_pool import prod_scores_all, save_db
from _parity import check_indices, check_signs, require_gpu, score_tolerance, to_np_words, unpack_z

pytestmark = pytest.mark.gpu

R128 = oracle.dense_rotation(128, 1)
W128 = oracle.wht_rotation(128, 1)
S128 = oracle.qjl_matrix(128, 2)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _to_dev_bf16(bits, n, d, dev):
    return torch.from_numpy(bits.reshape(n, d).view(np.int16)).to(dev).view(torch.bfloat16)


def _rows_f64(bits, rows, d):
    return wl.bf16_bits_to_f32(bits.reshape(-1, d)[rows]).astype(np.float64)


def test_kv_keys_full_size_sampled(dev):
    cfg = wl.CONFIGS["c2"]
    n = cfg.B * cfg.hkv * cfg.T
    print(f"kv keys: {n} keys, d={cfg.d}, MSE b={cfg.bits}", flush=True)
    bits = wl.kv_keys(cfg)
    rot = tq.make_rotation(cfg.d, cfg.rot_seed, "dense")
    cb, cb_o = tq.codebook(cfg.d, cfg.bits), oracle.codebook(cfg.d, cfg.bits)
    p = tq.alloc_packed(n, cfg.d, cfg.bits, "mse", device=dev)
    tq.encode(_to_dev_bf16(bits, n, cfg.d, dev), cfg.bits, "mse", cb, rot, out=p)
    q = wl.kv_queries(cfg)
    s = tq.scores(torch.from_numpy(q).to(dev), p, cfg.hkv, cb, rot)
    torch.cuda.synchronize()
    rng = np.random.default_rng(101)
    rows = np.sort(rng.choice(n, 4096, replace=False))
    words = to_np_words(p.idx)[rows]
    norms = p.norms.cpu().numpy()[rows].astype(np.float64)
    enc = oracle.encode_mse(_rows_f64(bits, rows, cfg.d), R128, cb_o)
    gidx = oracle.unpack_bits(words, cfg.d, cfg.bits)
    bad, _ = check_indices(gidx, enc.y, cb_o, "kv keys full size")
    np.testing.assert_array_equal(words[~bad], enc.words[~bad])
    np.testing.assert_allclose(norms, enc.norms, rtol=1e-6)
    # scores: sampled (head, token) pairs on the GPU's own packed keys
    got = s.cpu().numpy()
    ratio = cfg.hq // cfg.hkv
    hs = rng.integers(0, cfg.hq, 4096)
    ts = rng.integers(0, cfg.T, 4096)
    krow = (hs // ratio) * cfg.T + ts
    kidx = oracle.unpack_bits(to_np_words(p.idx)[krow], cfg.d, cfg.bits)
    kn = p.norms.cpu().numpy()[krow].astype(np.float64)
    for h in np.unique(hs):
        m = hs == h
        ref = oracle.scores_mse(q[0, h:h + 1].astype(np.float64), kidx[m], kn[m], R128, cb_o)[0]
        tol = score_tolerance(q[0, h:h + 1].astype(np.float64), kn[m])[0]
        err = np.abs(got[0, h, ts[m]] - ref)
        assert np.all(err <= tol), (int(h), float((err / tol).max()))


@pytest.mark.parametrize("kind", ["dense", "wht"])
def test_prod_keys_full_size_sampled(dev, kind):
    cfg = wl.CONFIGS["c3"]
    n = cfg.B * cfg.hkv * cfg.T
    print(f"prod keys: {n} keys, rotation {kind}", flush=True)
    bits = wl.kv_keys(cfg)
    rot = tq.make_rotation(cfg.d, cfg.rot_seed, kind)
    rmat = R128 if kind == "dense" else W128
    qjl = tq.make_qjl(cfg.d, cfg.qjl_seed, rot)
    cb, cb_o = tq.codebook(cfg.d, cfg.bits - 1), oracle.codebook(cfg.d, cfg.bits - 1)
    p = tq.alloc_packed(n, cfg.d, cfg.bits - 1, "prod", device=dev)
    tq.encode(_to_dev_bf16(bits, n, cfg.d, dev), cfg.bits, "prod", cb, rot, qjl, out=p)
    q = wl.kv_queries(cfg)
    s = tq.scores(torch.from_numpy(q).to(dev), p, cfg.hkv, cb, rot, qjl)
    torch.cuda.synchronize()
    rng = np.random.default_rng(102)
    rows = np.sort(rng.choice(n, 2048, replace=False))
    encp = oracle.encode_prod(_rows_f64(bits, rows, cfg.d), rmat, cb_o, S128)
    gidx = oracle.unpack_bits(to_np_words(p.idx)[rows], cfg.d, cfg.bits - 1)
    bad, _ = check_indices(gidx, encp.mse.y, cb_o, f"prod full size {kind}")
    gz = unpack_z(to_np_words(p.qjl)[rows], cfg.d)
    check_signs(gz, encp.proj, S128, encp.mse.norms, ~bad, f"prod signs full size {kind}")
    g = p.rnorms.cpu().numpy()[rows]
    assert np.all(np.abs(g[~bad] - encp.gamma[~bad]) <= 2e-5 * encp.mse.norms[~bad] + 1e-12)
    # scores: sampled (sequence, head, token) triples on the GPU's own packed keys
    got = s.cpu().numpy()
    ratio = cfg.hq // cfg.hkv
    bs = rng.integers(0, cfg.B, 4096)
    hs = rng.integers(0, cfg.hq, 4096)
    ts = rng.integers(0, cfg.T, 4096)
    krow = (bs * cfg.hkv + hs // ratio) * cfg.T + ts
    sub = oracle.EncodedProd(
        mse=oracle.EncodedMSE(idx=oracle.unpack_bits(to_np_words(p.idx)[krow], cfg.d, cfg.bits - 1), words=None,
                              norms=p.norms.cpu().numpy()[krow].astype(np.float64), y=None),
        z=unpack_z(to_np_words(p.qjl)[krow], cfg.d), qjl_words=None,
        gamma=p.rnorms.cpu().numpy()[krow].astype(np.float64), proj=None)
    qs = q[bs, hs].astype(np.float64)                        # one query per sampled key
    ref_all = oracle.scores_prod(qs, sub, rmat, cb_o, S128)   # [4096, 4096]; the diagonal is used
    ref = np.diagonal(ref_all)
    tol = 1e-3 * np.linalg.norm(qs, axis=1) * sub.mse.norms
    err = np.abs(got[bs, hs, ts] - ref)
    assert np.all(err <= tol), float((err / tol).max())


@pytest.mark.parametrize("b", [2, 4])
def test_decode_attention_full_size_sampled(dev, b):
    cfg = wl.CONFIGS["c4"]
    n = cfg.B * cfg.hkv * cfg.T
    print(f"decode attention: {cfg.B} x {cfg.hkv} x {cfg.T}, b={b}", flush=True)
    rot = tq.make_rotation(cfg.d, cfg.rot_seed)
    cb, cb_o = tq.codebook(cfg.d, b), oracle.codebook(cfg.d, b)
    K = tq.encode(_to_dev_bf16(wl.kv_keys(cfg), n, cfg.d, dev), b, "mse", cb, rot)
    V = tq.encode(_to_dev_bf16(wl.kv_values(cfg), n, cfg.d, dev), b, "mse", cb, rot, layout="blocked")
    q = wl.kv_queries(cfg)
    out = tq.decode_attn(torch.from_numpy(q).to(dev), K, V, cfg.hkv, cb, cb, rot, rot)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    kw, vw = to_np_words(K.idx), to_np_words(V.idx)
    kn_all, vn_all = K.norms.cpu().numpy(), V.norms.cpu().numpy()
    ratio = cfg.hq // cfg.hkv
    rng = np.random.default_rng(103)
    for _ in range(2):
        bi, g = int(rng.integers(0, cfg.B)), int(rng.integers(0, cfg.hkv))
        r0 = (bi * cfg.hkv + g) * cfg.T
        kidx = oracle.unpack_bits(kw[r0:r0 + cfg.T], cfg.d, b)
        blk0 = r0 // 32
        vidx = oracle.unpack_token_blocked(vw.reshape(-1, cfg.d * b)[blk0:blk0 + cfg.T // 32], cfg.T, cfg.d, b)
        kn = kn_all[r0:r0 + cfg.T].astype(np.float64)
        vn = vn_all[r0:r0 + cfg.T].astype(np.float64)
        heads = q[bi:bi + 1, g * ratio:(g + 1) * ratio].astype(np.float64)
        ref = oracle.decode_attention(heads, kidx[None, None], kn[None, None], vidx[None, None], vn[None, None],
                                      R128, R128, cb_o, cb_o, 1 / np.sqrt(cfg.d))[0]
        vmax = np.max(np.linalg.norm(oracle.decode_mse(vidx, vn, R128, cb_o), axis=1))
        err = np.abs(got[bi, g * ratio:(g + 1) * ratio] - ref)
        assert np.all(err <= 1e-3 * vmax), (bi, g, float(err.max()), vmax)


@pytest.mark.parametrize("b", [2, 4])
def test_decode_loop_full_size_sampled(dev, b):
    """The streaming decode loop as bench.py runs it: caches of 4 x 8 KV heads x 131072 tokens,
    prefilled to T0 = 131072 - 110 tokens in one append (fused encode on whole blocks, per-token
    tail), then three single-token decode steps, then attention over T0 + 3 tokens."""
    cfg = wl.CONFIGS["c4"]
    t_cap, t0, steps = cfg.T, cfg.T - 110, 3
    n_seq = cfg.B * cfg.hkv
    print(f"decode loop: {cfg.B} x {cfg.hkv} x {t_cap}, prefill {t0}, b={b}", flush=True)
    rot = tq.make_rotation(cfg.d, cfg.rot_seed)
    cb, cb_o = tq.codebook(cfg.d, b), oracle.codebook(cfg.d, b)
    kc = tq.alloc_cache(cfg.B, cfg.hkv, t_cap, cfg.d, b, "mse", device=dev)
    vc = tq.alloc_cache(cfg.B, cfg.hkv, t_cap, cfg.d, b, "mse", layout="blocked", device=dev)
    kbits, vbits = wl.kv_keys(cfg), wl.kv_values(cfg)
    as_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    tq.cache_append(kc, as_dev(kbits[:, :, :t0]), 0, cb, rot)
    tq.cache_append(vc, as_dev(vbits[:, :, :t0]), 0, cb, rot)
    for i in range(steps):
        tq.cache_append(kc, as_dev(kbits[:, :, t0 + i:t0 + i + 1]), t0 + i, cb, rot)
        tq.cache_append(vc, as_dev(vbits[:, :, t0 + i:t0 + i + 1]), t0 + i, cb, rot)
    T = t0 + steps
    q = wl.kv_queries(cfg)
    out = tq.decode_attn_cache(torch.from_numpy(q).to(dev), kc, vc, T, cb, cb, rot, rot)
    torch.cuda.synchronize()
    kw, vw = to_np_words(kc.packed.idx), to_np_words(vc.packed.idx)
    kn_all, vn_all = kc.packed.norms.cpu().numpy(), vc.packed.norms.cpu().numpy()
    rng = np.random.default_rng(107)
    # sampled prefill rows and every decode-step row, both caches, against the oracle's encode
    seq = np.concatenate([rng.integers(0, n_seq, 2048), np.repeat(np.arange(n_seq), steps)])
    tok = np.concatenate([rng.integers(0, t0, 2048), np.tile(np.arange(t0, T), n_seq)])
    rows = seq * t_cap + tok
    for bits_, words, norms, blocked in ((kbits, kw, kn_all, False), (vbits, vw, vn_all, True)):
        x = wl.bf16_bits_to_f32(bits_.reshape(n_seq, t_cap, cfg.d)[seq, tok]).astype(np.float64)
        enc = oracle.encode_mse(x, R128, cb_o)
        if blocked:
            gidx = np.stack([oracle.unpack_token_blocked(words.reshape(-1, cfg.d * b)[r // 32:r // 32 + 1], 32,
                                                         cfg.d, b)[r % 32] for r in rows])
        else:
            gidx = oracle.unpack_bits(words[rows], cfg.d, b)
        check_indices(gidx, enc.y, cb_o, f"decode loop {'V' if blocked else 'K'} b={b}")
        np.testing.assert_allclose(norms[rows], enc.norms, rtol=1e-6)
    got = out.cpu().numpy()
    ratio = cfg.hq // cfg.hkv
    for _ in range(2):
        bi, g = int(rng.integers(0, cfg.B)), int(rng.integers(0, cfg.hkv))
        r0 = (bi * cfg.hkv + g) * t_cap
        kidx = oracle.unpack_bits(kw[r0:r0 + T], cfg.d, b)
        vidx = oracle.unpack_token_blocked(vw.reshape(-1, cfg.d * b)[r0 // 32:(r0 + t_cap) // 32], t_cap, cfg.d, b)[:T]
        kn = kn_all[r0:r0 + T].astype(np.float64)
        vn = vn_all[r0:r0 + T].astype(np.float64)
        heads = q[bi:bi + 1, g * ratio:(g + 1) * ratio].astype(np.float64)
        ref = oracle.decode_attention(heads, kidx[None, None], kn[None, None], vidx[None, None], vn[None, None],
                                      R128, R128, cb_o, cb_o, 1 / np.sqrt(cfg.d))[0]
        vmax = np.max(np.linalg.norm(oracle.decode_mse(vidx, vn, R128, cb_o), axis=1))
        err = np.abs(got[bi, g * ratio:(g + 1) * ratio] - ref)
        assert np.all(err <= 1e-3 * vmax), (bi, g, float(err.max()), vmax)


def test_vector_index_full_size_sampled(dev, tmp_path):
    cfg = wl.CONFIGS["c5"]
    n, d = cfg.n, cfg.d
    nq, k = cfg.extra["queries"], cfg.extra["k"]
    print(f"vector index: {n} x {d}, {nq} queries, top-{k}", flush=True)
    rng = np.random.default_rng(104)
    rows = np.sort(rng.choice(n, 512, replace=False))
    x = torch.empty((n, d), dtype=torch.float32, device=dev)
    xs = []
    for lo, xc in wl.index_vectors(cfg):
        x[lo:lo + xc.shape[0]].copy_(torch.from_numpy(xc))
        sel = rows[(rows >= lo) & (rows < lo + xc.shape[0])]
        xs.append(xc[sel - lo])
    x_rows = np.concatenate(xs).astype(np.float64)
    qn = wl.index_queries(cfg)
    rot = tq.make_rotation(d, cfg.rot_seed, "dense")
    qjl = tq.make_qjl(d, cfg.qjl_seed, rot)
    cb, cb_o = tq.codebook(d, cfg.bits - 1), oracle.codebook(d, cfg.bits - 1)
    p = tq.alloc_packed(n, d, cfg.bits - 1, "prod", device=dev)
    ews = torch.empty((tq.encode_workspace(n, d, cfg.bits, "prod"),), dtype=torch.uint8, device=dev)
    tq.encode(x, cfg.bits, "prod", cb, rot, qjl, out=p, ws=ews)
    del x
    top_s, top_i = tq.search_topk(torch.from_numpy(qn).to(dev), p, k, cb, rot, qjl)
    torch.cuda.synchronize()
    print("encoded and searched; checking samples", flush=True)
    rmat, smat = oracle.dense_rotation(d, cfg.rot_seed), oracle.qjl_matrix(d, cfg.qjl_seed)
    # encode: sampled database rows
    words, qwords = to_np_words(p.idx), to_np_words(p.qjl)
    norms, rn = p.norms.cpu().numpy(), p.rnorms.cpu().numpy()
    encp = oracle.encode_prod(x_rows, rmat, cb_o, smat)
    gidx = oracle.unpack_bits(words[rows], d, cfg.bits - 1)
    bad, _ = check_indices(gidx, encp.mse.y, cb_o, "vector index encode")
    check_signs(unpack_z(qwords[rows], d), encp.proj, smat, encp.mse.norms, ~bad, "vector index signs")
    assert np.all(np.abs(rn[rows][~bad] - encp.gamma[~bad]) <= 2e-5 * encp.mse.norms[~bad] + 1e-12)

    # search: sampled queries; scores of returned keys, and the oracle's top-k over every key of
    # the database (its scores of the GPU's own packed rows, in chunks over worker processes)
    gs, gi = top_s.cpu().numpy(), top_i.cpu().numpy()
    qsel = np.sort(rng.choice(nq, 6, replace=False))
    qv = qn[qsel].astype(np.float64)
    path = str(tmp_path / "db")
    save_db(path, words=words, qwords=qwords, norms=norms, rnorms=rn, rmat=rmat, smat=smat, q=qv,
            meta=np.array([d, cfg.bits - 1]))
    print("oracle scores of all keys", flush=True)
    pool = np.arange(n)
    ref_pool = prod_scores_all(path, n, workers=min(16, os.cpu_count() or 1))   # [6, n]
    print("oracle scores done", flush=True)
    for j, qi in enumerate(qsel):
        tol = 1e-3 * np.linalg.norm(qv[j]) * np.max(norms)
        ret = gi[qi]
        assert np.all((ret >= 0) & (ret < n)) and len(set(ret.tolist())) == k
        assert np.all(np.diff(gs[qi]) <= 0)
        ref_ret = ref_pool[j, np.searchsorted(pool, ret)]
        assert np.all(np.abs(gs[qi] - ref_ret) <= tol), (int(qi), float(np.abs(gs[qi] - ref_ret).max()))
        # no key outside the returned set beats the k-th returned key beyond the tolerance, and every
        # returned key is within the tolerance of the oracle's k-th best over the whole database
        kth = np.min(ref_ret)
        outside = ~np.isin(pool, ret)
        assert np.all(ref_pool[j, outside] <= kth + 2 * tol), (int(qi), float(ref_pool[j, outside].max() - kth))
        best_k = np.partition(ref_pool[j], n - k)[n - k]
        assert np.all(ref_ret >= best_k - 2 * tol), (int(qi), float(best_k - ref_ret.min()))
