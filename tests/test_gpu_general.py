"""GPU parity of the general-d path (d a multiple of 128 above 128) and of the top-k search against
the fp64 oracle, through the C ABI: the vector-index workload's shape (d = 1536 unit vectors with
a low-rank component, fp32, prod b = 4) at sizes the oracle finishes in seconds, with ragged
tails against the 128-vector GEMM tiles, forced workspace chunking, and the edge cases."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _parity import check_indices, check_signs, require_gpu, to_np_words, unpack_z

pytestmark = pytest.mark.gpu

D = 1536


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def handles(dev):
    rot = tq.make_rotation(D, 1, "dense")
    qjl = tq.make_qjl(D, 2, rot)
    return rot, qjl


@pytest.fixture(scope="module")
def mats():
    return oracle.dense_rotation(D, 1), oracle.qjl_matrix(D, 2)


def _db(n, seed=0):
    """Unit vectors g + sqrt(24) U w (rank 64), fp32, as the vector-index workload."""
    return wl.lowrank_unit_vectors(n, D, 64, 24.0, seed, 30 + seed, 31 + seed)


def _queries(nq, seed=0):
    return wl.lowrank_unit_vectors(nq, D, 64, 24.0, 32 + seed, 30, 33 + seed)


@pytest.mark.parametrize("d,kind,dtype", [(1536, "dense", "f32"), (256, "wht", "f32"), (512, "dense", "bf16"),
                                          (1024, "wht", "bf16")])
def test_rotate_general(dev, d, kind, dtype):
    rot = tq.make_rotation(d, 1, kind)
    rmat = oracle.dense_rotation(d, 1) if kind == "dense" else oracle.wht_rotation(d, 1)
    x = wl.gaussian((300, d), 5) * np.float32(3.0)
    x[7] = 0.0
    if dtype == "bf16":
        bits = wl.f32_to_bf16_bits(x)
        x = wl.bf16_bits_to_f32(bits)
        xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        xt = torch.from_numpy(x)
    y, nr = tq.rotate(xt.to(dev), rot)
    torch.cuda.synchronize()
    ref = oracle.encode_mse(x.astype(np.float64), rmat, oracle.codebook(d, 1))
    assert np.max(np.abs(y.cpu().numpy() - ref.y)) <= 1e-5
    assert np.allclose(nr.cpu().numpy(), ref.norms, rtol=1e-6, atol=0)
    assert np.all(y.cpu().numpy()[7] == 0.0) and nr.cpu().numpy()[7] == 0.0


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_encode_mse_general(dev, handles, mats, b):
    rot, _ = handles
    rmat, _ = mats
    x = _db(1000 + b)
    cb_o = oracle.codebook(D, b)
    p = tq.encode(torch.from_numpy(x).to(dev), b, "mse", tq.codebook(D, b), rot)
    torch.cuda.synchronize()
    ref = oracle.encode_mse(x.astype(np.float64), rmat, cb_o)
    gidx = oracle.unpack_bits(to_np_words(p.idx), D, b)
    check_indices(gidx, ref.y, cb_o, f"mse d={D} b={b}")
    assert np.allclose(p.norms.cpu().numpy(), ref.norms, rtol=1e-6, atol=0)


@pytest.mark.parametrize("n,ws_vectors", [(1000, None), (1000, 256), (130, 128), (77, None)])
def test_encode_prod_general(dev, handles, mats, n, ws_vectors):
    rot, qjl = handles
    rmat, smat = mats
    x = _db(n, seed=1)
    x[3] = 0.0
    cb_o = oracle.codebook(D, 3)
    ws = None
    if ws_vectors is not None:
        per = tq.encode_workspace(1, D, 4, "prod")
        ws = torch.empty((per * ws_vectors,), dtype=torch.uint8, device=dev)
    p = tq.encode(torch.from_numpy(x).to(dev), 4, "prod", tq.codebook(D, 3), rot, qjl, ws=ws)
    torch.cuda.synchronize()
    encp = oracle.encode_prod(x.astype(np.float64), rmat, cb_o, smat)
    gidx = oracle.unpack_bits(to_np_words(p.idx), D, 3)
    bad_rows, _ = check_indices(gidx, encp.mse.y, cb_o, "prod stage d=1536")
    gz = unpack_z(to_np_words(p.qjl), D)
    check_signs(gz, encp.proj, smat, encp.mse.norms, ~bad_rows, "prod signs d=1536")
    g = p.rnorms.cpu().numpy()
    ok = ~bad_rows
    assert np.all(np.abs(g[ok] - encp.gamma[ok]) <= 2e-5 * encp.mse.norms[ok] + 1e-12)
    # the zero vector: norm 0, index K/2 everywhere, every sign +1, gamma 0
    assert p.norms.cpu().numpy()[3] == 0.0 and g[3] == 0.0
    assert np.all(gidx[3] == 4) and np.all(gz[3])


def test_encode_prod_workspace_too_small(dev, handles):
    rot, qjl = handles
    x = torch.from_numpy(_db(300)).to(dev)
    per = tq.encode_workspace(1, D, 4, "prod")
    ws = torch.empty((per * 100,), dtype=torch.uint8, device=dev)
    with pytest.raises(tq.TQError) as e:
        tq.encode(x, 4, "prod", tq.codebook(D, 3), rot, qjl, ws=ws)
    assert e.value.status == 4


def _packed_prod(p, d, bits):
    idx = oracle.unpack_bits(to_np_words(p.idx), d, bits)
    mse = oracle.EncodedMSE(idx=idx, words=None, norms=p.norms.cpu().numpy().astype(np.float64), y=None)
    return oracle.EncodedProd(mse=mse, z=unpack_z(to_np_words(p.qjl), d), qjl_words=None,
                              gamma=p.rnorms.cpu().numpy().astype(np.float64), proj=None)


def _check_topk(got_s, got_i, ref_scores, k, tol):
    """Scores of the returned indices within tol of the oracle's; the set equals the oracle's top-k
    except where ranks k and k + 1 are within tol (several correct answers); order descending."""
    ref_v, ref_i = oracle.topk(ref_scores, k)
    nq, n = ref_scores.shape
    kk = min(k, n)
    tols = np.broadcast_to(np.ravel(tol), (nq,))
    for i in range(nq):
        tol = float(tols[i])
        gi = got_i[i, :kk]
        assert np.all(gi >= 0) and np.all(gi < n) and len(set(gi.tolist())) == kk, i
        assert np.all(np.abs(got_s[i, :kk] - ref_scores[i, gi]) <= tol), (i, np.abs(got_s[i, :kk] - ref_scores[i, gi]).max())
        assert np.all(np.diff(got_s[i, :kk]) <= 0), i
        kth = ref_v[i, kk - 1]
        missing = set(ref_i[i].tolist()) - set(gi.tolist())
        for j in missing:
            assert ref_scores[i, j] <= kth + 2 * tol, (i, j)
        for j in set(gi.tolist()) - set(ref_i[i].tolist()):
            assert ref_scores[i, j] >= kth - 2 * tol, (i, j)
        if kk < k:
            assert np.all(got_i[i, kk:] == -1) and np.all(np.isneginf(got_s[i, kk:]))


@pytest.mark.parametrize("n,nq,k", [(3000, 100, 10), (70000, 20, 10), (5, 3, 10), (1000, 130, 32), (513, 1, 1),
                                    (4100, 7, 5)])
def test_search_topk(dev, handles, mats, n, nq, k):
    rot, qjl = handles
    rmat, smat = mats
    cb = tq.codebook(D, 3)
    cb_o = oracle.codebook(D, 3)
    x = _db(n, seed=2)
    p = tq.encode(torch.from_numpy(x).to(dev), 4, "prod", cb, rot, qjl)
    q = _queries(nq)
    q[0] *= 3.0  # a non-unit query
    top_s, top_i = tq.search_topk(torch.from_numpy(q).to(dev), p, k, cb, rot, qjl)
    torch.cuda.synchronize()
    encp = _packed_prod(p, D, 3)
    ref = oracle.scores_prod(q.astype(np.float64), encp, rmat, cb_o, smat)
    tol = 1e-3 * np.linalg.norm(q, axis=1) * np.max(p.norms.cpu().numpy())
    _check_topk(top_s.cpu().numpy(), top_i.cpu().numpy(), ref, k, tol)


def test_search_topk_d128(dev):
    rot = tq.make_rotation(128, 1, "wht")
    qjl = tq.make_qjl(128, 2, rot)
    cb = tq.codebook(128, 2)
    x = wl.gaussian((2000, 128), 7)
    p = tq.encode(torch.from_numpy(x).to(dev), 3, "prod", cb, rot, qjl)
    q = wl.gaussian((40, 128), 8)
    top_s, top_i = tq.search_topk(torch.from_numpy(q).to(dev), p, 10, cb, rot, qjl)
    torch.cuda.synchronize()
    encp = _packed_prod(p, 128, 2)
    ref = oracle.scores_prod(q.astype(np.float64), encp, oracle.wht_rotation(128, 1), oracle.codebook(128, 2),
                             oracle.qjl_matrix(128, 2))
    tol = 1e-3 * np.linalg.norm(q, axis=1) * np.max(p.norms.cpu().numpy())
    _check_topk(top_s.cpu().numpy(), top_i.cpu().numpy(), ref, 10, tol)


def _d128_handles():
    rot = tq.make_rotation(128, 3, "wht")
    return rot, tq.make_qjl(128, 4, rot), tq.codebook(128, 3)


def _d128_ref(p, q):
    encp = _packed_prod(p, 128, 3)
    return oracle.scores_prod(q.astype(np.float64), encp, oracle.wht_rotation(128, 3), oracle.codebook(128, 3),
                              oracle.qjl_matrix(128, 4))


def test_search_topk_rising_scores(dev):
    # Scores that rise with the index: every chunk after the first beats the running k-th result
    # many times over, so the kept-score masks carry many bits in every chunk (a short first
    # chunk, then chunks of 65536 vectors, the last one ragged).
    rot, qjl, cb = _d128_handles()
    n, nq = 230_000, 12
    rng = np.random.default_rng(11)
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    alpha = np.linspace(0.2, 3.0, n)[:, None]
    x = (alpha * u[None, :] + 0.3 * rng.standard_normal((n, 128))).astype(np.float32)
    q = (u[None, :] + 0.2 * rng.standard_normal((nq, 128))).astype(np.float32)
    p = tq.encode(torch.from_numpy(x).to(dev), 4, "prod", cb, rot, qjl)
    for k in (1, 10, 32):
        top_s, top_i = tq.search_topk(torch.from_numpy(q).to(dev), p, k, cb, rot, qjl)
        torch.cuda.synchronize()
        ref = _d128_ref(p, q)
        tol = 1e-3 * np.linalg.norm(q, axis=1) * np.max(p.norms.cpu().numpy())
        _check_topk(top_s.cpu().numpy(), top_i.cpu().numpy(), ref, k, tol)


def test_search_topk_equal_scores_across_chunks(dev):
    # Rows copied within a chunk and across chunks encode to the same bits and so score the same;
    # equal scores rank by the smaller index, and a copy in a later chunk that only equals the
    # running k-th result is not kept.  Query i gets its own strong row, copied three times: into
    # the next 512-vector block and into two later chunks (vectors 65536 and 131072 on lie in
    # different chunks whatever the first chunk's length, which is at most 65536).
    rot, qjl, cb = _d128_handles()
    n, nq = 140_000, 6
    x = wl.gaussian((n, 128), 21).astype(np.float32) * 0.05
    q = wl.gaussian((nq, 128), 22).astype(np.float32)
    copies = []
    for i in range(nq):
        src = 1000 + 7919 * i
        dst = [src + 600 + 3 * i,              # the next 512-vector block
               65536 + 123 * i + 5,
               131072 + 17 * i + 1]
        x[src] = 4.0 * q[i] / np.linalg.norm(q[i])
        for j in dst:
            x[j] = x[src]
        copies.append(sorted([src] + dst))
    p = tq.encode(torch.from_numpy(x).to(dev), 4, "prod", cb, rot, qjl)
    words, norms = to_np_words(p.idx), p.norms.cpu().numpy()
    for c in copies:
        assert all(np.array_equal(words[c[0]], words[j]) and norms[c[0]] == norms[j] for j in c[1:])
    ref = _d128_ref(p, q)
    for k in (1, 2, 3, 4, 5):
        top_s, top_i = tq.search_topk(torch.from_numpy(q).to(dev), p, k, cb, rot, qjl)
        torch.cuda.synchronize()
        gs, gi = top_s.cpu().numpy(), top_i.cpu().numpy()
        for i in range(nq):
            assert np.argmax(ref[i]) in copies[i]
            m = min(k, 4)
            assert gi[i, :m].tolist() == copies[i][:m], (k, i, gi[i].tolist(), copies[i])
            assert np.all(gs[i, :m] == gs[i, 0]), (k, i, gs[i].tolist())
            if k == 5:
                assert gi[i, 4] not in copies[i] and gs[i, 4] < gs[i, 0]


def test_search_errors(dev, handles):
    rot, qjl = handles
    cb = tq.codebook(D, 3)
    p = tq.encode(torch.from_numpy(_db(10)).to(dev), 4, "prod", cb, rot, qjl)
    q = torch.from_numpy(_queries(2)).to(dev)
    with pytest.raises(tq.TQError) as e:
        tq.search_topk(q, p, 33, cb, rot, qjl)
    assert e.value.status == 1
    pm = tq.encode(torch.from_numpy(_db(10)).to(dev), 3, "mse", cb, rot)
    with pytest.raises(tq.TQError) as e:
        tq.search_topk(q, pm, 10, cb, rot, qjl)
    assert e.value.status == 3
    with pytest.raises(tq.TQError) as e:
        tq.search_topk(q, p, 10, cb, rot, qjl, ws=torch.empty((16,), dtype=torch.uint8, device=dev))
    assert e.value.status == 4
