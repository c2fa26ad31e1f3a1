"""GPU parity of the outlier-channel split codes (two TurboQuant_mse codes per d = 128 key, the
outlier half at b_o bits, the other half at b_r bits) against the oracle, through the C ABI:
the encode (indices by the band rule, norms), the scores from the GPU's own codes and from
codes the oracle wrote, GQA ratios that are and are not multiples of 4, ragged token counts,
zero halves, errors, and seeded samples of the full-size key set."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _parity import check_indices, require_gpu, score_tolerance, to_np_words

pytestmark = pytest.mark.gpu

M = 64
R_O = oracle.dense_rotation(M, 3)
R_R = oracle.dense_rotation(M, 4)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def rots(dev):
    return tq.make_rotation(M, 3), tq.make_rotation(M, 4)


def _keys(B, H, T, seed=0):
    bits = wl.kv_tensor_bf16(B, H, T, 128, seed=seed, outlier_seed=10, scale_seed=11)
    x = wl.bf16_bits_to_f32(bits).astype(np.float64)
    return x, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def _outliers(x):
    """Per KV head, the 64 channels of largest mean square, largest first (a calibration rule of
    the tests; the library takes any list)."""
    ms = np.mean(x * x, axis=(0, 2))
    return np.argsort(-ms, axis=1, kind="stable")[:, :M].astype(np.int32)


def _check_codes(p, part, cb_o, label):
    gidx = oracle.unpack_bits(to_np_words(p.idx), M, cb_o.b)
    ref = part.y.reshape(-1, M)
    bad, _ = check_indices(gidx, ref, cb_o, label)
    np.testing.assert_array_equal(to_np_words(p.idx)[~bad], part.words.reshape(-1, part.words.shape[-1])[~bad])
    np.testing.assert_allclose(p.norms.cpu().numpy(), part.norms.reshape(-1), rtol=1e-6, atol=1e-30)
    return gidx


def _gpu_as_oracle(po, pr, B, H, T, order):
    """The GPU's codes as an oracle EncodedSplit, to score identical packed inputs."""
    mk = lambda p, b: oracle.EncodedMSE(idx=oracle.unpack_bits(to_np_words(p.idx), M, b).reshape(B, H, T, M),
                                        words=None, norms=p.norms.cpu().numpy().astype(np.float64).reshape(B, H, T),
                                        y=None)
    return oracle.EncodedSplit(order=order, outlier=mk(po, po.bits), rest=mk(pr, pr.bits))


@pytest.mark.parametrize("bo,br,dtype", [(3, 2, "bf16"), (4, 3, "bf16"), (2, 1, "bf16"), (4, 4, "f32"),
                                         (1, 4, "f32"), (3, 3, "bf16")])
def test_encode_split_matches_oracle(dev, rots, bo, br, dtype):
    B, H, T = 2, 2, 300                      # 300 tokens: one 512-token block of the MFMA kernel, ragged
    x, xt = _keys(B, H, T, seed=bo * 10 + br)
    if dtype == "f32":
        x = x * (1.0 + 1e-3 * wl.gaussian(x.shape, 9))   # values off the bf16 grid
        xt = torch.from_numpy(x.astype(np.float32))
        x = x.astype(np.float32).astype(np.float64)
    out = _outliers(x)
    sp = tq.make_split(out)
    cbo, cbr = tq.codebook(M, bo), tq.codebook(M, br)
    po, pr = tq.encode_split(xt.to(dev), sp, cbo, cbr, *rots)
    torch.cuda.synchronize()
    ocb_o, ocb_r = oracle.codebook(M, bo), oracle.codebook(M, br)
    enc = oracle.encode_split(x, out, R_O, R_R, ocb_o, ocb_r)
    _check_codes(po, enc.outlier, ocb_o, f"split outlier b={bo}")
    _check_codes(pr, enc.rest, ocb_r, f"split rest b={br}")


@pytest.mark.parametrize("bo,br", [(3, 2), (4, 3)])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (2, 2), (16, 2), (6, 2), (12, 3), (64, 1)])
def test_scores_split_matches_oracle(dev, rots, bo, br, hq, hkv):
    B, T = 2, 300
    x, xt = _keys(B, hkv, T, seed=3)
    out = _outliers(x)
    sp = tq.make_split(out)
    cbo, cbr = tq.codebook(M, bo), tq.codebook(M, br)
    K = tq.encode_split(xt.to(dev), sp, cbo, cbr, *rots)
    q = wl.gaussian((B, hq, 128), 21)
    s = tq.scores_split(torch.from_numpy(q).to(dev), K, hkv, sp, cbo, cbr, *rots)
    torch.cuda.synchronize()
    ocb_o, ocb_r = oracle.codebook(M, bo), oracle.codebook(M, br)
    enc = _gpu_as_oracle(K[0], K[1], B, hkv, T, oracle.channel_order(out, 128))
    ref = oracle.scores_split(q, enc, R_O, R_R, ocb_o, ocb_r)
    knorm = np.sqrt(enc.outlier.norms ** 2 + enc.rest.norms ** 2)           # [B, Hkv, T]
    ratio = hq // hkv
    for b in range(B):
        for h in range(hq):
            tol = score_tolerance(q[b, h][None], knorm[b, h // ratio])[0]
            assert np.all(np.abs(s[b, h].cpu().numpy() - ref[b, h]) <= tol), (b, h)


def test_scores_from_oracle_codes(dev, rots):
    # Codes the oracle wrote, uploaded as they are: the score kernel alone against the oracle.
    B, hkv, hq, T, bo, br = 1, 2, 8, 517, 4, 3
    x, _ = _keys(B, hkv, T, seed=7)
    out = _outliers(x)
    ocb_o, ocb_r = oracle.codebook(M, bo), oracle.codebook(M, br)
    enc = oracle.encode_split(x, out, R_O, R_R, ocb_o, ocb_r)
    up = lambda part, b: tq.Packed(M, b, "mse", B * hkv * T,
                                   torch.from_numpy(part.words.reshape(-1, 2 * b).view(np.int32)).to(dev),
                                   torch.from_numpy(part.norms.reshape(-1).astype(np.float32)).to(dev))
    K = (up(enc.outlier, bo), up(enc.rest, br))
    enc32 = oracle.EncodedSplit(order=enc.order, outlier=oracle.EncodedMSE(
        idx=enc.outlier.idx, words=None, norms=enc.outlier.norms.astype(np.float32).astype(np.float64), y=None),
        rest=oracle.EncodedMSE(idx=enc.rest.idx, words=None,
                               norms=enc.rest.norms.astype(np.float32).astype(np.float64), y=None))
    q = wl.gaussian((B, hq, 128), 22)
    s = tq.scores_split(torch.from_numpy(q).to(dev), K, hkv, tq.make_split(out), tq.codebook(M, bo),
                        tq.codebook(M, br), *rots)
    torch.cuda.synchronize()
    ref = oracle.scores_split(q, enc32, R_O, R_R, ocb_o, ocb_r)
    knorm = np.linalg.norm(x, axis=-1)
    for h in range(hq):
        tol = score_tolerance(q[0, h][None], knorm[0, h // 4])[0]
        assert np.all(np.abs(s[0, h].cpu().numpy() - ref[0, h]) <= tol), h


def test_zero_halves_and_empty(dev, rots):
    B, H, T, bo, br = 1, 1, 130, 3, 2
    x, _ = _keys(B, H, T, seed=5)
    out = _outliers(x)
    x[0, 0, 3] = 0.0                          # a zero key
    x[0, 0, 129][out[0]] = 0.0                # a key whose outlier half is zero
    xt = torch.from_numpy(x.astype(np.float32))
    sp = tq.make_split(out)
    po, pr = tq.encode_split(xt.to(dev), sp, tq.codebook(M, bo), tq.codebook(M, br), *rots)
    torch.cuda.synchronize()
    io = oracle.unpack_bits(to_np_words(po.idx), M, bo)
    ir = oracle.unpack_bits(to_np_words(pr.idx), M, br)
    assert np.all(io[3] == 1 << (bo - 1)) and np.all(ir[3] == 1 << (br - 1))
    assert np.all(io[129] == 1 << (bo - 1))
    assert po.norms[3].item() == 0.0 and pr.norms[3].item() == 0.0 and po.norms[129].item() == 0.0
    enc = oracle.encode_split(x, out, R_O, R_R, oracle.codebook(M, bo), oracle.codebook(M, br))
    _check_codes(pr, enc.rest, oracle.codebook(M, br), "rest with zero halves")
    # empty token range: nothing to do, success
    e = tq.encode_split(torch.empty((1, 1, 0, 128), dtype=torch.bfloat16, device=dev), sp, tq.codebook(M, bo),
                        tq.codebook(M, br), *rots)
    s = tq.scores_split(torch.zeros((1, 4, 128), device=dev), e, 1, sp, tq.codebook(M, bo), tq.codebook(M, br), *rots)
    assert s.shape == (1, 4, 0)


def test_split_errors(dev, rots):
    x, xt = _keys(1, 2, 64)
    sp = tq.make_split(_outliers(x))
    cbo, cbr = tq.codebook(M, 3), tq.codebook(M, 2)
    po, pr = tq.encode_split(xt.to(dev), sp, cbo, cbr, *rots)
    with pytest.raises(tq.TQError) as e:            # split for 2 heads, keys with 1
        tq.encode_split(xt[:, :1].contiguous().to(dev), sp, cbo, cbr, *rots)
    assert e.value.status == 2
    with pytest.raises(tq.TQError) as e:            # codebook of the wrong dimension
        tq.encode_split(xt.to(dev), sp, tq.codebook(128, 3), cbr, *rots)
    assert e.value.status == 2
    with pytest.raises(tq.TQError) as e:            # bits of the packed set and the codebook differ
        tq.scores_split(torch.zeros((1, 8, 128), device=dev), (po, pr), 2, sp, tq.codebook(M, 4), cbr, *rots)
    assert e.value.status == 2
    with pytest.raises(tq.TQError) as e:            # GQA ratio above the 64 the score kernel takes
        tq.scores_split(torch.zeros((1, 130, 128), device=dev), (po, pr), 2, sp, cbo, cbr, *rots)
    assert e.value.status == 3
    ws = torch.empty((16,), dtype=torch.uint8, device=dev)
    with pytest.raises(tq.TQError) as e:            # workspace too small
        tq.scores_split(torch.zeros((1, 8, 128), device=dev), (po, pr), 2, sp, cbo, cbr, *rots, ws=ws)
    assert e.value.status == 4


def test_split_full_size_sampled(dev, rots):
    # The KV-key workload at full size (1 x 8 KV heads x 32768 tokens, 32 query heads) at 2.5 bits:
    # 4096 sampled keys' codes and 4096 sampled scores against the oracle.
    cfg = wl.CONFIGS["c2"]
    bits = wl.kv_keys(cfg)
    x_all = wl.bf16_bits_to_f32(bits)
    out = _outliers(x_all[:, :, :4096].astype(np.float64))
    sp = tq.make_split(out)
    bo, br = 3, 2
    cbo, cbr = tq.codebook(M, bo), tq.codebook(M, br)
    xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    K = tq.encode_split(xt, sp, cbo, cbr, *rots)
    q = wl.kv_queries(cfg)
    s = tq.scores_split(torch.from_numpy(q).to(dev), K, cfg.hkv, sp, cbo, cbr, *rots)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = np.sort(rng.choice(cfg.B * cfg.hkv * cfg.T, 4096, replace=False))
    hh, tt = (rows // cfg.T) % cfg.hkv, rows % cfg.T
    ocb_o, ocb_r = oracle.codebook(M, bo), oracle.codebook(M, br)
    for h in range(cfg.hkv):
        sel = rows[hh == h]
        xs = x_all[0, h, tt[hh == h]].astype(np.float64)[None, None]
        enc = oracle.encode_split(xs, out[h:h + 1], R_O, R_R, ocb_o, ocb_r)
        for p, part, cb in ((K[0], enc.outlier, ocb_o), (K[1], enc.rest, ocb_r)):
            gw = to_np_words(p.idx)[sel]
            gidx = oracle.unpack_bits(gw, M, cb.b)
            bad, _ = check_indices(gidx, part.y.reshape(-1, M), cb, f"full-size split head {h}")
            np.testing.assert_array_equal(gw[~bad], part.words.reshape(-1, gw.shape[1])[~bad])
            np.testing.assert_allclose(p.norms.cpu().numpy()[sel], part.norms.reshape(-1), rtol=1e-6)
    # sampled scores on the GPU's own codes
    order = oracle.channel_order(out, 128)
    io = oracle.unpack_bits(to_np_words(K[0].idx), M, bo)
    ir = oracle.unpack_bits(to_np_words(K[1].idx), M, br)
    no, nr = K[0].norms.cpu().numpy().astype(np.float64), K[1].norms.cpu().numpy().astype(np.float64)
    sg = s.cpu().numpy()
    ratio = cfg.hq // cfg.hkv
    pick = rng.choice(cfg.hq * cfg.T, 4096, replace=False)
    for k in pick:
        h, t = divmod(int(k), cfg.T)
        hk = h // ratio
        r = hk * cfg.T + t
        qo = R_O @ q[0, h][order[hk, :M]]
        qr = R_R @ q[0, h][order[hk, M:]]
        ref = no[r] * qo @ ocb_o.centroids[io[r]] + nr[r] * qr @ ocb_r.centroids[ir[r]]
        tol = 1e-3 * np.linalg.norm(q[0, h]) * np.hypot(no[r], nr[r])
        assert abs(sg[0, h, t] - ref) <= tol, (h, t)


def test_split_cache_appends_and_scores(dev, rots):
    # Split codes as a streaming key cache: seeded garbage, then appends of 37, 1, 100 and 1 tokens
    # at increasing positions ("TurboQuant 详解", KV-cache example: prefill, then one token per
    # decode step).  Every appended row matches the oracle's encode of that token; every other
    # row keeps its garbage; scores over the written prefix match the oracle on the cache's codes.
    B, H, T_CAP, bo, br = 2, 2, 160, 3, 2
    plan = [(0, 37), (37, 1), (38, 100), (138, 1)]
    written = 139
    x, _ = _keys(B, H, T_CAP, seed=13)
    out = _outliers(x)
    sp = tq.make_split(out)
    cbo, cbr = tq.codebook(M, bo), tq.codebook(M, br)
    K = tq.alloc_split_cache(B, H, T_CAP, bo, br, device=dev)
    rng = np.random.default_rng(14)
    garbage = []
    for p in K:
        g = rng.integers(-2**31, 2**31, size=tuple(p.idx.shape), dtype=np.int64).astype(np.int32)
        p.idx.copy_(torch.from_numpy(g))
        p.norms.copy_(torch.from_numpy(rng.standard_normal(p.n).astype(np.float32)))
        garbage.append((g.view(np.uint32).copy(), p.norms.cpu().numpy().copy()))
    xb = torch.from_numpy(wl.f32_to_bf16_bits(x.astype(np.float32)).view(np.int16)).view(torch.bfloat16)
    x = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)
    for pos, n_new in plan:
        tq.cache_append_split(K, xb[:, :, pos:pos + n_new].contiguous().to(dev), pos, T_CAP, sp, cbo, cbr, *rots)
    q = wl.gaussian((B, 8, 128), 23)
    s = tq.scores_split_cache(torch.from_numpy(q).to(dev), K, H, written, T_CAP, sp, cbo, cbr, *rots)
    torch.cuda.synchronize()
    rows = (np.arange(B * H)[:, None] * T_CAP + np.arange(written)[None, :]).reshape(-1)
    untouched = np.setdiff1d(np.arange(B * H * T_CAP), rows)
    ocb = (oracle.codebook(M, bo), oracle.codebook(M, br))
    enc = oracle.encode_split(x[:, :, :written], out, R_O, R_R, *ocb)
    for p, part, cb, (gw, gn) in zip(K, (enc.outlier, enc.rest), ocb, garbage):
        words = to_np_words(p.idx)
        gidx = oracle.unpack_bits(words[rows], M, cb.b)
        bad, _ = check_indices(gidx, part.y.reshape(-1, M), cb, "split cache")
        np.testing.assert_array_equal(words[rows][~bad], part.words.reshape(-1, 2 * cb.b)[~bad])
        np.testing.assert_allclose(p.norms.cpu().numpy()[rows], part.norms.reshape(-1), rtol=1e-6)
        np.testing.assert_array_equal(words[untouched], gw[untouched])
        np.testing.assert_array_equal(p.norms.cpu().numpy()[untouched], gn[untouched])
    # scores over the prefix, on the cache's own codes
    mk = lambda p, b: oracle.EncodedMSE(
        idx=oracle.unpack_bits(to_np_words(p.idx)[rows], M, b).reshape(B, H, written, M), words=None,
        norms=p.norms.cpu().numpy().astype(np.float64)[rows].reshape(B, H, written), y=None)
    encg = oracle.EncodedSplit(order=oracle.channel_order(out, 128), outlier=mk(K[0], bo), rest=mk(K[1], br))
    ref = oracle.scores_split(q, encg, R_O, R_R, *ocb)
    knorm = np.sqrt(encg.outlier.norms ** 2 + encg.rest.norms ** 2)
    for b in range(B):
        for h in range(8):
            tol = score_tolerance(q[b, h][None], knorm[b, h // 4])[0]
            assert np.all(np.abs(s[b, h].cpu().numpy() - ref[b, h]) <= tol), (b, h)
    # errors: past the capacity, prefix longer than the capacity
    with pytest.raises(tq.TQError) as e:
        tq.cache_append_split(K, xb[:, :, :30].contiguous().to(dev), 140, T_CAP, sp, cbo, cbr, *rots)
    assert e.value.status == 1
    with pytest.raises(tq.TQError) as e:
        tq.scores_split_cache(torch.from_numpy(q).to(dev), K, H, T_CAP + 1, T_CAP, sp, cbo, cbr, *rots)
    assert e.value.status == 1


@pytest.mark.parametrize("bo,br", [(2, 1), (1, 4), (3, 2), (4, 3)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [9, 32, 33])
def test_short_encode_per_token_path(dev, rots, dtype, bo, br, T):
    # At most 32 tokens per sequence take the one-block-per-token kernel, 33 the MFMA kernel: the
    # codes against the oracle on both sides of the switch, with a zero key and a key whose outlier
    # half is zero among them.
    B, H = 2, 3
    x, _ = _keys(B, H, T, seed=17 + T)
    out = _outliers(x)
    x[1, 2, 4] = 0.0
    x[0, 1, 7][out[1]] = 0.0
    if dtype == "f32":
        x = x * (1.0 + 1e-3 * wl.gaussian(x.shape, 19))
        xt = torch.from_numpy(x.astype(np.float32))
        x = x.astype(np.float32).astype(np.float64)
    else:
        xt = torch.from_numpy(wl.f32_to_bf16_bits(x.astype(np.float32)).view(np.int16)).view(torch.bfloat16)
    sp = tq.make_split(out)
    po, pr = tq.encode_split(xt.to(dev), sp, tq.codebook(M, bo), tq.codebook(M, br), *rots)
    torch.cuda.synchronize()
    ocb_o, ocb_r = oracle.codebook(M, bo), oracle.codebook(M, br)
    enc = oracle.encode_split(x, out, R_O, R_R, ocb_o, ocb_r)
    _check_codes(po, enc.outlier, ocb_o, f"per-token outlier {dtype}")
    _check_codes(pr, enc.rest, ocb_r, f"per-token rest {dtype}")
    io = oracle.unpack_bits(to_np_words(po.idx), M, bo)
    zero_row = (1 * H + 2) * T + 4
    assert np.all(io[zero_row] == 1 << (bo - 1)) and po.norms[zero_row].item() == 0.0
    assert np.all(io[(0 * H + 1) * T + 7] == 1 << (bo - 1))


@pytest.mark.parametrize("bo,br,vb,hq,hkv,T", [(3, 2, 2, 8, 2, 300), (4, 3, 3, 4, 2, 77), (3, 2, 4, 2, 2, 33),
                                               (4, 3, 2, 4, 1, 1), (3, 2, 3, 4, 2, 1000)])
def test_decode_attn_split_matches_oracle(dev, rots, bo, br, vb, hq, hkv, T):
    # split keys inside decode attention, against the oracle on the GPU's own codes; T = 77 with
    # two sequences per batch puts sequences that start in the second half of a 32-token block
    B = 2
    x, xt = _keys(B, hkv, T, seed=bo * 10 + vb)
    out = _outliers(x)
    sp = tq.make_split(out)
    cbo, cbr, cbv = tq.codebook(M, bo), tq.codebook(M, br), tq.codebook(128, vb)
    rot_v = tq.make_rotation(128, 1)
    K = tq.encode_split(xt.to(dev), sp, cbo, cbr, *rots)
    vbits = wl.kv_tensor_bf16(B, hkv, T, 128, seed=33, outlier_seed=21, scale_seed=None)
    vt = torch.from_numpy(vbits.view(np.int16)).view(torch.bfloat16).reshape(-1, 128).to(dev)
    V = tq.encode(vt, vb, "mse", cbv, rot_v, layout="blocked")
    q = wl.gaussian((B, hq, 128), 44)
    got = tq.decode_attn_split(torch.from_numpy(q).to(dev), K, V, hkv, sp, cbo, cbr, cbv, *rots, rot_v).cpu().numpy()
    torch.cuda.synchronize()
    n = B * hkv * T
    enc = _gpu_as_oracle(K[0], K[1], B, hkv, T, oracle.channel_order(out, 128))
    R_V = oracle.dense_rotation(128, 1)
    ocbv = oracle.codebook(128, vb)
    vidx = oracle.unpack_token_blocked(to_np_words(V.idx), n, 128, vb).reshape(B, hkv, T, 128)
    vn = V.norms.cpu().numpy().astype(np.float64).reshape(B, hkv, T)
    ref = oracle.decode_attention_split(q, enc, vidx, vn, R_O, R_R, R_V, oracle.codebook(M, bo), oracle.codebook(M, br),
                                        ocbv, 1 / np.sqrt(128))
    ratio = hq // hkv
    for b in range(B):
        for g in range(hkv):
            vmax = np.max(np.linalg.norm(oracle.decode_mse(vidx[b, g], vn[b, g], R_V, ocbv), axis=1))
            err = np.max(np.abs(got[b, g * ratio:(g + 1) * ratio] - ref[b, g * ratio:(g + 1) * ratio]))
            assert err <= 1e-3 * vmax, (b, g, err, vmax)


def test_decode_attn_split_errors(dev, rots):
    x, xt = _keys(1, 2, 32, seed=1)
    sp = tq.make_split(_outliers(x))
    cbv, rot_v = tq.codebook(128, 2), tq.make_rotation(128, 1)
    V = tq.encode(xt.reshape(-1, 128).to(dev), 2, "mse", cbv, rot_v, layout="blocked")
    K = tq.encode_split(xt.to(dev), sp, tq.codebook(M, 2), tq.codebook(M, 2), *rots)
    with pytest.raises(tq.TQError) as e:       # (2, 2) halves: no kernel
        tq.decode_attn_split(torch.zeros((1, 4, 128), device=dev), K, V, 2, sp, tq.codebook(M, 2), tq.codebook(M, 2),
                             cbv, *rots, rot_v)
    assert e.value.status == 3
    K = tq.encode_split(xt.to(dev), sp, tq.codebook(M, 3), tq.codebook(M, 2), *rots)
    with pytest.raises(tq.TQError) as e:       # GQA ratio 3
        tq.decode_attn_split(torch.zeros((1, 6, 128), device=dev), K, V, 2, sp, tq.codebook(M, 3), tq.codebook(M, 2),
                             cbv, *rots, rot_v)
    assert e.value.status == 3
