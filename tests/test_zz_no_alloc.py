"""The allocation-free score entry point (tq_scores_noalloc), through the C ABI: its scores equal
those of tq_scores with a caller workspace on the same inputs, bit for bit (the same kernels run
on the same operands), on two calls in a row where the second is smaller than the first (so the
static scratch still holds the first call's contents), for MSE and TurboQuant_prod keys.  Also
checked against the oracle's scores of the GPU's own packed keys, and the size limit."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _parity import require_gpu, score_tolerance, to_np_words, unpack_z

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _keys(B, hkv, T, seed):
    bits = wl.kv_tensor_bf16(B, hkv, T, D, seed=seed, outlier_seed=10, scale_seed=11)
    return torch.from_numpy(bits.reshape(-1, D).view(np.int16)).view(torch.bfloat16)


def _oracle_scores(q, p, B, hkv, T, mode, cb_o, rmat, smat):
    idx = oracle.unpack_bits(to_np_words(p.idx), D, p.bits)
    norms = p.norms.cpu().numpy().astype(np.float64)
    ratio = q.shape[1] // hkv
    out = np.empty((B, q.shape[1], T))
    tol = np.empty_like(out)
    for b in range(B):
        for g in range(hkv):
            r0, r1 = (b * hkv + g) * T, (b * hkv + g + 1) * T
            heads = q[b, g * ratio:(g + 1) * ratio].astype(np.float64)
            if mode == "mse":
                ref = oracle.scores_mse(heads, idx[r0:r1], norms[r0:r1], rmat, cb_o)
            else:
                enc = oracle.EncodedProd(
                    mse=oracle.EncodedMSE(idx=idx[r0:r1], words=None, norms=norms[r0:r1], y=None),
                    z=unpack_z(to_np_words(p.qjl), D)[r0:r1], qjl_words=None,
                    gamma=p.rnorms.cpu().numpy().astype(np.float64)[r0:r1], proj=None)
                ref = oracle.scores_prod(heads, enc, rmat, cb_o, smat)
            out[b, g * ratio:(g + 1) * ratio] = ref
            tol[b, g * ratio:(g + 1) * ratio] = score_tolerance(heads, norms[r0:r1])
    return out, tol


@pytest.mark.parametrize("mode", ["mse", "prod"])
def test_noalloc_scores_match_workspace_entry_point(dev, mode):
    rot = tq.make_rotation(D, 1, "dense")
    qjl = tq.make_qjl(D, 2, rot) if mode == "prod" else None
    b_stage = 3
    cb = tq.codebook(D, b_stage)
    total = b_stage + (1 if mode == "prod" else 0)
    rmat = oracle.dense_rotation(D, 1)
    smat = oracle.qjl_matrix(D, 2)
    cb_o = oracle.codebook(D, b_stage)
    # first call: 3 sequences x 8 query heads (GQA 4) x 700 tokens; second: 1 x 4 (GQA 2) x 333
    for call, (B, hkv, hq, T) in enumerate([(3, 2, 8, 700), (1, 2, 4, 333)]):
        x = _keys(B, hkv, T, seed=40 + call).to(dev)
        p = tq.encode(x, total, mode, cb, rot, qjl)
        q = torch.from_numpy(wl.gaussian((B, hq, D), 50 + call)).to(dev)
        ref = tq.scores(q, p, hkv, cb, rot, qjl)
        got = tq.scores_noalloc(q, p, hkv, cb, rot, qjl)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {call}: scores differ from tq_scores"
        want, tol = _oracle_scores(q.cpu().numpy(), p, B, hkv, T, mode, cb_o, rmat, smat)
        err = np.abs(got.cpu().numpy() - want)
        assert np.all(err <= tol), f"call {call}: max err/tol {float((err / tol).max()):.3g}"


def test_noalloc_rejects_more_heads_than_the_scratch_holds(dev):
    lib = tq.lib()
    cap = int(lib.tq_scores_noalloc_max_bytes())
    assert cap == 4 << 20
    rot = tq.make_rotation(D, 1, "dense")
    cb = tq.codebook(D, 3)
    B, hkv, hq, T = 2, 64, 2048, 1      # 4096 query heads (GQA 32) need more than 4 MiB
    p = tq.alloc_packed(B * hkv * T, D, 3, "mse", device=dev)
    q = torch.zeros((B, hq, D), device=dev)
    with pytest.raises(tq.TQError) as e:
        tq.scores_noalloc(q, p, hkv, cb, rot)
    assert e.value.status == 4
    # 3072 query heads (3 sequences x 16 KV heads x GQA 64) fit in the scratch and run
    B, hkv, hq, T = 3, 16, 1024, 40
    assert tq.scores_workspace(B, hq, D) <= cap
    x = _keys(B, hkv, T, seed=7).to(dev)
    p = tq.encode(x, 3, "mse", cb, rot)
    q = torch.from_numpy(wl.gaussian((B, hq, D), 8)).to(dev)
    ref = tq.scores(q, p, hkv, cb, rot)
    got = tq.scores_noalloc(q, p, hkv, cb, rot)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
