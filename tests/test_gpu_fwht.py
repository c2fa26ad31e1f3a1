"""GPU parity of the d = 128 MSE encode with the randomized Hadamard rotations, which runs as a fast
Walsh-Hadamard transform in registers (butterflies, quad exchanges), against the oracle's explicit
matrices (1/sqrt(d)) H diag(sigma) and the block form with groups of 32:

* indices by the band rule (flips only next to a threshold, to the adjacent index), words bit for
  bit on the rows without a flip, norms to rtol 1e-6;
* bits 1..4, bf16 and fp32 inputs, several seeds (so sigma differs);
* ragged vector counts against the 64-vector blocks (1, 63, 65, 1000 + 3), a zero vector (index
  K/2 everywhere, norm 0), a vector with one non-zero coordinate, and tiny and huge scales."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_turboquant_amd as tq
from kv_cache_compression_turboquant_amd import workloads as wl
from _parity import check_indices, require_gpu, to_np_words

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _oracle_rot(kind, seed):
    return oracle.wht_rotation(128, seed) if kind == "wht" else oracle.block_wht_rotation(128, seed, 32)


def _inputs(n, dtype, seed):
    x = wl.gaussian((n, 128), seed) * np.float32(2.5)
    x[::7] *= np.float32(1e-3)
    if n > 3:
        x[1] = 0.0                       # zero vector
        x[2] = 0.0
        x[2, 77] = -4.0                  # one non-zero coordinate
    if n > 5:
        x[5] *= np.float32(1e15)
    if dtype == "bf16":
        bits = wl.f32_to_bf16_bits(x)
        return wl.bf16_bits_to_f32(bits).astype(np.float64), torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    return x.astype(np.float64), torch.from_numpy(x)


def _check(p, x, kind, seed, b, label):
    cb_o = oracle.codebook(128, b)
    enc = oracle.encode_mse(x, _oracle_rot(kind, seed), cb_o)
    words = to_np_words(p.idx)
    gidx = oracle.unpack_bits(words, 128, b)
    bad, _ = check_indices(gidx, enc.y, cb_o, label)
    np.testing.assert_array_equal(words[~bad], enc.words[~bad])
    np.testing.assert_allclose(p.norms.cpu().numpy(), enc.norms, rtol=1e-6, atol=0)
    return gidx


@pytest.mark.parametrize("kind", ["wht", "block_wht"])
@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwht_encode_matches_oracle(dev, kind, b, dtype):
    seed = 3 + b
    rot = tq.make_rotation(128, seed, kind)
    x, xt = _inputs(1000 + 3, dtype, seed=10 * b + (dtype == "f32"))
    p = tq.encode(xt.to(dev), b, "mse", tq.codebook(128, b), rot)
    torch.cuda.synchronize()
    gidx = _check(p, x, kind, seed, b, f"fwht {kind} b={b} {dtype}")
    assert np.all(gidx[1] == 1 << (b - 1)) and float(p.norms[1]) == 0.0


@pytest.mark.parametrize("n", [1, 63, 65])
def test_fwht_encode_ragged_counts(dev, n):
    rot = tq.make_rotation(128, 11, "wht")
    x, xt = _inputs(n, "bf16", seed=n)
    p = tq.encode(xt.to(dev), 3, "mse", tq.codebook(128, 3), rot)
    torch.cuda.synchronize()
    _check(p, x, "wht", 11, 3, f"fwht n={n}")


def test_fwht_encode_writes_only_its_rows(dev):
    # the packed buffer past n keeps its contents (rows are written by the quad that owns them)
    rot = tq.make_rotation(128, 2, "block_wht")
    x, xt = _inputs(70, "f32", seed=4)
    p = tq.alloc_packed(80, 128, 2, "mse", device=dev)
    p.idx.fill_(-1)
    p.norms.fill_(7.0)
    q = tq.Packed(128, 2, "mse", 70, p.idx[:70], p.norms[:70])
    tq.encode(xt.to(dev), 2, "mse", tq.codebook(128, 2), rot, out=q)
    torch.cuda.synchronize()
    assert torch.all(p.idx[70:] == -1) and torch.all(p.norms[70:] == 7.0)
    _check(q, x, "block_wht", 2, 2, "fwht rows")
