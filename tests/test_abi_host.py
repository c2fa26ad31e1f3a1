"""CPU tests of the C-ABI library: it loads, exports every symbol include/tq.h declares, and its
host-side math (generator, QR rotation, Lloyd-Max codebook, QJL matrix) agrees with the oracle.
No kernel is launched here."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")


@pytest.fixture(scope="module")
def tq():
    import kv_cache_compression_turboquant_amd as tq
    from kv_cache_compression_turboquant_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        pytest.fail("libtq.so is not built: run `python -m kv_cache_compression_turboquant_amd.build`")
    return tq


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(tq):
    from kv_cache_compression_turboquant_amd import _binding
    raw = ctypes.CDLL(_binding.LIB_PATH)
    names = _declared_functions()
    assert len(names) >= 20
    for name in names:
        assert hasattr(raw, name), name
        assert name in _binding.SIGNATURES, f"binding lacks {name}"
    assert tq.lib().tq_abi_version() == 7


def test_splitmix_bit_identical(tq):
    for seed in (0, 1, 2, 12345, 2 ** 64 - 1):
        np.testing.assert_array_equal(tq.host_splitmix64(seed, 1000, offset=7),
                                      oracle.splitmix64(seed, 1000, offset=7))


def test_gaussian_stream(tq):
    g = tq.host_gaussian(1, 200000)
    np.testing.assert_allclose(g, oracle.gaussian(1, 200000), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("d", [3, 64, 128, 1536])
@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_codebook_matches_oracle(tq, d, b):
    c, t = tq.host_codebook(d, b)
    cb = oracle.codebook(d, b)
    np.testing.assert_allclose(c, cb.centroids, rtol=0, atol=1e-12)
    np.testing.assert_allclose(t, cb.thresholds, rtol=0, atol=1e-12)
    # the float32 thresholds the kernels compare against are identical
    np.testing.assert_array_equal(t.astype(np.float32), cb.thresholds32)
    g, _ = tq.host_codebook(d, b, "gauss")
    np.testing.assert_allclose(g, oracle.codebook(d, b, "gauss").centroids, atol=1e-12)


def test_codebook_handle_host_only(tq):
    cb = tq.codebook(128, 3)
    c, t = cb.values()
    np.testing.assert_allclose(c, oracle.codebook(128, 3).centroids, atol=1e-12)
    cb.close()


@pytest.mark.parametrize("d", [2, 16, 128, 256])
def test_dense_rotation_matches_oracle(tq, d):
    r = tq.host_rotation(d, 1)
    np.testing.assert_allclose(r, oracle.dense_rotation(d, 1), rtol=0, atol=1e-12)


def test_dense_rotation_d1536(tq):
    r = tq.host_rotation(1536, 1)
    np.testing.assert_allclose(r, oracle.dense_rotation(1536, 1), rtol=0, atol=1e-12)


def test_wht_rotation_matches_oracle(tq):
    for d in (2, 64, 128):
        np.testing.assert_array_equal(tq.host_rotation(d, 1, "wht"), oracle.wht_rotation(d, 1))


def test_block_wht_rotation_matches_oracle(tq):
    for d in (32, 96, 128, 1536):
        np.testing.assert_array_equal(tq.host_rotation(d, 3, "block_wht"), oracle.block_wht_rotation(d, 3, 32))
    with pytest.raises(tq.TQError):
        tq.host_rotation(100, 1, "block_wht")


def test_qjl_matrix(tq):
    np.testing.assert_allclose(tq.host_qjl_matrix(128, 2), oracle.qjl_matrix(128, 2), rtol=1e-14, atol=1e-14)


def test_error_paths(tq):
    lib = tq.lib()
    c = np.empty(32)
    t = np.empty(32)
    P = lambda a: ctypes.c_void_p(a.ctypes.data)
    assert lib.tq_host_codebook(128, 5, 0, P(c), P(t)) == 1          # b out of range
    assert lib.tq_host_codebook(128, 0, 0, P(c), P(t)) == 1
    assert lib.tq_host_codebook(128, 2, 7, P(c), P(t)) == 1          # bad density
    assert lib.tq_host_codebook(128, 2, 0, None, P(t)) == 1
    r = np.empty(96 * 96)
    assert lib.tq_host_rotation(96, 1, 1, P(r)) == 3                 # Hadamard needs 2^k
    assert "Hadamard" in lib.tq_last_error().decode()
    assert lib.tq_host_splitmix64(0, 0, -1, None) == 1
    assert lib.tq_packed_words(128, 3) == 12 and lib.tq_packed_words(100, 3) == 0
    # hot-path entry points validate before touching the device
    desc = tq.tq_packed(128, 3, 0, 0, 10, None, None, None, None)
    assert lib.tq_encode(None, 1, 10, 128, 3, 0, None, None, None, ctypes.byref(desc), None, 0, None) == 1
    cbh = tq.codebook(128, 2)
    assert lib.tq_encode(None, 1, 10, 128, 3, 0, cbh.ptr, None, None, ctypes.byref(desc), None, 0, None) == 1
    # search validates its handles and k before anything else
    assert lib.tq_search_topk(None, 4, ctypes.byref(desc), None, None, None, 10, None, None, None, 0, None) == 1
    assert lib.tq_scores(None, 1, 32, 5, 10, ctypes.byref(desc), cbh.ptr, None, None, None, None, 0, None) == 1
    assert lib.tq_quantize_rotated(None, 10, 64, cbh.ptr, None, None) == 1   # null buffers
    assert lib.tq_quantize_rotated(None, -1, 128, cbh.ptr, None, None) == 1
    assert lib.tq_quantize_rotated(None, 0, 64, cbh.ptr, None, None) == 2    # d mismatch
    assert lib.tq_quantize_rotated(None, 0, 128, cbh.ptr, None, None) == 0   # empty is fine


def test_codebook_from_values_checks(tq):
    with pytest.raises(tq.TQError):
        tq.codebook_from_values(4, [0.5, -0.5])
    cb = tq.codebook_from_values(4, [-0.6, 0.6])
    c, t = cb.values()
    assert t.tolist() == [0.0]


def test_workspace_sizes(tq):
    lib = tq.lib()
    # encode: only prod away from d = 128 stages residual rows (d + d/128 floats per vector)
    assert lib.tq_encode_workspace(1000, 128, 4, 1) == 0
    assert lib.tq_encode_workspace(1000, 1536, 4, 0) == 0
    assert lib.tq_encode_workspace(1000, 1536, 4, 1) == 1000 * (1536 + 12) * 4
    assert lib.tq_encode_workspace(10 ** 6, 1536, 4, 1) == 131072 * (1536 + 12) * 4
    assert lib.tq_encode_workspace(0, 1536, 4, 1) == 0
    # search: rejected shapes report 0; the score chunk dominates at large n
    assert lib.tq_search_workspace(1024, 10 ** 6, 1536, 0) == 0
    assert lib.tq_search_workspace(1024, 10 ** 6, 1536, 33) == 0
    assert lib.tq_search_workspace(1024, 10 ** 6, 1000, 10) == 0
    big = lib.tq_search_workspace(1024, 10 ** 6, 1536, 10)
    assert big >= 1024 * 65536 * 4 + 2 * 1024 * 1536 * 4
    assert lib.tq_search_workspace(1024, 100, 1536, 10) < big


def test_split_score_entry_points_validate(tq):
    """The query-prologue and prepared-score entry points reject bad shapes before any launch."""
    lib = tq.lib()
    cbh = tq.codebook(128, 3)
    desc = tq.tq_packed(128, 3, 0, 0, 10, None, None, None, None)
    # null rotation / handles
    assert lib.tq_prepare_queries(None, 1, 32, 8, None, None, None, 0, None) == 1
    assert lib.tq_scores_prepared(None, 0, 1, 32, 8, 10, None, cbh.ptr, None, None) == 1
    # Hq not a multiple of Hkv; GQA ratio 6 unsupported
    assert lib.tq_scores_prepared(None, 0, 1, 30, 8, 10, ctypes.byref(desc), cbh.ptr, None, None) == 2
    assert lib.tq_scores_prepared(None, 0, 1, 48, 8, 10, ctypes.byref(desc), cbh.ptr, None, None) == 3
    # a descriptor of 10 keys without buffers is rejected before its shape is looked at
    assert lib.tq_scores_prepared(None, 0, 1, 32, 8, 10, ctypes.byref(desc), cbh.ptr, None, None) == 1
    # empty work is fine without buffers
    empty = tq.tq_packed(128, 3, 0, 0, 0, None, None, None, None)
    assert lib.tq_scores_prepared(None, 0, 0, 32, 8, 0, ctypes.byref(empty), cbh.ptr, None, None) == 0


def test_search_entry_point_validates(tq):
    lib = tq.lib()
    cbh = tq.codebook(128, 3)
    mse = tq.tq_packed(128, 3, 0, 0, 10, None, None, None, None)
    # handles first, then k range
    assert lib.tq_search_topk(None, 4, ctypes.byref(mse), cbh.ptr, None, None, 10, None, None, None, 0, None) == 1


def test_timer_entry_points(tq):
    lib = tq.lib()
    ms = ctypes.c_float()
    lib.tq_timer_reset()
    # ids never armed, or out of range, are rejected
    assert lib.tq_timer_read(0, ctypes.byref(ms)) == 1
    assert lib.tq_timer_read(-1, ctypes.byref(ms)) == 1
    assert lib.tq_timer_read(256, ctypes.byref(ms)) == 1
    assert lib.tq_timer_read(0, None) == 1
    # without a device no events can be created: arming fails cleanly
    t = lib.tq_timer_arm()
    assert t == -1 or 0 <= t < 256
    assert lib.tq_timer_arm_kernel(7) == -1          # unknown kernel kind
    assert b"unknown kernel kind" in lib.tq_last_error()
    lib.tq_timer_reset()


def test_peak_entry_points_validate(tq):
    """The measurement-ceiling kernels reject bad arguments before any launch."""
    lib = tq.lib()
    dummy = ctypes.c_void_p(16)
    assert lib.tq_peak_read(None, 1024, 4, None, None) == 1
    assert lib.tq_peak_read(dummy, 1000, 4, None, None) == 1      # not a multiple of 16
    assert lib.tq_peak_read(dummy, 1024, 0, None, None) == 1
    assert lib.tq_peak_copy(dummy, None, 1024, 4, None) == 1
    assert lib.tq_peak_copy(dummy, dummy, 0, 4, None) == 1
    assert lib.tq_peak_mfma(4, 10, 4, dummy, None) == 1           # unknown kind
    assert lib.tq_peak_mfma(0, 0, 4, dummy, None) == 1
    assert lib.tq_peak_mfma(0, 10, 4, None, None) == 1


def test_cache_entry_points_validate(tq):
    """The streaming-cache entry points reject missing handles and descriptors before any launch."""
    lib = tq.lib()
    cbh = tq.codebook(128, 3)
    desc = tq.tq_packed(128, 3, 0, 0, 2 * 64, None, None, None, None)
    # null rotation / cache
    assert lib.tq_cache_append(None, 1, 1, 2, 1, 0, 64, 3, 0, cbh.ptr, None, None, ctypes.byref(desc), None) == 1
    assert lib.tq_cache_append(None, 1, 1, 2, 1, 0, 64, 3, 0, cbh.ptr, None, None, None, None) == 1
    assert lib.tq_scores_cache(None, 1, 8, 2, 10, 64, ctypes.byref(desc), cbh.ptr, None, None, None, None, 0,
                               None) == 1
    assert lib.tq_decode_attn_cache(None, 1, 8, 2, 10, 64, ctypes.byref(desc), ctypes.byref(desc), cbh.ptr, cbh.ptr,
                                    None, None, ctypes.c_float(1.0), None, None, 0, None) == 1


def test_split_entry_points_validate(tq):
    """The outlier-channel split entry points reject bad channel lists and missing handles before
    any device work, and size their workspace."""
    lib = tq.lib()
    h = ctypes.c_void_p()
    good = np.tile(np.arange(64, dtype=np.int32), (2, 1))
    rep = good.copy()
    rep[1, 5] = rep[1, 6]                     # repeated channel
    out = good.copy()
    out[0, 0] = 128                           # outside [0, 128)
    P = lambda a: ctypes.c_void_p(a.ctypes.data)
    assert lib.tq_make_split(2, 128, P(rep), ctypes.byref(h)) == 1
    assert lib.tq_make_split(2, 128, P(out), ctypes.byref(h)) == 1
    assert lib.tq_make_split(0, 128, P(good), ctypes.byref(h)) == 1
    assert lib.tq_make_split(2, 96, P(good), ctypes.byref(h)) == 3
    assert lib.tq_make_split(2, 128, None, ctypes.byref(h)) == 1
    cbh = tq.codebook(64, 3)
    desc = tq.tq_packed(64, 3, 0, 0, 10, None, None, None, None)
    assert lib.tq_encode_split(None, 1, 1, 2, 5, None, cbh.ptr, cbh.ptr, None, None, ctypes.byref(desc),
                               ctypes.byref(desc), None) == 1
    assert lib.tq_scores_split(None, 1, 8, 2, 5, None, ctypes.byref(desc), ctypes.byref(desc), cbh.ptr, cbh.ptr,
                               None, None, None, None, 0, None) == 1
    assert lib.tq_scores_split_workspace(2, 32) == 2 * 32 * 128 * 4


def test_split_wrappers_reject_bad_tensors(tq):
    """The Python split wrappers check shapes, dtypes, contiguity, output size and devices before
    calling the library (its split functions take no d and read 128 values per key)."""
    import torch
    TQE = tq.TQError
    sp = object()                      # never reached: every case fails in the wrapper
    n = 1 * 2 * 5
    K = (tq.alloc_packed(n, 64, 3, device="cpu"), tq.alloc_packed(n, 64, 2, device="cpu"))
    # encode_split / cache_append_split: x must be contiguous [B, H, T, 128] bf16 or fp32
    for fn in (lambda x: tq.encode_split(x, sp, None, None, None, None, out=K),
               lambda x: tq.cache_append_split(K, x, 0, 5, sp, None, None, None, None)):
        with pytest.raises(TQE, match=r"\[B, H, T, 128\]"):
            fn(torch.zeros((1, 2, 5, 64)))
        with pytest.raises(TQE, match=r"\[B, H, T, 128\]"):
            fn(torch.zeros((2 * 5, 128)))
        with pytest.raises(TQE, match="bf16 or fp32"):
            fn(torch.zeros((1, 2, 5, 128), dtype=torch.float16))
        with pytest.raises(TQE, match="contiguous"):
            fn(torch.zeros((1, 5, 2, 128)).transpose(1, 2))
    # scores_split / scores_split_cache: q must be contiguous fp32 [B, Hq, 128]; out sized B*Hq*T
    for fn in (lambda q, out=None: tq.scores_split(q, K, 2, sp, None, None, None, None, out=out),
               lambda q, out=None: tq.scores_split_cache(q, K, 2, 5, 5, sp, None, None, None, None, out=out)):
        with pytest.raises(TQE, match=r"\[B, Hq, 128\]"):
            fn(torch.zeros((1, 8, 64)))
        with pytest.raises(TQE, match="fp32"):
            fn(torch.zeros((1, 8, 128), dtype=torch.bfloat16))
        with pytest.raises(TQE, match="contiguous"):
            fn(torch.zeros((1, 128, 8)).transpose(1, 2))
        with pytest.raises(TQE, match="out must be"):
            fn(torch.zeros((1, 8, 128)), out=torch.zeros((1, 8, 4)))
        with pytest.raises(TQE, match="out must be"):
            fn(torch.zeros((1, 8, 128)), out=torch.zeros((1, 8, 5), dtype=torch.float64))
