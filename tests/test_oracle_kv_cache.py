"""Pins of the oracle's streaming KV cache (prefill, per-token appends, decode over the prefix).

The appends are checked bit by bit against a per-bit walk of each layout's definition (not the
vectorized packers), against the one-shot encode of the same tokens (streaming is the same
quantizer applied token by token: "TurboQuant 详解", KV-cache example, and the section after it:
no online fitting), and for the untouched rows against the cache's previous contents."""

import numpy as np
import pytest

import oracle


def _setup(d, b, seed=0):
    return oracle.dense_rotation(d, 1), oracle.codebook(d, b)


def _token_blocked_bit(words, d, b, row, coord, j):
    """Bit j of the index of (row, coord) in a token-blocked array, walked per the definition:
    block row // 32, chunk position o d + c with o = (row % 32) // 8, field e = row % 8 at
    chunk bits [b e, b e + b), chunks of 8 b bits concatenated LSB-first."""
    blk, within = divmod(row, 32)
    o, e = divmod(within, 8)
    p = (o * d + coord) * 8 * b + b * e + j
    return (int(words[blk, p // 32]) >> (p % 32)) & 1


def _append_plan():
    # prefill 37 tokens, five single-token decode steps, then a 22-token burst
    return [(0, 37), (37, 1), (38, 1), (39, 1), (40, 1), (41, 1), (42, 22)]


@pytest.mark.parametrize("b", [2, 3])
def test_token_blocked_appends_bitwise(b):
    d, n_seq, t_cap = 32, 2, 64
    rot, cb = _setup(d, b)
    rng = np.random.default_rng(5)
    words0 = rng.integers(0, 2**32, size=(n_seq * t_cap // 32, d * b), dtype=np.uint64).astype(np.uint32)
    norms0 = rng.standard_normal(n_seq * t_cap)
    x = rng.standard_normal((n_seq, 64, d))
    words, norms = words0, norms0
    for pos, n_new in _append_plan():
        words, norms, _ = oracle.append_token_blocked_mse(words, norms, x[:, pos:pos + n_new], pos, t_cap, rot, cb)
    written = 64
    full = oracle.encode_mse(x.reshape(-1, d), rot, cb).idx.reshape(n_seq, 64, d)
    for s in range(n_seq):
        for t in range(t_cap):
            row = s * t_cap + t
            for c in range(d):
                for j in range(b):
                    got = _token_blocked_bit(words, d, b, row, c, j)
                    if t < written:
                        assert got == (int(full[s, t, c]) >> j) & 1
                    else:
                        assert got == _token_blocked_bit(words0, d, b, row, c, j)
    rows = oracle.live_rows(n_seq, t_cap, written).reshape(-1)
    np.testing.assert_allclose(norms[rows], np.linalg.norm(x.reshape(-1, d), axis=1), rtol=1e-15)


def test_token_blocked_append_keeps_other_rows():
    # a single append in the middle of a block touches exactly that row's d fields
    d, b, n_seq, t_cap = 32, 3, 1, 32
    rot, cb = _setup(d, b)
    rng = np.random.default_rng(9)
    words0 = rng.integers(0, 2**32, size=(1, d * b), dtype=np.uint64).astype(np.uint32)
    x = rng.standard_normal((1, 1, d))
    words, _, enc = oracle.append_token_blocked_mse(words0, np.zeros(32), x, 13, t_cap, rot, cb)
    diff = np.unpackbits((words ^ words0).view(np.uint8))
    changed = oracle.unpack_token_blocked(words ^ words0, 32, d, b)
    assert np.all(changed[np.arange(32) != 13] == 0)
    assert diff.sum() == np.count_nonzero(np.unpackbits(
        (oracle.unpack_token_blocked(words0, 32, d, b)[13] ^ enc.idx[0]).astype(np.uint8)))


@pytest.mark.parametrize("b", [3, 4])
def test_rows_appends_match_one_shot_encode(b):
    d, n_seq, t_cap = 128, 3, 50
    rot, cb = _setup(d, b)
    w_per = d * b // 32
    rng = np.random.default_rng(11)
    words0 = rng.integers(0, 2**32, size=(n_seq * t_cap, w_per), dtype=np.uint64).astype(np.uint32)
    norms0 = rng.standard_normal(n_seq * t_cap)
    x = rng.standard_normal((n_seq, 45, d))
    words, norms = words0, norms0
    for pos, n_new in [(0, 20), (20, 1), (21, 1), (22, 23)]:
        words, norms, _ = oracle.append_rows_mse(words, norms, x[:, pos:pos + n_new], pos, t_cap, rot, cb)
    full = oracle.encode_mse(x.reshape(-1, d), rot, cb)
    for s in range(n_seq):
        for t in range(t_cap):
            row = s * t_cap + t
            if t < 45:
                assert words[row].tolist() == full.words[s * 45 + t].tolist()
                assert norms[row] == full.norms[s * 45 + t]
            else:
                assert words[row].tolist() == words0[row].tolist()
                assert norms[row] == norms0[row]


def test_rows_prod_append_matches_one_shot_encode():
    d, n_seq, t_cap = 128, 2, 10
    rot = oracle.dense_rotation(d, 1)
    cb = oracle.codebook(d, 3)
    smat = oracle.qjl_matrix(d, 2)
    rng = np.random.default_rng(12)
    x = rng.standard_normal((n_seq, 6, d))
    words = np.zeros((n_seq * t_cap, 12), np.uint32)
    qw = np.zeros((n_seq * t_cap, 4), np.uint32)
    norms = np.zeros(n_seq * t_cap)
    rn = np.zeros(n_seq * t_cap)
    for pos, n_new in [(0, 4), (4, 1), (5, 1)]:
        words, norms, qw, rn, _ = oracle.append_rows_prod(words, norms, qw, rn, x[:, pos:pos + n_new], pos, t_cap,
                                                          rot, cb, smat)
    full = oracle.encode_prod(x.reshape(-1, d), rot, cb, smat)
    rows = oracle.live_rows(n_seq, t_cap, 6).reshape(-1)
    np.testing.assert_array_equal(words[rows], full.mse.words)
    np.testing.assert_array_equal(qw[rows], full.qjl_words)
    np.testing.assert_array_equal(rn[rows], full.gamma)
    assert not words[oracle.live_rows(n_seq, t_cap, t_cap).reshape(n_seq, t_cap)[:, 6:].reshape(-1)].any()


def test_append_bounds():
    with pytest.raises(ValueError):
        oracle.cache_rows(2, 16, 10, 7)
    with pytest.raises(ValueError):
        oracle.cache_rows(2, 16, -1, 1)
    rot, cb = _setup(32, 2)
    with pytest.raises(ValueError):
        oracle.append_token_blocked_mse(np.zeros((1, 64), np.uint32), np.zeros(48), np.zeros((1, 1, 32)), 0, 48,
                                        rot, cb)
    assert oracle.cache_rows(2, 16, 3, 2).tolist() == [[3, 4], [19, 20]]
