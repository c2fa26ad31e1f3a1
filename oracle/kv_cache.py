"""Streaming compressed KV cache: prefill, per-token append, and decode over the cache.

Test infrastructure only (see the package docstring).

* "TurboQuant 详解", the worked KV-cache example (prefill and decode): prefill compresses the
  prompt's keys and values token by token and head by head and writes the bit-packed result
  into the persistent cache; at each decode step the new token's key and value are produced
  and appended to the end of the cache at once, and the step's query attends to every cached
  key and takes the weighted sum of every cached value.  The section after it (what is special
  about TurboQuant here) adds that no online fitting is needed: a token is quantized and written
  as soon as it exists, with only rotation, lookup and packing online.
* Cache geometry (a reading; the pages fix no layout): B * H sequences of capacity T_cap rows
  each; sequence s = b * H + h owns rows [s T_cap, (s + 1) T_cap) of the packed arrays.  Keys use
  the rows layout, values the token-blocked layout (quantizer.pack_token_blocked), which needs
  T_cap to be a multiple of 32 so that every sequence owns whole blocks.  An append writes rows
  pos .. pos + n_new - 1 of every sequence and leaves every other stored bit unchanged.

The appends here are defined through the pinned primitives: the encoders of quantizer.py and
the two packers.  The rows-layout append is a row assignment; the token-blocked append unpacks
the whole array with the layout's inverse, assigns the rows and packs it again, so every field
of every other row passes through unchanged by construction.
"""

import numpy as np

from .quantizer import (encode_mse, encode_prod, pack_token_blocked, unpack_token_blocked)


def cache_rows(n_seq, t_cap, pos, n_new):
    """Cache rows written by an append: [n_seq, n_new] int64, row s T_cap + pos + t."""
    if pos < 0 or n_new < 0 or pos + n_new > t_cap:
        raise ValueError("append outside the cache capacity")
    return (np.arange(n_seq)[:, None] * t_cap + pos + np.arange(n_new)[None, :]).astype(np.int64)


def append_rows_mse(words, norms, x_new, pos, t_cap, rotation, cb):
    """Rows-layout MSE append.  words [n_seq T_cap, d b / 32] uint32, norms [n_seq T_cap];
    x_new [n_seq, n_new, d].  Returns updated copies (words, norms) and the encoding."""
    x_new = np.asarray(x_new, dtype=np.float64)
    n_seq, n_new, d = x_new.shape
    enc = encode_mse(x_new.reshape(-1, d), rotation, cb)
    rows = cache_rows(n_seq, t_cap, pos, n_new).reshape(-1)
    w = np.array(words, dtype=np.uint32, copy=True)
    nr = np.array(norms, dtype=np.float64, copy=True)
    w[rows] = enc.words
    nr[rows] = enc.norms
    return w, nr, enc


def append_rows_prod(words, norms, qwords, rnorms, x_new, pos, t_cap, rotation, cb_stage, s_matrix):
    """Rows-layout TurboQuant_prod append: indices, norms, QJL sign words and residual norms."""
    x_new = np.asarray(x_new, dtype=np.float64)
    n_seq, n_new, d = x_new.shape
    encp = encode_prod(x_new.reshape(-1, d), rotation, cb_stage, s_matrix)
    rows = cache_rows(n_seq, t_cap, pos, n_new).reshape(-1)
    w = np.array(words, dtype=np.uint32, copy=True)
    nr = np.array(norms, dtype=np.float64, copy=True)
    qw = np.array(qwords, dtype=np.uint32, copy=True)
    rn = np.array(rnorms, dtype=np.float64, copy=True)
    w[rows] = encp.mse.words
    nr[rows] = encp.mse.norms
    qw[rows] = encp.qjl_words
    rn[rows] = encp.gamma
    return w, nr, qw, rn, encp


def assign_token_blocked(words, n_rows, d, b, rows, idx):
    """Token-blocked words with the indices of `rows` replaced by idx [len(rows), d]; every other
    field is carried over unchanged (unpack everything, assign, pack again)."""
    all_idx = unpack_token_blocked(words, n_rows, d, b).copy()
    all_idx[np.asarray(rows, dtype=np.int64)] = np.asarray(idx, dtype=np.int64)
    return pack_token_blocked(all_idx, b)


def append_token_blocked_mse(words, norms, x_new, pos, t_cap, rotation, cb):
    """Token-blocked MSE append (the value cache).  words [n_seq T_cap / 32, d b] uint32."""
    if t_cap % 32 != 0:
        raise ValueError("the token-blocked cache needs T_cap to be a multiple of 32")
    x_new = np.asarray(x_new, dtype=np.float64)
    n_seq, n_new, d = x_new.shape
    enc = encode_mse(x_new.reshape(-1, d), rotation, cb)
    rows = cache_rows(n_seq, t_cap, pos, n_new).reshape(-1)
    w = assign_token_blocked(words, n_seq * t_cap, d, cb.b, rows, enc.idx)
    nr = np.array(norms, dtype=np.float64, copy=True)
    nr[rows] = enc.norms
    return w, nr, enc


def live_rows(n_seq, t_cap, length):
    """The first `length` rows of every sequence, [n_seq, length] (the attended prefix)."""
    return cache_rows(n_seq, t_cap, 0, length)
