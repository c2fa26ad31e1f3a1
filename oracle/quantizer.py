"""TurboQuant_mse and TurboQuant_prod encode/decode, the packed format and the scores.

Test infrastructure only (see the package docstring).

* Nearest centroid: "TurboQuant 详解", TurboQuant_mse official steps, step 3 -- each rotated
  coordinate maps to argmin_k |y_i - c_k|.  For a sorted codebook this is the cell
  #{k : y_i >= t_k} between midpoint thresholds (the Lloyd-Max example of the same page);
  a value exactly on a threshold goes to the upper index (reading: same rule as sign(0) = +1
  in the TurboQuant_prod example).  Pinned by brute-force argmin and the 1-bit example.
* Norm extraction: "TurboQuant 详解", the Q&A after Theorem 1 and the KV prefill example
  (steps 1-6): store s = ||x||, quantize u = x / s, rotate y = R u, pack the indices.
  Reading: a zero vector has u = 0 (its indices are those of y = 0; it decodes to 0).
* Packed format: the pages say only "compact bitstream" (prefill example, step 5).  Reading:
  per vector, coordinate i occupies stream bits [i b, i b + b), least significant bit first;
  stream bit p is bit (p mod 32) of 32-bit word floor(p / 32); W = d b / 32 words.  Norms are
  float32 (the configurations store fp32 norms; one page suggests fp16).
* Decode: "TurboQuant 详解", official step 5 -- x_hat = s R^T C[idx].
* TurboQuant_prod: "TurboQuant 详解", TurboQuant_prod section, and "TurboQuant
  first-principles walkthrough", QJL paragraph -- (b-1)-bit MSE stage, residual
  r = x - x_hat_mse, gamma = ||r||, sign bits z = sign(S r) with sign(0) = +1, correction
  gamma * sqrt(pi/2) / d * S^T z.  Reading: S has i.i.d. N(0, 1) entries (the only choice
  for which the printed constant makes the estimator unbiased); r and gamma are in the
  original scale.  Pinned by the page's 2-D example and by unbiasedness over S draws.
* Scores: <q, x_hat> = s <R q, C[idx]> (query rotated once, "Sub-byte KV cache quantization
  with TurboQuant", third layer: pre-rotate the query, then per position a lookup and a dot),
  plus gamma * sqrt(pi/2) / d * <S q, z> for prod.
"""

from dataclasses import dataclass

import numpy as np

from .rng import gaussian

QJL_CONST = float(np.sqrt(np.pi / 2.0))


def nearest_index(y, thresholds):
    """Index of the nearest centroid: #{k : y >= t_k} (ties to the upper index)."""
    t = np.asarray(thresholds, dtype=np.float64)
    return np.searchsorted(t, np.asarray(y, dtype=np.float64), side="right").astype(np.int64)


def pack_bits(idx, b):
    """Pack b-bit indices along the last axis into uint32 words, LSB-first stream."""
    idx = np.asarray(idx).astype(np.uint64)
    lead = idx.shape[:-1]
    d = idx.shape[-1]
    if (d * b) % 32 != 0:
        raise ValueError("d * b must be a multiple of 32")
    if np.any(idx >> np.uint64(b)):
        raise ValueError("index does not fit in b bits")
    bits = (idx[..., None] >> np.arange(b, dtype=np.uint64)) & np.uint64(1)
    stream = bits.reshape(*lead, d * b // 32, 32)
    words = (stream << np.arange(32, dtype=np.uint64)).sum(axis=-1)
    return words.astype(np.uint32)


def unpack_bits(words, d, b):
    """Inverse of pack_bits: uint32 words [..., d b / 32] -> indices [..., d] (int64)."""
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    lead = words.shape[:-1]
    if words.shape[-1] * 32 != d * b:
        raise ValueError("word count does not match d * b / 32")
    stream = (words[..., None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    bits = stream.reshape(*lead, d, b)
    idx = (bits << np.arange(b, dtype=np.uint64)).sum(axis=-1)
    return idx.astype(np.int64)


def pack_token_blocked(idx, b):
    """Token-blocked layout of b-bit indices idx [n, d] (the layout the decode-attention value
    cache uses; the pages fix no layout, this is the library's documented reading).

    Rows are grouped in blocks of 32 (rows past n are index 0).  Inside block beta, chunk
    (o, c) for octet o = 0..3 and coordinate c = 0..d-1 sits at chunk position o * d + c and
    holds the indices of rows 32 beta + 8 o + e, e = 0..7, at coordinate c, LSB-first (row e at
    chunk bits [b e, b e + b)).  Chunks of 8 b bits are concatenated LSB-first into the block's
    stream of 32 d b bits = d b words.  Returns uint32 [ceil(n / 32), d * b].
    """
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    nblk = (n + 31) // 32
    pad = np.zeros((nblk * 32, d), dtype=np.int64)
    pad[:n] = idx
    blocks = pad.reshape(nblk, 4, 8, d)                # [beta, o, e, c]
    chunks = blocks.transpose(0, 1, 3, 2)               # [beta, o, c, e]: chunk (o, c), row e
    return pack_bits(chunks.reshape(nblk, 4 * d * 8), b)


def unpack_token_blocked(words, n, d, b):
    """Inverse of pack_token_blocked: uint32 [ceil(n / 32), d b] -> indices [n, d]."""
    words = np.asarray(words, dtype=np.uint32)
    nblk = (n + 31) // 32
    chunks = unpack_bits(words.reshape(nblk, d * b), 4 * d * 8, b).reshape(nblk, 4, d, 8)
    return chunks.transpose(0, 1, 3, 2).reshape(nblk * 32, d)[:n]


@dataclass
class EncodedMSE:
    idx: np.ndarray      # [..., d] int64 centroid indices
    words: np.ndarray    # [..., d b / 32] uint32 packed indices (None if d b % 32 != 0)
    norms: np.ndarray    # [...] float64, s = ||x||
    y: np.ndarray        # [..., d] float64 rotated unit coordinates R u


@dataclass
class EncodedProd:
    mse: EncodedMSE      # the (b-1)-bit stage
    z: np.ndarray        # [..., d] bool, True where (S r)_i >= 0
    qjl_words: np.ndarray  # [..., d / 32] uint32, bit i = z_i (None if d % 32 != 0)
    gamma: np.ndarray    # [...] float64 residual norms ||r||
    proj: np.ndarray     # [..., d] float64, S r


def encode_mse(x, rotation, cb):
    """TurboQuant_mse encode of the rows of x (float64 [..., d])."""
    x = np.asarray(x, dtype=np.float64)
    s = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(s > 0.0, s, 1.0)
    u = np.where((s > 0.0)[..., None], x / safe[..., None], 0.0)
    y = u @ np.asarray(rotation, dtype=np.float64).T
    idx = nearest_index(y, cb.thresholds)
    words = pack_bits(idx, cb.b) if (idx.shape[-1] * cb.b) % 32 == 0 else None
    return EncodedMSE(idx=idx, words=words, norms=s, y=y)


def decode_mse(idx, norms, rotation, cb):
    """x_hat = s R^T C[idx] for each row."""
    yhat = cb.centroids[np.asarray(idx)]
    return np.asarray(norms, dtype=np.float64)[..., None] * (yhat @ np.asarray(rotation))


def qjl_matrix(d, seed):
    """QJL projection S: d x d i.i.d. N(0, 1) entries, row-major from the seeded stream."""
    return gaussian(seed, d * d).reshape(d, d)


def qjl_encode(r, s_matrix):
    """1-bit QJL of residuals r [..., d]: (z = (S r >= 0), gamma = ||r||, S r)."""
    r = np.asarray(r, dtype=np.float64)
    gamma = np.sqrt(np.sum(r * r, axis=-1))
    proj = r @ np.asarray(s_matrix, dtype=np.float64).T
    return proj >= 0.0, gamma, proj


def qjl_correction(z, gamma, s_matrix):
    """Correction vector gamma sqrt(pi/2) / d S^T z, with z mapped to {-1, +1}."""
    z = np.asarray(z, dtype=bool)
    d = z.shape[-1]
    zpm = np.where(z, 1.0, -1.0)
    return (np.asarray(gamma, dtype=np.float64) * QJL_CONST / d)[..., None] * (
        zpm @ np.asarray(s_matrix, dtype=np.float64))


def encode_prod(x, rotation, cb_stage, s_matrix):
    """TurboQuant_prod encode: MSE stage with ``cb_stage`` ((b-1) bits), then 1-bit QJL."""
    x = np.asarray(x, dtype=np.float64)
    enc = encode_mse(x, rotation, cb_stage)
    xhat = decode_mse(enc.idx, enc.norms, rotation, cb_stage)
    z, gamma, proj = qjl_encode(x - xhat, s_matrix)
    qw = pack_bits(z.astype(np.int64), 1) if z.shape[-1] % 32 == 0 else None
    return EncodedProd(mse=enc, z=z, qjl_words=qw, gamma=gamma, proj=proj)


def decode_prod(encp, rotation, cb_stage, s_matrix):
    """x_hat_prod = x_hat_mse + gamma sqrt(pi/2)/d S^T z (z in {-1, +1})."""
    base = decode_mse(encp.mse.idx, encp.mse.norms, rotation, cb_stage)
    return base + qjl_correction(encp.z, encp.gamma, s_matrix)


def scores_mse(q, idx, norms, rotation, cb):
    """<q_m, x_hat_n> = s_n <R q_m, C[idx_n]> for queries q [m, d] and keys [n, d] -> [m, n]."""
    q_rot = np.asarray(q, dtype=np.float64) @ np.asarray(rotation).T
    yhat = cb.centroids[np.asarray(idx)]
    return (q_rot @ yhat.T) * np.asarray(norms, dtype=np.float64)[None, :]


def scores_prod(q, encp, rotation, cb_stage, s_matrix):
    """Unbiased prod score: MSE part plus gamma sqrt(pi/2)/d <S q, z>."""
    d = encp.z.shape[-1]
    base = scores_mse(q, encp.mse.idx, encp.mse.norms, rotation, cb_stage)
    q_s = np.asarray(q, dtype=np.float64) @ np.asarray(s_matrix).T
    zpm = np.where(encp.z, 1.0, -1.0)
    return base + (q_s @ zpm.T) * (encp.gamma * QJL_CONST / d)[None, :]


def quantize_rotated(y32, cb):
    """Indices of given float32 rotated unit coordinates against the float32 thresholds.

    The decision is taken in the precision the device takes it (float32 operands; the
    comparison itself is exact), so packed bits can be compared bit for bit.
    """
    t32 = cb.thresholds.astype(np.float32).astype(np.float64)
    y = np.asarray(y32, dtype=np.float32).astype(np.float64)
    return np.searchsorted(t32, y, side="right").astype(np.int64)
