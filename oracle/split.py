"""Outlier-channel mixed precision: two TurboQuant_mse codes per key vector.

Test infrastructure only (see the package docstring).

* "TurboQuant 和 RotorQuant 的真相", the section on the asymmetric needs of K and V: keys need
  more bits than values, either a wider code or mixed precision, where the outlier channels
  get more bits than the others.
* "TurboQuant 详解", the engineering section (key data points): 3.5 bits per channel is
  quality neutral, 2.5 bits per channel degrades only slightly.

Readings (the pages fix no mechanism):
* The d channels of a key are split per KV head into an outlier set O of d/2 channels, chosen
  by the caller (fixed ahead of time, since the pages' KV flow fits nothing online), and the
  remaining d/2 channels.  Each part is a vector of its own, encoded by TurboQuant_mse with
  its own norm, its own rotation (d/2 x d/2) and the codebook for dimension d/2, the outlier
  part at b_o bits and the rest at b_r.  The bit budget per channel is (b_o + b_r) / 2, which
  gives the pages' 2.5 and 3.5 bits with (b_o, b_r) = (3, 2) and (4, 3).
* Coordinate order inside a part: the outlier part in the order the caller lists its
  channels, the rest in ascending channel order.
* Reconstruction puts each part's decoded vector back on its own channels; the score of a
  query is <q, x_hat>, as for a single code.

Parity status: the split, the reconstruction and the scores are pinned by the reduction to
two plain encodes, invariance under relabelling the channels, an element-by-element form of
the score in the two rotated domains, and the per-part distortion against the exact value of
each part's codebook.
"""

from dataclasses import dataclass

import numpy as np

from .quantizer import EncodedMSE, decode_mse, encode_mse


def channel_order(outliers, d):
    """[H, d] channel order per head: the outlier channels as listed, then the rest ascending."""
    outliers = np.asarray(outliers, dtype=np.int64)
    heads, m = outliers.shape
    if 2 * m != d:
        raise ValueError("the outlier set holds half of the channels")
    order = np.empty((heads, d), dtype=np.int64)
    for h in range(heads):
        o = outliers[h]
        if np.any(o < 0) or np.any(o >= d) or len(set(o.tolist())) != m:
            raise ValueError("outlier channels must be distinct channels of the vector")
        rest = np.setdiff1d(np.arange(d), o)
        order[h] = np.concatenate([o, rest])
    return order


@dataclass
class EncodedSplit:
    order: np.ndarray    # [H, d] channel order (outliers first)
    outlier: EncodedMSE  # codes of the outlier parts, [..., H, T, d/2]
    rest: EncodedMSE     # codes of the remaining parts, [..., H, T, d/2]


def encode_split(x, outliers, rot_o, rot_r, cb_o, cb_r):
    """Split encode of keys x [B, H, T, d]: two TurboQuant_mse codes per vector."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    order = channel_order(outliers, d)
    if order.shape[0] != x.shape[1]:
        raise ValueError("one outlier set per head")
    m = d // 2
    parts = np.stack([x[:, h][..., order[h]] for h in range(x.shape[1])], axis=1)
    return EncodedSplit(order=order, outlier=encode_mse(parts[..., :m], rot_o, cb_o),
                        rest=encode_mse(parts[..., m:], rot_r, cb_r))


def decode_split(enc, rot_o, rot_r, cb_o, cb_r):
    """x_hat [B, H, T, d]: each part decoded (s R^T C[idx]) and put back on its channels."""
    xo = decode_mse(enc.outlier.idx, enc.outlier.norms, rot_o, cb_o)
    xr = decode_mse(enc.rest.idx, enc.rest.norms, rot_r, cb_r)
    m = xo.shape[-1]
    xhat = np.zeros(xo.shape[:-1] + (2 * m,))
    for h in range(xo.shape[1]):
        xhat[:, h][..., enc.order[h, :m]] = xo[:, h]
        xhat[:, h][..., enc.order[h, m:]] = xr[:, h]
    return xhat


def scores_split(q, enc, rot_o, rot_r, cb_o, cb_r):
    """Scores [B, Hq, T] = <q, x_hat> of queries q [B, Hq, d] against split-coded keys; query
    head h reads KV head h // (Hq / Hkv)."""
    q = np.asarray(q, dtype=np.float64)
    xhat = decode_split(enc, rot_o, rot_r, cb_o, cb_r)
    ratio = q.shape[1] // xhat.shape[1]
    return np.stack([xhat[:, h // ratio] @ q[:, h][..., None] for h in range(q.shape[1])],
                    axis=1)[..., 0]


def decode_attention_split(q, enc, v_idx, v_norms, rot_o, rot_r, rot_v, cb_o, cb_r, cb_v, scale):
    """Decode attention with split-coded keys ("TurboQuant 和 RotorQuant 的真相", chapter 1 formula):
    out[b, h] = sum_t softmax_t(scale <q[b,h], k_hat[b,g,t]>) v_hat[b,g,t], g = h // ratio, with
    k_hat the split reconstruction (its logits are scores_split) and v_hat = s_v R_V^T C_V[idx].
    q [B, Hq, d]; v_idx [B, Hkv, T, d]; v_norms [B, Hkv, T].  Returns float64 [B, Hq, d]."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = v_idx.shape[1]
    ratio = hq // hkv
    logits = scale * scores_split(q, enc, rot_o, rot_r, cb_o, cb_r)      # [B, Hq, T]
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        for g in range(hkv):
            v_hat = decode_mse(v_idx[b, g], v_norms[b, g], rot_v, cb_v)
            for h in range(g * ratio, (g + 1) * ratio):
                p = np.exp(logits[b, h] - np.max(logits[b, h]))
                out[b, h] = (p / np.sum(p)) @ v_hat
    return out
