"""Outlier channels at 8 bits, the other channels TurboQuant_mse: keys with a few large channels.

Test infrastructure only (see the package docstring).

"TurboQuant 和 RotorQuant 的真相", the section on the different needs of K and V: keys need more
bits, and one community practice keeps the outlier channels at 8 bits and codes the rest at
3 bits.  The page fixes neither which channels are outliers nor what "8-bit" means; the reading
taken here (the plainest one):

* the caller names, per KV head, n_o outlier channels, fixed ahead of time (the KV flow of
  "TurboQuant 详解" fits nothing online);
* the outlier channels of a key are stored as symmetric 8-bit integers with one scale per key:
  scale = max |x_c| / 127 over the key's outlier channels, q_c = x_c / scale rounded to the
  nearest integer, ties to even (so q lies in [-127, 127]); an all-zero outlier part has scale 0
  and q = 0;
* the other channels are coded by TurboQuant_mse exactly as a whole key is ("TurboQuant 详解",
  official steps 1-5), applied to the key with its outlier channels set to zero: norm
  s = ||x_rest||, y = R (x_rest / s), nearest-centroid indices, at d = 128 with the d = 128
  codebook.  (A Haar rotation maps every fixed unit vector, this one included, to a uniform point
  of the sphere, so the coordinate density is the same Beta law and the d = 128 codebook applies
  as the deployment checklist of "Sub-byte KV cache quantization with TurboQuant" asks);
* the reconstruction takes the rest channels from the TurboQuant code and the outlier channels from
  the 8-bit part: x_hat[rest] = (s R^T C[idx])[rest], x_hat[c] = scale q_c for c an outlier.
  The score is <q, x_hat> = s <R (q with the outlier channels zeroed), C[idx]> + scale <q_O, q8>.

Pinned by brute force (the 8-bit quantizer against all 255 levels), the reconstruction split by
channel, the identity of the two score formulas, and the d = 128 distortion of the rest code.
"""

from dataclasses import dataclass

import numpy as np

from .quantizer import EncodedMSE, decode_mse, encode_mse


@dataclass
class EncodedOutlier8:
    outliers: np.ndarray     # [H, n_o] channels per KV head
    rest: EncodedMSE         # idx [B, H, T, 128], norms [B, H, T] of the masked keys
    q8: np.ndarray           # [B, H, T, n_o] int8 values
    scale: np.ndarray        # [B, H, T] float64


def int8_absmax(v, dtype=np.float64):
    """Symmetric 8-bit quantization of rows v [..., n_o]: scale = max |v| / 127, q = round(v / scale)
    (half to even).  Returns (q int8, scale); an all-zero row gives scale 0, q 0.

    dtype is the precision of the two divisions (each correctly rounded); the page fixes none.
    float64 is the reading; float32 takes the integer decisions in a float32 kernel's precision,
    so that its codes can be compared bit for bit."""
    v = np.asarray(v, dtype=dtype)
    amax = np.max(np.abs(v), axis=-1)
    scale = amax / dtype(127.0)
    safe = np.where(scale > 0, scale, dtype(1.0))
    q = np.rint(v / safe[..., None])                  # numpy rint: half to even
    q = np.where(scale[..., None] > 0, q, dtype(0.0))
    return np.clip(q, -127, 127).astype(np.int8), scale


def rest_mask(outliers, d=128):
    """[H, d] boolean: True on the channels coded by TurboQuant (the non-outlier channels)."""
    outliers = np.asarray(outliers)
    m = np.ones((outliers.shape[0], d), dtype=bool)
    for h in range(outliers.shape[0]):
        m[h, outliers[h]] = False
    return m


def encode_outlier8(x, outliers, rotation, cb, int8_dtype=np.float64):
    """x [B, H, T, 128]; outliers [H, n_o] (distinct channels per head); int8_dtype: the precision
    of the 8-bit decisions (see int8_absmax)."""
    x = np.asarray(x, dtype=np.float64)
    bsz, h, t, d = x.shape
    mask = rest_mask(outliers, d)
    xr = x * mask[None, :, None, :]
    enc = encode_mse(xr.reshape(-1, d), rotation, cb)
    rest = EncodedMSE(idx=enc.idx.reshape(bsz, h, t, d), words=None, norms=enc.norms.reshape(bsz, h, t), y=None)
    xo = np.stack([x[:, hh][..., np.asarray(outliers)[hh]] for hh in range(h)], axis=1)   # [B, H, T, n_o]
    q8, scale = int8_absmax(xo, int8_dtype)
    return EncodedOutlier8(outliers=np.asarray(outliers), rest=rest, q8=q8, scale=scale)


def decode_outlier8(enc, rotation, cb):
    """x_hat [B, H, T, 128]: rest channels from the TurboQuant code, outlier channels from q8."""
    bsz, h, t, d = enc.rest.idx.shape
    xr = decode_mse(enc.rest.idx.reshape(-1, d), enc.rest.norms.reshape(-1), rotation, cb).reshape(bsz, h, t, d)
    mask = rest_mask(enc.outliers, d)
    out = xr * mask[None, :, None, :]
    for hh in range(h):
        out[:, hh][..., enc.outliers[hh]] = enc.q8[:, hh].astype(np.float64) * enc.scale[:, hh][..., None]
    return out


def scores_outlier8(q, enc, rotation, cb):
    """Raw scores [B, Hq, T] of queries q [B, Hq, 128] against outlier-8 keys of [B, Hkv, T]
    (kv head h // (Hq / Hkv)): s <R (q masked), C[idx]> + scale <q_O, q8>."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = enc.rest.idx.shape[1]
    ratio = hq // hkv
    mask = rest_mask(enc.outliers, d)
    cent = cb.centroids
    out = np.empty((bsz, hq, enc.rest.idx.shape[2]))
    for b in range(bsz):
        for h in range(hq):
            g = h // ratio
            qr = rotation @ (q[b, h] * mask[g])
            main = enc.rest.norms[b, g] * (cent[enc.rest.idx[b, g]] @ qr)
            side = enc.scale[b, g] * (enc.q8[b, g].astype(np.float64) @ q[b, h][enc.outliers[g]])
            out[b, h] = main + side
    return out


def decode_attention_outlier8(q, enc_k, v_idx, v_norms, rot_k, rot_v, cb_k, cb_v, scale):
    """Decode attention with outlier-8 keys ("TurboQuant 和 RotorQuant 的真相", chapter 1 formula):
    out[b, h] = sum_t softmax_t(scale <q[b,h], k_hat[b,g,t]>) v_hat[b,g,t], g = h // ratio, with
    k_hat the outlier-8 reconstruction (its logits are scores_outlier8) and v_hat = s_v R_V^T C_V[idx].
    q [B, Hq, 128]; v_idx [B, Hkv, T, 128]; v_norms [B, Hkv, T].  Returns float64 [B, Hq, 128]."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = v_idx.shape[1]
    ratio = hq // hkv
    logits = scale * scores_outlier8(q, enc_k, rot_k, cb_k)              # [B, Hq, T]
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        for g in range(hkv):
            v_hat = decode_mse(v_idx[b, g], v_norms[b, g], rot_v, cb_v)
            for h in range(g * ratio, (g + 1) * ratio):
                p = np.exp(logits[b, h] - np.max(logits[b, h]))
                out[b, h] = (p / np.sum(p)) @ v_hat
    return out
