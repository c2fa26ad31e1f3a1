"""Decode-step attention over compressed K and V, and top-k retrieval.

Test infrastructure only (see the package docstring).

* Attention: "TurboQuant 和 RotorQuant 的真相", chapter 1 -- softmax(Q K^T / sqrt(d)) V; the
  decode flow of "TurboQuant 详解" (decode section): the new query attends to every cached
  key and takes the weighted sum of every cached value, read from the compressed cache.
  K and V are both stored TurboQuant_mse ("Sub-byte KV cache quantization with TurboQuant",
  precision/throughput section: store MSE, keep prod for custom score kernels).
  GQA head mapping kv_head = q_head // (Hq / Hkv) (same page, third layer).
  Computed as textbook dense attention on the dequantized K_hat, V_hat in float64, with a
  max-subtracted softmax.  Pinned by T = 1 (output = v_hat), equal logits (output = mean)
  and brute-force attention on tiny inputs.
* Top-k: the k largest scores per query, ties broken by the smaller database index
  ("TurboQuant 详解", pain point 3: retrieval ranks by inner product).  Brute force.
"""

import numpy as np

from .quantizer import decode_mse


def decode_attention(q, k_idx, k_norms, v_idx, v_norms, rot_k, rot_v, cb_k, cb_v, scale):
    """out[b, h] = sum_t softmax_t(scale <q[b,h], k_hat[b,g,t]>) v_hat[b,g,t], g = h // ratio.

    q: [B, Hq, d]; k_idx/v_idx: [B, Hkv, T, d] indices; k_norms/v_norms: [B, Hkv, T].
    Returns float64 [B, Hq, d].
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = k_idx.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    ratio = hq // hkv
    out = np.zeros((bsz, hq, d))
    for bi in range(bsz):
        for g in range(hkv):
            k_hat = decode_mse(k_idx[bi, g], k_norms[bi, g], rot_k, cb_k)   # [T, d]
            v_hat = decode_mse(v_idx[bi, g], v_norms[bi, g], rot_v, cb_v)   # [T, d]
            for h in range(g * ratio, (g + 1) * ratio):
                logits = scale * (k_hat @ q[bi, h])
                p = np.exp(logits - np.max(logits))
                p /= np.sum(p)
                out[bi, h] = p @ v_hat
    return out


def topk(scores, k):
    """Top-k per row of scores [m, n]: (values [m, k], indices [m, k]); ties -> smaller index."""
    scores = np.asarray(scores, dtype=np.float64)
    m, n = scores.shape
    k = min(k, n)
    vals = np.empty((m, k))
    inds = np.empty((m, k), dtype=np.int64)
    cols = np.arange(n)
    for i in range(m):
        order = np.lexsort((cols, -scores[i]))[:k]
        inds[i] = order
        vals[i] = scores[i, order]
    return vals, inds
