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
* Prefill attention: "TurboQuant 详解", the KV-cache example (prefill: the prompt's keys and
  values are compressed as they are written into the cache) and the decode section's second
  route (the packed cache is unpacked, looked up and scaled inside the attention itself, never
  materialised); "TurboQuant 和 RotorQuant 的真相", the Flash Attention fusion section (K and V
  dequantized inside the attention kernel).  A chunk of Tn new tokens is appended at positions
  pos .. pos + Tn - 1, and the query of chunk token i (absolute position pos + i) attends with
  the causal rule of autoregressive attention to cached tokens 0 .. pos + i, old and new alike,
  all read back dequantized.  Computed as textbook masked softmax attention on K_hat, V_hat in
  float64.  Pinned by torch's scaled_dot_product_attention (float64, explicit mask) on the same
  dequantized tensors, Tn = 1 against decode_attention, chunked against one-shot prefill, and
  causality (later keys leave earlier outputs unchanged).
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


def prefill_attention(q, k_idx, k_norms, v_idx, v_norms, pos, rot_k, rot_v, cb_k, cb_v, scale):
    """Causal attention of a chunk of Tn queries over a compressed cache.

    q: [B, Hq, Tn, d], query i of the chunk at absolute position pos + i; k_idx / v_idx:
    [B, Hkv, T, d] indices and k_norms / v_norms [B, Hkv, T] of the cache after the chunk's own
    keys and values were appended (T >= pos + Tn; rows past pos + Tn - 1 are never read).
    out[b, h, i] = sum_{t <= pos + i} softmax_t(scale <q[b,h,i], k_hat[b,g,t]>) v_hat[b,g,t],
    g = h // (Hq / Hkv).  Returns float64 [B, Hq, Tn, d].
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, tn, d = q.shape
    hkv = k_idx.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if k_idx.shape[2] < pos + tn:
        raise ValueError("the cache must hold the chunk")
    ratio = hq // hkv
    live = pos + tn
    out = np.zeros((bsz, hq, tn, d))
    for bi in range(bsz):
        for g in range(hkv):
            k_hat = decode_mse(k_idx[bi, g, :live], k_norms[bi, g, :live], rot_k, cb_k)   # [live, d]
            v_hat = decode_mse(v_idx[bi, g, :live], v_norms[bi, g, :live], rot_v, cb_v)
            for h in range(g * ratio, (g + 1) * ratio):
                for i in range(tn):
                    n_vis = pos + i + 1                      # tokens 0 .. pos + i
                    logits = scale * (k_hat[:n_vis] @ q[bi, h, i])
                    p = np.exp(logits - np.max(logits))
                    p /= np.sum(p)
                    out[bi, h, i] = p @ v_hat[:n_vis]
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
