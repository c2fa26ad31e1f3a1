"""TurboQuant encode and compressed-key score on MI355X (gfx950).

A thin Python layer over libtq.so (include/tq.h): handles for the codebook, rotation and QJL
matrix; torch tensors for device memory; torch's current stream for ordering.  Every step of the
encode / score path runs in the library's HIP kernels; if the library is missing, calls raise.
"""

import ctypes

import numpy as np

from ._binding import (DENSITY, LAYOUT, MODE, ROT_KIND, DTYPE_BF16, DTYPE_F32, TQError, check, lib,
                       tq_packed, host_splitmix64, host_gaussian, host_codebook, host_rotation,
                       host_qjl_matrix, SIGNATURES)

__all__ = [
    "Codebook", "Rotation", "QJL", "Packed", "codebook", "codebook_from_values", "make_rotation",
    "rotation_from_matrix", "make_qjl", "qjl_from_matrix", "alloc_packed", "encode", "rotate",
    "quantize_rotated", "decode", "scores", "scores_workspace", "packed_words", "TQError",
    "decode_attn", "decode_attn_workspace", "encode_workspace", "search_workspace", "search_topk",
    "prepare_queries", "scores_prepared", "scores_noalloc", "timer_arm", "timer_read", "timer_reset",
    "KVCache", "alloc_cache", "cache_append", "kv_append", "scores_cache", "decode_attn_cache",
    "prefill_attn", "prefill_attn_workspace",
    "Split", "make_split", "encode_split", "scores_split", "scores_split_workspace", "alloc_split_cache",
    "cache_append_split", "scores_split_cache", "peak_read", "peak_copy", "peak_mfma",
    "Outlier8", "make_outlier8", "encode_outlier8", "scores_outlier8", "scores_outlier8_workspace",
    "decode_attn_outlier8", "decode_attn_outlier8_workspace", "decode_attn_split", "decode_attn_split_workspace",
    "host_splitmix64", "host_gaussian", "host_codebook", "host_rotation", "host_qjl_matrix",
]


def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _np(a):
    return ctypes.c_void_p(a.ctypes.data)


class _Handle:
    _free = None

    def __init__(self, ptr):
        self._ptr = ptr

    @property
    def ptr(self):
        return self._ptr

    def close(self):
        if self._ptr:
            getattr(lib(), self._free)(self._ptr)
            self._ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Codebook(_Handle):
    _free = "tq_codebook_free"

    def __init__(self, ptr, d, b):
        super().__init__(ptr)
        self.d, self.b = d, b

    def values(self):
        c = np.empty(1 << self.b)
        t = np.empty((1 << self.b) - 1)
        check(lib().tq_codebook_values(self.ptr, _np(c), _np(t)))
        return c, t


class Rotation(_Handle):
    _free = "tq_rotation_free"

    def __init__(self, ptr, d, kind):
        super().__init__(ptr)
        self.d, self.kind = d, kind

    def matrix(self):
        r = np.empty((self.d, self.d))
        check(lib().tq_rotation_export(self.ptr, _np(r)))
        return r


class QJL(_Handle):
    _free = "tq_qjl_free"

    def __init__(self, ptr, d, rotation):
        super().__init__(ptr)
        self.d = d
        self.rotation = rotation


def codebook(d, b, density="beta"):
    h = ctypes.c_void_p()
    check(lib().tq_codebook(d, b, DENSITY[density], ctypes.byref(h)))
    return Codebook(h.value, d, b)


def codebook_from_values(d, centroids):
    c = np.ascontiguousarray(centroids, dtype=np.float64)
    b = int(round(np.log2(c.size)))
    h = ctypes.c_void_p()
    check(lib().tq_codebook_from_values(d, b, _np(c), ctypes.byref(h)))
    return Codebook(h.value, d, b)


def make_rotation(d, seed, kind="dense"):
    h = ctypes.c_void_p()
    check(lib().tq_make_rotation(d, seed, ROT_KIND[kind], ctypes.byref(h)))
    return Rotation(h.value, d, kind)


def rotation_from_matrix(m):
    m = np.ascontiguousarray(m, dtype=np.float64)
    h = ctypes.c_void_p()
    check(lib().tq_rotation_from_matrix(m.shape[0], _np(m), ctypes.byref(h)))
    return Rotation(h.value, m.shape[0], "dense")


def make_qjl(d, seed, rotation):
    h = ctypes.c_void_p()
    check(lib().tq_make_qjl(d, seed, rotation.ptr, ctypes.byref(h)))
    return QJL(h.value, d, rotation)


def qjl_from_matrix(s, rotation):
    s = np.ascontiguousarray(s, dtype=np.float64)
    h = ctypes.c_void_p()
    check(lib().tq_qjl_from_matrix(s.shape[0], _np(s), rotation.ptr, ctypes.byref(h)))
    return QJL(h.value, s.shape[0], rotation)


def packed_words(d, bits):
    return int(lib().tq_packed_words(d, bits))


class Packed:
    """Caller-owned packed storage: idx int32 (uint32 bits) [n, d*bits/32] (rows layout) or
    [ceil(n/32), d*bits] (token-blocked layout), norms [n] fp32, and for prod qjl [n, d/32]
    int32 and rnorms [n] fp32."""

    def __init__(self, d, bits, mode, n, idx, norms, qjl=None, rnorms=None, layout="rows"):
        self.d, self.bits, self.mode, self.n, self.layout = d, bits, mode, n, layout
        self.idx, self.norms, self.qjl, self.rnorms = idx, norms, qjl, rnorms

    def descriptor(self):
        return tq_packed(self.d, self.bits, MODE[self.mode], LAYOUT[self.layout], self.n, _dptr(self.idx),
                         _dptr(self.norms), _dptr(self.qjl), _dptr(self.rnorms))


def alloc_packed(n, d, bits, mode="mse", device="cuda", layout="rows"):
    torch = _torch()
    w = d * bits // 32
    if layout == "blocked":
        idx = torch.empty(((n + 31) // 32, d * bits), dtype=torch.int32, device=device)
        norms = torch.empty((n,), dtype=torch.float32, device=device)
        return Packed(d, bits, mode, n, idx, norms, layout="blocked")
    idx = torch.empty((n, w), dtype=torch.int32, device=device)
    norms = torch.empty((n,), dtype=torch.float32, device=device)
    qjl = rn = None
    if mode == "prod":
        qjl = torch.empty((n, d // 32), dtype=torch.int32, device=device)
        rn = torch.empty((n,), dtype=torch.float32, device=device)
    return Packed(d, bits, mode, n, idx, norms, qjl, rn)


def _dtype_code(x):
    torch = _torch()
    if x.dtype == torch.bfloat16:
        return DTYPE_BF16
    if x.dtype == torch.float32:
        return DTYPE_F32
    raise TQError(3, f"unsupported dtype {x.dtype}")


def encode_workspace(n, d, b, mode):
    return int(lib().tq_encode_workspace(n, d, b, MODE[mode]))


def encode(x, b, mode, cb, rot, qjl=None, out=None, layout="rows", ws=None):
    """Encode rows of x [n, d] (bf16 or fp32, contiguous, on the GPU) with b total bits.
    ws: optional uint8 device workspace (prod at d != 128 needs one; allocated if absent)."""
    torch = _torch()
    n, d = x.shape
    stage = b - 1 if mode == "prod" else b
    if out is None:
        out = alloc_packed(n, d, stage, mode, device=x.device, layout=layout)
    need = encode_workspace(n, d, b, mode)
    if ws is None and need > 0:
        ws = torch.empty((need,), dtype=torch.uint8, device=x.device)
    desc = out.descriptor()
    check(lib().tq_encode(_dptr(x), _dtype_code(x), n, d, b, MODE[mode], cb.ptr, rot.ptr,
                          qjl.ptr if qjl is not None else None, ctypes.byref(desc), _dptr(ws),
                          ws.numel() * ws.element_size() if ws is not None else 0, _stream()))
    return out


def rotate(x, rot):
    """(y_unit [n, d] fp32, norms [n] fp32) as formed inside the encode kernel."""
    torch = _torch()
    n, d = x.shape
    y = torch.empty((n, d), dtype=torch.float32, device=x.device)
    nr = torch.empty((n,), dtype=torch.float32, device=x.device)
    check(lib().tq_rotate(_dptr(x), _dtype_code(x), n, d, rot.ptr, _dptr(y), _dptr(nr), _stream()))
    return y, nr


def quantize_rotated(y, cb):
    torch = _torch()
    n, d = y.shape
    out = torch.empty((n, d * cb.b // 32), dtype=torch.int32, device=y.device)
    check(lib().tq_quantize_rotated(_dptr(y), n, d, cb.ptr, _dptr(out), _stream()))
    return out


def decode(p, cb, rot, qjl=None):
    torch = _torch()
    out = torch.empty((p.n, p.d), dtype=torch.float32, device=p.norms.device)
    desc = p.descriptor()
    check(lib().tq_decode(ctypes.byref(desc), cb.ptr, rot.ptr, qjl.ptr if qjl is not None else None,
                          _dptr(out), _stream()))
    return out


def scores_workspace(B, Hq, d):
    return int(lib().tq_scores_workspace(B, Hq, d))


def scores(q, K, Hkv, cb, rot, qjl=None, out=None, ws=None):
    """Raw scores [B, Hq, T] of q [B, Hq, d] fp32 against packed keys K laid out [B, Hkv, T]."""
    torch = _torch()
    B, Hq, d = q.shape
    T = K.n // max(B * Hkv, 1)
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    nbytes = scores_workspace(B, Hq, d)
    if ws is None:
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=q.device)
    desc = K.descriptor()
    check(lib().tq_scores(_dptr(q), B, Hq, Hkv, T, ctypes.byref(desc), cb.ptr, rot.ptr,
                          qjl.ptr if qjl is not None else None, _dptr(out), _dptr(ws),
                          ws.numel() * ws.element_size(), _stream()))
    return out


def scores_noalloc(q, K, Hkv, cb, rot, qjl=None, out=None):
    """tq_scores with the query workspace in the library's static device scratch (no allocation
    inside the call; `out` is allocated here only when not given).  Calls that overlap on one GPU
    race on that scratch."""
    torch = _torch()
    B, Hq, d = q.shape
    T = K.n // max(B * Hkv, 1)
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    desc = K.descriptor()
    check(lib().tq_scores_noalloc(_dptr(q), B, Hq, Hkv, T, ctypes.byref(desc), cb.ptr, rot.ptr,
                                  qjl.ptr if qjl is not None else None, _dptr(out), _stream()))
    return out


def prepare_queries(q, Hkv, rot, qjl=None, ws=None):
    """Query prologue of the score path into a workspace (returned): q [B, Hq, d] fp32."""
    torch = _torch()
    B, Hq, d = q.shape
    if ws is None:
        ws = torch.empty((max(scores_workspace(B, Hq, d), 1),), dtype=torch.uint8, device=q.device)
    check(lib().tq_prepare_queries(_dptr(q), B, Hq, Hkv, rot.ptr, qjl.ptr if qjl is not None else None, _dptr(ws),
                                   ws.numel() * ws.element_size(), _stream()))
    return ws


def scores_prepared(ws, B, Hq, K, Hkv, cb, out=None):
    """Scores [B, Hq, T] from a workspace filled by prepare_queries."""
    torch = _torch()
    T = K.n // max(B * Hkv, 1)
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=ws.device)
    desc = K.descriptor()
    check(lib().tq_scores_prepared(_dptr(ws), ws.numel() * ws.element_size(), B, Hq, Hkv, T, ctypes.byref(desc),
                                   cb.ptr, _dptr(out), _stream()))
    return out


def decode_attn_workspace(B, Hq, Hkv, T, d):
    return int(lib().tq_decode_attn_workspace(B, Hq, Hkv, T, d))


def decode_attn(q, K, V, Hkv, cb_k, cb_v, rot_k, rot_v, scale=None, out=None, ws=None):
    """softmax(scale <q, k_hat>) v_hat for q [B, Hq, d] fp32; K rows-layout, V blocked-layout at
    d = 128 (rows-layout at d = 64 or 256), both laid out [B, Hkv, T]."""
    torch = _torch()
    B, Hq, d = q.shape
    T = K.n // max(B * Hkv, 1)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    nbytes = decode_attn_workspace(B, Hq, Hkv, T, d)
    if ws is None:
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=q.device)
    kd, vd = K.descriptor(), V.descriptor()
    check(lib().tq_decode_attn(_dptr(q), B, Hq, Hkv, T, ctypes.byref(kd), ctypes.byref(vd), cb_k.ptr, cb_v.ptr,
                               rot_k.ptr, rot_v.ptr, ctypes.c_float(scale), _dptr(out), _dptr(ws),
                               ws.numel() * ws.element_size(), _stream()))
    return out


class KVCache:
    """A preallocated compressed cache of B*H sequences of capacity t_cap tokens (sequence
    b*H + h owns rows [(b*H + h) t_cap, (b*H + h + 1) t_cap) of `packed`)."""

    def __init__(self, B, H, t_cap, b, mode, packed):
        self.B, self.H, self.t_cap, self.b, self.mode, self.packed = B, H, t_cap, b, mode, packed


def alloc_cache(B, H, t_cap, d, b, mode="mse", layout="rows", device="cuda"):
    """Caller-owned cache storage (uninitialised): keys in the rows layout (MSE or prod), values
    in the token-blocked layout (MSE, t_cap a multiple of 32).  b is the total bit budget."""
    stage = b - 1 if mode == "prod" else b
    return KVCache(B, H, t_cap, b, mode, alloc_packed(B * H * t_cap, d, stage, mode, device=device, layout=layout))


def cache_append(cache, x, pos, cb, rot, qjl=None):
    """Encodes x [B, H, n_new, d] (bf16 or fp32, contiguous) into positions pos .. pos+n_new-1 of
    every sequence of the cache."""
    B, H, n_new, d = x.shape
    desc = cache.packed.descriptor()
    check(lib().tq_cache_append(_dptr(x), _dtype_code(x), B, H, n_new, pos, cache.t_cap, cache.b, MODE[cache.mode],
                                cb.ptr, rot.ptr, qjl.ptr if qjl is not None else None, ctypes.byref(desc),
                                _stream()))


def kv_append(kc, vc, k, v, pos, cb_k, cb_v, rot_k, rot_v):
    """Appends keys k and values v [B, H, n_new, d] (same dtype, contiguous) at position pos of a
    key cache (rows, MSE) and a value cache (token-blocked, MSE) in one call."""
    B, H, n_new, d = k.shape
    if v.shape != k.shape or v.dtype != k.dtype:
        raise TQError(2, "keys and values must have the same shape and dtype")
    kd, vd = kc.packed.descriptor(), vc.packed.descriptor()
    check(lib().tq_kv_append(_dptr(k), _dptr(v), _dtype_code(k), B, H, n_new, pos, kc.t_cap, kc.b, vc.b, cb_k.ptr,
                             cb_v.ptr, rot_k.ptr, rot_v.ptr, ctypes.byref(kd), ctypes.byref(vd), _stream()))


def scores_cache(q, cache, T, cb, rot, qjl=None, out=None, ws=None):
    """Raw scores [B, Hq, T] of q [B, Hq, d] against the first T keys of every sequence."""
    torch = _torch()
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty((max(scores_workspace(B, Hq, d), 1),), dtype=torch.uint8, device=q.device)
    desc = cache.packed.descriptor()
    check(lib().tq_scores_cache(_dptr(q), B, Hq, cache.H, T, cache.t_cap, ctypes.byref(desc), cb.ptr, rot.ptr,
                                qjl.ptr if qjl is not None else None, _dptr(out), _dptr(ws),
                                ws.numel() * ws.element_size(), _stream()))
    return out


def decode_attn_cache(q, kc, vc, T, cb_k, cb_v, rot_k, rot_v, scale=None, out=None, ws=None):
    """Decode attention of q [B, Hq, d] over the first T tokens of a key cache and a value cache."""
    torch = _torch()
    B, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty((max(decode_attn_workspace(B, Hq, kc.H, kc.t_cap, d), 1),), dtype=torch.uint8,
                         device=q.device)
    kd, vd = kc.packed.descriptor(), vc.packed.descriptor()
    check(lib().tq_decode_attn_cache(_dptr(q), B, Hq, kc.H, T, kc.t_cap, ctypes.byref(kd), ctypes.byref(vd), cb_k.ptr,
                                     cb_v.ptr, rot_k.ptr, rot_v.ptr, ctypes.c_float(scale), _dptr(out), _dptr(ws),
                                     ws.numel() * ws.element_size(), _stream()))
    return out



def _same_device(fn, *ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise TQError(1, f"{fn}: tensors on different devices {sorted(map(str, devs))}")


def _check_split_keys_x(fn, x):
    """Keys for the split entry points: contiguous [B, H, T, 128] bf16 or fp32 (the C functions
    take no d and read 128 values per key)."""
    torch = _torch()
    if x.dim() != 4 or x.shape[3] != 128:
        raise TQError(2, f"{fn}: x must be [B, H, T, 128], got {list(x.shape)}")
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TQError(3, f"{fn}: x must be bf16 or fp32, got {x.dtype}")
    if not x.is_contiguous():
        raise TQError(1, f"{fn}: x must be contiguous")


def _check_split_q(fn, q):
    """Queries for the split score entry points: contiguous fp32 [B, Hq, 128]."""
    torch = _torch()
    if q.dim() != 3 or q.shape[2] != 128:
        raise TQError(2, f"{fn}: q must be [B, Hq, 128], got {list(q.shape)}")
    if q.dtype != torch.float32:
        raise TQError(3, f"{fn}: q must be fp32, got {q.dtype}")
    if not q.is_contiguous():
        raise TQError(1, f"{fn}: q must be contiguous")


def _check_scores_out(fn, out, n):
    torch = _torch()
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != n:
        raise TQError(1, f"{fn}: out must be contiguous fp32 with {n} elements")

def prefill_attn_workspace(B, Hq, n_new, d=128):
    return int(lib().tq_prefill_attn_workspace(B, Hq, n_new, d))


def prefill_attn(q, kc, vc, k, v, pos, cb_k, cb_v, rot_k, rot_v, scale=None, out=None, ws=None):
    """Appends keys k and values v [B, Hkv, n_new, d] (same dtype, contiguous) at position pos of
    the key cache kc (rows, MSE) and value cache vc (token-blocked, MSE), then returns the causal
    attention [B, Hq, n_new, d] fp32 of the chunk's queries q [B, Hq, n_new, d] over the cache."""
    torch = _torch()
    B, Hq, n_new, d = q.shape
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4 or k.shape[2] != n_new:
        raise TQError(2, "prefill_attn: k and v must be [B, Hkv, n_new, d] of one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise TQError(1, "prefill_attn: q, k and v must be contiguous")
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if out is None:
        out = torch.empty((B, Hq, n_new, d), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty((max(prefill_attn_workspace(B, Hq, n_new, d), 1),), dtype=torch.uint8, device=q.device)
    kd, vd = kc.packed.descriptor(), vc.packed.descriptor()
    check(lib().tq_prefill_attn(_dptr(q), _dptr(k), _dptr(v), _dtype_code(k), B, Hq, Hkv, n_new, pos, kc.t_cap,
                                cb_k.ptr, cb_v.ptr, rot_k.ptr, rot_v.ptr, ctypes.byref(kd), ctypes.byref(vd),
                                ctypes.c_float(scale), _dptr(out), _dptr(ws), ws.numel() * ws.element_size(),
                                _stream()))
    return out


class Split(_Handle):
    """Per-KV-head channel split of d = 128 keys: 64 outlier channels, then the rest."""
    _free = "tq_split_free"

    def __init__(self, ptr, outliers):
        super().__init__(ptr)
        self.outliers = outliers
        self.H = outliers.shape[0]


def make_split(outliers):
    """outliers: [H, 64] integer channels (distinct per row, in [0, 128))."""
    o = np.ascontiguousarray(np.asarray(outliers), dtype=np.int32)
    if o.ndim != 2:
        raise TQError(1, "outliers must be [H, 64]")
    h = ctypes.c_void_p()
    check(lib().tq_make_split(o.shape[0], 2 * o.shape[1], _np(o), ctypes.byref(h)))
    return Split(h.value, o)


def encode_split(x, split, cb_o, cb_r, rot_o, rot_r, out=None):
    """Split encode of keys x [B, H, T, 128] (bf16 or fp32): (outlier codes, rest codes), each a
    rows-layout MSE Packed with d = 64 and n = B*H*T."""
    _check_split_keys_x("encode_split", x)
    B, H, T, _ = x.shape
    n = B * H * T
    if out is None:
        out = (alloc_packed(n, 64, cb_o.b, "mse", device=x.device), alloc_packed(n, 64, cb_r.b, "mse", device=x.device))
    _same_device("encode_split", x, out[0].idx, out[0].norms, out[1].idx, out[1].norms)
    do, dr = out[0].descriptor(), out[1].descriptor()
    check(lib().tq_encode_split(_dptr(x), _dtype_code(x), B, H, T, split.ptr, cb_o.ptr, cb_r.ptr, rot_o.ptr,
                                rot_r.ptr, ctypes.byref(do), ctypes.byref(dr), _stream()))
    return out


def scores_split_workspace(B, Hq):
    return int(lib().tq_scores_split_workspace(B, Hq))


def scores_split(q, K, Hkv, split, cb_o, cb_r, rot_o, rot_r, out=None, ws=None):
    """Raw scores [B, Hq, T] of q [B, Hq, 128] fp32 against split codes K = (K_o, K_r) of keys
    [B, Hkv, T]."""
    torch = _torch()
    _check_split_q("scores_split", q)
    B, Hq, _ = q.shape
    T = K[0].n // max(B * Hkv, 1)
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check_scores_out("scores_split", out, B * Hq * T)
    if ws is None:
        ws = torch.empty((max(scores_split_workspace(B, Hq), 1),), dtype=torch.uint8, device=q.device)
    _same_device("scores_split", q, out, ws, K[0].idx, K[0].norms, K[1].idx, K[1].norms)
    do, dr = K[0].descriptor(), K[1].descriptor()
    check(lib().tq_scores_split(_dptr(q), B, Hq, Hkv, T, split.ptr, ctypes.byref(do), ctypes.byref(dr), cb_o.ptr,
                                cb_r.ptr, rot_o.ptr, rot_r.ptr, _dptr(out), _dptr(ws),
                                ws.numel() * ws.element_size(), _stream()))
    return out


class Outlier8(_Handle):
    """Per-KV-head outlier channels of d = 128 keys kept at 8 bits (4, 8 or 16 per head)."""
    _free = "tq_outlier8_free"

    def __init__(self, ptr, outliers):
        super().__init__(ptr)
        self.outliers = outliers
        self.H, self.n_o = outliers.shape


def make_outlier8(outliers):
    """outliers: [H, n_o] integer channels (distinct per row, in [0, 128); n_o 4, 8 or 16).  Slot k
    of a key's 8-bit part is the head's k-th smallest outlier channel."""
    o = np.ascontiguousarray(np.asarray(outliers), dtype=np.int32)
    if o.ndim != 2:
        raise TQError(1, "outliers must be [H, n_o]")
    h = ctypes.c_void_p()
    check(lib().tq_make_outlier8(o.shape[0], 128, o.shape[1], _np(o), ctypes.byref(h)))
    return Outlier8(h.value, np.sort(o, axis=1))


def encode_outlier8(x, o, cb, rot, out=None):
    """Outlier-8 encode of keys x [B, H, T, 128] (bf16 or fp32): (rest, q8, scale) with rest a
    rows-layout MSE Packed (d = 128, n = B*H*T), q8 int8 [n, n_o] and scale fp32 [n]."""
    torch = _torch()
    _check_split_keys_x("encode_outlier8", x)
    B, H, T, _ = x.shape
    n = B * H * T
    if out is None:
        out = (alloc_packed(n, 128, cb.b, "mse", device=x.device),
               torch.empty((n, o.n_o), dtype=torch.int8, device=x.device),
               torch.empty((n,), dtype=torch.float32, device=x.device))
    rest, q8, scale = out
    if q8.dtype != torch.int8 or not q8.is_contiguous() or q8.numel() != n * o.n_o:
        raise TQError(1, f"encode_outlier8: q8 must be contiguous int8 with {n * o.n_o} elements")
    _check_scores_out("encode_outlier8", scale, n)
    _same_device("encode_outlier8", x, rest.idx, rest.norms, q8, scale)
    d = rest.descriptor()
    check(lib().tq_encode_outlier8(_dptr(x), _dtype_code(x), B, H, T, o.ptr, cb.ptr, rot.ptr, ctypes.byref(d),
                                   _dptr(q8), _dptr(scale), _stream()))
    return out


def scores_outlier8_workspace(B, Hq):
    return int(lib().tq_scores_outlier8_workspace(B, Hq))


def scores_outlier8(q, K, Hkv, o, cb, rot, out=None, ws=None):
    """Raw scores [B, Hq, T] of q [B, Hq, 128] fp32 against outlier-8 keys K = (rest, q8, scale)
    of keys [B, Hkv, T]."""
    torch = _torch()
    _check_split_q("scores_outlier8", q)
    rest, q8, scale = K
    B, Hq, _ = q.shape
    T = rest.n // max(B * Hkv, 1)
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check_scores_out("scores_outlier8", out, B * Hq * T)
    if q8.dtype != torch.int8 or not q8.is_contiguous() or q8.numel() != rest.n * o.n_o:
        raise TQError(1, f"scores_outlier8: q8 must be contiguous int8 with {rest.n * o.n_o} elements")
    _check_scores_out("scores_outlier8", scale, rest.n)
    if ws is None:
        ws = torch.empty((max(scores_outlier8_workspace(B, Hq), 1),), dtype=torch.uint8, device=q.device)
    _same_device("scores_outlier8", q, out, ws, rest.idx, rest.norms, q8, scale)
    d = rest.descriptor()
    check(lib().tq_scores_outlier8(_dptr(q), B, Hq, Hkv, T, o.ptr, ctypes.byref(d), _dptr(q8), _dptr(scale), cb.ptr,
                                   rot.ptr, _dptr(out), _dptr(ws), ws.numel() * ws.element_size(), _stream()))
    return out


def decode_attn_outlier8_workspace(B, Hq, Hkv, T):
    return int(lib().tq_decode_attn_outlier8_workspace(B, Hq, Hkv, T))


def decode_attn_outlier8(q, K, V, Hkv, o, cb_k, cb_v, rot_k, rot_v, scale=None, out=None, ws=None):
    """softmax(scale <q, k_hat>) v_hat for q [B, Hq, 128] fp32 with outlier-8 keys K = (rest, q8,
    scale) and blocked-layout values V, both laid out [B, Hkv, T]."""
    torch = _torch()
    _check_split_q("decode_attn_outlier8", q)
    rest, q8, sc = K
    B, Hq, d = q.shape
    T = rest.n // max(B * Hkv, 1)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check_scores_out("decode_attn_outlier8", out, B * Hq * d)
    if q8.dtype != torch.int8 or not q8.is_contiguous() or q8.numel() != rest.n * o.n_o:
        raise TQError(1, f"decode_attn_outlier8: q8 must be contiguous int8 with {rest.n * o.n_o} elements")
    _check_scores_out("decode_attn_outlier8", sc, rest.n)
    if ws is None:
        ws = torch.empty((max(decode_attn_outlier8_workspace(B, Hq, Hkv, T), 1),), dtype=torch.uint8, device=q.device)
    _same_device("decode_attn_outlier8", q, out, ws, rest.idx, rest.norms, q8, sc, V.idx, V.norms)
    kd, vd = rest.descriptor(), V.descriptor()
    check(lib().tq_decode_attn_outlier8(_dptr(q), B, Hq, Hkv, T, o.ptr, ctypes.byref(kd), _dptr(q8), _dptr(sc),
                                        ctypes.byref(vd), cb_k.ptr, cb_v.ptr, rot_k.ptr, rot_v.ptr,
                                        ctypes.c_float(scale), _dptr(out), _dptr(ws), ws.numel() * ws.element_size(),
                                        _stream()))
    return out


def decode_attn_split_workspace(B, Hq, Hkv, T):
    return int(lib().tq_decode_attn_split_workspace(B, Hq, Hkv, T))


def decode_attn_split(q, K, V, Hkv, split, cb_o, cb_r, cb_v, rot_o, rot_r, rot_v, scale=None, out=None, ws=None):
    """softmax(scale <q, k_hat>) v_hat for q [B, Hq, 128] fp32 with split keys K = (K_o, K_r) and
    blocked-layout values V, both laid out [B, Hkv, T]."""
    torch = _torch()
    _check_split_q("decode_attn_split", q)
    B, Hq, d = q.shape
    T = K[0].n // max(B * Hkv, 1)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check_scores_out("decode_attn_split", out, B * Hq * d)
    if ws is None:
        ws = torch.empty((max(decode_attn_split_workspace(B, Hq, Hkv, T), 1),), dtype=torch.uint8, device=q.device)
    _same_device("decode_attn_split", q, out, ws, K[0].idx, K[0].norms, K[1].idx, K[1].norms, V.idx, V.norms)
    do, dr, dv = K[0].descriptor(), K[1].descriptor(), V.descriptor()
    check(lib().tq_decode_attn_split(_dptr(q), B, Hq, Hkv, T, split.ptr, ctypes.byref(do), ctypes.byref(dr),
                                     ctypes.byref(dv), cb_o.ptr, cb_r.ptr, cb_v.ptr, rot_o.ptr, rot_r.ptr, rot_v.ptr,
                                     ctypes.c_float(scale), _dptr(out), _dptr(ws), ws.numel() * ws.element_size(),
                                     _stream()))
    return out


def alloc_split_cache(B, H, t_cap, b_o, b_r, device="cuda"):
    """Split codes of capacity t_cap per sequence: (outlier codes, rest codes), each with
    B*H*t_cap rows (contents undefined until appended)."""
    n = B * H * t_cap
    return (alloc_packed(n, 64, b_o, "mse", device=device), alloc_packed(n, 64, b_r, "mse", device=device))


def cache_append_split(K, x, pos, t_cap, split, cb_o, cb_r, rot_o, rot_r):
    """Append keys x [B, H, n_new, 128] (bf16 or fp32) at row pos of every sequence of the split
    cache K = (K_o, K_r) of capacity t_cap."""
    _check_split_keys_x("cache_append_split", x)
    B, H, n_new, _ = x.shape
    _same_device("cache_append_split", x, K[0].idx, K[0].norms, K[1].idx, K[1].norms)
    do, dr = K[0].descriptor(), K[1].descriptor()
    check(lib().tq_cache_append_split(_dptr(x), _dtype_code(x), B, H, n_new, pos, t_cap, split.ptr, cb_o.ptr,
                                      cb_r.ptr, rot_o.ptr, rot_r.ptr, ctypes.byref(do), ctypes.byref(dr), _stream()))
    return K


def scores_split_cache(q, K, Hkv, T, t_cap, split, cb_o, cb_r, rot_o, rot_r, out=None, ws=None):
    """Raw scores [B, Hq, T] of q [B, Hq, 128] fp32 over the first T rows of every sequence of the
    split cache K = (K_o, K_r) of capacity t_cap."""
    torch = _torch()
    _check_split_q("scores_split_cache", q)
    B, Hq, _ = q.shape
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check_scores_out("scores_split_cache", out, B * Hq * T)
    if ws is None:
        ws = torch.empty((max(scores_split_workspace(B, Hq), 1),), dtype=torch.uint8, device=q.device)
    _same_device("scores_split_cache", q, out, ws, K[0].idx, K[0].norms, K[1].idx, K[1].norms)
    do, dr = K[0].descriptor(), K[1].descriptor()
    check(lib().tq_scores_split_cache(_dptr(q), B, Hq, Hkv, T, t_cap, split.ptr, ctypes.byref(do), ctypes.byref(dr),
                                      cb_o.ptr, cb_r.ptr, rot_o.ptr, rot_r.ptr, _dptr(out), _dptr(ws),
                                      ws.numel() * ws.element_size(), _stream()))
    return out


def search_workspace(nq, n, d, k):
    return int(lib().tq_search_workspace(nq, n, d, k))


def search_topk(q, db, k, cb, rot, qjl, ws=None, out=None):
    """Top-k maximum inner-product search of q [nq, d] fp32 against a prod database (rows
    layout): (scores [nq, k] fp32 descending, indices [nq, k] int64)."""
    torch = _torch()
    nq, d = q.shape
    if out is None:
        out = (torch.empty((nq, k), dtype=torch.float32, device=q.device),
               torch.empty((nq, k), dtype=torch.int64, device=q.device))
    need = search_workspace(nq, db.n, d, k)
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    desc = db.descriptor()
    check(lib().tq_search_topk(_dptr(q), nq, ctypes.byref(desc), cb.ptr, rot.ptr, qjl.ptr, k, _dptr(out[0]),
                               _dptr(out[1]), _dptr(ws), ws.numel() * ws.element_size(), _stream()))
    return out


_TIMED = {"encode": 0, "scores": 1}


def timer_arm(kernel="encode"):
    """Arm a kernel timer for the next launch on this thread of the d = 128 rows-layout encode
    kernel ("encode") or of the d = 128 score kernel ("scores"); returns its id (measurement
    helper: the events are attached to the kernel's own dispatch)."""
    t = int(lib().tq_timer_arm_kernel(_TIMED[kernel]))
    if t < 0:
        raise TQError(4, lib().tq_last_error().decode())
    return t


def timer_read(t):
    """Duration in ms of the kernel launched under timer t (waits for it)."""
    ms = ctypes.c_float()
    check(lib().tq_timer_read(int(t), ctypes.byref(ms)))
    return float(ms.value)


def timer_reset():
    lib().tq_timer_reset()


def peak_read(src, blocks, sink=None):
    """Measurement ceiling: a streaming read of the bytes of `src` (device tensor, size a multiple
    of 16) by `blocks` blocks of 256 threads."""
    nbytes = src.numel() * src.element_size()
    check(lib().tq_peak_read(_dptr(src), nbytes, int(blocks), _dptr(sink), _stream()))


def peak_copy(dst, src, blocks):
    """Measurement ceiling: a streaming copy of src into dst (same byte size, a multiple of 16)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise TQError(1, "peak_copy: dst and src differ in size")
    check(lib().tq_peak_copy(_dptr(dst), _dptr(src), nbytes, int(blocks), _stream()))


PEAK_MFMA_KINDS = {"bf16_16x16x32": (0, 8, 16384), "bf16_32x32x16": (1, 4, 32768),
                   "f16_16x16x32": (2, 8, 16384), "f16_32x32x16": (3, 4, 32768)}


def peak_mfma(kind, iters, blocks, out):
    """Measurement ceiling: independent MFMA chains, `out` a device fp32 tensor of blocks * 256
    elements.  Returns the flops the launch issues."""
    code, chains, per_inst = PEAK_MFMA_KINDS[kind]
    if out.numel() < blocks * 256:
        raise TQError(1, "peak_mfma: out needs blocks * 256 floats")
    check(lib().tq_peak_mfma(code, int(iters), int(blocks), _dptr(out), _stream()))
    return float(blocks) * 4 * iters * chains * per_inst
