"""ctypes binding of libtq.so (include/tq.h).  Argument marshalling only: every step of the
encode / score path runs in the library's HIP kernels.  Tensors are torch tensors on the current
HIP device; work is enqueued on torch's current stream."""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_ESHAPE, TQ_EUNSUPPORTED, TQ_ENOMEM, TQ_EDEVICE = range(6)
STATUS_NAMES = {0: "TQ_OK", 1: "TQ_EINVAL", 2: "TQ_ESHAPE", 3: "TQ_EUNSUPPORTED",
                4: "TQ_ENOMEM", 5: "TQ_EDEVICE"}
DENSITY = {"beta": 0, "gauss": 1}
ROT_KIND = {"dense": 0, "wht": 1, "block_wht": 2}
DTYPE_F32, DTYPE_BF16 = 0, 1
MODE = {"mse": 0, "prod": 1}
LAYOUT = {"rows": 0, "blocked": 1}


class TQError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class tq_packed(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("n", ctypes.c_int64),
                ("idx", ctypes.c_void_p), ("norms", ctypes.c_void_p),
                ("qjl", ctypes.c_void_p), ("rnorms", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); every symbol declared in include/tq.h
SIGNATURES = {
    "tq_abi_version": (_I, []),
    "tq_last_error": (ctypes.c_char_p, []),
    "tq_host_splitmix64": (_I, [_U64, _U64, _I64, _P]),
    "tq_host_gaussian": (_I, [_U64, _I64, _P]),
    "tq_host_codebook": (_I, [_I, _I, _I, _P, _P]),
    "tq_host_rotation": (_I, [_I, _U64, _I, _P]),
    "tq_host_qjl_matrix": (_I, [_I, _U64, _P]),
    "tq_codebook": (_I, [_I, _I, _I, ctypes.POINTER(_P)]),
    "tq_codebook_from_values": (_I, [_I, _I, _P, ctypes.POINTER(_P)]),
    "tq_codebook_values": (_I, [_P, _P, _P]),
    "tq_codebook_free": (None, [_P]),
    "tq_make_rotation": (_I, [_I, _U64, _I, ctypes.POINTER(_P)]),
    "tq_rotation_from_matrix": (_I, [_I, _P, ctypes.POINTER(_P)]),
    "tq_rotation_export": (_I, [_P, _P]),
    "tq_rotation_free": (None, [_P]),
    "tq_make_qjl": (_I, [_I, _U64, _P, ctypes.POINTER(_P)]),
    "tq_qjl_from_matrix": (_I, [_I, _P, _P, ctypes.POINTER(_P)]),
    "tq_qjl_free": (None, [_P]),
    "tq_packed_words": (_SZ, [_I, _I]),
    "tq_packed_idx_words": (_SZ, [_I64, _I, _I, _I]),
    "tq_decode_attn_workspace": (_SZ, [_I, _I, _I, _I64, _I]),
    "tq_decode_attn": (_I, [_P, _I, _I, _I, _I64, ctypes.POINTER(tq_packed), ctypes.POINTER(tq_packed), _P, _P,
                            _P, _P, ctypes.c_float, _P, _P, _SZ, _P]),
    "tq_encode": (_I, [_P, _I, _I64, _I, _I, _I, _P, _P, _P, ctypes.POINTER(tq_packed), _P, _SZ, _P]),
    "tq_encode_workspace": (_SZ, [_I64, _I, _I, _I]),
    "tq_search_workspace": (_SZ, [_I64, _I64, _I, _I]),
    "tq_search_topk": (_I, [_P, _I64, ctypes.POINTER(tq_packed), _P, _P, _P, _I, _P, _P, _P, _SZ, _P]),
    "tq_timer_arm": (_I, []),
    "tq_timer_read": (_I, [_I, ctypes.POINTER(ctypes.c_float)]),
    "tq_timer_reset": (None, []),
    "tq_timer_arm_kernel": (_I, [_I]),
    "tq_scores_noalloc": (_I, [_P, _I, _I, _I, _I64, ctypes.POINTER(tq_packed), _P, _P, _P, _P, _P]),
    "tq_scores_noalloc_max_bytes": (_SZ, []),
    "tq_prefill_attn_workspace": (_SZ, [_I, _I, _I64, _I]),
    "tq_prefill_attn": (_I, [_P, _P, _P, _I, _I, _I, _I, _I64, _I64, _I64, _P, _P, _P, _P, ctypes.POINTER(tq_packed),
                             ctypes.POINTER(tq_packed), ctypes.c_float, _P, _P, _SZ, _P]),
    "tq_peak_read": (_I, [_P, _SZ, _I, _P, _P]),
    "tq_peak_copy": (_I, [_P, _P, _SZ, _I, _P]),
    "tq_peak_mfma": (_I, [_I, _I, _I, _P, _P]),
    "tq_rotate": (_I, [_P, _I, _I64, _I, _P, _P, _P, _P]),
    "tq_quantize_rotated": (_I, [_P, _I64, _I, _P, _P, _P]),
    "tq_decode": (_I, [ctypes.POINTER(tq_packed), _P, _P, _P, _P, _P]),
    "tq_scores_workspace": (_SZ, [_I, _I, _I]),
    "tq_prepare_queries": (_I, [_P, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "tq_scores_prepared": (_I, [_P, _SZ, _I, _I, _I, _I64, ctypes.POINTER(tq_packed), _P, _P, _P]),
    "tq_scores": (_I, [_P, _I, _I, _I, _I64, ctypes.POINTER(tq_packed), _P, _P, _P, _P, _P, _SZ, _P]),
    "tq_kv_append": (_I, [_P, _P, _I, _I, _I, _I64, _I64, _I64, _I, _I, _P, _P, _P, _P, ctypes.POINTER(tq_packed),
                          ctypes.POINTER(tq_packed), _P]),
    "tq_cache_append": (_I, [_P, _I, _I, _I, _I64, _I64, _I64, _I, _I, _P, _P, _P, ctypes.POINTER(tq_packed), _P]),
    "tq_scores_cache": (_I, [_P, _I, _I, _I, _I64, _I64, ctypes.POINTER(tq_packed), _P, _P, _P, _P, _P, _SZ, _P]),
    "tq_decode_attn_cache": (_I, [_P, _I, _I, _I, _I64, _I64, ctypes.POINTER(tq_packed), ctypes.POINTER(tq_packed),
                                  _P, _P, _P, _P, ctypes.c_float, _P, _P, _SZ, _P]),
    "tq_make_split": (_I, [_I, _I, _P, ctypes.POINTER(_P)]),
    "tq_split_free": (None, [_P]),
    "tq_encode_split": (_I, [_P, _I, _I, _I, _I64, _P, _P, _P, _P, _P, ctypes.POINTER(tq_packed),
                             ctypes.POINTER(tq_packed), _P]),
    "tq_scores_split_workspace": (_SZ, [_I, _I]),
    "tq_cache_append_split": (_I, [_P, _I, _I, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P, ctypes.POINTER(tq_packed),
                                   ctypes.POINTER(tq_packed), _P]),
    "tq_scores_split_cache": (_I, [_P, _I, _I, _I, _I64, _I64, _P, ctypes.POINTER(tq_packed),
                                   ctypes.POINTER(tq_packed), _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "tq_scores_split": (_I, [_P, _I, _I, _I, _I64, _P, ctypes.POINTER(tq_packed), ctypes.POINTER(tq_packed), _P, _P,
                             _P, _P, _P, _P, _SZ, _P]),
    "tq_make_outlier8": (_I, [_I, _I, _I, _P, ctypes.POINTER(_P)]),
    "tq_outlier8_free": (None, [_P]),
    "tq_encode_outlier8": (_I, [_P, _I, _I, _I, _I64, _P, _P, _P, ctypes.POINTER(tq_packed), _P, _P, _P]),
    "tq_scores_outlier8_workspace": (_SZ, [_I, _I]),
    "tq_decode_attn_outlier8_workspace": (_SZ, [_I, _I, _I, _I64]),
    "tq_decode_attn_split_workspace": (_SZ, [_I, _I, _I, _I64]),
    "tq_decode_attn_split": (_I, [_P, _I, _I, _I, _I64, _P, ctypes.POINTER(tq_packed), ctypes.POINTER(tq_packed),
                                  ctypes.POINTER(tq_packed), _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _SZ, _P]),
    "tq_decode_attn_outlier8": (_I, [_P, _I, _I, _I, _I64, _P, ctypes.POINTER(tq_packed), _P, _P,
                                     ctypes.POINTER(tq_packed), _P, _P, _P, _P, ctypes.c_float, _P, _P, _SZ, _P]),
    "tq_scores_outlier8": (_I, [_P, _I, _I, _I, _I64, _P, ctypes.POINTER(tq_packed), _P, _P, _P, _P, _P, _P, _SZ,
                                _P]),
}

_lib = None


def lib():
    """The loaded library; raises if libtq.so has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m kv_cache_compression_turboquant_amd.build` "
                "(or __graft_entry__.build()).  There is no non-HIP fallback.")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status):
    if status != TQ_OK:
        msg = lib().tq_last_error().decode(errors="replace")
        raise TQError(status, msg)


def _ptr(arr):
    return ctypes.c_void_p(arr.ctypes.data)


# ---- host-only math ------------------------------------------------------------------

def host_splitmix64(seed, n, offset=0):
    out = np.empty(n, dtype=np.uint64)
    check(lib().tq_host_splitmix64(seed, offset, n, _ptr(out)))
    return out


def host_gaussian(seed, n):
    out = np.empty(n, dtype=np.float64)
    check(lib().tq_host_gaussian(seed, n, _ptr(out)))
    return out


def host_codebook(d, b, density="beta"):
    c = np.empty(1 << b, dtype=np.float64)
    t = np.empty((1 << b) - 1 if b > 0 else 1, dtype=np.float64)
    check(lib().tq_host_codebook(d, b, DENSITY[density], _ptr(c), _ptr(t)))
    return c, t


def host_rotation(d, seed, kind="dense"):
    r = np.empty((d, d), dtype=np.float64)
    check(lib().tq_host_rotation(d, seed, ROT_KIND[kind], _ptr(r)))
    return r


def host_qjl_matrix(d, seed):
    s = np.empty((d, d), dtype=np.float64)
    check(lib().tq_host_qjl_matrix(d, seed, _ptr(s)))
    return s
