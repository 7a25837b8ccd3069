"""ctypes declarations mirroring include/tq.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EHIP = 0, -1, -2, -3
TQ_F32, TQ_BF16 = 0, 1
TQ_BETA_HALF_D, TQ_GAUSS_1_OVER_D = 0, 1
TQ_FLAG_GAUSS_1_OVER_D, TQ_FLAG_TWO_SIDED = 1, 2
TQ_MAX_LAYERS = 256

# every symbol include/tq.h declares
EXPORTS = [
    "tq_last_error", "tq_version", "tq_codebook_init", "tq_codebook_init_density", "tq_signs",
    "tq_packed_row_bytes", "tq_rotate", "tq_encode", "tq_decode", "tq_append_row",
    "tq_attn_workspace_bytes", "tq_attn_decode", "tq_layer_bits_boundary",
    "tq_attn_decode_noalloc", "tq_cache_decode",
]
TQ_ATTN_NOALLOC_MAX_BYTES = 16 << 20


class TqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class TqCodebook(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("levels", ctypes.c_int32),
                ("density", ctypes.c_int32), ("centroids", ctypes.c_float * 16),
                ("boundaries", ctypes.c_float * 15), ("distortion_per_coord", ctypes.c_double)]


class TqCacheDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("window", ctypes.c_int32),
                ("bits_k", ctypes.c_int32), ("bits_v", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("flags", ctypes.c_uint32), ("head_dim", ctypes.c_void_p), ("k_packed", ctypes.c_void_p),
                ("k_norms", ctypes.c_void_p), ("v_packed", ctypes.c_void_p),
                ("v_norms", ctypes.c_void_p), ("layer_bits_k", ctypes.c_void_p),
                ("layer_bits_v", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libtq.so (built in-tree by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it first (python -c "
                              "'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(_LIB_PATH)
        P, i32, i64, u64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                ctypes.c_size_t)
        L.tq_last_error.restype = ctypes.c_char_p
        L.tq_last_error.argtypes = []
        L.tq_version.restype = ctypes.c_char_p
        L.tq_version.argtypes = []
        L.tq_codebook_init.argtypes = [i32, i32, P]
        L.tq_codebook_init_density.argtypes = [i32, i32, i32, P]
        L.tq_signs.argtypes = [i32, u64, P]
        L.tq_packed_row_bytes.argtypes = [i32, i32]
        L.tq_packed_row_bytes.restype = sz
        u32 = ctypes.c_uint32
        L.tq_rotate.argtypes = [P, i32, i64, i32, u64, u32, i32, P, P]
        L.tq_encode.argtypes = [P, P, i32, i64, i32, i32, i32, u64, u32, P, P, P, P, P]
        L.tq_decode.argtypes = [P, P, i64, i32, i32, u64, u32, P, P]
        L.tq_append_row.argtypes = [P, i32, P, P, i32, i64, P]
        L.tq_cache_decode.argtypes = [P, i32, i64, i64, P, P, P]
        L.tq_attn_workspace_bytes.argtypes = [P, i32, i32, i64, ctypes.c_float]
        L.tq_attn_workspace_bytes.restype = sz
        L.tq_attn_decode.argtypes = [P, i32, P, i32, i64, ctypes.c_float, ctypes.c_float, P, P, sz, P]
        L.tq_layer_bits_boundary.argtypes = [i32, i32, i32, i32, P]
        L.tq_attn_decode_noalloc.argtypes = [P, i32, P, i32, i64, ctypes.c_float, ctypes.c_float,
                                             P, P]
        for name in ("tq_codebook_init", "tq_codebook_init_density", "tq_signs", "tq_rotate",
                     "tq_encode", "tq_decode", "tq_append_row", "tq_attn_decode",
                     "tq_layer_bits_boundary", "tq_attn_decode_noalloc", "tq_cache_decode"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib
