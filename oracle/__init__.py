"""Python access to the fp64 CPU oracle (``tq_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline leg may import this package; the library package never does.
Argument marshalling only -- every number is computed by the C oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BETA = 0
GAUSS = 1

_lib = None


def build() -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, u64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        L.orc_splitmix64_stream.argtypes = [u64, i32, P]
        L.orc_signs.argtypes = [u64, i32, P]
        L.orc_signs2.argtypes = [u64, i32, P, P]
        L.orc_fwht.argtypes = [P, i32]
        L.orc_rotate.argtypes = [P, i32, P, P, P]
        L.orc_unrotate.argtypes = [P, i32, P, P, P]
        L.orc_pack.argtypes = [P, i32, i32, P]
        L.orc_unpack.argtypes = [P, i32, i32, P]
        L.orc_codebook.argtypes = [i32, i32, i32, P, P, P]
        L.orc_codebook.restype = i32
        L.orc_sphere_mse.argtypes = [i32, i32, P, P]
        L.orc_sphere_mse.restype = f64
        L.orc_codebook_float.argtypes = [i32, i32, i32, P, P]
        L.orc_padded_dim.argtypes = [i32]
        L.orc_padded_dim.restype = i32
        L.orc_encode.argtypes = [P, i64, i32, i32, i32, i32, u64, P, P, P]
        L.orc_encode.restype = i32
        L.orc_decode.argtypes = [P, P, i64, i32, i32, i32, i32, u64, P]
        L.orc_decode.restype = i32
        L.orc_decode_f64.argtypes = [P, P, i64, i32, i32, i32, i32, u64, P]
        L.orc_decode_f64.restype = i32
        L.orc_attention.argtypes = [P, i32, P, P, P, P, i32, i32, i32, i32, i32,
                                    i32, i32, u64, f64, f64, P]
        L.orc_attention.restype = i32
        L.orc_attention_rotated.argtypes = [P, i32, P, P, P, P, i32, i32, i32,
                                            i32, i32, i32, i32, u64, f64, P]
        L.orc_attention_rotated.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def splitmix64_stream(seed: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.uint64)
    lib().orc_splitmix64_stream(seed, n, _p(out))
    return out


def signs(seed: int, d: int) -> np.ndarray:
    out = np.zeros(d, np.int8)
    lib().orc_signs(seed, d, _p(out))
    return out


def signs2(seed: int, d: int):
    """(s1, s2): the sign vectors before and after the butterfly."""
    s1 = np.zeros(d, np.int8)
    s2 = np.zeros(d, np.int8)
    lib().orc_signs2(seed, d, _p(s1), _p(s2))
    return s1, s2


def _rotation_signs(seed: int, d: int, two_sided: bool):
    if two_sided:
        return signs2(seed, d)
    return signs(seed, d), None


def fwht(x) -> np.ndarray:
    x = _c(x, np.float64).copy()
    lib().orc_fwht(_p(x), x.shape[-1])
    return x


def rotate(x, seed: int, two_sided: bool = False) -> np.ndarray:
    x = _c(x, np.float64)
    d = x.shape[-1]
    s, s2 = _rotation_signs(seed, d, two_sided)
    y = np.empty_like(x)
    for r in range(x.reshape(-1, d).shape[0]):
        lib().orc_rotate(_p(x.reshape(-1, d)[r]), d, _p(s), None if s2 is None else _p(s2),
                         _p(y.reshape(-1, d)[r]))
    return y


def unrotate(y, seed: int, two_sided: bool = False) -> np.ndarray:
    y = _c(y, np.float64)
    d = y.shape[-1]
    s, s2 = _rotation_signs(seed, d, two_sided)
    x = np.empty_like(y)
    for r in range(y.reshape(-1, d).shape[0]):
        lib().orc_unrotate(_p(y.reshape(-1, d)[r]), d, _p(s), None if s2 is None else _p(s2),
                           _p(x.reshape(-1, d)[r]))
    return x


def pack(idx, bits: int) -> np.ndarray:
    idx = _c(idx, np.uint8)
    n = idx.size
    out = np.zeros((n * bits + 7) // 8, np.uint8)
    lib().orc_pack(_p(idx), n, bits, _p(out))
    return out


def unpack(buf, n: int, bits: int) -> np.ndarray:
    buf = _c(buf, np.uint8)
    out = np.zeros(n, np.uint8)
    lib().orc_unpack(_p(buf), n, bits, _p(out))
    return out


def codebook(d: int, bits: int, density: int = BETA):
    """fp64 (centroids, boundaries, iterations) in unit-norm coordinates."""
    L = 1 << bits
    c = np.zeros(L, np.float64)
    b = np.zeros(max(L - 1, 1), np.float64)
    it = ctypes.c_int(0)
    rc = lib().orc_codebook(d, bits, density, _p(c), _p(b), ctypes.byref(it))
    if rc != 0:
        raise RuntimeError(f"orc_codebook({d},{bits},{density}) -> {rc}")
    return c, b[: L - 1], it.value


def sphere_mse(d, bits, c, b) -> float:
    c = _c(c, np.float64)
    b = _c(b, np.float64)
    return lib().orc_sphere_mse(d, bits, _p(c), _p(b))


def codebook_float(d: int, bits: int, density: int = BETA):
    L = 1 << bits
    cf = np.zeros(L, np.float32)
    bf = np.zeros(max(L - 1, 1), np.float32)
    if lib().orc_codebook_float(d, bits, density, _p(cf), _p(bf)) != 0:
        raise RuntimeError("orc_codebook_float failed")
    return cf, bf[: L - 1]


def padded_dim(d: int) -> int:
    """The length rows of d coordinates are rotated and stored at."""
    return int(lib().orc_padded_dim(d))


def encode(x, d: int, bits: int, seed: int, density: int = BETA, want_u=False,
           two_sided: bool = False):
    """x: float32 [n, d] (bf16 callers convert exactly first).  With
    dp = padded_dim(d): returns packed uint8 [n, dp*bits/8], norms float32 [n]
    (and u fp64 [n, dp])."""
    x = _c(x, np.float32).reshape(-1, d)
    n = x.shape[0]
    dp = padded_dim(d)
    packed = np.zeros((n, dp * bits // 8), np.uint8)
    norms = np.zeros(n, np.float32)
    u = np.zeros((n, dp), np.float64) if want_u else None
    rc = lib().orc_encode(_p(x), n, d, bits, density, int(two_sided), seed, _p(packed), _p(norms),
                          _p(u) if want_u else None)
    if rc != 0:
        raise RuntimeError(f"orc_encode -> {rc}")
    return (packed, norms, u) if want_u else (packed, norms)


def decode(packed, norms, d: int, bits: int, seed: int, density: int = BETA,
           f64: bool = False, two_sided: bool = False):
    packed = _c(packed, np.uint8).reshape(-1, padded_dim(d) * bits // 8)
    norms = _c(norms, np.float32).reshape(-1)
    n = packed.shape[0]
    if f64:
        out = np.zeros((n, d), np.float64)
        rc = lib().orc_decode_f64(_p(packed), _p(norms), n, d, bits, density, int(two_sided),
                                  seed, _p(out))
    else:
        out = np.zeros((n, d), np.float32)
        rc = lib().orc_decode(_p(packed), _p(norms), n, d, bits, density, int(two_sided),
                              seed, _p(out))
    if rc != 0:
        raise RuntimeError(f"orc_decode -> {rc}")
    return out


def attention(q, k_packed, k_norms, v_packed, v_norms, n_kv, T, d, bits_k, bits_v,
              seed, scale, density=BETA, sparse_v_threshold=0.0, rotated=False,
              two_sided=False):
    """One sequence: q [n_q, d] float32; cache rows [n_kv, T]. Returns fp64 [n_q, d]."""
    q = _c(q, np.float32).reshape(-1, d)
    n_q = q.shape[0]
    kp = _c(k_packed, np.uint8)
    kn = _c(k_norms, np.float32)
    vp = _c(v_packed, np.uint8)
    vn = _c(v_norms, np.float32)
    dp = padded_dim(d)
    assert kp.size == n_kv * T * dp * bits_k // 8 and vp.size == n_kv * T * dp * bits_v // 8
    assert kn.size == n_kv * T and vn.size == n_kv * T
    out = np.zeros((n_q, d), np.float64)
    if rotated:
        rc = lib().orc_attention_rotated(_p(q), n_q, _p(kp), _p(kn), _p(vp), _p(vn), n_kv,
                                         T, d, bits_k, bits_v, density, int(two_sided), seed,
                                         scale, _p(out))
    else:
        rc = lib().orc_attention(_p(q), n_q, _p(kp), _p(kn), _p(vp), _p(vn), n_kv, T, d,
                                 bits_k, bits_v, density, int(two_sided), seed, scale,
                                 sparse_v_threshold, _p(out))
    if rc != 0:
        raise RuntimeError(f"orc_attention -> {rc}")
    return out
