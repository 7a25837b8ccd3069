"""TurboQuant KV-cache codec on AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of ``libtq.so`` (declared in include/tq.h).
The functions here only marshal arguments -- torch tensors supply device
memory and the current HIP stream -- and every step of the codec runs in the
library's HIP kernels.  There is no CPU fallback: if the library or a GPU is
missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import _abi
from ._abi import (TQ_ATTN_NOALLOC_MAX_BYTES, TQ_BETA_HALF_D, TQ_BF16, TQ_EHIP, TQ_EINVAL,
                   TQ_EUNSUPPORTED, TQ_F32,
                   TQ_FLAG_GAUSS_1_OVER_D, TQ_FLAG_TWO_SIDED, TQ_GAUSS_1_OVER_D, TQ_MAX_LAYERS,
                   TQ_OK, TqCodebook, TqError, lib, library_path)

__all__ = [
    "TqError", "TQCache", "lib", "library_path", "tq_codebook_init", "tq_signs",
    "tq_packed_row_bytes", "tq_rotate", "tq_encode", "tq_decode", "tq_append_row",
    "tq_cache_decode", "tq_attn_workspace_bytes", "tq_attn_decode", "tq_last_error", "tq_version",
    "tq_layer_bits_boundary", "tq_attn_decode_noalloc", "TQ_ATTN_NOALLOC_MAX_BYTES",
    "TQ_F32", "TQ_BF16", "TQ_BETA_HALF_D", "TQ_GAUSS_1_OVER_D", "TQ_OK", "TQ_EINVAL",
    "TQ_EUNSUPPORTED", "TQ_EHIP", "TQ_MAX_LAYERS", "TQ_FLAG_GAUSS_1_OVER_D", "TQ_FLAG_TWO_SIDED",
]

_DTYPES = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}


def _check(rc: int, fn: str):
    if rc != TQ_OK:
        raise TqError(rc, f"{fn}: {lib().tq_last_error().decode()}")


def _stream(stream=None) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def tq_last_error() -> str:
    return lib().tq_last_error().decode()


def tq_version() -> str:
    return lib().tq_version().decode()


def tq_codebook_init(d: int, bits: int, density: int = TQ_BETA_HALF_D) -> dict:
    cb = TqCodebook()
    _check(lib().tq_codebook_init_density(d, bits, density, ctypes.byref(cb)),
           "tq_codebook_init")
    L = cb.levels
    return {
        "d": cb.d, "bits": cb.bits, "levels": L, "density": cb.density,
        "centroids": np.array(cb.centroids[:L], np.float32),
        "boundaries": np.array(cb.boundaries[: L - 1], np.float32),
        "distortion_per_coord": cb.distortion_per_coord,
    }


def tq_signs(d: int, seed: int) -> np.ndarray:
    out = np.zeros(d, np.int8)
    _check(lib().tq_signs(d, ctypes.c_uint64(seed), out.ctypes.data_as(ctypes.c_void_p)),
           "tq_signs")
    return out


def tq_packed_row_bytes(d: int, bits: int) -> int:
    return int(lib().tq_packed_row_bytes(d, bits))


def tq_layer_bits_boundary(n_layers: int, bits_inner: int, bits_boundary: int,
                           n_boundary: int = -1) -> list:
    """Per-layer widths: the first and last n_boundary layers (default 2) at
    bits_boundary, the others at bits_inner."""
    out = (ctypes.c_int32 * max(n_layers, 1))()
    _check(lib().tq_layer_bits_boundary(n_layers, n_boundary, bits_inner, bits_boundary, out),
           "tq_layer_bits_boundary")
    return list(out[:n_layers])


def tq_rotate(x: torch.Tensor, seed: int, inverse: bool = False, out=None, stream=None,
              flags: int = 0):
    """Rotation only: out = H(D x)/sqrt(d) (or D H x / sqrt(d) when inverse);
    S2 H S1 and S1 H S2 with TQ_FLAG_TWO_SIDED."""
    d = x.shape[-1]
    n = x.numel() // d if d else 0
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _check_shape(out, x.shape, "out", "tq_rotate")
    _check(lib().tq_rotate(_dev(x, "x"), _DTYPES[x.dtype], n, d, ctypes.c_uint64(seed), flags,
                           1 if inverse else 0, _dev(out, "out", torch.float32), _stream(stream)),
           "tq_rotate")
    return out


def tq_encode(k: torch.Tensor | None, v: torch.Tensor | None, bits_k: int, bits_v: int,
              seed: int, k_packed=None, k_norms=None, v_packed=None, v_norms=None,
              stream=None, flags: int = 0):
    """Encode K and/or V rows ([..., d], fp32 or bf16) in one launch.
    Returns (k_packed, k_norms, v_packed, v_norms) with None for a missing side."""
    ref = k if k is not None else v
    if ref is None:
        raise ValueError("tq_encode: k and v are both None")
    d = ref.shape[-1]
    n = ref.numel() // d
    lead = ref.shape[:-1]
    if k is not None and v is not None and (k.shape != v.shape or k.dtype != v.dtype):
        raise ValueError("tq_encode: k and v must have the same shape and dtype")
    dt = _DTYPES[ref.dtype]
    args = []
    outs = []
    for x, bits, pk, nm in ((k, bits_k, k_packed, k_norms), (v, bits_v, v_packed, v_norms)):
        if x is None:
            args += [None, None, None]
            outs += [None, None]
            continue
        rb = tq_packed_row_bytes(d, bits)
        if pk is None:
            pk = torch.empty(*lead, rb, dtype=torch.uint8, device=x.device)
        if nm is None:
            nm = torch.empty(*lead, dtype=torch.float32, device=x.device)
        if pk.numel() != n * rb or nm.numel() != n:
            raise ValueError("tq_encode: output buffers have the wrong size")
        args += [_dev(x, "rows"), _dev(pk, "packed", torch.uint8), _dev(nm, "norms", torch.float32)]
        outs += [pk, nm]
    _check(lib().tq_encode(args[0], args[3], dt, n, d, bits_k, bits_v, ctypes.c_uint64(seed),
                           flags, args[1], args[2], args[4], args[5], _stream(stream)),
           "tq_encode")
    return tuple(outs)


def tq_decode(packed: torch.Tensor, norms: torch.Tensor, d: int, bits: int, seed: int,
              out=None, stream=None, flags: int = 0):
    n = norms.numel()
    rb = tq_packed_row_bytes(d, bits)
    if packed.numel() != n * rb:
        raise ValueError("tq_decode: packed size does not match norms")
    if out is None:
        out = torch.empty(*norms.shape, d, dtype=torch.float32, device=packed.device)
    if out.numel() != n * d:
        raise ValueError("tq_decode: out has the wrong size")
    _check(lib().tq_decode(_dev(packed, "packed", torch.uint8), _dev(norms, "norms", torch.float32),
                           n, d, bits, ctypes.c_uint64(seed), flags,
                           _dev(out, "out", torch.float32), _stream(stream)), "tq_decode")
    return out


class TQCache:
    """Ring-buffer compressed KV cache; buffers are torch device tensors.

    Per layer l: k_packed[l] uint8 [batch, n_kv, window, d_l*bk_l/8],
    k_norms[l] float32 [batch, n_kv, window] (likewise for V).  head_dim,
    bits_k and bits_v are one value for every layer or a list per layer.  The
    C descriptor holds host arrays of their device pointers."""

    def __init__(self, n_layers, batch, n_kv_heads, window, head_dim, bits_k, bits_v,
                 seed=42, device="cuda", flags=0):
        def per_layer(v, name):
            out = [v] * n_layers if isinstance(v, int) else list(v)
            if len(out) != n_layers:
                raise ValueError(f"{name} list must have n_layers entries")
            return out
        hd = per_layer(head_dim, "head_dim")
        self.n_layers, self.batch, self.n_kv_heads, self.window = n_layers, batch, n_kv_heads, window
        self.head_dim, self.bits_k, self.bits_v, self.seed = hd, bits_k, bits_v, seed
        self.layer_bits_k, self.layer_bits_v = per_layer(bits_k, "bits_k"), per_layer(bits_v, "bits_v")
        self._uniform = isinstance(bits_k, int) and isinstance(bits_v, int)
        self.flags = flags
        self.k_packed, self.k_norms, self.v_packed, self.v_norms = [], [], [], []
        for d, bk, bv in zip(hd, self.layer_bits_k, self.layer_bits_v):
            self.k_packed.append(torch.zeros(batch, n_kv_heads, window, tq_packed_row_bytes(d, bk),
                                             dtype=torch.uint8, device=device))
            self.v_packed.append(torch.zeros(batch, n_kv_heads, window, tq_packed_row_bytes(d, bv),
                                             dtype=torch.uint8, device=device))
            self.k_norms.append(torch.zeros(batch, n_kv_heads, window, dtype=torch.float32, device=device))
            self.v_norms.append(torch.zeros(batch, n_kv_heads, window, dtype=torch.float32, device=device))
        self._refresh()

    def _refresh(self):
        n = self.n_layers
        self._hd = (ctypes.c_int32 * n)(*self.head_dim)
        self._kp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in self.k_packed])
        self._kn = (ctypes.c_void_p * n)(*[t.data_ptr() for t in self.k_norms])
        self._vp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in self.v_packed])
        self._vn = (ctypes.c_void_p * n)(*[t.data_ptr() for t in self.v_norms])
        self._lbk = (ctypes.c_int32 * n)(*self.layer_bits_k)
        self._lbv = (ctypes.c_int32 * n)(*self.layer_bits_v)
        per = None if self._uniform else (ctypes.cast(self._lbk, ctypes.c_void_p),
                                          ctypes.cast(self._lbv, ctypes.c_void_p))
        self.desc = _abi.TqCacheDesc(
            n, self.batch, self.n_kv_heads, self.window, self.layer_bits_k[0],
            self.layer_bits_v[0], self.seed, self.flags, ctypes.cast(self._hd, ctypes.c_void_p),
            ctypes.cast(self._kp, ctypes.c_void_p), ctypes.cast(self._kn, ctypes.c_void_p),
            ctypes.cast(self._vp, ctypes.c_void_p), ctypes.cast(self._vn, ctypes.c_void_p),
            *(per if per else (None, None)))

    def layer_bits(self, layer: int):
        """(K width, V width) of a layer."""
        return self.layer_bits_k[layer], self.layer_bits_v[layer]


def _check_shape(t, shape, name, fn):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{fn}: {name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def tq_append_row(cache: TQCache, layer: int, k_new, v_new, pos: int, stream=None):
    """k_new / v_new: a list of per-layer tensors [batch, n_kv, d_l] (layer = -1)
    or one tensor (a single layer)."""
    fn = "tq_append_row"
    if layer < 0:
        if layer != -1:
            raise ValueError(f"{fn}: layer must be -1 (every layer) or a layer index")
        ks, vs = list(k_new), list(v_new)
        layers = range(cache.n_layers)
        if len(ks) != cache.n_layers or len(vs) != cache.n_layers:
            raise ValueError(f"{fn}: layer = -1 needs {cache.n_layers} K and V tensors "
                             f"(got {len(ks)} and {len(vs)})")
    else:
        if layer >= cache.n_layers:
            raise ValueError(f"{fn}: layer {layer} out of range (n_layers {cache.n_layers})")
        ks, vs = [k_new], [v_new]
        layers = [layer]
    for l, kt, vt in zip(layers, ks, vs):
        want = (cache.batch, cache.n_kv_heads, cache.head_dim[l])
        _check_shape(kt, want, f"k_new[{l}]", fn)
        _check_shape(vt, want, f"v_new[{l}]", fn)
    if ks[0].dtype not in _DTYPES:
        raise ValueError(f"{fn}: rows must be float32 or bfloat16")
    dt = _DTYPES[ks[0].dtype]
    for t in ks + vs:
        if t.dtype != ks[0].dtype:
            raise ValueError(f"{fn}: mixed dtypes")
    kp = (ctypes.c_void_p * len(ks))(*[_dev(t, "k_new").value for t in ks])
    vp = (ctypes.c_void_p * len(vs))(*[_dev(t, "v_new").value for t in vs])
    _check(lib().tq_append_row(ctypes.byref(cache.desc), layer, kp, vp, dt, pos, _stream(stream)),
           fn)


def tq_cache_decode(cache: TQCache, layer: int, start: int = 0, count: int | None = None,
                    k_out=None, v_out=None, sides: str = "kv", stream=None):
    """Decode ring slots [start, start + count) (default: the whole window) of
    one layer, or of every layer (layer = -1), to fp32.  k_out / v_out: a list
    of per-layer tensors [batch, n_kv, count, d_l] (layer = -1) or one tensor;
    allocated when None for the sides named in `sides`.  Returns (k_out, v_out)
    with None for a side not decoded."""
    fn = "tq_cache_decode"
    if count is None:
        count = cache.window - start
    if layer < 0:
        if layer != -1:
            raise ValueError(f"{fn}: layer must be -1 (every layer) or a layer index")
        layers = list(range(cache.n_layers))
    else:
        if layer >= cache.n_layers:
            raise ValueError(f"{fn}: layer {layer} out of range (n_layers {cache.n_layers})")
        layers = [layer]
    if start < 0 or count < 0 or start + count > cache.window:
        raise ValueError(f"{fn}: slots [{start}, {start + count}) outside [0, {cache.window})")

    def alloc(outs, want):
        if outs is not None or not want:
            return outs
        outs = [torch.empty(cache.batch, cache.n_kv_heads, count, cache.head_dim[l],
                            dtype=torch.float32, device=cache.k_packed[l].device) for l in layers]
        return outs if layer < 0 else outs[0]

    k_out = alloc(k_out, "k" in sides)
    v_out = alloc(v_out, "v" in sides)
    lists = []
    for outs, name in ((k_out, "k_out"), (v_out, "v_out")):
        if outs is None:
            lists.append(None)
            continue
        lst = list(outs) if layer < 0 else [outs]
        if len(lst) != len(layers):
            raise ValueError(f"{fn}: {name} needs {len(layers)} tensors (got {len(lst)})")
        for l, t in zip(layers, lst):
            _check_shape(t, (cache.batch, cache.n_kv_heads, count, cache.head_dim[l]),
                         f"{name}[{l}]", fn)
        lists.append(lst)
    arrays = [None if lst is None else (ctypes.c_void_p * len(lst))(
        *[_dev(t, name, torch.float32).value for t in lst])
        for lst, name in zip(lists, ("k_out", "v_out"))]
    _check(lib().tq_cache_decode(ctypes.byref(cache.desc), layer, start, count, arrays[0],
                                 arrays[1], _stream(stream)), fn)
    return k_out, v_out


def tq_attn_workspace_bytes(cache: TQCache, layer: int, n_q_heads: int, ctx_len: int,
                            sparse_v: float = 0.0) -> int:
    return int(lib().tq_attn_workspace_bytes(ctypes.byref(cache.desc), layer, n_q_heads, ctx_len,
                                             ctypes.c_float(sparse_v)))


def tq_attn_decode(cache: TQCache, layer: int, q: torch.Tensor, ctx_len: int, scale: float = 0.0,
                   out=None, workspace=None, stream=None, sparse_v: float = 0.0):
    """q: bf16 [batch, n_q_heads, d]; returns fp32 [batch, n_q_heads, d].
    sparse_v: the sparse-V gate threshold (0 = off)."""
    fn = "tq_attn_decode"
    if not 0 <= layer < cache.n_layers:
        raise ValueError(f"{fn}: layer {layer} out of range (n_layers {cache.n_layers})")
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError(f"{fn}: q must be a 3-D tensor [batch, n_q_heads, head_dim]")
    n_q = q.shape[1]
    _check_shape(q, (cache.batch, n_q, cache.head_dim[layer]), "q", fn)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check_shape(out, q.shape, "out", fn)
    ws = tq_attn_workspace_bytes(cache, layer, n_q, ctx_len, sparse_v)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    _check(lib().tq_attn_decode(ctypes.byref(cache.desc), layer, _dev(q, "q", torch.bfloat16), n_q,
                                ctx_len, ctypes.c_float(scale), ctypes.c_float(sparse_v),
                                _dev(out, "out", torch.float32),
                                _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                _stream(stream)), fn)
    return out


def tq_attn_decode_noalloc(cache: TQCache, layer: int, q: torch.Tensor, ctx_len: int,
                           out: torch.Tensor, scale: float = 0.0, stream=None,
                           sparse_v: float = 0.0):
    """tq_attn_decode without a workspace: the library's static device scratch
    (TQ_ATTN_NOALLOC_MAX_BYTES per GPU) takes its place, and nothing is
    allocated -- `out` (fp32 [batch, n_q_heads, d]) must be given.  Calls that
    overlap on one GPU share the scratch and race."""
    fn = "tq_attn_decode_noalloc"
    if not 0 <= layer < cache.n_layers:
        raise ValueError(f"{fn}: layer {layer} out of range (n_layers {cache.n_layers})")
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError(f"{fn}: q must be a 3-D tensor [batch, n_q_heads, head_dim]")
    n_q = q.shape[1]
    _check_shape(q, (cache.batch, n_q, cache.head_dim[layer]), "q", fn)
    _check_shape(out, q.shape, "out", fn)
    _check(lib().tq_attn_decode_noalloc(ctypes.byref(cache.desc), layer,
                                        _dev(q, "q", torch.bfloat16), n_q, ctx_len,
                                        ctypes.c_float(scale), ctypes.c_float(sparse_v),
                                        _dev(out, "out", torch.float32), _stream(stream)), fn)
    return out
