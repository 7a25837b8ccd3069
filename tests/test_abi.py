"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
its host-side pieces agree with the oracle, and argument validation and the
HIP-error path behave as the header states.  No kernel is launched."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tq():
    import kv_cache_vector_rotate_amd as tq
    tq.lib()
    return tq


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(tq):
    names = _declared_functions()
    assert "tq_encode" in names and "tq_attn_decode" in names
    L = ctypes.CDLL(tq.library_path())
    for n in names:
        assert hasattr(L, n), n
    from kv_cache_vector_rotate_amd import _abi
    assert sorted(_abi.EXPORTS) == names


def test_version_and_row_bytes(tq):
    assert "gfx950" in tq.tq_version()
    for d in (64, 128, 256):
        for b in (2, 3, 4):
            assert tq.tq_packed_row_bytes(d, b) == d * b // 8
    # a head_dim that is not a power of two is stored at the next one
    assert tq.tq_packed_row_bytes(96, 3) == 48 and tq.tq_packed_row_bytes(160, 4) == 128
    assert tq.tq_packed_row_bytes(100, 2) == 32 and tq.tq_packed_row_bytes((1 << 20) + 1, 4) == 0
    assert tq.tq_packed_row_bytes(0, 4) == 0 and tq.tq_packed_row_bytes(64, 9) == 0


@pytest.mark.parametrize("d", [2, 64, 128, 256, 1024])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_matches_oracle(tq, orc, d, bits):
    """Library (incomplete-beta continued fraction) vs oracle (quadrature):
    independent computations of the same Lloyd-Max fixed point; float tables
    equal or at most 1 ulp apart."""
    cb = tq.tq_codebook_init(d, bits)
    cf, bf = orc.codebook_float(d, bits)
    assert cb["levels"] == 1 << bits
    for a, b in ((cb["centroids"], cf), (cb["boundaries"], bf)):
        ua = a.view(np.int32).astype(np.int64)
        ub = b.view(np.int32).astype(np.int64)
        assert np.all(np.abs(ua - ub) <= 1), (a, b)
    assert cb["boundaries"][(1 << bits) // 2 - 1] == 0.0
    # distortion: E[X^2] - sum P c^2 under the Beta density; compare with a
    # direct quadrature of the squared error (scipy)
    import scipy.integrate
    import scipy.stats
    if d >= 4:
        a = d / 2
        c = cb["centroids"].astype(np.float64)
        edges = np.concatenate([[-1.0], cb["boundaries"].astype(np.float64), [1.0]])
        f = lambda x: scipy.stats.beta.pdf((x + 1) / 2, a, a) / 2
        tot = sum(scipy.integrate.quad(lambda x: (x - c[j]) ** 2 * f(x), edges[j], edges[j + 1],
                                       epsabs=1e-15, limit=200)[0] for j in range(len(c)))
        assert abs(cb["distortion_per_coord"] - tot) < 1e-9 + 1e-6 * tot


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_density_codebook(tq, orc, bits):
    cb = tq.tq_codebook_init(128, bits, tq.TQ_GAUSS_1_OVER_D)
    cf, _ = orc.codebook_float(128, bits, orc.GAUSS)
    assert np.all(np.abs(cb["centroids"].view(np.int32).astype(np.int64)
                         - cf.view(np.int32).astype(np.int64)) <= 1)


def test_signs_match_oracle(tq, orc):
    for seed in (0, 1, 42, 2 ** 63 + 5):
        assert np.array_equal(tq.tq_signs(256, seed), orc.signs(seed, 256))
    assert np.array_equal(tq.tq_signs(64, 42), orc.signs(42, 256)[:64])


def test_codebook_and_sign_validation(tq):
    with pytest.raises(tq.TqError) as e:
        tq.tq_codebook_init(96, 3)
    assert e.value.status == tq.TQ_EINVAL and "power of two" in str(e.value)
    for d, b in ((1, 2), (128, 0), (128, 5), (1 << 21, 2)):
        with pytest.raises(tq.TqError):
            tq.tq_codebook_init(d, b)
    with pytest.raises(tq.TqError):
        tq.tq_codebook_init(128, 2, 7)
    L = tq.lib()
    assert L.tq_signs(0, 1, None) == tq.TQ_EINVAL


def _c(v):
    return ctypes.c_void_p(v)


def test_encode_decode_validation_without_launch(tq):
    """Every rejected argument is rejected before any HIP call (no GPU here)."""
    L = tq.lib()
    A = _c(4096)          # fake, 16-byte aligned pointers: never dereferenced
    N = _c(8192)
    assert L.tq_encode(None, None, 0, 10, 128, 4, 2, 42, 0, A, N, A, N, None) == tq.TQ_EINVAL
    assert "both" in tq.tq_last_error()
    assert L.tq_encode(A, None, 7, 10, 128, 4, 2, 42, 0, A, N, None, None, None) == tq.TQ_EINVAL
    assert L.tq_encode(A, None, 0, 10, 1, 4, 2, 42, 0, A, N, None, None, None) == tq.TQ_EINVAL
    assert L.tq_encode(A, None, 0, 10, 100, 4, 2, 42, 0, A, N, None, None, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_encode(A, None, 0, 10, 32, 4, 2, 42, 0, A, N, None, None, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_encode(A, None, 0, 10, 288, 4, 2, 42, 0, A, N, None, None, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_encode(A, None, 0, 10, 512, 4, 2, 42, 0, A, N, None, None, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_encode(A, None, 0, 10, 128, 1, 2, 42, 0, A, N, None, None, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_encode(A, None, 0, 10, 128, 5, 2, 42, 0, A, N, None, None, None) == tq.TQ_EINVAL
    assert L.tq_encode(A, None, 0, -1, 128, 4, 2, 42, 0, A, N, None, None, None) == tq.TQ_EINVAL
    assert L.tq_encode(_c(4100), None, 0, 10, 128, 4, 2, 42, 0, A, N, None, None, None) == tq.TQ_EINVAL
    assert "aligned" in tq.tq_last_error()
    assert L.tq_encode(A, None, 0, 10, 128, 4, 2, 42, 0, None, N, None, None, None) == tq.TQ_EINVAL
    # n_rows == 0 succeeds and launches nothing, NULL buffers included
    assert L.tq_encode(A, A, 1, 0, 128, 4, 2, 42, 0, A, N, A, N, None) == tq.TQ_OK
    assert L.tq_encode(None, None, 1, 0, 128, 4, 2, 42, 0, None, None, None, None, None) == tq.TQ_OK
    assert L.tq_decode(A, N, 0, 128, 4, 42, 0, A, None) == tq.TQ_OK
    assert L.tq_decode(A, N, 5, 128, 1, 42, 0, A, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_decode(None, N, 5, 128, 4, 42, 0, A, None) == tq.TQ_EINVAL
    assert L.tq_rotate(A, 0, 0, 128, 42, 0, 0, A, None) == tq.TQ_OK
    assert L.tq_rotate(A, 0, 3, 1, 42, 0, 0, A, None) == tq.TQ_EINVAL
    assert L.tq_rotate(A, 0, 3, 96, 42, 0, 0, A, None) == tq.TQ_EUNSUPPORTED   # codec calls only
    # padded head_dims pass validation (n_rows = 0: nothing launched)
    for d in (96, 160, 192, 224):
        assert L.tq_encode(A, None, 0, 0, d, 4, 2, 42, 0, A, N, None, None, None) == tq.TQ_OK
        assert L.tq_decode(A, N, 0, d, 3, 42, 0, A, None) == tq.TQ_OK
    # option bits: the two known ones pass validation, any other is rejected
    for fn, args in (("tq_encode", lambda f: (A, None, 0, 0, 128, 4, 2, 42, f, A, N, None, None,
                                              None)),
                     ("tq_decode", lambda f: (A, N, 0, 128, 4, 42, f, A, None)),
                     ("tq_rotate", lambda f: (A, 0, 0, 128, 42, f, 0, A, None))):
        for f in (0, 1, 2, 3):
            assert getattr(L, fn)(*args(f)) == tq.TQ_OK
        for f in (4, 8, 0x80000000):
            assert getattr(L, fn)(*args(f)) == tq.TQ_EINVAL
            assert "flag" in tq.tq_last_error()


def _desc(tq, n_layers=2, batch=2, n_kv=2, window=8, head_dim=128, bk=4, bv=2, flags=0,
          layer_bk=None, layer_bv=None):
    from kv_cache_vector_rotate_amd import _abi
    hd = (ctypes.c_int32 * n_layers)(*([head_dim] * n_layers))
    ptrs = [(ctypes.c_void_p * n_layers)(*([4096 * (i + 1)] * n_layers)) for i in range(4)]
    lb = [None if a is None else (ctypes.c_int32 * n_layers)(*a) for a in (layer_bk, layer_bv)]
    d = _abi.TqCacheDesc(n_layers, batch, n_kv, window, bk, bv, 42, flags,
                         ctypes.cast(hd, ctypes.c_void_p),
                         *[ctypes.cast(p, ctypes.c_void_p) for p in ptrs],
                         *[None if a is None else ctypes.cast(a, ctypes.c_void_p) for a in lb])
    d._keep = (hd, ptrs, lb)
    return d


def test_cache_and_attention_validation(tq):
    L = tq.lib()
    d = _desc(tq)
    A = _c(4096)
    arr = (ctypes.c_void_p * 2)(4096, 4096)
    assert L.tq_append_row(None, -1, arr, arr, 0, 0, None) == tq.TQ_EINVAL
    assert L.tq_append_row(ctypes.byref(d), 2, arr, arr, 0, 0, None) == tq.TQ_EINVAL
    assert L.tq_append_row(ctypes.byref(d), -1, arr, arr, 0, -1, None) == tq.TQ_EINVAL
    assert L.tq_attn_decode(ctypes.byref(d), 0, A, 3, 5, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_EINVAL
    assert "multiple" in tq.tq_last_error()
    assert L.tq_attn_decode(ctypes.byref(d), 0, A, 6, 5, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_attn_decode(ctypes.byref(d), 0, A, 4, 0, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_EINVAL
    assert L.tq_attn_decode(ctypes.byref(d), 0, A, 4, 5, 0.0, 0.0, A, A, 16, None) == tq.TQ_EINVAL
    assert "workspace" in tq.tq_last_error()
    ws = L.tq_attn_workspace_bytes(ctypes.byref(d), 0, 4, 5, 0.0)
    # 2 sequences x 4 query heads x 1 chunk x (128 + 4) floats
    assert ws == 2 * 4 * 1 * 132 * 4
    # with the sparse-V gate: + the chunk maxima (2 x 4 x 1 floats, padded to
    # 16 bytes) + every context row's scores (2 x 4 x 5 floats)
    assert L.tq_attn_workspace_bytes(ctypes.byref(d), 0, 4, 5, 1e-3) == ws + 32 + 2 * 4 * 5 * 4
    assert L.tq_attn_workspace_bytes(ctypes.byref(d), 5, 4, 5, 0.0) == 0
    for bad in (-0.1, 1.0, float("nan")):
        assert L.tq_attn_workspace_bytes(ctypes.byref(d), 0, 4, 5, bad) == 0
    for bad in (-0.1, 1.0, float("nan")):
        assert L.tq_attn_decode(ctypes.byref(d), 0, A, 4, 5, 0.0, bad, A, A, 1 << 20, None) == tq.TQ_EINVAL
    assert "sparse_v" in tq.tq_last_error()
    d2 = _desc(tq, head_dim=100)
    assert L.tq_attn_decode(ctypes.byref(d2), 0, A, 4, 5, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_EUNSUPPORTED
    d2 = _desc(tq, head_dim=1)
    assert L.tq_attn_decode(ctypes.byref(d2), 0, A, 4, 5, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_EINVAL
    d2 = _desc(tq, head_dim=96, batch=0)
    assert L.tq_attn_decode(ctypes.byref(d2), 0, A, 4, 5, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_OK
    # the workspace holds the padded length: 2 x 4 x 1 x (128 + 4) floats
    assert L.tq_attn_workspace_bytes(ctypes.byref(_desc(tq, head_dim=96)), 0, 4, 5, 0.0) == 2 * 4 * 132 * 4
    d3 = _desc(tq, bk=1)
    assert L.tq_attn_decode(ctypes.byref(d3), 0, A, 4, 5, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_EUNSUPPORTED
    d4 = _desc(tq, flags=4)
    assert L.tq_attn_decode(ctypes.byref(d4), 0, A, 4, 5, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_EINVAL
    assert "flag" in tq.tq_last_error()
    # one KV head's packed rows (window x head_dim / 2 bytes) must stay below 2 GiB
    d5 = _desc(tq, head_dim=256, window=1 << 24)
    assert L.tq_attn_decode(ctypes.byref(d5), 0, A, 4, 5, 0.0, 0.0, A, A, 1 << 30, None) == tq.TQ_EUNSUPPORTED
    assert "window" in tq.tq_last_error()
    assert L.tq_append_row(ctypes.byref(d4), -1, arr, arr, 0, 0, None) == tq.TQ_EINVAL
    assert "flag" in tq.tq_last_error()


def test_cache_decode_validation_without_launch(tq):
    """tq_cache_decode rejects bad descriptors, layers, slot ranges, widths and
    buffers before launching anything; empty requests succeed and launch
    nothing."""
    L = tq.lib()
    d = _desc(tq)                                   # 2 layers, window 8, K4/V2, d 128
    outs = (ctypes.c_void_p * 2)(8192, 8192)
    assert L.tq_cache_decode(None, -1, 0, 8, outs, outs, None) == tq.TQ_EINVAL
    for layer in (-2, 2):
        assert L.tq_cache_decode(ctypes.byref(d), layer, 0, 8, outs, outs, None) == tq.TQ_EINVAL
        assert "layer" in tq.tq_last_error()
    for start, count in ((-1, 4), (0, -1), (4, 5), (9, 0)):
        assert L.tq_cache_decode(ctypes.byref(d), -1, start, count, outs, outs, None) == tq.TQ_EINVAL
        assert "slots" in tq.tq_last_error()
    mis = (ctypes.c_void_p * 2)(8192 + 4, 8192)
    assert L.tq_cache_decode(ctypes.byref(d), -1, 0, 8, mis, None, None) == tq.TQ_EINVAL
    assert "misaligned" in tq.tq_last_error()
    assert L.tq_cache_decode(ctypes.byref(_desc(tq, bv=1)), -1, 0, 8, None, outs,
                             None) == tq.TQ_EUNSUPPORTED
    assert L.tq_cache_decode(ctypes.byref(_desc(tq, head_dim=100)), 0, 0, 8, outs, None,
                             None) == tq.TQ_EUNSUPPORTED
    assert L.tq_cache_decode(ctypes.byref(_desc(tq, flags=4)), 0, 0, 8, outs, None,
                             None) == tq.TQ_EINVAL
    # nothing to decode: no launch
    assert L.tq_cache_decode(ctypes.byref(d), -1, 3, 0, outs, outs, None) == tq.TQ_OK
    assert L.tq_cache_decode(ctypes.byref(d), -1, 0, 8, None, None, None) == tq.TQ_OK
    nulls = (ctypes.c_void_p * 2)(None, None)
    assert L.tq_cache_decode(ctypes.byref(d), -1, 0, 8, nulls, None, None) == tq.TQ_OK
    assert L.tq_cache_decode(ctypes.byref(_desc(tq, batch=0)), -1, 0, 8, outs, outs,
                             None) == tq.TQ_OK
    # the binding checks counts and shapes first
    cache = tq.TQCache(2, 2, 2, 8, [128, 64], 4, 2, device="cpu")
    with pytest.raises(ValueError, match="slots"):
        tq.tq_cache_decode(cache, -1, 4, 5)
    with pytest.raises(ValueError, match="2 tensors"):
        tq.tq_cache_decode(cache, -1, 0, 8, k_out=[torch.zeros(2, 2, 8, 128)])
    with pytest.raises(ValueError, match=r"k_out\[1\]"):
        tq.tq_cache_decode(cache, -1, 0, 8, k_out=[torch.zeros(2, 2, 8, 128)] * 2)
    with pytest.raises(ValueError, match=r"v_out\[0\]"):
        tq.tq_cache_decode(cache, 0, 2, 4, k_out=torch.zeros(2, 2, 4, 128),
                           v_out=torch.zeros(2, 2, 8, 128))


def test_binding_rejects_mismatched_shapes(tq):
    """The Python binding checks every tensor against the cache before any
    pointer reaches the library (host-only: CPU tensors, so a shape that
    passed would fail the device check instead, with another message)."""
    cache = tq.TQCache(3, 2, 2, 16, [128, 64, 128], 4, 2, device="cpu")
    bf = torch.bfloat16
    for q in (torch.zeros(1, 4, 128, dtype=bf),       # batch 1, cache batch 2
              torch.zeros(2, 4, 64, dtype=bf),        # head_dim of another layer
              torch.zeros(2, 4, 128, 1, dtype=bf),    # not 3-D
              torch.zeros(8, 128, dtype=bf)):
        with pytest.raises(ValueError, match="q"):
            tq.tq_attn_decode(cache, 0, q, 16)
    with pytest.raises(ValueError, match="out"):
        tq.tq_attn_decode(cache, 0, torch.zeros(2, 4, 128, dtype=bf), 16,
                          out=torch.zeros(2, 4, 64))
    with pytest.raises(ValueError, match="layer"):
        tq.tq_attn_decode(cache, 3, torch.zeros(2, 4, 128, dtype=bf), 16)
    rows = [torch.zeros(2, 2, d) for d in (128, 64, 128)]
    with pytest.raises(ValueError, match="3 K and V"):
        tq.tq_append_row(cache, -1, rows[:2], rows[:2], 0)
    with pytest.raises(ValueError, match="3 K and V"):
        tq.tq_append_row(cache, -1, rows, rows[:2], 0)
    with pytest.raises(ValueError, match=r"k_new\[1\]"):
        tq.tq_append_row(cache, -1, [rows[0], rows[0], rows[2]], rows, 0)
    with pytest.raises(ValueError, match=r"v_new\[0\]"):
        tq.tq_append_row(cache, 0, rows[0], torch.zeros(2, 3, 128), 0)
    with pytest.raises(ValueError, match="out of range"):
        tq.tq_append_row(cache, 3, rows[0], rows[0], 0)
    with pytest.raises(ValueError, match="device"):   # shapes pass, then the device check
        tq.tq_append_row(cache, 1, rows[1], rows[1], 0)
    with pytest.raises(ValueError, match="out"):
        tq.tq_rotate(torch.zeros(4, 128), 42, out=torch.zeros(4, 64))


def test_noalloc_validation_without_launch(tq):
    """tq_attn_decode_noalloc checks its arguments like tq_attn_decode and
    rejects a call whose workspace would exceed its static scratch before
    touching the device."""
    L = tq.lib()
    A = _c(4096)
    d = _desc(tq, window=1 << 20)
    assert L.tq_attn_workspace_bytes(ctypes.byref(d), 0, 4, 1 << 20, 1e-3) > tq.TQ_ATTN_NOALLOC_MAX_BYTES
    assert L.tq_attn_decode_noalloc(ctypes.byref(d), 0, A, 4, 1 << 20, 0.0, 1e-3, A, None) == tq.TQ_EINVAL
    assert "scratch" in tq.tq_last_error()
    assert L.tq_attn_decode_noalloc(ctypes.byref(d), 0, A, 4, 5, 0.0, 0.0, None, None) == tq.TQ_EINVAL
    assert "NULL" in tq.tq_last_error()
    assert L.tq_attn_decode_noalloc(ctypes.byref(d), 0, A, 3, 5, 0.0, 0.0, A, None) == tq.TQ_EINVAL
    assert L.tq_attn_decode_noalloc(ctypes.byref(d), 0, A, 4, 5, 0.0, 2.0, A, None) == tq.TQ_EINVAL
    assert L.tq_attn_decode_noalloc(ctypes.byref(_desc(tq, batch=0)), 0, A, 4, 5, 0.0, 0.0, A,
                                    None) == tq.TQ_OK


def test_layer_bits_boundary_policy(tq):
    assert tq.tq_layer_bits_boundary(10, 2, 4) == [4, 4, 2, 2, 2, 2, 2, 2, 4, 4]
    assert tq.tq_layer_bits_boundary(10, 3, 4, n_boundary=1) == [4] + [3] * 8 + [4]
    assert tq.tq_layer_bits_boundary(5, 2, 4, n_boundary=0) == [2] * 5
    assert tq.tq_layer_bits_boundary(3, 2, 4) == [4, 4, 4]       # boundaries overlap
    L = tq.lib()
    out = (ctypes.c_int32 * 4)()
    for args in ((0, 2, 2, 4), (tq.TQ_MAX_LAYERS + 1, 2, 2, 4), (4, 2, 0, 4), (4, 2, 2, 5)):
        assert L.tq_layer_bits_boundary(*args, out) == tq.TQ_EINVAL
    assert L.tq_layer_bits_boundary(4, 2, 2, 4, None) == tq.TQ_EINVAL


def test_per_layer_bits_validation(tq):
    """The descriptor's per-layer widths are what append and attention check
    (no launch: every case is rejected, or has no rows)."""
    L = tq.lib()
    A = _c(4096)
    arr = (ctypes.c_void_p * 2)(4096, 4096)
    # uniform widths invalid, per-layer widths valid: the arrays win
    d = _desc(tq, batch=0, bk=9, bv=9, layer_bk=[4, 3], layer_bv=[2, 2])
    assert L.tq_append_row(ctypes.byref(d), -1, arr, arr, 0, 0, None) == tq.TQ_OK
    d = _desc(tq, batch=0, layer_bk=[4, 5], layer_bv=[2, 2])
    assert L.tq_append_row(ctypes.byref(d), -1, arr, arr, 0, 0, None) == tq.TQ_EINVAL
    assert L.tq_append_row(ctypes.byref(d), 0, arr, arr, 0, 0, None) == tq.TQ_OK
    d = _desc(tq, batch=0, layer_bk=[4, 4], layer_bv=[2, 1])
    assert L.tq_append_row(ctypes.byref(d), 1, arr, arr, 0, 0, None) == tq.TQ_EUNSUPPORTED
    d = _desc(tq, layer_bk=[4, 1], layer_bv=[2, 2])
    assert L.tq_attn_decode(ctypes.byref(d), 1, A, 4, 5, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_EUNSUPPORTED
    d = _desc(tq, bk=1, layer_bk=[4, 4], layer_bv=[2, 2], batch=0)
    assert L.tq_attn_decode(ctypes.byref(d), 0, A, 4, 5, 0.0, 0.0, A, A, 1 << 20, None) == tq.TQ_OK


def test_injected_hip_error_path():
    """TQ_TEST_FAIL_LAUNCH=1 makes the next launch report TQ_EHIP without
    launching; the following call is unaffected (one shot)."""
    code = r"""
import ctypes, sys
sys.path.insert(0, %r)
import kv_cache_vector_rotate_amd as tq
L = tq.lib()
A = ctypes.c_void_p(4096); N = ctypes.c_void_p(8192)
rc = L.tq_encode(A, None, 0, 10, 128, 4, 2, 42, 0, A, N, None, None, None)
msg = tq.tq_last_error()
rc2 = L.tq_decode(None, N, 5, 128, 4, 42, 0, A, None)
print(rc, rc2, msg)
""" % ROOT
    env = dict(os.environ, TQ_TEST_FAIL_LAUNCH="1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    rc, rc2, msg = r.stdout.split(" ", 2)
    assert int(rc) == -3 and "injected" in msg
    assert int(rc2) == -1
