"""tq_attn_decode_noalloc (the library's static scratch in place of a
workspace; nothing allocated) against tq_attn_decode on the same inputs:
the same kernels and split, so the outputs must be identical.  Two calls in
a row on each path, the second with a smaller input than the first."""
import math

import numpy as np
import pytest
import torch

import kvgen

pytestmark = pytest.mark.gpu
SEED = 42


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_rotate_amd as tq
    tq.lib()
    return tq


def _case(tq, B, Hkv, G, d, T, bk, bv, seed, kscale=1.0):
    cache = tq.TQCache(1, B, Hkv, T, d, bk, bv, SEED)
    k = kvgen.normal((B, Hkv, T, d), seed, "cuda") * kscale
    v = kvgen.normal((B, Hkv, T, d), seed + 1, "cuda")
    tq.tq_encode(k, v, bk, bv, SEED, cache.k_packed[0], cache.k_norms[0], cache.v_packed[0],
                 cache.v_norms[0])
    q = kvgen.normal((B, Hkv * G, d), seed + 2, "cuda", torch.bfloat16)
    return cache, q


@pytest.mark.parametrize("gate", [0.0, 1e-3])
def test_noalloc_equals_workspace_entry_point(tq, orc, gate):
    big = _case(tq, 8, 4, 4, 128, 5000, 4, 2, 11, kscale=3.0)
    small = _case(tq, 2, 2, 1, 64, 700, 3, 2, 21, kscale=3.0)
    outs = []
    for cache, q in (big, small):       # two calls in a row, the second smaller
        o = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        tq.tq_attn_decode_noalloc(cache, 0, q, cache.window, o, sparse_v=gate)
        outs.append(o)
    torch.cuda.synchronize()
    for (cache, q), o in zip((big, small), outs):
        ref = tq.tq_attn_decode(cache, 0, q, cache.window, sparse_v=gate)
        assert torch.equal(o, ref)
    # and the smaller call against the oracle, to the parity bar
    from _parity import check_attention
    cache, q = small
    o = outs[1].cpu().numpy()
    d, T = 64, cache.window
    for h in (0, 1):
        kp = cache.k_packed[0][1, h].cpu().numpy()
        kn = cache.k_norms[0][1, h].cpu().numpy()
        vp = cache.v_packed[0][1, h].cpu().numpy()
        vn = cache.v_norms[0][1, h].cpu().numpy()
        ref = orc.attention(q[1, h:h + 1].float().cpu().numpy(), kp, kn, vp, vn, 1, T, d, 3, 2,
                            SEED, 1 / math.sqrt(d), sparse_v_threshold=gate)[0]
        check_attention(o[1, h], ref)


def test_noalloc_rejects_oversize_and_keeps_working(tq):
    """A call whose workspace would exceed the static scratch is rejected
    before any launch; the next call runs normally."""
    cache, q = _case(tq, 32, 8, 4, 128, 16384, 4, 2, 31)
    assert tq.tq_attn_workspace_bytes(cache, 0, 32, 16384, 1e-3) > tq.TQ_ATTN_NOALLOC_MAX_BYTES
    o = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TqError) as e:
        tq.tq_attn_decode_noalloc(cache, 0, q, 16384, o, sparse_v=1e-3)
    assert e.value.status == tq.TQ_EINVAL and "scratch" in str(e.value)
    assert torch.count_nonzero(o) == 0
    tq.tq_attn_decode_noalloc(cache, 0, q, 16384, o)     # ungated: fits
    assert torch.equal(o, tq.tq_attn_decode(cache, 0, q, 16384))
