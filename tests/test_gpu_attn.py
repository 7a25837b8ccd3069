"""GPU parity of tq_attn_decode against the oracle's plain definition
(decode every cached row, softmax attention in fp64)."""
import math

import numpy as np
import pytest
import torch

import kvgen
from _parity import check_attention

pytestmark = pytest.mark.gpu
SEED = 42


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_rotate_amd as tq
    tq.lib()
    return tq


def _fill(tq, cache, layer, seed, kscale=1.0, dist="normal"):
    B, H, W, d = cache.batch, cache.n_kv_heads, cache.window, cache.head_dim[layer]
    if dist == "normal":
        k = kvgen.normal((B, H, W, d), seed, "cuda") * kscale
        v = kvgen.normal((B, H, W, d), seed + 1, "cuda")
    else:
        k = kvgen.student_t((B, H, W, d), seed, device="cuda") * kscale
        v = kvgen.student_t((B, H, W, d), seed + 1, device="cuda")
    bk, bv = cache.layer_bits(layer)
    tq.tq_encode(k, v, bk, bv, SEED, cache.k_packed[layer],
                 cache.k_norms[layer], cache.v_packed[layer], cache.v_norms[layer],
                 flags=cache.flags)


def _oracle(orc, cache, layer, q, b, heads, T, scale, sparse_v=0.0):
    """Oracle output for sequence b, the given query heads, context slots [0, T)."""
    d = cache.head_dim[layer]
    G = q.shape[1] // cache.n_kv_heads
    out = {}
    for h in heads:
        g = h // G
        kp = cache.k_packed[layer][b, g, :T].cpu().numpy()
        kn = cache.k_norms[layer][b, g, :T].cpu().numpy()
        vp = cache.v_packed[layer][b, g, :T].cpu().numpy()
        vn = cache.v_norms[layer][b, g, :T].cpu().numpy()
        qh = q[b, h:h + 1].float().cpu().numpy()
        bk, bv = cache.layer_bits(layer)
        out[h] = orc.attention(qh, kp, kn, vp, vn, 1, T, d, bk, bv, SEED,
                               scale, sparse_v_threshold=sparse_v,
                               density=orc.GAUSS if cache.flags & 1 else orc.BETA,
                               two_sided=bool(cache.flags & 2))[0]
    return out


@pytest.mark.parametrize("d,bk,bv,G", [(128, 4, 2, 4), (64, 3, 2, 1), (256, 4, 4, 2),
                                       (128, 2, 3, 8), (256, 3, 2, 8), (64, 4, 4, 2),
                                       (128, 3, 4, 1), (128, 4, 2, 2), (64, 2, 2, 4),
                                       (256, 2, 3, 1), (256, 4, 2, 4), (64, 4, 2, 8),
                                       (256, 3, 2, 1), (128, 2, 2, 1)])
@pytest.mark.parametrize("T", [1, 7, 256, 300, 1100])
def test_attention_small(tq, orc, d, bk, bv, G, T):
    B, Hkv = 2, 2
    Hq = Hkv * G
    W = max(T, 16)
    cache = tq.TQCache(1, B, Hkv, W, d, bk, bv, SEED)
    _fill(tq, cache, 0, 7 + T + d)
    q = kvgen.normal((B, Hq, d), 3 + T, "cuda", torch.bfloat16)
    o = tq.tq_attn_decode(cache, 0, q, T).cpu().numpy()
    for b in range(B):
        ref = _oracle(orc, cache, 0, q, b, range(Hq), T, 1 / math.sqrt(d))
        for h in range(Hq):
            check_attention(o[b, h], ref[h])


@pytest.mark.parametrize("d,G,bk,bv", [(128, 4, 4, 2), (256, 1, 3, 2), (64, 1, 3, 2)])
def test_attention_ring_window_and_scale(tq, orc, d, G, bk, bv):
    """ctx_len beyond the window reads every slot; explicit scale; a peaked
    softmax (keys x 8); the exchange scan and the row scan."""
    B, Hkv, W = 1, 2, 700
    cache = tq.TQCache(1, B, Hkv, W, d, bk, bv, SEED)
    _fill(tq, cache, 0, 21, kscale=8.0)
    q = (kvgen.normal((B, Hkv * G, d), 22, "cuda") * 2.0).to(torch.bfloat16)
    o = tq.tq_attn_decode(cache, 0, q, 5000, scale=0.3).cpu().numpy()
    ref = _oracle(orc, cache, 0, q, 0, range(Hkv * G), W, 0.3)
    for h in range(Hkv * G):
        check_attention(o[0, h], ref[h])
    # the softmax is peaked: outputs are O(1), the bound is still met
    assert max(np.abs(ref[h]).max() for h in ref) > 0.5


@pytest.mark.parametrize("d,G", [(64, 4), (128, 1), (128, 4), (256, 2)])
def test_attention_peaked_row_groups(tq, orc, d, G):
    """Keys x 8 and queries x 2 (a peaked softmax whose largest scores sit in
    different rows of each tile), a context with a ragged last tile."""
    B, Hkv, T = 2, 2, 1100
    cache = tq.TQCache(1, B, Hkv, T, d, 4, 2, SEED)
    _fill(tq, cache, 0, 61 + d + G, kscale=8.0)
    q = (kvgen.normal((B, Hkv * G, d), 62 + G, "cuda") * 2.0).to(torch.bfloat16)
    o = tq.tq_attn_decode(cache, 0, q, T).cpu().numpy()
    for b in range(B):
        ref = _oracle(orc, cache, 0, q, b, range(Hkv * G), T, 1 / math.sqrt(d))
        for h in range(Hkv * G):
            check_attention(o[b, h], ref[h])


def test_attention_determinism(tq):
    d, B, Hkv, G, W = 128, 3, 2, 4, 5000
    cache = tq.TQCache(1, B, Hkv, W, d, 4, 2, SEED)
    _fill(tq, cache, 0, 31)
    q = kvgen.normal((B, Hkv * G, d), 32, "cuda", torch.bfloat16)
    a = tq.tq_attn_decode(cache, 0, q, W)
    b = tq.tq_attn_decode(cache, 0, q, W)
    assert torch.equal(a, b)


def test_config4_fused_decode_attention_full_size_sampled(tq, orc):
    """batch 32, 32 query heads on 8 KV heads, head_dim 128, context 16384,
    K4/V2 cache from N(0,1) rows, bf16 queries, scale 1/sqrt(128): the bench's
    launch; the oracle checks 6 sampled (sequence, KV head) groups (24 query
    heads)."""
    B, Hq, Hkv, d, T = 32, 32, 8, 128, 16384
    cache = tq.TQCache(1, B, Hkv, T, d, 4, 2, SEED)
    _fill(tq, cache, 0, 4)
    q = kvgen.normal((B, Hq, d), 44, "cuda", torch.bfloat16)
    o = tq.tq_attn_decode(cache, 0, q, T).cpu().numpy()
    rng = np.random.default_rng(4)
    errs = []
    for b in rng.choice(B, 6, replace=False):
        g = int(rng.integers(Hkv))
        heads = range(g * 4, g * 4 + 4)
        ref = _oracle(orc, cache, 0, q, int(b), heads, T, 1 / math.sqrt(d))
        for h in heads:
            errs.append(check_attention(o[b, h], ref[h]))
    print("config 4 max abs err %.3g, max rel L2 %.3g" % (max(e[0] for e in errs),
                                                          max(e[1] for e in errs)))


def test_config5_long_context_attention_sampled(tq, orc):
    """K3/V2, one sequence, 131072 tokens, 8 KV heads (G = 1), bf16
    Student-t(3) rows; one head_dim-64 and one head_dim-256 layer, 2 heads each
    checked against the oracle."""
    T, H = 131072, 8
    cache = tq.TQCache(2, 1, H, T, [64, 256], 3, 2, SEED)
    for l in range(2):
        _fill(tq, cache, l, 50 + l, dist="t")
    for l, d in enumerate((64, 256)):
        q = kvgen.student_t((1, H, d), 70 + l, device="cuda")
        o = tq.tq_attn_decode(cache, l, q, T).cpu().numpy()
        ref = _oracle(orc, cache, l, q, 0, (1, 6), T, 1 / math.sqrt(d))
        for h in (1, 6):
            check_attention(o[0, h], ref[h])


@pytest.mark.parametrize("d,bk,bv,G", [(128, 4, 2, 4), (64, 3, 3, 2), (256, 2, 4, 1),
                                       (128, 3, 2, 2), (128, 4, 4, 8), (256, 4, 2, 2),
                                       (64, 2, 3, 4), (256, 3, 3, 8)])
def test_attention_sparse_v(tq, orc, d, bk, bv, G):
    """Sparse-V gate (threshold 1e-3) against the oracle's rule, on a peaked
    softmax over several 256-slot blocks and a ragged last block; a large
    fraction of the rows is gated."""
    B, Hkv, T = 2, 2, 1100
    Hq = Hkv * G
    cache = tq.TQCache(1, B, Hkv, T, d, bk, bv, SEED)
    _fill(tq, cache, 0, 80 + d, kscale=6.0)
    q = (kvgen.normal((B, Hq, d), 81 + d, "cuda") * 2.0).to(torch.bfloat16)
    scale = 0.5
    o = tq.tq_attn_decode(cache, 0, q, T, scale=scale, sparse_v=1e-3).cpu().numpy()
    o0 = tq.tq_attn_decode(cache, 0, q, T, scale=scale).cpu().numpy()
    for b in range(B):
        ref = _oracle(orc, cache, 0, q, b, range(Hq), T, scale, sparse_v=1e-3)
        for h in range(Hq):
            check_attention(o[b, h], ref[h])
    # the gate changes the result (rows were dropped) but only slightly
    assert np.abs(o - o0).max() > 0
    assert np.abs(o - o0).max() < 0.05


@pytest.mark.parametrize("d,G", [(128, 4), (64, 2)])
@pytest.mark.parametrize("T", [1, 7, 256, 300])
def test_attention_sparse_v_short(tq, orc, d, G, T):
    """The gate on contexts of one row, a few rows, one whole block and one
    block plus a ragged part (keys x 6: many rows gated)."""
    B, Hkv = 2, 2
    Hq = Hkv * G
    cache = tq.TQCache(1, B, Hkv, max(T, 16), d, 4, 2, SEED)
    _fill(tq, cache, 0, 90 + T + d, kscale=6.0)
    q = (kvgen.normal((B, Hq, d), 91 + T, "cuda") * 2.0).to(torch.bfloat16)
    o = tq.tq_attn_decode(cache, 0, q, T, scale=0.5, sparse_v=1e-3).cpu().numpy()
    for b in range(B):
        ref = _oracle(orc, cache, 0, q, b, range(Hq), T, 0.5, sparse_v=1e-3)
        for h in range(Hq):
            check_attention(o[b, h], ref[h])


@pytest.mark.parametrize("t_dom", [5, 2900])
def test_attention_sparse_v_dominant_row_across_chunks(tq, orc, t_dom):
    """One dominant row, early or late, in a 3000-slot context that the
    kernels split over many chunks: against the context's largest score
    every other row of the four query heads that share it is gated, in every
    chunk (a reference maximum per chunk or per 256-row block would keep
    hundreds of them).  The other KV head's heads see ordinary scores."""
    d, B, Hkv, G, T = 128, 1, 2, 4, 3000
    cache = tq.TQCache(1, B, Hkv, T, d, 4, 2, SEED)
    _fill(tq, cache, 0, 95 + t_dom)
    kp = cache.k_packed[0][0, 0].cpu().numpy()
    kn = cache.k_norms[0][0, 0].cpu().numpy()
    Kh = orc.decode(kp, kn, d, 4, SEED, f64=True)
    qd = Kh[t_dom] / np.linalg.norm(Kh[t_dom]) * 3.0
    q = kvgen.normal((B, Hkv * G, d), 96, "cuda", torch.bfloat16)
    q[0, :G] = torch.from_numpy(qd).to(torch.bfloat16).cuda()
    qf = q[0, 0].float().cpu().numpy().astype(np.float64)
    scale = 1 / math.sqrt(d)
    s = scale * Kh @ qf
    # raise the row's key norm until its score leads every other by 10
    f = (np.delete(s, t_dom).max() + 10.0) / s[t_dom]
    assert f > 1
    cache.k_norms[0][0, 0, t_dom] *= float(f)
    kn = cache.k_norms[0][0, 0].cpu().numpy()
    s = scale * orc.decode(kp, kn, d, 4, SEED, f64=True) @ qf
    rel = np.exp(s - s.max())
    assert (rel > 1e-3).sum() == 1
    per_block = sum(int((np.exp(s[b0:b0 + 256] - s[b0:b0 + 256].max()) > 1e-3).sum())
                    for b0 in range(0, T, 256))
    assert per_block > 100
    o = tq.tq_attn_decode(cache, 0, q, T, sparse_v=1e-3).cpu().numpy()
    ref = _oracle(orc, cache, 0, q, 0, range(Hkv * G), T, scale, sparse_v=1e-3)
    for h in range(Hkv * G):
        check_attention(o[0, h], ref[h])


@pytest.mark.parametrize("t_dom", [5, 19990])
def test_attention_dominant_row_one_query_head(tq, orc, t_dom):
    """One query head per KV head (the row scan) over a 20000-slot context
    split into 79 chunks per head, with one row whose score leads every other
    by 10 early or late in the context: the merge's running maximum is set by
    the first chunk, or raised by the last and every earlier sum rescaled."""
    d, B, Hkv, G, T, bk, bv = 256, 1, 2, 1, 20000, 3, 2
    cache = tq.TQCache(1, B, Hkv, T, d, bk, bv, SEED)
    _fill(tq, cache, 0, 97 + t_dom)
    kp = cache.k_packed[0][0, 0].cpu().numpy()
    kn = cache.k_norms[0][0, 0].cpu().numpy()
    Kh = orc.decode(kp, kn, d, bk, SEED, f64=True)
    q = kvgen.normal((B, Hkv * G, d), 98, "cuda", torch.bfloat16)
    q[0, 0] = torch.from_numpy(Kh[t_dom] / np.linalg.norm(Kh[t_dom]) * 3.0).to(torch.bfloat16).cuda()
    qf = q[0, 0].float().cpu().numpy().astype(np.float64)
    scale = 1 / math.sqrt(d)
    s = scale * Kh @ qf
    f = (np.delete(s, t_dom).max() + 10.0) / s[t_dom]
    assert f > 1
    cache.k_norms[0][0, 0, t_dom] *= float(f)
    o = tq.tq_attn_decode(cache, 0, q, T).cpu().numpy()
    ref = _oracle(orc, cache, 0, q, 0, range(Hkv * G), T, scale)
    for h in range(Hkv * G):
        check_attention(o[0, h], ref[h])


def test_config4_attention_sparse_v_sampled(tq, orc):
    """The bench's attention launch with the sparse-V gate at 1e-3, sampled."""
    B, Hq, Hkv, d, T = 32, 32, 8, 128, 16384
    cache = tq.TQCache(1, B, Hkv, T, d, 4, 2, SEED)
    _fill(tq, cache, 0, 4)
    q = kvgen.normal((B, Hq, d), 44, "cuda", torch.bfloat16)
    o = tq.tq_attn_decode(cache, 0, q, T, sparse_v=1e-3).cpu().numpy()
    rng = np.random.default_rng(5)
    for b in rng.choice(B, 3, replace=False):
        g = int(rng.integers(Hkv))
        heads = range(g * 4, g * 4 + 4)
        ref = _oracle(orc, cache, 0, q, int(b), heads, T, 1 / math.sqrt(d), sparse_v=1e-3)
        for h in heads:
            check_attention(o[b, h], ref[h])


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("d,bk,bv,G", [(128, 4, 2, 4), (64, 3, 3, 2), (256, 2, 4, 1)])
def test_attention_flags(tq, orc, d, bk, bv, G, flags):
    """N(0, 1/d) codebooks and the two-sided rotation: the cache written with
    the flags, q rotated and the output rotated back with the same ones."""
    B, Hkv, T = 2, 2, 1100
    cache = tq.TQCache(1, B, Hkv, T, d, bk, bv, SEED, flags=flags)
    _fill(tq, cache, 0, 40 + d + flags)
    q = kvgen.normal((B, Hkv * G, d), 41 + flags, "cuda", torch.bfloat16)
    o = tq.tq_attn_decode(cache, 0, q, T).cpu().numpy()
    for b in range(B):
        ref = _oracle(orc, cache, 0, q, b, range(Hkv * G), T, 1 / math.sqrt(d))
        for h in range(Hkv * G):
            check_attention(o[b, h], ref[h])
    # with the gate on as well
    o = tq.tq_attn_decode(cache, 0, q, T, sparse_v=1e-2).cpu().numpy()
    ref = _oracle(orc, cache, 0, q, 1, range(Hkv * G), T, 1 / math.sqrt(d), sparse_v=1e-2)
    for h in range(Hkv * G):
        check_attention(o[1, h], ref[h])


def test_attention_per_layer_bits(tq, orc):
    """A cache whose layers have their own K and V widths (boundary layers at
    4 bits, the others lower) and head_dims: each layer's attention reads
    its own widths."""
    hd = [128, 64, 128, 256, 128]
    bk = [4, 3, 2, 3, 4]
    bv = tq.tq_layer_bits_boundary(5, 2, 4, n_boundary=1)      # [4, 2, 2, 2, 4]
    B, Hkv, G, T = 2, 2, 2, 600
    cache = tq.TQCache(5, B, Hkv, T, hd, bk, bv, SEED, flags=3)
    for layer in range(5):
        assert cache.k_packed[layer].shape[-1] == hd[layer] * bk[layer] // 8
        _fill(tq, cache, layer, 70 + layer)
    for layer in (0, 2, 3):
        q = kvgen.normal((B, Hkv * G, hd[layer]), 80 + layer, "cuda", torch.bfloat16)
        o = tq.tq_attn_decode(cache, layer, q, T).cpu().numpy()
        ref = _oracle(orc, cache, layer, q, 1, range(Hkv * G), T, 1 / math.sqrt(hd[layer]))
        for h in range(Hkv * G):
            check_attention(o[1, h], ref[h])


@pytest.mark.parametrize("flags", [0, 3])
@pytest.mark.parametrize("d,G", [(96, 4), (160, 2), (224, 8)])
def test_attention_padded_head_dim(tq, orc, d, G, flags):
    """head_dim that is not a power of two: q and out hold d values; the
    cache rows are stored at the padded length."""
    B, Hkv, T = 2, 2, 700
    cache = tq.TQCache(1, B, Hkv, T, d, 4, 2, SEED, flags=flags)
    _fill(tq, cache, 0, 90 + d)
    q = kvgen.normal((B, Hkv * G, d), 91 + d, "cuda", torch.bfloat16)
    o = tq.tq_attn_decode(cache, 0, q, T)
    assert o.shape == (B, Hkv * G, d)
    o = o.cpu().numpy()
    for b in range(B):
        ref = _oracle(orc, cache, 0, q, b, range(Hkv * G), T, 1 / math.sqrt(d))
        for h in range(Hkv * G):
            check_attention(o[b, h], ref[h])
