"""GPU parity of the append-only ring cache (tq_append_row) and of decoding
the whole window, against the oracle."""
import math

import numpy as np
import pytest
import torch

import kvgen
from _parity import BandTally, check_attention, check_decoded, check_indices, check_norms

pytestmark = pytest.mark.gpu
SEED = 42


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_rotate_amd as tq
    tq.lib()
    return tq


def _check_slot(orc, rows, packed, norms, d, bits, flags=0, tally=None):
    density = orc.GAUSS if flags & 1 else orc.BETA
    op, on, u = orc.encode(rows.astype(np.float32), d, bits, SEED, want_u=True,
                           density=density, two_sided=bool(flags & 2))
    dp = orc.padded_dim(d)          # rows are stored at the padded length
    _, bnd = orc.codebook_float(dp, bits, density)
    check_norms(norms, on)
    check_indices(packed, op, u, dp, bits, bnd, tally=tally)


@pytest.mark.parametrize("flags", [0, 3])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_append_ring_small_mixed_head_dims(tq, orc, dtype, flags):
    """3 layers (head_dim 256, 64, 256), batch 3, 2 KV heads, window 5;
    appends positions 0..11 (the ring wraps twice), all layers per call; the
    cache must hold exactly the last `window` rows of every (layer, seq, head)
    and untouched slots must stay as they were.  flags 3: N(0, 1/d) codebooks
    and the two-sided rotation."""
    hd = [256, 64, 256]
    B, H, W, bk, bv = 3, 2, 5, 4, 3
    cache = tq.TQCache(3, B, H, W, hd, bk, bv, SEED, flags=flags)
    hist = {}
    for pos in range(12):
        ks = [kvgen.unit_dirs_lognormal((B, H, d), 1000 * pos + l, "cuda").to(dtype)
              for l, d in enumerate(hd)]
        vs = [kvgen.unit_dirs_lognormal((B, H, d), 5000 + 1000 * pos + l, "cuda").to(dtype)
              for l, d in enumerate(hd)]
        tq.tq_append_row(cache, -1, ks, vs, pos)
        hist[pos % W] = (ks, vs)
        if pos == 2:
            # slots 3, 4 never written yet: still zero
            assert torch.count_nonzero(cache.k_norms[0][:, :, 3:]).item() == 0
    torch.cuda.synchronize()
    tally = BandTally()
    for slot, (ks, vs) in hist.items():
        for l, d in enumerate(hd):
            for x, bits, pk, nm in ((ks[l], bk, cache.k_packed[l], cache.k_norms[l]),
                                    (vs[l], bv, cache.v_packed[l], cache.v_norms[l])):
                rows = x.float().cpu().numpy().reshape(B * H, d)
                _check_slot(orc, rows, pk[:, :, slot].cpu().numpy().reshape(B * H, -1),
                            nm[:, :, slot].cpu().numpy().reshape(-1), d, bits, flags, tally)
    tally.check()


def test_append_single_layer(tq, orc):
    B, H, W, d = 2, 4, 7, 128
    cache = tq.TQCache(2, B, H, W, d, 4, 2, SEED)
    k = kvgen.normal((B, H, d), 1, "cuda")
    v = kvgen.normal((B, H, d), 2, "cuda")
    tq.tq_append_row(cache, 1, k, v, 9)
    torch.cuda.synchronize()
    assert torch.count_nonzero(cache.k_norms[0]).item() == 0
    slot = 9 % W
    tally = BandTally()
    _check_slot(orc, k.cpu().numpy().reshape(-1, d),
                cache.k_packed[1][:, :, slot].cpu().numpy().reshape(B * H, -1),
                cache.k_norms[1][:, :, slot].cpu().numpy().reshape(-1), d, 4, tally=tally)
    _check_slot(orc, v.cpu().numpy().reshape(-1, d),
                cache.v_packed[1][:, :, slot].cpu().numpy().reshape(B * H, -1),
                cache.v_norms[1][:, :, slot].cpu().numpy().reshape(-1), d, 2, tally=tally)
    tally.check()


def test_config2_gemma_shaped_step_full_size_sampled(tq, orc):
    """34 layers, 4 KV heads, head_dim 256, window 512, batch 64, K4/V4, fp32
    rows with random directions and lognormal(0, 0.5) norms.  Prefill fills
    the window (one encode per layer), then one step appends a row to every
    layer at pos 512 (slot 0) and decodes the whole window of every layer
    (tq_cache_decode)."""
    NL, B, H, W, d = 34, 64, 4, 512, 256
    cache = tq.TQCache(NL, B, H, W, d, 4, 4, SEED)
    rng = np.random.default_rng(2)
    for l in range(NL):
        k = kvgen.unit_dirs_lognormal((B, H, W, d), 10 + l, "cuda")
        v = kvgen.unit_dirs_lognormal((B, H, W, d), 100 + l, "cuda")
        tq.tq_encode(k, v, 4, 4, SEED, cache.k_packed[l], cache.k_norms[l], cache.v_packed[l],
                     cache.v_norms[l])
    ks = [kvgen.unit_dirs_lognormal((B, H, d), 300 + l, "cuda") for l in range(NL)]
    vs = [kvgen.unit_dirs_lognormal((B, H, d), 400 + l, "cuda") for l in range(NL)]
    tq.tq_append_row(cache, -1, ks, vs, W)
    # the whole window of every layer, K and V, in one call (68 buffers: two
    # launches of at most 64)
    kos, vos = tq.tq_cache_decode(cache, -1)
    torch.cuda.synchronize()
    tally = BandTally()
    for l in rng.choice(NL, 3, replace=False):
        for x, pk, nm, out in ((ks[l], cache.k_packed[l], cache.k_norms[l], kos[l]),
                               (vs[l], cache.v_packed[l], cache.v_norms[l], vos[l])):
            _check_slot(orc, x.cpu().numpy().reshape(-1, d),
                        pk[:, :, 0].cpu().numpy().reshape(B * H, -1),
                        nm[:, :, 0].cpu().numpy().reshape(-1), d, 4, tally=tally)
            sel = rng.choice(B * H * W, 2048, replace=False)
            gp = pk.reshape(-1, d // 2)[torch.from_numpy(sel).cuda()].cpu().numpy()
            gn = nm.reshape(-1)[torch.from_numpy(sel).cuda()].cpu().numpy()
            gx = out.reshape(-1, d)[torch.from_numpy(sel).cuda()].cpu().numpy()
            check_decoded(gx, orc.decode(gp, gn, d, 4, SEED))
    # the last layer's V through tq_decode as well: the same rows
    out = torch.empty(B, H, W, d, device="cuda")
    tq.tq_decode(cache.v_packed[NL - 1], cache.v_norms[NL - 1], d, 4, SEED, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, vos[NL - 1])
    tally.check()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_append_per_layer_bits(tq, orc, dtype):
    """Layers with their own (head_dim, K width, V width): one append call
    launches once per distinct triple; every slot matches the oracle at its
    layer's widths and untouched slots stay zero."""
    hd = [128, 64, 128, 256, 128, 64]
    bk = [4, 3, 2, 4, 4, 3]
    bv = tq.tq_layer_bits_boundary(6, 2, 4)                    # [4, 4, 2, 2, 4, 4]
    assert bv == [4, 4, 2, 2, 4, 4]
    B, H, W = 2, 3, 4
    cache = tq.TQCache(6, B, H, W, hd, bk, bv, SEED)
    tally = BandTally()
    for pos in (5, 6):
        ks = [kvgen.normal((B, H, d), 900 + 10 * pos + l, "cuda").to(dtype) for l, d in enumerate(hd)]
        vs = [kvgen.normal((B, H, d), 950 + 10 * pos + l, "cuda").to(dtype) for l, d in enumerate(hd)]
        tq.tq_append_row(cache, -1, ks, vs, pos)
        torch.cuda.synchronize()
        slot = pos % W
        for l, d in enumerate(hd):
            for x, bits, pk, nm in ((ks[l], bk[l], cache.k_packed[l], cache.k_norms[l]),
                                    (vs[l], bv[l], cache.v_packed[l], cache.v_norms[l])):
                assert pk.shape[-1] == d * bits // 8
                _check_slot(orc, x.float().cpu().numpy().reshape(-1, d),
                            pk[:, :, slot].cpu().numpy().reshape(B * H, -1),
                            nm[:, :, slot].cpu().numpy().reshape(-1), d, bits, tally=tally)
    tally.check()
    for l in range(6):
        assert torch.count_nonzero(cache.k_norms[l][:, :, [0, 3]]).item() == 0
        assert torch.count_nonzero(cache.v_packed[l][:, :, [0, 3]]).item() == 0


def test_append_padded_head_dims(tq, orc):
    """Layers of head_dim 96, 160 and 128 in one cache: rows of d values are
    appended at the padded length of their layer."""
    hd = [96, 160, 128, 96]
    B, H, W = 2, 2, 3
    cache = tq.TQCache(4, B, H, W, hd, 4, 3, SEED, flags=2)
    tally = BandTally()
    ks = [kvgen.normal((B, H, d), 1200 + l, "cuda") for l, d in enumerate(hd)]
    vs = [kvgen.normal((B, H, d), 1300 + l, "cuda").to(torch.bfloat16) for l, d in enumerate(hd)]
    tq.tq_append_row(cache, -1, ks, [v.float() for v in vs], 4)
    torch.cuda.synchronize()
    for l, d in enumerate(hd):
        dp = orc.padded_dim(d)
        assert cache.k_packed[l].shape[-1] == dp * 4 // 8
        for x, bits, pk, nm in ((ks[l], 4, cache.k_packed[l], cache.k_norms[l]),
                                (vs[l].float(), 3, cache.v_packed[l], cache.v_norms[l])):
            _check_slot(orc, x.cpu().numpy().reshape(-1, d),
                        pk[:, :, 1].cpu().numpy().reshape(B * H, -1),
                        nm[:, :, 1].cpu().numpy().reshape(-1), d, bits, flags=2, tally=tally)
    tally.check()


@pytest.mark.parametrize("d,bk,bv", [(64, 3, 2), (256, 4, 4), (96, 3, 3)])
def test_eviction_moves_packed_rows(tq, orc, d, bk, bv):
    """Evicting the oldest E positions of a linear cache is a plain move of
    packed bytes and norms: after shifting slots [E, W) down to [0, W - E),
    decoding and attention over the moved rows give what the oracle gives for
    the original rows, and a row appended at the freed position W - E joins
    them (TurboQuant KV Cache Compression — Spec, "Integration Points" and
    "Testing Strategy" item 7)."""
    B, H, W, E, G = 2, 2, 300, 37, 2
    cache = tq.TQCache(1, B, H, W, d, bk, bv, SEED)
    k = kvgen.normal((B, H, W, d), 61, "cuda")
    v = kvgen.normal((B, H, W, d), 62, "cuda")
    tq.tq_encode(k, v, bk, bv, SEED, cache.k_packed[0], cache.k_norms[0],
                 cache.v_packed[0], cache.v_norms[0])
    torch.cuda.synchronize()
    before = [t.clone() for t in (cache.k_packed[0], cache.k_norms[0],
                                   cache.v_packed[0], cache.v_norms[0])]
    for t in (cache.k_packed[0], cache.k_norms[0], cache.v_packed[0], cache.v_norms[0]):
        t[:, :, :W - E] = t[:, :, E:].clone()
    kn = kvgen.normal((B, H, d), 63, "cuda")
    vn = kvgen.normal((B, H, d), 64, "cuda")
    tq.tq_append_row(cache, 0, kn, vn, W - E)
    T = W - E + 1
    q = kvgen.normal((B, H * G, d), 65, "cuda", torch.bfloat16)
    o = tq.tq_attn_decode(cache, 0, q, T).cpu().numpy()
    dp = orc.padded_dim(d)
    out = torch.empty(B, H, W - E, dp, device="cuda")
    for pk, nm, bits, src_p, src_n in ((cache.k_packed[0], cache.k_norms[0], bk, before[0], before[1]),
                                       (cache.v_packed[0], cache.v_norms[0], bv, before[2], before[3])):
        tq.tq_decode(pk[:, :, :W - E].contiguous(), nm[:, :, :W - E].contiguous(), dp, bits,
                     SEED, out=out)
        torch.cuda.synchronize()
        gp = src_p[:, :, E:].cpu().numpy().reshape(-1, pk.shape[-1])
        gn = src_n[:, :, E:].cpu().numpy().reshape(-1)
        check_decoded(out.cpu().numpy().reshape(-1, dp), orc.decode(gp, gn, dp, bits, SEED))
    tally = BandTally()
    _check_slot(orc, kn.cpu().numpy().reshape(-1, d),
                cache.k_packed[0][:, :, W - E].cpu().numpy().reshape(B * H, -1),
                cache.k_norms[0][:, :, W - E].cpu().numpy().reshape(-1), d, bk, tally=tally)
    tally.check()
    # attention over the original rows E..W-1 followed by the appended row
    for b in range(B):
        for h in range(H * G):
            g = h // G
            kp = np.concatenate([before[0][b, g, E:].cpu().numpy(),
                                 cache.k_packed[0][b, g, W - E:W - E + 1].cpu().numpy()])
            kq = np.concatenate([before[1][b, g, E:].cpu().numpy(),
                                 cache.k_norms[0][b, g, W - E:W - E + 1].cpu().numpy()])
            vp = np.concatenate([before[2][b, g, E:].cpu().numpy(),
                                 cache.v_packed[0][b, g, W - E:W - E + 1].cpu().numpy()])
            vq = np.concatenate([before[3][b, g, E:].cpu().numpy(),
                                 cache.v_norms[0][b, g, W - E:W - E + 1].cpu().numpy()])
            ref = orc.attention(q[b, h:h + 1].float().cpu().numpy(), kp, kq, vp, vq, 1, T, d, bk, bv,
                                SEED, 1.0 / math.sqrt(d))[0]
            check_attention(o[b, h], ref)


def _decode_ref(orc, cache, l, side, start, count):
    bits = cache.layer_bits(l)[side]
    pk = (cache.k_packed if side == 0 else cache.v_packed)[l][:, :, start:start + count]
    nm = (cache.k_norms if side == 0 else cache.v_norms)[l][:, :, start:start + count]
    return orc.decode(pk.cpu().numpy(), nm.cpu().numpy(), cache.head_dim[l], bits, SEED,
                      density=orc.GAUSS if cache.flags & 1 else orc.BETA,
                      two_sided=bool(cache.flags & 2))


@pytest.mark.parametrize("flags", [0, 3])
def test_cache_decode_slot_ranges(tq, orc, flags):
    """tq_cache_decode over layers of head_dim 256, 64, 96 (padded to 128) and
    128 with their own K and V widths: every (layer, side) in one call (one
    launch per (head_dim, bits)), slot ranges that are not a multiple of the
    rows per wave, a single layer and a single side; each output matches the
    oracle's decode of the same packed rows."""
    hd = [256, 64, 96, 128, 256]
    bk = [4, 3, 4, 2, 4]
    bv = [2, 2, 3, 4, 2]
    B, H, W = 2, 3, 37
    cache = tq.TQCache(5, B, H, W, hd, bk, bv, SEED, flags=flags)
    for l, d in enumerate(hd):
        k = kvgen.normal((B, H, W, d), 70 + l, "cuda")
        v = kvgen.normal((B, H, W, d), 80 + l, "cuda").to(torch.bfloat16)
        tq.tq_encode(k, v.float(), bk[l], bv[l], SEED, cache.k_packed[l], cache.k_norms[l],
                     cache.v_packed[l], cache.v_norms[l], flags=flags)
    for layer, start, count, sides in ((-1, 0, W, "kv"), (-1, 5, 19, "kv"), (2, 36, 1, "kv"),
                                       (0, 3, 30, "v"), (-1, 1, 7, "k")):
        ko, vo = tq.tq_cache_decode(cache, layer, start, count, sides=sides)
        torch.cuda.synchronize()
        layers = list(range(5)) if layer < 0 else [layer]
        for side, outs in ((0, ko), (1, vo)):
            if "kv"[side] not in sides:
                assert outs is None
                continue
            outs = outs if layer < 0 else [outs]
            for l, o in zip(layers, outs):
                assert o.shape == (B, H, count, hd[l])
                check_decoded(o.cpu().numpy().reshape(-1, hd[l]),
                              _decode_ref(orc, cache, l, side, start, count))


def test_cache_decode_many_heads(tq, orc):
    """More (sequence, head) pairs than one launch's grid holds (65600 >
    65535): the call splits them over launches."""
    B, H, W, d = 16400, 4, 3, 64
    cache = tq.TQCache(1, B, H, W, d, 3, 2, SEED)
    k = kvgen.normal((B, H, W, d), 91, "cuda")
    tq.tq_encode(k, k, 3, 2, SEED, cache.k_packed[0], cache.k_norms[0], cache.v_packed[0],
                 cache.v_norms[0])
    ko, vo = tq.tq_cache_decode(cache, 0, 1, 2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for side, o in ((0, ko), (1, vo)):
        ref = _decode_ref(orc, cache, 0, side, 1, 2).reshape(B * H, 2, d)
        got = o.cpu().numpy().reshape(B * H, 2, d)
        sel = np.concatenate([rng.choice(B * H, 2000, replace=False), [0, 65534, 65535, B * H - 1]])
        check_decoded(got[sel].reshape(-1, d), ref[sel].reshape(-1, d))
