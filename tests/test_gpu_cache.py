"""GPU parity of the append-only ring cache (tq_append_row) and of decoding
the whole window, against the oracle."""
import numpy as np
import pytest
import torch

import kvgen
from _parity import BandTally, check_decoded, check_indices, check_norms

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
    layer at pos 512 (slot 0) and decodes the whole window of every layer."""
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
    out = torch.empty(B, H, W, d, device="cuda")
    tally = BandTally()
    for l in rng.choice(NL, 3, replace=False):
        for x, pk, nm in ((ks[l], cache.k_packed[l], cache.k_norms[l]),
                          (vs[l], cache.v_packed[l], cache.v_norms[l])):
            _check_slot(orc, x.cpu().numpy().reshape(-1, d),
                        pk[:, :, 0].cpu().numpy().reshape(B * H, -1),
                        nm[:, :, 0].cpu().numpy().reshape(-1), d, 4, tally=tally)
            tq.tq_decode(pk, nm, d, 4, SEED, out=out)
            torch.cuda.synchronize()
            sel = rng.choice(B * H * W, 2048, replace=False)
            gp = pk.reshape(-1, d // 2)[torch.from_numpy(sel).cuda()].cpu().numpy()
            gn = nm.reshape(-1)[torch.from_numpy(sel).cuda()].cpu().numpy()
            gx = out.reshape(-1, d)[torch.from_numpy(sel).cuda()].cpu().numpy()
            check_decoded(gx, orc.decode(gp, gn, d, 4, SEED))
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
