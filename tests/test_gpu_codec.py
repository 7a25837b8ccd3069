"""GPU parity of rotate / encode / decode against the fp64 oracle.

Every case calls the HIP kernels through the C ABI (via the thin binding) and
compares element by element with the oracle on the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

import kvgen
from _parity import (BandTally, check_decoded, check_indices, check_indices_with_ties, check_norms,
                     unpack_rows)

pytestmark = pytest.mark.gpu
SEED = 42


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_rotate_amd as tq
    tq.lib()
    return tq


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def _encode_check(tq, orc, x, d, bits, density_seed=SEED):
    """Encode x (device, [n, d]) on the GPU, compare with the oracle; returns
    (gpu packed, gpu norms)."""
    kp, kn, _, _ = tq.tq_encode(x, None, bits, 2, density_seed)
    torch.cuda.synchronize()
    xh = _np(x).reshape(-1, d).astype(np.float32)
    op, on, u = orc.encode(xh, d, bits, density_seed, want_u=True)
    _, bnd = orc.codebook_float(d, bits)
    gp, gn = kp.cpu().numpy().reshape(-1, d * bits // 8), kn.cpu().numpy().reshape(-1)
    check_norms(gn, on)
    check_indices(gp, op, u, d, bits, bnd)
    return gp, gn


def test_config1_round_trip_full(tq, orc):
    """4096 rows x 128, fp32 N(0,1), K4, seed 42: encode, decode, cosine."""
    d, bits = 128, 4
    x = kvgen.normal((4096, d), 1, "cuda")
    gp, gn = _encode_check(tq, orc, x, d, bits)
    kp = torch.from_numpy(gp).cuda()
    kn = torch.from_numpy(gn).cuda()
    xd = tq.tq_decode(kp, kn, d, bits, SEED).cpu().numpy()
    check_decoded(xd, orc.decode(gp, gn, d, bits, SEED))
    xs = _np(x)
    cos = (xd * xs).sum(1) / np.linalg.norm(xd, axis=1) / np.linalg.norm(xs, axis=1)
    assert cos.min() >= 0.88


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_encode_decode_all_bits_ragged(tq, orc, d, dtype):
    """K and V in one launch with different bit widths; row counts that leave
    a ragged tail in the last workgroup pass."""
    n = 1000 + 37
    tally = BandTally()
    k = kvgen.normal((n, d), 11 + d, "cuda", dtype)
    v = kvgen.normal((n, d), 12 + d, "cuda", dtype) * 3.0
    for bk, bv in ((4, 2), (3, 3), (2, 4)):
        kp, kn, vp, vn = tq.tq_encode(k, v, bk, bv, SEED)
        torch.cuda.synchronize()
        for x, bits, p, nm in ((k, bk, kp, kn), (v, bv, vp, vn)):
            xh = _np(x).astype(np.float32)
            op, on, u = orc.encode(xh, d, bits, SEED, want_u=True)
            _, bnd = orc.codebook_float(d, bits)
            gp, gn = p.cpu().numpy(), nm.cpu().numpy()
            check_norms(gn, on)
            check_indices(gp, op, u, d, bits, bnd, tally=tally)
            xd = tq.tq_decode(p, nm, d, bits, SEED).cpu().numpy()
            check_decoded(xd, orc.decode(gp, gn, d, bits, SEED))
    tally.check()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_encode_bf16_row_counts_at_block_edges(tq, orc, d):
    """bf16 rows in counts around the matrix-core encode's 16-row blocks and
    64-row groups (a launch of 256 rows per workgroup and side): partial first
    blocks, partial groups, workgroups whose later waves start past the last
    row; K and V of different widths in one launch, against the oracle."""
    tally = BandTally()
    for n in (1, 5, 15, 16, 17, 33, 63, 64, 65, 127, 255, 256, 257, 300, 513):
        k = kvgen.normal((n, d), 900 + n, "cuda", torch.bfloat16)
        v = kvgen.normal((n, d), 901 + n, "cuda", torch.bfloat16)
        for bk, bv in ((4, 2), (3, 3)):
            kp, kn, vp, vn = tq.tq_encode(k, v, bk, bv, SEED)
            torch.cuda.synchronize()
            for x, bits, pk, nm in ((k, bk, kp, kn), (v, bv, vp, vn)):
                op, on, u = orc.encode(_np(x).astype(np.float32), d, bits, SEED, want_u=True)
                _, bnd = orc.codebook_float(d, bits)
                check_norms(nm.cpu().numpy(), on)
                check_indices(pk.cpu().numpy(), op, u, d, bits, bnd, tally=tally)
    tally.check()


@pytest.mark.parametrize("d", [64, 128])
def test_encode_rows_at_high_low_word_addresses(tq, orc, d):
    """bf16 rows whose device addresses have the low 32-bit word at or above
    2^31 (a view into a buffer past such a boundary): the encode builds its
    load addresses from 32-bit halves, which must widen without sign."""
    n = 300
    nbytes = n * d * 2
    buf = torch.empty((1 << 32) + nbytes + 4096, dtype=torch.uint8, device="cuda")
    base = buf.data_ptr()
    # first 16-byte aligned offset whose address has the low word >= 2^31
    lo = base & 0xFFFFFFFF
    off = 0 if lo >= (1 << 31) else (1 << 31) - lo
    off = (off + 15) // 16 * 16
    assert ((base + off) & 0xFFFFFFFF) >= (1 << 31) and off + nbytes <= buf.numel()
    k = buf[off:off + nbytes].view(torch.bfloat16).view(n, d)
    k.copy_(kvgen.normal((n, d), 41 + d, "cuda", torch.bfloat16))
    v = kvgen.normal((n, d), 42 + d, "cuda", torch.bfloat16)
    tally = BandTally()
    kp, kn, vp, vn = tq.tq_encode(k, v, 4, 2, SEED)
    torch.cuda.synchronize()
    for x, bits, pk, nm in ((k, 4, kp, kn), (v, 2, vp, vn)):
        op, on, u = orc.encode(_np(x).astype(np.float32), d, bits, SEED, want_u=True)
        _, bnd = orc.codebook_float(d, bits)
        check_norms(nm.cpu().numpy(), on)
        check_indices(pk.cpu().numpy(), op, u, d, bits, bnd, tally=tally)
    tally.check()
    del k, buf


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotate_forward_inverse(tq, orc, d):
    x = kvgen.normal((333, d), 5, "cuda")
    y = tq.tq_rotate(x, SEED).cpu().numpy()
    yo = orc.rotate(_np(x).astype(np.float64), SEED)
    assert np.abs(y - yo).max() <= 1e-6 * np.abs(yo).max()
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(_np(x), axis=1), rtol=1e-5)
    xb = tq.tq_rotate(torch.from_numpy(y).cuda(), SEED, inverse=True).cpu().numpy()
    assert np.abs(xb - _np(x)).max() <= 1e-5
    xi = orc.unrotate(_np(x).astype(np.float64), SEED)
    yi = tq.tq_rotate(x, SEED, inverse=True).cpu().numpy()
    assert np.abs(yi - xi).max() <= 1e-6 * np.abs(xi).max()
    xb16 = x.to(torch.bfloat16)
    y16 = tq.tq_rotate(xb16, SEED).cpu().numpy()
    yo16 = orc.rotate(_np(xb16).astype(np.float64), SEED)
    assert np.abs(y16 - yo16).max() <= 1e-6 * np.abs(yo16).max()


def test_edge_rows(tq, orc):
    """Zero, constant, tiny, huge and single-spike rows; power-of-two scale
    invariance on the device."""
    d, bits = 128, 4
    rng = np.random.default_rng(3)
    base = rng.standard_normal((8, d)).astype(np.float32)
    rows = [np.zeros(d, np.float32), np.ones(d, np.float32), -np.ones(d, np.float32),
            np.eye(d, dtype=np.float32)[5] * 7.0, base[0] * np.float32(1e-30),
            base[1] * np.float32(1e30), base[2] * np.float32(2.0 ** -126),
            base[3] * np.float32(3e-41)]
    x = torch.from_numpy(np.stack(rows + list(base))).cuda()
    gp, gn = _encode_check(tq, orc, x, d, bits)
    L = 1 << bits
    assert gn[0] == 0 and np.all(unpack_rows(gp[:1], d, bits) == L // 2 - 1)
    xd = tq.tq_decode(torch.from_numpy(gp).cuda(), torch.from_numpy(gn).cuda(), d, bits,
                      SEED).cpu().numpy()
    assert np.all(xd[0] == 0)
    finite = np.isfinite(gn) & (gn > 1e-30) & (gn < 1e30)
    check_decoded(xd[finite], orc.decode(gp[finite], gn[finite], d, bits, SEED))
    # constant row: the sign-first order spreads it; round trip keeps cos >= 0.88
    c = (xd[1] @ rows[1]) / np.linalg.norm(xd[1]) / np.linalg.norm(rows[1])
    assert c >= 0.88
    # exact power-of-two scaling leaves the indices unchanged
    for k in (-90, -20, 20, 90):
        xs = torch.from_numpy(base * np.float32(2.0 ** k)).cuda()
        sp, sn, _, _ = tq.tq_encode(xs, None, bits, 2, SEED)
        assert np.array_equal(sp.cpu().numpy(), gp[8:])
        assert np.array_equal(sn.cpu().numpy(), gn[8:] * np.float32(2.0 ** k))


@pytest.mark.parametrize("sides", [1, 2])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_edge_rows(tq, orc, bits, d, dtype, sides):
    """Zero, constant, spike, exact-tie, tiny and huge rows against the
    oracle; rows holding an Inf or a NaN encode as the zero row with a
    non-finite norm; power-of-two scale invariance (indices identical, norms
    scaled exactly, except that the bf16 matrix-core kernels sum a rescaled
    row's squares in another order: there within 1e-6).  sides = 2 encodes
    the rows as K and as V in one call (the two results must be
    identical)."""
    def tq_encode(rows, bits_k, bits_v, seed):
        if sides == 1:
            return tq.tq_encode(rows, None, bits_k, bits_v, seed)
        kp_, kn_, vp_, vn_ = tq.tq_encode(rows, rows, bits_k, bits_k, seed)
        assert torch.equal(kp_, vp_)
        assert torch.equal(kn_.nan_to_num(), vn_.nan_to_num())
        return kp_, kn_, None, None

    bf16_rows = dtype == torch.bfloat16
    rng = np.random.default_rng(5)
    e = np.eye(d, dtype=np.float32)
    base = rng.standard_normal((6, d)).astype(np.float32)
    rows = [np.zeros(d, np.float32), np.ones(d, np.float32), e[d - 56] * 3.0, e[0] + e[1],
            e[3] - e[d // 2 + 2], base[0] * np.float32(1e-30), base[1] * np.float32(1e30)]
    x = torch.from_numpy(np.stack(rows + list(base))).cuda().to(dtype)
    kp, kn, _, _ = tq_encode(x, bits, 2, SEED)
    torch.cuda.synchronize()
    op, on, u = orc.encode(_np(x).astype(np.float32), d, bits, SEED, want_u=True)
    gp, gn = kp.cpu().numpy(), kn.cpu().numpy()
    check_norms(gn, on)
    # rows with exactly zero rotated coordinates sit on the middle boundary
    # (either neighbouring cell is as near); every other index is bit-exact
    # outside the 1e-6 band, in-band mismatches counted
    _, bnd = orc.codebook_float(d, bits)
    tally = BandTally()
    check_indices_with_ties(gp, op, u, d, bits, bnd, tally)
    tally.check()
    ig = unpack_rows(gp, d, bits)
    L = 1 << bits
    assert gn[0] == 0 and np.all(ig[0] == L // 2 - 1)
    xd = tq.tq_decode(kp, kn, d, bits, SEED).cpu().numpy()
    assert np.all(xd[0] == 0)
    check_decoded(xd[1:], orc.decode(gp[1:], gn[1:], d, bits, SEED))
    # exact power-of-two scaling leaves the indices unchanged
    for k in (-60, -20, 20, 60):  # +-60 take the rescaled path
        xs = x[7:] * float(2.0 ** k)
        sp, sn, _, _ = tq_encode(xs, bits, 2, SEED)
        assert np.array_equal(sp.cpu().numpy(), gp[7:])
        want = gn[7:] * np.float32(2.0 ** k)
        if abs(k) > 20 and bf16_rows:
            np.testing.assert_allclose(sn.cpu().numpy(), want, rtol=1e-6)
        else:
            assert np.array_equal(sn.cpu().numpy(), want)
    # Inf and NaN rows
    bad = x[7:9].clone()
    bad[0, 17] = float("inf")
    bad[1, d - 6] = float("nan")
    bp, bn, _, _ = tq_encode(bad, bits, 2, SEED)
    bn = bn.cpu().numpy()
    assert not np.isfinite(bn).any()
    assert np.all(unpack_rows(bp.cpu().numpy(), d, bits) == L // 2 - 1)


def test_empty_and_single_row(tq, orc):
    d = 128
    x = torch.empty(0, d, device="cuda")
    kp, kn, _, _ = tq.tq_encode(x, None, 4, 2, SEED)
    assert kp.numel() == 0 and kn.numel() == 0
    one = kvgen.normal((1, d), 9, "cuda")
    _encode_check(tq, orc, one, d, 4)


def test_determinism(tq):
    d = 256
    x = kvgen.normal((5000, d), 17, "cuda", torch.bfloat16)
    a = tq.tq_encode(x, x, 3, 2, SEED)
    b = tq.tq_encode(x, x, 3, 2, SEED)
    for s, t in zip(a, b):
        assert torch.equal(s, t)
    da = tq.tq_decode(a[0], a[1], d, 3, SEED)
    db = tq.tq_decode(b[0], b[1], d, 3, SEED)
    assert torch.equal(da, db)


def test_config3_bulk_prefill_full_size_sampled(tq, orc):
    """32 layers x 8 KV heads x 32768 tokens x 128, bf16 AR(1) rho 0.6 with 4
    outlier channels (x8) per head, K4/V2 in one launch -- the bench's launch
    -- compared on 4096 sampled rows per side."""
    L, H, T, d = 32, 8, 32768, 128
    k = kvgen.ar1_outliers((L, H, T, d), 3, "cuda")
    v = kvgen.ar1_outliers((L, H, T, d), 103, "cuda")
    kp, kn, vp, vn = tq.tq_encode(k, v, 4, 2, SEED)
    torch.cuda.synchronize()
    n = L * H * T
    rows = np.sort(np.random.default_rng(3).choice(n, 4096, replace=False))
    ridx = torch.from_numpy(rows).cuda()
    tally = BandTally()
    for x, bits, p, nm in ((k, 4, kp, kn), (v, 2, vp, vn)):
        xs = x.reshape(n, d)[ridx].float().cpu().numpy()
        op, on, u = orc.encode(xs, d, bits, SEED, want_u=True)
        _, bnd = orc.codebook_float(d, bits)
        gp = p.reshape(n, -1)[ridx].cpu().numpy()
        gn = nm.reshape(n)[ridx].cpu().numpy()
        check_norms(gn, on)
        check_indices(gp, op, u, d, bits, bnd, tally=tally)
    tally.check()


def test_config5_long_context_codec_sampled(tq, orc):
    """K3/V2, one sequence, 131072 tokens, 8 KV heads, head_dim 64 and 256,
    bf16 Student-t(3): encode and decode per layer (two layers of each head_dim
    here), compared on sampled rows."""
    T, H = 131072, 8
    rng = np.random.default_rng(5)
    tally = BandTally()
    for li, d in enumerate((64, 256, 64, 256)):
        k = kvgen.student_t((H, T, d), 500 + li, device="cuda")
        v = kvgen.student_t((H, T, d), 600 + li, device="cuda")
        kp, kn, vp, vn = tq.tq_encode(k, v, 3, 2, SEED)
        n = H * T
        rows = np.sort(rng.choice(n, 2048, replace=False))
        ridx = torch.from_numpy(rows).cuda()
        for x, bits, p, nm in ((k, 3, kp, kn), (v, 2, vp, vn)):
            xs = x.reshape(n, d)[ridx].float().cpu().numpy()
            op, on, u = orc.encode(xs, d, bits, SEED, want_u=True)
            _, bnd = orc.codebook_float(d, bits)
            gp = p.reshape(n, -1)[ridx].cpu().numpy()
            gn = nm.reshape(n)[ridx].cpu().numpy()
            check_norms(gn, on)
            check_indices(gp, op, u, d, bits, bnd, tally=tally)
            out = tq.tq_decode(p, nm, d, bits, SEED)
            xd = out.reshape(n, d)[ridx].cpu().numpy()
            check_decoded(xd, orc.decode(gp, gn, d, bits, SEED))
            del out
        del k, v, kp, kn, vp, vn
    tally.check()


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_encode_decode_flags(tq, orc, d, dtype, flags):
    """N(0, 1/d) codebooks (flag 1) and the two-sided rotation (flag 2): every
    bit width on both sides of one launch (the matrix-core kernel for bf16
    rows, the lane-slice kernel for fp32), then decode."""
    density = orc.GAUSS if flags & 1 else orc.BETA
    two = bool(flags & 2)
    n = 4096 + 29
    tally = BandTally()
    k = kvgen.normal((n, d), 31 + d + flags, "cuda", dtype)
    v = kvgen.normal((n, d), 32 + d + flags, "cuda", dtype) * 2.0
    for bk, bv in ((4, 2), (3, 3), (2, 4)):
        kp, kn, vp, vn = tq.tq_encode(k, v, bk, bv, SEED, flags=flags)
        torch.cuda.synchronize()
        for x, bits, p, nm in ((k, bk, kp, kn), (v, bv, vp, vn)):
            xh = _np(x).astype(np.float32)
            op, on, u = orc.encode(xh, d, bits, SEED, density=density, want_u=True,
                                   two_sided=two)
            _, bnd = orc.codebook_float(d, bits, density)
            gp, gn = p.cpu().numpy(), nm.cpu().numpy()
            check_norms(gn, on)
            check_indices(gp, op, u, d, bits, bnd, tally=tally)
            xd = tq.tq_decode(p, nm, d, bits, SEED, flags=flags).cpu().numpy()
            check_decoded(xd, orc.decode(gp, gn, d, bits, SEED, density=density,
                                         two_sided=two))
    tally.check()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotate_two_sided(tq, orc, d):
    x = kvgen.normal((333, d), 6, "cuda")
    xs = _np(x).astype(np.float64)
    for inverse in (False, True):
        y = tq.tq_rotate(x, SEED, inverse=inverse, flags=2).cpu().numpy()
        yo = (orc.unrotate if inverse else orc.rotate)(xs, SEED, two_sided=True)
        assert np.abs(y - yo).max() <= 1e-6 * np.abs(yo).max()
    y = tq.tq_rotate(x, SEED, flags=2)
    xb = tq.tq_rotate(y, SEED, inverse=True, flags=2).cpu().numpy()
    assert np.abs(xb - xs).max() <= 1e-5
    # the density bit does not change the rotation
    assert torch.equal(tq.tq_rotate(x, SEED, flags=3), y)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_edge_rows_two_sided(tq, orc, dtype, bits):
    """Rows whose rotated coordinates are exactly zero (u = +-0 after the
    second diagonal), zero rows and spikes, two-sided with both densities."""
    d = 128
    e = np.eye(d, dtype=np.float32)
    rows = [np.zeros(d, np.float32), e[0] + e[1], e[3] - e[7], e[5] * 3.0,
            e[0] + e[1] + e[2] + e[3], np.ones(d, np.float32)]
    x = torch.from_numpy(np.stack(rows)).cuda().to(dtype)
    for flags in (2, 3):
        density = orc.GAUSS if flags & 1 else orc.BETA
        kp, kn, _, _ = tq.tq_encode(x, None, bits, 2, SEED, flags=flags)
        torch.cuda.synchronize()
        op, on, u = orc.encode(_np(x).astype(np.float32), d, bits, SEED, density=density,
                               want_u=True, two_sided=True)
        gp, gn = kp.cpu().numpy(), kn.cpu().numpy()
        # exact zeros sit on the middle boundary: the two cells next to it are
        # equally near, and the kernel's fused last stage (a*t + b*t as one
        # fma over a rounded product) may leave that product's rounding error,
        # a tiny value of either sign, there; every other index is bit-exact
        _, bnd = orc.codebook_float(d, bits, density)
        tally = BandTally()
        check_indices_with_ties(gp, op, u, d, bits, bnd, tally)
        tally.check()
        ig, io = unpack_rows(gp, d, bits), unpack_rows(op, d, bits)
        assert np.array_equal(ig[0], io[0])           # zero row: u = 0 exactly, t = 0
        check_norms(gn, on)
        xd = tq.tq_decode(kp, kn, d, bits, SEED, flags=flags).cpu().numpy()
        assert np.all(xd[0] == 0)
        check_decoded(xd[1:], orc.decode(gp[1:], gn[1:], d, bits, SEED, density=density,
                                         two_sided=True))


@pytest.mark.parametrize("flags", [0, 3])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [96, 160, 192, 224])
def test_padded_head_dim(tq, orc, d, dtype, flags):
    """head_dim that is not a power of two: rows of d values, packed at the
    next power of two, decoded back to d values."""
    dp = orc.padded_dim(d)
    density = orc.GAUSS if flags & 1 else orc.BETA
    two = bool(flags & 2)
    n = 1000 + 37
    tally = BandTally()
    k = kvgen.normal((n, d), 61 + d, "cuda", dtype)
    v = kvgen.normal((n, d), 62 + d, "cuda", dtype) * 0.5
    for bk, bv in ((4, 2), (3, 3), (2, 4)):
        kp, kn, vp, vn = tq.tq_encode(k, v, bk, bv, SEED, flags=flags)
        torch.cuda.synchronize()
        for x, bits, p, nm in ((k, bk, kp, kn), (v, bv, vp, vn)):
            assert p.shape == (n, dp * bits // 8)
            xh = _np(x).astype(np.float32)
            op, on, u = orc.encode(xh, d, bits, SEED, density=density, want_u=True,
                                   two_sided=two)
            _, bnd = orc.codebook_float(dp, bits, density)
            gp, gn = p.cpu().numpy(), nm.cpu().numpy()
            check_norms(gn, on)
            check_indices(gp, op, u, dp, bits, bnd, tally=tally)
            xd = tq.tq_decode(p, nm, d, bits, SEED, flags=flags)
            assert xd.shape == (n, d)
            check_decoded(xd.cpu().numpy(), orc.decode(gp, gn, d, bits, SEED, density=density,
                                                       two_sided=two))
    tally.check()


@pytest.mark.parametrize("flags", [2, 3])
def test_flags_large_launch_sampled(tq, orc, flags):
    """K4/V2 bf16 d = 128 with the flags at 600k rows (a launch of thousands of
    workgroups per side, the second side's after the first's, and a ragged
    last group), compared on sampled rows."""
    d, n = 128, 600_000 + 37
    density = orc.GAUSS if flags & 1 else orc.BETA
    k = kvgen.ar1_outliers((1, 1, n, d), 70 + flags, "cuda").reshape(n, d)
    v = kvgen.ar1_outliers((1, 1, n, d), 80 + flags, "cuda").reshape(n, d)
    kp, kn, vp, vn = tq.tq_encode(k, v, 4, 2, SEED, flags=flags)
    torch.cuda.synchronize()
    rows = np.sort(np.concatenate([np.random.default_rng(flags).choice(n - 64, 3000, replace=False),
                                   np.arange(n - 64, n)]))
    ridx = torch.from_numpy(rows).cuda()
    tally = BandTally()
    for x, bits, p, nm in ((k, 4, kp, kn), (v, 2, vp, vn)):
        xs = x[ridx].float().cpu().numpy()
        op, on, u = orc.encode(xs, d, bits, SEED, density=density, want_u=True,
                               two_sided=bool(flags & 2))
        _, bnd = orc.codebook_float(d, bits, density)
        gp, gn = p[ridx].cpu().numpy(), nm[ridx].cpu().numpy()
        check_norms(gn, on)
        check_indices(gp, op, u, d, bits, bnd, tally=tally)
        xd = tq.tq_decode(p, nm, d, bits, SEED, flags=flags)[ridx].cpu().numpy()
        check_decoded(xd, orc.decode(gp, gn, d, bits, SEED, density=density,
                                     two_sided=bool(flags & 2)))
    tally.check()
