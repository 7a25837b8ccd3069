// Decode-step attention over the compressed cache, in the rotated domain.
//
// Pages (cited by title and section):
//   "TurboQuant KV Cache Compression — Spec", Optimization: Fused
//     dequant-dot -- since the rotation R is orthogonal, <q, R^T k'> =
//     <R q, k'>: rotate q once, score against centroid values directly,
//     accumulate the V sum in the rotated domain, rotate the output back once.
//   "TurboQuantEngine — Specification", 6 P1 follow-ups, "Compressed-domain
//     attention".
//
// With k_t = D H (n_t c_K[idx_t]) / sqrt(d) (decode), the score is
//   scale <q, k_t> = scale n_t <H (D q) / sqrt(d), c_K[idx_t]>,
// and sum_t p_t v_t = D H (sum_t p_t n^V_t c_V[idx^V_t]) / sqrt(d).
//
// Split over the context: workgroup (chunk, kv head, sequence) handles the G
// query heads of one KV head (or four of eight) over one chunk of rows with
// an online softmax (scores in log2 units) and writes (o', max, sum) for its
// chunk.  Two scans: the exchange scan (two or more query heads per KV head)
// passes each tile's partial scores through LDS so that one lane per row
// takes the row's softmax; the per-lane scan (one query head per KV head)
// keeps every row's scores on all the lanes that hold the row.  With the
// sparse-V gate each wave takes whole 256-row blocks (the gate compares each
// row with its block's maximum) and loads V only for kept rows.  A second
// kernel merges the chunks of each (sequence, query head) in chunk order
// (log-sum-exp) and applies the single inverse rotation.  No atomics; the
// order of every sum is fixed.  With the two-sided rotation S2 H S1, q' takes
// S2 after H and o' takes S2 before it.
//
// Centroid lookup: neighbouring indices address a table of centroid tuples in
// LDS, one read per lookup: pairs (2*bits bits) for 3/4-bit sides,
// quadruples for 2-bit sides.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <mutex>
#include <string>
#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

using namespace tqd;

namespace {

constexpr int kTile = 256;           // rows per online-softmax tile (= threads)
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
    const uint16_t *q;        // [B][Hq][D] bf16
    const uint8_t *kp;        // layer K packed rows [B][Hkv][window][D*BK/8]
    const float *kn;          // [B][Hkv][window]
    const uint8_t *vp;
    const float *vn;
    float *part;              // [B][Hq][n_chunks][D + 4]: o'[D], max, sum
    float *cmax;              // sparse-V gate: [B][Hq][n_chunks] chunk maxima of the scores
    float *scores;            // sparse-V gate: [B][Hkv * gsplit][T][G / gsplit] scores
    float *out;               // [B][Hq][D]
    int Hq, Hkv, window, T, n_chunks, chunk_len;
    int gsplit;               // workgroups per KV head, each taking G of its query heads
    int d_in;                 // head_dim of q and out (<= D; padded to D inside)
    float qscale;             // scale * log2(e) / sqrt(D)
    float gate_log2;          // sparse-V gate: log2(threshold), -inf when off
    float centK[16];
    float centV[16];
    uint32_t signs[8];
    uint32_t signs2[8];       // second diagonal (two-sided rotation), else zero
};

// The workgroup's (chunk, group y, sequence).  With two workgroups per KV
// head (gsplit = 2) both read the KV head's rows: the launch's linear
// workgroup ids are remapped so that the two of a pair are 8 ids apart, which
// puts them on the same XCD (workgroups go to the 8 XCDs in turn) at about the
// same time, and the second read of the rows hits that XCD's L2.  A bijection:
// each run of 16 ids holds 8 pairs; the last, shorter run pairs neighbours.
struct AttnBlock {
    int chunk, y, b;
};

__device__ __forceinline__ AttnBlock attn_block(const AttnParams &p)
{
    if (p.gsplit != 2)
        return AttnBlock{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
    const uint32_t nx = gridDim.x, ny = gridDim.y, n = nx * ny * gridDim.z;
    const uint32_t L = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const uint32_t full = n & ~15u;
    uint32_t pair, half;
    if (L < full) {
        half = (L >> 3) & 1u;
        pair = (L >> 4) * 8u + (L & 7u);
    } else {
        half = (L - full) & 1u;
        pair = full / 2u + (L - full) / 2u;
    }
    const uint32_t nyp = ny / 2u, rest = pair / nx;
    return AttnBlock{(int)(pair % nx), (int)(2u * (rest % nyp) + half), (int)(rest / nyp)};
}

template <int M>
__device__ __forceinline__ float lane_xor_any(float v)
{
    if constexpr (M >= 32)
        return __shfl_xor(v, M);
    else
        return lane_xor<M>(v);
}

// x, with its known bits hidden from the compiler: keeps a value built for
// byte-wise use (fields already shifted into place) from being folded back
// into its inputs at every use
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x)
{
    asm("" : "+v"(x));
    return x;
}

__device__ __forceinline__ float wave_max(float x)
{
    x = max_across<32>(x);
    return fmaxf(x, __shfl_xor(x, 32));
}

// Bits of one lane's slice of a packed row: CPL indices of BITS bits starting
// at byte `off` from `base` (the slice never crosses the row end; rows are a
// multiple of 4 bytes, of 8 where the slice is 8 bytes).  Reads the 4-byte
// words that cover it and shifts the slice down to bit 0.  One unsigned
// 32-bit offset from a uniform base: a scalar base and a vector offset per
// load, no 64-bit address arithmetic.
template <int BITS, int CPL>
__device__ __forceinline__ uint64_t load_slice_bits(const uint8_t *base, uint32_t off)
{
    constexpr int NB = CPL * BITS / 8;  // bytes in the slice
    if constexpr (NB == 8) {
        return *reinterpret_cast<const uint64_t *>(base + off);  // off % 8 == 0
    } else if constexpr (NB == 4) {
        return *reinterpret_cast<const uint32_t *>(base + off);  // off % 4 == 0
    } else if constexpr (NB == 2) {
        return *reinterpret_cast<const uint16_t *>(base + off);  // off % 2 == 0
    } else {
        const uint32_t a = off & ~3u, sh = off & 3u;
        const uint32_t *w = reinterpret_cast<const uint32_t *>(base + a);
        uint64_t v = w[0];
        if (sh + NB > 4)
            v |= (uint64_t)w[1] << 32;
        return (v >> (8 * sh)) & ((1ull << (8 * NB)) - 1ull);
    }
}

// Centroid lookups: neighbouring indices address a table of centroid tuples
// in LDS, one read per lookup.  3- and 4-bit indices go in pairs (64- and
// 256-entry tables of float2).  2-bit indices go in quadruples (one byte, a
// 256-entry table of float4: one address instruction per four coordinates)
// where four or more query heads share a KV head, which makes the scan
// vector-ALU bound; with one or two the scan is bound by the LDS, and pairs
// (a 16-entry, 128-byte table whose reads hit distinct banks) measured faster
// than the 4 KB quadruple table's bank conflicts.
template <int BITS, int G>
struct Lookup {
    static constexpr int W = BITS == 2 && G >= 4 ? 4 : 2;  // coordinates per lookup
    static constexpr int N = 1 << (W * BITS);              // table entries
};

template <int BITS, int G>
__device__ __forceinline__ void fill_lookup(float *tab, const float *cent)
{
    constexpr int W = Lookup<BITS, G>::W, N = Lookup<BITS, G>::N;
    for (int e = threadIdx.x; e < N; e += kBlock)
#pragma unroll
        for (int j = 0; j < W; j++)
            tab[W * e + j] = cent[(e >> (BITS * j)) & ((1 << BITS) - 1)];
}

// the W centroids of lookup m of a lane's slice bits
template <int BITS, int G>
__device__ __forceinline__ void lookup(const float *tab, uint64_t bits, int m, float *cc)
{
    constexpr int W = Lookup<BITS, G>::W, N = Lookup<BITS, G>::N;
    const int e = (int)((bits >> (W * BITS * m)) & (N - 1));
    if constexpr (W == 4) {
        const float4 v = *reinterpret_cast<const float4 *>(tab + 4 * e);
        cc[0] = v.x; cc[1] = v.y; cc[2] = v.z; cc[3] = v.w;
    } else {
        const float2 v = *reinterpret_cast<const float2 *>(tab + 2 * e);
        cc[0] = v.x; cc[1] = v.y;
    }
}

// Layout of the exchange scan: P lanes share a row (CPL coordinates each), a
// step covers one 256-row tile in P row passes, and lane `sub` of a row group
// owns the softmax of the group's row in pass `sub`.  It takes this path when
// the partial scores of a step (P x G per row) fit a small LDS block and there
// are at least two query heads per KV head: with one, the per-lane softmax it
// removes is too small to pay for the two LDS round trips per tile (measured
// slower at head_dim 64, 128 and 256 with long contexts).
template <int D, int G>
struct Xch {
    static constexpr int CPL = G >= 8 ? 8 : 16;
    static constexpr int P = D / CPL;
    static constexpr int RPW = 64 / P;
    static constexpr int RPB = RPW * (kBlock / 64);
    static constexpr bool ON = P * G <= 32 && G >= 2;
    static constexpr int XS = P * G + 4;  // floats per (row group, pass): P partials x G heads, padded
    static constexpr int XW = P * G + 4;  // floats per row group of weights, padded
    static constexpr int FLOATS = RPW * P * XS + RPW * XW;  // per wave
};

// G consecutive floats (LDS or global memory), as one access where the
// width allows
template <int G>
__device__ __forceinline__ void put_vec(float *dst, const float (&v)[G])
{
    if constexpr (G == 4) {
        *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (G == 2) {
        *reinterpret_cast<float2 *>(dst) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
        for (int h = 0; h < G; h++)
            dst[h] = v[h];
    }
}

template <int G>
__device__ __forceinline__ void get_vec(const float *src, float (&v)[G])
{
    if constexpr (G == 4) {
        const float4 t = *reinterpret_cast<const float4 *>(src);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else if constexpr (G == 2) {
        const float2 t = *reinterpret_cast<const float2 *>(src);
        v[0] = t.x; v[1] = t.y;
    } else {
#pragma unroll
        for (int h = 0; h < G; h++)
            v[h] = src[h];
    }
}

// Exchange scan, first half: the partial scores of the P rows of this lane's
// row group over its coordinate slice, into the group's LDS block (`xrow`,
// pass-major), then this lane's row's G scores as the P partials added in
// lane order.
template <int D, int BK, int G>
__device__ __forceinline__ void xch_scores(const float *tabK, float *xrow,
                                           const float (&qr)[G][Xch<D, G>::CPL],
                                           const uint64_t (&kb)[Xch<D, G>::P], int sub,
                                           float (&sc)[G])
{
    using X = Xch<D, G>;
    constexpr int CPL = X::CPL, P = X::P, WK = Lookup<BK, G>::W;
#pragma unroll
    for (int c = 0; c < P; c++) {
        float s[G];
#pragma unroll
        for (int h = 0; h < G; h++)
            s[h] = 0.0f;
#pragma unroll
        for (int m = 0; m < CPL / WK; m++) {
            float cc[WK];
            lookup<BK, G>(tabK, kb[c], m, cc);
#pragma unroll
            for (int j = 0; j < WK; j++)
#pragma unroll
                for (int h = 0; h < G; h++)
                    s[h] = fmaf(qr[h][WK * m + j], cc[j], s[h]);
        }
        put_vec<G>(xrow + c * X::XS + sub * G, s);
    }
    wave_lds_fence();
#pragma unroll
    for (int h = 0; h < G; h++)
        sc[h] = 0.0f;
#pragma unroll
    for (int j = 0; j < P; j++) {
        float v[G];
        get_vec<G>(xrow + sub * X::XS + j * G, v);
#pragma unroll
        for (int h = 0; h < G; h++)
            sc[h] += v[h];
    }
}

// Exchange scan, second half: the weighted V slice of one row pass (rotated
// domain) added to this lane's accumulators
template <int D, int BV, int G>
__device__ __forceinline__ void xch_accumulate(const float *tabV, uint64_t vbits,
                                               const float (&wc)[G],
                                               float (&acc)[G][Xch<D, G>::CPL])
{
    constexpr int CPL = Xch<D, G>::CPL, WV = Lookup<BV, G>::W;
#pragma unroll
    for (int m = 0; m < CPL / WV; m++) {
        float cc[WV];
        lookup<BV, G>(tabV, vbits, m, cc);
#pragma unroll
        for (int j = 0; j < WV; j++)
#pragma unroll
            for (int h = 0; h < G; h++)
                acc[h][WV * m + j] = fmaf(wc[h], cc[j], acc[h][WV * m + j]);
    }
}

// One tile of the exchange scan.  The lanes of a row group first score their
// coordinate slices of the group's P rows and write the partial sums to LDS;
// lane `sub` then adds the P partials of row `sub` (in lane order), takes the
// row's G scores and the group's running maximum, and forms the row's weights,
// which go back through LDS so that every lane of the group can accumulate
// the P rows' V slices.  The exponentials are taken once per (row, head)
// rather than on each of the P lanes holding the row.  The running maximum is
// per row group (the groups are merged after the scan).  TAIL: the tile runs
// past the context; those rows read a valid row and are masked.
template <int D, int BK, int BV, int G, bool TAIL>
__device__ __forceinline__ void xch_step(const float *tabK, const float *tabV, float *xs,
                                         float *xw, const float (&qr)[G][Xch<D, G>::CPL],
                                         float (&acc)[G][Xch<D, G>::CPL], float (&m_run)[G],
                                         float (&l_part)[G], const uint8_t *kbase,
                                         const uint8_t *vbase, const float *knb,
                                         const float *vnb, int tw, int t_begin, int t_end,
                                         int sub, int rig)
{
    using X = Xch<D, G>;
    constexpr int CPL = X::CPL, P = X::P, RPB = X::RPB;
    constexpr int RBK = D * BK / 8, RBV = D * BV / 8;
    constexpr int SBK = CPL * BK / 8, SBV = CPL * BV / 8;
    uint64_t kb[P], vb[P];
#pragma unroll
    for (int c = 0; c < P; c++) {
        int t = tw + c * RPB;
        if constexpr (TAIL)
            t = t < t_end ? t : t_begin;
        kb[c] = load_slice_bits<BK, CPL>(kbase, (uint32_t)t * RBK + (uint32_t)(sub * SBK));
        vb[c] = load_slice_bits<BV, CPL>(vbase, (uint32_t)t * RBV + (uint32_t)(sub * SBV));
    }
    int to = tw + sub * RPB;  // the row this lane takes the softmax of
    const bool valid = to < t_end;
    if constexpr (TAIL)
        to = valid ? to : t_begin;
    const float kn = knb[to], vn = vnb[to];

    float *xrow = xs + rig * P * X::XS;
    float sc[G];
    xch_scores<D, BK, G>(tabK, xrow, qr, kb, sub, sc);
    float w[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        sc[h] *= kn;
        if constexpr (TAIL)
            sc[h] = valid ? sc[h] : -__builtin_huge_valf();
        const float mx = max_across<P>(sc[h]);  // the row group's maximum
        if (mx > m_run[h]) {
            const float fac = exp2f(m_run[h] - mx);  // 0 on the group's first valid tile
            l_part[h] *= fac;
#pragma unroll
            for (int k = 0; k < CPL; k++)
                acc[h][k] *= fac;
            m_run[h] = mx;
        }
        float pr = __builtin_amdgcn_exp2f(sc[h] - m_run[h]);
        if constexpr (TAIL)
            pr = m_run[h] == -__builtin_huge_valf() ? 0.0f : pr;  // no valid row yet
        l_part[h] += pr;
        w[h] = pr * vn;
    }
    float *wrow = xw + rig * X::XW;
    put_vec<G>(wrow + sub * G, w);
    wave_lds_fence();
#pragma unroll
    for (int c = 0; c < P; c++) {
        float wc[G];
        get_vec<G>(wrow + c * G, wc);
        xch_accumulate<D, BV, G>(tabV, vb[c], wc, acc);
    }
    wave_lds_fence();  // every lane is done with this tile's LDS blocks
}

// q' = S2 H (D q) * scale * log2(e) / sqrt(d) for query heads h0 .. h0 + G - 1
// of sequence b (S2 = identity for the one-sided rotation), into qs[G][D].
// Wave 0 rotates; the caller synchronises the workgroup before reading qs.
template <int D, int G>
__device__ __forceinline__ void rotate_queries(const AttnParams &p, float (*qs)[D], int b, int h0,
                                               int wave, int lane)
{
    if (wave != 0)
        return;
    constexpr int P2 = D / kCPL;
    const int sub2 = lane % P2, r2 = lane / P2;
    float v[kCPL];
    const int h = h0 + (r2 < G ? r2 : 0);
    if (sub2 * kCPL < p.d_in) {
        load_slice(p.q + ((int64_t)b * p.Hq + h) * p.d_in + sub2 * kCPL, v);
    } else {
#pragma unroll
        for (int k = 0; k < kCPL; k++)
            v[k] = 0.0f;  // the zero padding of a head_dim below D
    }
    apply_signs(v, p.signs[sub2]);
    fwht_row<P2>(v, sub2);
    apply_signs(v, p.signs2[sub2]);
    if (r2 < G) {
#pragma unroll
        for (int k = 0; k < kCPL; k++)
            qs[r2][sub2 * kCPL + k] = v[k] * p.qscale;
    }
}

// This lane's coordinate slice of the G rotated queries
template <int D, int G, int CPL>
__device__ __forceinline__ void query_slices(const float (*qs)[D], int sub, float (&qr)[G][CPL])
{
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int k = 0; k < CPL; k++)
            qr[h][k] = qs[h][sub * CPL + k];
}

// The end of a chunk: each wave's (o', max, sum) reduced over its row groups
// (every lane of a row group holds the same sum, so the sums reduce across
// row groups only), the waves merged by log-sum-exp through LDS (accs holds
// wave w's o' at w * AST), and the chunk's record (o'[D], max, sum) of each
// of the G query heads written to the workspace.
template <int D, int G, int CPL, int AST>
__device__ __forceinline__ void write_chunk_record(const AttnParams &p, float (&acc)[G][CPL],
                                                   const float (&m_run)[G], float (&l_part)[G],
                                                   float *accs, float (*red_m)[G],
                                                   float (*red_l)[G], int b, int h0, int chunk)
{
    constexpr int P = D / CPL, RS = D + 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane % P, rig = lane / P;
#pragma unroll
    for (int h = 0; h < G; h++) {
        float l = l_part[h];
        if constexpr (P <= 1) l += lane_xor_any<1>(l);
        if constexpr (P <= 2) l += lane_xor_any<2>(l);
        if constexpr (P <= 4) l += lane_xor_any<4>(l);
        if constexpr (P <= 8) l += lane_xor_any<8>(l);
        if constexpr (P <= 16) l += lane_xor_any<16>(l);
        if constexpr (P <= 32) l += lane_xor_any<32>(l);
        l_part[h] = l;
#pragma unroll
        for (int k = 0; k < CPL; k++) {
            float a = acc[h][k];
            if constexpr (P <= 1) a += lane_xor_any<1>(a);
            if constexpr (P <= 2) a += lane_xor_any<2>(a);
            if constexpr (P <= 4) a += lane_xor_any<4>(a);
            if constexpr (P <= 8) a += lane_xor_any<8>(a);
            if constexpr (P <= 16) a += lane_xor_any<16>(a);
            if constexpr (P <= 32) a += lane_xor_any<32>(a);
            acc[h][k] = a;
        }
    }
    if (rig == 0) {
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int k = 0; k < CPL; k++)
                accs[wave * AST + h * D + sub * CPL + k] = acc[h][k];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; h++) {
            red_m[wave][h] = m_run[h];
            red_l[wave][h] = l_part[h];
        }
    }
    __syncthreads();
    float *rec0 = p.part + (((int64_t)b * p.Hq + h0) * p.n_chunks + chunk) * RS;
    const int64_t hstride = (int64_t)p.n_chunks * RS;
    for (int i = tid; i < G * D; i += kBlock) {
        const int h = i / D, j = i % D;
        float M = red_m[0][h];
#pragma unroll
        for (int w = 1; w < kBlock / 64; w++)
            M = fmaxf(M, red_m[w][h]);
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < kBlock / 64; w++) {
            const float mw = red_m[w][h];
            o += mw == -__builtin_huge_valf() ? 0.0f : exp2f(mw - M) * accs[w * AST + h * D + j];
        }
        rec0[h * hstride + j] = o;
    }
    if (tid < G) {
        float M = red_m[0][tid];
#pragma unroll
        for (int w = 1; w < kBlock / 64; w++)
            M = fmaxf(M, red_m[w][tid]);
        float l = 0.0f;
#pragma unroll
        for (int w = 0; w < kBlock / 64; w++) {
            const float mw = red_m[w][tid];
            l += mw == -__builtin_huge_valf() ? 0.0f : exp2f(mw - M) * red_l[w][tid];
        }
        rec0[tid * hstride + D] = M;
        rec0[tid * hstride + D + 1] = l;
    }
}

// Partial results of one chunk.  The exchange scan (above) runs where its LDS
// blocks fit and there are at least two query heads per KV head; otherwise
// the per-lane scan: each wave keeps its rows' scores in registers (every lane
// of a row holds the row's sums), runs its own running maximum (wave-uniform)
// and sum, and accumulates V right after each step of CH row passes, with no
// LDS traffic for scores and no barrier inside the scan.  Either way the four
// waves' (o', max, sum) are merged once at the end.  Per-lane rows of wave w:
// t_begin + it * RPB + w * RPW + (lane / P).
template <int D, int BK, int BV, int G>
__global__ __launch_bounds__(kBlock) void attn_partial_wave_kernel(AttnParams p)
{
    constexpr int CPL = G >= 8 ? 8 : 16;  // coordinates per lane in the scan
    constexpr int P = D / CPL;            // lanes per row
    constexpr int RPW = 64 / P;
    constexpr int RPB = RPW * (kBlock / 64);
    constexpr int RBK = D * BK / 8, RBV = D * BV / 8;
    constexpr int CH = G >= 8 ? 4 : 8;    // row passes per step
    constexpr int WK = Lookup<BK, G>::W, WV = Lookup<BV, G>::W;

    __shared__ __attribute__((aligned(16))) float tabK[Lookup<BK, G>::N * WK];
    __shared__ __attribute__((aligned(16))) float tabV[Lookup<BV, G>::N * WV];
    __shared__ float qs[G][D];
    __shared__ float red_m[kBlock / 64][G];
    __shared__ float red_l[kBlock / 64][G];
    // exchange scan: each wave's LDS blocks of partial scores and weights;
    // after the scan the same wave-owned region holds the wave's o' (accs)
    constexpr bool XON = Xch<D, G>::ON;
    constexpr int XFL = Xch<D, G>::FLOATS;
    constexpr int AST = XON && XFL > G * D ? XFL : G * D;
    __shared__ __attribute__((aligned(16))) float accs[kBlock / 64 * AST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const AttnBlock blk = attn_block(p);
    const int chunk = blk.chunk, b = blk.b;
    const int g = blk.y / p.gsplit;  // KV head
    const int h0 = blk.y * G;        // first of this workgroup's G query heads

    fill_lookup<BK, G>(tabK, p.centK);
    fill_lookup<BV, G>(tabV, p.centV);
    rotate_queries<D, G>(p, qs, b, h0, wave, lane);
    __syncthreads();

    const int sub = lane % P, rig = lane / P;
    float qr[G][CPL];
    query_slices<D, G, CPL>(qs, sub, qr);

    float acc[G][CPL];
    float m_run[G], l_part[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        m_run[h] = -__builtin_huge_valf();
        l_part[h] = 0.0f;
#pragma unroll
        for (int k = 0; k < CPL; k++)
            acc[h][k] = 0.0f;
    }

    const int64_t rowbase = ((int64_t)b * p.Hkv + g) * p.window;
    const int t_begin = chunk * p.chunk_len;
    const int t_end = min(p.T, t_begin + p.chunk_len);

    if constexpr (XON) {
        using X = Xch<D, G>;
        float *xs = accs + wave * AST;
        float *xw = xs + X::RPW * X::P * X::XS;
        const uint8_t *kbase = p.kp + rowbase * RBK;
        const uint8_t *vbase = p.vp + rowbase * RBV;
        const float *knb = p.kn + rowbase, *vnb = p.vn + rowbase;
        // tiles of 256 rows (chunks start on tile boundaries); the last one
        // may run past the context
        int t0 = t_begin;
#pragma unroll 1
        for (; t0 + kTile <= t_end; t0 += kTile)
            xch_step<D, BK, BV, G, false>(tabK, tabV, xs, xw, qr, acc, m_run, l_part, kbase, vbase,
                                          knb, vnb, t0 + wave * RPW + rig, t_begin, t_end, sub,
                                          rig);
        if (t0 < t_end)
            xch_step<D, BK, BV, G, true>(tabK, tabV, xs, xw, qr, acc, m_run, l_part, kbase, vbase,
                                         knb, vnb, t0 + wave * RPW + rig, t_begin, t_end, sub,
                                         rig);
        // bring the row groups to the wave's maximum; each lane's sum covers
        // its own rows, so the sums add within the group first
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float M = wave_max(m_run[h]);
            const float f = m_run[h] == -__builtin_huge_valf() ? 0.0f : exp2f(m_run[h] - M);
            l_part[h] = sum_across<P>(l_part[h] * f);
#pragma unroll
            for (int k = 0; k < CPL; k++)
                acc[h][k] *= f;
            m_run[h] = M;
        }
    } else {
    // steps of CH row passes (CH * RPB rows); 32-bit row offsets from uniform
    // bases; only a step that runs past the context (the last) masks rows
    const uint8_t *kbase = p.kp + rowbase * RBK;
    const uint8_t *vbase = p.vp + rowbase * RBV;
    const float *knb = p.kn + rowbase, *vnb = p.vn + rowbase;
    auto step = [&](const int s0, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const int t0 = s0 + wave * RPW + rig;  // this lane's row in pass 0
        // every K and V load of the step in flight before any arithmetic;
        // rows past the context read the last row and are masked below
        uint64_t kb[CH], vb[CH];
        float kn[CH], vn[CH];
#pragma unroll
        for (int c = 0; c < CH; c++) {
            int t = t0 + c * RPB;
            if constexpr (TAIL)
                t = min(t, t_end - 1);
            kb[c] = load_slice_bits<BK, CPL>(kbase,
                                             (uint32_t)t * RBK + (uint32_t)(sub * (CPL * BK / 8)));
            kn[c] = knb[t];
            vb[c] = load_slice_bits<BV, CPL>(vbase,
                                             (uint32_t)t * RBV + (uint32_t)(sub * (CPL * BV / 8)));
            vn[c] = vnb[t];
        }
        // scores (log2 units), every lane of a row holding its row's value
        float sc[CH][G];
#pragma unroll
        for (int c = 0; c < CH; c++) {
            float s[G];
#pragma unroll
            for (int h = 0; h < G; h++)
                s[h] = 0.0f;
#pragma unroll
            for (int m = 0; m < CPL / WK; m++) {
                float cc[WK];
                lookup<BK, G>(tabK, kb[c], m, cc);
#pragma unroll
                for (int j = 0; j < WK; j++)
#pragma unroll
                    for (int h = 0; h < G; h++)
                        s[h] = fmaf(qr[h][WK * m + j], cc[j], s[h]);
            }
            // the row's sum is taken whether or not the row is valid: a
            // select afterwards, not a branch around the cross-lane sum
#pragma unroll
            for (int h = 0; h < G; h++)
                s[h] = sum_across<P>(s[h]) * kn[c];
            const bool valid = !TAIL || t0 + c * RPB < t_end;
#pragma unroll
            for (int h = 0; h < G; h++)
                sc[c][h] = valid ? s[h] : -__builtin_huge_valf();
        }
        // running maximum of the wave; rescale only when it grows
#pragma unroll
        for (int h = 0; h < G; h++) {
            float mx = sc[0][h];
#pragma unroll
            for (int c = 1; c < CH; c++)
                mx = fmaxf(mx, sc[c][h]);
            mx = wave_max(mx);
            if (mx > m_run[h]) {
                const float fac = exp2f(m_run[h] - mx);  // 0 on the first valid step
                l_part[h] *= fac;
#pragma unroll
                for (int k = 0; k < CPL; k++)
                    acc[h][k] *= fac;
                m_run[h] = mx;
            }
        }
        // weights and the V sum of the step (rotated domain)
#pragma unroll
        for (int c = 0; c < CH; c++) {
            float w[G];
#pragma unroll
            for (int h = 0; h < G; h++) {
                // weights below 2^-126 flush to 0 (v_exp_f32); m_run is -inf
                // only while the wave has seen no valid row, which a step
                // inside the context cannot leave behind
                float pr = __builtin_amdgcn_exp2f(sc[c][h] - m_run[h]);
                if constexpr (TAIL)
                    pr = m_run[h] == -__builtin_huge_valf() ? 0.0f : pr;
                l_part[h] += pr;
                w[h] = pr * vn[c];
            }
#pragma unroll
            for (int m = 0; m < CPL / WV; m++) {
                float cc[WV];
                lookup<BV, G>(tabV, vb[c], m, cc);
#pragma unroll
                for (int j = 0; j < WV; j++)
#pragma unroll
                    for (int h = 0; h < G; h++)
                        acc[h][WV * m + j] = fmaf(w[h], cc[j], acc[h][WV * m + j]);
            }
        }
    };
    constexpr int SR = CH * RPB;  // rows per step of the workgroup
    int s0 = t_begin;
#pragma unroll 1
    for (; s0 + SR <= t_end; s0 += SR)
        step(s0, std::integral_constant<bool, false>{});
    if (s0 < t_end)
        step(s0, std::integral_constant<bool, true>{});
    }

    write_chunk_record<D, G, CPL, AST>(p, acc, m_run, l_part, accs, red_m, red_l, b, h0, chunk);
}

// ---- One query head per KV head: the row scan.  With a single query the
// score of a key row is a sum over its coordinate pairs of a value that
// depends only on the pair's two indices: the workgroup tabulates the
// query's partial score for every pair position and index pair, (D/2) x
// 4^BK floats ([Foundry] "Optimization: Fused dequant-dot": the rotated
// query against centroid values, here taken two coordinates at a time).
// Each lane then scores one whole row, one LDS read and one add per pair
// (all lanes of a read address the same table row, so lanes with equal
// index pairs share a read), and the row's softmax terms are computed once,
// not on every lane that holds a slice of it.  The V sum
// keeps the coordinate split of the per-lane scan (P lanes per row, CPL
// coordinates each); the weights of a wave's 64 rows reach those lanes
// through a small per-wave LDS buffer.  Wave w takes rows
// t_begin + 256 i + 64 w + lane of its chunk.
template <int D, int BK>
struct RowScan {
    static constexpr int QN = 1 << (2 * BK);  // table entries per coordinate pair
    static constexpr bool ON = BK <= 3 || D * QN * 2 <= 32768;  // table <= 32 KB
};

template <int D, int BK, int BV>
__global__ __launch_bounds__(kBlock) void attn_partial_row_kernel(AttnParams p)
{
    constexpr int QN = RowScan<D, BK>::QN;
    constexpr int NPAIR = D / 2;
    constexpr int RBK = D * BK / 8, RBV = D * BV / 8;
    constexpr int KW = RBK / 4;               // 32-bit words of a key row
    constexpr int CPL = 16, P = D / CPL;      // V: lanes per row, coordinates per lane
    constexpr int RPW = 64 / P;               // V: rows per pass of a wave
    constexpr int NPASS = 64 / RPW;           // V: passes per 64 rows
    constexpr int WV = Lookup<BV, 1>::W;
    static_assert(RBK % 8 == 0 && QN <= kBlock, "row scan layout");

    __shared__ float qtab[NPAIR * QN];
    __shared__ __attribute__((aligned(16))) float tabV[Lookup<BV, 1>::N * WV];
    __shared__ float qs[1][D];
    __shared__ float wbuf[kBlock];            // each wave's 64 weights of the current rows
    __shared__ float red_m[kBlock / 64][1];
    __shared__ float red_l[kBlock / 64][1];
    __shared__ __attribute__((aligned(16))) float accs[kBlock / 64 * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;

    fill_lookup<BV, 1>(tabV, p.centV);
    rotate_queries<D, 1>(p, qs, b, g, wave, lane);
    __syncthreads();
    {
        // entry e of pair m: q'[2m] c[e's low BK bits] + q'[2m+1] c[its high
        // BK bits]; thread t fills the entries e = t % QN of pairs
        // m = t / QN, + kBlock / QN, ...
        const int e = tid % QN;
        const float c0 = p.centK[e & ((1 << BK) - 1)], c1 = p.centK[e >> BK];
        for (int m = tid / QN; m < NPAIR; m += kBlock / QN)
            qtab[m * QN + e] = fmaf(qs[0][2 * m + 1], c1, qs[0][2 * m] * c0);
    }
    __syncthreads();

    const int sub = lane % P, rig = lane / P;
    float acc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; k++)
        acc[k] = 0.0f;
    float m_run = -__builtin_huge_valf();  // the wave's running maximum
    float l_run = 0.0f;                     // this lane's rows' weights

    const int64_t rowbase = ((int64_t)b * p.Hkv + g) * p.window;
    const uint8_t *kbase = p.kp + rowbase * RBK;
    const uint8_t *vbase = p.vp + rowbase * RBV;
    const float *knb = p.kn + rowbase, *vnb = p.vn + rowbase;
    const int t_begin = chunk * p.chunk_len;
    const int t_end = min(p.T, t_begin + p.chunk_len);
    float *wrow = wbuf + wave * 64;

#pragma unroll 1
    for (int t0 = t_begin + 64 * wave; t0 < t_end; t0 += kBlock) {
        // this lane's key row and both norms; the V slices of the wave's
        // NPASS passes; rows past the context read the last row (masked)
        const int t = t0 + lane;
        const bool valid = t < t_end;
        const int tt = valid ? t : t_end - 1;
        uint32_t kw[KW];
        {
            const uint2 *kr = reinterpret_cast<const uint2 *>(kbase + (uint32_t)tt * RBK);
#pragma unroll
            for (int i = 0; i < KW / 2; i++) {
                const uint2 v = kr[i];
                kw[2 * i] = v.x;
                kw[2 * i + 1] = v.y;
            }
        }
        const float kn = knb[tt], vn = vnb[tt];
        uint64_t vb[NPASS];  // CPL * BV bits each
#pragma unroll
        for (int j = 0; j < NPASS; j++) {
            const int tv = min(t0 + j * RPW + rig, t_end - 1);
            vb[j] = load_slice_bits<BV, CPL>(vbase,
                                             (uint32_t)tv * RBV + (uint32_t)(sub * (CPL * BV / 8)));
        }
        // the row's score (log2 units): pair m's field, shifted to bit 2,
        // addresses entry e of table row m (row offset in the instruction)
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int m = 0; m < NPAIR; m++) {
            constexpr int FW = 2 * BK;
            const int o = FW * m, wi = o / 32, ob = o % 32;
            uint32_t f;
            if (ob + FW > 32)
                f = __builtin_amdgcn_alignbit(kw[wi + 1], kw[wi], ob - 2);
            else if (ob >= 2)
                f = kw[wi] >> (ob - 2);
            else
                f = kw[wi] << (2 - ob);
            const float v = *reinterpret_cast<const float *>(
                reinterpret_cast<const char *>(qtab + m * QN) + (f & (uint32_t)((QN - 1) << 2)));
            if (m & 1)
                s1 += v;
            else
                s0 += v;
        }
        const float sc = valid ? (s0 + s1) * kn : -__builtin_huge_valf();
        // running maximum of the wave (lane 0's row is always valid)
        const float mx = wave_max(sc);
        if (mx > m_run) {
            const float fac = exp2f(m_run - mx);  // 0 on the first rows
            l_run *= fac;
#pragma unroll
            for (int k = 0; k < CPL; k++)
                acc[k] *= fac;
            m_run = mx;
        }
        // weights below 2^-126 flush to 0 (v_exp_f32); invalid rows give 0
        const float pr = __builtin_amdgcn_exp2f(sc - m_run);
        l_run += pr;
        // the weights go to the V lanes through this wave's LDS buffer (one
        // wave writes and reads it; its LDS accesses complete in order)
        wrow[lane] = pr * vn;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < NPASS; j++) {
            const float w = wrow[j * RPW + rig];
            if constexpr (BV == 2) {
                // the eight 4-bit pair indices, times the entry size (8
                // bytes), one to a byte: a table address is one byte extract
                const uint32_t v32 = (uint32_t)vb[j];  // 32 bits at BV = 2
                const uint32_t ev = opaque_u32((v32 << 3) & 0x78787878u);  // pairs 0, 2, 4, 6
                const uint32_t od = opaque_u32((v32 >> 1) & 0x78787878u);  // pairs 1, 3, 5, 7
#pragma unroll
                for (int m = 0; m < 8; m++) {
                    const uint32_t a = __builtin_amdgcn_ubfe(m & 1 ? od : ev, 8 * (m >> 1), 8);
                    const float2 cv = *reinterpret_cast<const float2 *>(
                        reinterpret_cast<const char *>(tabV) + a);
                    acc[2 * m] = fmaf(w, cv.x, acc[2 * m]);
                    acc[2 * m + 1] = fmaf(w, cv.y, acc[2 * m + 1]);
                }
            } else {
#pragma unroll
                for (int m = 0; m < CPL / WV; m++) {
                    float cc[WV];
                    lookup<BV, 1>(tabV, vb[j], m, cc);
#pragma unroll
                    for (int q = 0; q < WV; q++)
                        acc[WV * m + q] = fmaf(w, cc[q], acc[WV * m + q]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // the chunk record: the epilogue sums each coordinate slice over the
    // lanes of its rig and expects the weight sum the same way, so the
    // wave's total goes to the rig-0 lanes
    float l_tot = l_run;
    l_tot += lane_xor_any<1>(l_tot);
    l_tot += lane_xor_any<2>(l_tot);
    l_tot += lane_xor_any<4>(l_tot);
    l_tot += lane_xor_any<8>(l_tot);
    l_tot += lane_xor_any<16>(l_tot);
    l_tot += lane_xor_any<32>(l_tot);
    float acc1[1][CPL], m1[1] = {m_run}, l1[1] = {rig == 0 ? l_tot : 0.0f};
#pragma unroll
    for (int k = 0; k < CPL; k++)
        acc1[0][k] = acc[k];
    write_chunk_record<D, 1, CPL, D>(p, acc1, m1, l1, accs, red_m, red_l, b, g, chunk);
}

// ---- The sparse-V gate ([Atlas] "Sparse V dequant"): the V row of a slot is
// loaded and decoded only where the row's weight relative to the largest
// weight of the context, exp(score - max score), exceeds the threshold;
// every row stays in the softmax denominator.  The maximum needs every score
// of the context, so the gated path runs two passes over the chunks.
// attn_scores_kernel reads K only: each row's scores (log2 units) go to the
// workspace, [B][n_grp][T][G] (the G query heads of a workgroup together;
// n_grp = Hkv * gsplit), and each chunk's largest score per head to cmax.
// attn_gated_v_kernel takes the context maximum from all chunk maxima, adds
// every row's weight to the denominator and loads V only for the rows some
// head keeps.  Its chunk records carry the context maximum, and the combine
// kernel merges them like the ungated ones.
template <int D, int BK, int G>
__global__ __launch_bounds__(kBlock) void attn_scores_kernel(AttnParams p)
{
    constexpr int CPL = G >= 8 ? 8 : 16;
    constexpr int P = D / CPL, RPW = 64 / P, RPB = RPW * (kBlock / 64);
    constexpr int RBK = D * BK / 8, SBK = CPL * BK / 8;
    constexpr int WK = Lookup<BK, G>::W;
    constexpr int CH = G >= 8 ? 4 : 8;  // row passes per step of the per-lane form
    using X = Xch<D, G>;
    constexpr bool XON = X::ON;

    __shared__ __attribute__((aligned(16))) float tabK[Lookup<BK, G>::N * WK];
    __shared__ float qs[G][D];
    __shared__ float red_m[kBlock / 64][G];
    __shared__ __attribute__((aligned(16))) float xbuf[XON ? kBlock / 64 * X::FLOATS : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const AttnBlock blk = attn_block(p);
    const int chunk = blk.chunk, b = blk.b;
    const int g = blk.y / p.gsplit;
    const int h0 = blk.y * G;
    fill_lookup<BK, G>(tabK, p.centK);
    rotate_queries<D, G>(p, qs, b, h0, wave, lane);
    __syncthreads();
    const int sub = lane % P, rig = lane / P;
    float qr[G][CPL];
    query_slices<D, G, CPL>(qs, sub, qr);

    const int64_t rowbase = ((int64_t)b * p.Hkv + g) * p.window;
    const uint8_t *kbase = p.kp + rowbase * RBK;
    const float *knb = p.kn + rowbase;
    float *srow = p.scores + ((int64_t)b * gridDim.y + blk.y) * p.T * G;
    const int t_begin = chunk * p.chunk_len;
    const int t_end = min(p.T, t_begin + p.chunk_len);
    float mx[G];
#pragma unroll
    for (int h = 0; h < G; h++)
        mx[h] = -__builtin_huge_valf();

    if constexpr (XON) {
        // tiles of 256 rows: P row passes per wave, lane `sub` of a row group
        // sums the partials of the group's row of pass `sub` (exchange scan)
        float *xrow = xbuf + wave * X::FLOATS + rig * P * X::XS;
#pragma unroll 1
        for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
            const int tw = t0 + wave * RPW + rig;
            uint64_t kb[P];
#pragma unroll
            for (int c = 0; c < P; c++) {
                const int t = min(tw + c * RPB, t_end - 1);
                kb[c] = load_slice_bits<BK, CPL>(kbase, (uint32_t)t * RBK + (uint32_t)(sub * SBK));
            }
            const int to = tw + sub * RPB;
            const float kn = knb[min(to, t_end - 1)];
            float sc[G];
            xch_scores<D, BK, G>(tabK, xrow, qr, kb, sub, sc);
            if (to < t_end) {
#pragma unroll
                for (int h = 0; h < G; h++) {
                    sc[h] *= kn;
                    mx[h] = fmaxf(mx[h], sc[h]);
                }
                put_vec<G>(srow + (int64_t)to * G, sc);
            }
            wave_lds_fence();  // the tile's partials are read before the next tile's
        }
    } else {
        // steps of CH row passes; every lane of a row holds the row's sums
#pragma unroll 1
        for (int s0 = t_begin; s0 < t_end; s0 += CH * RPB) {
            const int t0 = s0 + wave * RPW + rig;
            uint64_t kb[CH];
            float kn[CH];
#pragma unroll
            for (int c = 0; c < CH; c++) {
                const int t = min(t0 + c * RPB, t_end - 1);
                kb[c] = load_slice_bits<BK, CPL>(kbase, (uint32_t)t * RBK + (uint32_t)(sub * SBK));
                kn[c] = knb[t];
            }
#pragma unroll
            for (int c = 0; c < CH; c++) {
                float sc[G];
#pragma unroll
                for (int h = 0; h < G; h++)
                    sc[h] = 0.0f;
#pragma unroll
                for (int m = 0; m < CPL / WK; m++) {
                    float cc[WK];
                    lookup<BK, G>(tabK, kb[c], m, cc);
#pragma unroll
                    for (int j = 0; j < WK; j++)
#pragma unroll
                        for (int h = 0; h < G; h++)
                            sc[h] = fmaf(qr[h][WK * m + j], cc[j], sc[h]);
                }
#pragma unroll
                for (int h = 0; h < G; h++)
                    sc[h] = sum_across<P>(sc[h]) * kn[c];
                const int t = t0 + c * RPB;
                if (t < t_end) {
#pragma unroll
                    for (int h = 0; h < G; h++)
                        mx[h] = fmaxf(mx[h], sc[h]);
                    if (sub == 0)
                        put_vec<G>(srow + (int64_t)t * G, sc);
                }
            }
        }
    }
    // the chunk's largest score per head
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float m = wave_max(mx[h]);
        if (lane == 0)
            red_m[wave][h] = m;
    }
    __syncthreads();
    if (tid < G) {
        float m = red_m[0][tid];
#pragma unroll
        for (int w = 1; w < kBlock / 64; w++)
            m = fmaxf(m, red_m[w][tid]);
        p.cmax[((int64_t)b * p.Hq + h0 + tid) * p.n_chunks + chunk] = m;
    }
}

template <int D, int BV, int G>
__global__ __launch_bounds__(kBlock) void attn_gated_v_kernel(AttnParams p)
{
    constexpr int CPL = G >= 8 ? 8 : 16;
    constexpr int P = D / CPL, RPW = 64 / P, RPB = RPW * (kBlock / 64);
    constexpr int RBV = D * BV / 8, SBV = CPL * BV / 8;
    constexpr int WV = Lookup<BV, G>::W;
    constexpr int CH = G >= 8 ? 4 : 8;  // row passes per step
    constexpr int AST = G * D;

    __shared__ __attribute__((aligned(16))) float tabV[Lookup<BV, G>::N * WV];
    __shared__ float red_m[kBlock / 64][G];
    __shared__ float red_l[kBlock / 64][G];
    __shared__ __attribute__((aligned(16))) float accs[kBlock / 64 * AST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const AttnBlock blk = attn_block(p);
    const int chunk = blk.chunk, b = blk.b;
    const int g = blk.y / p.gsplit;
    const int h0 = blk.y * G;
    fill_lookup<BV, G>(tabV, p.centV);
    // the context's largest score of each head: the largest chunk maximum
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float *cm = p.cmax + ((int64_t)b * p.Hq + h0 + h) * p.n_chunks;
        float m = -__builtin_huge_valf();
        for (int c = tid; c < p.n_chunks; c += kBlock)
            m = fmaxf(m, cm[c]);
        m = wave_max(m);
        if (lane == 0)
            red_m[wave][h] = m;
    }
    __syncthreads();
    float M[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        M[h] = red_m[0][h];
#pragma unroll
        for (int w = 1; w < kBlock / 64; w++)
            M[h] = fmaxf(M[h], red_m[w][h]);
    }
    __syncthreads();  // red_m is reused by the record

    const int sub = lane % P, rig = lane / P;
    float acc[G][CPL], l_part[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        l_part[h] = 0.0f;
#pragma unroll
        for (int k = 0; k < CPL; k++)
            acc[h][k] = 0.0f;
    }
    const int64_t rowbase = ((int64_t)b * p.Hkv + g) * p.window;
    const uint8_t *vbase = p.vp + rowbase * RBV;
    const float *vnb = p.vn + rowbase;
    const float *srow = p.scores + ((int64_t)b * gridDim.y + blk.y) * p.T * G;
    const int t_begin = chunk * p.chunk_len;
    const int t_end = min(p.T, t_begin + p.chunk_len);
#pragma unroll 1
    for (int s0 = t_begin; s0 < t_end; s0 += CH * RPB) {
        const int t0 = s0 + wave * RPW + rig;
        float sc[CH][G];
#pragma unroll
        for (int c = 0; c < CH; c++)
            get_vec<G>(srow + (int64_t)min(t0 + c * RPB, t_end - 1) * G, sc[c]);
        // V of the rows some head keeps (the same decision on every lane of a
        // row); no branch around the load: rows nobody keeps read the chunk's
        // first row, which is not used
        uint64_t vb[CH];
        float vn[CH];
        bool kept[CH];
#pragma unroll
        for (int c = 0; c < CH; c++) {
            const int t = t0 + c * RPB;
            bool k = false;
#pragma unroll
            for (int h = 0; h < G; h++)
                k |= sc[c][h] - M[h] > p.gate_log2;
            kept[c] = k && t < t_end;
            const int tv = kept[c] ? t : t_begin;
            vb[c] = load_slice_bits<BV, CPL>(vbase, (uint32_t)tv * RBV + (uint32_t)(sub * SBV));
            vn[c] = vnb[tv];
        }
#pragma unroll
        for (int c = 0; c < CH; c++) {
            const bool valid = t0 + c * RPB < t_end;
            float w[G];
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float pr = valid ? __builtin_amdgcn_exp2f(sc[c][h] - M[h]) : 0.0f;
                l_part[h] += pr;
                w[h] = kept[c] && sc[c][h] - M[h] > p.gate_log2 ? pr * vn[c] : 0.0f;
            }
            if (__ballot(kept[c]) == 0)
                continue;  // no lane keeps its row of this pass
#pragma unroll
            for (int m = 0; m < CPL / WV; m++) {
                float cc[WV];
                lookup<BV, G>(tabV, vb[c], m, cc);
#pragma unroll
                for (int j = 0; j < WV; j++)
#pragma unroll
                    for (int h = 0; h < G; h++)
                        acc[h][WV * m + j] = fmaf(w[h], cc[j], acc[h][WV * m + j]);
            }
        }
    }
    write_chunk_record<D, G, CPL, AST>(p, acc, M, l_part, accs, red_m, red_l, b, h0, chunk);
}

// Merge the chunks of one (sequence, query head) and rotate back.  One
// workgroup per (sequence, query head): thread t takes coordinates
// 4 (t % (D/4)) .. +3 of the chunks c = t / (D/4), + NG, + 2 NG, ... (NG
// groups of chunks in parallel, every record read whole-line), the groups'
// sums meet in LDS in a fixed order, and the first wave applies the single
// inverse rotation (its first D/32 lanes hold the row).  The records are read
// in one pass: each group keeps a running maximum of the chunk maxima and
// rescales its sums when it grows (the log-sum-exp merge of [Foundry]
// "Optimization: Fused dequant-dot" taken over chunks), and the groups are
// brought to the common maximum where they meet.
// Threads per merge workgroup: 512 at head_dim 256 (eight chunk groups), so
// that a long context's records load in one batch per thread, else 256.
template <int D>
constexpr int combine_threads()
{
    return D >= 256 ? 512 : 256;
}

template <int D>
__global__ __launch_bounds__(combine_threads<D>()) void attn_combine_kernel(AttnParams p)
{
    constexpr int CT = combine_threads<D>();
    constexpr int P = D / kCPL, RS = D + 4, Q = D / 4, NG = CT / Q;
    __shared__ __attribute__((aligned(16))) float part[NG][D];
    __shared__ float lsum[NG], gmax[NG];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j4 = tid % Q, grp = tid / Q;
    const int64_t bh = blockIdx.x;
    const float *rec = p.part + bh * p.n_chunks * RS;
    constexpr float kNegInf = -__builtin_huge_valf();
    // the records of UN chunks are loaded together (one latency per batch:
    // with few (sequence, head) pairs this kernel is latency-bound); every
    // thread of a group reads the same chunks, so the group's maximum is the
    // same in all of them
    constexpr int UN = D >= 256 ? 16 : 8;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float L = 0.0f, m = kNegInf;
    auto raise_to = [&](float mn) {  // mn >= m; from m = -inf the sums are 0
        const float s = mn == m ? 1.0f : exp2f(m - mn);
        o.x *= s;
        o.y *= s;
        o.z *= s;
        o.w *= s;
        L *= s;
        m = mn;
    };
    auto add = [&](float mx, const float4 &t, float lv) {
        const float w = mx == kNegInf ? 0.0f : exp2f(mx - m);
        o.x = fmaf(w, t.x, o.x);
        o.y = fmaf(w, t.y, o.y);
        o.z = fmaf(w, t.z, o.z);
        o.w = fmaf(w, t.w, o.w);
        L = fmaf(w, lv, L);  // lv = 0 except on the thread holding coordinates 0..3
    };
    int c = grp;
    for (; c + (UN - 1) * NG < p.n_chunks; c += UN * NG) {
        float mx[UN], lv[UN];
        float4 t[UN];
#pragma unroll
        for (int u = 0; u < UN; u++) {
            const float *r = rec + (c + u * NG) * RS;
            mx[u] = r[D];
            lv[u] = j4 == 0 ? r[D + 1] : 0.0f;
            t[u] = reinterpret_cast<const float4 *>(r)[j4];
        }
        float mn = m;
#pragma unroll
        for (int u = 0; u < UN; u++)
            mn = fmaxf(mn, mx[u]);
        raise_to(mn);
#pragma unroll
        for (int u = 0; u < UN; u++)
            add(mx[u], t[u], lv[u]);
    }
    for (; c < p.n_chunks; c += NG) {
        const float *r = rec + c * RS;
        const float mx = r[D];
        raise_to(fmaxf(m, mx));
        add(mx, reinterpret_cast<const float4 *>(r)[j4], j4 == 0 ? r[D + 1] : 0.0f);
    }
    reinterpret_cast<float4 *>(part[grp])[j4] = o;
    if (j4 == 0) {
        lsum[grp] = L;
        gmax[grp] = m;
    }
    __syncthreads();
    if (wave == 0) {
        const int sub = lane % P;
        float M = kNegInf;
#pragma unroll
        for (int g2 = 0; g2 < NG; g2++)
            M = fmaxf(M, gmax[g2]);
        float gs[NG];  // each group's factor to the common maximum
#pragma unroll
        for (int g2 = 0; g2 < NG; g2++)
            gs[g2] = gmax[g2] == M ? 1.0f : exp2f(gmax[g2] - M);
        float v[kCPL];
#pragma unroll
        for (int k = 0; k < kCPL; k++) {
            float a = 0.0f;
#pragma unroll
            for (int g2 = 0; g2 < NG; g2++)
                a = fmaf(gs[g2], part[g2][sub * kCPL + k], a);
            v[k] = a;
        }
        float Lt = 0.0f;
#pragma unroll
        for (int g2 = 0; g2 < NG; g2++)
            Lt = fmaf(gs[g2], lsum[g2], Lt);
        apply_signs(v, p.signs2[sub]);
        fwht_row<P>(v, sub);
        const float sc = 1.0f / (Lt * sqrtf((float)D));
#pragma unroll
        for (int k = 0; k < kCPL; k++)
            v[k] *= sc;
        apply_signs(v, p.signs[sub]);
        if (lane < P && sub * kCPL < p.d_in)  // padded coordinates are dropped
            store_slice(p.out + bh * p.d_in + sub * kCPL, v);
    }
}

int check_cache(const tq_cache_desc *c, int layer, const char *fn)
{
    if (!c)
        return tq::fail(TQ_EINVAL, std::string(fn) + ": cache is NULL");
    if (c->n_layers < 1 || c->n_layers > TQ_MAX_LAYERS || c->batch < 0 || c->n_kv_heads < 1 ||
        c->window < 1 || !c->head_dim || !c->k_packed || !c->k_norms || !c->v_packed ||
        !c->v_norms)
        return tq::fail(TQ_EINVAL, std::string(fn) + ": invalid cache descriptor");
    if (layer < 0 || layer >= c->n_layers)
        return tq::fail(TQ_EINVAL, std::string(fn) + ": layer out of range");
    return tq::check_flags(c->flags, fn);
}

struct Split {
    int T, n_chunks, chunk_len;
};

// Which scan a launch runs (the host's mirror of the kernels' choice): the
// exchange scan for two or four query heads per KV head where its LDS blocks
// fit, and for eight as two workgroups of four; the per-lane scan otherwise.
template <int D>
bool exchange_scan(int G)
{
    switch (G) {
    case 2: return Xch<D, 2>::ON;
    case 4: return Xch<D, 4>::ON;
    case 8: return Xch<D, 8>::ON || Xch<D, 4>::ON;
    default: return false;
    }
}

bool exchange_scan_for(int D, int G)
{
    return D == 64 ? exchange_scan<64>(G) : D == 128 ? exchange_scan<128>(G) : exchange_scan<256>(G);
}

// Workgroups per KV head (eight query heads on the exchange scan: two of four)
int groups_per_kv_head(int D, int G)
{
    if (G == 8) {
        const bool split = D == 64    ? Xch<64, 4>::ON && !Xch<64, 8>::ON
                           : D == 128 ? Xch<128, 4>::ON && !Xch<128, 8>::ON
                                      : Xch<256, 4>::ON && !Xch<256, 8>::ON;
        return split ? 2 : 1;
    }
    return 1;
}

// Context split: enough chunks for about `target` workgroups, chunks a whole
// number of tiles.  The target is one round of resident workgroups over the
// 256 CUs: two per CU for the exchange scan (its registers and LDS), four for
// the per-lane scan; measured, 512 and 1024 beat the other choice and 2048 for
// each.  Depends only on the arguments, so results are the same on every
// device.
Split split_for(int batch, int n_kv, int64_t ctx_len, int window, int D, int G)
{
    Split s;
    s.T = (int)(ctx_len < window ? ctx_len : window);
    const int target = exchange_scan_for(D, G) ? 512 : 1024;
    const int units =
        batch * n_kv * groups_per_kv_head(D, G) > 0 ? batch * n_kv * groups_per_kv_head(D, G) : 1;
    const int tiles = (s.T + kTile - 1) / kTile;
    int want = (target + units - 1) / units;
    if (want > tiles)
        want = tiles;
    if (want < 1)
        want = 1;
    const int tiles_per_chunk = (tiles + want - 1) / want;
    s.chunk_len = tiles_per_chunk * kTile;
    s.n_chunks = (s.T + s.chunk_len - 1) / s.chunk_len;
    return s;
}

template <int D, int BK, int BV>
void launch_attn_wave(int G, dim3 grid, AttnParams p, hipStream_t st)
{
    dim3 block(kBlock);
    p.gsplit = 1;
    switch (G) {
    case 1:
        if constexpr (RowScan<D, BK>::ON)
            hipLaunchKernelGGL((attn_partial_row_kernel<D, BK, BV>), grid, block, 0, st, p);
        else
            hipLaunchKernelGGL((attn_partial_wave_kernel<D, BK, BV, 1>), grid, block, 0, st, p);
        break;
    case 2: hipLaunchKernelGGL((attn_partial_wave_kernel<D, BK, BV, 2>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((attn_partial_wave_kernel<D, BK, BV, 4>), grid, block, 0, st, p); break;
    default:
        if constexpr (Xch<D, 4>::ON && !Xch<D, 8>::ON) {
            // eight query heads per KV head: two workgroups of four each (the
            // exchange scan, which needs more LDS than a workgroup of eight
            // could have); each reads the KV head's rows
            p.gsplit = 2;
            grid.y *= 2;
            hipLaunchKernelGGL((attn_partial_wave_kernel<D, BK, BV, 4>), grid, block, 0, st, p);
        } else {
            hipLaunchKernelGGL((attn_partial_wave_kernel<D, BK, BV, 8>), grid, block, 0, st, p);
        }
        break;
    }
}

// the sparse-V gate's two passes for workgroups of GW query heads
template <int D, int BK, int BV, int GW>
void launch_gated(dim3 grid, const AttnParams &p, hipStream_t st)
{
    hipLaunchKernelGGL((attn_scores_kernel<D, BK, GW>), grid, dim3(kBlock), 0, st, p);
    hipLaunchKernelGGL((attn_gated_v_kernel<D, BV, GW>), grid, dim3(kBlock), 0, st, p);
}

// Query heads per workgroup of the sparse-V passes: as on the ungated path
// (eight query heads as two workgroups of four where the exchange scan runs)
template <int D, int BK, int BV>
void launch_attn_g(int G, dim3 grid, AttnParams p, hipStream_t st)
{
    if (!(p.gate_log2 > -__builtin_huge_valf())) {
        launch_attn_wave<D, BK, BV>(G, grid, p, st);
        return;
    }
    switch (G) {
    case 1: p.gsplit = 1; launch_gated<D, BK, BV, 1>(grid, p, st); break;
    case 2: p.gsplit = 1; launch_gated<D, BK, BV, 2>(grid, p, st); break;
    case 4: p.gsplit = 1; launch_gated<D, BK, BV, 4>(grid, p, st); break;
    default:
        if constexpr (Xch<D, 4>::ON && !Xch<D, 8>::ON) {
            p.gsplit = 2;
            grid.y *= 2;
            launch_gated<D, BK, BV, 4>(grid, p, st);
        } else {
            p.gsplit = 1;
            launch_gated<D, BK, BV, 8>(grid, p, st);
        }
        break;
    }
}

template <int D, int BK>
void launch_attn_bv(int BV, int G, dim3 grid, const AttnParams &p, hipStream_t st)
{
    switch (BV) {
    case 2: launch_attn_g<D, BK, 2>(G, grid, p, st); break;
    case 3: launch_attn_g<D, BK, 3>(G, grid, p, st); break;
    default: launch_attn_g<D, BK, 4>(G, grid, p, st); break;
    }
}

template <int D>
void launch_attn_d(int BK, int BV, int G, dim3 grid, const AttnParams &p, hipStream_t st)
{
    switch (BK) {
    case 2: launch_attn_bv<D, 2>(BV, G, grid, p, st); break;
    case 3: launch_attn_bv<D, 3>(BV, G, grid, p, st); break;
    default: launch_attn_bv<D, 4>(BV, G, grid, p, st); break;
    }
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)(grid.z * p.Hq)),
                       dim3(combine_threads<D>()), 0, st, p);
}

// Workspace layout: the chunk records [B][Hq][n_chunks][D + 4] floats; with
// the sparse-V gate also the chunk maxima [B][Hq][n_chunks] (padded to 16
// bytes) and every row's scores [B][Hq][T] floats.
struct WsLayout {
    size_t part, cmax, scores, total;  // byte offsets and the size
};

WsLayout ws_layout(int batch, int n_q_heads, const Split &s, int D, bool gated)
{
    WsLayout w;
    const size_t bh = (size_t)batch * (size_t)n_q_heads;
    w.part = 0;
    w.cmax = bh * s.n_chunks * (size_t)(D + 4) * sizeof(float);
    w.scores = w.cmax + (gated ? (bh * s.n_chunks * sizeof(float) + 15) / 16 * 16 : 0);
    w.total = w.scores + (gated ? bh * (size_t)s.T * sizeof(float) : 0);
    return w;
}

}  // namespace

extern "C" size_t tq_attn_workspace_bytes(const tq_cache_desc *c, int layer, int n_q_heads,
                                          int64_t ctx_len, float sparse_v_threshold)
{
    if (!c || layer < 0 || layer >= c->n_layers || !c->head_dim || n_q_heads < 1 ||
        ctx_len < 1 || c->window < 1 || c->batch < 0 || c->n_kv_heads < 1 ||
        !(sparse_v_threshold >= 0.0f && sparse_v_threshold < 1.0f))
        return 0;
    const int D = tq::padded_dim(c->head_dim[layer]);
    if (D == 0)
        return 0;
    Split s = split_for(c->batch, c->n_kv_heads, ctx_len, c->window, D, n_q_heads / c->n_kv_heads);
    return ws_layout(c->batch, n_q_heads, s, D, sparse_v_threshold > 0.0f).total;
}

// ---- Scratch of the allocation-free entry point: one file-scope device
// array per GPU (each device that loads the library holds its own copy until
// the process ends).  Host code never names `scratch` in a kernel argument or
// a copy: in host code the name is a host-side stand-in, not a device
// address.  Its device address is taken once per device with that device
// current and kept in scratch_ptr.
constexpr size_t kScratchBytes = TQ_ATTN_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void *scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up on its first use)
static int scratch_for_current_device(void **ptr, const char *fn)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return tq::fail(TQ_EHIP, std::string(fn) + ": hipGetDevice: " + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": device index above " +
                                             std::to_string(kMaxDevices - 1));
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return tq::fail(TQ_EHIP, std::string(fn) + ": hipGetSymbolAddress(scratch): " +
                                         hipGetErrorString(e));
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return TQ_OK;
}

// tq_attn_decode, and (noalloc) the same with the static scratch in place of
// the caller's workspace
static int attn_decode_impl(const tq_cache_desc *c, int layer, const uint16_t *q_bf16,
                            int n_q_heads, int64_t ctx_len, float scale, float sparse_v_threshold,
                            float *out, void *workspace, size_t ws_bytes, void *stream,
                            bool noalloc, const char *fn)
{
    tq::clear_error();
    int rc = check_cache(c, layer, fn);
    if (rc != TQ_OK)
        return rc;
    if (!(sparse_v_threshold >= 0.0f && sparse_v_threshold < 1.0f))
        return tq::fail(TQ_EINVAL, std::string(fn) + ": sparse_v_threshold must be in [0, 1)");
    if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0)
        return tq::fail(TQ_EINVAL, std::string(fn) + ": n_q_heads must be a positive multiple of n_kv_heads");
    const int G = n_q_heads / c->n_kv_heads;
    if (ctx_len < 1)
        return tq::fail(TQ_EINVAL, std::string(fn) + ": ctx_len must be >= 1");
    const int d = c->head_dim[layer], D = tq::padded_dim(d);
    if (D == 0)
        return tq::fail(TQ_EINVAL, std::string(fn) + ": head_dim outside 2..2^20");
    if (!((D == 64 || D == 128 || D == 256) && (d == D || d % 32 == 0)))
        return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": device kernels take head_dim in "
                                         + "{64, 128, 256} or a multiple of 32 between them");
    const int bits_k = tq::layer_bits(c, layer, 0), bits_v = tq::layer_bits(c, layer, 1);
    for (int bits : {bits_k, bits_v}) {
        if (bits < 1 || bits > 4)
            return tq::fail(TQ_EINVAL, std::string(fn) + ": bits must be in 1..4");
        if (bits == 1)
            return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": device kernels take bits in {2, 3, 4}");
    }
    if (!(G == 1 || G == 2 || G == 4 || G == 8))
        return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": query/KV head ratio must be 1, 2, 4 or 8");
    // the kernels address one KV head's packed rows with 32-bit byte offsets
    if ((uint64_t)c->window * (uint64_t)(D / 2) >= (1ull << 31))
        return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": window too large (one KV head's packed "
                                         + "rows must span less than 2 GiB)");
    if (c->batch == 0)
        return TQ_OK;
    if (!q_bf16 || !out || (!noalloc && !workspace) || !c->k_packed[layer] ||
        !c->k_norms[layer] || !c->v_packed[layer] || !c->v_norms[layer])
        return tq::fail(TQ_EINVAL, std::string(fn) + ": NULL buffer");
    if (((uintptr_t)q_bf16 | (uintptr_t)out | (uintptr_t)workspace |
         (uintptr_t)c->k_packed[layer] | (uintptr_t)c->v_packed[layer]) % 16 != 0 ||
        ((uintptr_t)c->k_norms[layer] | (uintptr_t)c->v_norms[layer]) % 4 != 0)
        return tq::fail(TQ_EINVAL, std::string(fn) + ": misaligned buffer");
    const size_t need = tq_attn_workspace_bytes(c, layer, n_q_heads, ctx_len, sparse_v_threshold);
    if (noalloc) {
        if (need > kScratchBytes)
            return tq::fail(TQ_EINVAL, std::string(fn) + ": this call needs " + std::to_string(need) +
                                           " bytes of scratch; the library's static scratch holds " +
                                           std::to_string(kScratchBytes) +
                                           " (use tq_attn_decode with a workspace)");
        if ((rc = scratch_for_current_device(&workspace, fn)) != TQ_OK)
            return rc;
        ws_bytes = kScratchBytes;
    } else if (ws_bytes < need) {
        return tq::fail(TQ_EINVAL, std::string(fn) + ": workspace too small (need " +
                                       std::to_string(need) + " bytes)");
    }
    if (tq::take_injected_launch_failure())
        return tq::fail(TQ_EHIP, std::string(fn) + ": injected launch failure (TQ_TEST_FAIL_LAUNCH)");
    tq_codebook ck, cv;
    if ((rc = tq::get_codebook(D, bits_k, tq::density_of(c->flags), &ck)) != TQ_OK ||
        (rc = tq::get_codebook(D, bits_v, tq::density_of(c->flags), &cv)) != TQ_OK)
        return rc;
    Split s = split_for(c->batch, c->n_kv_heads, ctx_len, c->window, D, G);
    AttnParams p;
    p.q = q_bf16;
    p.kp = c->k_packed[layer];
    p.kn = c->k_norms[layer];
    p.vp = c->v_packed[layer];
    p.vn = c->v_norms[layer];
    const WsLayout wl = ws_layout(c->batch, n_q_heads, s, D, sparse_v_threshold > 0.0f);
    p.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + wl.part);
    p.cmax = reinterpret_cast<float *>(static_cast<char *>(workspace) + wl.cmax);
    p.scores = reinterpret_cast<float *>(static_cast<char *>(workspace) + wl.scores);
    p.out = out;
    p.Hq = n_q_heads;
    p.Hkv = c->n_kv_heads;
    p.window = c->window;
    p.T = s.T;
    p.n_chunks = s.n_chunks;
    p.chunk_len = s.chunk_len;
    p.gsplit = 1;
    p.d_in = d;
    // the default scale is 1/sqrt(head_dim); the rotation's 1/sqrt is of the
    // padded length
    const float sc = scale > 0.0f ? scale : 1.0f / sqrtf((float)d);
    p.qscale = sc * kLog2e / sqrtf((float)D);
    p.gate_log2 = sparse_v_threshold > 0.0f ? log2f(sparse_v_threshold) : -__builtin_huge_valf();
    for (int j = 0; j < 16; j++) {
        p.centK[j] = j < ck.levels ? ck.centroids[j] : 0.0f;
        p.centV[j] = j < cv.levels ? cv.centroids[j] : 0.0f;
    }
    tq::sign_words(D, c->seed, p.signs);
    tq::sign_words2(D, c->seed, c->flags, p.signs2);
    dim3 grid((unsigned)s.n_chunks, (unsigned)c->n_kv_heads, (unsigned)c->batch);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (D) {
    case 64: launch_attn_d<64>(bits_k, bits_v, G, grid, p, st); break;
    case 128: launch_attn_d<128>(bits_k, bits_v, G, grid, p, st); break;
    default: launch_attn_d<256>(bits_k, bits_v, G, grid, p, st); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return tq::fail(TQ_EHIP, std::string(std::string(fn) + ": ") + hipGetErrorString(e));
    return TQ_OK;
}

extern "C" int tq_attn_decode(const tq_cache_desc *c, int layer, const uint16_t *q_bf16,
                              int n_q_heads, int64_t ctx_len, float scale,
                              float sparse_v_threshold, float *out, void *workspace,
                              size_t ws_bytes, void *stream)
{
    return attn_decode_impl(c, layer, q_bf16, n_q_heads, ctx_len, scale, sparse_v_threshold, out,
                            workspace, ws_bytes, stream, false, "tq_attn_decode");
}

extern "C" int tq_attn_decode_noalloc(const tq_cache_desc *c, int layer, const uint16_t *q_bf16,
                                      int n_q_heads, int64_t ctx_len, float scale,
                                      float sparse_v_threshold, float *out, void *stream)
{
    return attn_decode_impl(c, layer, q_bf16, n_q_heads, ctx_len, scale, sparse_v_threshold, out,
                            nullptr, 0, stream, true, "tq_attn_decode_noalloc");
}
