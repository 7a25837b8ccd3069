// Codec kernels of libtq.so: rotate, encode (K and V in one launch), decode
// and the append-only ring-cache encode.
//
// Pages (cited by title and section):
//   "TurboQuant KV Cache Compression — Spec" -- As-Built Notes 1 (signs
//     before the Hadamard) and 2 (L2-norm normalisation); Algorithm Detail
//     steps 1-3; Hadamard Transform Detail; Integration Points (pos % max_seq).
//   "TurboQuantEngine — Specification" -- 2.2 Memory contract (fp32 norm and
//     packed indices per head row); 6 P1 follow-ups, W3 (encode only the new
//     row each step).
//
// Work decomposition: each row is owned by P = d/32 lanes (32 coordinates per
// lane, see tq_device.h); workgroups of 256 threads walk the rows with a grid
// stride.  Nothing is shared between rows, so there are no atomics and the
// result does not depend on the launch shape.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <mutex>
#include <string>

#include "tq_device.h"
#include "tq_internal.h"

using namespace tqd;

namespace {

// ----------------------------------------------------------------- encode

struct CodeTable {
    float bnd[15];
    int bits;
};

// One row: norm, sign, rotate, normalise, bucketize, pack.  `valid` false
// lanes compute on zeros and store nothing.  `key` addresses the bucketize
// table built for BITS.
template <int D, int BITS, typename T>
__device__ __forceinline__ void encode_row(const RawSlice<T> &raw, bool valid, int sub,
                                           const SignMasks<T> &sm, uint32_t key,
                                           uint8_t *dst_row, float *dst_norm)
{
    constexpr int P = Shape<D>::P;
    float v[kCPL];
    float ss;
    convert_signed(raw, sm.xm, v, ss);  // invalid lanes carry a zeroed slice
    ss = sum_across<P>(ss);
    // Rows whose sum of squares leaves [2^-100, 2^100] (tiny, huge, zero or
    // non-finite) are rescaled by an exact power of two first (ldexpf per
    // element: 2^-e is not representable for e < -126); indices do not change
    // under such scaling and the norm is scaled back.  Non-finite rows are
    // encoded as the zero row (their stored norm is not finite).
    int nexp = 0;
    float nbad = 0.0f;
    if (!(ss >= 0x1p-100f && ss <= 0x1p100f)) {
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < kCPL; k++)
            m = fmaxf(m, fabsf(v[k]));
        m = max_across<P>(m);
        if (m > 0.0f && m <= FLT_MAX) {
            (void)frexpf(m, &nexp);
#pragma unroll
            for (int k = 0; k < kCPL; k++)
                v[k] = ldexpf(v[k], -nexp);
            ss = 0.0f;
#pragma unroll
            for (int k = 0; k < kCPL; k++)
                ss = fmaf(v[k], v[k], ss);
            ss = sum_across<P>(ss);
        } else if (!(m <= FLT_MAX)) {
            nbad = ss + m;  // inf or NaN
#pragma unroll
            for (int k = 0; k < kCPL; k++)
                v[k] = 0.0f;
            ss = 0.0f;
        }
    }
    const float n = sqrtf(ss);
    // u = H(D x) / (sqrt(d) n); zero rows get u = 0
    const float inv = ss > 0.0f ? 1.0f / sqrtf((float)D * ss) : 0.0f;
    fwht_row<P>(v, sub);
    uint32_t w[BITS];
#pragma unroll
    for (int j = 0; j < BITS; j++)
        w[j] = 0u;
#pragma unroll
    for (int k = 0; k < kCPL; k++)
        put_index<BITS>(w, k, bucketize(v[k] * inv, key));
    if (valid) {
        store_words<BITS>(dst_row + sub * 4 * BITS, w);
        if (sub == 0)
            *dst_norm = nbad != 0.0f ? nbad : ldexpf(n, nexp);
    }
}

struct EncodeSide {
    const void *src;
    uint8_t *packed;
    float *norms;
    CodeTable code;
};

struct EncodeParams {
    EncodeSide side[2];
    int64_t n_rows;
    uint32_t signs[8];
};

template <int D, typename T, int BITS>
__device__ __forceinline__ void encode_contig_loop(const EncodeSide &s, int64_t n_rows,
                                                   const SignMasks<T> &sm, uint32_t key)
{
    constexpr int P = Shape<D>::P, RPW = Shape<D>::RPW, RPB = Shape<D>::RPB;
    constexpr int RB = D * BITS / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % P, rig = lane / P;
    const T *src = static_cast<const T *>(s.src);
    const int64_t stride = (int64_t)gridDim.x * RPB;
    int64_t row = (int64_t)blockIdx.x * RPB + wave * RPW + rig;
    RawSlice<T> cur;
    if (row < n_rows)
        load_raw(src + row * D + sub * kCPL, cur);
    else
        zero_raw(cur);
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < n_rows; base += stride) {
        // issue the next pass's loads before transforming this one
        const int64_t nrow = row + stride;
        RawSlice<T> nxt;
        if (nrow < n_rows)
            load_raw(src + nrow * D + sub * kCPL, nxt);
        else
            zero_raw(nxt);
        const bool valid = row < n_rows;
        const int64_t r = valid ? row : 0;
        encode_row<D, BITS, T>(cur, valid, sub, sm, key, s.packed + r * RB, s.norms + r);
        cur = nxt;
        row = nrow;
    }
}

// blockIdx.y selects the side (0 = first non-NULL side, 1 = second)
template <int D, typename T>
__global__ __launch_bounds__(kBlock) void encode_kernel(EncodeParams p)
{
    __shared__ float2 lut[kLutBins];
    const EncodeSide &s = p.side[blockIdx.y];
    build_lut(lut, s.code.bnd, (1 << s.code.bits) - 1);
    __syncthreads();
    const int sub = (threadIdx.x & 63) % Shape<D>::P;
    const SignMasks<T> sm(p.signs[sub]);
    const uint32_t key = lut_key(lut);
    switch (s.code.bits) {
    case 2: encode_contig_loop<D, T, 2>(s, p.n_rows, sm, key); break;
    case 3: encode_contig_loop<D, T, 3>(s, p.n_rows, sm, key); break;
    default: encode_contig_loop<D, T, 4>(s, p.n_rows, sm, key); break;
    }
}

// ------------------------------------------- encode, 64 coordinates per lane
// For bf16 rows of d in {64, 128} each lane produces 64 output coordinates
// of one row: with d = 64 a lane owns a row; with d = 128 lanes l and l + 32
// share row l, lane l + 32 producing the second half of the outputs.  Every
// lane thus works on the same coordinate indices and the sign diagonal is
// wave-uniform; it is folded into the butterflies: writing the signed input
// as s_i x_i and carrying one sign per block, merging blocks [j, j+h) and
// [j+h, j+2h) (signs s_j and s_{j+h}) gives
//   a' = s_j (a + r b),  b' = s_j (a - r b),   r = s_j s_{j+h},
// so a butterfly is two fmas with a uniform r (a scalar register) and every
// output carries the single sign s_0, which joins 1/||x||.  For d = 128 the
// stage across the two halves goes first (the stages commute): lane l forms
// x_k + r_k x_{k+64}, lane l + 32 forms x_k - r_k x_{k+64} (its minus sign
// applied as an xor on the bf16 words), after which both lanes carry the
// signs s_0..s_63 and run the same six remaining stages.
// Global memory is read and written through a per-wave LDS stage so that
// every load and store instruction covers whole 128-byte lines.

constexpr int kPiece = 128;            // bytes of 64 bf16 coordinates
constexpr int kPieceStride = kPiece + 16;
constexpr int kRowStage = 64 * kPieceStride;  // per wave

struct EncodeRowsParams {
    EncodeSide side[2];
    int64_t n_rows;
    uint32_t rbits[4];  // butterfly signs r in the order used (d - 1 bits; 1 = -1)
    float s0;           // sign carried by every output
};

// r as a float from the packed bits (uniform: scalar instructions)
__device__ __forceinline__ float butterfly_sign(const uint32_t (&rb)[4], int i)
{
    return __uint_as_float(0x3F800000u | (((rb[i >> 5] >> (i & 31)) & 1u) << 31));
}

template <int D, int BITS>
__device__ __forceinline__ void encode_rows_loop(const EncodeSide s, const int64_t n_rows,
                                                 const uint32_t (&rb)[4], const float s0,
                                                 uint32_t key, uint8_t *stg)
{
    constexpr int NH = D / 64;                 // lanes per row
    constexpr int RPW = 64 / NH;               // rows per wave
    constexpr int CB = D * 2;                  // input bytes per row (bf16)
    constexpr int RB = D * BITS / 8;           // packed bytes per row
    constexpr int HB = 64 * BITS / 8;          // packed bytes per lane
    constexpr int NWL = 2 * BITS;              // packed words per lane
    constexpr int G = HB % 16 == 0 ? 16 : 8;   // store granule (divides HB)
    constexpr int CROSS = NH - 1;              // signs used by the stage across halves
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane % RPW, half = lane / RPW;
    const int64_t stride = (int64_t)gridDim.x * (kBlock / 64) * RPW;
    const uint8_t *src = static_cast<const uint8_t *>(s.src);
    const uint32_t flip = half ? 0x80008000u : 0u;

    for (int64_t row0 = ((int64_t)blockIdx.x * (kBlock / 64) + wave) * RPW; row0 < n_rows;
         row0 += stride) {
        const int nvalid = (int)min<int64_t>(RPW, n_rows - row0);
        // ---- stage the group (8 KiB): 128-byte piece pc of row r at slot pc*RPW + r
        {
            u32x4 t[8];
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const int c = 8 * q + (lane >> 3);  // 128-byte chunk of the group
                if (c / NH < nvalid)
                    t[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                        src + row0 * CB + c * kPiece + (lane & 7) * 16));
                else
                    t[q] = 0;
            }
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const int c = 8 * q + (lane >> 3);
                *reinterpret_cast<u32x4 *>(stg + ((c % NH) * RPW + c / NH) * kPieceStride +
                                           (lane & 7) * 16) = t[q];
            }
        }
        wave_lds_fence();
        const uint8_t *sa = stg + row * kPieceStride;              // coordinates 0..63
        const uint8_t *sb = stg + (RPW + row) * kPieceStride;      // 64..127 (d = 128)
        // ---- read, convert; sum of squares of this lane's input half
        float v[64];
        float ss = 0.0f, mx = 0.0f;
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const u32x4 wa = *reinterpret_cast<const u32x4 *>(sa + m * 16);
            const uint32_t aa[4] = {wa.x, wa.y, wa.z, wa.w};
            if constexpr (NH == 1) {
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    const bf16x2_t hv = __builtin_bit_cast(bf16x2_t, aa[c]);
                    ss = __builtin_amdgcn_fdot2_f32_bf16(hv, hv, ss, false);
                    v[8 * m + 2 * c] = __uint_as_float(aa[c] << 16);
                    v[8 * m + 2 * c + 1] = __uint_as_float(aa[c] & 0xFFFF0000u);
                }
            } else {
                const u32x4 wb = *reinterpret_cast<const u32x4 *>(sb + m * 16);
                const uint32_t bw[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    const uint32_t own = half ? bw[c] : aa[c];
                    const bf16x2_t hv = __builtin_bit_cast(bf16x2_t, own);
                    ss = __builtin_amdgcn_fdot2_f32_bf16(hv, hv, ss, false);
                    const uint32_t bb = bw[c] ^ flip;
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) {
                        const int k = 8 * m + 2 * c + hh;
                        const float xa = __uint_as_float(hh ? (aa[c] & 0xFFFF0000u) : (aa[c] << 16));
                        const float xb = __uint_as_float(hh ? (bb & 0xFFFF0000u) : (bb << 16));
                        v[k] = fmaf(butterfly_sign(rb, k), xb, xa);
                    }
                }
            }
        }
        if constexpr (NH == 2)
            ss += __shfl_xor(ss, 32);
        // Rows whose sum of squares leaves [2^-100, 2^100] (tiny, huge, zero or
        // non-finite) get an exact power-of-two rescale of the transformed
        // values; rows holding Inf or NaN encode as the zero row and store a
        // non-finite norm.
        int nexp = 0;
        bool bad = false;
        if (!(ss >= 0x1p-100f && ss <= 0x1p100f)) {
            // largest magnitude of the row (both halves)
#pragma unroll
            for (int m = 0; m < 8; m++)
#pragma unroll
                for (int pc = 0; pc < NH; pc++) {
                    const u32x4 w4 = *reinterpret_cast<const u32x4 *>((pc ? sb : sa) + m * 16);
                    const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                    for (int c = 0; c < 4; c++)
                        mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(ww[c] << 16)),
                                             fabsf(__uint_as_float(ww[c] & 0xFFFF0000u))));
                }
            if (!(mx <= FLT_MAX)) {
                bad = true;
            } else if (mx > 0.0f) {
                (void)frexpf(mx, &nexp);
                ss = 0.0f;
#pragma unroll
                for (int m = 0; m < 8; m++)
#pragma unroll
                    for (int pc = 0; pc < NH; pc++) {
                        const u32x4 w4 = *reinterpret_cast<const u32x4 *>((pc ? sb : sa) + m * 16);
                        const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                        for (int c = 0; c < 4; c++) {
                            const float x0 = ldexpf(__uint_as_float(ww[c] << 16), -nexp);
                            const float x1 = ldexpf(__uint_as_float(ww[c] & 0xFFFF0000u), -nexp);
                            ss = fmaf(x0, x0, ss);
                            ss = fmaf(x1, x1, ss);
                        }
                    }
#pragma unroll
                for (int k = 0; k < 64; k++)
                    v[k] = ldexpf(v[k], -nexp);
            }
        }
        const float n = sqrtf(ss);
        const float inv = ss > 0.0f ? s0 / sqrtf((float)D * ss) : 0.0f;
        // ---- remaining stages; the last one is fused with bucketize/pack
        uint32_t w[NWL];
#pragma unroll
        for (int q = 0; q < NWL; q++)
            w[q] = 0u;
        int off = 64 * CROSS;
#pragma unroll
        for (int h = 1; h < 32; h *= 2) {
#pragma unroll
            for (int j = 0; j < 64; j += 2 * h) {
                const float rr = butterfly_sign(rb, off + j / (2 * h));
#pragma unroll
                for (int i = j; i < j + h; i++) {
                    const float a = v[i], b = v[i + h];
                    v[i] = fmaf(rr, b, a);
                    v[i + h] = fmaf(-rr, b, a);
                }
            }
            off += 64 / (2 * h);
        }
        const float rl = butterfly_sign(rb, off);
        const float sc = bad ? 0.0f : inv;   // bad rows: u = 0 (the zero-row code)
#pragma unroll
        for (int i = 0; i < 32; i++) {
            const float a = v[i], b = v[i + 32];
            const uint32_t i0 = bucketize(fmaf(rl, b, a) * sc, key);
            const uint32_t i1 = bucketize(fmaf(-rl, b, a) * sc, key);
#pragma unroll
            for (int t2 = 0; t2 < 2; t2++) {
                const int k = t2 ? i + 32 : i;
                const uint32_t idx = t2 ? i1 : i0;
                const int bit = k * BITS, wd = bit >> 5, sh = bit & 31;
                w[wd] |= idx << sh;
                if (sh + BITS > 32)
                    w[wd + 1] |= idx >> (32 - sh);
            }
        }
        if (half == 0 && row < nvalid)
            s.norms[row0 + row] = bad ? ss : ldexpf(n, nexp);
        wave_lds_fence();
        // ---- packed rows through LDS, then whole-line stores
        constexpr int PS = HB + 16;  // padded stride of a lane's packed bytes
        const int chunk = row * NH + half;  // lane's packed bytes sit at chunk * HB
#pragma unroll
        for (int q = 0; q < NWL; q++)
            *reinterpret_cast<uint32_t *>(stg + chunk * PS + 4 * q) = w[q];
        wave_lds_fence();
        uint8_t *dst = s.packed + row0 * RB;
#pragma unroll
        for (int q = 0; q < (64 * HB + 64 * G - 1) / (64 * G); q++) {
            const int e = 64 * q + lane;          // granule index in the region
            if (e * G < nvalid * RB) {
                const int owner = (e * G) / HB, o = (e * G) % HB;
                if constexpr (G == 16) {
                    const u32x4 t = *reinterpret_cast<const u32x4 *>(stg + owner * PS + o);
                    __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(dst) + e);
                } else {
                    const uint2 t = *reinterpret_cast<const uint2 *>(stg + owner * PS + o);
                    reinterpret_cast<uint2 *>(dst)[e] = t;
                }
            }
        }
        wave_lds_fence();
    }
}

template <int D>
__device__ __forceinline__ void encode_rows_side(const EncodeSide s, const int64_t n_rows,
                                                 const uint32_t (&rb)[4], const float s0,
                                                 float2 *lut, uint8_t *stg)
{
    build_lut(lut, s.code.bnd, (1 << s.code.bits) - 1);
    __syncthreads();
    const uint32_t key = lut_key(lut);
    switch (s.code.bits) {
    case 2: encode_rows_loop<D, 2>(s, n_rows, rb, s0, key, stg); break;
    case 3: encode_rows_loop<D, 3>(s, n_rows, rb, s0, key, stg); break;
    default: encode_rows_loop<D, 4>(s, n_rows, rb, s0, key, stg); break;
    }
}

template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2)))
void encode_rows_kernel(EncodeRowsParams p)
{
    __shared__ float2 lut[kLutBins];
    __shared__ __attribute__((aligned(16))) uint8_t stage[kBlock / 64][kRowStage];
    // the side is chosen by a uniform branch: indexing the kernel argument
    // struct with blockIdx.y would copy it to scratch memory
    const uint32_t rb[4] = {p.rbits[0], p.rbits[1], p.rbits[2], p.rbits[3]};
    if (blockIdx.y == 0)
        encode_rows_side<D>(p.side[0], p.n_rows, rb, p.s0, lut, stage[threadIdx.x >> 6]);
    else
        encode_rows_side<D>(p.side[1], p.n_rows, rb, p.s0, lut, stage[threadIdx.x >> 6]);
}

// ----------------------------------------------------------------- append

constexpr int kMaxAppendLayers = 48;

struct AppendSide {
    const void *src[kMaxAppendLayers];
    uint8_t *packed[kMaxAppendLayers];
    float *norms[kMaxAppendLayers];
    CodeTable code;
};

struct AppendParams {
    AppendSide side[2];
    int n_layers;     // layers in this launch (all of head_dim D)
    int bh;           // batch * n_kv_heads
    int window;
    int slot;         // pos % window
    uint32_t signs[8];
};

template <int D, typename T, int BITS>
__device__ __forceinline__ void append_loop(const AppendSide &s, const AppendParams &p,
                                            const SignMasks<T> &sm, uint32_t key)
{
    constexpr int P = Shape<D>::P, RPW = Shape<D>::RPW, RPB = Shape<D>::RPB;
    constexpr int RB = D * BITS / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % P, rig = lane / P;
    const int64_t n_rows = (int64_t)p.n_layers * p.bh;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < n_rows;
         base += (int64_t)gridDim.x * RPB) {
        const int64_t row = base + wave * RPW + rig;
        const bool valid = row < n_rows;
        const int64_t r = valid ? row : 0;
        const int li = (int)(r / p.bh), j = (int)(r % p.bh);
        const T *src = static_cast<const T *>(s.src[li]) + (int64_t)j * D + sub * kCPL;
        const int64_t dst = (int64_t)j * p.window + p.slot;
        RawSlice<T> raw;
        if (valid)
            load_raw(src, raw);
        else
            zero_raw(raw);
        encode_row<D, BITS, T>(raw, valid, sub, sm, key, s.packed[li] + dst * RB,
                               s.norms[li] + dst);
    }
}

template <int D, typename T>
__global__ __launch_bounds__(kBlock) void append_kernel(AppendParams p)
{
    __shared__ float2 lut[kLutBins];
    const AppendSide &s = p.side[blockIdx.y];
    build_lut(lut, s.code.bnd, (1 << s.code.bits) - 1);
    __syncthreads();
    const int sub = (threadIdx.x & 63) % Shape<D>::P;
    const SignMasks<T> sm(p.signs[sub]);
    const uint32_t key = lut_key(lut);
    switch (s.code.bits) {
    case 2: append_loop<D, T, 2>(s, p, sm, key); break;
    case 3: append_loop<D, T, 3>(s, p, sm, key); break;
    default: append_loop<D, T, 4>(s, p, sm, key); break;
    }
}

// ----------------------------------------------------------------- decode

struct DecodeParams {
    const uint8_t *packed;
    const float *norms;
    float *out;
    int64_t n_rows;
    float cent[16];
    uint32_t signs[8];
};

template <int D, int BITS>
__global__ __launch_bounds__(kBlock) void decode_kernel(DecodeParams p)
{
    constexpr int P = Shape<D>::P, RPW = Shape<D>::RPW, RPB = Shape<D>::RPB;
    constexpr int RB = D * BITS / 8;
    __shared__ float cent[16];
    __shared__ __attribute__((aligned(16))) float stage[kBlock / 64][kStageFloats];
    if (threadIdx.x < 16)
        cent[threadIdx.x] = p.cent[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % P, rig = lane / P;
    const uint32_t smask = p.signs[sub];
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const int64_t stride = (int64_t)gridDim.x * RPB;
    int64_t row = (int64_t)blockIdx.x * RPB + wave * RPW + rig;
    uint32_t w[BITS];
    float n;
    {
        const int64_t r = row < p.n_rows ? row : 0;
        load_words<BITS>(p.packed + r * RB + sub * 4 * BITS, w);
        n = p.norms[r];
    }
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < p.n_rows; base += stride) {
        const int64_t row0 = base + wave * RPW;
        // next pass's packed words and norm, issued before this pass's work
        const int64_t nrow = row + stride;
        uint32_t wn[BITS];
        float nn;
        {
            const int64_t r = nrow < p.n_rows ? nrow : 0;
            load_words<BITS>(p.packed + r * RB + sub * 4 * BITS, wn);
            nn = p.norms[r];
        }
        float v[kCPL];
#pragma unroll
        for (int k = 0; k < kCPL; k++)
            v[k] = cent[get_index<BITS>(w, k)];
        fwht_row<P>(v, sub);
        const float sc = n * inv_sqrt_d;
#pragma unroll
        for (int k = 0; k < kCPL; k++)
            v[k] *= sc;
        apply_signs(v, smask);
        const int64_t left = (p.n_rows - row0) * D;
        if (left > 0)
            store_region_coalesced(p.out + row0 * D, v, stage[wave], lane, left);
#pragma unroll
        for (int j = 0; j < BITS; j++)
            w[j] = wn[j];
        n = nn;
        row = nrow;
    }
}

// ----------------------------------------------------------------- rotate

struct RotateParams {
    const void *in;
    float *out;
    int64_t n_rows;
    int inverse;
    uint32_t signs[8];
};

template <int D, typename T>
__global__ __launch_bounds__(kBlock) void rotate_kernel(RotateParams p)
{
    constexpr int P = Shape<D>::P, RPW = Shape<D>::RPW, RPB = Shape<D>::RPB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % P, rig = lane / P;
    const uint32_t smask = p.signs[sub];
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const T *in = static_cast<const T *>(p.in);
    __shared__ __attribute__((aligned(16))) float stage[kBlock / 64][kStageFloats];
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < p.n_rows;
         base += (int64_t)gridDim.x * RPB) {
        const int64_t row0 = base + wave * RPW;
        const int64_t row = row0 + rig;
        const bool valid = row < p.n_rows;
        const int64_t r = valid ? row : 0;
        float v[kCPL];
        load_slice(in + r * D + sub * kCPL, v);
        if (!p.inverse)
            apply_signs(v, smask);
        fwht_row<P>(v, sub);
#pragma unroll
        for (int k = 0; k < kCPL; k++)
            v[k] *= inv_sqrt_d;
        if (p.inverse)
            apply_signs(v, smask);
        const int64_t left = (p.n_rows - row0) * D;
        if (left > 0)
            store_region_coalesced(p.out + row0 * D, v, stage[wave], lane, left);
    }
}

// ------------------------------------------------------------ host helpers

int device_cus()
{
    static std::mutex mu;
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

unsigned grid_for(int64_t n_rows, int rows_per_block)
{
    const int64_t need = (n_rows + rows_per_block - 1) / rows_per_block;
    const int64_t cap = (int64_t)device_cus() * 16;
    return (unsigned)(need < cap ? (need > 0 ? need : 1) : cap);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// d supported by the device kernels, else the status to return
int check_d(int d, const char *fn)
{
    if (d == 64 || d == 128 || d == 256)
        return TQ_OK;
    if (tq::is_pow2(d) && d >= 2 && d <= (1 << 20))
        return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": device kernels take d in {64, 128, 256}");
    return tq::fail(TQ_EINVAL, std::string(fn) + ": d must be a power of two");
}

int check_bits(int bits, const char *fn)
{
    if (bits >= 2 && bits <= 4)
        return TQ_OK;
    if (bits == 1)
        return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": device kernels take bits in {2, 3, 4}");
    return tq::fail(TQ_EINVAL, std::string(fn) + ": bits must be in 1..4");
}

// boundaries for the device table; checks that no widened bin holds two
int code_table(int d, int bits, CodeTable *t, const char *fn)
{
    tq_codebook cb;
    int rc = tq::get_codebook(d, bits, TQ_BETA_HALF_D, &cb);
    if (rc != TQ_OK)
        return rc;
    t->bits = bits;
    for (int j = 0; j < 15; j++)
        t->bnd[j] = j < cb.levels - 1 ? cb.boundaries[j] : 0.0f;
    for (int j = 0; j + 1 < cb.levels - 1; j++)
        if (cb.boundaries[j + 1] - cb.boundaries[j] <= 1.0f / kLutScale + 2.0f * kLutSlack)
            return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": codebook boundaries too close for the bucketize table");
    return TQ_OK;
}

int launch_status(const char *fn)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return tq::fail(TQ_EHIP, std::string(fn) + ": " + hipGetErrorString(e));
    return TQ_OK;
}

int injected(const char *fn)
{
    if (tq::take_injected_launch_failure())
        return tq::fail(TQ_EHIP, std::string(fn) + ": injected launch failure (TQ_TEST_FAIL_LAUNCH)");
    return TQ_OK;
}

// butterfly signs for the row-per-lane encode, in the order the kernel uses:
// for d = 128 first the 64 signs s_k s_{k+64} of the stage across halves, then
// (for both d) the stages h = 1, 2, .., 32 over the first 64 signs
void fill_row_signs(int d, uint64_t seed, EncodeRowsParams &q)
{
    int8_t s[128];
    tq_signs(d, seed, s);
    for (int w = 0; w < 4; w++)
        q.rbits[w] = 0u;
    int off = 0;
    auto put = [&](int i, int sign) {
        if (sign < 0)
            q.rbits[i >> 5] |= 1u << (i & 31);
    };
    if (d == 128) {
        for (int k = 0; k < 64; k++)
            put(off + k, s[k] * s[k + 64]);
        off += 64;
    }
    for (int h = 1; h < 64; h *= 2) {
        for (int m = 0; m < 64 / (2 * h); m++)
            put(off + m, s[2 * h * m] * s[2 * h * m + h]);
        off += 64 / (2 * h);
    }
    q.s0 = (float)s[0];
}

// workgroups of `kern` that fit on one CU at once (queried once per kernel)
template <typename K>
int resident_blocks(K kern)
{
    static int v = 0;
    if (v == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kBlock, 0) != hipSuccess || n < 1)
            n = 1;
        v = n;
    }
    return v;
}

template <int D>
void launch_encode_rows_d(const EncodeRowsParams &q, int sides, hipStream_t st)
{
    auto kern = encode_rows_kernel<D>;
    const int rpw = 64 / (D / 64);  // rows per wave
    const int64_t groups = (q.n_rows + rpw - 1) / rpw;
    const int64_t need = (groups + kBlock / 64 - 1) / (kBlock / 64);
    // the resident workgroups (split between the sides), each looping
    int64_t cap = (int64_t)device_cus() * resident_blocks(kern) / sides;
    if (cap < 1)
        cap = 1;
    dim3 grid((unsigned)(need < cap ? need : cap), sides), block(kBlock);
    hipLaunchKernelGGL(kern, grid, block, 0, st, q);
}

template <typename T>
void launch_encode(int d, const EncodeParams &p, int sides, hipStream_t st)
{
    dim3 block(kBlock);
    switch (d) {
    case 64: hipLaunchKernelGGL((encode_kernel<64, T>), dim3(grid_for(p.n_rows, Shape<64>::RPB), sides), block, 0, st, p); break;
    case 128: hipLaunchKernelGGL((encode_kernel<128, T>), dim3(grid_for(p.n_rows, Shape<128>::RPB), sides), block, 0, st, p); break;
    default: hipLaunchKernelGGL((encode_kernel<256, T>), dim3(grid_for(p.n_rows, Shape<256>::RPB), sides), block, 0, st, p); break;
    }
}

template <typename T>
void launch_append(int d, const AppendParams &p, int sides, hipStream_t st)
{
    dim3 block(kBlock);
    const int64_t rows = (int64_t)p.n_layers * p.bh;
    switch (d) {
    case 64: hipLaunchKernelGGL((append_kernel<64, T>), dim3(grid_for(rows, Shape<64>::RPB), sides), block, 0, st, p); break;
    case 128: hipLaunchKernelGGL((append_kernel<128, T>), dim3(grid_for(rows, Shape<128>::RPB), sides), block, 0, st, p); break;
    default: hipLaunchKernelGGL((append_kernel<256, T>), dim3(grid_for(rows, Shape<256>::RPB), sides), block, 0, st, p); break;
    }
}

template <int D>
void launch_decode_d(int bits, const DecodeParams &p, hipStream_t st)
{
    dim3 grid(grid_for(p.n_rows, Shape<D>::RPB)), block(kBlock);
    switch (bits) {
    case 2: hipLaunchKernelGGL((decode_kernel<D, 2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((decode_kernel<D, 3>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((decode_kernel<D, 4>), grid, block, 0, st, p); break;
    }
}

template <typename T>
void launch_rotate(int d, const RotateParams &p, hipStream_t st)
{
    dim3 block(kBlock);
    switch (d) {
    case 64: hipLaunchKernelGGL((rotate_kernel<64, T>), dim3(grid_for(p.n_rows, Shape<64>::RPB)), block, 0, st, p); break;
    case 128: hipLaunchKernelGGL((rotate_kernel<128, T>), dim3(grid_for(p.n_rows, Shape<128>::RPB)), block, 0, st, p); break;
    default: hipLaunchKernelGGL((rotate_kernel<256, T>), dim3(grid_for(p.n_rows, Shape<256>::RPB)), block, 0, st, p); break;
    }
}

}  // namespace

// ------------------------------------------------------------ C entry points

extern "C" int tq_rotate(const void *in, int dtype, int64_t n_rows, int d, uint64_t seed,
                         int inverse, float *out, void *stream)
{
    static const char *fn = "tq_rotate";
    tq::clear_error();
    if (dtype != TQ_F32 && dtype != TQ_BF16)
        return tq::fail(TQ_EINVAL, "tq_rotate: unknown dtype");
    if (n_rows < 0)
        return tq::fail(TQ_EINVAL, "tq_rotate: n_rows < 0");
    int rc = check_d(d, fn);
    if (rc != TQ_OK)
        return rc;
    if (n_rows == 0)
        return TQ_OK;
    if (!in || !out)
        return tq::fail(TQ_EINVAL, "tq_rotate: NULL buffer");
    if (!aligned(in, 16) || !aligned(out, 16))
        return tq::fail(TQ_EINVAL, "tq_rotate: buffers must be 16-byte aligned");
    if ((rc = injected(fn)) != TQ_OK)
        return rc;
    RotateParams p;
    p.in = in;
    p.out = out;
    p.n_rows = n_rows;
    p.inverse = inverse ? 1 : 0;
    tq::sign_words(d, seed, p.signs);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == TQ_F32)
        launch_rotate<float>(d, p, st);
    else
        launch_rotate<uint16_t>(d, p, st);
    return launch_status(fn);
}

extern "C" int tq_encode(const void *k_rows, const void *v_rows, int dtype, int64_t n_rows,
                         int d, int bits_k, int bits_v, uint64_t seed, uint8_t *k_packed,
                         float *k_norms, uint8_t *v_packed, float *v_norms, void *stream)
{
    static const char *fn = "tq_encode";
    tq::clear_error();
    if (dtype != TQ_F32 && dtype != TQ_BF16)
        return tq::fail(TQ_EINVAL, "tq_encode: unknown dtype");
    if (n_rows < 0)
        return tq::fail(TQ_EINVAL, "tq_encode: n_rows < 0");
    int rc = check_d(d, fn);
    if (rc != TQ_OK)
        return rc;
    if (n_rows == 0)
        return TQ_OK;  // nothing to do; buffers may be NULL
    if (!k_rows && !v_rows)
        return tq::fail(TQ_EINVAL, "tq_encode: both k_rows and v_rows are NULL");
    EncodeParams p;
    int sides = 0;
    const void *src[2] = {k_rows, v_rows};
    uint8_t *pk[2] = {k_packed, v_packed};
    float *nm[2] = {k_norms, v_norms};
    int bits[2] = {bits_k, bits_v};
    for (int s = 0; s < 2; s++) {
        if (!src[s])
            continue;
        if ((rc = check_bits(bits[s], fn)) != TQ_OK)
            return rc;
        if (!pk[s] || !nm[s])
            return tq::fail(TQ_EINVAL, "tq_encode: NULL output buffer for a non-NULL input");
        if (!aligned(src[s], 16) || !aligned(pk[s], 16) || !aligned(nm[s], 4))
            return tq::fail(TQ_EINVAL, "tq_encode: misaligned buffer (rows and packed need 16 bytes, norms 4)");
        EncodeSide &e = p.side[sides++];
        e.src = src[s];
        e.packed = pk[s];
        e.norms = nm[s];
        if ((rc = code_table(d, bits[s], &e.code, fn)) != TQ_OK)
            return rc;
    }
    if ((rc = injected(fn)) != TQ_OK)
        return rc;
    p.n_rows = n_rows;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == TQ_BF16 && d <= 128) {
        EncodeRowsParams q;
        q.side[0] = p.side[0];
        q.side[1] = p.side[1];
        q.n_rows = n_rows;
        fill_row_signs(d, seed, q);
        if (d == 64)
            launch_encode_rows_d<64>(q, sides, st);
        else
            launch_encode_rows_d<128>(q, sides, st);
        return launch_status(fn);
    }
    tq::sign_words(d, seed, p.signs);
    if (dtype == TQ_F32)
        launch_encode<float>(d, p, sides, st);
    else
        launch_encode<uint16_t>(d, p, sides, st);
    return launch_status(fn);
}

extern "C" int tq_decode(const uint8_t *packed, const float *norms, int64_t n_rows, int d,
                         int bits, uint64_t seed, float *out, void *stream)
{
    static const char *fn = "tq_decode";
    tq::clear_error();
    if (n_rows < 0)
        return tq::fail(TQ_EINVAL, "tq_decode: n_rows < 0");
    int rc = check_d(d, fn);
    if (rc != TQ_OK)
        return rc;
    if ((rc = check_bits(bits, fn)) != TQ_OK)
        return rc;
    if (n_rows == 0)
        return TQ_OK;
    if (!packed || !norms || !out)
        return tq::fail(TQ_EINVAL, "tq_decode: NULL buffer");
    if (!aligned(packed, 16) || !aligned(out, 16) || !aligned(norms, 4))
        return tq::fail(TQ_EINVAL, "tq_decode: misaligned buffer (packed and out need 16 bytes, norms 4)");
    if ((rc = injected(fn)) != TQ_OK)
        return rc;
    tq_codebook cb;
    if ((rc = tq::get_codebook(d, bits, TQ_BETA_HALF_D, &cb)) != TQ_OK)
        return rc;
    DecodeParams p;
    p.packed = packed;
    p.norms = norms;
    p.out = out;
    p.n_rows = n_rows;
    for (int j = 0; j < 16; j++)
        p.cent[j] = j < cb.levels ? cb.centroids[j] : 0.0f;
    tq::sign_words(d, seed, p.signs);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (d) {
    case 64: launch_decode_d<64>(bits, p, st); break;
    case 128: launch_decode_d<128>(bits, p, st); break;
    default: launch_decode_d<256>(bits, p, st); break;
    }
    return launch_status(fn);
}

extern "C" int tq_append_row(const tq_cache_desc *c, int layer, const void *const *k_new,
                             const void *const *v_new, int dtype, int64_t pos, void *stream)
{
    static const char *fn = "tq_append_row";
    tq::clear_error();
    if (!c)
        return tq::fail(TQ_EINVAL, "tq_append_row: cache is NULL");
    if (dtype != TQ_F32 && dtype != TQ_BF16)
        return tq::fail(TQ_EINVAL, "tq_append_row: unknown dtype");
    if (c->n_layers < 1 || c->n_layers > TQ_MAX_LAYERS || c->batch < 0 || c->n_kv_heads < 0 ||
        c->window < 1 || !c->head_dim || !c->k_packed || !c->k_norms || !c->v_packed ||
        !c->v_norms)
        return tq::fail(TQ_EINVAL, "tq_append_row: invalid cache descriptor");
    if (layer < -1 || layer >= c->n_layers)
        return tq::fail(TQ_EINVAL, "tq_append_row: layer out of range");
    if (pos < 0)
        return tq::fail(TQ_EINVAL, "tq_append_row: pos < 0");
    if (!k_new || !v_new)
        return tq::fail(TQ_EINVAL, "tq_append_row: k_new / v_new is NULL");
    int rc;
    if ((rc = check_bits(c->bits_k, fn)) != TQ_OK || (rc = check_bits(c->bits_v, fn)) != TQ_OK)
        return rc;
    const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->n_layers : layer + 1;
    for (int l = l0; l < l1; l++) {
        const int i = l - l0;
        if ((rc = check_d(c->head_dim[l], fn)) != TQ_OK)
            return rc;
        if (!k_new[i] || !v_new[i] || !c->k_packed[l] || !c->k_norms[l] || !c->v_packed[l] ||
            !c->v_norms[l])
            return tq::fail(TQ_EINVAL, "tq_append_row: NULL layer buffer");
        if (!aligned(k_new[i], 16) || !aligned(v_new[i], 16) || !aligned(c->k_packed[l], 16) ||
            !aligned(c->v_packed[l], 16) || !aligned(c->k_norms[l], 4) || !aligned(c->v_norms[l], 4))
            return tq::fail(TQ_EINVAL, "tq_append_row: misaligned layer buffer");
    }
    const int bh = c->batch * c->n_kv_heads;
    if (bh == 0)
        return TQ_OK;
    if ((rc = injected(fn)) != TQ_OK)
        return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int slot = (int)(pos % c->window);
    // one launch per distinct head_dim (and per kMaxAppendLayers layers)
    const int dims[3] = {64, 128, 256};
    for (int di = 0; di < 3; di++) {
        const int d = dims[di];
        AppendParams p;
        p.bh = bh;
        p.window = c->window;
        p.slot = slot;
        tq::sign_words(d, c->seed, p.signs);
        if ((rc = code_table(d, c->bits_k, &p.side[0].code, fn)) != TQ_OK ||
            (rc = code_table(d, c->bits_v, &p.side[1].code, fn)) != TQ_OK)
            return rc;
        p.n_layers = 0;
        for (int l = l0; l <= l1; l++) {
            const bool flush = (l == l1) || (p.n_layers == kMaxAppendLayers);
            if (flush && p.n_layers > 0) {
                if (dtype == TQ_F32)
                    launch_append<float>(d, p, 2, st);
                else
                    launch_append<uint16_t>(d, p, 2, st);
                if ((rc = launch_status(fn)) != TQ_OK)
                    return rc;
                p.n_layers = 0;
            }
            if (l == l1)
                break;
            if (c->head_dim[l] != d)
                continue;
            const int i = l - l0, n = p.n_layers++;
            p.side[0].src[n] = k_new[i];
            p.side[0].packed[n] = c->k_packed[l];
            p.side[0].norms[n] = c->k_norms[l];
            p.side[1].src[n] = v_new[i];
            p.side[1].packed[n] = c->v_packed[l];
            p.side[1].norms[n] = c->v_norms[l];
        }
    }
    return TQ_OK;
}
