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
//   "CITATIONS" -- Two-sided Rademacher signs in WHT (a second sign vector
//     after the butterfly); N(0, 1/d) codebook replacement.
//
// Work decomposition: the lane-slice kernels give each row P = d/32 lanes (32
// coordinates per lane, see tq_device.h); the bf16 encode for d in {64, 128}
// gives each row one lane (below).  Nothing is shared between rows, so there
// are no atomics and the result does not depend on the launch shape.  A
// head_dim that is not a power of two runs at the next one, its rows
// zero-padded ("TurboQuant KV Cache Compression — Spec", Hadamard Transform
// Detail).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <mutex>
#include <string>

#include <vector>

#include "tq_device.h"
#include "tq_internal.h"

using namespace tqd;

namespace {

// ----------------------------------------------------------------- encode

struct CodeTable {
    float bnd[15];
    int bits;
    float istep;  // 2 bits: 1 / (128 b) for the boundaries (-b, 0, b); else 0
};

// One row: norm, sign, rotate, normalise, bucketize, pack.  `valid` false
// lanes compute on zeros and store nothing.  `key` addresses the bucketize
// table built for BITS.
template <int D, int BITS, typename T>
__device__ __forceinline__ void encode_row(const RawSlice<T> &raw, bool valid, int sub,
                                           const SignMasks<T> &sm, uint32_t s2, uint32_t key,
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
        if (m > 0.0f && m <= FLT_MAX && ss == ss) {
            (void)frexpf(m, &nexp);
#pragma unroll
            for (int k = 0; k < kCPL; k++)
                v[k] = ldexpf(v[k], -nexp);
            ss = 0.0f;
#pragma unroll
            for (int k = 0; k < kCPL; k++)
                ss = fmaf(v[k], v[k], ss);
            ss = sum_across<P>(ss);
        } else if (!(m <= FLT_MAX) || ss != ss) {  // an Inf or a NaN (the max skips NaN)
            nbad = ss + m;  // inf or NaN
#pragma unroll
            for (int k = 0; k < kCPL; k++)
                v[k] = 0.0f;
            ss = 0.0f;
        }
    }
    const float n = sqrtf(ss);
    // u = H(D x) / (sqrt(d) n) (S2 H (D x) / (sqrt(d) n) with the second
    // diagonal of the two-sided rotation); zero rows get u = 0
    const float inv = ss > 0.0f ? 1.0f / sqrtf((float)D * ss) : 0.0f;
    fwht_row<P>(v, sub);
    if (s2 != 0u)
        apply_signs(v, s2);
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
    int d_in;            // coordinates per input row (<= D; the rest are zero)
    uint32_t signs[8];
    uint32_t signs2[8];  // second diagonal (two-sided rotation), else zero
};

// Coalesced input for the lane-slice encode (rows of exactly D values): the
// RPW rows of a wave's pass are contiguous, lane l loads 16-byte pieces
// l + 64 q of them (whole cache lines per instruction), and the pass goes
// through LDS into the lane-slice layout (slices of SB bytes at a skewed
// stride SS, against bank conflicts on the slice reads).
template <int D, typename T>
struct PassIO {
    static constexpr int P = Shape<D>::P, RPW = Shape<D>::RPW;
    static constexpr int SB = kCPL * (int)sizeof(T);  // bytes of one lane's slice
    static constexpr int SS = SB + 16;                // LDS slice stride
    static constexpr int RS = P * SS;                 // LDS row stride
    static constexpr int RB = D * (int)sizeof(T);     // input bytes per row
    static constexpr int NQ = RPW * RB / 1024;        // 16-byte pieces per lane
    static constexpr int LDS = RPW * RS;              // LDS bytes per wave
};

template <int D, typename T>
__device__ __forceinline__ void load_pass(const uint8_t *src, int64_t row0, int64_t n_rows,
                                          int lane, u32x4 (&ch)[PassIO<D, T>::NQ])
{
    using IO = PassIO<D, T>;
    const int64_t avail = (n_rows - row0) * IO::RB;  // bytes of real rows from row0 on
    const u32x4 *g = reinterpret_cast<const u32x4 *>(src + row0 * IO::RB) + lane;
    if (avail >= (int64_t)IO::RPW * IO::RB) {  // a whole pass (uniform branch)
#pragma unroll
        for (int q = 0; q < IO::NQ; q++)
            ch[q] = __builtin_nontemporal_load(g + 64 * q);
    } else {
#pragma unroll
        for (int q = 0; q < IO::NQ; q++)
            ch[q] = 16 * (int64_t)(lane + 64 * q) < avail ? __builtin_nontemporal_load(g + 64 * q)
                                                          : u32x4{0u, 0u, 0u, 0u};
    }
}

// The pass from registers into this wave's LDS, then this lane's slice back.
template <int D, typename T>
__device__ __forceinline__ void stage_pass(const u32x4 (&ch)[PassIO<D, T>::NQ], uint8_t *stg,
                                           int lane, int rig, int sub, RawSlice<T> &raw)
{
    using IO = PassIO<D, T>;
    wave_lds_fence();  // every lane is done with the previous pass
#pragma unroll
    for (int q = 0; q < IO::NQ; q++) {
        const int o = 16 * (lane + 64 * q);
        const int row = o / IO::RB, w = o % IO::RB;
        *reinterpret_cast<u32x4 *>(stg + row * IO::RS + (w / IO::SB) * IO::SS + w % IO::SB) = ch[q];
    }
    wave_lds_fence();
    using V = typename std::remove_reference<decltype(raw.q[0])>::type;
    const uint8_t *mine = stg + rig * IO::RS + sub * IO::SS;
#pragma unroll
    for (int j = 0; j < (int)(sizeof(raw.q) / sizeof(raw.q[0])); j++)
        raw.q[j] = *reinterpret_cast<const V *>(mine + 16 * j);
}

template <int D, typename T, int BITS, bool PAD>
__device__ __forceinline__ void encode_contig_loop(const EncodeSide &s, int64_t n_rows,
                                                   int d_in, const SignMasks<T> &sm,
                                                   uint32_t s2, uint32_t key, uint8_t *stg)
{
    constexpr int P = Shape<D>::P, RPW = Shape<D>::RPW, RPB = Shape<D>::RPB;
    constexpr int RB = D * BITS / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % P, rig = lane / P;
    const int64_t stride = (int64_t)gridDim.x * RPB;
    if constexpr (!PAD) {
        using IO = PassIO<D, T>;
        const uint8_t *src = static_cast<const uint8_t *>(s.src);
        int64_t row0 = (int64_t)blockIdx.x * RPB + wave * RPW;  // this wave's pass
        u32x4 ch[IO::NQ];
        load_pass<D, T>(src, row0, n_rows, lane, ch);
        for (int64_t base = (int64_t)blockIdx.x * RPB; base < n_rows; base += stride) {
            // the next pass's loads are issued before this one is transformed
            u32x4 nx[IO::NQ];
            load_pass<D, T>(src, row0 + stride, n_rows, lane, nx);
            RawSlice<T> raw;
            stage_pass<D, T>(ch, stg, lane, rig, sub, raw);
            const int64_t row = row0 + rig;
            const bool valid = row < n_rows;
            const int64_t r = valid ? row : 0;
            encode_row<D, BITS, T>(raw, valid, sub, sm, s2, key, s.packed + r * RB, s.norms + r);
#pragma unroll
            for (int q = 0; q < IO::NQ; q++)
                ch[q] = nx[q];
            row0 += stride;
        }
        return;
    }
    // rows of d_in < D values (padded): each lane loads its own slice
    const T *src = static_cast<const T *>(s.src);
    // a head_dim below D (padded to D) leaves whole slices of zeros
    const bool live = sub * kCPL < d_in;
    int64_t row = (int64_t)blockIdx.x * RPB + wave * RPW + rig;
    RawSlice<T> cur;
    if (row < n_rows && live)
        load_raw(src + row * d_in + sub * kCPL, cur);
    else
        zero_raw(cur);
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < n_rows; base += stride) {
        // issue the next pass's loads before transforming this one
        const int64_t nrow = row + stride;
        RawSlice<T> nxt;
        if (nrow < n_rows && live)
            load_raw(src + nrow * d_in + sub * kCPL, nxt);
        else
            zero_raw(nxt);
        const bool valid = row < n_rows;
        const int64_t r = valid ? row : 0;
        encode_row<D, BITS, T>(cur, valid, sub, sm, s2, key, s.packed + r * RB, s.norms + r);
        cur = nxt;
        row = nrow;
    }
}

// blockIdx.y selects the side (0 = first non-NULL side, 1 = second)
template <int D, typename T, bool PAD>
__global__ __launch_bounds__(kBlock) void encode_kernel(EncodeParams p)
{
    __shared__ float2 lut[kLutBins];
    __shared__ __attribute__((aligned(16))) uint8_t stage[PAD ? 16 : (kBlock / 64) * PassIO<D, T>::LDS];
    uint8_t *stg = stage + (PAD ? 0 : (threadIdx.x >> 6) * PassIO<D, T>::LDS);
    const EncodeSide &s = p.side[blockIdx.y];
    build_lut(lut, s.code.bnd, (1 << s.code.bits) - 1);
    __syncthreads();
    const int sub = (threadIdx.x & 63) % Shape<D>::P;
    const SignMasks<T> sm(p.signs[sub]);
    const uint32_t s2 = p.signs2[sub];
    const uint32_t key = lut_key(lut);
    switch (s.code.bits) {
    case 2: encode_contig_loop<D, T, 2, PAD>(s, p.n_rows, p.d_in, sm, s2, key, stg); break;
    case 3: encode_contig_loop<D, T, 3, PAD>(s, p.n_rows, p.d_in, sm, s2, key, stg); break;
    default: encode_contig_loop<D, T, 4, PAD>(s, p.n_rows, p.d_in, sm, s2, key, stg); break;
    }
}

// ------------------------------------------------- encode, shared helpers
// idx (nbits wide) into the little-endian bit stream w at bit `bit`
template <int NWORDS>
__device__ __forceinline__ void put_bits(uint32_t (&w)[NWORDS], int bit, int nbits, uint32_t idx)
{
    const int wd = bit >> 5, sh = bit & 31;
    w[wd] = lshl_or(idx, sh, w[wd]);
    if (sh + nbits > 32)
        w[wd + 1] |= idx >> (32 - sh);
}

// The table entry (boundary inside the bin, count below it) for T = 128 u,
// from a table built with boundary scale 128
__device__ __forceinline__ f32x2 lut_entry(float t, uint32_t key)
{
    const float g = t + kLutMagic;
    const uint32_t a = (__float_as_uint(g) << 3) + key;
    return *reinterpret_cast<const __attribute__((address_space(3))) f32x2 *>((uintptr_t)a);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------- encode, shared types
struct SignBits8 {
    uint32_t w[8];  // bit k of w[k / 32] set: coordinate k is negated
};

typedef const __attribute__((address_space(3))) uint8_t LdsBytes;
typedef const __attribute__((address_space(3))) u32x4 LdsU32x4;

// ------------------------------------- encode, bf16 rows on the matrix cores
// For d = 32 Q the Hadamard matrix (Sylvester order) factors over coordinate
// k = 32 a + b (segment a, place b) as H_d = H_Q (x) H_32, so the rotation of
// a row is
//   Y_a = H_32 S_a x_a                 (each segment on its own)
//   y_{32 a' + b'} = sum_a (H_Q)_{a' a} Y_a[b']
// with S_a the segment's part of the sign diagonal.  Y_a is a product with a
// fixed +-1 matrix: for 16 rows at a time, two 16 x 16 x 32 bf16 matrix-core
// products per segment (exact products, fp32 sums), S_a folded into the
// constant operand.  The Q-point transform across segments, scaled to
// T = 128 u in its last stage, the table bucketize and the packing then run
// on the vector ALUs: log2 Q add/sub stages per output instead of the whole
// butterfly's log2 d.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (lane l, kq = l / 16):
//   A (16 x 32): lane l holds A[l % 16][8 kq + j], j < 8
//   B (32 x 16): lane l holds B[8 kq + j][l % 16]
//   C (16 x 16): lane l holds C[4 kq + i][l % 16], i < 4
// B is the block's rows: column n = l % 16 is row n of the block, and lane
// l's eight values are coordinates 32 a + 8 kq .. + 7 of it (one 16-byte
// load).  Row m of the constant operand in M-block mb stands for output
// b' = 8 (m / 4) + 4 mb + m % 4, so that lane l ends with outputs
// b' = 8 kq + j (j = 4 mb + i) of row n: eight consecutive coordinates of
// every segment, a byte-aligned field of 8 BITS bits of the packed row.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

struct EncodeMfmaParams {
    EncodeSide side[2];
    int64_t n_rows;
    SignBits8 s1;  // the sign diagonal: bit k set where s_k = -1
    SignBits8 s2;  // second diagonal of the two-sided rotation
    // the bucketize table of side lut_side (-1: none), built on the host
    // (the same entries build_lut computes); a workgroup of that side copies
    // it from the kernel arguments instead of building it
    int lut_side;
    float2 lut[kLutBins];
};

// The constant operand of segment a, M-block mb for this lane: bf16 pairs
// (H_32)[b'][k] s_{32 a + k} for its row m = lane % 16 and k = 8 kq + j.
// (H_32)[b'][k] = (-1)^parity(b' & k) splits over the bits of b' =
// 8 (m / 4) + 4 mb + m % 4 and k = 8 kq + j: parity((m / 4) & kq) for every
// j, j >= 4 when mb = 1, and parity((m % 4) & j), whose masks over j are
// 0x00, 0xAA, 0xCC, 0x66.  With the segment's signs (bits 8 kq .. 8 kq + 7
// of s1.w[a]) that is one byte of negations per (a, mb); `spread` maps each
// nibble of it to two words of bf16 (+-1, +-1) pairs.
__device__ __forceinline__ uint32_t spread_word(uint32_t t)
{
    return 0x3F803F80u | ((t & 1u) << 15) | ((t & 2u) << 30);
}

__device__ __forceinline__ void fill_spread(u32x2 *spread)
{
    if (threadIdx.x < 16)
        spread[threadIdx.x] = u32x2{spread_word(threadIdx.x & 3u), spread_word(threadIdx.x >> 2)};
}

template <int Q>
__device__ __forceinline__ void mfma_rotation_operand(const SignBits8 &s1, int lane,
                                                      const u32x2 *spread, u32x4 (&am)[Q][2])
{
    const int m = lane & 15, kq = lane >> 4;
    const uint32_t h0 = ((__popc((m >> 2) & kq) & 1) ? 0xFFu : 0u) ^
                        ((0x66CCAA00u >> (8 * (m & 3))) & 0xFFu);
    const __attribute__((address_space(3))) u32x2 *sp =
        (const __attribute__((address_space(3))) u32x2 *)spread;
#pragma unroll
    for (int a = 0; a < Q; a++) {
        const uint32_t sg = (s1.w[a] >> (8 * kq)) & 0xFFu;
#pragma unroll
        for (int mb = 0; mb < 2; mb++) {
            const uint32_t neg = h0 ^ sg ^ (mb ? 0xF0u : 0u);
            const u32x2 lo = sp[neg & 15u], hi = sp[neg >> 4];
            am[a][mb] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
    }
}

// Ring of block inputs in LDS: the loads of a block go straight from memory
// to its slot (no registers held while they are in flight).  Instruction i
// of a block reads the block's rows RPI i .. RPI i + RPI - 1 (RPI =
// 1024 / (2 D)), 1 KiB of memory in one piece, whole lines, and puts lane
// l's 16 bytes at byte 16 l of the slot's region i; the regions are kSeg
// bytes apart (1024 + 16), so that the B operands read back without bank
// conflicts.  Lane l = 16 kq + Q r + s fetches row RPI i + r, the 16 bytes
// 8 kq .. 8 kq + 7 of segment s.  The operand of segment a for lane (n, kq)
// is then granule 16 kq + Q r + a of region i = n / RPI (r = n % RPI), at
// 16-byte bank group i + Q r + a (mod 16): for each (a, kq) the 16 rows fall
// in 16 different groups.  Rows past n_rows load row n_rows - 1 instead
// (every block issues the same loads, so the wait counts below hold) and
// read as zeros.
constexpr int kSeg = 1024 + 16;

template <int D>
__device__ __forceinline__ void issue_block_lds(const uint8_t *src, int64_t r0, int64_t n_rows,
                                                int lane, uint8_t *slot)
{
    constexpr int Q = D / 32, RPI = 512 / D;
    // a uniform base (the block's first row, or the last row) and a 32-bit
    // offset per lane
    const int64_t b0 = r0 < n_rows ? r0 : n_rows - 1;
    const uint64_t ga = (uint64_t)(uintptr_t)(src + b0 * (2 * D));
    // uniform (scalar registers); the builtin returns int: both halves are
    // widened as unsigned, or a low word at or above 2^31 would sign-extend
    // into the high one
    const uint32_t ga_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ga >> 32));
    const uint32_t ga_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ga);
    const uint8_t *gb = (const uint8_t *)(uintptr_t)(((uint64_t)ga_hi << 32) | (uint64_t)ga_lo);
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LdsBytes *)slot);
    const int kq = lane >> 4, r = (lane & 15) / Q, sg = lane & (Q - 1);
    const uint32_t lane_off = (uint32_t)(r * (2 * D) + 64 * sg + 16 * kq);
    // Written out rather than through the compiler's builtin, whose tracking
    // of loads into LDS makes every later LDS read wait for all of them: the
    // waits for these are placed by hand (wait_vmcnt).  No register is
    // written: the data goes to LDS at M0 + 16 lane (the instruction's offset
    // field would move the LDS address as well, so it stays 0).
    auto dma = [](uint32_t voff, const uint8_t *g, uint32_t m0) {
        asm volatile("s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dwordx4 %0, %1"
                     :
                     : "v"(voff), "s"(g), "s"(m0)
                     : "memory", "m0");
    };
    if (b0 + 16 <= n_rows) {  // uniform: a whole block, instruction i lane_off past row RPI i
#pragma unroll
        for (int i = 0; i < Q; i++)
            dma(lane_off, gb + 1024 * i, base + kSeg * i);
    } else {  // at the end: rows clamped to the last one
        const int last = (int)(n_rows - 1 - b0);
#pragma unroll
        for (int i = 0; i < Q; i++)
            dma((uint32_t)(min(RPI * i + r, last) * (2 * D) + 64 * sg + 16 * kq), gb,
                base + kSeg * i);
    }
}

template <int D>
__device__ __forceinline__ void read_block_lds(const uint8_t *slot, int64_t r0, int64_t n_rows,
                                               int lane, u32x4 (&x)[D / 32])
{
    constexpr int Q = D / 32, RPI = 512 / D;
    const int n = lane & 15, kq = lane >> 4;
    LdsBytes *rp = (LdsBytes *)slot + kSeg * (n / RPI) + 16 * (16 * kq + Q * (n % RPI));
#pragma unroll
    for (int a = 0; a < Q; a++)
        x[a] = *reinterpret_cast<LdsU32x4 *>(rp + 16 * a);
    if (r0 + 16 > n_rows) {  // uniform: a block at the end
        const bool ok = r0 + n < n_rows;
#pragma unroll
        for (int a = 0; a < Q; a++)
            x[a] = ok ? x[a] : u32x4{0u, 0u, 0u, 0u};
    }
}

// op over the four lanes holding parts of one row (lanes n, n + 16, n + 32,
// n + 48): the swaps of 16-lane rows and of 32-lane halves pair each lane
// with its partners in registers, and both lanes of a pair combine the same
// two values in the same order, so the four lanes end with identical bits.
template <typename F>
__device__ __forceinline__ float row_across_kq(float v, F op)
{
    const uint32_t u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = op(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const uint32_t w = __float_as_uint(v);
    const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return op(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Sum of squares of row lane % 16 of a block: each of the four lanes holding
// a part of it adds its 8 Q values, then the parts are exchanged, so the
// four lanes end with the same value (products exact, fp32 sums)
template <int Q>
__device__ __forceinline__ float mfma_block_sumsq(const u32x4 (&x)[Q])
{
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int a = 0; a < Q; a++) {
        s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(x[a].x), as_bf16x2(x[a].x), s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(x[a].y), as_bf16x2(x[a].y), s1, false);
        s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(x[a].z), as_bf16x2(x[a].z), s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(x[a].w), as_bf16x2(x[a].w), s1, false);
    }
    return row_across_kq(s0 + s1, [](float a, float b) { return a + b; });
}

// the block's 2 Q products, M-block by M-block (the first M-block's results,
// which the transform takes first, are ready first)
template <int Q>
__device__ __forceinline__ void mfma_block_products(const u32x4 (&am)[Q][2], const u32x4 (&x)[Q],
                                                    f32x4 (&acc)[Q][2])
{
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int a = 0; a < Q; a++)
            acc[a][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, am[a][mb]), __builtin_bit_cast(bf16x8_t, x[a]),
                f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
}

// Where byte o of row n of a block's packed rows sits in the wave's LDS stage
// (16 rows of RB bytes): its 16-byte granule is exchanged with granule
// c ^ f(n), so that the lanes of one store (rows n, four lanes each) fall in
// different banks where RB / 4 words per row divide the 64 banks; the
// readback undoes the exchange.
template <int RB>
constexpr bool stage_swizzled()
{
    return RB % 16 == 0 && ((RB / 4) & (RB / 4 - 1)) == 0 && RB / 4 <= 64;
}

template <int RB>
__device__ __forceinline__ int stage_offset(int n, int o)
{
    if constexpr (stage_swizzled<RB>()) {
        constexpr int G = RB / 16, P = 256 / RB;  // granules per row; rows per bank cycle
        const int f = (n / P) % G;
        return n * RB + (((o >> 4) ^ f) << 4) + (o & 15);
    } else {
        return n * RB + o;
    }
}

// where granule e of the block's dense packed rows sits in the stage
template <int RB>
__device__ __forceinline__ int stage_granule(int e)
{
    if constexpr (stage_swizzled<RB>())
        return stage_offset<RB>(e / (RB / 16), 16 * (e % (RB / 16)));
    else
        return 16 * e;
}

// store instructions of a whole block's packed rows (RB granules of 16 bytes)
template <int RB>
constexpr int kMfmaStores = (RB + 63) / 64;

// Encode one block (16 rows starting at r0) of one side: the rows arrive in
// x in the B layout; packed rows and norms go to memory through the wave's
// LDS stage.
template <int D, int BITS, bool S2>
__device__ __forceinline__ void mfma_block(u32x4 (&x)[D / 32], const u32x4 (&am)[D / 32][2],
                                           const EncodeSide &s, uint32_t key, const SignBits8 &s2,
                                           int64_t r0, int64_t n_rows, uint8_t *stg, int lane)
{
    constexpr int Q = D / 32, RB = D * BITS / 8, H = Q / 2;
    const int n = lane & 15, kq = lane >> 4;
    // the products first: the sum of squares and the scale are worked out
    // while the matrix cores run
    f32x4 acc[Q][2];
    mfma_block_products<Q>(am, x, acc);
    __builtin_amdgcn_sched_barrier(0);
    float ss = mfma_block_sumsq<Q>(x);
    int nexp = 0;
    bool bad = false;
    const bool rare = !(ss >= 0x1p-100f && ss <= 0x1p100f);
    if (__builtin_amdgcn_ballot_w64(rare) != 0) {
        // rare (a wave-uniform branch): rows out of range are rewritten as
        // x * 2^-nexp (max |x| in [1/2, 1)), or zeros if they hold an Inf or
        // a NaN, and the block's products are taken again
        float mx = 0.0f;
#pragma unroll
        for (int a = 0; a < Q; a++) {
            const uint32_t xw[4] = {x[a].x, x[a].y, x[a].z, x[a].w};
#pragma unroll
            for (int c = 0; c < 4; c++)
                mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(xw[c])), fabsf(bf16_hi(xw[c]))));
        }
        mx = row_across_kq(mx, [](float a, float b) { return fmaxf(a, b); });
        const float ss0 = ss;  // the fast path's sum
        bad = rare && (!(mx <= FLT_MAX) || ss0 != ss0);  // an Inf or a NaN (the max skips NaN)
        if (rare && !bad && mx > 0.0f)
            (void)frexpf(mx, &nexp);
        if (rare) {
#pragma unroll
            for (int a = 0; a < Q; a++) {
                uint32_t xw[4] = {x[a].x, x[a].y, x[a].z, x[a].w};
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    // exact for normal results; parts below 2^-126 of the
                    // largest magnitude may round, far under fp32 precision
                    const float x0 = bad ? 0.0f : ldexpf(bf16_lo(xw[c]), -nexp);
                    const float x1 = bad ? 0.0f : ldexpf(bf16_hi(xw[c]), -nexp);
                    xw[c] = (__float_as_uint(x1) & 0xFFFF0000u) | (__float_as_uint(x0) >> 16);
                }
                x[a] = u32x4{xw[0], xw[1], xw[2], xw[3]};
            }
        }
        ss = mfma_block_sumsq<Q>(x);
        if (bad)
            ss = ss0 + mx;  // stored as the norm: not finite
        mfma_block_products<Q>(am, x, acc);
    }
    // the hardware reciprocal square root and square root (about 1 ulp):
    // every block takes them, four lanes per row, so the correctly rounded
    // expansions would cost a fifth of the block; their error stays two
    // orders under the tolerance of u and of the norm
    const float t = (ss > 0.0f && !bad) ? 128.0f * __builtin_amdgcn_rsqf((float)D * ss) : 0.0f;
    const float nrm = bad ? ss : ldexpf(__builtin_amdgcn_sqrtf(ss), nexp);
    // the Q-point transform across segments for each of the lane's eight
    // places j = 4 mb + i; the last stage carries the scale
    const float ts = BITS == 2 ? t * s.code.istep : t;
    float T[Q][8];
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float v[Q];
#pragma unroll
            for (int a = 0; a < Q; a++)
                v[a] = acc[a][mb][i];
#pragma unroll
            for (int h = 1; h < H; h *= 2)
#pragma unroll
                for (int j = 0; j < Q; j += 2 * h)
#pragma unroll
                    for (int a = j; a < j + h; a++) {
                        const float u = v[a], w = v[a + h];
                        v[a] = u + w;
                        v[a + h] = u - w;
                    }
#pragma unroll
            for (int a = 0; a < H; a++) {
                const float bt = v[a + H] * ts;
                T[a][4 * mb + i] = fmaf(v[a], ts, bt);
                T[a + H][4 * mb + i] = fmaf(v[a], ts, -bt);
            }
        }
#pragma unroll
    for (int a = 0; a < Q; a++) {
        if constexpr (S2) {
            // the second diagonal's signs of coordinates 32 a + 8 kq + j
            // (taken per block: hoisted, the Q words would stay in registers)
            int kql = kq;
            asm volatile("" : "+v"(kql));
            const uint32_t sb = s2.w[a] >> (8 * kql);
#pragma unroll
            for (int j = 0; j < 8; j++)
                T[a][j] = __uint_as_float(__float_as_uint(T[a][j]) ^ ((sb << (31 - j)) & 0x80000000u));
        }
        uint32_t w;
        if constexpr (BITS == 2) {
            // boundaries -b, 0, b equally spaced (T scaled by 1 / b): the
            // field collects sum c 4^j with c = clamp(floor(-T), -2, 1) and
            // takes 0x5555 - that
            uint32_t we = 0u, wo = 0u;
#pragma unroll
            for (int j = 0; j < 8; j += 2)
                pack_c2(T[a][j], T[a][j + 1], 2 * j, 2 * j + 2, we, wo);
            w = 0x5555u - (we + wo);
        } else {
            uint32_t idx[8];
#pragma unroll
            for (int h = 0; h < 8; h += 4) {
                float tt[4], bb[4];
                uint32_t base[4], id4[4];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    tt[r] = T[a][h + r];
                    const f32x2 e = lut_entry(tt[r], key);
                    bb[r] = e.x;
                    base[r] = __float_as_uint(e.y);
                }
                bucket_add4(tt, bb, base, id4);
#pragma unroll
                for (int r = 0; r < 4; r++)
                    idx[h + r] = id4[r];
            }
            w = idx[0];
#pragma unroll
            for (int j = 1; j < 8; j++)
                w = lshl_or(idx[j], BITS * j, w);
        }
        // the field: 8 BITS bits at byte BITS (4 a + kq) of row n
        if constexpr (BITS == 4) {
            *reinterpret_cast<uint32_t *>(stg + stage_offset<RB>(n, 16 * a + 4 * kq)) = w;
        } else if constexpr (BITS == 2) {
            *reinterpret_cast<uint16_t *>(stg + stage_offset<RB>(n, 8 * a + 2 * kq)) = (uint16_t)w;
        } else {
            // three bytes at 12 a + 3 kq: a halfword and a byte, the
            // halfword at the even address
            const bool odd = (kq & 1) != 0;
            uint8_t *f = stg + stage_offset<RB>(n, 12 * a + 3 * kq);
            *reinterpret_cast<uint16_t *>(f + (odd ? 1 : 0)) = (uint16_t)(odd ? w >> 8 : w);
            f[odd ? 0 : 2] = (uint8_t)(odd ? w : w >> 16);
        }
    }
    // the block's packed rows (dense, as in memory: whole lines where the
    // block is whole) and norms
    const int nvalid = (int)min<int64_t>(16, n_rows - r0);
    wave_lds_fence();
    if (nvalid == 16) {
        // a whole block: every lane stores, without branches; the four
        // lanes of a row store the same norm, and lanes past the block's RB
        // granules repeat granules
        *as_global(s.norms + r0 + n) = nrm;
        __attribute__((address_space(1))) u32x4 *dst =
            reinterpret_cast<__attribute__((address_space(1))) u32x4 *>(as_global(s.packed + r0 * RB));
#pragma unroll
        for (int q = 0; q < kMfmaStores<RB>; q++) {
            const int e = (64 * q + lane) % RB;  // granule (16 rows of RB bytes: RB granules)
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + stage_granule<RB>(e));
            __builtin_nontemporal_store(v, dst + e);
        }
    } else {
        if (kq == 0 && n < nvalid)
            *as_global(s.norms + r0 + n) = nrm;
        const int bytes = nvalid * RB;
        __attribute__((address_space(1))) uint8_t *dst = as_global(s.packed + r0 * RB);
#pragma unroll
        for (int q = 0; q < (16 * RB + 1023) / 1024; q++) {
            const int e = 64 * q + lane;  // 16-byte granule of the block's packed rows
            if (16 * e + 16 <= bytes) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + stage_granule<RB>(e));
                __builtin_nontemporal_store(v, reinterpret_cast<__attribute__((address_space(1))) u32x4 *>(dst) + e);
            } else if (16 * e < bytes) {  // an 8-byte tail (RB is a multiple of 8, not of 16)
                *reinterpret_cast<__attribute__((address_space(1))) u32x2 *>(dst + 16 * e) =
                    *reinterpret_cast<const u32x2 *>(stg + 16 * e);
            }
        }
    }
    wave_lds_fence();
}

// Waits on the vector-memory count or the LDS count alone (memory clobbers: no memory access moves across them)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkmcnt0()
{
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
}

template <int D>
constexpr int ring_slots()
{
    return D == 64 ? 3 : 2;
}

// One group of 64 rows of one side per wave: its four blocks pass through
// the wave's ring of R slots, a slot refilled with the group's next block as
// soon as it has been read into registers.
template <int D, int BITS, bool S2>
__device__ __forceinline__ void mfma_group(const EncodeSide &s, int64_t g0, int64_t n_rows,
                                           uint32_t key, const SignBits8 &s2,
                                           const u32x4 (&am)[D / 32][2], uint8_t *slots,
                                           uint8_t *stg, int lane)
{
    constexpr int Q = D / 32, R = ring_slots<D>(), SLOT = Q * kSeg;
    const uint8_t *src = static_cast<const uint8_t *>(s.src);
    // (the first R blocks' loads were issued by the caller)
#pragma unroll 1
    for (int u = 0; u < 4; u++) {
        const int64_t r0 = g0 + 16 * u;
        uint8_t *slot = slots + (u % R) * SLOT;
        // this block's loads are done once at most those issued after them
        // are outstanding: the group's next R - 1 blocks (loads complete in
        // order; stores are not ordered with them and are left out, which
        // can only wait longer).  Near the group's end fewer follow: all.
        if (u + R <= 4)
            wait_vmcnt<(R - 1) * Q>();
        else
            wait_vmcnt<0>();
        u32x4 x[Q];
        read_block_lds<D>(slot, r0, n_rows, lane, x);
        if (u + R < 4) {
            wait_lgkmcnt0();  // the slot is read before it is refilled
            issue_block_lds<D>(src, g0 + 16 * (u + R), n_rows, lane, slot);
        }
        if (r0 < n_rows)
            mfma_block<D, BITS, S2>(x, am, s, key, s2, r0, n_rows, stg, lane);
    }
}

// One launch, one group of 64 rows per wave, every group of the first side
// before any of the second (workgroups [0, nb) take the first side, [nb, 2 nb)
// the second): the launch walks memory as one compact window, side by side.
// Measured on the bulk workload, a streaming kernel of this traffic with no
// arithmetic reaches 76% of HBM in this order and about 70% when each wave
// loops over many groups or alternates the sides.
template <int D, int B0, int B1, bool S2>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(D == 256 ? 2 : 4)))
void encode_mfma_kernel(EncodeMfmaParams p)
{
    constexpr int Q = D / 32, R = ring_slots<D>();
    constexpr int RBM = D * B0 / 8;  // B0 >= B1
    constexpr int SLOT = Q * kSeg;   // Q regions of 1 KiB, padded
    __shared__ float2 lut[(B0 > 2 || B1 > 2) ? kLutBins : 1];
    __shared__ u32x2 spread[16];
    __shared__ __attribute__((aligned(16))) uint8_t ring[kBlock / 64][R * SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t stage[kBlock / 64][16 * RBM];
    const int64_t n_rows = p.n_rows;
    const int64_t nb = (n_rows + 255) / 256;  // workgroups per side
    const bool second = B1 > 0 && (int64_t)blockIdx.x >= nb;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t g0 = (((int64_t)blockIdx.x - (second ? nb : 0)) * (kBlock / 64) + wave) * 64;
    // the group's first loads go out before the set-up below (rows past the
    // end load the last row, so a wave past n_rows issues them too)
    {
        const uint8_t *src = static_cast<const uint8_t *>(second ? p.side[1].src : p.side[0].src);
#pragma unroll
        for (int u = 0; u < R; u++)
            issue_block_lds<D>(src, g0 + 16 * u, n_rows, lane, ring[wave] + u * SLOT);
    }
    if (p.lut_side == (second ? 1 : 0)) {
        // the table from the kernel arguments (one 8-byte load per entry)
        typedef const __attribute__((address_space(4))) u32x2 KU32x2;
        KU32x2 *klut = (KU32x2 *)((const __attribute__((address_space(4))) char *)
                                      __builtin_amdgcn_kernarg_segment_ptr() +
                                  offsetof(EncodeMfmaParams, lut));
        for (int i = threadIdx.x; i < kLutBins; i += kBlock)
            reinterpret_cast<u32x2 *>(lut)[i] = klut[i];
    } else if (second) {
        if constexpr (B1 > 2)
            build_lut(lut, p.side[1].code.bnd, (1 << B1) - 1, kLutScale);
    } else {
        if constexpr (B0 > 2)
            build_lut(lut, p.side[0].code.bnd, (1 << B0) - 1, kLutScale);
    }
    fill_spread(spread);
    __syncthreads();
    if (g0 >= n_rows) {
        wait_vmcnt<0>();  // no load into LDS outlives the wave
        return;
    }
    u32x4 am[Q][2];
    mfma_rotation_operand<Q>(p.s1, lane, spread, am);
    const uint32_t key = lut_key(lut);
    if constexpr (B1 > 0) {
        if (second) {
            mfma_group<D, (B1 > 0 ? B1 : B0), S2>(p.side[1], g0, n_rows, key, p.s2, am, ring[wave],
                                                  stage[wave], lane);
            return;
        }
    }
    mfma_group<D, B0, S2>(p.side[0], g0, n_rows, key, p.s2, am, ring[wave], stage[wave], lane);
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
    int d_in;         // coordinates per new row (<= D; the rest are zero)
    uint32_t signs[8];
    uint32_t signs2[8];  // second diagonal (two-sided rotation), else zero
};

template <int D, typename T, int BITS>
__device__ __forceinline__ void append_loop(const AppendSide &s, const AppendParams &p,
                                            const SignMasks<T> &sm, uint32_t s2, uint32_t key)
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
        const T *src = static_cast<const T *>(s.src[li]) + (int64_t)j * p.d_in + sub * kCPL;
        const int64_t dst = (int64_t)j * p.window + p.slot;
        RawSlice<T> raw;
        if (valid && sub * kCPL < p.d_in)
            load_raw(src, raw);
        else
            zero_raw(raw);
        encode_row<D, BITS, T>(raw, valid, sub, sm, s2, key, s.packed[li] + dst * RB,
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
    const uint32_t s2 = p.signs2[sub];
    const uint32_t key = lut_key(lut);
    switch (s.code.bits) {
    case 2: append_loop<D, T, 2>(s, p, sm, s2, key); break;
    case 3: append_loop<D, T, 3>(s, p, sm, s2, key); break;
    default: append_loop<D, T, 4>(s, p, sm, s2, key); break;
    }
}

// ----------------------------------------------------------------- decode

// Per-call tables of a decode: centroids, the sign words of this lane's
// slice, and the xor masks of the two-sided rotation
struct DecodeTables {
    float cent[16];
    uint32_t signs[8];
    // packed-row xor mask: all bits of index i set where the second diagonal
    // of the two-sided rotation is -1 (else zero).  The centroid table is
    // exactly symmetric, c[L-1-k] = -c[k], so flipping the index bits is the
    // exact negation of n c[idx].
    uint32_t flip[32];
    int two_sided;  // flip is nonzero
    int d_out;      // coordinates kept per output row (PAD kernels; else D)
};

struct DecodeParams {
    DecodeTables t;
    const uint8_t *packed;
    const float *norms;
    float *out;
    int64_t n_rows;
    int64_t row_base;  // first row of this launch
};

// One wave per workgroup, one pass of RPW rows per wave, and one launch (or
// a few, for grids beyond the launch limit) covering all rows: short-lived
// workgroups keep the write stream in few DRAM pages at a time, which a
// persistent grid-stride loop does not.  The packed words and the norm are
// both requested before either is used (one memory round trip, not two).
constexpr int kDecodeBlock = 64;

// The wave's RPW consecutive rows: packed rows from `in`, norms from `nrm`,
// `valid` (1..RPW) of them written to `out` (rows of D floats, or of d_out
// for PAD).  Rows past `valid` read row 0 and are not stored.
template <int D, int BITS, bool PAD>
__device__ __forceinline__ void decode_wave(const DecodeTables &t, const uint8_t *in,
                                            const float *nrm, float *out, int valid)
{
    constexpr int P = Shape<D>::P, RPW = Shape<D>::RPW;
    constexpr int RB = D * BITS / 8;
    __shared__ float cent[16];
    __shared__ __attribute__((aligned(16))) float stage[kStageFloats];
    if (threadIdx.x < 16)
        cent[threadIdx.x] = t.cent[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x;
    const int sub = lane % P, rig = lane / P;
    const uint32_t smask = t.signs[sub];
    uint32_t w[BITS];
    float n;
    {
        const int r = rig < valid ? rig : 0;
        load_words<BITS>(in + (int64_t)r * RB + sub * 4 * BITS, w);
        n = nrm[r];
    }
    if (t.two_sided) {
#pragma unroll
        for (int j = 0; j < BITS; j++)
            w[j] ^= t.flip[sub * BITS + j];
    }
    float v[kCPL];
#pragma unroll
    for (int k = 0; k < kCPL; k++)
        v[k] = cent[get_index<BITS>(w, k)];
    fwht_row<P>(v, sub);
    const float sc = n * (1.0f / sqrtf((float)D));
#pragma unroll
    for (int k = 0; k < kCPL; k++)
        v[k] *= sc;
    apply_signs(v, smask);
    if constexpr (PAD) {
        // head_dim d_out < D: rows of d_out floats, the padded slices dropped
        store_region_padded<P>(out, v, stage, lane, (int64_t)valid * t.d_out, t.d_out / kCPL);
    } else {
        (void)RPW;
        store_region_coalesced(out, v, stage, lane, (int64_t)valid * D);
    }
}

template <int D, int BITS, bool PAD>
__global__ __launch_bounds__(kDecodeBlock) void decode_kernel(DecodeParams p)
{
    constexpr int RPW = Shape<D>::RPW, RB = D * BITS / 8;
    const int64_t row0 = p.row_base + (int64_t)blockIdx.x * RPW;
    if (row0 >= p.n_rows)
        return;
    const int valid = (int)min<int64_t>(RPW, p.n_rows - row0);
    decode_wave<D, BITS, PAD>(p.t, p.packed + row0 * RB, p.norms + row0,
                              p.out + row0 * (PAD ? p.t.d_out : D), valid);
}

// ---- Decode of a range of ring slots of cache layers ([Foundry] API
// "Quantize / Dequantize": dequantize a range of cached positions of a
// layer).  One launch covers up to kMaxDecodeSegs (layer, K or V) buffers of
// one (D, bits, padding): blockIdx.z picks the buffer, blockIdx.y the
// (sequence, head) (plus bh_base), blockIdx.x a run of RPW slots.  Slots
// [start, start + count) of every (sequence, head) go to out rows
// [bh][count][d_out].
constexpr int kMaxDecodeSegs = 64;

struct CacheDecodeParams {
    DecodeTables t;
    const uint8_t *packed[kMaxDecodeSegs];
    const float *norms[kMaxDecodeSegs];
    float *out[kMaxDecodeSegs];
    int window, start, count, bh_base;
};

template <int D, int BITS, bool PAD>
__global__ __launch_bounds__(kDecodeBlock) void cache_decode_kernel(CacheDecodeParams p)
{
    constexpr int RPW = Shape<D>::RPW, RB = D * BITS / 8;
    const int seg = blockIdx.z;
    const int64_t bh = (int64_t)p.bh_base + blockIdx.y;
    const int slot0 = blockIdx.x * RPW;
    const int valid = min(RPW, p.count - slot0);
    const int64_t row = bh * p.window + p.start + slot0;  // first packed row
    decode_wave<D, BITS, PAD>(p.t, p.packed[seg] + row * RB, p.norms[seg] + row,
                              p.out[seg] + (bh * p.count + slot0) * (PAD ? p.t.d_out : D), valid);
}

// ----------------------------------------------------------------- rotate

struct RotateParams {
    const void *in;
    float *out;
    int64_t n_rows;
    int64_t row_base;  // first row of this launch
    int inverse;
    uint32_t signs[8];
    uint32_t signs2[8];  // second diagonal (two-sided rotation), else zero
};

template <int D, typename T>
__global__ __launch_bounds__(kBlock) void rotate_kernel(RotateParams p)
{
    constexpr int P = Shape<D>::P, RPW = Shape<D>::RPW, RPB = Shape<D>::RPB;
    __shared__ __attribute__((aligned(16))) float stage[kBlock / 64][kStageFloats];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % P, rig = lane / P;
    const int64_t row0 = p.row_base + (int64_t)blockIdx.x * RPB + wave * RPW;
    if (row0 >= p.n_rows)
        return;
    const int64_t row = row0 + rig;
    const int64_t r = row < p.n_rows ? row : row0;
    const uint32_t smask = p.signs[sub], s2 = p.signs2[sub];
    float v[kCPL];
    load_slice(static_cast<const T *>(p.in) + r * D + sub * kCPL, v);
    // forward S2 H S1, inverse S1 H S2 (S2 = identity when one-sided)
    apply_signs(v, p.inverse ? s2 : smask);
    fwht_row<P>(v, sub);
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
#pragma unroll
    for (int k = 0; k < kCPL; k++)
        v[k] *= inv_sqrt_d;
    apply_signs(v, p.inverse ? smask : s2);
    store_region_coalesced(p.out + row0 * D, v, stage[wave], lane, (p.n_rows - row0) * D);
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

// One workgroup per `rpb` rows, in launches of at most kMaxGrid workgroups:
// calls launch(grid, first_row) for each.
constexpr int64_t kMaxGrid = 1 << 30;

template <typename F>
void launch_all(int64_t n_rows, int rpb, F launch)
{
    const int64_t per = kMaxGrid * rpb;
    for (int64_t first = 0; first < n_rows; first += per) {
        const int64_t rows = n_rows - first < per ? n_rows - first : per;
        launch(dim3((unsigned)((rows + rpb - 1) / rpb)), first);
    }
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// d supported by the device kernels, else the status to return: 64, 128,
// 256, and (allow_pad) the multiples of 32 between them, which run padded to
// the next power of two
int check_d(int d, const char *fn, bool allow_pad = true)
{
    const int dp = tq::padded_dim(d);
    if (dp == 0)
        return tq::fail(TQ_EINVAL, std::string(fn) + ": d outside 2..2^20");
    if ((dp == 64 || dp == 128 || dp == 256) && (d == dp || (allow_pad && d % 32 == 0)))
        return TQ_OK;
    return tq::fail(TQ_EUNSUPPORTED,
                    std::string(fn) + (allow_pad ? ": device kernels take d in {64, 128, 256} "
                                                   "or a multiple of 32 between 64 and 256"
                                                 : ": device kernels take d in {64, 128, 256}"));
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
int code_table(int d, int bits, int density, CodeTable *t, const char *fn)
{
    tq_codebook cb;
    int rc = tq::get_codebook(d, bits, density, &cb);
    if (rc != TQ_OK)
        return rc;
    t->bits = bits;
    for (int j = 0; j < 15; j++)
        t->bnd[j] = j < cb.levels - 1 ? cb.boundaries[j] : 0.0f;
    for (int j = 0; j + 1 < cb.levels - 1; j++)
        if (cb.boundaries[j + 1] - cb.boundaries[j] <= 1.0f / kLutScale + 2.0f * kLutSlack)
            return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": codebook boundaries too close for the bucketize table");
    t->istep = 0.0f;
    if (bits == 2) {
        // the three boundaries are -b, 0, b (the codebook is symmetric)
        if (!(cb.boundaries[1] == 0.0f && cb.boundaries[0] == -cb.boundaries[2] && cb.boundaries[2] > 0.0f))
            return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": 2-bit codebook is not symmetric");
        t->istep = 1.0f / (kLutScale * cb.boundaries[2]);
    }
    return TQ_OK;
}

// The decode kernel's packed-row xor mask (DecodeParams::flip): the packed
// row (LSB-first bitstream) of indices L-1 where the second diagonal is -1,
// 0 elsewhere; all zero for the one-sided rotation.
void flip_words(int d, int bits, uint64_t seed, uint32_t flags, uint32_t *flip)
{
    uint32_t s2[8];
    tq::sign_words2(d, seed, flags, s2);
    for (int j = 0; j < 32; j++)
        flip[j] = 0u;
    const uint32_t all = (1u << bits) - 1u;
    for (int i = 0; i < d; i++) {
        if (!((s2[i / 32] >> (i % 32)) & 1u))
            continue;
        const int bit = i * bits, wd = bit / 32, sh = bit % 32;
        flip[wd] |= all << sh;
        if (sh + bits > 32)
            flip[wd + 1] |= all >> (32 - sh);
    }
}

void fill_decode_tables(const tq_codebook &cb, int d, int D, int bits, uint64_t seed,
                        uint32_t flags, DecodeTables *t)
{
    for (int j = 0; j < 16; j++)
        t->cent[j] = j < cb.levels ? cb.centroids[j] : 0.0f;
    tq::sign_words(D, seed, t->signs);
    flip_words(D, bits, seed, flags, t->flip);
    t->two_sided = (flags & TQ_FLAG_TWO_SIDED) ? 1 : 0;
    t->d_out = d;
}

// The decode kernels negate through the index bits: the codebook must be
// exactly symmetric
int decode_codebook(int D, int bits, uint32_t flags, tq_codebook *cb, const char *fn)
{
    int rc = tq::get_codebook(D, bits, tq::density_of(flags), cb);
    if (rc != TQ_OK)
        return rc;
    for (int j = 0; j < cb->levels; j++)
        if (cb->centroids[cb->levels - 1 - j] != -cb->centroids[j])
            return tq::fail(TQ_EUNSUPPORTED, std::string(fn) + ": codebook is not symmetric");
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

// workgroups of `kern` that fit on one CU at once (queried once per kernel
// and device)
template <typename K>
int resident_blocks(K kern, int block = kBlock)
{
    static std::mutex mu;
    static const void *keys[64];
    static int vals[64];
    static int nkeys = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const void *key = reinterpret_cast<const void *>(kern);
    std::lock_guard<std::mutex> lk(mu);
    for (int i = 0; i < nkeys; i++)
        if (keys[i] == key && vals[i] >> 16 == dev)
            return vals[i] & 0xFFFF;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, block, 0) != hipSuccess || n < 1)
        n = 1;
    if (nkeys < 64) {
        keys[nkeys] = key;
        vals[nkeys++] = (dev << 16) | (n & 0xFFFF);
    }
    return n;
}

// The bucketize table as build_lut fills it on the device (the same float
// operations: the bin edges are exact multiples of 1/128 less or more the
// slack, each rounded once, so the entries are identical)
void host_lut(const float *bnd, int nbnd, float bscale, float2 *lut)
{
    for (int i = 0; i < kLutBins; i++) {
        const float lo = ((float)(i - kLutZero) - 0.5f) * (1.0f / kLutScale) - kLutSlack;
        const float hi = ((float)(i - kLutZero) + 0.5f) * (1.0f / kLutScale) + kLutSlack;
        int base = 0;
        float inside = __builtin_huge_valf();
        for (int j = 0; j < nbnd; j++) {
            const float b = bnd[j];
            if (b < lo)
                base++;
            else if (b <= hi && inside == __builtin_huge_valf())
                inside = b;
        }
        float base_bits;
        std::memcpy(&base_bits, &base, sizeof base_bits);
        lut[i] = make_float2(inside * bscale, base_bits);
    }
}

template <int D, int B0, int B1, bool S2>
void launch_encode_mfma_k(const EncodeMfmaParams &q, hipStream_t st)
{
    auto kern = encode_mfma_kernel<D, B0, B1, S2>;
    // 256 rows per workgroup and side, every group of the first side first
    const int64_t per_side = (q.n_rows + 255) / 256;
    const int64_t blocks = per_side * (B1 > 0 ? 2 : 1);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kBlock), 0, st, q);
}

// sides ordered so that side[0] has the larger width (B0 >= B1; B1 = 0: one side)
template <int D, bool S2>
void launch_encode_mfma_d(const EncodeMfmaParams &q, int b0, int b1, hipStream_t st)
{
    switch (b0 * 10 + b1) {
    case 40: launch_encode_mfma_k<D, 4, 0, S2>(q, st); break;
    case 30: launch_encode_mfma_k<D, 3, 0, S2>(q, st); break;
    case 20: launch_encode_mfma_k<D, 2, 0, S2>(q, st); break;
    case 44: launch_encode_mfma_k<D, 4, 4, S2>(q, st); break;
    case 43: launch_encode_mfma_k<D, 4, 3, S2>(q, st); break;
    case 42: launch_encode_mfma_k<D, 4, 2, S2>(q, st); break;
    case 33: launch_encode_mfma_k<D, 3, 3, S2>(q, st); break;
    case 32: launch_encode_mfma_k<D, 3, 2, S2>(q, st); break;
    default: launch_encode_mfma_k<D, 2, 2, S2>(q, st); break;
    }
}

template <typename T, bool PAD>
void launch_encode_pad(int d, const EncodeParams &p, int sides, hipStream_t st)
{
    dim3 block(kBlock);
    switch (d) {
    case 64: hipLaunchKernelGGL((encode_kernel<64, T, PAD>), dim3(grid_for(p.n_rows, Shape<64>::RPB), sides), block, 0, st, p); break;
    case 128: hipLaunchKernelGGL((encode_kernel<128, T, PAD>), dim3(grid_for(p.n_rows, Shape<128>::RPB), sides), block, 0, st, p); break;
    default: hipLaunchKernelGGL((encode_kernel<256, T, PAD>), dim3(grid_for(p.n_rows, Shape<256>::RPB), sides), block, 0, st, p); break;
    }
}

// rows of exactly d values take coalesced loads; padded ones per-lane loads
template <typename T>
void launch_encode(int d, const EncodeParams &p, int sides, hipStream_t st)
{
    if (p.d_in == d)
        launch_encode_pad<T, false>(d, p, sides, st);
    else
        launch_encode_pad<T, true>(d, p, sides, st);
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

template <int D, bool PAD>
void launch_decode_d(int bits, const DecodeParams &p0, hipStream_t st)
{
    launch_all(p0.n_rows, Shape<D>::RPW, [&](dim3 grid, int64_t first) {
        DecodeParams p = p0;
        p.row_base = first;
        const dim3 block(kDecodeBlock);
        switch (bits) {
        case 2: hipLaunchKernelGGL((decode_kernel<D, 2, PAD>), grid, block, 0, st, p); break;
        case 3: hipLaunchKernelGGL((decode_kernel<D, 3, PAD>), grid, block, 0, st, p); break;
        default: hipLaunchKernelGGL((decode_kernel<D, 4, PAD>), grid, block, 0, st, p); break;
        }
    });
}

// grid.y holds at most 65535 (sequence, head) pairs per launch
constexpr int64_t kMaxGridY = 65535;

template <int D, bool PAD>
void launch_cache_decode_d(int bits, int nseg, int64_t n_bh, const CacheDecodeParams &p0,
                           hipStream_t st)
{
    const unsigned gx = (unsigned)((p0.count + Shape<D>::RPW - 1) / Shape<D>::RPW);
    for (int64_t b0 = 0; b0 < n_bh; b0 += kMaxGridY) {
        CacheDecodeParams p = p0;
        p.bh_base = (int)b0;
        const dim3 grid(gx, (unsigned)std::min<int64_t>(kMaxGridY, n_bh - b0), (unsigned)nseg);
        const dim3 block(kDecodeBlock);
        switch (bits) {
        case 2: hipLaunchKernelGGL((cache_decode_kernel<D, 2, PAD>), grid, block, 0, st, p); break;
        case 3: hipLaunchKernelGGL((cache_decode_kernel<D, 3, PAD>), grid, block, 0, st, p); break;
        default: hipLaunchKernelGGL((cache_decode_kernel<D, 4, PAD>), grid, block, 0, st, p); break;
        }
    }
}

template <typename T>
void launch_rotate(int d, const RotateParams &p0, hipStream_t st)
{
    const int rpb = d == 64 ? Shape<64>::RPB : d == 128 ? Shape<128>::RPB : Shape<256>::RPB;
    launch_all(p0.n_rows, rpb, [&](dim3 grid, int64_t first) {
        RotateParams p = p0;
        p.row_base = first;
        switch (d) {
        case 64: hipLaunchKernelGGL((rotate_kernel<64, T>), grid, dim3(kBlock), 0, st, p); break;
        case 128: hipLaunchKernelGGL((rotate_kernel<128, T>), grid, dim3(kBlock), 0, st, p); break;
        default: hipLaunchKernelGGL((rotate_kernel<256, T>), grid, dim3(kBlock), 0, st, p); break;
        }
    });
}

}  // namespace

// ------------------------------------------------------------ C entry points

extern "C" int tq_rotate(const void *in, int dtype, int64_t n_rows, int d, uint64_t seed,
                         uint32_t flags, int inverse, float *out, void *stream)
{
    static const char *fn = "tq_rotate";
    tq::clear_error();
    if (dtype != TQ_F32 && dtype != TQ_BF16)
        return tq::fail(TQ_EINVAL, "tq_rotate: unknown dtype");
    if (n_rows < 0)
        return tq::fail(TQ_EINVAL, "tq_rotate: n_rows < 0");
    int rc = tq::check_flags(flags, fn);
    if (rc != TQ_OK)
        return rc;
    if ((rc = check_d(d, fn, false)) != TQ_OK)
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
    tq::sign_words2(d, seed, flags, p.signs2);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == TQ_F32)
        launch_rotate<float>(d, p, st);
    else
        launch_rotate<uint16_t>(d, p, st);
    return launch_status(fn);
}

extern "C" int tq_encode(const void *k_rows, const void *v_rows, int dtype, int64_t n_rows,
                         int d, int bits_k, int bits_v, uint64_t seed, uint32_t flags,
                         uint8_t *k_packed, float *k_norms, uint8_t *v_packed, float *v_norms,
                         void *stream)
{
    static const char *fn = "tq_encode";
    tq::clear_error();
    if (dtype != TQ_F32 && dtype != TQ_BF16)
        return tq::fail(TQ_EINVAL, "tq_encode: unknown dtype");
    if (n_rows < 0)
        return tq::fail(TQ_EINVAL, "tq_encode: n_rows < 0");
    int rc = tq::check_flags(flags, fn);
    if (rc != TQ_OK)
        return rc;
    if ((rc = check_d(d, fn)) != TQ_OK)
        return rc;
    const int D = tq::padded_dim(d);  // rotated and stored length
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
        if ((rc = code_table(D, bits[s], tq::density_of(flags), &e.code, fn)) != TQ_OK)
            return rc;
    }
    if ((rc = injected(fn)) != TQ_OK)
        return rc;
    p.n_rows = n_rows;
    p.d_in = d;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == TQ_BF16 && d == D) {
        // bf16 rows of exactly 64, 128 or 256 values: the matrix-core encode
        EncodeMfmaParams q;
        q.side[0] = p.side[0];
        q.side[1] = p.side[1];
        if (sides == 2 && q.side[1].code.bits > q.side[0].code.bits) {
            q.side[0] = p.side[1];
            q.side[1] = p.side[0];
        }
        const int b0 = q.side[0].code.bits, b1 = sides == 2 ? q.side[1].code.bits : 0;
        if (sides == 1)
            q.side[1] = q.side[0];  // unused
        q.n_rows = n_rows;
        for (int w = 0; w < 8; w++)
            q.s1.w[w] = q.s2.w[w] = 0u;
        tq::sign_words(d, seed, q.s1.w);
        tq::sign_words2(d, seed, flags, q.s2.w);
        // one side's table travels with the arguments (the first side with
        // more than two bits); the other side, if it needs one, builds it
        q.lut_side = b0 > 2 ? 0 : b1 > 2 ? 1 : -1;
        if (q.lut_side >= 0) {
            const CodeTable &c = q.side[q.lut_side].code;
            host_lut(c.bnd, (1 << c.bits) - 1, kLutScale, q.lut);
        }
        const bool two = (flags & TQ_FLAG_TWO_SIDED) != 0;
        switch (d) {
        case 64:
            two ? launch_encode_mfma_d<64, true>(q, b0, b1, st)
                : launch_encode_mfma_d<64, false>(q, b0, b1, st);
            break;
        case 128:
            two ? launch_encode_mfma_d<128, true>(q, b0, b1, st)
                : launch_encode_mfma_d<128, false>(q, b0, b1, st);
            break;
        default:
            two ? launch_encode_mfma_d<256, true>(q, b0, b1, st)
                : launch_encode_mfma_d<256, false>(q, b0, b1, st);
            break;
        }
        return launch_status(fn);
    }
    tq::sign_words(D, seed, p.signs);
    tq::sign_words2(D, seed, flags, p.signs2);
    if (dtype == TQ_F32)
        launch_encode<float>(D, p, sides, st);
    else
        launch_encode<uint16_t>(D, p, sides, st);
    return launch_status(fn);
}

extern "C" int tq_decode(const uint8_t *packed, const float *norms, int64_t n_rows, int d,
                         int bits, uint64_t seed, uint32_t flags, float *out, void *stream)
{
    static const char *fn = "tq_decode";
    tq::clear_error();
    if (n_rows < 0)
        return tq::fail(TQ_EINVAL, "tq_decode: n_rows < 0");
    int rc = tq::check_flags(flags, fn);
    if (rc != TQ_OK)
        return rc;
    if ((rc = check_d(d, fn)) != TQ_OK)
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
    const int D = tq::padded_dim(d);  // rotated and stored length
    tq_codebook cb;
    if ((rc = decode_codebook(D, bits, flags, &cb, fn)) != TQ_OK)
        return rc;
    DecodeParams p;
    p.packed = packed;
    p.norms = norms;
    p.out = out;
    p.n_rows = n_rows;
    fill_decode_tables(cb, d, D, bits, seed, flags, &p.t);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool pad = d != D;
    switch (D) {
    case 64: launch_decode_d<64, false>(bits, p, st); break;
    case 128:
        pad ? launch_decode_d<128, true>(bits, p, st) : launch_decode_d<128, false>(bits, p, st);
        break;
    default:
        pad ? launch_decode_d<256, true>(bits, p, st) : launch_decode_d<256, false>(bits, p, st);
        break;
    }
    return launch_status(fn);
}

extern "C" int tq_cache_decode(const tq_cache_desc *c, int layer, int64_t start,
                               int64_t count, float *const *k_out, float *const *v_out,
                               void *stream)
{
    static const char *fn = "tq_cache_decode";
    tq::clear_error();
    if (!c)
        return tq::fail(TQ_EINVAL, "tq_cache_decode: cache is NULL");
    if (c->n_layers < 1 || c->n_layers > TQ_MAX_LAYERS || c->batch < 0 || c->n_kv_heads < 0 ||
        c->window < 1 || !c->head_dim || !c->k_packed || !c->k_norms || !c->v_packed ||
        !c->v_norms)
        return tq::fail(TQ_EINVAL, "tq_cache_decode: invalid cache descriptor");
    if (layer < -1 || layer >= c->n_layers)
        return tq::fail(TQ_EINVAL, "tq_cache_decode: layer out of range");
    if (start < 0 || count < 0 || start + count > c->window)
        return tq::fail(TQ_EINVAL, "tq_cache_decode: slots [start, start + count) must lie in "
                                   "[0, window)");
    if (tq::check_flags(c->flags, fn) != TQ_OK)
        return TQ_EINVAL;
    int rc;
    const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->n_layers : layer + 1;
    // the (layer, side) buffers to decode: side 0 = K, 1 = V
    struct Seg {
        int layer, side, d, D, bits;
        const uint8_t *packed;
        const float *norms;
        float *out;
    };
    std::vector<Seg> segs;
    for (int l = l0; l < l1; l++) {
        if ((rc = check_d(c->head_dim[l], fn)) != TQ_OK)
            return rc;
        for (int side = 0; side < 2; side++) {
            float *const *outs = side == 0 ? k_out : v_out;
            float *o = outs ? outs[l - l0] : nullptr;
            if (!o)
                continue;  // side or layer not requested
            const int bits = tq::layer_bits(c, l, side);
            if ((rc = check_bits(bits, fn)) != TQ_OK)
                return rc;
            const uint8_t *pk = side == 0 ? c->k_packed[l] : c->v_packed[l];
            const float *nm = side == 0 ? c->k_norms[l] : c->v_norms[l];
            if (!pk || !nm)
                return tq::fail(TQ_EINVAL, "tq_cache_decode: NULL layer buffer");
            if (!aligned(pk, 16) || !aligned(o, 16) || !aligned(nm, 4))
                return tq::fail(TQ_EINVAL, "tq_cache_decode: misaligned buffer (packed and out "
                                           "need 16 bytes, norms 4)");
            const int d = c->head_dim[l];
            segs.push_back({l, side, d, tq::padded_dim(d), bits, pk, nm, o});
        }
    }
    const int64_t n_bh = (int64_t)c->batch * c->n_kv_heads;
    if (n_bh == 0 || count == 0 || segs.empty())
        return TQ_OK;
    if ((rc = injected(fn)) != TQ_OK)
        return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // one launch per distinct (head_dim, bits) and per kMaxDecodeSegs buffers
    // of it, in the order of their first buffers
    std::vector<bool> done(segs.size(), false);
    for (size_t first = 0; first < segs.size(); first++) {
        if (done[first])
            continue;
        const Seg &f = segs[first];
        tq_codebook cb;
        if ((rc = decode_codebook(f.D, f.bits, c->flags, &cb, fn)) != TQ_OK)
            return rc;
        CacheDecodeParams p;
        fill_decode_tables(cb, f.d, f.D, f.bits, c->seed, c->flags, &p.t);
        p.window = c->window;
        p.start = (int)start;
        p.count = (int)count;
        p.bh_base = 0;
        int n = 0;
        for (size_t i = first; i <= segs.size(); i++) {
            const bool flush = i == segs.size() || n == kMaxDecodeSegs;
            if (flush && n > 0) {
                const bool pad = f.d != f.D;
                switch (f.D) {
                case 64: launch_cache_decode_d<64, false>(f.bits, n, n_bh, p, st); break;
                case 128:
                    pad ? launch_cache_decode_d<128, true>(f.bits, n, n_bh, p, st)
                        : launch_cache_decode_d<128, false>(f.bits, n, n_bh, p, st);
                    break;
                default:
                    pad ? launch_cache_decode_d<256, true>(f.bits, n, n_bh, p, st)
                        : launch_cache_decode_d<256, false>(f.bits, n, n_bh, p, st);
                    break;
                }
                if ((rc = launch_status(fn)) != TQ_OK)
                    return rc;
                n = 0;
            }
            if (i == segs.size())
                break;
            if (done[i] || segs[i].d != f.d || segs[i].bits != f.bits)
                continue;
            done[i] = true;
            p.packed[n] = segs[i].packed;
            p.norms[n] = segs[i].norms;
            p.out[n] = segs[i].out;
            n++;
        }
    }
    return TQ_OK;
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
    if (tq::check_flags(c->flags, fn) != TQ_OK)
        return TQ_EINVAL;
    if (!k_new || !v_new)
        return tq::fail(TQ_EINVAL, "tq_append_row: k_new / v_new is NULL");
    int rc;
    const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->n_layers : layer + 1;
    for (int l = l0; l < l1; l++) {
        const int i = l - l0;
        if ((rc = check_d(c->head_dim[l], fn)) != TQ_OK)
            return rc;
        if ((rc = check_bits(tq::layer_bits(c, l, 0), fn)) != TQ_OK ||
            (rc = check_bits(tq::layer_bits(c, l, 1), fn)) != TQ_OK)
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
    // one launch per distinct (head_dim, K width, V width), in the order of
    // their first layers, and per kMaxAppendLayers layers of it
    auto same = [&](int a, int b) {
        return c->head_dim[a] == c->head_dim[b] &&
               tq::layer_bits(c, a, 0) == tq::layer_bits(c, b, 0) &&
               tq::layer_bits(c, a, 1) == tq::layer_bits(c, b, 1);
    };
    for (int first = l0; first < l1; first++) {
        bool seen = false;
        for (int l = l0; l < first && !seen; l++)
            seen = same(l, first);
        if (seen)
            continue;
        const int d = c->head_dim[first], D = tq::padded_dim(d);
        const int bk = tq::layer_bits(c, first, 0), bv = tq::layer_bits(c, first, 1);
        AppendParams p;
        p.bh = bh;
        p.window = c->window;
        p.slot = slot;
        p.d_in = d;
        tq::sign_words(D, c->seed, p.signs);
        tq::sign_words2(D, c->seed, c->flags, p.signs2);
        const int dens = tq::density_of(c->flags);
        if ((rc = code_table(D, bk, dens, &p.side[0].code, fn)) != TQ_OK ||
            (rc = code_table(D, bv, dens, &p.side[1].code, fn)) != TQ_OK)
            return rc;
        p.n_layers = 0;
        for (int l = l0; l <= l1; l++) {
            const bool flush = (l == l1) || (p.n_layers == kMaxAppendLayers);
            if (flush && p.n_layers > 0) {
                if (dtype == TQ_F32)
                    launch_append<float>(D, p, 2, st);
                else
                    launch_append<uint16_t>(D, p, 2, st);
                if ((rc = launch_status(fn)) != TQ_OK)
                    return rc;
                p.n_layers = 0;
            }
            if (l == l1)
                break;
            if (!same(l, first))
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
