// Device building blocks shared by the codec and attention kernels (gfx950,
// wave64).
//
// Row layout in registers: a row of D coordinates is held by P = D / 32
// neighbouring lanes of one wavefront, 32 consecutive coordinates per lane
// (lane `sub` of the group holds coordinates [32*sub, 32*sub + 32)).  A wave
// therefore carries 64 / P rows at once: 8 rows of 256, 16 rows of 128 or 32
// rows of 64 coordinates (Shape<D>).  Each lane loads and stores one
// contiguous slice, so global accesses are contiguous per lane and per row.
//
// Walsh-Hadamard transform ("TurboQuant KV Cache Compression — Spec",
// "Hadamard Transform Detail": Sylvester butterflies over log2(d) stages):
// the five stages over coordinate bits 0..4 run inside a lane on registers;
// the stages over bits 5.. pair lane `sub` with lane `sub ^ m` and run with
// DPP quad permutes (m = 1, 2) or ds_swizzle xor (m = 4, 8), never through
// LDS memory.  A butterfly keeps (a + b) in the lower lane and (a - b) in the
// upper lane of the pair, exactly as the in-lane stages do.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tqd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kCPL = 32;          // coordinates per lane
constexpr int kBlock = 256;       // threads per workgroup (4 waves)

// Bucketize table.  u is mapped to bin round(128 u) + 136 by one fma whose
// float result lands in [2^23, 2^24) (unit spacing), so the bin is the low
// bits of the float and the table address is one shift-add of those bits.
// Bin i covers u in [(i - 136.5)/128, (i - 135.5)/128); |u| <= 1 up to
// rounding for every finite row, so bins 0..271 are the ones reached and
// the table has slack bins on both ends.  Entry i holds the number of
// boundaries below its (slightly widened) lower edge and the single boundary
// that may fall inside it, so idx(u) = base + (u > boundary_in_bin).  The
// host checks that boundaries are further apart than a widened bin, so a bin
// never holds two.
constexpr int kLutBins = 280;
constexpr float kLutScale = 128.0f;        // bins per unit of u
constexpr int kLutZero = 136;              // bin of u = 0
constexpr float kLutMagic = 12583048.0f;   // 1.5 * 2^23 + 136
constexpr uint32_t kLutMagicBits = 0x4B400000u;  // bits of 1.5 * 2^23
constexpr float kLutSlack = 1e-5f;         // widening of each bin, in units of u

template <int D>
struct Shape {
    static constexpr int P = D / kCPL;        // lanes per row
    static constexpr int RPW = 64 / P;        // rows per wave
    static constexpr int RPB = RPW * (kBlock / 64);  // rows per workgroup pass
};

// value of lane (lane ^ M) within the wave, for M in {1, 2, 4, 8, 16}
template <int M>
__device__ __forceinline__ float lane_xor(float v)
{
    int x = __float_as_int(v);
    if constexpr (M == 1)
        x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    else if constexpr (M == 2)
        x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    else if constexpr (M == 4)
        x = __builtin_amdgcn_ds_swizzle(x, 0x101F);             // and 0x1f, xor 4
    else if constexpr (M == 8)
        x = __builtin_amdgcn_ds_swizzle(x, 0x201F);             // and 0x1f, xor 8
    else
        x = __builtin_amdgcn_ds_swizzle(x, 0x401F);             // and 0x1f, xor 16
    return __int_as_float(x);
}

// Partner of step M of a butterfly reduction: once steps 1 .. M/2 are done,
// every lane of an aligned group of M lanes holds the same partial, so any
// lane of the neighbouring group will do.  Steps 4 and 8 take the mirrored
// lane of the 8- or 16-lane row (DPP row_half_mirror / row_mirror, a vector
// instruction) instead of lane ^ M (a swizzle through the LDS unit); the
// values, and so the results, are the same.  Not for exchanges that need
// lane ^ M itself (the Hadamard stages).
template <int M>
__device__ __forceinline__ float reduce_partner(float v)
{
    if constexpr (M == 4)
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
    else if constexpr (M == 8)
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
    else
        return lane_xor<M>(v);
}

template <int P>
__device__ __forceinline__ float sum_across(float x)
{
    if constexpr (P > 1) x += reduce_partner<1>(x);
    if constexpr (P > 2) x += reduce_partner<2>(x);
    if constexpr (P > 4) x += reduce_partner<4>(x);
    if constexpr (P > 8) x += reduce_partner<8>(x);
    if constexpr (P > 16) x += reduce_partner<16>(x);
    return x;
}

template <int P>
__device__ __forceinline__ float max_across(float x)
{
    if constexpr (P > 1) x = fmaxf(x, reduce_partner<1>(x));
    if constexpr (P > 2) x = fmaxf(x, reduce_partner<2>(x));
    if constexpr (P > 4) x = fmaxf(x, reduce_partner<4>(x));
    if constexpr (P > 8) x = fmaxf(x, reduce_partner<8>(x));
    if constexpr (P > 16) x = fmaxf(x, reduce_partner<16>(x));
    return x;
}

// in-lane stages (coordinate bits 0..4), unnormalised
__device__ __forceinline__ void fwht_lane(float (&v)[kCPL])
{
#pragma unroll
    for (int h = 1; h < kCPL; h *= 2) {
#pragma unroll
        for (int i = 0; i < kCPL; i++) {
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
}

template <int M>
__device__ __forceinline__ void fwht_cross_stage(float (&v)[kCPL], int sub)
{
    // lower lane of the pair: a + b; upper lane: a - b = partner - own
    const float sg = (sub & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < kCPL; i++)
        v[i] = fmaf(sg, v[i], lane_xor<M>(v[i]));
}

// full unnormalised transform of a row held by P lanes
template <int P>
__device__ __forceinline__ void fwht_row(float (&v)[kCPL], int sub)
{
    fwht_lane(v);
    if constexpr (P > 1) fwht_cross_stage<1>(v, sub);
    if constexpr (P > 2) fwht_cross_stage<2>(v, sub);
    if constexpr (P > 4) fwht_cross_stage<4>(v, sub);
    if constexpr (P > 8) fwht_cross_stage<8>(v, sub);
}

// negate coordinate k when bit k of mask is set (sign diagonal D)
__device__ __forceinline__ void apply_signs(float (&v)[kCPL], uint32_t mask)
{
#pragma unroll
    for (int k = 0; k < kCPL; k++)
        v[k] = __uint_as_float(__float_as_uint(v[k]) ^ ((mask << (31 - k)) & 0x80000000u));
}

// ---------------------------------------------------------------- row I/O

__device__ __forceinline__ void load_slice(const float *p, float (&v)[kCPL])
{
    const f32x4 *q = reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int j = 0; j < kCPL / 4; j++) {
        f32x4 t = __builtin_nontemporal_load(q + j);
        v[4 * j + 0] = t.x;
        v[4 * j + 1] = t.y;
        v[4 * j + 2] = t.z;
        v[4 * j + 3] = t.w;
    }
}

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits
__device__ __forceinline__ void load_slice(const uint16_t *p, float (&v)[kCPL])
{
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int j = 0; j < kCPL / 8; j++) {
        u32x4 t = __builtin_nontemporal_load(q + j);
        uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int m = 0; m < 4; m++) {
            v[8 * j + 2 * m] = __uint_as_float(w[m] << 16);
            v[8 * j + 2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
        }
    }
}

__device__ __forceinline__ void store_slice(float *p, const float (&v)[kCPL])
{
    f32x4 *q = reinterpret_cast<f32x4 *>(p);
#pragma unroll
    for (int j = 0; j < kCPL / 4; j++) {
        f32x4 t = {v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
        __builtin_nontemporal_store(t, q + j);
    }
}

// A wave's P-lane row groups cover 64 * 32 consecutive floats of a row-major
// [rows][D] array (lane l holds floats [32 l, 32 l + 32) of the wave's
// region).  Storing that straight from registers sends 16 bytes to each of 64
// different cache lines per instruction; instead the region is passed through
// a per-wave LDS buffer (rows padded by 4 floats) and written back so that
// each store instruction covers 1 KiB contiguously.  `valid_floats` limits the
// stores to the rows that exist.  Wave-local: no workgroup barrier.
constexpr int kStageStride = kCPL + 4;                 // floats per lane in LDS
constexpr int kStageFloats = 64 * kStageStride;        // per wave

__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void store_region_coalesced(float *region, const float (&v)[kCPL],
                                                       float *stage, int lane,
                                                       int64_t valid_floats)
{
#pragma unroll
    for (int j = 0; j < kCPL / 4; j++) {
        f32x4 t = {v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
        *reinterpret_cast<f32x4 *>(stage + lane * kStageStride + 4 * j) = t;
    }
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < kCPL / 4; j++) {
        const int e = 64 * j + lane;  // float4 index inside the region
        const f32x4 t = *reinterpret_cast<const f32x4 *>(stage + (e >> 3) * kStageStride + 4 * (e & 7));
        if ((int64_t)e * 4 < valid_floats)
            __builtin_nontemporal_store(t, reinterpret_cast<f32x4 *>(region) + e);
    }
    wave_lds_fence();
}

// The same for rows padded to D = P * kCPL of which only the first nv * kCPL
// coordinates are kept: the region holds RPW rows of nv * kCPL floats, built
// from the slices sub < nv of each row.
template <int P>
__device__ __forceinline__ void store_region_padded(float *region, const float (&v)[kCPL],
                                                    float *stage, int lane, int64_t valid_floats,
                                                    int nv)
{
#pragma unroll
    for (int j = 0; j < kCPL / 4; j++) {
        f32x4 t = {v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
        *reinterpret_cast<f32x4 *>(stage + lane * kStageStride + 4 * j) = t;
    }
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < kCPL / 4; j++) {
        const int e = 64 * j + lane;      // float4 index inside the region
        const int q = e >> 3;             // kept slice: row q / nv, slice q % nv
        const int r = q / nv;
        const int src = r * P + (q - r * nv);
        if ((int64_t)e * 4 < valid_floats && q < (64 / P) * nv) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(stage + src * kStageStride + 4 * (e & 7));
            __builtin_nontemporal_store(t, reinterpret_cast<f32x4 *>(region) + e);
        }
    }
    wave_lds_fence();
}

// ------------------------------------------------------------ bit packing
// Index k of a lane's slice occupies bits [k*BITS, (k+1)*BITS) of the lane's
// BITS 32-bit words (little-endian), which is the row's bitstream restricted
// to that slice: the slice starts at bit 32*BITS*sub of the row, a multiple
// of 32.

template <int BITS>
__device__ __forceinline__ void put_index(uint32_t (&w)[BITS], int k, uint32_t idx)
{
    const int bit = k * BITS, word = bit >> 5, off = bit & 31;
    w[word] |= idx << off;
    if (off + BITS > 32)
        w[word + 1] |= idx >> (32 - off);
}

template <int BITS>
__device__ __forceinline__ uint32_t get_index(const uint32_t (&w)[BITS], int k)
{
    const int bit = k * BITS, word = bit >> 5, off = bit & 31;
    uint32_t v = w[word] >> off;
    if (off + BITS > 32)
        v |= w[word + 1] << (32 - off);
    return v & ((1u << BITS) - 1u);
}

template <int BITS>
__device__ __forceinline__ void store_words(uint8_t *p, const uint32_t (&w)[BITS])
{
    if constexpr (BITS == 4) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (BITS == 2) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    } else {
        uint32_t *q = reinterpret_cast<uint32_t *>(p);
#pragma unroll
        for (int j = 0; j < BITS; j++)
            q[j] = w[j];
    }
}

template <int BITS>
__device__ __forceinline__ void load_words(const uint8_t *p, uint32_t (&w)[BITS])
{
    if constexpr (BITS == 4) {
        uint4 t = *reinterpret_cast<const uint4 *>(p);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else if constexpr (BITS == 2) {
        uint2 t = *reinterpret_cast<const uint2 *>(p);
        w[0] = t.x; w[1] = t.y;
    } else {
        const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
        for (int j = 0; j < BITS; j++)
            w[j] = q[j];
    }
}

// ----------------------------------------------------------- bucketize

// LDS byte address of a pointer into LDS
__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Fill the bucketize table from the (levels - 1) boundaries.  Every thread of
// the block takes part; the caller synchronises afterwards.  The stored
// boundary is multiplied by `bscale` (a power of two: 1 for tables looked up
// with u, kLutScale for tables looked up with 128 u).
__device__ __forceinline__ void build_lut(float2 *lut, const float *bnd, int nbnd,
                                          float bscale = 1.0f)
{
    for (int i = threadIdx.x; i < kLutBins; i += blockDim.x) {
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
        lut[i] = make_float2(inside * bscale, __int_as_float(base));
    }
}

// Base for bucketize(): LDS address of the table minus the magic offset.
__device__ __forceinline__ uint32_t lut_key(const float2 *lut)
{
    return lds_address(lut) - (kLutMagicBits << 3);
}

// idx = #{j : b_j < u} for finite |u| <= 1.09
__device__ __forceinline__ uint32_t bucketize(float u, uint32_t key)
{
    const float g = fmaf(u, kLutScale, kLutMagic);
    const uint32_t a = (__float_as_uint(g) << 3) + key;
    const f32x2 e = *reinterpret_cast<const __attribute__((address_space(3))) f32x2 *>(
        (uintptr_t)a);
    return (uint32_t)__float_as_int(e.y) + (u > e.x ? 1u : 0u);
}

// ------------------------------------------------------- signed row loads
// The sign diagonal is applied while loading, as an xor of the sign bits.
// For bf16 one mask per 32-bit word covers two coordinates (bits 15 and 31).

// per-lane xor masks for a lane's 32 coordinates (bit k of `mask` = coord k)
__device__ __forceinline__ void sign_masks_bf16(uint32_t mask, uint32_t (&xm)[kCPL / 2])
{
#pragma unroll
    for (int m = 0; m < kCPL / 2; m++)
        xm[m] = (((mask >> (2 * m)) & 1u) << 15) | (((mask >> (2 * m + 1)) & 1u) << 31);
}

__device__ __forceinline__ void sign_masks_f32(uint32_t mask, uint32_t (&xm)[kCPL])
{
#pragma unroll
    for (int k = 0; k < kCPL; k++)
        xm[k] = ((mask >> k) & 1u) << 31;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// idx_k = base_k + (t_k > b_k) for four outputs.  Each compare writes its own
// scalar register pair, so no compare waits for the previous add (the
// compiler puts every compare in VCC, and a compare's result must be two wait
// states old before an add reads it as carry; here each is at least three).
__device__ __forceinline__ void bucket_add4(const float (&t)[4], const float (&b)[4],
                                            const uint32_t (&base)[4], uint32_t (&idx)[4])
{
    uint64_t m0, m1, m2, m3;
    asm("v_cmp_gt_f32_e64 %4, %8, %12\n\t"
        "v_cmp_gt_f32_e64 %5, %9, %13\n\t"
        "v_cmp_gt_f32_e64 %6, %10, %14\n\t"
        "v_cmp_gt_f32_e64 %7, %11, %15\n\t"
        "v_addc_co_u32_e64 %0, %4, %16, 0, %4\n\t"
        "v_addc_co_u32_e64 %1, %5, %17, 0, %5\n\t"
        "v_addc_co_u32_e64 %2, %6, %18, 0, %6\n\t"
        "v_addc_co_u32_e64 %3, %7, %19, 0, %7"
        : "=&v"(idx[0]), "=&v"(idx[1]), "=&v"(idx[2]), "=v"(idx[3]), "=&s"(m0), "=&s"(m1),
          "=&s"(m2), "=&s"(m3)
        : "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]),
          "v"(b[3]), "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]));
}

// (a << sh) | b and (a << sh) + b as single instructions (the compiler tends
// to split them into a shift and a three-input or/add)
__device__ __forceinline__ uint32_t lshl_or(uint32_t a, uint32_t sh, uint32_t b)
{
    uint32_t r;
    asm("v_lshl_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "i"(sh), "v"(b));
    return r;
}
__device__ __forceinline__ uint32_t lshl_add(uint32_t a, uint32_t sh, uint32_t b)
{
    uint32_t r;
    asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "i"(sh), "v"(b));
    return r;
}

// 2-bit packing step for two outputs: wa += c_a << sa, wb += c_b << sb with
// c = clamp(floor(-t), -2, 1) (three instructions per output; the compiler
// emits floor and convert separately)
__device__ __forceinline__ void pack_c2(float ta, float tb, uint32_t sa, uint32_t sb_, uint32_t &wa,
                                        uint32_t &wb)
{
    uint32_t ca, cb;
    asm("v_cvt_flr_i32_f32_e64 %0, -%4\n\t"
        "v_cvt_flr_i32_f32_e64 %1, -%5\n\t"
        "v_med3_i32 %0, %0, -2, 1\n\t"
        "v_med3_i32 %1, %1, -2, 1\n\t"
        "v_lshl_add_u32 %2, %0, %6, %2\n\t"
        "v_lshl_add_u32 %3, %1, %7, %3"
        : "=&v"(ca), "=&v"(cb), "+v"(wa), "+v"(wb)
        : "v"(ta), "v"(tb), "i"(sa), "i"(sb_));
}

// a[i] for a lane-varying i < N from a uniform array (kernel arguments): a
// select chain on scalar values rather than an indexed load
template <int N>
__device__ __forceinline__ uint32_t pick(const uint32_t *a, int i)
{
    uint32_t v = a[0];
#pragma unroll
    for (int j = 1; j < N; j++)
        v = i == j ? a[j] : v;
    return v;
}

// cache policy of streaming buffer loads: non-temporal
constexpr int kCpolNT = 2;

// A pointer to device memory as a global-address-space pointer (plain global
// loads and stores instead of flat ones).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T *as_global(T *p)
{
    return (__attribute__((address_space(1))) T *)p;
}

// Reinterpret a 32-bit word as two bf16 (taken by value: __builtin_bit_cast
// applied directly to an element of an ext_vector_type value reads element 0
// with this compiler).
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

// Raw slice of one lane (loaded ahead of use to keep loads in flight while
// the previous row is being transformed).
template <typename T>
struct RawSlice;
template <>
struct RawSlice<uint16_t> {
    u32x4 q[kCPL / 8];
};
template <>
struct RawSlice<float> {
    f32x4 q[kCPL / 4];
};

template <typename T>
__device__ __forceinline__ void load_raw(const T *p, RawSlice<T> &r)
{
    using V = typename std::remove_reference<decltype(r.q[0])>::type;
    const V *q = reinterpret_cast<const V *>(p);
#pragma unroll
    for (int j = 0; j < (int)(sizeof(r.q) / sizeof(r.q[0])); j++)
        r.q[j] = __builtin_nontemporal_load(q + j);
}

template <typename T>
__device__ __forceinline__ void zero_raw(RawSlice<T> &r)
{
#pragma unroll
    for (int j = 0; j < (int)(sizeof(r.q) / sizeof(r.q[0])); j++)
        r.q[j] = 0;
}

// bf16 slice -> sign-flipped fp32 values and their sum of squares (the sum
// of squares uses the bf16 dot-product instruction, fp32 accumulate)
__device__ __forceinline__ void convert_signed(const RawSlice<uint16_t> &r,
                                               const uint32_t (&xm)[kCPL / 2],
                                               float (&v)[kCPL], float &ss)
{
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kCPL / 8; j++) {
        const uint32_t w[4] = {r.q[j].x, r.q[j].y, r.q[j].z, r.q[j].w};
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const bf16x2_t h = __builtin_bit_cast(bf16x2_t, w[m]);
            acc = __builtin_amdgcn_fdot2_f32_bf16(h, h, acc, false);
            const uint32_t s = w[m] ^ xm[4 * j + m];
            v[8 * j + 2 * m] = __uint_as_float(s << 16);
            v[8 * j + 2 * m + 1] = __uint_as_float(s & 0xFFFF0000u);
        }
    }
    ss = acc;
}

__device__ __forceinline__ void convert_signed(const RawSlice<float> &r,
                                               const uint32_t (&xm)[kCPL],
                                               float (&v)[kCPL], float &ss)
{
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kCPL / 4; j++) {
        const float x[4] = {r.q[j].x, r.q[j].y, r.q[j].z, r.q[j].w};
#pragma unroll
        for (int m = 0; m < 4; m++) {
            acc = fmaf(x[m], x[m], acc);
            v[4 * j + m] = __uint_as_float(__float_as_uint(x[m]) ^ xm[4 * j + m]);
        }
    }
    ss = acc;
}

template <typename T>
struct SignMasks;
template <>
struct SignMasks<uint16_t> {
    uint32_t xm[kCPL / 2];
    __device__ __forceinline__ explicit SignMasks(uint32_t mask) { sign_masks_bf16(mask, xm); }
};
template <>
struct SignMasks<float> {
    uint32_t xm[kCPL];
    __device__ __forceinline__ explicit SignMasks(uint32_t mask) { sign_masks_f32(mask, xm); }
};

}  // namespace tqd
