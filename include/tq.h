/*
 * tq.h -- C ABI of the TurboQuant KV-cache codec for AMD Instinct MI355X
 * (gfx950).  One shared library, libtq.so; plain pointers and sizes only.
 *
 * Pages this interface follows (cited by title and section):
 *   [Engine]  "TurboQuantEngine — Specification": 2.1 Accuracy contract,
 *             2.2 Memory contract (fp32 norm + ceil(d*bits/8) packed bytes per
 *             head row), 3 Codec, 6 P1 follow-ups (append-only encode of the
 *             new row; compressed-domain attention).
 *   [Foundry] "TurboQuant KV Cache Compression — Spec": Overview, As-Built
 *             Notes (signs before the Hadamard; L2-norm normalisation),
 *             Algorithm Detail steps 1-3, API (init / cache / quantize /
 *             dequantize / attention), Integration Points (circular
 *             addressing pos % max_seq), Hadamard Transform Detail,
 *             Optimization: Fused dequant-dot.
 *   [Atlas]   "CITATIONS" (TurboQuant+ integration notes): Prior art item 4
 *             (N(0, 1/d) codebooks); "Two-sided Rademacher signs in WHT";
 *             "N(0, 1/d) codebook replacement"; "Sparse V dequant";
 *             "LA-V7 boundary-V protection" (first and last layers at higher
 *             precision).
 *   [KVC]     "Implementation specification: TurboAngle and TurboQuant-style
 *             KV compression": Core implementation contract (rows [B, d],
 *             power-of-two d, K and V may use different codecs).
 *
 * Conventions shared by every call
 *   - Return value: TQ_OK (0) or a negative tq_status.  The message of the
 *     last failure on the calling thread is returned by tq_last_error().
 *     Nothing is printed; no C++ exception crosses this boundary.
 *   - Device pointers are HIP device allocations owned by the caller; the
 *     library allocates no device memory and keeps no device state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device calls are asynchronous on that stream and never synchronise;
 *     faults during execution surface at the caller's next synchronisation.
 *   - Row layout: a row is one head vector of d coordinates.  Packed row r of
 *     a buffer starts at byte r * tq_packed_row_bytes(d, bits); index i of a
 *     row occupies bits [i*bits, (i+1)*bits) of the row's little-endian
 *     bitstream (3-bit rows are dense: 8 indices per 3 bytes).
 *   - Alignment: fp32/bf16 row buffers and packed buffers 16-byte aligned;
 *     norm buffers 4-byte aligned.  Misaligned pointers -> TQ_EINVAL.
 *   - Device kernels accept d in {64, 128, 256} and bits in {2, 3, 4};
 *     other valid values return TQ_EUNSUPPORTED.  Codec calls (not
 *     tq_rotate) also accept a d that is a multiple of 32 between 64 and 256
 *     (96, 160, 192, 224): such rows are zero-padded to the next power of two
 *     D, rotated, quantised and stored at length D (D*bits/8 packed bytes,
 *     the signs and codebook of D); decode and attention return the first d
 *     coordinates ([Foundry] Hadamard Transform Detail: pad a head_dim that is
 *     not a power of two).  Row buffers of such d hold d values per row.
 *   - n_rows == 0 (or an empty context) succeeds and launches nothing.
 *   - Non-finite inputs: a row holding an Inf or a NaN encodes as the zero
 *     row (every index L/2 - 1) with a non-finite stored norm (tq_encode,
 *     tq_append_row); decode and attention pass such norms on as IEEE
 *     arithmetic does.  Every access stays inside the buffers described here.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TQ_OK = 0,
    TQ_EINVAL = -1,        /* invalid argument (null, size, alignment, shape) */
    TQ_EUNSUPPORTED = -2,  /* valid, but no device kernel for this case */
    TQ_EHIP = -3           /* the HIP runtime reported an error at launch */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

/* Coordinate density a codebook is optimised for.
 *   TQ_BETA_HALF_D    Beta(d/2, d/2) mapped to [-1, 1]: [Foundry] Step 2.
 *   TQ_GAUSS_1_OVER_D N(0, 1/d): [Atlas] "Prior art" item 4 and "N(0, 1/d)
 *                     codebook replacement".
 * The codec calls below select the density with TQ_FLAG_GAUSS_1_OVER_D. */
typedef enum { TQ_BETA_HALF_D = 0, TQ_GAUSS_1_OVER_D = 1 } tq_density;

/* Option bits (`flags` of tq_rotate / tq_encode / tq_decode and of
 * tq_cache_desc).  0 = the default codec: Beta(d/2, d/2) codebooks and the
 * one-sided rotation H (D x) / sqrt(d).  Other bits -> TQ_EINVAL.
 *   TQ_FLAG_GAUSS_1_OVER_D  codebooks for N(0, 1/d) instead of Beta(d/2, d/2).
 *   TQ_FLAG_TWO_SIDED       rotation S2 H (S1 x) / sqrt(d), inverse
 *                           S1 H (S2 y) / sqrt(d) ([Atlas] "Two-sided
 *                           Rademacher signs in WHT").  S1 is the one-sided
 *                           diagonal (SplitMix64 outputs 0..d-1 of the seed);
 *                           S2 takes outputs d..2d-1 of the same stream, i.e.
 *                           S2 = entries d..2d-1 of tq_signs(2d, seed).
 * Rows encoded with some flags decode correctly only with the same flags. */
#define TQ_FLAG_GAUSS_1_OVER_D 1u
#define TQ_FLAG_TWO_SIDED 2u

/* Lloyd-Max scalar quantiser for one (d, bits, density), in units of a
 * unit-norm coordinate ([Foundry] Step 2's fa_tq_codebook, plus d, density
 * and the expected per-coordinate squared error under the density).
 * centroids[0..levels-1] increase; boundaries[0..levels-2] are midpoints of
 * neighbouring centroids; the table is symmetric and the middle boundary is
 * exactly 0. Unused trailing entries are 0. */
typedef struct {
    int32_t d;
    int32_t bits;
    int32_t levels;
    int32_t density;
    float centroids[16];
    float boundaries[15];
    double distortion_per_coord;
} tq_codebook;

/* Thread-local message of the last failing call on this thread ("" if none). */
const char *tq_last_error(void);

/* Library version string. */
const char *tq_version(void);

/* Host only, synchronous, thread-safe, memoised.  d: power of two in
 * [2, 2^20]; bits: 1..4.  [Foundry] "Codebook Generation": Lloyd iteration
 * (boundaries = midpoints, centroids = conditional means) run to
 * convergence.  TQ_EINVAL on bad d/bits/density or a NULL out. */
int tq_codebook_init(int d, int bits, tq_codebook *out);
int tq_codebook_init_density(int d, int bits, int density, tq_codebook *out);

/* Host only.  The rotation's sign diagonal D ([Foundry] Step 1: generated once
 * from a seed and reused for every row, head and layer): out_pm1[i] = -1 when
 * the top bit of the i-th SplitMix64 output for `seed` is set, else +1.
 * d in [1, 2^20]. */
int tq_signs(int d, uint64_t seed, int8_t *out_pm1);

/* Bytes of one packed row: D * bits / 8 rounded up ([Engine] 2.2), D = d
 * for a power of two and the next power of two otherwise (the padded length
 * rows are stored at).  0 when d <= 0, d > 2^20 or bits outside 1..8. */
size_t tq_packed_row_bytes(int d, int bits);

/* Rotation only, for checking the transform on the device.
 * Forward (inverse == 0): out = H (D x) / sqrt(d)   ([Foundry] As-Built 1).
 * Inverse (inverse != 0): out = D (H x) / sqrt(d)    ([Foundry] Hadamard
 * Transform Detail: H/sqrt(d) and D are each their own inverse).
 * With TQ_FLAG_TWO_SIDED: S2 H (S1 x) / sqrt(d) and S1 H (S2 x) / sqrt(d);
 * TQ_FLAG_GAUSS_1_OVER_D has no effect here.
 * in: [n_rows][d] of `dtype` (device); out: [n_rows][d] fp32 (device). */
int tq_rotate(const void *in, int dtype, int64_t n_rows, int d, uint64_t seed,
              uint32_t flags, int inverse, float *out, void *stream);

/* Encode K and/or V rows ([Foundry] Steps 1-3 with As-Built 2; [KVC] K and V
 * may use different bit widths).  Per row x: n = ||x||_2 (fp32, stored),
 * u = H (D x) / (sqrt(d) n) (u = 0 when n = 0), idx_i = #{j : b_j < u_i}
 * against the (d, bits) boundaries, indices bit-packed.
 * k_rows / v_rows: [n_rows][d] of `dtype` (device); either side may be NULL
 * (its outputs are then ignored) but not both.
 * k_packed: [n_rows][d*bits_k/8], k_norms: [n_rows] (device, written).
 * Same for v_*.  One kernel launch covers both sides.  `flags` selects the
 * codebook density and the rotation (TQ_FLAG_*; u then uses S2 H S1). */
int tq_encode(const void *k_rows, const void *v_rows, int dtype, int64_t n_rows,
              int d, int bits_k, int bits_v, uint64_t seed, uint32_t flags,
              uint8_t *k_packed, float *k_norms, uint8_t *v_packed, float *v_norms,
              void *stream);

/* Decode ([Foundry] Step 2 lookup, then the inverse rotation):
 * out = D H (n * c[idx]) / sqrt(d), fp32 [n_rows][d] (device); with
 * TQ_FLAG_TWO_SIDED out = S1 H (S2 n c[idx]) / sqrt(d).  `flags` must be the
 * ones the rows were encoded with.
 * packed: [n_rows][d*bits/8], norms: [n_rows] (device, read). */
int tq_decode(const uint8_t *packed, const float *norms, int64_t n_rows, int d,
              int bits, uint64_t seed, uint32_t flags, float *out, void *stream);

/* ---------------------------------------------------------------------- */
/* Ring-buffer KV cache ([Foundry] API "Cache" and Integration Points:
 * per-head [n_kv_heads, max_seq, head_dim] layout, slot = pos % window).
 * The descriptor is a host struct; every buffer it points to is a caller-
 * owned device allocation.  Layer l holds, for K and for V,
 *   packed [batch][n_kv_heads][window][head_dim[l] * bits / 8] bytes
 *   norms  [batch][n_kv_heads][window] floats,
 * with bits the layer's K or V width (layer_bits_k[l] / layer_bits_v[l], or
 * bits_k / bits_v for every layer when those arrays are NULL).               */
#define TQ_MAX_LAYERS 256

typedef struct {
    int32_t n_layers;         /* 1..TQ_MAX_LAYERS */
    int32_t batch;            /* sequences */
    int32_t n_kv_heads;
    int32_t window;           /* ring slots per (sequence, head) */
    int32_t bits_k, bits_v;
    uint64_t seed;            /* sign seed shared by K, V and q */
    uint32_t flags;           /* TQ_FLAG_* for every layer, K and V */
    const int32_t *head_dim;  /* host array [n_layers] */
    uint8_t *const *k_packed; /* host array [n_layers] of device pointers */
    float *const *k_norms;
    uint8_t *const *v_packed;
    float *const *v_norms;
    /* Per-layer bit widths, host arrays [n_layers] in 2..4, or NULL for
     * bits_k / bits_v on every layer ([Atlas] "LA-V7 boundary-V protection":
     * boundary layers at a higher precision; [KVC] K and V codecs chosen per
     * layer).  See tq_layer_bits_boundary. */
    const int32_t *layer_bits_k;
    const int32_t *layer_bits_v;
} tq_cache_desc;

/* Host only.  The boundary-layer policy of [Atlas] "LA-V7 boundary-V
 * protection" as bit widths: out[l] = bits_boundary for the first and the
 * last n_boundary layers, bits_inner for the others (n_boundary < 0 selects
 * the page's default of 2).  out: host array [n_layers].  TQ_EINVAL when
 * n_layers is outside 1..TQ_MAX_LAYERS, a width is outside 1..4 or out is
 * NULL. */
int tq_layer_bits_boundary(int n_layers, int n_boundary, int bits_inner,
                           int bits_boundary, int32_t *out);

/* Append-only encode of the new K and V rows ([Engine] 6, W3: encode only the
 * new row) into slot pos % window ([Foundry] Integration Points).
 * layer = -1 appends to every layer (one launch per distinct (head_dim,
 * K width, V width));
 * otherwise only that layer.  k_new / v_new are host arrays of device
 * pointers with n_layers entries (layer = -1) or 1 entry; entry i points to
 * [batch][n_kv_heads][head_dim] rows of `dtype`.  pos >= 0. */
int tq_append_row(const tq_cache_desc *cache, int layer, const void *const *k_new,
                  const void *const *v_new, int dtype, int64_t pos, void *stream);

/* Decode ring slots [start, start + count) of every (sequence, KV head) of a
 * layer back to fp32 ([Foundry] API "Quantize / Dequantize": dequantize a
 * range of cached positions of a layer; Performance Budget: the full-window
 * dequantize).  layer = -1 decodes every layer; otherwise only that layer.
 * k_out / v_out are host arrays of device pointers with n_layers entries
 * (layer = -1) or 1 entry; entry i receives [batch][n_kv_heads][count]
 * [head_dim] floats, the rows tq_decode gives for the same packed rows.  A
 * NULL array skips that side, a NULL entry that (layer, side).  One launch
 * covers up to 64 (layer, side) buffers of the same (head_dim, bits).
 * 0 <= start, 0 <= count, start + count <= window, else TQ_EINVAL; count = 0
 * decodes nothing.  Slots hold whatever was last written there (zero rows
 * where nothing was). */
int tq_cache_decode(const tq_cache_desc *cache, int layer, int64_t start, int64_t count,
                    float *const *k_out, float *const *v_out, void *stream);

/* Workspace bytes tq_attn_decode needs for this (cache, layer, n_q_heads,
 * ctx_len, sparse_v_threshold): the chunk records of the split over the
 * context and, with the sparse-V gate on (threshold > 0), also every context
 * row's scores (4 bytes per row and query head) and the chunk maxima.  0 on
 * invalid arguments. */
size_t tq_attn_workspace_bytes(const tq_cache_desc *cache, int layer,
                               int n_q_heads, int64_t ctx_len,
                               float sparse_v_threshold);

/* Decode-step attention over the compressed cache of one layer, in the
 * rotated domain ([Foundry] Optimization: Fused dequant-dot; [Engine] 6
 * "Compressed-domain attention"): q' = H (D q) / sqrt(d) once per head;
 * score_t = scale * n_t <q', c_K[idx_t]>; softmax over t; o' = sum_t p_t
 * n^V_t c_V[idx^V_t]; out = D H o' / sqrt(d).  Equal, up to rounding, to
 * softmax attention over the decoded rows.  The cache's flags select the
 * codebooks and the rotation (S2 H S1 q and S1 H S2 o' when two-sided); the
 * layer's K and V widths come from the descriptor.
 * q_bf16: [batch][n_q_heads][d] bf16 (device).  Query head h reads KV head
 * h / (n_q_heads / n_kv_heads); n_q_heads must be a multiple of n_kv_heads
 * with a ratio of 1, 2, 4 or 8.  Context = slots [0, min(ctx_len, window)).
 * scale <= 0 selects 1/sqrt(d).  out: [batch][n_q_heads][d] fp32 (device).
 * sparse_v_threshold in [0, 1): 0 disables the gate; otherwise the V row of
 * slot t contributes only where exp(score_t - m) > sparse_v_threshold, m the
 * largest score of the whole context of the same query head, i.e. where the
 * row's weight relative to the largest weight exceeds the threshold ([Atlas]
 * "Sparse V dequant": V of rows whose softmax exponent against the maximum
 * is below the threshold is neither loaded nor decoded).  Gated rows stay in
 * the softmax denominator.  The gated path first scores the whole context
 * (K only), then reads V for the kept rows.  Invalid (negative, >= 1 or NaN)
 * -> TQ_EINVAL.
 * workspace: device buffer of at least tq_attn_workspace_bytes(...) bytes,
 * 16-byte aligned; its contents need no initialisation.  ctx_len >= 1.
 * window * head_dim / 2 (one KV head's packed rows at 4 bits, padded
 * head_dim) must stay below 2^31, else TQ_EUNSUPPORTED. */
int tq_attn_decode(const tq_cache_desc *cache, int layer, const uint16_t *q_bf16,
                   int n_q_heads, int64_t ctx_len, float scale, float sparse_v_threshold,
                   float *out, void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * attention as tq_attn_decode -- same kernels, same results -- with the
 * library's own static device scratch in place of the caller's workspace.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the caller still passes q, out and the cache.
 * Scratch: one file-scope device array of TQ_ATTN_NOALLOC_MAX_BYTES per GPU,
 * held from the library's load on that GPU until the process ends.  A call
 * whose tq_attn_workspace_bytes(...) exceeds it returns TQ_EINVAL (the
 * ungated path needs B * n_q_heads * n_chunks * (D + 4) * 4 bytes, about
 * 1 MiB at batch 32 x 32 query heads; the sparse-V gate adds 4 bytes per
 * context row and query head).  Every call on a GPU shares that GPU's
 * scratch, which keeps the last call's contents (the kernels need no
 * initialisation): calls that overlap on one GPU (several streams or host
 * threads without ordering between them) race.  Arguments and errors
 * otherwise as tq_attn_decode; the first call on a device also looks up the
 * scratch's address there (TQ_EHIP if the runtime fails). */
#define TQ_ATTN_NOALLOC_MAX_BYTES (16u << 20)

int tq_attn_decode_noalloc(const tq_cache_desc *cache, int layer, const uint16_t *q_bf16,
                           int n_q_heads, int64_t ctx_len, float scale,
                           float sparse_v_threshold, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
