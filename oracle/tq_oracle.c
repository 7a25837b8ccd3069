/*
 * Plain, slow, fp64 CPU oracle for the TurboQuant KV-cache codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this file's library.  It shares no source, header,
 * table or constant with the GPU library, and neither includes the other.
 *
 * Pages followed (cited by title and section):
 *   [Engine]   "TurboQuantEngine — Specification" (larql)
 *   [Foundry]  "TurboQuant KV Cache Compression — Spec" (Foundry attention)
 *   [Atlas]    "CITATIONS" (atlas, TurboQuant+ integration notes)
 *   [KVC]      "Implementation specification: TurboAngle and TurboQuant-style
 *               KV compression" (kvcompress)
 *
 * What each function follows:
 *   orc_signs      [Foundry] "Step 1: Random Orthogonal Rotation" (one +-1
 *                  diagonal generated once from a seed); the generator is
 *                  SplitMix64 (Steele, Lea & Flood 2014), sign = top bit.
 *   orc_fwht       [Foundry] "Hadamard Transform Detail" (unnormalised
 *                  Sylvester butterfly, log2 d stages).
 *   orc_rotate     [Foundry] "As-Built Notes" item 1 (signs before the
 *                  Hadamard: y = H (D x) / sqrt(d)); [KVC] "TurboAngle
 *                  reference path" steps 1-2 (D then orthonormal H).
 *                  Optional second sign vector after the Hadamard: [Atlas]
 *                  "Two-sided Rademacher signs in WHT" (orc_signs2).
 *   orc_codebook   [Foundry] "Step 2: Lloyd-Max Scalar Quantization" and
 *                  "Codebook Generation" (Lloyd iteration on Beta(d/2, d/2)
 *                  mapped to [-1, 1]); [Atlas] "Prior art" item 4 for the
 *                  N(0, 1/d) alternative.
 *   orc_pack       [Foundry] "Step 3: Packing" (LSB-first; dense 3-bit, the
 *                  "8 values into 3 bytes" alternative).
 *   orc_padded_dim [Foundry] "Hadamard Transform Detail" (a head_dim that is
 *                  not a power of two is padded to the next one).
 *   orc_encode     [Foundry] "As-Built Notes" item 2 (L2-norm normalisation),
 *                  [Engine] "2.2 Memory contract" (fp32 norm + packed indices
 *                  per head).
 *   orc_decode     [Foundry] "Step 2" (centroid lookup) and "Hadamard
 *                  Transform Detail" (inverse = signs after H).
 *   orc_attention  [Foundry] "Attention with TurboQuant cache" (dequantise,
 *                  then standard attention) -- the plain definition.
 *   orc_attention_rotated
 *                  [Foundry] "Optimization: Fused dequant-dot" (q rotated
 *                  once, dots and V-sum in the rotated domain, one inverse
 *                  rotation) -- used only to check that identity.
 *
 * Readings where the pages are silent or disagree are listed in the design
 * notes of the repository; the ones that change arithmetic are restated at
 * the function that takes them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MAX_LEVELS 16

/* ------------------------------------------------------------------ */
/* Signs                                                               */
/* ------------------------------------------------------------------ */

/* SplitMix64: state advances by the golden-ratio increment, output is the
 * state passed through the two xor-shift-multiply mixing rounds. */
static uint64_t orc_splitmix64(uint64_t *state)
{
    uint64_t z;
    *state += 0x9E3779B97F4A7C15ULL;
    z = *state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* First n raw SplitMix64 outputs for a seed (exposed for the generator pin). */
void orc_splitmix64_stream(uint64_t seed, int n, uint64_t *out)
{
    uint64_t st = seed;
    for (int i = 0; i < n; i++)
        out[i] = orc_splitmix64(&st);
}

/* Reading: sign i is -1 when the top bit of output i is set, else +1.  One
 * vector per (seed, d); a smaller d takes a prefix of the same stream. */
void orc_signs(uint64_t seed, int d, int8_t *out)
{
    uint64_t st = seed;
    for (int i = 0; i < d; i++) {
        uint64_t r = orc_splitmix64(&st);
        out[i] = (r >> 63) ? (int8_t)-1 : (int8_t)1;
    }
}

/* Two-sided rotation ([Atlas] "Two-sided Rademacher signs in WHT": one sign
 * vector before the butterfly and another after it).  The page does not
 * print the two vectors; reading: s1 is the one-sided vector above (outputs
 * 0..d-1) and s2 takes the next d outputs of the same stream (d..2d-1). */
void orc_signs2(uint64_t seed, int d, int8_t *s1, int8_t *s2)
{
    int8_t *all = (int8_t *)malloc((size_t)2 * d);
    orc_signs(seed, 2 * d, all);
    memcpy(s1, all, (size_t)d);
    memcpy(s2, all + d, (size_t)d);
    free(all);
}

/* The sign vectors a codec call uses: s always, s2 only when two_sided
 * (else *s2 = NULL).  Both are malloc'd; free with free(). */
static void orc_rotation_signs(uint64_t seed, int d, int two_sided, int8_t **s,
                               int8_t **s2)
{
    *s = (int8_t *)malloc((size_t)d);
    *s2 = NULL;
    if (two_sided) {
        *s2 = (int8_t *)malloc((size_t)d);
        orc_signs2(seed, d, *s, *s2);
    } else {
        orc_signs(seed, d, *s);
    }
}

/* ------------------------------------------------------------------ */
/* Rotation                                                            */
/* ------------------------------------------------------------------ */

/* Unnormalised Sylvester Walsh-Hadamard transform, in place: at each stage
 * of half-width h, every pair (i, i+h) inside a block of 2h becomes
 * (a+b, a-b).  d must be a power of two. */
void orc_fwht(double *x, int d)
{
    for (int h = 1; h < d; h *= 2) {
        for (int blk = 0; blk < d; blk += 2 * h) {
            for (int i = blk; i < blk + h; i++) {
                double a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
        }
    }
}

/* Forward rotation y = H (s .* x) / sqrt(d), and with a second sign vector
 * s2 (not NULL) y = s2 .* H (s .* x) / sqrt(d). */
void orc_rotate(const double *x, int d, const int8_t *s, const int8_t *s2,
                double *y)
{
    double inv = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; i++)
        y[i] = (double)s[i] * x[i];
    orc_fwht(y, d);
    for (int i = 0; i < d; i++)
        y[i] *= inv;
    if (s2)
        for (int i = 0; i < d; i++)
            y[i] *= (double)s2[i];
}

/* Inverse rotation x = s .* (H y) / sqrt(d): H/sqrt(d) is symmetric and
 * orthogonal, so it is its own inverse, and D is its own inverse; the order
 * is the reverse of the forward one.  With s2: x = s .* H (s2 .* y) / sqrt(d). */
void orc_unrotate(const double *y, int d, const int8_t *s, const int8_t *s2,
                  double *x)
{
    double inv = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; i++)
        x[i] = s2 ? (double)s2[i] * y[i] : y[i];
    orc_fwht(x, d);
    for (int i = 0; i < d; i++)
        x[i] = (double)s[i] * x[i] * inv;
}

/* ------------------------------------------------------------------ */
/* Packing                                                             */
/* ------------------------------------------------------------------ */

/* Index i occupies bits [i*bits, (i+1)*bits) of a little-endian bitstream:
 * bit k of the stream is bit (k mod 8) of byte k/8.  Reading of the pages'
 * packing table: the first value sits in the low bits; 3-bit is dense. */
void orc_pack(const uint8_t *idx, int n, int bits, uint8_t *out)
{
    int nbytes = (n * bits + 7) / 8;
    memset(out, 0, (size_t)nbytes);
    for (int i = 0; i < n; i++) {
        for (int b = 0; b < bits; b++) {
            int k = i * bits + b;
            if ((idx[i] >> b) & 1)
                out[k / 8] |= (uint8_t)(1u << (k % 8));
        }
    }
}

void orc_unpack(const uint8_t *in, int n, int bits, uint8_t *idx)
{
    for (int i = 0; i < n; i++) {
        unsigned v = 0;
        for (int b = 0; b < bits; b++) {
            int k = i * bits + b;
            v |= (unsigned)((in[k / 8] >> (k % 8)) & 1) << b;
        }
        idx[i] = (uint8_t)v;
    }
}

/* ------------------------------------------------------------------ */
/* Lloyd-Max codebook                                                  */
/* ------------------------------------------------------------------ */

/* Densities of a rotated, norm-divided coordinate.
 *   ORC_BETA : Beta(d/2, d/2) mapped from [0, 1] to [-1, 1], i.e.
 *              f(x) ~ (1 - x^2)^(d/2 - 1)                    ([Foundry] Step 2)
 *   ORC_GAUSS: N(0, 1/d)                                      ([Atlas] item 4)
 * Both are symmetric, so the quantiser is computed on the positive half and
 * mirrored; the middle boundary is exactly 0 and c[j] = -c[L-1-j] exactly. */
enum { ORC_BETA = 0, ORC_GAUSS = 1 };

/* Gauss-Legendre rule on [-1, 1], nodes by Newton's method on P_n. */
#define GL_N 20
static double gl_x[GL_N], gl_w[GL_N];
static int gl_ready = 0;

static void gl_init(void)
{
    if (gl_ready)
        return;
    const double pi = 3.14159265358979323846;
    for (int i = 0; i < GL_N; i++) {
        double z = cos(pi * (i + 0.75) / (GL_N + 0.5));
        double dp = 0.0;
        for (int it = 0; it < 100; it++) {
            double p0 = 1.0, p1 = z;
            for (int k = 2; k <= GL_N; k++) {
                double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
                p0 = p1;
                p1 = p2;
            }
            /* p1 = P_n(z), p0 = P_{n-1}(z) */
            dp = GL_N * (z * p1 - p0) / (z * z - 1.0);
            double dz = p1 / dp;
            z -= dz;
            if (fabs(dz) < 1e-16)
                break;
        }
        gl_x[i] = z;
        gl_w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
    gl_ready = 1;
}

/* Beta density in z = x / sigma units, sigma = 1/sqrt(d+1), up to a constant:
 * g(z) = (1 - sigma^2 z^2)^(expo), expo = d/2 - 1 for the codebook density
 * and (d-3)/2 for the exact marginal of a uniform point on the sphere. */
typedef struct {
    double sigma;  /* scale from x to z */
    double expo;   /* exponent of (1 - x^2) */
    double zmax;   /* end of the support in z units (or a cut-off) */
} orc_beta_z;

static double beta_z_logg(const orc_beta_z *p, double z)
{
    double t = p->sigma * z;
    if (p->expo == 0.0)
        return 0.0;
    return p->expo * log1p(-t * t);
}

/* integrals of g, z g and z^2 g over [lo, hi] (composite Gauss-Legendre,
 * pieces no wider than 0.25 in z) */
static void beta_z_moments(const orc_beta_z *p, double lo, double hi,
                           double *m0, double *m1, double *m2)
{
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
    if (hi > p->zmax)
        hi = p->zmax;
    if (lo < -p->zmax)
        lo = -p->zmax;
    if (hi > lo) {
        int pieces = (int)ceil((hi - lo) / 0.25);
        if (pieces < 1)
            pieces = 1;
        double w = (hi - lo) / pieces;
        for (int k = 0; k < pieces; k++) {
            double a = lo + k * w, mid = a + 0.5 * w;
            for (int i = 0; i < GL_N; i++) {
                double z = mid + 0.5 * w * gl_x[i];
                double g = exp(beta_z_logg(p, z)) * 0.5 * w * gl_w[i];
                s0 += g;
                s1 += z * g;
                s2 += z * z * g;
            }
        }
    }
    *m0 = s0;
    *m1 = s1;
    *m2 = s2;
}

static orc_beta_z beta_z_codebook_density(int d)
{
    orc_beta_z p;
    p.sigma = 1.0 / sqrt((double)d + 1.0);
    p.expo = 0.5 * d - 1.0;
    /* beyond |z| = 40 the density is below exp(-790) relative to its peak
     * for every d >= 4; for small d the support ends first */
    p.zmax = 1.0 / p.sigma;
    if (p.zmax > 40.0)
        p.zmax = 40.0;
    return p;
}

/* Standard normal cell moments by the closed forms
 * P = Phi(hi) - Phi(lo), E[Z 1cell] = phi(lo) - phi(hi). */
static void gauss_moments(double lo, double hi, double *m0, double *m1)
{
    const double rs2 = 0.70710678118654752440;
    const double rs2pi = 0.39894228040143267794;
    *m0 = 0.5 * (erfc(lo * rs2) - erfc(hi * rs2));
    *m1 = rs2pi * (exp(-0.5 * lo * lo) - exp(-0.5 * hi * hi));
}

/* Lloyd iteration on the positive half.  pos_c[0..h-1] are the positive
 * centroids (z units, increasing), pos_b[0..h-2] the positive boundaries
 * between them; the cell of pos_c[0] starts at the middle boundary 0.
 * Reading: initialise at evenly spaced points inside (0, 2) z units (clamped
 * into the support) and iterate until the largest centroid move is below
 * 1e-13 z units, rather than a fixed count of iterations. */
static int lloyd_half(int density, const orc_beta_z *bp, int h, double *pos_c,
                      double *pos_b, int *iters_out)
{
    double zend = density == ORC_BETA ? bp->zmax : 40.0;
    for (int j = 0; j < h; j++) {
        double c = 2.0 * (2.0 * j + 1.0) / (2.0 * h);
        if (c > 0.95 * zend)
            c = 0.95 * zend * (j + 1.0) / (h + 1.0);
        pos_c[j] = c;
    }
    int it;
    for (it = 0; it < 200000; it++) {
        for (int j = 0; j + 1 < h; j++)
            pos_b[j] = 0.5 * (pos_c[j] + pos_c[j + 1]);
        double moved = 0.0;
        for (int j = 0; j < h; j++) {
            double lo = j == 0 ? 0.0 : pos_b[j - 1];
            double hi = j == h - 1 ? zend : pos_b[j];
            double m0, m1, m2;
            if (density == ORC_BETA)
                beta_z_moments(bp, lo, hi, &m0, &m1, &m2);
            else
                gauss_moments(lo, hi, &m0, &m1);
            if (!(m0 > 0.0))
                return -1;
            double c = m1 / m0;
            double dc = fabs(c - pos_c[j]);
            if (dc > moved)
                moved = dc;
            pos_c[j] = c;
        }
        if (moved < 1e-13)
            break;
    }
    for (int j = 0; j + 1 < h; j++)
        pos_b[j] = 0.5 * (pos_c[j] + pos_c[j + 1]);
    if (iters_out)
        *iters_out = it + 1;
    return it < 200000 ? 0 : -2;
}

/* Full codebook in x units (unit-norm coordinates).
 * c[0..L-1] increasing; b[0..L-2] increasing, b[L/2-1] = 0.
 * bits in 1..4, d a power of two >= 2 (for ORC_GAUSS d only sets 1/sqrt(d)).
 * Returns 0, or < 0 on bad arguments / no convergence. */
int orc_codebook(int d, int bits, int density, double *c, double *b, int *iters)
{
    if (bits < 1 || bits > 4 || d < 2 || (d & (d - 1)) != 0)
        return -3;
    if (density != ORC_BETA && density != ORC_GAUSS)
        return -3;
    gl_init();
    int L = 1 << bits, h = L / 2;
    double pc[8], pb[8];
    orc_beta_z bp = beta_z_codebook_density(d);
    int rc = lloyd_half(density, &bp, h, pc, pb, iters);
    if (rc != 0)
        return rc;
    double scale = density == ORC_BETA ? bp.sigma : 1.0 / sqrt((double)d);
    for (int j = 0; j < h; j++) {
        c[h + j] = pc[j] * scale;
        c[h - 1 - j] = -pc[j] * scale;
    }
    b[h - 1] = 0.0;
    for (int j = 0; j + 1 < h; j++) {
        b[h + j] = pb[j] * scale;
        b[h - 2 - j] = -pb[j] * scale;
    }
    return 0;
}

/* Expected squared reconstruction error of a unit vector drawn uniformly
 * from the sphere: d * integral (x - Q(x))^2 f_true(x) dx, where f_true is
 * the exact marginal of one coordinate, ~ (1 - x^2)^((d-3)/2).  Rotation is
 * orthogonal and decode applies its exact inverse, so this is the mean of
 * ||u - c[idx]||^2 over rows.  Requires d >= 8. */
double orc_sphere_mse(int d, int bits, const double *c, const double *b)
{
    gl_init();
    if (d < 8)
        return -1.0;
    int L = 1 << bits;
    orc_beta_z p;
    p.sigma = 1.0 / sqrt((double)d + 1.0);
    p.expo = 0.5 * (d - 3.0);
    p.zmax = 1.0 / p.sigma;
    if (p.zmax > 40.0)
        p.zmax = 40.0;
    double tot0 = 0.0, err = 0.0;
    for (int j = 0; j < L; j++) {
        double lo = j == 0 ? -p.zmax : b[j - 1] / p.sigma;
        double hi = j == L - 1 ? p.zmax : b[j] / p.sigma;
        double m0, m1, m2;
        beta_z_moments(&p, lo, hi, &m0, &m1, &m2);
        double cz = c[j] / p.sigma;
        /* integral (z - cz)^2 g = m2 - 2 cz m1 + cz^2 m0 */
        err += m2 - 2.0 * cz * m1 + cz * cz * m0;
        tot0 += m0;
    }
    return d * p.sigma * p.sigma * err / tot0;
}

/* Memoised float tables (the form the pages' codebook struct stores). */
typedef struct {
    int d, bits, density, ok;
    float cf[ORC_MAX_LEVELS];
    float bf[ORC_MAX_LEVELS - 1];
} orc_cb_entry;
static orc_cb_entry orc_cb_cache[64];
static int orc_cb_count = 0;

static const orc_cb_entry *orc_cb_get(int d, int bits, int density)
{
    for (int i = 0; i < orc_cb_count; i++)
        if (orc_cb_cache[i].d == d && orc_cb_cache[i].bits == bits &&
            orc_cb_cache[i].density == density)
            return &orc_cb_cache[i];
    double c[ORC_MAX_LEVELS], b[ORC_MAX_LEVELS];
    if (orc_codebook(d, bits, density, c, b, NULL) != 0)
        return NULL;
    orc_cb_entry e;
    memset(&e, 0, sizeof e);
    e.d = d;
    e.bits = bits;
    e.density = density;
    e.ok = 1;
    int L = 1 << bits;
    for (int j = 0; j < L; j++)
        e.cf[j] = (float)c[j];
    for (int j = 0; j + 1 < L; j++)
        e.bf[j] = (float)b[j];
    int slot = orc_cb_count < 64 ? orc_cb_count++ : 63;
    orc_cb_cache[slot] = e;
    return &orc_cb_cache[slot];
}

/* float tables as used by encode/decode */
int orc_codebook_float(int d, int bits, int density, float *cf, float *bf)
{
    const orc_cb_entry *e = orc_cb_get(d, bits, density);
    if (!e)
        return -1;
    int L = 1 << bits;
    memcpy(cf, e->cf, sizeof(float) * L);
    memcpy(bf, e->bf, sizeof(float) * (L - 1));
    return 0;
}

/* ------------------------------------------------------------------ */
/* Encode / decode                                                     */
/* ------------------------------------------------------------------ */

/* Length a row is rotated and stored at: d itself when it is a power of two,
 * else the next power of two (reading of [Foundry] Hadamard Transform Detail,
 * which pads a head_dim that is not a power of two and drops the extra
 * coordinates: the padded vector is rotated, quantised and stored whole, and
 * only decode drops coordinates d..d_pad-1, since dropping rotated
 * coordinates would lose information beyond the quantisation).  0 when d is
 * out of range. */
int orc_padded_dim(int d)
{
    if (d < 2 || d > (1 << 20))
        return 0;
    int p = 1;
    while (p < d)
        p *= 2;
    return p;
}

/* Encode rows x[n_rows][d] (fp32 values; bf16 inputs arrive converted
 * exactly).  With dp = orc_padded_dim(d), per row:
 *   x'  = x followed by dp - d zeros
 *   n   = ||x||_2 of the input row, stored as float         (reading: the
 *         norm of the input row, not of the rotated one; equal in exact
 *         arithmetic)
 *   y   = H (s .* x') / sqrt(dp), or s2 .* H (s .* x') / sqrt(dp) when
 *         two_sided ([Atlas] "Two-sided Rademacher signs in WHT"); s, s2 and
 *         the codebook are those of dp
 *   u   = y / n, and u = 0 when n = 0                        (reading)
 *   idx = #{ j : b_j < u }  with b_j the float boundaries    (a u exactly on
 *         a boundary takes the lower cell; reading)
 *   packed = LSB-first bitstream of the dp indices, dp*bits/8 bytes
 *         (dp*bits % 8 == 0 for bits in 2..4 and dp >= 8).
 * u_out, when not NULL, receives u[n_rows][dp] (for boundary-band accounting).
 * Returns 0 or a negative error. */
int orc_encode(const float *x, int64_t n_rows, int d, int bits, int density,
               int two_sided, uint64_t seed, uint8_t *packed, float *norms,
               double *u_out)
{
    const int dp = orc_padded_dim(d);
    if (dp == 0 || bits < 1 || bits > 4 || (dp * bits) % 8 != 0)
        return -3;
    const orc_cb_entry *cb = orc_cb_get(dp, bits, density);
    if (!cb)
        return -1;
    int L = 1 << bits;
    int row_bytes = dp * bits / 8;
    int8_t *s, *s2;
    double *xr = (double *)malloc(sizeof(double) * dp);
    double *y = (double *)malloc(sizeof(double) * dp);
    uint8_t *idx = (uint8_t *)malloc((size_t)dp);
    orc_rotation_signs(seed, dp, two_sided, &s, &s2);
    for (int64_t r = 0; r < n_rows; r++) {
        const float *xrow = x + r * d;
        double ss = 0.0;
        for (int i = 0; i < dp; i++) {
            xr[i] = i < d ? (double)xrow[i] : 0.0;
            ss += xr[i] * xr[i];
        }
        double n = sqrt(ss);
        orc_rotate(xr, dp, s, s2, y);
        for (int i = 0; i < dp; i++) {
            double u = n > 0.0 ? y[i] / n : 0.0;
            if (u_out)
                u_out[r * dp + i] = u;
            int k = 0;
            for (int j = 0; j < L - 1; j++)
                if ((double)cb->bf[j] < u)
                    k++;
            idx[i] = (uint8_t)k;
        }
        orc_pack(idx, dp, bits, packed + r * row_bytes);
        norms[r] = (float)n;
    }
    free(s);
    free(s2);
    free(xr);
    free(y);
    free(idx);
    return 0;
}

/* Decode one row into fp64 at the padded length dp: yhat = n * c[idx],
 * xhat = s .* H yhat / sqrt(dp) (s .* H (s2 .* yhat) / sqrt(dp) with a second
 * sign vector). */
static void orc_decode_row_f64(const uint8_t *packed_row, float norm, int dp,
                               int bits, const orc_cb_entry *cb,
                               const int8_t *s, const int8_t *s2, uint8_t *idx,
                               double *yh, double *out)
{
    orc_unpack(packed_row, dp, bits, idx);
    for (int i = 0; i < dp; i++)
        yh[i] = (double)norm * (double)cb->cf[idx[i]];
    orc_unrotate(yh, dp, s, s2, out);
}

/* Decode rows ([n_rows][dp*bits/8] packed) to [n_rows][d]: the first d of the
 * dp decoded coordinates, in fp64 (out64) or rounded once to float (out32);
 * exactly one of the two is not NULL. */
static int orc_decode_any(const uint8_t *packed, const float *norms,
                          int64_t n_rows, int d, int bits, int density,
                          int two_sided, uint64_t seed, float *out32,
                          double *out64)
{
    const int dp = orc_padded_dim(d);
    if (dp == 0 || bits < 1 || bits > 4 || (dp * bits) % 8 != 0)
        return -3;
    const orc_cb_entry *cb = orc_cb_get(dp, bits, density);
    if (!cb)
        return -1;
    int row_bytes = dp * bits / 8;
    int8_t *s, *s2;
    double *yh = (double *)malloc(sizeof(double) * dp);
    double *xo = (double *)malloc(sizeof(double) * dp);
    uint8_t *idx = (uint8_t *)malloc((size_t)dp);
    orc_rotation_signs(seed, dp, two_sided, &s, &s2);
    for (int64_t r = 0; r < n_rows; r++) {
        orc_decode_row_f64(packed + r * row_bytes, norms[r], dp, bits, cb, s, s2,
                           idx, yh, xo);
        for (int i = 0; i < d; i++) {
            if (out32)
                out32[r * d + i] = (float)xo[i];
            else
                out64[r * d + i] = xo[i];
        }
    }
    free(s);
    free(s2);
    free(yh);
    free(xo);
    free(idx);
    return 0;
}

int orc_decode(const uint8_t *packed, const float *norms, int64_t n_rows, int d,
               int bits, int density, int two_sided, uint64_t seed, float *out)
{
    return orc_decode_any(packed, norms, n_rows, d, bits, density, two_sided,
                          seed, out, NULL);
}

/* Same, but keeps fp64 output (used by the attention definition). */
int orc_decode_f64(const uint8_t *packed, const float *norms, int64_t n_rows,
                   int d, int bits, int density, int two_sided, uint64_t seed,
                   double *out)
{
    return orc_decode_any(packed, norms, n_rows, d, bits, density, two_sided,
                          seed, NULL, out);
}

/* ------------------------------------------------------------------ */
/* Attention                                                           */
/* ------------------------------------------------------------------ */

/* Softmax attention of n_q query heads over T cached rows, plain definition:
 *   khat_t, vhat_t = decode of the stored K, V rows (fp64, not rounded)
 *   score_t = scale * <q, khat_t>,  p = softmax(score) (max subtracted)
 *   o = sum_t p_t vhat_t
 * Query head h reads KV head g = h / (n_q / n_kv) (contiguous groups;
 * reading).  q[n_q][d] are the query values (bf16 inputs arrive converted
 * exactly).  Cache rows are [n_kv][T] with row strides of one packed row
 * (dp*bits/8 bytes, dp = orc_padded_dim(d)); khat, vhat are the d decoded
 * coordinates.
 * sparse_v_threshold > 0 gates the V sum ([Atlas] "Sparse V dequant"): the
 * V row of a position contributes only when its softmax exponent, taken
 * against the softmax's maximum, exceeds the threshold.  Reading: the
 * maximum is that of the whole context (of this query head), so
 *   keep_t = exp(score_t - max_t' score_t') > threshold,
 * i.e. the row's attention weight relative to the largest weight; the
 * running maximum of an online softmax only ever approaches it from below,
 * and this is the one choice that does not depend on the loop order.  Gated
 * rows still count in the softmax denominator (their V is left at zero; the
 * kept weights are not renormalised).  0 disables the gate. */
int orc_attention(const float *q, int n_q, const uint8_t *k_packed,
                  const float *k_norms, const uint8_t *v_packed,
                  const float *v_norms, int n_kv, int T, int d, int bits_k,
                  int bits_v, int density, int two_sided, uint64_t seed,
                  double scale, double sparse_v_threshold, double *out)
{
    if (n_kv <= 0 || n_q % n_kv != 0 || T < 1)
        return -3;
    int G = n_q / n_kv;
    const int dp = orc_padded_dim(d);
    if (dp == 0)
        return -3;
    int kb = dp * bits_k / 8, vb = dp * bits_v / 8;
    double *K = (double *)malloc(sizeof(double) * (size_t)T * d);
    double *V = (double *)malloc(sizeof(double) * (size_t)T * d);
    double *sc = (double *)malloc(sizeof(double) * (size_t)T);
    if (!K || !V || !sc)
        return -1;
    int rc = 0;
    for (int g = 0; g < n_kv && rc == 0; g++) {
        rc = orc_decode_f64(k_packed + (size_t)g * T * kb, k_norms + (size_t)g * T,
                            T, d, bits_k, density, two_sided, seed, K);
        if (rc == 0)
            rc = orc_decode_f64(v_packed + (size_t)g * T * vb,
                                v_norms + (size_t)g * T, T, d, bits_v, density,
                                two_sided, seed, V);
        for (int hh = 0; hh < G && rc == 0; hh++) {
            int h = g * G + hh;
            const float *qh = q + (size_t)h * d;
            double m = -INFINITY;
            for (int t = 0; t < T; t++) {
                double acc = 0.0;
                for (int i = 0; i < d; i++)
                    acc += (double)qh[i] * K[(size_t)t * d + i];
                sc[t] = scale * acc;
                if (sc[t] > m)
                    m = sc[t];
            }
            double denom = 0.0;
            for (int t = 0; t < T; t++) {
                sc[t] = exp(sc[t] - m);
                denom += sc[t];
            }
            double *oh = out + (size_t)h * d;
            for (int i = 0; i < d; i++)
                oh[i] = 0.0;
            for (int t = 0; t < T; t++) {
                double p = sc[t] / denom;
                /* sc holds exp(score - m), m the context's largest score */
                if (sparse_v_threshold > 0.0 && !(sc[t] > sparse_v_threshold))
                    continue;
                for (int i = 0; i < d; i++)
                    oh[i] += p * V[(size_t)t * d + i];
            }
        }
    }
    free(K);
    free(V);
    free(sc);
    return rc;
}

/* The same attention evaluated in the rotated domain at the padded length
 * dp: q' = H (s .* q) / sqrt(dp) (q zero-padded), score_t = scale * n_t
 * <q', c_K[idx_t]>, o' = sum_t p_t n^V_t c_V[idx^V_t], o = the first d of
 * s .* H o' / sqrt(dp) (the rotation and its inverse take the second sign
 * vector when two_sided).  Equal to orc_attention up to rounding: the padded
 * coordinates of q are zero, so <q', c_K> only sees the first d coordinates of
 * the decoded key. */
int orc_attention_rotated(const float *q, int n_q, const uint8_t *k_packed,
                          const float *k_norms, const uint8_t *v_packed,
                          const float *v_norms, int n_kv, int T, int d,
                          int bits_k, int bits_v, int density, int two_sided,
                          uint64_t seed, double scale, double *out)
{
    const int dp = orc_padded_dim(d);
    if (n_kv <= 0 || n_q % n_kv != 0 || T < 1 || dp == 0)
        return -3;
    const orc_cb_entry *cbk = orc_cb_get(dp, bits_k, density);
    const orc_cb_entry *cbv = orc_cb_get(dp, bits_v, density);
    if (!cbk || !cbv)
        return -1;
    int G = n_q / n_kv;
    int kb = dp * bits_k / 8, vb = dp * bits_v / 8;
    int8_t *s, *s2;
    double *qd = (double *)malloc(sizeof(double) * dp);
    double *qr = (double *)malloc(sizeof(double) * dp);
    double *orot = (double *)malloc(sizeof(double) * dp);
    double *ofull = (double *)malloc(sizeof(double) * dp);
    double *sc = (double *)malloc(sizeof(double) * (size_t)T);
    uint8_t *idx = (uint8_t *)malloc((size_t)dp);
    orc_rotation_signs(seed, dp, two_sided, &s, &s2);
    for (int h = 0; h < n_q; h++) {
        int g = h / G;
        for (int i = 0; i < dp; i++)
            qd[i] = i < d ? (double)q[(size_t)h * d + i] : 0.0;
        orc_rotate(qd, dp, s, s2, qr);
        double m = -INFINITY;
        for (int t = 0; t < T; t++) {
            size_t row = (size_t)g * T + t;
            orc_unpack(k_packed + row * kb, dp, bits_k, idx);
            double acc = 0.0;
            for (int i = 0; i < dp; i++)
                acc += qr[i] * (double)cbk->cf[idx[i]];
            sc[t] = scale * (double)k_norms[row] * acc;
            if (sc[t] > m)
                m = sc[t];
        }
        double denom = 0.0;
        for (int t = 0; t < T; t++) {
            sc[t] = exp(sc[t] - m);
            denom += sc[t];
        }
        for (int i = 0; i < dp; i++)
            orot[i] = 0.0;
        for (int t = 0; t < T; t++) {
            size_t row = (size_t)g * T + t;
            orc_unpack(v_packed + row * vb, dp, bits_v, idx);
            double w = sc[t] / denom * (double)v_norms[row];
            for (int i = 0; i < dp; i++)
                orot[i] += w * (double)cbv->cf[idx[i]];
        }
        orc_unrotate(orot, dp, s, s2, ofull);
        for (int i = 0; i < d; i++)
            out[(size_t)h * d + i] = ofull[i];
    }
    free(ofull);
    free(s);
    free(s2);
    free(qd);
    free(qr);
    free(orot);
    free(sc);
    free(idx);
    return 0;
}
