// Host half of libtq.so: errors, codebooks, signs and sizes.
//
// Codebook ([Foundry] = "TurboQuant KV Cache Compression — Spec", sections
// "Step 2: Lloyd-Max Scalar Quantization" and "Codebook Generation"): the
// Lloyd-Max quantiser of the coordinate density, found by Lloyd's iteration
// (boundaries at midpoints of neighbouring centroids, centroids at the
// conditional means of their cells) run until it stops moving.
//
// For the Beta(d/2, d/2) density mapped to [-1, 1], f(x) ~ (1 - x^2)^(a-1)
// with a = d/2, each cell [lo, hi] needs
//   P = I_{(1+hi)/2}(a, a) - I_{(1+lo)/2}(a, a)      (regularised incomplete
//       beta, evaluated by its continued fraction with the modified Lentz
//       method; DLMF 8.17.22)
//   M = integral x f = ((1-lo^2)^a - (1-hi^2)^a) / (2a * 2^(2a-1) B(a, a))
// and the centroid is M / P.  For N(0, 1/d) the same quantities come from
// erfc and the normal density.  The iteration runs on the positive half; the
// negative half is its mirror image, so the table is exactly symmetric and
// the middle boundary is exactly 0.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "tq_internal.h"

namespace tq {

static thread_local std::string g_last_error;

int fail(int status, const std::string &msg)
{
    g_last_error = msg;
    return status;
}

void clear_error() { g_last_error.clear(); }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

bool take_injected_launch_failure()
{
    static std::mutex mu;
    static int state = -1;  // -1 unread, 0 off, 1 armed
    std::lock_guard<std::mutex> lk(mu);
    if (state < 0) {
        const char *e = std::getenv("TQ_TEST_FAIL_LAUNCH");
        state = (e && std::strcmp(e, "1") == 0) ? 1 : 0;
    }
    if (state == 1) {
        state = 0;
        return true;
    }
    return false;
}

// ---------------------------------------------------------------- signs

static inline uint64_t splitmix64_next(uint64_t &s)
{
    s += 0x9E3779B97F4A7C15ULL;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

void sign_words(int d, uint64_t seed, uint32_t *words)
{
    int nw = (d + 31) / 32;
    for (int w = 0; w < nw; w++)
        words[w] = 0;
    uint64_t s = seed;
    for (int i = 0; i < d; i++)
        if (splitmix64_next(s) >> 63)
            words[i / 32] |= 1u << (i % 32);
}

void sign_words2(int d, uint64_t seed, uint32_t flags, uint32_t *words)
{
    int nw = (d + 31) / 32;
    for (int w = 0; w < nw; w++)
        words[w] = 0;
    if (!(flags & TQ_FLAG_TWO_SIDED))
        return;
    uint64_t s = seed;
    for (int i = 0; i < d; i++)
        (void)splitmix64_next(s);
    for (int i = 0; i < d; i++)
        if (splitmix64_next(s) >> 63)
            words[i / 32] |= 1u << (i % 32);
}

int check_flags(uint32_t flags, const char *fn)
{
    if (flags & ~(TQ_FLAG_GAUSS_1_OVER_D | TQ_FLAG_TWO_SIDED))
        return fail(TQ_EINVAL, std::string(fn) + ": unknown flag bits");
    return TQ_OK;
}

// ------------------------------------------------------------- codebook

// Continued fraction of I_x(a, b) (valid for x < (a+1)/(a+b+2)).
static double betacf(double a, double b, double x)
{
    const double tiny = 1e-300, eps = 1e-16;
    double qab = a + b, qap = a + 1.0, qam = a - 1.0;
    double c = 1.0, dd = 1.0 - qab * x / qap;
    if (std::fabs(dd) < tiny)
        dd = tiny;
    dd = 1.0 / dd;
    double h = dd;
    for (int m = 1; m < 100000; m++) {
        double m2 = 2.0 * m;
        double num = m * (b - m) * x / ((qam + m2) * (a + m2));
        dd = 1.0 + num * dd;
        if (std::fabs(dd) < tiny)
            dd = tiny;
        c = 1.0 + num / c;
        if (std::fabs(c) < tiny)
            c = tiny;
        dd = 1.0 / dd;
        h *= dd * c;
        num = -(a + m) * (qab + m) * x / ((a + m2) * (qap + m2));
        dd = 1.0 + num * dd;
        if (std::fabs(dd) < tiny)
            dd = tiny;
        c = 1.0 + num / c;
        if (std::fabs(c) < tiny)
            c = tiny;
        dd = 1.0 / dd;
        double del = dd * c;
        h *= del;
        if (std::fabs(del - 1.0) < eps)
            break;
    }
    return h;
}

// Regularised incomplete beta I_x(a, a) for the symmetric case.
static double ibeta_sym(double a, double x)
{
    if (x <= 0.0)
        return 0.0;
    if (x >= 1.0)
        return 1.0;
    if (x == 0.5)
        return 0.5;
    double lnpre = a * std::log(x) + a * std::log1p(-x) -
                   (2.0 * std::lgamma(a) - std::lgamma(2.0 * a));
    if (x < 0.5)
        return std::exp(lnpre) * betacf(a, a, x) / a;
    return 1.0 - std::exp(lnpre) * betacf(a, a, 1.0 - x) / a;
}

struct CellMoments {
    double p;  // probability of the cell
    double m;  // integral of x over the cell (first moment)
};

// Beta(d/2, d/2) on [-1, 1]; 0 <= lo < hi <= 1.
static CellMoments beta_cell(double a, double lo, double hi)
{
    CellMoments r;
    r.p = ibeta_sym(a, 0.5 * (1.0 + hi)) - ibeta_sym(a, 0.5 * (1.0 + lo));
    // ln(2a * 2^(2a-1) * B(a, a))
    double lnC = std::log(2.0 * a) + (2.0 * a - 1.0) * std::log(2.0) +
                 2.0 * std::lgamma(a) - std::lgamma(2.0 * a);
    double t_lo = a * std::log1p(-lo * lo) - lnC;
    double t_hi = hi >= 1.0 ? -INFINITY : a * std::log1p(-hi * hi) - lnC;
    r.m = std::exp(t_lo) - std::exp(t_hi);
    return r;
}

// N(0, s^2); 0 <= lo < hi (hi may be +inf).
static CellMoments gauss_cell(double s, double lo, double hi)
{
    CellMoments r;
    const double r2 = 0.70710678118654752440, rpi2 = 0.39894228040143267794;
    double zl = lo / s, zh = hi / s;
    r.p = 0.5 * (std::erfc(zl * r2) - (std::isinf(zh) ? 0.0 : std::erfc(zh * r2)));
    r.m = s * rpi2 * (std::exp(-0.5 * zl * zl) - (std::isinf(zh) ? 0.0 : std::exp(-0.5 * zh * zh)));
    return r;
}

static int build_codebook(int d, int bits, int density, tq_codebook *cb)
{
    const int L = 1 << bits, h = L / 2;
    const double a = 0.5 * d;
    // spread of the density, used only to place the starting centroids
    const double spread = density == TQ_BETA_HALF_D ? 1.0 / std::sqrt(d + 1.0)
                                                    : 1.0 / std::sqrt((double)d);
    const double top = density == TQ_BETA_HALF_D ? 1.0 : INFINITY;
    double c[8], b[8];
    // start: positive centroids at the midpoints of h equal slices of
    // [0, min(2.5 * spread, 0.9 * top)]
    double span = std::fmin(2.5 * spread, 0.9 * (std::isinf(top) ? 1e300 : top));
    for (int j = 0; j < h; j++)
        c[j] = span * (j + 0.5) / h;
    double distortion_sum = 0.0;
    int it = 0;
    // Stop when no centroid moved by more than 1e-13 of the density's spread
    // (the map's own rounding noise is about 1e-14 relative).
    for (; it < 200000; it++) {
        for (int j = 0; j + 1 < h; j++)
            b[j] = 0.5 * (c[j] + c[j + 1]);
        double move = 0.0;
        distortion_sum = 0.0;
        for (int j = 0; j < h; j++) {
            double lo = j == 0 ? 0.0 : b[j - 1];
            double hi = j == h - 1 ? top : b[j];
            CellMoments cm = density == TQ_BETA_HALF_D ? beta_cell(a, lo, hi)
                                                       : gauss_cell(spread, lo, hi);
            if (!(cm.p > 0.0))
                return fail(TQ_EINVAL, "codebook: empty cell during Lloyd iteration");
            double cn = cm.m / cm.p;
            move = std::fmax(move, std::fabs(cn - c[j]));
            c[j] = cn;
            distortion_sum += cm.p * cn * cn;
        }
        if (move <= 1e-13 * spread)
            break;
    }
    for (int j = 0; j + 1 < h; j++)
        b[j] = 0.5 * (c[j] + c[j + 1]);
    std::memset(cb, 0, sizeof(*cb));
    cb->d = d;
    cb->bits = bits;
    cb->levels = L;
    cb->density = density;
    for (int j = 0; j < h; j++) {
        cb->centroids[h + j] = (float)c[j];
        cb->centroids[h - 1 - j] = (float)-c[j];
    }
    cb->boundaries[h - 1] = 0.0f;
    for (int j = 0; j + 1 < h; j++) {
        cb->boundaries[h + j] = (float)b[j];
        cb->boundaries[h - 2 - j] = (float)-b[j];
    }
    // E[(X - Q(X))^2] = E[X^2] - sum_j P_j c_j^2 for conditional-mean
    // centroids; the half-line sum counts each mirrored cell once.
    double ex2 = density == TQ_BETA_HALF_D ? 1.0 / (d + 1.0) : 1.0 / d;
    cb->distortion_per_coord = ex2 - 2.0 * distortion_sum;
    return TQ_OK;
}

int get_codebook(int d, int bits, int density, tq_codebook *out)
{
    static std::mutex mu;
    static std::map<std::tuple<int, int, int>, tq_codebook> memo;
    auto key = std::make_tuple(d, bits, density);
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = memo.find(key);
        if (it != memo.end()) {
            *out = it->second;
            return TQ_OK;
        }
    }
    tq_codebook cb;
    int rc = build_codebook(d, bits, density, &cb);
    if (rc != TQ_OK)
        return rc;
    std::lock_guard<std::mutex> lk(mu);
    memo[key] = cb;
    *out = cb;
    return TQ_OK;
}

}  // namespace tq

// ------------------------------------------------------------- C entry points

extern "C" const char *tq_last_error(void) { return tq::g_last_error.c_str(); }

extern "C" const char *tq_version(void) { return "tq 0.1.0 gfx950"; }

extern "C" int tq_codebook_init_density(int d, int bits, int density, tq_codebook *out)
{
    tq::clear_error();
    if (!out)
        return tq::fail(TQ_EINVAL, "tq_codebook_init: out is NULL");
    if (d < 2 || d > (1 << 20) || !tq::is_pow2(d))
        return tq::fail(TQ_EINVAL, "tq_codebook_init: d must be a power of two in [2, 2^20]");
    if (bits < 1 || bits > 4)
        return tq::fail(TQ_EINVAL, "tq_codebook_init: bits must be in 1..4");
    if (density != TQ_BETA_HALF_D && density != TQ_GAUSS_1_OVER_D)
        return tq::fail(TQ_EINVAL, "tq_codebook_init: unknown density");
    return tq::get_codebook(d, bits, density, out);
}

extern "C" int tq_codebook_init(int d, int bits, tq_codebook *out)
{
    return tq_codebook_init_density(d, bits, TQ_BETA_HALF_D, out);
}

extern "C" int tq_signs(int d, uint64_t seed, int8_t *out_pm1)
{
    tq::clear_error();
    if (!out_pm1)
        return tq::fail(TQ_EINVAL, "tq_signs: out is NULL");
    if (d < 1 || d > (1 << 20))
        return tq::fail(TQ_EINVAL, "tq_signs: d must be in [1, 2^20]");
    uint64_t s = seed;
    for (int i = 0; i < d; i++)
        out_pm1[i] = (tq::splitmix64_next(s) >> 63) ? (int8_t)-1 : (int8_t)1;
    return TQ_OK;
}

namespace tq {
int padded_dim(int d)
{
    if (d < 2 || d > (1 << 20))
        return 0;
    int p = 1;
    while (p < d)
        p *= 2;
    return p;
}
}  // namespace tq

extern "C" size_t tq_packed_row_bytes(int d, int bits)
{
    const int dp = d == 1 ? 1 : tq::padded_dim(d);
    if (dp == 0 || bits < 1 || bits > 8)
        return 0;
    return ((size_t)dp * (size_t)bits + 7) / 8;
}

extern "C" int tq_layer_bits_boundary(int n_layers, int n_boundary, int bits_inner,
                                      int bits_boundary, int32_t *out)
{
    tq::clear_error();
    if (n_layers < 1 || n_layers > TQ_MAX_LAYERS)
        return tq::fail(TQ_EINVAL, "tq_layer_bits_boundary: n_layers outside 1..TQ_MAX_LAYERS");
    if (bits_inner < 1 || bits_inner > 4 || bits_boundary < 1 || bits_boundary > 4)
        return tq::fail(TQ_EINVAL, "tq_layer_bits_boundary: bits must be in 1..4");
    if (!out)
        return tq::fail(TQ_EINVAL, "tq_layer_bits_boundary: out is NULL");
    const int nb = n_boundary < 0 ? 2 : n_boundary;  // the page's "auto"
    for (int l = 0; l < n_layers; l++)
        out[l] = (l < nb || l >= n_layers - nb) ? bits_boundary : bits_inner;
    return TQ_OK;
}
