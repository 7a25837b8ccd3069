// Internal declarations shared by the host half (tq_host.cpp) and the device
// half (tq_codec.hip, tq_attn.hip) of libtq.so.  Not installed; not part of the ABI.
#pragma once

#include <cstdint>
#include <string>

#include "../../include/tq.h"

namespace tq {

// Thread-local error reporting: every public entry point returns through
// fail() on error so that tq_last_error() has a message.
int fail(int status, const std::string &msg);
void clear_error();

// Memoised host codebook (validated arguments assumed).
int get_codebook(int d, int bits, int density, tq_codebook *out);

// Sign diagonal of the rotation as a bitmask: bit i of words[i / 32] is set
// when coordinate i is negated.  d <= 256 for device use.
void sign_words(int d, uint64_t seed, uint32_t *words /* d/32 rounded up */);

// The second diagonal of the two-sided rotation (S2: stream outputs d..2d-1),
// same layout; all zero unless `flags` has TQ_FLAG_TWO_SIDED.
void sign_words2(int d, uint64_t seed, uint32_t flags, uint32_t *words);

// Codebook density selected by `flags`.
inline int density_of(uint32_t flags)
{
    return (flags & TQ_FLAG_GAUSS_1_OVER_D) ? TQ_GAUSS_1_OVER_D : TQ_BETA_HALF_D;
}

// TQ_OK, or TQ_EINVAL (with a message naming fn) for unknown option bits.
int check_flags(uint32_t flags, const char *fn);

// Bit width of layer l of a cache, side 0 = K, 1 = V (the per-layer arrays
// when present, else the uniform widths).
inline int layer_bits(const tq_cache_desc *c, int l, int side)
{
    const int32_t *a = side ? c->layer_bits_v : c->layer_bits_k;
    return a ? a[l] : (side ? c->bits_v : c->bits_k);
}

bool is_pow2(int64_t v);

// Length a row of d coordinates is rotated and stored at: d when it is a
// power of two, else the next power of two; 0 when d is outside 2..2^20.
int padded_dim(int d);

// Test-only fault injection: when the environment variable TQ_TEST_FAIL_LAUNCH
// is "1" at the first query, the next device launch reports TQ_EHIP without
// launching anything (one shot), so host tests can reach the HIP error path.
bool take_injected_launch_failure();

}  // namespace tq
