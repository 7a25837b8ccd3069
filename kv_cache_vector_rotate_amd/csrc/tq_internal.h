// Internal declarations shared by the host half (tq_host.cpp) and the device
// half (tq_kernels.hip) of libtq.so.  Not installed; not part of the ABI.
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

bool is_pow2(int64_t v);

// Test-only fault injection: when the environment variable TQ_TEST_FAIL_LAUNCH
// is "1" at the first query, the next device launch reports TQ_EHIP without
// launching anything (one shot), so host tests can reach the HIP error path.
bool take_injected_launch_failure();

}  // namespace tq
