// Device arithmetic of the n-gram hash shared by the hash kernel and the fused
// hash-and-gather kernel (engram API page, Qwen3_8_FlashNextNGramEmbedding:
// _hash_input_ids takes the positive remainder of each order's mix by the
// head's modulus).
#pragma once

#include "engram_internal.h"

namespace engram {

// Positive remainder of a signed 64-bit value by p (2 <= p <= 2^62), with
// magic = floor(2^64 / p) (Barrett).  For m < 0, m mod p = p - 1 - ((-m - 1)
// mod p), and -m - 1 = ~m fits in [0, 2^63), so both signs reduce a value
// below 2^63, for which umulhi(v, magic) is floor(v / p) or one less.
__device__ __forceinline__ uint64_t floor_mod(int64_t m, uint64_t p, uint64_t magic) {
    const bool neg = m < 0;
    const uint64_t v = neg ? ~(uint64_t)m : (uint64_t)m;
    const uint64_t q = __umul64hi(v, magic);
    uint64_t r = v - q * p;
    if (r >= p) r -= p;
    return neg ? p - 1 - r : r;
}

}  // namespace engram
