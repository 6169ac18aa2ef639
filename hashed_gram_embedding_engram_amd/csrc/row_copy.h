// The copy half of the row gather, shared by the gather kernel and the fused
// hash-and-gather kernel: one wave moves G consecutive lookups' rows of CPR
// 16-byte chunks (G * CPR = 64 * PER_LANE), each lane PER_LANE chunks with
// dwordx4 loads and non-temporal dwordx4 stores.  Lane i < G holds the local
// row of lookup n0 + i (~0 for a lookup outside the shard, whose output row
// is zero).  Every load is issued unconditionally (a lane with nothing to copy
// reads `zero`), so all PER_LANE loads of the wave are in flight together;
// each load instruction reads 64 consecutive chunks of the wave's rows and
// each store instruction writes 1 KB of consecutive output.
#pragma once

#include "engram_internal.h"

namespace engram {

template <int CPR, int G, bool ROW32, bool NT_LOAD>
__device__ __forceinline__ void copy_wave_rows(const u32x4* __restrict__ table, uint64_t local, int64_t n0, int64_t n,
                                               u32x4* __restrict__ out, int lane, const u32x4* zero) {
    constexpr int PER_LANE = CPR * G / 64;
    static_assert(CPR * G % 64 == 0 && G <= 64, "wave tile must be whole dwordx4 per lane");
    const int rem = (int)(n - n0 < G ? n - n0 : G);
    const u32x4* src[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
        const int c = lane + 64 * j;
        const int i = c / CPR, k = c % CPR;
        if (ROW32) {
            const uint32_t r = __shfl((uint32_t)local, i, 64);
            src[j] = (i < rem && r != 0xFFFFFFFFu) ? table + ((uint64_t)r * CPR + k) : zero;
        } else {
            const uint64_t r = __shfl(local, i, 64);
            src[j] = (i < rem && r != ~0ull) ? table + (r * CPR + k) : zero;
        }
    }
    u32x4 v[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) v[j] = NT_LOAD ? __builtin_nontemporal_load(src[j]) : *src[j];
    u32x4* dst = out + n0 * CPR + lane;
    if (rem == G) {  // every wave but the last: no per-store condition
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j) __builtin_nontemporal_store(v[j], dst + 64 * j);
    } else {
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j)
            if ((lane + 64 * j) / CPR < rem) __builtin_nontemporal_store(v[j], dst + 64 * j);
    }
}

}  // namespace engram
