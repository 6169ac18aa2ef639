// Stable LSD radix sort of (32-bit key, 32-bit index) pairs for gfx950: the
// pieces shared by the backward's sort by row (scatter.hip) and the routing
// sort by owner (route.hip).  Included by both; everything is internal.
//
// A tile of kTile pairs is owned by one 256-thread block, each wave owning a
// contiguous span of 64 * kItems pairs.  Per 8-bit digit pass:
//   histogram   per-tile digit counts (per-wave LDS atomics, then summed),
//               stored per tile and added into the totals of the tile's
//               chunk and group (see DigitCounts);
//   downsweep   finds where each of its digits starts from those counts,
//               ranks every key among the equal digits before it in its wave
//               span with ballots (no atomics, hence stable), orders the tile
//               by digit in LDS and writes each digit's run to its global slot.
// A pass's histogram usually comes from the kernel that wrote its keys.
#pragma once

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kBlock = 256;                       // threads per block, 4 waves
constexpr int kItems = 16;                        // keys per thread in a sort tile
constexpr int kTile = kBlock * kItems;            // 4096 keys per sort tile
constexpr int kWaveSpan = 64 * kItems;            // contiguous keys owned by one wave
constexpr int kRadix = 256;

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Lanes of the wave whose 8-bit digit equals this lane's, among lanes with `live`.
// Per bit: the lanes whose bit matches this lane's are ~(ballot ^ rep), rep
// being this lane's bit spread over a word; keeping them is one three-input
// bitwise instruction per half of the mask.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool live) {
    const uint64_t l = __ballot(live);
    uint32_t lo = (uint32_t)l, hi = (uint32_t)(l >> 32);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int32_t srep = (int32_t)(d << (31 - b)) >> 31;  // one signed bit-field extract
        const uint32_t rep = (uint32_t)srep;
        const uint64_t bb = __ballot(srep < 0);
        // a & ~(b ^ c): truth table 0x90 with a, b, c as index bits 2, 1, 0
        lo = __builtin_amdgcn_bitop3_b32(lo, (uint32_t)bb, rep, 0x90);
        hi = __builtin_amdgcn_bitop3_b32(hi, (uint32_t)(bb >> 32), rep, 0x90);
    }
    return (uint64_t)hi << 32 | lo;
}

// Exclusive prefix sum over the 256 threads of a block; *total gets the sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total, uint32_t* s_tmp) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    uint32_t wave_off = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) {
        const uint32_t t = s_tmp[k];
        if (k < w) wave_off += t;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return wave_off + x - v;
}

__device__ __forceinline__ void report_bad(int64_t* status, int64_t idx) {
    if (status) atomicMin((unsigned long long*)status, (unsigned long long)idx);
}

// Where a tile's keys of digit d go, without a scan kernel between the
// histogram and the scatter.  Tiles form chunks of 2^chunk_shift tiles and
// chunks form groups of 2^group_shift chunks (each level about the cube root
// of the tile count).  The histogram kernel stores each tile's count per
// digit and adds it into the totals of its chunk and of its group (sums of
// counts: the order of the atomic adds does not matter).  Tile t's digit-d
// keys then start after
//   every key of a smaller digit (the digit totals, scanned over digits),
//   the digit-d keys of the groups before t's group,
//   those of the chunks before t's chunk inside its group, and
//   those of the tiles before t inside its chunk.
// All three arrays hold the 256 digits of one tile (chunk, group)
// contiguously, so a block reads one count per thread per entry in one
// coalesced load.
struct DigitCounts {
    uint32_t* hist;    // [num_tiles][kRadix]
    uint32_t* chunk;   // [num_chunks][kRadix], zero before the histogram kernel
    uint32_t* group;   // [num_groups][kRadix], zero before the histogram kernel
    uint32_t num_groups, chunk_shift, group_shift;
};

struct CountShape {
    int64_t num_chunks, num_groups;
    uint32_t chunk_shift, group_shift;
};
inline CountShape count_shape(int64_t num_tiles) {
    uint32_t lg = 0;
    while (((int64_t)1 << lg) < num_tiles) ++lg;
    CountShape c;
    c.chunk_shift = lg / 3;
    c.group_shift = lg / 3;
    c.num_chunks = (num_tiles + ((int64_t)1 << c.chunk_shift) - 1) >> c.chunk_shift;
    c.num_groups = (c.num_chunks + ((int64_t)1 << c.group_shift) - 1) >> c.group_shift;
    return c;
}
// Words of chunk and group totals for one pass.
inline size_t count_words(int64_t num_tiles) {
    const CountShape c = count_shape(num_tiles);
    return (size_t)kRadix * (size_t)(c.num_chunks + c.num_groups);
}
// `totals` holds count_words(num_tiles) words: the chunk totals, then the group totals.
inline DigitCounts make_digit_counts(void* hist, uint32_t* totals, int64_t num_tiles) {
    const CountShape c = count_shape(num_tiles);
    return DigitCounts{(uint32_t*)hist, totals, totals + (size_t)kRadix * (size_t)c.num_chunks,
                       (uint32_t)c.num_groups, c.chunk_shift, c.group_shift};
}

__device__ __forceinline__ void publish_tile_counts(const DigitCounts& dc, uint32_t tile, int d, uint32_t c) {
    dc.hist[(size_t)tile * kRadix + d] = c;
    if (c) {
        const uint32_t chunk = tile >> dc.chunk_shift;
        atomicAdd(&dc.chunk[(size_t)chunk * kRadix + d], c);
        atomicAdd(&dc.group[(size_t)(chunk >> dc.group_shift) * kRadix + d], c);
    }
}

// The counts that place thread d's digit for one tile: the digit's total over
// all tiles and its keys in the tiles before this one.  With at most
// kCapTiles tiles per chunk, kCapChunks chunks per group and kCapGroups
// groups (up to 2^22 keys), every count is loaded at once by clamped,
// unguarded loads issued before the tile's keys, so both sets of loads are in
// flight together; larger sorts sum them in loops.
constexpr uint32_t kCapTiles = 8, kCapChunks = 8, kCapGroups = 16;
struct TileCounts {
    uint32_t tile[kCapTiles];     // this chunk's tiles (clamped)
    uint32_t chunk[kCapChunks];   // this group's chunks (clamped)
    uint32_t group[kCapGroups];   // all groups (clamped)
};

inline bool small_counts(const DigitCounts& dc) {
    return (1u << dc.chunk_shift) <= kCapTiles && (1u << dc.group_shift) <= kCapChunks && dc.num_groups <= kCapGroups;
}

template <bool SMALL>
__device__ __forceinline__ void load_tile_counts(const DigitCounts& dc, uint32_t tile, int d, TileCounts& tc) {
    if (!SMALL) return;
    const uint32_t chunk = tile >> dc.chunk_shift, group = chunk >> dc.group_shift;
    const uint32_t t0 = chunk << dc.chunk_shift, c0 = group << dc.group_shift;
    const uint32_t t_last = tile > t0 ? tile - t0 - 1 : 0u;     // entries before this one (t0 itself exists)
    const uint32_t c_last = chunk > c0 ? chunk - c0 - 1 : 0u;
    const uint32_t g_last = dc.num_groups - 1;
#pragma unroll
    for (uint32_t k = 0; k < kCapTiles; ++k) tc.tile[k] = dc.hist[(size_t)(t0 + min(k, t_last)) * kRadix + d];
#pragma unroll
    for (uint32_t k = 0; k < kCapChunks; ++k) tc.chunk[k] = dc.chunk[(size_t)(c0 + min(k, c_last)) * kRadix + d];
#pragma unroll
    for (uint32_t k = 0; k < kCapGroups; ++k) tc.group[k] = dc.group[(size_t)min(k, g_last) * kRadix + d];
}

template <bool SMALL>
__device__ __forceinline__ void sum_tile_counts(const DigitCounts& dc, uint32_t tile, int d, const TileCounts& tc,
                                                uint32_t* total, uint32_t* before) {
    const uint32_t chunk = tile >> dc.chunk_shift, group = chunk >> dc.group_shift;
    const uint32_t t0 = chunk << dc.chunk_shift, c0 = group << dc.group_shift;
    uint32_t t = 0, b = 0;
    if (SMALL) {
#pragma unroll
        for (uint32_t k = 0; k < kCapTiles; ++k) b += k < tile - t0 ? tc.tile[k] : 0u;
#pragma unroll
        for (uint32_t k = 0; k < kCapChunks; ++k) b += k < chunk - c0 ? tc.chunk[k] : 0u;
#pragma unroll
        for (uint32_t k = 0; k < kCapGroups; ++k) {
            const uint32_t x = k < dc.num_groups ? tc.group[k] : 0u;
            t += x;
            b += k < group ? x : 0u;
        }
    } else {
#pragma unroll 4
        for (uint32_t k = t0; k < tile; ++k) b += dc.hist[(size_t)k * kRadix + d];
#pragma unroll 4
        for (uint32_t k = c0; k < chunk; ++k) b += dc.chunk[(size_t)k * kRadix + d];
#pragma unroll 8
        for (uint32_t k = 0; k < dc.num_groups; ++k) {
            const uint32_t x = dc.group[(size_t)k * kRadix + d];
            t += x;
            b += k < group ? x : 0u;
        }
    }
    *total = t;
    *before = b;
}

// Tile histograms of the digit at `shift` (passes after the first).
__global__ __launch_bounds__(kBlock) void upsweep_kernel(const uint32_t* __restrict__ keys, uint32_t n, int shift,
                                                         DigitCounts dc) {
    __shared__ uint32_t s_cnt[kBlock / 64][kRadix];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) s_cnt[k][tid] = 0;
    __syncthreads();
    const uint32_t base = blockIdx.x * (uint32_t)kTile + (uint32_t)w * kWaveSpan;
    uint32_t key[kItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const uint32_t e = base + (uint32_t)it * 64 + (uint32_t)lane;
        key[it] = e < n ? keys[min(e, n - 1)] : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int it = 0; it < kItems; ++it)
        if (base + (uint32_t)it * 64 + (uint32_t)lane < n) atomicAdd(&s_cnt[w][(key[it] >> shift) & 0xFFu], 1u);
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) c += s_cnt[k][tid];
    publish_tile_counts(dc, blockIdx.x, tid, c);
}

// Exclusive prefix sum over the threads of a BLOCK-thread block; *total gets the sum.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_exclusive_scan_n(uint32_t v, uint32_t* total, uint32_t* s_tmp) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    uint32_t wave_off = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < BLOCK / 64; ++k) {
        const uint32_t t = s_tmp[k];
        if (k < w) wave_off += t;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return wave_off + x - v;
}

// One stable scatter pass of the LSD radix sort.  vals_in == nullptr means
// the value of entry e is e itself.  SMALL as for load_tile_counts.
template <bool SMALL>
__global__ __launch_bounds__(kBlock) void downsweep_kernel(const uint32_t* __restrict__ keys_in,
                                                           const uint32_t* __restrict__ vals_in,
                                                           uint32_t* __restrict__ keys_out,
                                                           uint32_t* __restrict__ vals_out, uint32_t n, int shift,
                                                           DigitCounts dc) {
    __shared__ uint32_t s_keys[kTile];
    __shared__ uint32_t s_vals[kTile];
    __shared__ uint32_t s_wave_cnt[kBlock / 64][kRadix];
    __shared__ uint32_t s_digit_start[kRadix];
    __shared__ uint32_t s_global[kRadix];
    __shared__ uint32_t s_tmp[kBlock / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < (kBlock / 64) * kRadix; i += kBlock) (&s_wave_cnt[0][0])[i] = 0;
    __syncthreads();

    const uint32_t tile_base = blockIdx.x * (uint32_t)kTile;
    const uint32_t base = tile_base + (uint32_t)w * kWaveSpan;
    TileCounts tc;
    load_tile_counts<SMALL>(dc, blockIdx.x, tid, tc);
    uint32_t key[kItems], val[kItems], rank[kItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const uint32_t e = min(base + (uint32_t)it * 64 + (uint32_t)lane, n - 1);
        key[it] = keys_in[e];
        val[it] = vals_in ? vals_in[e] : e;  // no values: the input order itself (a first pass)
    }
    // Thread tid's digit: its total over all tiles and its keys in earlier tiles.
    uint32_t digit_total, digit_before;
    sum_tile_counts<SMALL>(dc, blockIdx.x, tid, tc, &digit_total, &digit_before);
    // Sum here, not next to the use: the loaded counts then die before the
    // ranking needs its registers.
    asm volatile("" : "+v"(digit_total), "+v"(digit_before));
    // Rank every key among the equal digits before it in this wave's span:
    // items are visited in index order and the lowest lane of each digit group
    // advances the wave's counter for that digit.
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const bool live = base + (uint32_t)it * 64 + (uint32_t)lane < n;
        const uint32_t d = (key[it] >> shift) & 0xFFu;
        const uint64_t peers = match_digit(d, live);
        const uint32_t before = (uint32_t)__popcll(peers & lanemask_lt(lane));
        uint32_t cnt = 0;
        if (live) cnt = s_wave_cnt[w][d];
        rank[it] = cnt + before;
        if (live && before == 0) s_wave_cnt[w][d] = cnt + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    // Per digit: offsets of the waves inside the tile and the tile total.
    {
        const int d = tid;
        uint32_t sum = 0;
#pragma unroll
        for (int k = 0; k < kBlock / 64; ++k) {
            const uint32_t c = s_wave_cnt[k][d];
            s_wave_cnt[k][d] = sum;
            sum += c;
        }
        uint32_t tot;
        s_digit_start[d] = block_exclusive_scan(sum, &tot, s_tmp);
        s_global[d] = block_exclusive_scan(digit_total, &tot, s_tmp) + digit_before;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const bool live = base + (uint32_t)it * 64 + (uint32_t)lane < n;
        if (live) {
            const uint32_t d = (key[it] >> shift) & 0xFFu;
            const uint32_t pos = s_digit_start[d] + s_wave_cnt[w][d] + rank[it];
            s_keys[pos] = key[it];
            s_vals[pos] = val[it];
        }
    }
    __syncthreads();
    const uint32_t count = min((uint32_t)kTile, n - tile_base);
    for (uint32_t j = tid; j < count; j += kBlock) {
        const uint32_t k = s_keys[j];
        const uint32_t d = (k >> shift) & 0xFFu;
        const uint32_t g = s_global[d] + (j - s_digit_start[d]);
        if (g < n) {  // always true for a consistent histogram; keeps every store in bounds
            keys_out[g] = k;
            vals_out[g] = s_vals[j];
        }
    }
}

}  // namespace
}  // namespace engram
