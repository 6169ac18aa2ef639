// Stable LSD radix sort of (32-bit key, 32-bit index) pairs for gfx950: the
// pieces shared by the backward's sort by row (scatter.hip) and the routing
// sort by owner (route.hip).  Included by both; everything is internal.
//
// A tile of kTile pairs is owned by one 256-thread block, each wave owning a
// contiguous span of 64 * kItems pairs.  Per 8-bit digit pass:
//   upsweep     per-tile digit histograms (per-wave LDS atomics, then summed);
//   digit_scan  for every digit, an exclusive prefix over the tiles;
//   downsweep   ranks every key among the equal digits before it in its wave
//               span with ballots (no atomics, hence stable), orders the tile
//               by digit in LDS and writes each digit's run to its global slot.
// A pass's first histogram usually comes from the kernel that builds the keys.
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
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool live) {
    uint64_t m = __ballot(live);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
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

// Tile histograms of the digit at `shift` (passes after the first).
__global__ __launch_bounds__(kBlock) void upsweep_kernel(const uint32_t* __restrict__ keys, uint32_t n, int shift,
                                                         uint32_t* __restrict__ hist, uint32_t num_tiles) {
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
    hist[(size_t)tid * num_tiles + blockIdx.x] = c;
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

// hist[d][tile] -> exclusive prefix over tiles (in place); digit_total[d] = sum.
// One 256-thread block per digit.  Small blocks on purpose: the plan usually
// runs beside the gather, and a block that needs few wave slots starts as
// soon as a compute unit has room.
__global__ __launch_bounds__(kBlock) void digit_scan_kernel(uint32_t* __restrict__ hist, uint32_t num_tiles,
                                                            uint32_t* __restrict__ digit_total) {
    __shared__ uint32_t s_tmp[kBlock / 64];
    uint32_t* row = hist + (size_t)blockIdx.x * num_tiles;
    uint32_t running = 0;
    for (uint32_t b = 0; b < num_tiles; b += kBlock) {
        const uint32_t i = b + threadIdx.x;
        const uint32_t raw = row[min(i, num_tiles - 1)];
        const uint32_t v = i < num_tiles ? raw : 0u;
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan(v, &tot, s_tmp);
        if (i < num_tiles) row[i] = running + ex;
        running += tot;
    }
    if (threadIdx.x == 0) digit_total[blockIdx.x] = running;
}

// One stable scatter pass of the LSD radix sort.  vals_in == nullptr means
// the value of entry e is e itself.
__global__ __launch_bounds__(kBlock) void downsweep_kernel(const uint32_t* __restrict__ keys_in,
                                                           const uint32_t* __restrict__ vals_in,
                                                           uint32_t* __restrict__ keys_out,
                                                           uint32_t* __restrict__ vals_out, uint32_t n, int shift,
                                                           const uint32_t* __restrict__ hist,
                                                           const uint32_t* __restrict__ digit_total,
                                                           uint32_t num_tiles) {
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
    uint32_t key[kItems], val[kItems], rank[kItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const uint32_t e = min(base + (uint32_t)it * 64 + (uint32_t)lane, n - 1);
        key[it] = keys_in[e];
        val[it] = vals_in ? vals_in[e] : e;  // no values: the input order itself (a first pass)
    }
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
        const uint32_t start = block_exclusive_scan(sum, &tot, s_tmp);
        s_digit_start[d] = start;
        uint32_t tot2;
        const uint32_t digit_base = block_exclusive_scan(digit_total[d], &tot2, s_tmp);
        s_global[d] = digit_base + hist[(size_t)d * num_tiles + blockIdx.x];
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
