// Stable LSD radix sort of (32-bit key, 32-bit index) pairs for gfx950: the
// pieces shared by the backward's sort by row (scatter.hip) and the routing
// sort by owner (route.hip).  Included by both; everything is internal.
//
// A tile of kTile pairs is owned by one 256-thread block, each wave owning a
// contiguous span of 64 * kItems pairs.  Per digit pass (8 bits, or 9 for a
// last pass that needs one bit more):
//   histogram   per-tile digit counts (per-wave LDS atomics, then summed),
//               stored per tile and added into the totals of the tile's
//               chunk and group (see DigitCounts);
//   downsweep   finds where each of its digits starts from those counts,
//               ranks every key among the equal digits before it in its wave
//               span with ballots (no atomics, hence stable), orders the tile
//               by digit in LDS and writes each digit's run to its global slot.
// A pass's histogram usually comes from the kernel that wrote its keys.
//
// A sort may also be segmented: several independent sorts of equal length,
// laid out one after another, each sorted in place (see Segments).
#pragma once

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kBlock = 256;                       // threads per block, 4 waves
// Keys per thread in a sort tile is a template parameter of the sort kernels
// (ITEMS); these are the defaults, which the routing sort uses.
constexpr int kItems = 16;                        // keys per thread in a sort tile
constexpr int kTile = kBlock * kItems;            // 4096 keys per sort tile
constexpr int kWaveSpan = 64 * kItems;            // contiguous keys owned by one wave
constexpr int kRadix = 256;

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Lanes of the wave whose BITS-bit digit equals this lane's, among lanes with
// `live`.  Per bit: the lanes whose bit matches this lane's are ~(ballot ^ rep),
// rep being this lane's bit spread over a word; keeping them is one three-input
// bitwise instruction per half of the mask.
template <int BITS = 8>
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool live) {
    const uint64_t l = __ballot(live);
    uint32_t lo = (uint32_t)l, hi = (uint32_t)(l >> 32);
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
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
// All three arrays hold the R digits of one tile (chunk, group) contiguously
// (R = 256 or 512, the pass's radix), so a block reads its counts for one
// entry in coalesced loads.
struct DigitCounts {
    uint32_t* hist;    // [num_tiles][R]
    uint32_t* chunk;   // [num_chunks][R], zero before the histogram kernel
    uint32_t* group;   // [num_groups][R], zero before the histogram kernel
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
// Words of chunk and group totals for one pass of radix `radix`.
inline size_t count_words(int64_t num_tiles, int radix = kRadix) {
    const CountShape c = count_shape(num_tiles);
    return (size_t)radix * (size_t)(c.num_chunks + c.num_groups);
}
// `totals` holds count_words(num_tiles, radix) words: the chunk totals, then the group totals.
inline DigitCounts make_digit_counts(void* hist, uint32_t* totals, int64_t num_tiles, int radix = kRadix) {
    const CountShape c = count_shape(num_tiles);
    return DigitCounts{(uint32_t*)hist, totals, totals + (size_t)radix * (size_t)c.num_chunks,
                       (uint32_t)c.num_groups, c.chunk_shift, c.group_shift};
}

// A segmented sort: segments of `len` keys each (as many as the grid holds,
// `tiles` blocks per segment), segment s holding
// entries [s * len, (s + 1) * len) of every key and value array and sorted
// in place, so no key leaves its segment.  Segment s owns grid blocks
// [s * tiles, (s + 1) * tiles) and its own digit counts, `hist_words` and
// `total_words` further on than those of segment s - 1.  Its digits are
// taken from key - base[s]: every key of segment s lies in
// [base[s], base[s] + 2^bits), so fewer digit passes cover it than the whole
// key range would need.  A first pass without a value array gives entry e of
// segment s the value e * val_mul + s.  An unsegmented sort is one segment
// with base 0 and val_mul 1.
constexpr int kMaxSegs = 16;
struct Segments {
    uint32_t len, tiles, val_mul, hist_words, total_words;
    uint32_t base[kMaxSegs];
};
inline Segments one_segment(uint32_t n, uint32_t tiles) {
    Segments sg{};
    sg.len = n;
    sg.tiles = tiles;
    sg.val_mul = 1;
    return sg;
}
// base[s] for a block-uniform s, selected with compile-time indices so the
// array stays in kernel arguments.
__device__ __forceinline__ uint32_t segment_base(const Segments& sg, uint32_t s) {
    uint32_t b = sg.base[0];
#pragma unroll
    for (int k = 1; k < kMaxSegs; ++k)
        if (s == (uint32_t)k) b = sg.base[k];
    return b;
}
__device__ __forceinline__ DigitCounts segment_counts(DigitCounts dc, const Segments& sg, uint32_t s) {
    dc.hist += (size_t)s * sg.hist_words;
    dc.chunk += (size_t)s * sg.total_words;
    dc.group += (size_t)s * sg.total_words;
    return dc;
}

template <int R = kRadix>
__device__ __forceinline__ void publish_tile_counts(const DigitCounts& dc, uint32_t tile, int d, uint32_t c) {
    dc.hist[(size_t)tile * R + d] = c;
    if (c) {
        const uint32_t chunk = tile >> dc.chunk_shift;
        atomicAdd(&dc.chunk[(size_t)chunk * R + d], c);
        atomicAdd(&dc.group[(size_t)(chunk >> dc.group_shift) * R + d], c);
    }
}

// The counts that place one digit for one tile: the digit's total over all
// tiles and its keys in the tiles before this one.  With at most kCapTiles
// tiles per chunk, kCapChunks chunks per group and kCapGroups groups (up to
// 2^22 keys), every count is loaded at once by clamped, unguarded loads
// issued before the tile's keys, so both sets of loads are in flight
// together; larger sorts sum them in loops.
constexpr uint32_t kCapTiles = 8, kCapChunks = 8, kCapGroups = 16;
struct TileCounts {
    uint32_t tile[kCapTiles];     // this chunk's tiles (clamped)
    uint32_t chunk[kCapChunks];   // this group's chunks (clamped)
    uint32_t group[kCapGroups];   // all groups (clamped)
};

inline bool small_counts(const DigitCounts& dc) {
    return (1u << dc.chunk_shift) <= kCapTiles && (1u << dc.group_shift) <= kCapChunks && dc.num_groups <= kCapGroups;
}

template <bool SMALL, int R = kRadix>
__device__ __forceinline__ void load_tile_counts(const DigitCounts& dc, uint32_t tile, int d, TileCounts& tc) {
    if (!SMALL) return;
    const uint32_t chunk = tile >> dc.chunk_shift, group = chunk >> dc.group_shift;
    const uint32_t t0 = chunk << dc.chunk_shift, c0 = group << dc.group_shift;
    const uint32_t t_last = tile > t0 ? tile - t0 - 1 : 0u;     // entries before this one (t0 itself exists)
    const uint32_t c_last = chunk > c0 ? chunk - c0 - 1 : 0u;
    const uint32_t g_last = dc.num_groups - 1;
#pragma unroll
    for (uint32_t k = 0; k < kCapTiles; ++k) tc.tile[k] = dc.hist[(size_t)(t0 + min(k, t_last)) * R + d];
#pragma unroll
    for (uint32_t k = 0; k < kCapChunks; ++k) tc.chunk[k] = dc.chunk[(size_t)(c0 + min(k, c_last)) * R + d];
#pragma unroll
    for (uint32_t k = 0; k < kCapGroups; ++k) tc.group[k] = dc.group[(size_t)min(k, g_last) * R + d];
}

template <bool SMALL, int R = kRadix>
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
        for (uint32_t k = t0; k < tile; ++k) b += dc.hist[(size_t)k * R + d];
#pragma unroll 4
        for (uint32_t k = c0; k < chunk; ++k) b += dc.chunk[(size_t)k * R + d];
#pragma unroll 8
        for (uint32_t k = 0; k < dc.num_groups; ++k) {
            const uint32_t x = dc.group[(size_t)k * R + d];
            t += x;
            b += k < group ? x : 0u;
        }
    }
    *total = t;
    *before = b;
}

// The counts of one digit straight from the tile histograms of a short
// segment (at most kDirectTiles tiles, so no chunk or group totals are
// needed, nor zeroed): its total over the segment's tiles and its keys in the
// tiles before `tile`.
constexpr uint32_t kDirectTiles = 64;
template <int R>
__device__ __forceinline__ void direct_tile_counts(const DigitCounts& dc, uint32_t tiles, uint32_t tile, int d,
                                                   uint32_t* total, uint32_t* before) {
    uint32_t t = 0, b = 0;
#pragma unroll 8
    for (uint32_t k = 0; k < tiles; ++k) {
        const uint32_t x = dc.hist[(size_t)k * R + d];
        t += x;
        b += k < tile ? x : 0u;
    }
    *total = t;
    *before = b;
}

// Tile histograms of the BITS-bit digit at `shift` (passes after the first).
// Thread tid owns digits tid * DPT .. tid * DPT + DPT - 1.
template <int ITEMS = kItems, int BITS = 8>
__global__ __launch_bounds__(kBlock) void upsweep_kernel(const uint32_t* __restrict__ keys, int shift,
                                                         DigitCounts dc, Segments sg) {
    constexpr int R = 1 << BITS, DPT = R / kBlock;
    static_assert(DPT >= 1, "at least one digit per thread");
    __shared__ uint32_t s_cnt[kBlock / 64][R];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint32_t seg = blockIdx.x / sg.tiles, tile = blockIdx.x - seg * sg.tiles;
    const uint32_t n = sg.len, sb = segment_base(sg, seg);
    keys += (size_t)seg * n;
    dc = segment_counts(dc, sg, seg);
    for (int i = tid; i < (kBlock / 64) * R; i += kBlock) (&s_cnt[0][0])[i] = 0;
    __syncthreads();
    const uint32_t base = tile * (uint32_t)(kBlock * ITEMS) + (uint32_t)w * (64 * ITEMS);
    uint32_t key[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const uint32_t e = base + (uint32_t)it * 64 + (uint32_t)lane;
        key[it] = keys[min(e, n - 1)];
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it)
        if (base + (uint32_t)it * 64 + (uint32_t)lane < n)
            atomicAdd(&s_cnt[w][((key[it] - sb) >> shift) & (uint32_t)(R - 1)], 1u);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < DPT; ++q) {
        const int d = tid * DPT + q;
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < kBlock / 64; ++k) c += s_cnt[k][d];
        publish_tile_counts<R>(dc, tile, d, c);
    }
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

// Where the routing sort's single pass puts its result: each entry's ID
// (ids[value]) and request position (the value) as int64 at its sorted slot,
// and the per-owner counts (digit totals below `world`) from block 0.
struct GroupedOut {
    const int64_t* ids;
    int64_t* sorted_ids;
    int64_t* order;
    int64_t* send_counts;
    int world;
};

// One stable scatter pass of the LSD radix sort over the BITS-bit digit at
// `shift`.  vals_in == nullptr means the value of an entry is its index (see
// Segments).  SMALL as for load_tile_counts; DIRECT takes the counts from the
// tile histograms alone (direct_tile_counts).  With GROUPED (one unsegmented
// 8-bit pass) the pass writes `go`'s outputs instead of keys_out / vals_out.
// Thread tid owns digits tid * DPT .. tid * DPT + DPT - 1.
template <bool SMALL, int ITEMS = kItems, bool GROUPED = false, int BITS = 8, bool DIRECT = false>
__global__ __launch_bounds__(kBlock) void downsweep_kernel(const uint32_t* __restrict__ keys_in,
                                                           const uint32_t* __restrict__ vals_in,
                                                           uint32_t* __restrict__ keys_out,
                                                           uint32_t* __restrict__ vals_out, int shift,
                                                           DigitCounts dc, Segments sg, GroupedOut go) {
    constexpr int R = 1 << BITS, DPT = R / kBlock;
    static_assert(DPT >= 1 && (!GROUPED || DPT == 1), "grouped output takes 8-bit digits");
    __shared__ uint32_t s_keys[kBlock * ITEMS];
    __shared__ uint32_t s_vals[kBlock * ITEMS];
    // per wave and digit: the wave's count, then where the wave's keys of the
    // digit start inside the tile (row 0: where the tile's digit run starts);
    // both below the tile size, so 16 bits each (a 9-bit pass of 24 keys per
    // thread then fits three blocks per compute unit).  Once the tile is
    // ordered, the same words hold, per digit, where the tile's digit run goes
    // globally less where it starts in the tile (s_run_off, 32 bits).
    static_assert(kBlock * ITEMS <= 0xFFFF, "tile offsets fit 16 bits");
    __shared__ uint16_t s_wave_cnt[kBlock / 64][R];
    uint32_t* const s_run_off = reinterpret_cast<uint32_t*>(&s_wave_cnt[0][0]);  // R of the array's 2R words
    uint32_t* const s_tmp = s_keys;  // the scans' scratch: s_keys is written only after them
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint32_t seg = blockIdx.x / sg.tiles, tile = blockIdx.x - seg * sg.tiles;
    const uint32_t n = sg.len, sb = segment_base(sg, seg);
    const size_t so = (size_t)seg * n;  // the segment's first entry
    dc = segment_counts(dc, sg, seg);
    for (int i = tid; i < (kBlock / 64) * R; i += kBlock) (&s_wave_cnt[0][0])[i] = 0;
    __syncthreads();

    const uint32_t tile_base = tile * (uint32_t)(kBlock * ITEMS);
    const uint32_t base = tile_base + (uint32_t)w * (64 * ITEMS);
    TileCounts tc[DPT];
#pragma unroll
    for (int q = 0; q < DPT; ++q) load_tile_counts<SMALL && !DIRECT, R>(dc, tile, tid * DPT + q, tc[q]);
    uint32_t key[ITEMS], val[ITEMS], rank[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const uint32_t e = min(base + (uint32_t)it * 64 + (uint32_t)lane, n - 1);
        key[it] = keys_in[so + e];
        val[it] = vals_in ? vals_in[so + e] : e * sg.val_mul + seg;  // no values: the input order (a first pass)
    }
    // Per owned digit: its total over the segment's tiles and its keys in earlier tiles.
    uint32_t digit_total[DPT], digit_before[DPT];
#pragma unroll
    for (int q = 0; q < DPT; ++q) {
        if (DIRECT)
            direct_tile_counts<R>(dc, sg.tiles, tile, tid * DPT + q, &digit_total[q], &digit_before[q]);
        else
            sum_tile_counts<SMALL, R>(dc, tile, tid * DPT + q, tc[q], &digit_total[q], &digit_before[q]);
        // Sum here, not next to the use: the loaded counts then die before the
        // ranking needs its registers.
        asm volatile("" : "+v"(digit_total[q]), "+v"(digit_before[q]));
    }
    // Rank every key among the equal digits before it in this wave's span:
    // items are visited in index order and the lowest lane of each digit group
    // advances the wave's counter for that digit.
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const bool live = base + (uint32_t)it * 64 + (uint32_t)lane < n;
        const uint32_t d = ((key[it] - sb) >> shift) & (uint32_t)(R - 1);
        const uint64_t peers = match_digit<BITS>(d, live);
        const uint32_t before = (uint32_t)__popcll(peers & lanemask_lt(lane));
        uint32_t cnt = 0;
        if (live) cnt = s_wave_cnt[w][d];
        rank[it] = cnt + before;
        if (live && before == 0) s_wave_cnt[w][d] = (uint16_t)(cnt + (uint32_t)__popcll(peers));
    }
    __syncthreads();
    // Per owned digit: where each wave's keys of it start inside the tile, and
    // where the tile's keys of it go globally.
    uint32_t global_start[DPT];
    {
        uint32_t tile_cnt[DPT], tile_sum = 0, seg_sum = 0;
#pragma unroll
        for (int q = 0; q < DPT; ++q) {
            const int d = tid * DPT + q;
            uint32_t sum = 0;
#pragma unroll
            for (int k = 0; k < kBlock / 64; ++k) {
                const uint32_t c = s_wave_cnt[k][d];
                s_wave_cnt[k][d] = (uint16_t)sum;
                sum += c;
            }
            tile_cnt[q] = sum;
            tile_sum += sum;
            seg_sum += digit_total[q];
        }
        uint32_t tot;
        uint32_t tile_run = block_exclusive_scan(tile_sum, &tot, s_tmp);
        uint32_t seg_run = block_exclusive_scan(seg_sum, &tot, s_tmp);
#pragma unroll
        for (int q = 0; q < DPT; ++q) {
            const int d = tid * DPT + q;
#pragma unroll
            for (int k = 0; k < kBlock / 64; ++k) s_wave_cnt[k][d] = (uint16_t)(s_wave_cnt[k][d] + tile_run);
            global_start[q] = seg_run + digit_before[q] - tile_run;
            tile_run += tile_cnt[q];
            seg_run += digit_total[q];
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const bool live = base + (uint32_t)it * 64 + (uint32_t)lane < n;
        if (live) {
            const uint32_t d = ((key[it] - sb) >> shift) & (uint32_t)(R - 1);
            const uint32_t pos = s_wave_cnt[w][d] + rank[it];
            s_keys[pos] = key[it];
            s_vals[pos] = val[it];
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < DPT; ++q) s_run_off[tid * DPT + q] = global_start[q];  // the wave offsets are no longer read
    __syncthreads();
    const uint32_t count = min((uint32_t)(kBlock * ITEMS), n - tile_base);
    for (uint32_t j = tid; j < count; j += kBlock) {
        const uint32_t k = s_keys[j];
        const uint32_t d = ((k - sb) >> shift) & (uint32_t)(R - 1);
        const uint32_t g = s_run_off[d] + j;  // unsigned wrap-around cancels
        if (g < n) {  // always true for a consistent histogram; keeps every store in its segment
            if (GROUPED) {
                const uint32_t v = min(s_vals[j], n - 1);
                go.sorted_ids[g] = go.ids[v];
                go.order[g] = v;
            } else {
                keys_out[so + g] = k;
                vals_out[so + g] = s_vals[j];
            }
        }
    }
    if (GROUPED && blockIdx.x == 0 && tid < go.world) {
        uint32_t total = 0;  // every group's count of owner tid
        for (uint32_t gi = 0; gi < dc.num_groups; ++gi) total += dc.group[(size_t)gi * R + tid];
        go.send_counts[tid] = total;
    }
}

}  // namespace
}  // namespace engram
