// Owner routing on one GPU: the single-GPU half of the row-owner exchange.
//
// Engram API page ("nemo_automodel.components.models.qwen3_8_flash_next.engram"),
// Qwen3_8_FlashNextOwnerShardedEmbedding: rank r owns rows
// [r * local_rows, (r + 1) * local_rows); a request rank groups its global row
// IDs by owner and sends them in a first All-to-All (_exchange_ids); owners
// look up their local rows; a second, autograd-aware All-to-All returns the
// values (and the gradients the other way).  _validate_sorted_send_ids checks
// that each destination segment holds only that owner's IDs;
// _fixed_capacity_all_to_all pads every peer segment to one agreed capacity
// with a fill value, exchanges equal splits, and restores the compact,
// source-ordered result.
//
// Kernels here:
//   route plan     owner = id / local_rows; a stable one-digit radix pass
//                  groups the IDs by owner (request order kept inside each
//                  segment); send counts = the owner histogram.
//   validate       every ID of segment w lies in owner w's row range.
//   pack / unpack  compact segments <-> [world][capacity] padded blocks.
//   permute        rows into / out of the grouped order.
//   unpack_unpermute  the requester's unpack and the move back to request
//                  order in one pass; permute_pack  the move into grouped
//                  order and the pack in one pass (the backward's send);
//   gather_padded  the owner's lookup from the received padded ID blocks
//                  straight into padded value blocks.
// The collective itself (RCCL all-to-all over xGMI) is outside this library.
#include <algorithm>

#include "radix_sort.h"
#include "row_copy.h"

// Units (16 or 4 bytes) per thread and loop step of the fused unpack: 2
// measured best on the world-64 value rows (79 us against 87 us with 1).
#ifndef ENGRAM_UNPERMUTE_K
#define ENGRAM_UNPERMUTE_K 2
#endif

namespace engram {
namespace {

// World sizes are 1..255 (checked by the API): owners fit one 8-bit digit with
// 255 left for out-of-range IDs, and one thread per count fits a block.

struct RouteLayout {
    size_t keys_a, hist, count_totals, counters, total;
    int64_t num_tiles;
};

RouteLayout route_layout(int64_t n) {
    RouteLayout L;
    L.num_tiles = (n + kTile - 1) / kTile;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = (off + bytes + 255) & ~(size_t)255; return at; };
    L.keys_a = take(4 * (size_t)n);
    L.hist = take(4 * (size_t)kRadix * (size_t)L.num_tiles);
    L.count_totals = take(4 * count_words(L.num_tiles));
    L.counters = take(16);
    L.total = off;
    return L;
}

__global__ void zero_counts_kernel(int64_t* counts, int world) {
    if (threadIdx.x < (unsigned)world) counts[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kBlock) void route_init_kernel(int64_t* status, uint32_t* counters,
                                                            uint32_t* count_totals, uint32_t total_words) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (status) *status = -1;
        counters[0] = 0;
    }
    for (uint32_t i = blockIdx.x * kBlock + threadIdx.x; i < total_words; i += gridDim.x * kBlock)
        count_totals[i] = 0;
}

// Owner keys (sentinel `world` for an ID outside the table) and the per-tile
// owner histogram; the request index of each key is its position.
__global__ __launch_bounds__(kBlock) void route_keys_kernel(const int64_t* __restrict__ ids, uint32_t n,
                                                            int64_t local_rows, int world, uint32_t* __restrict__ keys,
                                                            DigitCounts dc, int64_t* __restrict__ status) {
    __shared__ uint32_t s_cnt[kBlock / 64][kRadix];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) s_cnt[k][tid] = 0;
    __syncthreads();
    const uint32_t base = blockIdx.x * (uint32_t)kTile + (uint32_t)w * kWaveSpan;
    const uint64_t table_rows = (uint64_t)local_rows * (uint64_t)world;
    int64_t r[kItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) r[it] = ids[min(base + (uint32_t)it * 64 + (uint32_t)lane, n - 1)];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const uint32_t e = base + (uint32_t)it * 64 + (uint32_t)lane;
        if (e < n) {
            uint32_t key = (uint32_t)world;
            if ((uint64_t)r[it] < table_rows)
                key = (uint32_t)((uint64_t)r[it] / (uint64_t)local_rows);
            else
                report_bad(status, e);
            keys[e] = key;
            atomicAdd(&s_cnt[w][key], 1u);
        }
    }
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) c += s_cnt[k][tid];
    publish_tile_counts(dc, blockIdx.x, tid, c);
}

// Per-segment facts every block of segment w needs, from the counts (up to
// 255, one per thread) by one block reduction:
//   off      sum over v < w of the segment lengths before w
//   total    sum over every segment
//   any_bad  some count is negative
// A segment's length is its count clamped below at 0 and, with clamp_cap,
// above at the capacity.
struct SegmentInfo {
    int64_t off, total;
    bool any_bad;
};

__device__ SegmentInfo segment_info(const int64_t* __restrict__ counts, int world, int w, int64_t capacity,
                                    bool clamp_cap) {
    __shared__ int64_t s_off[kBlock / 64], s_tot[kBlock / 64];
    __shared__ int s_bad[kBlock / 64];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int64_t c = t < world ? counts[t] : 0;
    const int bad = c < 0;
    c = c < 0 ? 0 : (clamp_cap && c > capacity ? capacity : c);
    int64_t before = t < w ? c : 0, all = c;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        before += __shfl_xor(before, o, 64);
        all += __shfl_xor(all, o, 64);
    }
    const int any = __any(bad);
    if (lane == 0) {
        s_off[wv] = before;
        s_tot[wv] = all;
        s_bad[wv] = any;
    }
    __syncthreads();
    SegmentInfo r{0, 0, false};
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) {
        r.off += s_off[k];
        r.total += s_tot[k];
        r.any_bad = r.any_bad || s_bad[k];
    }
    return r;
}

// Blocks are laid out as grid (x, world): blockIdx.y is the segment, x strides
// over its units.  Segment offsets come from segment_info; unit indices are
// 32-bit when a segment has fewer than 2^31 units (I = uint32_t), which keeps
// the per-unit division cheap.

// Segment w of sorted_ids must hold only owner w's IDs.  Counts that are
// negative or add up to more than n are reported as n and nothing is checked.
template <typename I>
__global__ __launch_bounds__(kBlock) void route_validate_kernel(const int64_t* __restrict__ sorted_ids, int64_t n,
                                                                const int64_t* __restrict__ send_counts, int world,
                                                                int64_t local_rows, int64_t* __restrict__ status) {
    const int w = blockIdx.y;
    const SegmentInfo si = segment_info(send_counts, world, w, 0, false);
    if (si.any_bad || si.total > n) {
        if (blockIdx.x == 0 && w == 0 && threadIdx.x == 0) report_bad(status, n);
        return;
    }
    const I len = (I)send_counts[w];
    const int64_t lo = (int64_t)w * local_rows, hi = lo + local_rows;
    for (I e = (I)blockIdx.x * kBlock + threadIdx.x; e < len; e += (I)gridDim.x * kBlock) {
        const int64_t id = sorted_ids[si.off + (int64_t)e];
        if (id < lo || id >= hi) report_bad(status, si.off + (int64_t)e);
    }
}

// The fill of unit k of a row: `fill` is the fill element repeated over 16
// bytes, and rows start on a multiple of the element, so a 4-byte unit at byte
// 4k of the row takes word k mod 4 and a 16-byte unit takes all of it.
template <typename U>
__device__ __forceinline__ U fill_unit(u32x4 fill, uint32_t k);
template <>
__device__ __forceinline__ u32x4 fill_unit<u32x4>(u32x4 fill, uint32_t) { return fill; }
template <>
__device__ __forceinline__ uint32_t fill_unit<uint32_t>(u32x4 fill, uint32_t k) {
    const uint32_t j = k & 3u;
    return j == 0 ? fill[0] : (j == 1 ? fill[1] : (j == 2 ? fill[2] : fill[3]));
}

// Copy unit U: 16 bytes when rows allow it, else 4 bytes.  Segment w's
// min(count, capacity) rows go to block w, the rest of the block is the fill.
// Only the first src_rows source rows are read: a block row whose source lies
// past them takes the fill too (status world, unless a bad count is lower).
// The copy kernels move K 16-byte (or 4-byte) units per thread per loop
// step, all loads issued before the stores; the stores of consecutive units
// are non-temporal (the world-64 value pack went from 81 to 64 us with them).  Measured on the world-64 step:
// K = 4 helps the unpack (the compact side is written sequentially) and the
// 4-byte units; the pack of 16-byte units gains little and the scattering
// permute loses, so each launch picks its own K.
template <typename U, typename I, int K>
__global__ __launch_bounds__(kBlock) void pack_kernel(const U* __restrict__ src, int64_t src_rows, int64_t row_units,
                                                      const int64_t* __restrict__ counts, int world, int64_t capacity,
                                                      u32x4 fill, U* __restrict__ dst, int64_t* __restrict__ status) {
    const int w = blockIdx.y;
    const SegmentInfo si = segment_info(counts, world, w, capacity, false);
    const int64_t c = counts[w];
    const int64_t kept = c < 0 ? 0 : (c > capacity ? capacity : c);
    const int64_t avail = min(kept, max((int64_t)0, src_rows - si.off));  // kept rows that exist in src
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (c < 0 || c > capacity) report_bad(status, w);
        if (avail < kept) report_bad(status, world);
    }
    const I rows = (I)avail;
    const I units = (I)row_units, seg_units = (I)(capacity * row_units);
    const U* __restrict__ s = src + si.off * row_units;
    U* __restrict__ d = dst + (int64_t)w * capacity * row_units;
    const I step = (I)gridDim.x * (I)(kBlock * K);
    for (I e0 = (I)blockIdx.x * (I)(kBlock * K) + threadIdx.x; e0 < seg_units; e0 += step) {
        U v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const I e = e0 + (I)(k * kBlock);
            const I r = e / units;
            v[k] = (e < seg_units && r < rows) ? s[e] : fill_unit<U>(fill, (uint32_t)(e - r * units));
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const I e = e0 + (I)(k * kBlock);
            if (e < seg_units) __builtin_nontemporal_store(v[k], d + e);
        }
    }
}

// Segment w's first min(count, capacity) rows of block w, appended in rank
// order to the compact output; rows at or past dst_rows are dropped (status
// world).
template <typename U, typename I, int K>
__global__ __launch_bounds__(kBlock) void unpack_kernel(const U* __restrict__ src, int64_t row_units,
                                                        const int64_t* __restrict__ counts, int world, int64_t capacity,
                                                        U* __restrict__ dst, int64_t dst_rows,
                                                        int64_t* __restrict__ status) {
    const int w = blockIdx.y;
    const SegmentInfo si = segment_info(counts, world, w, capacity, true);
    const int64_t c = counts[w];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (c < 0 || c > capacity) report_bad(status, w);
        if (w == world - 1 && si.total > dst_rows) report_bad(status, world);
    }
    const int64_t rows = c < 0 ? 0 : (c > capacity ? capacity : c);
    const int64_t fit = min(rows, max((int64_t)0, dst_rows - si.off));  // rows of this segment that fit
    const I seg_units = (I)(fit * row_units);
    const U* __restrict__ s = src + (int64_t)w * capacity * row_units;
    U* __restrict__ d = dst + si.off * row_units;
    const I step = (I)gridDim.x * (I)(kBlock * K);
    for (I e0 = (I)blockIdx.x * (I)(kBlock * K) + threadIdx.x; e0 < seg_units; e0 += step) {
        U v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const I e = e0 + (I)(k * kBlock);
            if (e < seg_units) v[k] = s[e];
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const I e = e0 + (I)(k * kBlock);
            if (e < seg_units) __builtin_nontemporal_store(v[k], d + e);
        }
    }
}

// The move into grouped order and the pack in one pass (the requester's send
// of gradient rows in the backward): block w's row r is grouped row
// k = offset of w + r, read from request position order[k]; rows past the
// kept count, past n, or whose order entry lies outside [0, n) take the fill.
// Block rows are written in order, so the stores are non-temporal (as the
// pack's).
template <typename U, typename I, int K>
__global__ __launch_bounds__(kBlock) void permute_pack_kernel(const U* __restrict__ src, int64_t row_units,
                                                              const int64_t* __restrict__ order, int64_t n,
                                                              const int64_t* __restrict__ counts, int world,
                                                              int64_t capacity, u32x4 fill, U* __restrict__ dst,
                                                              int64_t* __restrict__ status) {
    const int w = blockIdx.y;
    const SegmentInfo si = segment_info(counts, world, w, capacity, false);
    const int64_t c = counts[w];
    const int64_t kept = c < 0 ? 0 : (c > capacity ? capacity : c);
    const int64_t avail = min(kept, max((int64_t)0, n - si.off));  // kept rows that exist in the grouped order
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (c < 0 || c > capacity) report_bad(status, w);
        if (avail < kept) report_bad(status, world);
    }
    const I rows = (I)avail;
    const I units = (I)row_units, seg_units = (I)(capacity * row_units);
    const int64_t* __restrict__ ord = order + min(si.off, n);
    U* __restrict__ d = dst + (int64_t)w * capacity * row_units;
    const I step = (I)gridDim.x * (I)(kBlock * K);
    for (I e0 = (I)blockIdx.x * (I)(kBlock * K) + threadIdx.x; e0 < seg_units; e0 += step) {
        U v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const I e = e0 + (I)(k * kBlock);
            const I r = e / units;
            const I q = e - r * units;
            const int64_t o = (e < seg_units && r < rows) ? ord[r] : -1;
            v[k] = (uint64_t)o < (uint64_t)n ? src[o * row_units + (int64_t)q] : fill_unit<U>(fill, (uint32_t)q);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const I e = e0 + (I)(k * kBlock);
            if (e < seg_units) __builtin_nontemporal_store(v[k], d + e);
        }
    }
}

// The unpack and the move back to request order in one pass: compact row k
// (segment w's row r, k = offset of w + r, k < n) goes to dst row order[k];
// an order entry outside [0, n) is skipped.  The block rows are read in
// order and each row is written whole; its stores land at a random row, so
// they are plain stores (as the scattering permute).
template <typename U, typename I, int K>
__global__ __launch_bounds__(kBlock) void unpack_unpermute_kernel(const U* __restrict__ src, int64_t row_units,
                                                                  const int64_t* __restrict__ counts, int world,
                                                                  int64_t capacity, const int64_t* __restrict__ order,
                                                                  int64_t n, U* __restrict__ dst,
                                                                  int64_t* __restrict__ status) {
    const int w = blockIdx.y;
    const SegmentInfo si = segment_info(counts, world, w, capacity, true);
    const int64_t c = counts[w];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (c < 0 || c > capacity) report_bad(status, w);
        if (w == world - 1 && si.total > n) report_bad(status, world);
    }
    const int64_t rows = c < 0 ? 0 : (c > capacity ? capacity : c);
    const int64_t fit = min(rows, max((int64_t)0, n - si.off));  // compact rows of this segment below n
    const I units = (I)row_units, seg_units = (I)(fit * row_units);
    const U* __restrict__ s = src + (int64_t)w * capacity * row_units;
    const int64_t* __restrict__ ord = order + min(si.off, n);  // fit is 0 past n
    const I step = (I)gridDim.x * (I)(kBlock * K);
    for (I e0 = (I)blockIdx.x * (I)(kBlock * K) + threadIdx.x; e0 < seg_units; e0 += step) {
        int64_t at[K];  // destination unit, or -1
        U v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const I e = e0 + (I)(k * kBlock);
            at[k] = -1;
            if (e < seg_units) {
                const I r = e / units;
                const int64_t o = ord[r];
                if ((uint64_t)o < (uint64_t)n) at[k] = o * row_units + (int64_t)(e - r * units);
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (at[k] >= 0) v[k] = s[e0 + (I)(k * kBlock)];
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (at[k] >= 0) dst[at[k]] = v[k];
    }
}

__device__ u32x4 kZeroRowChunk = {0u, 0u, 0u, 0u};  // never written

// The owner's lookup on the exchange's padded blocks: padded entry e = (w, r)
// holds a received ID when r < split_sizes[w] (a negative count has none),
// otherwise padding.  Received IDs are looked up as the gather does (one
// wave per G entries, the row copy of row_copy.h); padding and IDs outside
// the shard give zero rows, and the lowest padded index holding an ID
// outside the shard goes to status.  Same four-wave cap as the gather.
template <int CPR, int G, bool ROW32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void gather_padded_kernel(
    const u32x4* __restrict__ table, int64_t row_begin, uint64_t num_rows, const int64_t* __restrict__ ids,
    const int64_t* __restrict__ counts, int64_t capacity, int64_t total, u32x4* __restrict__ out,
    int64_t* __restrict__ status) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t n0 = wave * G;
    if (n0 >= total) return;
    uint64_t local = ~0ull;
    if (lane < G && n0 + lane < total) {
        const int64_t e = n0 + lane;
        const int64_t w = e / capacity;
        if (e - w * capacity < counts[w]) {
            local = (uint64_t)ids[e] - (uint64_t)row_begin;
            if (local >= num_rows) {
                report_bad(status, e);
                local = ~0ull;
            }
        }
    }
    copy_wave_rows<CPR, G, ROW32, false>(table, local, n0, total, out, lane, &kZeroRowChunk);
}

// Other row sizes: one 16-byte chunk per lane over the flattened output,
// striding by the whole grid.
__global__ __launch_bounds__(256) void gather_padded_generic_kernel(const u32x4* __restrict__ table,
                                                                    int64_t row_begin, uint64_t num_rows,
                                                                    const int64_t* __restrict__ ids,
                                                                    const int64_t* __restrict__ counts,
                                                                    int64_t capacity, int64_t total, int cpr,
                                                                    u32x4* __restrict__ out,
                                                                    int64_t* __restrict__ status) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; f < total * cpr; f += stride) {
        const int64_t e = f / cpr;
        const int k = (int)(f - e * cpr);
        const int64_t w = e / capacity;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (e - w * capacity < counts[w]) {
            const uint64_t local = (uint64_t)ids[e] - (uint64_t)row_begin;
            if (local < num_rows)
                v = table[(int64_t)local * cpr + k];
            else if (k == 0)
                report_bad(status, e);
        }
        __builtin_nontemporal_store(v, out + f);
    }
}

// dst[i] = src[order[i]] (gather) or dst[order[i]] = src[i] (scatter); an
// index outside [0, n) is skipped.
template <typename U, bool GATHER, int K>
__global__ __launch_bounds__(kBlock) void permute_kernel(const U* __restrict__ src, int64_t row_units,
                                                         const int64_t* __restrict__ order, int64_t n,
                                                         U* __restrict__ dst) {
    const int64_t total = n * row_units;
    const int64_t step = (int64_t)gridDim.x * (kBlock * K);
    for (int64_t e0 = (int64_t)blockIdx.x * (kBlock * K) + threadIdx.x; e0 < total; e0 += step) {
        int64_t at[K];  // the other side's unit, or -1
        U v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t e = e0 + k * kBlock;
            at[k] = -1;
            if (e < total) {
                const int64_t i = e / row_units;
                const int64_t o = order[i];
                if ((uint64_t)o < (uint64_t)n) at[k] = o * row_units + (e - i * row_units);
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (at[k] >= 0) v[k] = GATHER ? src[at[k]] : src[e0 + k * kBlock];
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (at[k] >= 0) {
                if (GATHER)  // consecutive units: streamed past the caches
                    __builtin_nontemporal_store(v[k], dst + e0 + k * kBlock);
                else         // scattered units: plain stores (non-temporal ones measured slower)
                    dst[at[k]] = v[k];
            }
    }
}

unsigned grid_for(int64_t units) {
    const int64_t blocks = (units + kBlock - 1) / kBlock;
    return (unsigned)(blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks));
}

}  // namespace

size_t route_workspace_bytes(int64_t n) { return route_layout(n).total; }

hipError_t launch_route_plan(const int64_t* ids, int64_t n, int64_t local_rows, int world, int64_t* sorted_ids,
                             int64_t* order, int64_t* send_counts, void* workspace, int64_t* status,
                             hipStream_t stream) {
    const RouteLayout L = route_layout(n);
    char* ws = (char*)workspace;
    uint32_t* counters = (uint32_t*)(ws + L.counters);
    uint32_t* count_totals = (uint32_t*)(ws + L.count_totals);
    const uint32_t total_words = (uint32_t)count_words(L.num_tiles);
    const uint32_t init_grid = std::max(1u, std::min(64u, (total_words + kBlock - 1) / kBlock));
    hipLaunchKernelGGL(route_init_kernel, dim3(init_grid), dim3(kBlock), 0, stream, status, counters, count_totals,
                       total_words);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (n == 0) {  // no lookups: every send count is zero
        hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(kBlock), 0, stream, send_counts, world);
        return hipGetLastError();
    }
    const uint32_t nn = (uint32_t)n, tiles = (uint32_t)L.num_tiles;
    const DigitCounts dc = make_digit_counts(ws + L.hist, count_totals, L.num_tiles);
    uint32_t* ka = (uint32_t*)(ws + L.keys_a);
    hipLaunchKernelGGL(route_keys_kernel, dim3(tiles), dim3(kBlock), 0, stream, ids, nn, local_rows, world, ka, dc,
                       status);
    // One digit pass (owners fit 8 bits), writing the grouped IDs, their
    // request positions and the send counts directly.
    const GroupedOut go{ids, sorted_ids, order, send_counts, world};
    if (small_counts(dc))
        hipLaunchKernelGGL((downsweep_kernel<true, kItems, true>), dim3(tiles), dim3(kBlock), 0, stream, ka,
                           (const uint32_t*)nullptr, (uint32_t*)nullptr, (uint32_t*)nullptr, 0, dc,
                           one_segment(nn, tiles), go);
    else
        hipLaunchKernelGGL((downsweep_kernel<false, kItems, true>), dim3(tiles), dim3(kBlock), 0, stream, ka,
                           (const uint32_t*)nullptr, (uint32_t*)nullptr, (uint32_t*)nullptr, 0, dc,
                           one_segment(nn, tiles), go);
    return hipGetLastError();
}

// x blocks per segment for `units` units: enough to cover them, at most 4096 (the rest by striding).
dim3 segment_grid(int64_t units, int world) {
    int64_t x = (units + kBlock - 1) / kBlock;
    x = x < 1 ? 1 : (x > 4096 ? 4096 : x);
    return dim3((unsigned)x, (unsigned)world);
}

hipError_t launch_route_validate(const int64_t* sorted_ids, int64_t n, const int64_t* send_counts, int world,
                                 int64_t local_rows, int64_t* status, hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess) return err;
    // A segment holds at most n IDs when the counts are consistent (n < 2^31 by the API).
    hipLaunchKernelGGL((route_validate_kernel<uint32_t>), segment_grid(n / world + 1, world), dim3(kBlock), 0, stream,
                       sorted_ids, n, send_counts, world, local_rows, status);
    return hipGetLastError();
}

#define ENGRAM_SEGMENT_LAUNCH(KERNEL, U, K, UNITS, ...)                                                    \
    do {                                                                                                   \
        const dim3 grid = segment_grid(((UNITS) + (K) - 1) / (K), world);                                 \
        if ((UNITS) < ((int64_t)1 << 31) - (int64_t)grid.x * kBlock * (K))                                 \
            hipLaunchKernelGGL((KERNEL<U, uint32_t, K>), grid, dim3(kBlock), 0, stream, __VA_ARGS__);     \
        else                                                                                               \
            hipLaunchKernelGGL((KERNEL<U, uint64_t, K>), grid, dim3(kBlock), 0, stream, __VA_ARGS__);     \
    } while (0)

hipError_t launch_pack(const void* src, int64_t src_rows, int64_t row_bytes, const int64_t* counts, int world,
                       int64_t capacity, const uint32_t fill16[4], void* dst, int64_t* status, hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess) return err;
    const bool wide = row_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0;
    if (wide) {
        const int64_t units = row_bytes / 16;
        const u32x4 f = {fill16[0], fill16[1], fill16[2], fill16[3]};
        ENGRAM_SEGMENT_LAUNCH(pack_kernel, u32x4, 2, capacity * units, (const u32x4*)src, src_rows, units, counts, world,
                              capacity, f, (u32x4*)dst, status);
    } else {
        const int64_t units = row_bytes / 4;
        const u32x4 f = {fill16[0], fill16[1], fill16[2], fill16[3]};
        ENGRAM_SEGMENT_LAUNCH(pack_kernel, uint32_t, 4, capacity * units, (const uint32_t*)src, src_rows, units, counts,
                              world, capacity, f, (uint32_t*)dst, status);
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const void* src, int64_t row_bytes, const int64_t* counts, int world, int64_t capacity,
                         void* dst, int64_t dst_rows, int64_t* status, hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess) return err;
    const bool wide = row_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0;
    const int64_t rows = capacity < dst_rows ? capacity : dst_rows;  // at most per segment
    if (wide) {
        const int64_t units = row_bytes / 16;
        ENGRAM_SEGMENT_LAUNCH(unpack_kernel, u32x4, 4, rows * units, (const u32x4*)src, units, counts, world, capacity,
                              (u32x4*)dst, dst_rows, status);
    } else {
        const int64_t units = row_bytes / 4;
        ENGRAM_SEGMENT_LAUNCH(unpack_kernel, uint32_t, 4, rows * units, (const uint32_t*)src, units, counts, world,
                              capacity, (uint32_t*)dst, dst_rows, status);
    }
    return hipGetLastError();
}

hipError_t launch_unpack_unpermute(const void* src, int64_t row_bytes, const int64_t* counts, int world,
                                  int64_t capacity, const int64_t* order, int64_t n, void* dst, int64_t* status,
                                  hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess) return err;
    const bool wide = row_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0;
    const int64_t rows = capacity < n ? capacity : n;  // at most per segment
    if (wide) {
        const int64_t units = row_bytes / 16;
        ENGRAM_SEGMENT_LAUNCH(unpack_unpermute_kernel, u32x4, ENGRAM_UNPERMUTE_K, rows * units, (const u32x4*)src,
                              units, counts, world, capacity, order, n, (u32x4*)dst, status);
    } else {
        const int64_t units = row_bytes / 4;
        ENGRAM_SEGMENT_LAUNCH(unpack_unpermute_kernel, uint32_t, ENGRAM_UNPERMUTE_K, rows * units,
                              (const uint32_t*)src, units, counts, world, capacity, order, n, (uint32_t*)dst, status);
    }
    return hipGetLastError();
}

hipError_t launch_permute_pack(const void* src, int64_t row_bytes, const int64_t* order, int64_t n,
                               const int64_t* counts, int world, int64_t capacity, const uint32_t fill16[4], void* dst,
                               int64_t* status, hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess) return err;
    const bool wide = row_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0;
    const u32x4 f = {fill16[0], fill16[1], fill16[2], fill16[3]};
    if (wide) {
        const int64_t units = row_bytes / 16;
        ENGRAM_SEGMENT_LAUNCH(permute_pack_kernel, u32x4, 2, capacity * units, (const u32x4*)src, units, order, n,
                              counts, world, capacity, f, (u32x4*)dst, status);
    } else {
        const int64_t units = row_bytes / 4;
        ENGRAM_SEGMENT_LAUNCH(permute_pack_kernel, uint32_t, 4, capacity * units, (const uint32_t*)src, units, order,
                              n, counts, world, capacity, f, (uint32_t*)dst, status);
    }
    return hipGetLastError();
}

hipError_t launch_gather_padded(const void* table, int elem_bytes, int64_t row_begin, int64_t num_rows, int dim,
                                const int64_t* ids, const int64_t* counts, int world, int64_t capacity, void* out,
                                int64_t* status, hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    const int64_t total = (int64_t)world * capacity;
    if (err != hipSuccess || total == 0) return err;
    const int cpr = dim * elem_bytes / 16;
    const u32x4* t = (const u32x4*)table;
    u32x4* o = (u32x4*)out;
    const bool row32 = (uint64_t)num_rows < 0xFFFFFFFFull;
    const int64_t kMaxItems = (int64_t)1 << 31;
    const int g = cpr == 20 ? 16 : 8;
    if ((cpr == 20 || cpr == 40) && (total + g - 1) / g * 64 <= kMaxItems) {
        const int64_t waves = (total + g - 1) / g;
        const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
        if (cpr == 20 && row32)
            hipLaunchKernelGGL((gather_padded_kernel<20, 16, true>), grid, block, 0, stream, t, row_begin,
                               (uint64_t)num_rows, ids, counts, capacity, total, o, status);
        else if (cpr == 20)
            hipLaunchKernelGGL((gather_padded_kernel<20, 16, false>), grid, block, 0, stream, t, row_begin,
                               (uint64_t)num_rows, ids, counts, capacity, total, o, status);
        else if (row32)
            hipLaunchKernelGGL((gather_padded_kernel<40, 8, true>), grid, block, 0, stream, t, row_begin,
                               (uint64_t)num_rows, ids, counts, capacity, total, o, status);
        else
            hipLaunchKernelGGL((gather_padded_kernel<40, 8, false>), grid, block, 0, stream, t, row_begin,
                               (uint64_t)num_rows, ids, counts, capacity, total, o, status);
    } else {
        const int64_t grid = std::min((total * cpr + 255) / 256, kMaxItems / 256);
        hipLaunchKernelGGL(gather_padded_generic_kernel, dim3((unsigned)grid), dim3(256), 0, stream, t, row_begin,
                           (uint64_t)num_rows, ids, counts, capacity, total, cpr, o, status);
    }
    return hipGetLastError();
}

hipError_t launch_permute(const void* src, int64_t row_bytes, const int64_t* order, int64_t n, void* dst, bool gather,
                          hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const bool wide = row_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0;
    const int64_t units = wide ? row_bytes / 16 : row_bytes / 4;
    const dim3 grid(grid_for(n * units)), block(kBlock);
    if (wide && gather)
        hipLaunchKernelGGL((permute_kernel<u32x4, true, 1>), grid, block, 0, stream, (const u32x4*)src, units, order, n,
                           (u32x4*)dst);
    else if (wide)
        hipLaunchKernelGGL((permute_kernel<u32x4, false, 1>), grid, block, 0, stream, (const u32x4*)src, units, order, n,
                           (u32x4*)dst);
    else if (gather)
        hipLaunchKernelGGL((permute_kernel<uint32_t, true, 1>), grid, block, 0, stream, (const uint32_t*)src, units,
                           order, n, (uint32_t*)dst);
    else
        hipLaunchKernelGGL((permute_kernel<uint32_t, false, 1>), grid, block, 0, stream, (const uint32_t*)src, units,
                           order, n, (uint32_t*)dst);
    return hipGetLastError();
}

}  // namespace engram
