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
// The collective itself (RCCL all-to-all over xGMI) is outside this library.
#include "radix_sort.h"

namespace engram {
namespace {

constexpr int kMaxWorld = 255;  // owners fit one 8-bit digit, with 255 left for out-of-range IDs

struct RouteLayout {
    size_t keys_a, keys_b, vals_a, vals_b, hist, digit_total, counters, total;
    int64_t num_tiles;
};

RouteLayout route_layout(int64_t n) {
    RouteLayout L;
    L.num_tiles = (n + kTile - 1) / kTile;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = (off + bytes + 255) & ~(size_t)255; return at; };
    L.keys_a = take(4 * (size_t)n);
    L.keys_b = take(4 * (size_t)n);
    L.vals_a = take(4 * (size_t)n);
    L.vals_b = take(4 * (size_t)n);
    L.hist = take(4 * (size_t)kRadix * (size_t)L.num_tiles);
    L.digit_total = take(4 * kRadix);
    L.counters = take(16);
    L.total = off;
    return L;
}

__global__ void zero_counts_kernel(int64_t* counts, int world) {
    if (threadIdx.x < (unsigned)world) counts[threadIdx.x] = 0;
}

__global__ void route_init_kernel(int64_t* status, uint32_t* counters) {
    if (status) *status = -1;
    counters[0] = 0;
}

// Owner keys (sentinel `world` for an ID outside the table), request indices,
// and the per-tile owner histogram.
__global__ __launch_bounds__(kBlock) void route_keys_kernel(const int64_t* __restrict__ ids, uint32_t n,
                                                            int64_t local_rows, int world, uint32_t* __restrict__ keys,
                                                            uint32_t* __restrict__ vals, uint32_t* __restrict__ hist,
                                                            uint32_t num_tiles, int64_t* __restrict__ status) {
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
            vals[e] = e;
            atomicAdd(&s_cnt[w][key], 1u);
        }
    }
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) c += s_cnt[k][tid];
    hist[(size_t)tid * num_tiles + blockIdx.x] = c;
}

// Grouped IDs, their request positions, and the per-owner send counts.
__global__ __launch_bounds__(kBlock) void route_output_kernel(const uint32_t* __restrict__ sorted_vals,
                                                              const int64_t* __restrict__ ids, uint32_t n, int world,
                                                              const uint32_t* __restrict__ digit_total,
                                                              int64_t* __restrict__ sorted_ids,
                                                              int64_t* __restrict__ order,
                                                              int64_t* __restrict__ send_counts) {
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (blockIdx.x == 0 && threadIdx.x < (unsigned)world) send_counts[threadIdx.x] = digit_total[threadIdx.x];
    if (i >= n) return;
    const uint32_t v = min(sorted_vals[i], n - 1);
    sorted_ids[i] = ids[v];
    order[i] = v;
}

// Exclusive prefix of up to 255 int64 counts into LDS (offs[0..world]);
// returns false (and leaves the block consistent) if any count is negative.
__device__ bool load_segment_offsets(const int64_t* counts, int world, int64_t* offs) {
    __shared__ int s_bad;
    if (threadIdx.x == 0) {
        int64_t acc = 0;
        int bad = 0;
        for (int w = 0; w < world; ++w) {
            const int64_t c = counts[w];
            if (c < 0) bad = 1;
            offs[w] = acc;
            acc += c < 0 ? 0 : c;
        }
        offs[world] = acc;
        s_bad = bad;
    }
    __syncthreads();
    return s_bad == 0;
}

__device__ __forceinline__ int segment_of(const int64_t* offs, int world, int64_t i) {
    int lo = 0, hi = world;  // offs[lo] <= i < offs[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= i) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(kBlock) void route_validate_kernel(const int64_t* __restrict__ sorted_ids, int64_t n,
                                                                const int64_t* __restrict__ send_counts, int world,
                                                                int64_t local_rows, int64_t* __restrict__ status) {
    __shared__ int64_t offs[kMaxWorld + 1];
    const bool ok = load_segment_offsets(send_counts, world, offs);
    if (!ok || offs[world] > n) {
        if (blockIdx.x == 0 && threadIdx.x == 0) report_bad(status, n);
        return;
    }
    const int64_t total = offs[world];
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBlock) {
        const int w = segment_of(offs, world, i);
        const int64_t id = sorted_ids[i];
        if (id < (int64_t)w * local_rows || id >= ((int64_t)w + 1) * local_rows) report_bad(status, i);
    }
}

// Copy unit: 16 bytes when rows allow it, else 4 bytes.
template <typename U>
__global__ __launch_bounds__(kBlock) void pack_kernel(const U* __restrict__ src, int64_t row_units,
                                                      const int64_t* __restrict__ counts, int world, int64_t capacity,
                                                      U fill, U* __restrict__ dst, int64_t* __restrict__ status) {
    __shared__ int64_t offs[kMaxWorld + 1];
    const bool ok = load_segment_offsets(counts, world, offs);
    const int64_t total_units = (int64_t)world * capacity * row_units;
    if (blockIdx.x == 0 && threadIdx.x < (unsigned)world) {
        const int64_t c = counts[threadIdx.x];
        if (c < 0 || c > capacity) report_bad(status, threadIdx.x);
    }
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < total_units; e += (int64_t)gridDim.x * kBlock) {
        const int64_t row = e / row_units, k = e - row * row_units;
        const int w = (int)(row / capacity);
        const int64_t s = row - (int64_t)w * capacity;
        const int64_t c = counts[w];
        U v = fill;
        if (ok && s < c) v = src[(offs[w] + s) * row_units + k];
        dst[e] = v;
    }
}

template <typename U>
__global__ __launch_bounds__(kBlock) void unpack_kernel(const U* __restrict__ src, int64_t row_units,
                                                        const int64_t* __restrict__ counts, int world, int64_t capacity,
                                                        U* __restrict__ dst, int64_t dst_rows,
                                                        int64_t* __restrict__ status) {
    __shared__ int64_t offs[kMaxWorld + 1];
    const bool ok = load_segment_offsets(counts, world, offs);
    if (blockIdx.x == 0 && threadIdx.x <= (unsigned)world) {
        if (threadIdx.x < (unsigned)world) {
            const int64_t c = counts[threadIdx.x];
            if (c < 0 || c > capacity) report_bad(status, threadIdx.x);
        } else if (ok && offs[world] > dst_rows) {
            report_bad(status, world);
        }
    }
    if (!ok) return;
    const int64_t total_units = min(offs[world], dst_rows) * row_units;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < total_units; e += (int64_t)gridDim.x * kBlock) {
        const int64_t i = e / row_units, k = e - i * row_units;
        const int w = segment_of(offs, world, i);
        const int64_t s = i - offs[w];
        if (s < capacity) dst[e] = src[((int64_t)w * capacity + s) * row_units + k];
    }
}

// dst[i] = src[order[i]] (gather) or dst[order[i]] = src[i] (scatter); an
// index outside [0, n) is skipped.
template <typename U, bool GATHER>
__global__ __launch_bounds__(kBlock) void permute_kernel(const U* __restrict__ src, int64_t row_units,
                                                         const int64_t* __restrict__ order, int64_t n,
                                                         U* __restrict__ dst) {
    const int64_t total = n * row_units;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < total; e += (int64_t)gridDim.x * kBlock) {
        const int64_t i = e / row_units, k = e - i * row_units;
        const int64_t o = order[i];
        if ((uint64_t)o >= (uint64_t)n) continue;
        if (GATHER)
            dst[e] = src[o * row_units + k];
        else
            dst[o * row_units + k] = src[e];
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
    hipLaunchKernelGGL(route_init_kernel, dim3(1), dim3(1), 0, stream, status, counters);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (n == 0) {  // no lookups: every send count is zero
        hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(kBlock), 0, stream, send_counts, world);
        return hipGetLastError();
    }
    const uint32_t nn = (uint32_t)n, tiles = (uint32_t)L.num_tiles;
    uint32_t* hist = (uint32_t*)(ws + L.hist);
    uint32_t* digit_total = (uint32_t*)(ws + L.digit_total);
    uint32_t *ka = (uint32_t*)(ws + L.keys_a), *kb = (uint32_t*)(ws + L.keys_b);
    uint32_t *va = (uint32_t*)(ws + L.vals_a), *vb = (uint32_t*)(ws + L.vals_b);
    hipLaunchKernelGGL(route_keys_kernel, dim3(tiles), dim3(kBlock), 0, stream, ids, nn, local_rows, world, ka, va,
                       hist, tiles, status);
    hipLaunchKernelGGL(digit_scan_kernel, dim3(kRadix), dim3(kBlock), 0, stream, hist, tiles, digit_total);
    hipLaunchKernelGGL(downsweep_kernel, dim3(tiles), dim3(kBlock), 0, stream, ka, va, kb, vb, nn, 0, hist,
                       digit_total, tiles);
    hipLaunchKernelGGL(route_output_kernel, dim3((nn + kBlock - 1) / kBlock), dim3(kBlock), 0, stream, vb, ids, nn,
                       world, digit_total, sorted_ids, order, send_counts);
    return hipGetLastError();
}

hipError_t launch_route_validate(const int64_t* sorted_ids, int64_t n, const int64_t* send_counts, int world,
                                 int64_t local_rows, int64_t* status, hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_validate_kernel, dim3(grid_for(n)), dim3(kBlock), 0, stream, sorted_ids, n, send_counts,
                       world, local_rows, status);
    return hipGetLastError();
}

hipError_t launch_pack(const void* src, int64_t row_bytes, const int64_t* counts, int world, int64_t capacity,
                       const uint32_t fill16[4], void* dst, int64_t* status, hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess) return err;
    const bool wide = row_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0;
    if (wide) {
        const int64_t units = row_bytes / 16;
        const u32x4 f = {fill16[0], fill16[1], fill16[2], fill16[3]};
        hipLaunchKernelGGL((pack_kernel<u32x4>), dim3(grid_for((int64_t)world * capacity * units)), dim3(kBlock), 0,
                           stream, (const u32x4*)src, units, counts, world, capacity, f, (u32x4*)dst, status);
    } else {
        const int64_t units = row_bytes / 4;
        hipLaunchKernelGGL((pack_kernel<uint32_t>), dim3(grid_for((int64_t)world * capacity * units)), dim3(kBlock),
                           0, stream, (const uint32_t*)src, units, counts, world, capacity, fill16[0],
                           (uint32_t*)dst, status);
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const void* src, int64_t row_bytes, const int64_t* counts, int world, int64_t capacity,
                         void* dst, int64_t dst_rows, int64_t* status, hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess) return err;
    const int64_t max_rows = dst_rows < (int64_t)world * capacity ? dst_rows : (int64_t)world * capacity;
    const bool wide = row_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0;
    if (wide) {
        const int64_t units = row_bytes / 16;
        hipLaunchKernelGGL((unpack_kernel<u32x4>), dim3(grid_for(max_rows * units)), dim3(kBlock), 0, stream,
                           (const u32x4*)src, units, counts, world, capacity, (u32x4*)dst, dst_rows, status);
    } else {
        const int64_t units = row_bytes / 4;
        hipLaunchKernelGGL((unpack_kernel<uint32_t>), dim3(grid_for(max_rows * units)), dim3(kBlock), 0, stream,
                           (const uint32_t*)src, units, counts, world, capacity, (uint32_t*)dst, dst_rows, status);
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
        hipLaunchKernelGGL((permute_kernel<u32x4, true>), grid, block, 0, stream, (const u32x4*)src, units, order, n,
                           (u32x4*)dst);
    else if (wide)
        hipLaunchKernelGGL((permute_kernel<u32x4, false>), grid, block, 0, stream, (const u32x4*)src, units, order, n,
                           (u32x4*)dst);
    else if (gather)
        hipLaunchKernelGGL((permute_kernel<uint32_t, true>), grid, block, 0, stream, (const uint32_t*)src, units,
                           order, n, (uint32_t*)dst);
    else
        hipLaunchKernelGGL((permute_kernel<uint32_t, false>), grid, block, 0, stream, (const uint32_t*)src, units,
                           order, n, (uint32_t*)dst);
    return hipGetLastError();
}

}  // namespace engram
