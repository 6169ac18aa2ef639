// Owner-local row gather for gfx950: out[i] = table[rows[i] - row_begin].
//
// Engram API page ("nemo_automodel.components.models.qwen3_8_flash_next.engram"):
// Qwen3_8_FlashNextOwnerShardedEmbedding (an owner looks up only its contiguous
// rows) and Qwen3_8_FlashNextNGramEmbedding._lookup_ngram_ids (the H head rows of
// a position, concatenated).  A row outside the owned range is never read: its
// output is zero and the lowest such lookup index is reported through `status`
// (_validate_received_ids raises instead of clamping).
//
// The copy is pure HBM traffic: one random table row read and one sequential
// output row written per lookup.  A row is cut into 16-byte chunks (CPR chunks
// per row).  One wave copies G consecutive lookups, G * CPR = 64 * PER_LANE
// chunks, so each lane moves PER_LANE chunks with dwordx4 loads and stores:
//   bf16 x 160 -> CPR = 20, G = 16 (one position's 16 heads, 5,120 B out per wave)
//   fp32 x 160 -> CPR = 40, G = 8
// Each store instruction covers 1 KB of contiguous output; each load
// instruction reads 64 consecutive chunks of the wave's rows (every row is
// fully read by consecutive lanes).  Output stores are non-temporal: the
// output is not re-read by this kernel and should not evict table rows that
// repeat (hot n-grams) from L2 and the Infinity Cache.
#include <algorithm>

#include "engram_internal.h"
#include "row_copy.h"

// Build-time switch for non-temporal table loads; off, because the gather then
// ran 20% slower (repeated hot rows lose their cache hits).
#ifndef ENGRAM_GATHER_NT_LOAD
#define ENGRAM_GATHER_NT_LOAD 0
#endif

namespace engram {
namespace {

// Read by lanes that have no row to copy, so loads never need a branch.
__device__ u32x4 kZeroChunk = {0u, 0u, 0u, 0u};  // never written

__device__ __forceinline__ void report_bad(int64_t* status, int64_t idx) {
    if (status) atomicMin((unsigned long long*)status, (unsigned long long)idx);
}

// ROW32: the shard has fewer than 2^32 - 1 rows, so a local row id (or the
// out-of-range marker 0xFFFFFFFF) fits one 32-bit shuffle.
// At most four of these waves share a SIMD: amdgpu_waves_per_eu's upper bound
// makes the compiler reserve the registers of a four-wave occupancy (128
// VGPRs; the body needs about 34).  Sixteen waves per compute unit, each with
// PER_LANE 16-byte loads per lane in flight, already cover HBM latency; with
// fewer of them resident the gather alone runs faster (less cache thrashing),
// and a plan running beside it on another stream finds room to run.
template <int CPR, int G, bool ROW32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void gather_rows_kernel(
    const u32x4* __restrict__ table, int64_t row_begin, uint64_t num_rows, const int64_t* __restrict__ rows,
    int64_t n, u32x4* __restrict__ out, int64_t* __restrict__ status) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t n0 = wave * G;
    if (n0 >= n) return;

    // Lane i < G reads and checks row id n0 + i; the others fetch it by shuffle.
    const bool mine_live = lane < G && n0 + lane < n;
    uint64_t local = ~0ull;
    if (mine_live) {
        local = (uint64_t)rows[n0 + lane] - (uint64_t)row_begin;
        if (local >= num_rows) {
            report_bad(status, n0 + lane);
            local = ~0ull;
        }
    }
    copy_wave_rows<CPR, G, ROW32, ENGRAM_GATHER_NT_LOAD != 0>(table, local, n0, n, out, lane, &kZeroChunk);
}

// Any row size (multiple of 16 B, at most 64 chunks): one chunk per lane over
// the flattened output, striding by the whole grid (a launch holds fewer than
// 2^32 work-items, and n * cpr can exceed that).
__global__ __launch_bounds__(256) void gather_rows_generic_kernel(const u32x4* __restrict__ table,
                                                                  int64_t row_begin, uint64_t num_rows,
                                                                  const int64_t* __restrict__ rows, int64_t n,
                                                                  int cpr, u32x4* __restrict__ out,
                                                                  int64_t* __restrict__ status) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n * cpr; e += stride) {
        const int64_t i = e / cpr;
        const int k = (int)(e - i * cpr);
        const uint64_t local = (uint64_t)rows[i] - (uint64_t)row_begin;
        u32x4 v = (u32x4){0u, 0u, 0u, 0u};
        if (local < num_rows)
            v = table[(int64_t)local * cpr + k];
        else if (k == 0)
            report_bad(status, i);
        __builtin_nontemporal_store(v, out + e);
    }
}

__global__ void status_init_kernel(int64_t* status) { *status = -1; }

}  // namespace

hipError_t launch_status_init(int64_t* status, hipStream_t stream) {
    if (!status) return hipSuccess;
    hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(1), 0, stream, status);
    return hipGetLastError();
}

hipError_t launch_gather(const void* table, int elem_bytes, int64_t row_begin, int64_t num_rows, int dim,
                         const int64_t* rows, int64_t n, void* out, int64_t* status, hipStream_t stream) {
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess || n == 0) return err;
    const int cpr = dim * elem_bytes / 16;
    const u32x4* t = (const u32x4*)table;
    u32x4* o = (u32x4*)out;
    const int block = 256, waves_per_block = block / 64;
    const bool row32 = (uint64_t)num_rows < 0xFFFFFFFFull;
    // Work-items per launch must stay below 2^32: the one-wave-per-G-lookups
    // kernels take 64 / G per lookup (fewer lookups than fit in HBM at these
    // row sizes); the generic kernel strides over any count.
    const int64_t kMaxItems = (int64_t)1 << 31;
    const int gw = cpr == 20 ? 16 : 8;
    if ((cpr == 20 || cpr == 40) && (n + gw - 1) / gw * 64 <= kMaxItems) {
        const int g = gw;
        const int64_t waves = (n + g - 1) / g;
        const dim3 grid((unsigned)((waves + waves_per_block - 1) / waves_per_block));
        if (cpr == 20 && row32)
            hipLaunchKernelGGL((gather_rows_kernel<20, 16, true>), grid, dim3(block), 0, stream, t, row_begin,
                               (uint64_t)num_rows, rows, n, o, status);
        else if (cpr == 20)
            hipLaunchKernelGGL((gather_rows_kernel<20, 16, false>), grid, dim3(block), 0, stream, t, row_begin,
                               (uint64_t)num_rows, rows, n, o, status);
        else if (row32)
            hipLaunchKernelGGL((gather_rows_kernel<40, 8, true>), grid, dim3(block), 0, stream, t, row_begin,
                               (uint64_t)num_rows, rows, n, o, status);
        else
            hipLaunchKernelGGL((gather_rows_kernel<40, 8, false>), grid, dim3(block), 0, stream, t, row_begin,
                               (uint64_t)num_rows, rows, n, o, status);
    } else {
        const int64_t grid = std::min((n * cpr + block - 1) / block, kMaxItems / block);
        hipLaunchKernelGGL(gather_rows_generic_kernel, dim3((unsigned)grid), dim3(block), 0, stream, t,
                           row_begin, (uint64_t)num_rows, rows, n, cpr, o, status);
    }
    return hipGetLastError();
}

}  // namespace engram
