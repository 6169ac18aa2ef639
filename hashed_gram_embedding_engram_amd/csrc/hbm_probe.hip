// HBM ceilings of the machine the benchmark runs on: four plain kernels whose
// achieved bandwidth bounds what the lookup path's kernels can reach.  Built
// into its own library (libengram_probe.so), used by the benchmark only.
//   read     streaming 16-byte loads of a buffer (nothing written)
//   write    streaming 16-byte non-temporal stores
//   gather   the forward gather's traffic: 16 rows of 320 bytes per wave read
//            at positions given by an index array, written consecutively
//   expand   the backward's traffic: bf16 rows of 320 bytes read at indexed
//            positions, written as fp32 rows of 640 bytes; each wave stages its
//            16 output rows in LDS so that every store instruction writes 1 KiB
//   rmw      the dense backward's traffic: each of a set of distinct fp32 rows
//            of 640 bytes, at random places in a large array, gets the sum of
//            kRmwReads random bf16 rows of 320 bytes added to it (read,
//            add, write back); 16 rows per wave
// Every kernel strides over its work with a fixed grid.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBlock = 256;
constexpr int kRowChunks = 20;  // 16-byte chunks in a 320-byte row

__global__ __launch_bounds__(kBlock) void read_kernel(const u32x4* __restrict__ src, uint64_t n,
                                                      u32x4* __restrict__ sink) {
    constexpr int K = 8;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const uint64_t stride = (uint64_t)gridDim.x * kBlock * K;
    for (uint64_t e0 = (uint64_t)blockIdx.x * kBlock * K + threadIdx.x; e0 < n; e0 += stride) {
        u32x4 v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint64_t e = e0 + (uint64_t)k * kBlock;
            v[k] = e < n ? src[e] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < K; ++k) acc ^= v[k];
    }
    // Every lane's loads stay live: the block's XOR of everything it read is
    // stored, one 16-byte word per block (the words of all blocks XOR to the
    // XOR of the whole buffer).
    __shared__ u32x4 s_part[kBlock / 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        acc.x ^= __shfl_xor(acc.x, o, 64);
        acc.y ^= __shfl_xor(acc.y, o, 64);
        acc.z ^= __shfl_xor(acc.z, o, 64);
        acc.w ^= __shfl_xor(acc.w, o, 64);
    }
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        u32x4 b = s_part[0];
#pragma unroll
        for (int w = 1; w < kBlock / 64; ++w) b ^= s_part[w];
        sink[blockIdx.x] = b;
    }
}

__global__ __launch_bounds__(kBlock) void write_kernel(u32x4* __restrict__ dst, uint64_t n, uint32_t value) {
    constexpr int K = 8;
    const u32x4 v = {value, value, value, value};
    const uint64_t stride = (uint64_t)gridDim.x * kBlock * K;
    for (uint64_t e0 = (uint64_t)blockIdx.x * kBlock * K + threadIdx.x; e0 < n; e0 += stride) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint64_t e = e0 + (uint64_t)k * kBlock;
            if (e < n) __builtin_nontemporal_store(v, dst + e);
        }
    }
}

// Output row r (of `rows`) takes input row idx[r]; 16 rows per wave.
__global__ __launch_bounds__(kBlock) void gather_kernel(const u32x4* __restrict__ src, const uint32_t* __restrict__ idx,
                                                        uint64_t rows, u32x4* __restrict__ dst) {
    const int lane = threadIdx.x & 63;
    const uint64_t waves = (uint64_t)gridDim.x * (kBlock / 64);
    for (uint64_t t = (uint64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6); t * 16 < rows; t += waves) {
        const uint64_t r0 = t * 16;
        const uint32_t mine = lane < 16 && r0 + lane < rows ? idx[r0 + lane] : 0u;
        u32x4 x[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int c = lane + 64 * j, k = c / kRowChunks, q = c % kRowChunks;
            const uint32_t row = __shfl(mine, k, 64);
            x[j] = r0 + k < rows ? src[(uint64_t)row * kRowChunks + q] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int c = lane + 64 * j;
            if (r0 + c / kRowChunks < rows) __builtin_nontemporal_store(x[j], dst + r0 * kRowChunks + c);
        }
    }
}

__global__ __launch_bounds__(kBlock) void expand_kernel(const u32x4* __restrict__ src, const uint32_t* __restrict__ idx,
                                                        uint64_t rows, u32x4* __restrict__ dst) {
    __shared__ u32x4 s_out[kBlock / 64][2 * 5 * 64];
    const int lane = threadIdx.x & 63;
    u32x4* so = s_out[threadIdx.x >> 6];
    const uint64_t waves = (uint64_t)gridDim.x * (kBlock / 64);
    for (uint64_t t = (uint64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6); t * 16 < rows; t += waves) {
        const uint64_t r0 = t * 16;
        const uint32_t mine = lane < 16 && r0 + lane < rows ? idx[r0 + lane] : 0u;
        u32x4 x[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int c = lane + 64 * j, k = c / kRowChunks, q = c % kRowChunks;
            const uint32_t row = __shfl(mine, k, 64);
            x[j] = r0 + k < rows ? src[(uint64_t)row * kRowChunks + q] : u32x4{0u, 0u, 0u, 0u};
        }
        // bf16 chunk c (8 values) -> fp32 chunks 2c and 2c + 1 of the tile
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int c = lane + 64 * j;
            so[2 * c] = u32x4{x[j][0] << 16, x[j][0] & 0xFFFF0000u, x[j][1] << 16, x[j][1] & 0xFFFF0000u};
            so[2 * c + 1] = u32x4{x[j][2] << 16, x[j][2] & 0xFFFF0000u, x[j][3] << 16, x[j][3] & 0xFFFF0000u};
        }
        // other lanes' LDS writes are read below: order them at wavefront scope
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int m = 0; m < 10; ++m) {
            const int f = lane + 64 * m;  // fp32 chunk f of the tile: row f / 40
            if (r0 + f / (2 * kRowChunks) < rows) __builtin_nontemporal_store(so[f], dst + r0 * 2 * kRowChunks + f);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

constexpr int kRmwReads = 4;  // bf16 rows added into each fp32 row

// Row r of the work adds src rows idx[kRmwReads r + i] into dst row
// idx[kRmwReads rows + r].  A lane holding bf16 chunk q of a row (8 values)
// updates fp32 chunks 2q and 2q + 1 of the same row, so no data moves
// between lanes.
__global__ __launch_bounds__(kBlock) void rmw_kernel(const u32x4* __restrict__ src, const uint32_t* __restrict__ idx,
                                                     uint64_t rows, float* __restrict__ dst) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    const uint64_t waves = (uint64_t)gridDim.x * (kBlock / 64);
    const uint32_t* dst_idx = idx + (uint64_t)kRmwReads * rows;
    for (uint64_t t = (uint64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6); t * 16 < rows; t += waves) {
        const uint64_t r0 = t * 16;
        u32x4 x[5][kRmwReads];
        f32x4 old[5][2];
        f32x4* rowp[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int c = lane + 64 * j, k = c / kRowChunks, q = c % kRowChunks;
            const bool live = r0 + k < rows;
            const uint64_t r = live ? r0 + k : 0;
#pragma unroll
            for (int i = 0; i < kRmwReads; ++i) {
                const uint32_t s_row = idx[r * kRmwReads + i];
                x[j][i] = live ? src[(uint64_t)s_row * kRowChunks + q] : u32x4{0u, 0u, 0u, 0u};
            }
            rowp[j] = (f32x4*)(dst + (uint64_t)dst_idx[r] * (2 * kRowChunks * 4)) + 2 * q;
            old[j][0] = live ? rowp[j][0] : f32x4{0.f, 0.f, 0.f, 0.f};
            old[j][1] = live ? rowp[j][1] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int c = lane + 64 * j, k = c / kRowChunks;
            if (r0 + k >= rows) continue;
            f32x4 a = old[j][0], b = old[j][1];
#pragma unroll
            for (int i = 0; i < kRmwReads; ++i) {
                const u32x4 v = x[j][i];
                a += f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                           __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
                b += f32x4{__uint_as_float(v[2] << 16), __uint_as_float(v[2] & 0xFFFF0000u),
                           __uint_as_float(v[3] << 16), __uint_as_float(v[3] & 0xFFFF0000u)};
            }
            rowp[j][0] = a;
            rowp[j][1] = b;
        }
    }
}

}  // namespace

// kind 0 read (src, bytes; dst: one 16-byte word per block of the grid),
// 1 write (dst, bytes), 2 gather and 3 expand (src rows of 320 bytes, idx
// [rows] < the rows of src, dst [rows] output rows), 4 rmw (src rows of 320
// bytes; idx: 4 * count src rows, then count distinct dst rows; dst fp32 rows
// of 640 bytes).  Returns a hipError_t.
extern "C" int engram_probe(int kind, const void* src, const uint32_t* idx, uint64_t count, void* dst, int grid,
                            hipStream_t stream) {
    if (grid < 1) return (int)hipErrorInvalidValue;
    if (kind == 0)
        hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kBlock), 0, stream, (const u32x4*)src, count / 16,
                           (u32x4*)dst);
    else if (kind == 1)
        hipLaunchKernelGGL(write_kernel, dim3(grid), dim3(kBlock), 0, stream, (u32x4*)dst, count / 16, 0x3f803f80u);
    else if (kind == 2)
        hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(kBlock), 0, stream, (const u32x4*)src, idx, count,
                           (u32x4*)dst);
    else if (kind == 3)
        hipLaunchKernelGGL(expand_kernel, dim3(grid), dim3(kBlock), 0, stream, (const u32x4*)src, idx, count,
                           (u32x4*)dst);
    else if (kind == 4)
        hipLaunchKernelGGL(rmw_kernel, dim3(grid), dim3(kBlock), 0, stream, (const u32x4*)src, idx, count,
                           (float*)dst);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}
