// Internal declarations shared by the kernels and the C-ABI layer of libengram.
// Not installed; the public interface is include/engram.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace engram {

constexpr int kMaxNgram = 8;
constexpr int kMaxHeads = 64;

// Hash parameters passed by value as a kernel argument (1.6 KB, read through
// the scalar cache).  magic[h] = floor(2^64 / mod[h]) drives a Barrett
// reduction: for v < 2^63 and 2 <= p <= 2^62, q = umulhi(v, magic) is
// floor(v / p) or one less, so v - q*p needs at most one correction.
struct HashParams {
    int64_t eos;
    int64_t fill;
    int64_t mult[kMaxNgram];
    uint64_t mod[kMaxHeads];
    uint64_t magic[kMaxHeads];
    int64_t off[kMaxHeads];
    int32_t ngram_size;
    int32_t heads_per_ngram;
};

// 16-byte vector used for every bulk copy (one dwordx4 per lane).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

hipError_t launch_hash(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                       int64_t seq_end, const HashParams& p, int64_t* rows_out, hipStream_t stream);

hipError_t launch_gather(const void* table, int elem_bytes, int64_t row_begin, int64_t num_rows, int dim,
                         const int64_t* rows, int64_t n, void* out, int64_t* status, hipStream_t stream);

size_t scatter_workspace_bytes(int64_t n, int64_t num_rows, int dim);

// Backward phase 1: sort the lookups by row, count the runs, optionally write
// the distinct rows; the plan stays in the workspace.
hipError_t launch_scatter_plan(const int64_t* rows, int64_t n, int64_t row_begin, int64_t num_rows, int dim,
                               int64_t* uniq_rows, int64_t* num_uniq, void* workspace, int64_t* status,
                               hipStream_t stream);

// Backward phase 2: per-row fp64 sums of grad_out along a plan.
hipError_t launch_scatter_apply(const void* grad_out, int elem_bytes, int dim, int64_t n, int64_t num_rows,
                                float* grad_dense, float* uniq_grad, const void* workspace, hipStream_t stream);

// Owner routing (route.hip).
size_t route_workspace_bytes(int64_t n);
hipError_t launch_route_plan(const int64_t* ids, int64_t n, int64_t local_rows, int world, int64_t* sorted_ids,
                             int64_t* order, int64_t* send_counts, void* workspace, int64_t* status,
                             hipStream_t stream);
hipError_t launch_route_validate(const int64_t* sorted_ids, int64_t n, const int64_t* send_counts, int world,
                                 int64_t local_rows, int64_t* status, hipStream_t stream);
hipError_t launch_pack(const void* src, int64_t src_rows, int64_t row_bytes, const int64_t* counts, int world,
                       int64_t capacity, const uint32_t fill16[4], void* dst, int64_t* status, hipStream_t stream);
hipError_t launch_unpack(const void* src, int64_t row_bytes, const int64_t* counts, int world, int64_t capacity,
                         void* dst, int64_t dst_rows, int64_t* status, hipStream_t stream);
hipError_t launch_permute(const void* src, int64_t row_bytes, const int64_t* order, int64_t n, void* dst, bool gather,
                          hipStream_t stream);

// PLE short convolution and grouped RMSNorm (ple.hip).
size_t short_conv_workspace_bytes(int64_t batch, int64_t seq, int64_t channels, int kernel);
size_t rms_norm_workspace_bytes(int64_t rows, int64_t hidden);
bool rms_norm_group_ok(int elem_bytes, int64_t group);
hipError_t launch_short_conv(const void* x, int elem_bytes, int64_t B, int64_t S, int64_t C, const float* w,
                             const float* bias, int K, int d, const void* halo, void* y, hipStream_t stream);
hipError_t launch_short_conv_backward(const void* x, const void* dy, int elem_bytes, int64_t B, int64_t S, int64_t C,
                                      const float* w, int K, int d, const void* halo, void* dx, float* dw, float* db,
                                      void* dhalo, void* workspace, hipStream_t stream);
hipError_t launch_rms_norm(const void* x, int elem_bytes, int64_t rows, int64_t hidden, int64_t group, const float* w,
                           float eps, void* y, hipStream_t stream);
hipError_t launch_rms_norm_backward(const void* x, const void* dy, int elem_bytes, int64_t rows, int64_t hidden,
                                    int64_t group, const float* w, float eps, void* dx, float* dw, void* workspace,
                                    hipStream_t stream);

// Sets *status = -1 on the stream (a kernel, not a memset, so the call can be
// captured in a graph).
hipError_t launch_status_init(int64_t* status, hipStream_t stream);

}  // namespace engram
