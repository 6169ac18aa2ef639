// engram_scatter_add_noalloc: the scatter-add for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  It runs the same plan and apply kernels as
// engram_scatter_add, with the workspace taken from a fixed device array of
// this library instead of from the caller.
//
// Every GPU holds its own copy of the array, at its own address, until the
// process ends.  The host-side name `scratch` is only a stand-in for the
// symbol, never a device address: the address is looked up once per device
// with hipGetSymbolAddress (with that device current) and kept in a per-device
// table, and only that address is ever passed to a kernel.
#include <mutex>

#include "engram.h"
#include "engram_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)ENGRAM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up

// The scratch address on the current device, or nullptr when it cannot be had.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int engram_scatter_add_noalloc(const int64_t* rows, int64_t n, const void* grad_out, int32_t dtype,
                                          int32_t dim, int64_t row_begin, int64_t num_rows, float* grad_dense,
                                          int64_t* uniq_rows, float* uniq_grad, int64_t* num_uniq, int64_t* status,
                                          hipStream_t stream) {
    // Sizes the scratch cannot hold are refused before anything else is touched.
    if (n >= 0 && dim > 0 && n < ((int64_t)1 << 31) && engram_scatter_add_workspace(n, num_rows, dim) > kScratchBytes)
        return ENGRAM_EWORKSPACE;
    void* ws = scratch_on_current_device();
    if (!ws) return ENGRAM_ELAUNCH;
    // The same checks and kernels as engram_scatter_add, on the scratch array.
    return engram_scatter_add(rows, n, grad_out, dtype, dim, row_begin, num_rows, grad_dense, uniq_rows, uniq_grad,
                              num_uniq, ws, kScratchBytes, status, stream);
}
