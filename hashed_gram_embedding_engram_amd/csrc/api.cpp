// C ABI of libengram (include/engram.h): argument checks, hash-spec upload as
// a kernel argument, and dispatch to the kernels.  Nothing here allocates or
// keeps state; every check that can be made on the host is made before any
// work is enqueued.
#include "engram.h"

#include "engram_internal.h"

namespace {

bool row_bytes_ok(int32_t dtype, int32_t dim, int* elem_bytes) {
    const int eb = dtype == ENGRAM_F32 ? 4 : 2;
    *elem_bytes = eb;
    if (dim <= 0) return false;
    const int64_t bytes = (int64_t)dim * eb;
    return bytes % 16 == 0 && bytes <= 1024;
}

bool dtype_ok(int32_t dtype) { return dtype == ENGRAM_F32 || dtype == ENGRAM_BF16; }

int launch_result(hipError_t e) { return e == hipSuccess ? ENGRAM_OK : ENGRAM_ELAUNCH; }

// Validates the spec and fills the kernel parameters (with Barrett reciprocals).
int build_params(const engram_hash_spec* spec, engram::HashParams* p) {
    if (!spec) return ENGRAM_EINVAL;
    if (spec->ngram_size < 2 || spec->ngram_size > ENGRAM_MAX_NGRAM) return ENGRAM_ESPEC;
    if (spec->heads_per_ngram < 1) return ENGRAM_ESPEC;
    const int64_t heads = (int64_t)(spec->ngram_size - 1) * spec->heads_per_ngram;
    if (heads > ENGRAM_MAX_HEADS) return ENGRAM_ESPEC;
    *p = engram::HashParams{};
    p->eos = spec->eos_id;
    p->fill = spec->fill_id;
    p->ngram_size = spec->ngram_size;
    p->heads_per_ngram = spec->heads_per_ngram;
    for (int k = 0; k < ENGRAM_MAX_NGRAM; ++k) p->mult[k] = spec->multipliers[k];
    for (int64_t h = 0; h < heads; ++h) {
        const int64_t m = spec->head_mod[h], o = spec->head_offset[h];
        if (m < 2 || m > ((int64_t)1 << 62)) return ENGRAM_ESPEC;
        if (o < 0 || o > INT64_MAX - (m - 1)) return ENGRAM_ESPEC;
        p->mod[h] = (uint64_t)m;
        p->magic[h] = (uint64_t)(((unsigned __int128)1 << 64) / (unsigned __int128)(uint64_t)m);
        p->off[h] = o;
    }
    return ENGRAM_OK;
}

int hash_common(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin, int64_t seq_end,
                const engram_hash_spec* spec, int64_t* rows_out, hipStream_t stream) {
    if (batch < 0 || seq_len < 0) return ENGRAM_EINVAL;
    if (seq_begin < 0 || seq_begin > seq_end || seq_end > seq_len) return ENGRAM_EINVAL;
    engram::HashParams p;
    const int rc = build_params(spec, &p);
    if (rc != ENGRAM_OK) return rc;
    const int64_t width = seq_end - seq_begin;
    if (batch == 0 || width == 0) return ENGRAM_OK;
    if (!tokens || !rows_out) return ENGRAM_EINVAL;
    if (batch > INT64_MAX / width / ENGRAM_MAX_HEADS || batch * width > ((int64_t)1 << 40)) return ENGRAM_EINVAL;
    return launch_result(engram::launch_hash(tokens, batch, seq_len, seq_begin, seq_end, p, rows_out, stream));
}

}  // namespace

extern "C" {

int engram_hash(const int64_t* tokens, int64_t batch, int64_t seq_len, const engram_hash_spec* spec,
                int64_t* rows_out, hipStream_t stream) {
    return hash_common(tokens, batch, seq_len, 0, seq_len, spec, rows_out, stream);
}

int engram_hash_slice(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin, int64_t seq_end,
                      const engram_hash_spec* spec, int64_t* rows_out, hipStream_t stream) {
    return hash_common(tokens, batch, seq_len, seq_begin, seq_end, spec, rows_out, stream);
}

int engram_gather(const void* table, int32_t dtype, int64_t row_begin, int64_t num_rows, int32_t dim,
                  const int64_t* rows, int64_t n, void* out, int64_t* status, hipStream_t stream) {
    if (!dtype_ok(dtype)) return ENGRAM_EDTYPE;
    int eb;
    if (!row_bytes_ok(dtype, dim, &eb)) return ENGRAM_EINVAL;
    if (n < 0 || num_rows < 0 || row_begin < 0) return ENGRAM_EINVAL;
    if (n > ((int64_t)1 << 40)) return ENGRAM_EINVAL;
    if (n > 0 && (!rows || !out || (num_rows > 0 && !table))) return ENGRAM_EINVAL;
    return launch_result(engram::launch_gather(table, eb, row_begin, num_rows, dim, rows, n, out, status, stream));
}

size_t engram_scatter_add_workspace(int64_t n, int64_t num_rows, int32_t dim) {
    if (n < 0 || dim <= 0) return 0;
    return engram::scatter_workspace_bytes(n, num_rows, dim);
}

namespace {

int scatter_check_common(int32_t dtype, int32_t dim, int64_t n, int64_t row_begin, int64_t num_rows, int* eb) {
    if (!dtype_ok(dtype)) return ENGRAM_EDTYPE;
    if (!row_bytes_ok(dtype, dim, eb)) return ENGRAM_EINVAL;
    if (n < 0 || n >= ((int64_t)1 << 31)) return ENGRAM_EINVAL;
    if (num_rows < 0 || num_rows >= (int64_t)0xFFFFFFFFll || row_begin < 0) return ENGRAM_EINVAL;
    return ENGRAM_OK;
}

int workspace_check(const void* workspace, size_t workspace_bytes, int64_t n, int64_t num_rows, int32_t dim) {
    if (((uintptr_t)workspace & 255) != 0) return ENGRAM_EWORKSPACE;
    if (!workspace || workspace_bytes < engram::scatter_workspace_bytes(n, num_rows, dim)) return ENGRAM_EWORKSPACE;
    return ENGRAM_OK;
}

}  // namespace

int engram_scatter_add_plan(const int64_t* rows, int64_t n, int64_t row_begin, int64_t num_rows, int32_t dim,
                            int64_t* uniq_rows, int64_t* num_uniq, void* workspace, size_t workspace_bytes,
                            int64_t* status, hipStream_t stream) {
    int eb;
    int rc = scatter_check_common(ENGRAM_F32, dim, n, row_begin, num_rows, &eb);
    if (rc != ENGRAM_OK) return rc;
    if (n > 0 && !rows) return ENGRAM_EINVAL;
    if ((rc = workspace_check(workspace, workspace_bytes, n, num_rows, dim)) != ENGRAM_OK) return rc;
    return launch_result(engram::launch_scatter_plan(rows, n, row_begin, num_rows, dim, uniq_rows, num_uniq,
                                                     workspace, status, stream));
}

int engram_scatter_add_apply(const void* grad_out, int32_t dtype, int32_t dim, int64_t n, int64_t row_begin,
                             int64_t num_rows, float* grad_dense, float* uniq_grad, const void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    int eb;
    int rc = scatter_check_common(dtype, dim, n, row_begin, num_rows, &eb);
    if (rc != ENGRAM_OK) return rc;
    if ((grad_dense != nullptr) == (uniq_grad != nullptr)) return ENGRAM_EINVAL;
    if (n > 0 && !grad_out) return ENGRAM_EINVAL;
    if ((rc = workspace_check(workspace, workspace_bytes, n, num_rows, dim)) != ENGRAM_OK) return rc;
    return launch_result(engram::launch_scatter_apply(grad_out, eb, dim, n, num_rows, grad_dense, uniq_grad,
                                                      workspace, stream));
}

int engram_scatter_add(const int64_t* rows, int64_t n, const void* grad_out, int32_t dtype, int32_t dim,
                       int64_t row_begin, int64_t num_rows, float* grad_dense, int64_t* uniq_rows, float* uniq_grad,
                       int64_t* num_uniq, void* workspace, size_t workspace_bytes, int64_t* status,
                       hipStream_t stream) {
    int eb;
    int rc = scatter_check_common(dtype, dim, n, row_begin, num_rows, &eb);
    if (rc != ENGRAM_OK) return rc;
    const bool dense = grad_dense != nullptr;
    const bool compact = uniq_rows != nullptr || uniq_grad != nullptr || num_uniq != nullptr;
    if (dense == compact) return ENGRAM_EINVAL;
    if (compact && (!uniq_rows || !uniq_grad || !num_uniq)) return ENGRAM_EINVAL;
    if (n > 0 && (!rows || !grad_out)) return ENGRAM_EINVAL;
    if ((rc = workspace_check(workspace, workspace_bytes, n, num_rows, dim)) != ENGRAM_OK) return rc;
    hipError_t e = engram::launch_scatter_plan(rows, n, row_begin, num_rows, dim, uniq_rows, num_uniq, workspace,
                                               status, stream);
    if (e != hipSuccess) return ENGRAM_ELAUNCH;
    return launch_result(engram::launch_scatter_apply(grad_out, eb, dim, n, num_rows, grad_dense, uniq_grad,
                                                      workspace, stream));
}

const char* engram_strerror(int code) {
    switch (code) {
        case ENGRAM_OK: return "success";
        case ENGRAM_EINVAL: return "invalid argument (null pointer, size out of range or unsupported row width)";
        case ENGRAM_EDTYPE: return "unsupported element type";
        case ENGRAM_EWORKSPACE: return "scatter-add workspace missing, misaligned or too small";
        case ENGRAM_ELAUNCH: return "kernel launch failed";
        case ENGRAM_ESPEC: return "hash spec out of range (ngram_size, heads, moduli or offsets)";
        default: return "unknown engram status";
    }
}

}  // extern "C"
