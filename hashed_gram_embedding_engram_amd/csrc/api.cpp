// C ABI of libengram (include/engram.h): argument checks, hash-spec upload as
// a kernel argument, and dispatch to the kernels.  Nothing here allocates or
// keeps state; every check that can be made on the host is made before any
// work is enqueued.
#include "engram.h"

#include <initializer_list>

#include "engram_internal.h"
#include "lookup.h"

namespace {

bool row_bytes_ok(int32_t dtype, int32_t dim, int* elem_bytes) {
    const int eb = dtype == ENGRAM_F32 ? 4 : 2;
    *elem_bytes = eb;
    if (dim <= 0) return false;
    const int64_t bytes = (int64_t)dim * eb;
    return bytes % 16 == 0 && bytes <= 1024;
}

bool dtype_ok(int32_t dtype) { return dtype == ENGRAM_F32 || dtype == ENGRAM_BF16; }

// Device arrays must be aligned to their access width: 16 bytes for row data
// (loaded and stored as 16-byte chunks), 8 for int64 and fp64, 4 for fp32.
// NULL passes (the callers check which pointers are required).
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

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
    // rows are stored as 16-byte pairs of int64
    if (!tokens || !rows_out || !aligned(tokens, 8) || !aligned(rows_out, 16)) return ENGRAM_EINVAL;
    // one work-item per position: a launch holds fewer than 2^32
    if (batch > INT64_MAX / width / ENGRAM_MAX_HEADS || batch * width > ((int64_t)1 << 32) - 64) return ENGRAM_EINVAL;
    return launch_result(engram::launch_hash(tokens, batch, seq_len, seq_begin, seq_end, p, rows_out, stream));
}

}  // namespace

namespace engram {
// Work-items of the largest launch a convolution call makes (ple.hip).
int64_t short_conv_launch_items(int64_t batch, int64_t seq, int64_t channels, int kernel, int dilation,
                                int elem_bytes);
// The fused routing copies (route.hip): the unpack with the move to request
// order, and the move to grouped order with the pack.
hipError_t launch_unpack_unpermute(const void* src, int64_t row_bytes, const int64_t* counts, int world,
                                  int64_t capacity, const int64_t* order, int64_t n, void* dst, int64_t* status,
                                  hipStream_t stream);
hipError_t launch_permute_pack(const void* src, int64_t row_bytes, const int64_t* order, int64_t n,
                               const int64_t* counts, int world, int64_t capacity, const uint32_t fill16[4], void* dst,
                               int64_t* status, hipStream_t stream);
hipError_t launch_gather_padded(const void* table, int elem_bytes, int64_t row_begin, int64_t num_rows, int dim,
                                const int64_t* ids, const int64_t* counts, int world, int64_t capacity, void* out,
                                int64_t* status, hipStream_t stream);
// The backward's plan for rows as the exchange delivers them (scatter.hip).
hipError_t launch_scatter_plan_padded(const int64_t* ids, const int64_t* counts, int world, int64_t capacity,
                                      int64_t row_begin, int64_t num_rows, int dim, int64_t* uniq_rows,
                                      int64_t* num_uniq, void* workspace, int64_t* status, hipStream_t stream);
}  // namespace engram

namespace {
// The fill element (1, 2, 4 or 8 bytes) repeated over 16 bytes, as four words.
void fill_words(const void* fill, int fill_bytes, uint32_t fill16[4]) {
    unsigned char bytes[16];
    for (int i = 0; i < 16; ++i) bytes[i] = ((const unsigned char*)fill)[i % fill_bytes];
    for (int i = 0; i < 4; ++i)
        fill16[i] = (uint32_t)bytes[4 * i] | ((uint32_t)bytes[4 * i + 1] << 8) | ((uint32_t)bytes[4 * i + 2] << 16) |
                    ((uint32_t)bytes[4 * i + 3] << 24);
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
    if (!aligned(table, 16) || !aligned(out, 16) || !aligned(rows, 8) || !aligned(status, 8)) return ENGRAM_EINVAL;
    return launch_result(engram::launch_gather(table, eb, row_begin, num_rows, dim, rows, n, out, status, stream));
}

namespace {
int hash_gather_common(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin, int64_t seq_end,
                       const engram_hash_spec* spec, const void* table, int32_t dtype, int64_t row_begin,
                       int64_t num_rows, int32_t dim, void* out, int64_t* rows_out, int64_t* status,
                       hipStream_t stream) {
    if (!dtype_ok(dtype)) return ENGRAM_EDTYPE;
    int eb;
    if (!row_bytes_ok(dtype, dim, &eb)) return ENGRAM_EINVAL;
    if (batch < 0 || seq_len < 0 || num_rows < 0 || row_begin < 0) return ENGRAM_EINVAL;
    if (seq_begin < 0 || seq_begin > seq_end || seq_end > seq_len) return ENGRAM_EINVAL;
    engram::HashParams p;
    const int rc = build_params(spec, &p);
    if (rc != ENGRAM_OK) return rc;
    const int64_t width = seq_end - seq_begin;
    // one hash work-item per position: a launch holds fewer than 2^32
    if (width > 0 && (batch > INT64_MAX / width / ENGRAM_MAX_HEADS || batch * width > ((int64_t)1 << 32) - 64))
        return ENGRAM_EINVAL;
    const int64_t positions = batch * width;
    if (!aligned(tokens, 8) || !aligned(table, 16) || !aligned(out, 16) || !aligned(rows_out, 16) ||
        !aligned(status, 8))
        return ENGRAM_EINVAL;
    if (positions == 0) return launch_result(engram::launch_status_init(status, stream));
    if (!tokens || !out || (num_rows > 0 && !table)) return ENGRAM_EINVAL;
    if (!rows_out && !engram::hash_gather_fused(p, eb, dim, positions)) return ENGRAM_EINVAL;
    return launch_result(engram::launch_hash_gather(tokens, batch, seq_len, seq_begin, seq_end, p, table, eb,
                                                    row_begin, num_rows, dim, out, rows_out, status, stream));
}
}  // namespace

int engram_hash_gather(const int64_t* tokens, int64_t batch, int64_t seq_len, const engram_hash_spec* spec,
                       const void* table, int32_t dtype, int64_t row_begin, int64_t num_rows, int32_t dim,
                       void* out, int64_t* rows_out, int64_t* status, hipStream_t stream) {
    return hash_gather_common(tokens, batch, seq_len, 0, seq_len, spec, table, dtype, row_begin, num_rows, dim, out,
                              rows_out, status, stream);
}

int engram_hash_gather_slice(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                             int64_t seq_end, const engram_hash_spec* spec, const void* table, int32_t dtype,
                             int64_t row_begin, int64_t num_rows, int32_t dim, void* out, int64_t* rows_out,
                             int64_t* status, hipStream_t stream) {
    return hash_gather_common(tokens, batch, seq_len, seq_begin, seq_end, spec, table, dtype, row_begin, num_rows,
                              dim, out, rows_out, status, stream);
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
    if (!aligned(rows, 8) || !aligned(uniq_rows, 8) || !aligned(num_uniq, 8) || !aligned(status, 8))
        return ENGRAM_EINVAL;
    if ((rc = workspace_check(workspace, workspace_bytes, n, num_rows, dim)) != ENGRAM_OK) return rc;
    return launch_result(engram::launch_scatter_plan(rows, n, row_begin, num_rows, dim, uniq_rows, num_uniq,
                                                     workspace, status, stream));
}

int engram_scatter_add_plan_padded(const int64_t* ids, const int64_t* split_sizes, int32_t world, int64_t capacity,
                                   int64_t row_begin, int64_t num_rows, int32_t dim, int64_t* uniq_rows,
                                   int64_t* num_uniq, void* workspace, size_t workspace_bytes, int64_t* status,
                                   hipStream_t stream) {
    if (world < 1 || world > 255 || capacity < 0 || !split_sizes) return ENGRAM_EINVAL;
    if (capacity > ((int64_t)1 << 31) / world) return ENGRAM_EINVAL;
    const int64_t n = (int64_t)world * capacity;
    int eb;
    int rc = scatter_check_common(ENGRAM_F32, dim, n, row_begin, num_rows, &eb);
    if (rc != ENGRAM_OK) return rc;
    if (n > 0 && !ids) return ENGRAM_EINVAL;
    if (!aligned(ids, 8) || !aligned(split_sizes, 8) || !aligned(uniq_rows, 8) || !aligned(num_uniq, 8) ||
        !aligned(status, 8))
        return ENGRAM_EINVAL;
    if ((rc = workspace_check(workspace, workspace_bytes, n, num_rows, dim)) != ENGRAM_OK) return rc;
    return launch_result(engram::launch_scatter_plan_padded(ids, split_sizes, world, capacity, row_begin, num_rows,
                                                            dim, uniq_rows, num_uniq, workspace, status, stream));
}

namespace {

static int plan_from_tokens_common(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                            int64_t seq_end, const engram_hash_spec* spec, int64_t row_begin, int64_t num_rows,
                            int32_t dim, int64_t* uniq_rows, int64_t* num_uniq, void* workspace,
                            size_t workspace_bytes, int64_t* status, hipStream_t stream) {
    if (batch < 0 || seq_len < 0 || seq_begin < 0 || seq_end < seq_begin || seq_end > seq_len) return ENGRAM_EINVAL;
    if (seq_len >= ((int64_t)1 << 32)) return ENGRAM_EINVAL;
    engram::HashParams p;
    int rc = build_params(spec, &p);
    if (rc != ENGRAM_OK) return rc;
    if (p.ngram_size != 3 || p.heads_per_ngram != 8) return ENGRAM_EINVAL;  // 16 rows per position only
    const int64_t width = seq_end - seq_begin;
    if (width > 0 && batch > (((int64_t)1 << 31) - 1) / 16 / width) return ENGRAM_EINVAL;
    const int64_t n = batch * width * 16;
    int eb;
    if ((rc = scatter_check_common(ENGRAM_F32, dim, n, row_begin, num_rows, &eb)) != ENGRAM_OK) return rc;
    if (n > 0 && !tokens) return ENGRAM_EINVAL;
    if (!aligned(tokens, 8) || !aligned(uniq_rows, 8) || !aligned(num_uniq, 8) || !aligned(status, 8))
        return ENGRAM_EINVAL;
    if ((rc = workspace_check(workspace, workspace_bytes, n, num_rows, dim)) != ENGRAM_OK) return rc;
    return launch_result(engram::launch_scatter_plan_tokens(tokens, batch, seq_len, seq_begin, seq_end, p,
                                                            row_begin, num_rows, dim, uniq_rows, num_uniq,
                                                            workspace, status, stream));
}

}  // namespace

int engram_scatter_add_plan_from_tokens(const int64_t* tokens, int64_t batch, int64_t seq_len,
                                        const engram_hash_spec* spec, int64_t row_begin, int64_t num_rows, int32_t dim,
                                        int64_t* uniq_rows, int64_t* num_uniq, void* workspace,
                                        size_t workspace_bytes, int64_t* status, hipStream_t stream) {
    return plan_from_tokens_common(tokens, batch, seq_len, 0, seq_len, spec, row_begin, num_rows, dim, uniq_rows,
                                   num_uniq, workspace, workspace_bytes, status, stream);
}

int engram_scatter_add_plan_from_tokens_slice(const int64_t* tokens, int64_t batch, int64_t seq_len,
                                              int64_t seq_begin, int64_t seq_end, const engram_hash_spec* spec,
                                              int64_t row_begin, int64_t num_rows, int32_t dim, int64_t* uniq_rows,
                                              int64_t* num_uniq, void* workspace, size_t workspace_bytes,
                                              int64_t* status, hipStream_t stream) {
    return plan_from_tokens_common(tokens, batch, seq_len, seq_begin, seq_end, spec, row_begin, num_rows, dim,
                                   uniq_rows, num_uniq, workspace, workspace_bytes, status, stream);
}

int engram_scatter_add_apply(const void* grad_out, int32_t dtype, int32_t dim, int64_t n, int64_t row_begin,
                             int64_t num_rows, float* grad_dense, float* uniq_grad, const void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    int eb;
    int rc = scatter_check_common(dtype, dim, n, row_begin, num_rows, &eb);
    if (rc != ENGRAM_OK) return rc;
    if ((grad_dense != nullptr) == (uniq_grad != nullptr)) return ENGRAM_EINVAL;
    if (n > 0 && !grad_out) return ENGRAM_EINVAL;
    if (!aligned(grad_out, 16) || !aligned(grad_dense, 16) || !aligned(uniq_grad, 16)) return ENGRAM_EINVAL;
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
    if (!aligned(rows, 8) || !aligned(grad_out, 16) || !aligned(grad_dense, 16) || !aligned(uniq_grad, 16) ||
        !aligned(uniq_rows, 8) || !aligned(num_uniq, 8) || !aligned(status, 8))
        return ENGRAM_EINVAL;
    if ((rc = workspace_check(workspace, workspace_bytes, n, num_rows, dim)) != ENGRAM_OK) return rc;
    hipError_t e = engram::launch_scatter_plan(rows, n, row_begin, num_rows, dim, uniq_rows, num_uniq, workspace,
                                               status, stream);
    if (e != hipSuccess) return ENGRAM_ELAUNCH;
    return launch_result(engram::launch_scatter_apply(grad_out, eb, dim, n, num_rows, grad_dense, uniq_grad,
                                                      workspace, stream));
}

size_t engram_route_workspace(int64_t n) { return n < 0 ? 0 : engram::route_workspace_bytes(n); }

namespace {

int route_geometry(int64_t num_embeddings, int32_t world, int64_t* local_rows) {
    if (world < 1 || world > 255 || num_embeddings < 1 || num_embeddings % world != 0) return ENGRAM_EINVAL;
    *local_rows = num_embeddings / world;
    return ENGRAM_OK;
}

bool row_layout_ok(int64_t row_bytes) { return row_bytes > 0 && row_bytes % 4 == 0 && row_bytes <= (1 << 20); }

}  // namespace

int engram_route_plan(const int64_t* global_ids, int64_t n, int64_t num_embeddings, int32_t world,
                      int64_t* sorted_ids, int64_t* order, int64_t* send_counts, void* workspace,
                      size_t workspace_bytes, int64_t* status, hipStream_t stream) {
    int64_t local_rows;
    if (route_geometry(num_embeddings, world, &local_rows) != ENGRAM_OK) return ENGRAM_EINVAL;
    if (n < 0 || n >= ((int64_t)1 << 31) || !send_counts) return ENGRAM_EINVAL;
    if (n > 0 && (!global_ids || !sorted_ids || !order)) return ENGRAM_EINVAL;
    if (!aligned(global_ids, 8) || !aligned(sorted_ids, 8) || !aligned(order, 8) || !aligned(send_counts, 8) ||
        !aligned(status, 8))
        return ENGRAM_EINVAL;
    if (((uintptr_t)workspace & 255) != 0 || !workspace || workspace_bytes < engram::route_workspace_bytes(n))
        return ENGRAM_EWORKSPACE;
    return launch_result(engram::launch_route_plan(global_ids, n, local_rows, world, sorted_ids, order, send_counts,
                                                   workspace, status, stream));
}

int engram_route_validate(const int64_t* sorted_ids, int64_t n, const int64_t* send_counts, int32_t world,
                          int64_t num_embeddings, int64_t* status, hipStream_t stream) {
    int64_t local_rows;
    if (route_geometry(num_embeddings, world, &local_rows) != ENGRAM_OK) return ENGRAM_EINVAL;
    if (n < 0 || !send_counts || !status || (n > 0 && !sorted_ids)) return ENGRAM_EINVAL;
    if (!aligned(sorted_ids, 8) || !aligned(send_counts, 8) || !aligned(status, 8)) return ENGRAM_EINVAL;
    return launch_result(engram::launch_route_validate(sorted_ids, n, send_counts, world, local_rows, status, stream));
}

int engram_pack_fixed_capacity(const void* src, int64_t src_rows, int64_t row_bytes, const int64_t* split_sizes,
                               int32_t world, int64_t capacity, const void* fill, int32_t fill_bytes, void* dst,
                               int64_t* status, hipStream_t stream) {
    if (world < 1 || world > 255 || capacity < 0 || src_rows < 0 || !row_layout_ok(row_bytes) || !split_sizes)
        return ENGRAM_EINVAL;
    if (!(fill_bytes == 1 || fill_bytes == 2 || fill_bytes == 4 || fill_bytes == 8) || !fill) return ENGRAM_EINVAL;
    if (row_bytes % fill_bytes != 0) return ENGRAM_EINVAL;
    if (capacity > 0 && (!dst || (src_rows > 0 && !src))) return ENGRAM_EINVAL;
    if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(split_sizes, 8) || !aligned(status, 8)) return ENGRAM_EINVAL;
    if ((int64_t)world * capacity > ((int64_t)1 << 40) / row_bytes || src_rows > ((int64_t)1 << 40) / row_bytes)
        return ENGRAM_EINVAL;
    uint32_t fill16[4];
    fill_words(fill, fill_bytes, fill16);
    return launch_result(
        engram::launch_pack(src, src_rows, row_bytes, split_sizes, world, capacity, fill16, dst, status, stream));
}

int engram_permute_pack_rows(const void* src, int64_t row_bytes, const int64_t* order, int64_t n,
                             const int64_t* split_sizes, int32_t world, int64_t capacity, const void* fill,
                             int32_t fill_bytes, void* dst, int64_t* status, hipStream_t stream) {
    if (world < 1 || world > 255 || capacity < 0 || n < 0 || !row_layout_ok(row_bytes) || !split_sizes)
        return ENGRAM_EINVAL;
    if (!(fill_bytes == 1 || fill_bytes == 2 || fill_bytes == 4 || fill_bytes == 8) || !fill) return ENGRAM_EINVAL;
    if (row_bytes % fill_bytes != 0) return ENGRAM_EINVAL;
    if (capacity > 0 && (!dst || (n > 0 && (!src || !order)))) return ENGRAM_EINVAL;
    if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(order, 8) || !aligned(split_sizes, 8) || !aligned(status, 8))
        return ENGRAM_EINVAL;
    if ((int64_t)world * capacity > ((int64_t)1 << 40) / row_bytes || n > ((int64_t)1 << 40) / row_bytes)
        return ENGRAM_EINVAL;
    uint32_t fill16[4];
    fill_words(fill, fill_bytes, fill16);
    return launch_result(engram::launch_permute_pack(src, row_bytes, order, n, split_sizes, world, capacity, fill16,
                                                     dst, status, stream));
}

int engram_unpack_fixed_capacity(const void* src, int64_t row_bytes, const int64_t* split_sizes, int32_t world,
                                 int64_t capacity, void* dst, int64_t dst_rows, int64_t* status, hipStream_t stream) {
    if (world < 1 || world > 255 || capacity < 0 || dst_rows < 0 || !row_layout_ok(row_bytes) || !split_sizes)
        return ENGRAM_EINVAL;
    if (capacity > 0 && dst_rows > 0 && (!dst || !src)) return ENGRAM_EINVAL;
    if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(split_sizes, 8) || !aligned(status, 8)) return ENGRAM_EINVAL;
    if ((int64_t)world * capacity > ((int64_t)1 << 40) / row_bytes || dst_rows > ((int64_t)1 << 40) / row_bytes)
        return ENGRAM_EINVAL;
    return launch_result(engram::launch_unpack(src, row_bytes, split_sizes, world, capacity, dst, dst_rows, status,
                                               stream));
}

int engram_unpack_unpermute_rows(const void* src, int64_t row_bytes, const int64_t* split_sizes, int32_t world,
                                 int64_t capacity, const int64_t* order, int64_t n, void* dst, int64_t* status,
                                 hipStream_t stream) {
    if (world < 1 || world > 255 || capacity < 0 || n < 0 || !row_layout_ok(row_bytes) || !split_sizes)
        return ENGRAM_EINVAL;
    if (capacity > 0 && n > 0 && (!dst || !src || !order)) return ENGRAM_EINVAL;
    if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(order, 8) || !aligned(split_sizes, 8) || !aligned(status, 8))
        return ENGRAM_EINVAL;
    if ((int64_t)world * capacity > ((int64_t)1 << 40) / row_bytes || n > ((int64_t)1 << 40) / row_bytes)
        return ENGRAM_EINVAL;
    return launch_result(engram::launch_unpack_unpermute(src, row_bytes, split_sizes, world, capacity, order, n, dst,
                                                         status, stream));
}

int engram_gather_padded(const void* table, int32_t dtype, int64_t row_begin, int64_t num_rows, int32_t dim,
                         const int64_t* ids, const int64_t* split_sizes, int32_t world, int64_t capacity, void* out,
                         int64_t* status, hipStream_t stream) {
    if (!dtype_ok(dtype)) return ENGRAM_EDTYPE;
    int eb;
    if (!row_bytes_ok(dtype, dim, &eb)) return ENGRAM_EINVAL;
    if (world < 1 || world > 255 || capacity < 0 || num_rows < 0 || row_begin < 0 || !split_sizes)
        return ENGRAM_EINVAL;
    if (capacity > ((int64_t)1 << 40) / world) return ENGRAM_EINVAL;
    if (capacity > 0 && (!ids || !out || (num_rows > 0 && !table))) return ENGRAM_EINVAL;
    if (!aligned(table, 16) || !aligned(out, 16) || !aligned(ids, 8) || !aligned(split_sizes, 8) ||
        !aligned(status, 8))
        return ENGRAM_EINVAL;
    return launch_result(engram::launch_gather_padded(table, eb, row_begin, num_rows, dim, ids, split_sizes, world,
                                                      capacity, out, status, stream));
}

int engram_permute_rows(const void* src, int64_t row_bytes, const int64_t* order, int64_t n, void* dst,
                        hipStream_t stream) {
    if (n < 0 || !row_layout_ok(row_bytes) || (n > 0 && (!src || !order || !dst))) return ENGRAM_EINVAL;
    if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(order, 8) || n > ((int64_t)1 << 40) / row_bytes)
        return ENGRAM_EINVAL;
    return launch_result(engram::launch_permute(src, row_bytes, order, n, dst, true, stream));
}

int engram_unpermute_rows(const void* src, int64_t row_bytes, const int64_t* order, int64_t n, void* dst,
                          hipStream_t stream) {
    if (n < 0 || !row_layout_ok(row_bytes) || (n > 0 && (!src || !order || !dst))) return ENGRAM_EINVAL;
    if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(order, 8) || n > ((int64_t)1 << 40) / row_bytes)
        return ENGRAM_EINVAL;
    return launch_result(engram::launch_permute(src, row_bytes, order, n, dst, false, stream));
}

namespace {

// Sizes of a PLE call over a x b rows of `channels` features: every row a
// whole number of 16-byte chunks, at most 2^26 features per row and 2^36
// elements in all (137 GB of bf16 per tensor).  A convolution call also
// needs each of its launches below kConvLaunchItems work-items, which short
// sequences over many batch rows can reach first.
constexpr int64_t kConvLaunchItems = (int64_t)1 << 32;
int ple_dims_ok(int32_t dtype, int64_t a, int64_t b, int64_t channels, int* eb) {
    if (!dtype_ok(dtype)) return ENGRAM_EDTYPE;
    *eb = dtype == ENGRAM_F32 ? 4 : 2;
    if (a < 0 || b < 0 || channels <= 0 || channels > ((int64_t)1 << 26) || (channels * *eb) % 16 != 0)
        return ENGRAM_EINVAL;
    if (a > 0 && b > 0 && (b > ((int64_t)1 << 36) / a || a * b > ((int64_t)1 << 36) / channels)) return ENGRAM_EINVAL;
    return ENGRAM_OK;
}

// The norm runs one wave per (row, group): rows x groups at most 2^25 keeps
// its launches below 2^31 work-items.
bool norm_groups_ok(int64_t rows, int64_t hidden, int64_t group) {
    return rows <= (((int64_t)1 << 25) / (hidden / group));
}

bool ple_ptrs_ok(std::initializer_list<const void*> rows16, std::initializer_list<const void*> words4) {
    for (const void* p : rows16)
        if (!aligned(p, 16)) return false;
    for (const void* p : words4)
        if (!aligned(p, 4)) return false;
    return true;
}

}  // namespace

size_t engram_short_conv_workspace(int64_t batch, int64_t seq, int64_t channels, int32_t kernel) {
    if (batch < 0 || seq < 0 || channels <= 0 || kernel < 1 || kernel > 4) return 0;
    return engram::short_conv_workspace_bytes(batch, seq, channels, kernel);
}

int engram_short_conv(const void* x, int32_t dtype, int64_t batch, int64_t seq, int64_t channels,
                      const float* weight, const float* bias, int32_t kernel, int32_t dilation, const void* halo,
                      void* y, hipStream_t stream) {
    int eb;
    int rc = ple_dims_ok(dtype, batch, seq, channels, &eb);
    if (rc != ENGRAM_OK) return rc;
    if (kernel < 1 || kernel > 4 || dilation < 1 || !weight) return ENGRAM_EINVAL;
    if (engram::short_conv_launch_items(batch, seq, channels, kernel, dilation, eb) >= kConvLaunchItems)
        return ENGRAM_EINVAL;
    if (batch * seq > 0 && (!x || !y)) return ENGRAM_EINVAL;
    if (!ple_ptrs_ok({x, y, halo}, {weight, bias})) return ENGRAM_EINVAL;
    return launch_result(engram::launch_short_conv(x, eb, batch, seq, channels, weight, bias, kernel, dilation, halo,
                                                   y, stream));
}

int engram_short_conv_backward(const void* x, const void* dy, int32_t dtype, int64_t batch, int64_t seq,
                               int64_t channels, const float* weight, int32_t kernel, int32_t dilation,
                               const void* halo, void* dx, float* dweight, float* dbias, void* dhalo, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    int eb;
    int rc = ple_dims_ok(dtype, batch, seq, channels, &eb);
    if (rc != ENGRAM_OK) return rc;
    if (kernel < 1 || kernel > 4 || dilation < 1 || !weight || !dweight) return ENGRAM_EINVAL;
    if (engram::short_conv_launch_items(batch, seq, channels, kernel, dilation, eb) >= kConvLaunchItems)
        return ENGRAM_EINVAL;
    if (batch * seq > 0 && (!x || !dy || !dx)) return ENGRAM_EINVAL;
    if (!ple_ptrs_ok({x, dy, halo, dx, dhalo}, {weight, dweight, dbias})) return ENGRAM_EINVAL;
    if (((uintptr_t)workspace & 255) != 0) return ENGRAM_EWORKSPACE;
    const size_t need = engram::short_conv_workspace_bytes(batch, seq, channels, kernel);
    if (need > 0 && (!workspace || workspace_bytes < need)) return ENGRAM_EWORKSPACE;
    return launch_result(engram::launch_short_conv_backward(x, dy, eb, batch, seq, channels, weight, kernel, dilation,
                                                            halo, dx, dweight, dbias, dhalo, workspace, stream));
}

size_t engram_grouped_rms_norm_workspace(int64_t rows, int64_t hidden) {
    if (rows < 0 || hidden <= 0) return 0;
    return engram::rms_norm_workspace_bytes(rows, hidden);
}

int engram_grouped_rms_norm(const void* x, int32_t dtype, int64_t rows, int64_t hidden, int64_t group_size,
                            const float* weight, float eps, void* y, hipStream_t stream) {
    int eb;
    int rc = ple_dims_ok(dtype, rows, 1, hidden, &eb);
    if (rc != ENGRAM_OK) return rc;
    if (group_size <= 0 || hidden % group_size != 0 || !engram::rms_norm_group_ok(eb, group_size) || !weight ||
        !(eps >= 0.0f))
        return ENGRAM_EINVAL;
    if (rows > 0 && (!x || !y)) return ENGRAM_EINVAL;
    if (!norm_groups_ok(rows, hidden, group_size)) return ENGRAM_EINVAL;
    if (!ple_ptrs_ok({x, y}, {weight})) return ENGRAM_EINVAL;
    return launch_result(engram::launch_rms_norm(x, eb, rows, hidden, group_size, weight, eps, y, stream));
}

int engram_grouped_rms_norm_backward(const void* x, const void* dy, int32_t dtype, int64_t rows, int64_t hidden,
                                     int64_t group_size, const float* weight, float eps, void* dx, float* dweight,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int eb;
    int rc = ple_dims_ok(dtype, rows, 1, hidden, &eb);
    if (rc != ENGRAM_OK) return rc;
    if (group_size <= 0 || hidden % group_size != 0 || !engram::rms_norm_group_ok(eb, group_size) || !weight ||
        !dweight || !(eps >= 0.0f))
        return ENGRAM_EINVAL;
    if (rows > 0 && (!x || !dy || !dx)) return ENGRAM_EINVAL;
    if (!norm_groups_ok(rows, hidden, group_size)) return ENGRAM_EINVAL;
    if (!ple_ptrs_ok({x, dy, dx}, {weight, dweight})) return ENGRAM_EINVAL;
    if (((uintptr_t)workspace & 255) != 0) return ENGRAM_EWORKSPACE;
    const size_t need = engram::rms_norm_workspace_bytes(rows, hidden);
    if (need > 0 && (!workspace || workspace_bytes < need)) return ENGRAM_EWORKSPACE;
    return launch_result(engram::launch_rms_norm_backward(x, dy, eb, rows, hidden, group_size, weight, eps, dx,
                                                          dweight, workspace, stream));
}

const char* engram_strerror(int code) {
    switch (code) {
        case ENGRAM_OK: return "success";
        case ENGRAM_EINVAL: return "invalid argument (null or misaligned pointer, size out of range or unsupported row width)";
        case ENGRAM_EDTYPE: return "unsupported element type";
        case ENGRAM_EWORKSPACE: return "workspace missing, misaligned or too small";
        case ENGRAM_ELAUNCH: return "kernel launch failed";
        case ENGRAM_ESPEC: return "hash spec out of range (ngram_size, heads, moduli or offsets)";
        default: return "unknown engram status";
    }
}

}  // extern "C"
