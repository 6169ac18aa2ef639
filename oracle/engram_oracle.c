/*
 * Oracle of the Engram n-gram embedding hot path in plain C — TEST INFRASTRUCTURE.
 *
 * Plain scalar loops, no blocking or fusion, fp64 sums.  Shares no code or
 * header with the product library; only tests, the smoke check and the
 * benchmark's CPU-baseline leg load it (through oracle/c_oracle.py).
 *
 * Passages followed ("engram API page" = the page titled
 * nemo_automodel.components.models.qwen3_8_flash_next.engram):
 *   hash    — Qwen3_8_FlashNextNGramEmbedding class description,
 *             _shift_right_after_eos, _hash_input_ids;
 *   gather  — Qwen3_8_FlashNextOwnerShardedEmbedding class description and
 *             forward (owner-local lookup of rows [row_begin, row_begin+rows)),
 *             _validate_received_ids (an ID outside the owned range is an
 *             error, never clamped);
 *   scatter — the same class description: only the owner accumulates a row's
 *             gradient (backward of the lookup = sum of the output gradients
 *             of every lookup of that row).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Signed 64-bit product with wrap-around, done on unsigned integers because
 * signed overflow is undefined in C. */
static int64_t wrap_mul(int64_t a, int64_t b) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    return (int64_t)p;
}

/* Positive (floor) remainder of a signed value by a positive modulus.  C's %
 * truncates toward zero, so a negative result is moved up by one modulus. */
static int64_t positive_mod(int64_t v, int64_t p) {
    int64_t r = v % p;
    if (r < 0) r += p;
    return r;
}

/* _shift_right_after_eos for one batch row. */
static void shift_right_after_eos(const int64_t* ids, int64_t seq, int shift, int64_t eos,
                                  int64_t fill, int64_t* out) {
    for (int64_t t = 0; t < seq; ++t) {
        if (t < shift) { out[t] = fill; continue; }
        int crosses = 0;
        for (int64_t u = t - shift; u < t; ++u)
            if (ids[u] == eos) crosses = 1;
        out[t] = crosses ? fill : ids[t - shift];
    }
}

/* _hash_input_ids: ids [batch][seq] -> rows [batch][seq][(ngram_size-1)*heads_per_ngram].
 * Returns 0, or -1 for an unusable configuration. */
int oracle_hash(const int64_t* ids, int64_t batch, int64_t seq, int32_t ngram_size,
                int32_t heads_per_ngram, int64_t eos, int64_t fill, const int64_t* multipliers,
                const int64_t* vocab_sizes, const int64_t* offsets, int64_t* rows) {
    if (ngram_size < 2 || ngram_size > 8 || heads_per_ngram < 1) return -1;
    const int64_t heads = (int64_t)(ngram_size - 1) * heads_per_ngram;
    int64_t* shifted = (int64_t*)malloc(sizeof(int64_t) * (size_t)(seq > 0 ? seq : 1) * (size_t)ngram_size);
    if (!shifted) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t* row_ids = ids + b * seq;
        memcpy(shifted, row_ids, sizeof(int64_t) * (size_t)seq);
        for (int s = 1; s < ngram_size; ++s)
            shift_right_after_eos(row_ids, seq, s, eos, fill, shifted + (int64_t)s * seq);
        for (int64_t t = 0; t < seq; ++t) {
            int64_t* out = rows + (b * seq + t) * heads;
            int64_t mix = wrap_mul(shifted[t], multipliers[0]);
            for (int order = 2; order <= ngram_size; ++order) {
                mix ^= wrap_mul(shifted[(int64_t)(order - 1) * seq + t], multipliers[order - 1]);
                for (int j = 0; j < heads_per_ngram; ++j) {
                    int64_t h = (int64_t)(order - 2) * heads_per_ngram + j;
                    out[h] = positive_mod(mix, vocab_sizes[h]) + offsets[h];
                }
            }
        }
    }
    free(shifted);
    return 0;
}

/* Owner-local lookup: out[i] = table[rows[i] - row_begin] (bytes copied).
 * A row outside [row_begin, row_begin + num_rows) gives a zero output row.
 * Returns the lowest offending lookup index, or -1. */
int64_t oracle_gather(const void* table, int32_t elem_bytes, int32_t dim, int64_t row_begin,
                      int64_t num_rows, const int64_t* rows, int64_t n, void* out) {
    const size_t row_bytes = (size_t)elem_bytes * (size_t)dim;
    int64_t first_bad = -1;
    for (int64_t i = 0; i < n; ++i) {
        char* dst = (char*)out + (size_t)i * row_bytes;
        if (rows[i] < row_begin || rows[i] - row_begin >= num_rows) {
            memset(dst, 0, row_bytes);
            if (first_bad < 0) first_bad = i;
            continue;
        }
        memcpy(dst, (const char*)table + (size_t)(rows[i] - row_begin) * row_bytes, row_bytes);
    }
    return first_bad;
}

static double load_grad(const void* dy, int32_t dy_is_bf16, size_t idx) {
    if (dy_is_bf16) {
        /* bfloat16 is the upper half of an IEEE binary32 value. */
        uint32_t bits = (uint32_t)((const uint16_t*)dy)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float*)dy)[idx];
}

typedef struct { int64_t row; int64_t idx; } row_ref;

static int cmp_row_ref(const void* a, const void* b) {
    const row_ref* x = (const row_ref*)a;
    const row_ref* y = (const row_ref*)b;
    if (x->row != y->row) return x->row < y->row ? -1 : 1;
    if (x->idx != y->idx) return x->idx < y->idx ? -1 : 1;
    return 0;
}

/* Collect the in-range lookups sorted by (local row, lookup index). */
static int64_t sorted_valid(const int64_t* rows, int64_t n, int64_t row_begin, int64_t num_rows,
                            row_ref** out_refs, int64_t* first_bad) {
    row_ref* refs = (row_ref*)malloc(sizeof(row_ref) * (size_t)(n > 0 ? n : 1));
    int64_t m = 0;
    *first_bad = -1;
    for (int64_t i = 0; i < n; ++i) {
        if (rows[i] < row_begin || rows[i] - row_begin >= num_rows) {
            if (*first_bad < 0) *first_bad = i;
            continue;
        }
        refs[m].row = rows[i] - row_begin;
        refs[m].idx = i;
        ++m;
    }
    qsort(refs, (size_t)m, sizeof(row_ref), cmp_row_ref);
    *out_refs = refs;
    return m;
}

/* Dense backward: grad[r] = grad_in[r] + sum of dy[i] over lookups i of row r, in
 * fp64 with the lookups taken in ascending index order.  grad_in is fp32
 * [num_rows][dim]; grad_out is fp64 [num_rows][dim] (rows never looked up
 * keep grad_in).  Returns the lowest out-of-range lookup index, or -1. */
int64_t oracle_scatter_add_dense(const int64_t* rows, int64_t n, const void* dy, int32_t dy_is_bf16,
                                 int32_t dim, int64_t row_begin, int64_t num_rows,
                                 const float* grad_in, double* grad_out) {
    for (int64_t r = 0; r < num_rows; ++r)
        for (int32_t c = 0; c < dim; ++c)
            grad_out[r * dim + c] = (double)grad_in[r * dim + c];
    row_ref* refs;
    int64_t first_bad;
    int64_t m = sorted_valid(rows, n, row_begin, num_rows, &refs, &first_bad);
    double* acc = (double*)malloc(sizeof(double) * (size_t)dim);
    int64_t i = 0;
    while (i < m) {
        int64_t r = refs[i].row;
        for (int32_t c = 0; c < dim; ++c) acc[c] = 0.0;
        while (i < m && refs[i].row == r) {
            for (int32_t c = 0; c < dim; ++c)
                acc[c] += load_grad(dy, dy_is_bf16, (size_t)refs[i].idx * dim + c);
            ++i;
        }
        for (int32_t c = 0; c < dim; ++c) grad_out[r * dim + c] += acc[c];
    }
    free(acc);
    free(refs);
    return first_bad;
}

/* Compact backward: the distinct looked-up rows in ascending order (global row
 * IDs) with their fp64 gradient sums.  uniq_rows has room for n entries and
 * uniq_grad for n*dim.  Returns the lowest out-of-range lookup index, or -1. */
int64_t oracle_scatter_add_compact(const int64_t* rows, int64_t n, const void* dy, int32_t dy_is_bf16,
                                   int32_t dim, int64_t row_begin, int64_t num_rows,
                                   int64_t* uniq_rows, double* uniq_grad, int64_t* num_uniq) {
    row_ref* refs;
    int64_t first_bad;
    int64_t m = sorted_valid(rows, n, row_begin, num_rows, &refs, &first_bad);
    int64_t u = 0, i = 0;
    while (i < m) {
        int64_t r = refs[i].row;
        double* acc = uniq_grad + u * dim;
        for (int32_t c = 0; c < dim; ++c) acc[c] = 0.0;
        while (i < m && refs[i].row == r) {
            for (int32_t c = 0; c < dim; ++c)
                acc[c] += load_grad(dy, dy_is_bf16, (size_t)refs[i].idx * dim + c);
            ++i;
        }
        uniq_rows[u] = r + row_begin;
        ++u;
    }
    *num_uniq = u;
    free(refs);
    return first_bad;
}
