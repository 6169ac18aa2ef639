/*
 * The oracle's hash, gather and compact scatter-add spread over every host
 * core with OpenMP — TEST INFRASTRUCTURE (the CPU baseline beside the GPU
 * timing).  Each function computes exactly what its single-threaded twin in
 * engram_oracle.c computes, from the same passages:
 *   hash    — engram API page, Qwen3_8_FlashNextNGramEmbedding class
 *             description, _shift_right_after_eos, _hash_input_ids;
 *   gather  — Qwen3_8_FlashNextOwnerShardedEmbedding (owner-local rows,
 *             _validate_received_ids: an ID outside the owned range is an error);
 *   scatter — the same class: only the owner sums a row's gradients.
 * Work is split so that no result depends on the thread count: positions and
 * lookups are independent, and every row's gradients are still summed in
 * fp64 in ascending lookup order, so the outputs equal the single-threaded
 * oracle's bit for bit.  Shares no code with the product library.
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int oracle_mt_threads(void) { return omp_get_max_threads(); }

static int64_t mt_wrap_mul(int64_t a, int64_t b) { return (int64_t)((uint64_t)a * (uint64_t)b); }

static int64_t mt_positive_mod(int64_t v, int64_t p) {
    int64_t r = v % p;
    return r < 0 ? r + p : r;
}

/* The token s positions back, or the fill when that lies before the row start
 * or an EOS sits in [t - s, t - 1] (the context resets after EOS). */
static int64_t context(const int64_t* row, int64_t t, int s, int64_t eos, int64_t fill) {
    if (t < s) return fill;
    for (int64_t u = t - s; u < t; ++u)
        if (row[u] == eos) return fill;
    return row[t - s];
}

int oracle_mt_hash(const int64_t* ids, int64_t batch, int64_t seq, int32_t ngram_size, int32_t heads_per_ngram,
                   int64_t eos, int64_t fill, const int64_t* multipliers, const int64_t* vocab_sizes,
                   const int64_t* offsets, int64_t* rows) {
    if (ngram_size < 2 || ngram_size > 8 || heads_per_ngram < 1) return -1;
    const int64_t heads = (int64_t)(ngram_size - 1) * heads_per_ngram;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < batch * seq; ++g) {
        const int64_t b = g / seq, t = g - b * seq;
        const int64_t* row = ids + b * seq;
        int64_t* out = rows + g * heads;
        int64_t mix = mt_wrap_mul(row[t], multipliers[0]);
        for (int order = 2; order <= ngram_size; ++order) {
            mix ^= mt_wrap_mul(context(row, t, order - 1, eos, fill), multipliers[order - 1]);
            for (int j = 0; j < heads_per_ngram; ++j) {
                const int64_t h = (int64_t)(order - 2) * heads_per_ngram + j;
                out[h] = mt_positive_mod(mix, vocab_sizes[h]) + offsets[h];
            }
        }
    }
    return 0;
}

int64_t oracle_mt_gather(const void* table, int32_t elem_bytes, int32_t dim, int64_t row_begin, int64_t num_rows,
                         const int64_t* rows, int64_t n, void* out) {
    const size_t row_bytes = (size_t)elem_bytes * (size_t)dim;
    int64_t first_bad = n;
#pragma omp parallel for schedule(static) reduction(min : first_bad)
    for (int64_t i = 0; i < n; ++i) {
        char* dst = (char*)out + (size_t)i * row_bytes;
        if (rows[i] < row_begin || rows[i] - row_begin >= num_rows) {
            memset(dst, 0, row_bytes);
            if (i < first_bad) first_bad = i;
            continue;
        }
        memcpy(dst, (const char*)table + (size_t)(rows[i] - row_begin) * row_bytes, row_bytes);
    }
    return first_bad == n ? -1 : first_bad;
}

static double mt_load_grad(const void* dy, int32_t dy_is_bf16, size_t idx) {
    if (dy_is_bf16) {
        const uint32_t bits = (uint32_t)((const uint16_t*)dy)[idx] << 16;  /* bf16 = upper half of binary32 */
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float*)dy)[idx];
}

typedef struct { int64_t row; int64_t idx; } mt_ref;

static int mt_cmp(const void* a, const void* b) {
    const mt_ref* x = (const mt_ref*)a;
    const mt_ref* y = (const mt_ref*)b;
    if (x->row != y->row) return x->row < y->row ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx ? 1 : 0);
}

/* Compact backward.  The parallel sort cuts the local row range into buckets
 * of equal width: each thread counts its contiguous share of the lookups per
 * bucket, the counts give every (thread, bucket) pair its slot range, the
 * lookups are copied there, and each bucket is sorted by (row, index) on its
 * own.  A row lies in exactly one bucket, so the buckets in order are the
 * whole sorted list, and each bucket's distinct rows and sums can be written
 * once the distinct rows of the buckets before it are counted. */
int64_t oracle_mt_scatter_add_compact(const int64_t* rows, int64_t n, const void* dy, int32_t dy_is_bf16,
                                      int32_t dim, int64_t row_begin, int64_t num_rows, int64_t* uniq_rows,
                                      double* uniq_grad, int64_t* num_uniq) {
    const int T = omp_get_max_threads();
    const int64_t NB = 4096;
    int64_t* count = (int64_t*)calloc((size_t)T * (size_t)NB, sizeof(int64_t));
    int64_t* bucket_start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(NB + 1));
    int64_t* bucket_uniq = (int64_t*)malloc(sizeof(int64_t) * (size_t)(NB + 1));
    mt_ref* refs = (mt_ref*)malloc(sizeof(mt_ref) * (size_t)(n > 0 ? n : 1));
    int64_t first_bad = n;
#define BUCKET_OF(local) ((int64_t)(((unsigned __int128)(uint64_t)(local) * (uint64_t)NB) / (uint64_t)num_rows))
#pragma omp parallel num_threads(T) reduction(min : first_bad)
    {
        const int th = omp_get_thread_num();
        const int64_t i0 = n * th / T, i1 = n * (th + 1) / T;
        int64_t* mine = count + (int64_t)th * NB;
        for (int64_t i = i0; i < i1; ++i) {
            if (rows[i] < row_begin || rows[i] - row_begin >= num_rows) {
                if (i < first_bad) first_bad = i;
                continue;
            }
            ++mine[BUCKET_OF(rows[i] - row_begin)];
        }
#pragma omp barrier
#pragma omp single
        {
            int64_t at = 0;
            for (int64_t k = 0; k < NB; ++k) {
                bucket_start[k] = at;
                for (int t = 0; t < T; ++t) {
                    const int64_t c = count[(int64_t)t * NB + k];
                    count[(int64_t)t * NB + k] = at;  /* now this (thread, bucket) pair's first slot */
                    at += c;
                }
            }
            bucket_start[NB] = at;
        }
        for (int64_t i = i0; i < i1; ++i) {
            if (rows[i] < row_begin || rows[i] - row_begin >= num_rows) continue;
            const int64_t local = rows[i] - row_begin;
            const int64_t slot = mine[BUCKET_OF(local)]++;
            refs[slot].row = local;
            refs[slot].idx = i;
        }
#pragma omp barrier
#pragma omp for schedule(dynamic, 8)
        for (int64_t k = 0; k < NB; ++k) {
            const int64_t a = bucket_start[k], b = bucket_start[k + 1];
            qsort(refs + a, (size_t)(b - a), sizeof(mt_ref), mt_cmp);
            int64_t u = 0;
            for (int64_t i = a; i < b; ++i)
                if (i == a || refs[i].row != refs[i - 1].row) ++u;
            bucket_uniq[k] = u;
        }
#pragma omp single
        {
            int64_t at = 0;
            for (int64_t k = 0; k < NB; ++k) {
                const int64_t u = bucket_uniq[k];
                bucket_uniq[k] = at;
                at += u;
            }
            bucket_uniq[NB] = at;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t k = 0; k < NB; ++k) {
            int64_t u = bucket_uniq[k];
            int64_t i = bucket_start[k];
            const int64_t end = bucket_start[k + 1];
            while (i < end) {
                const int64_t r = refs[i].row;
                double* acc = uniq_grad + u * dim;
                for (int32_t c = 0; c < dim; ++c) acc[c] = 0.0;
                while (i < end && refs[i].row == r) {
                    for (int32_t c = 0; c < dim; ++c)
                        acc[c] += mt_load_grad(dy, dy_is_bf16, (size_t)refs[i].idx * dim + c);
                    ++i;
                }
                uniq_rows[u] = r + row_begin;
                ++u;
            }
        }
    }
#undef BUCKET_OF
    *num_uniq = bucket_uniq[NB];
    free(refs);
    free(bucket_uniq);
    free(bucket_start);
    free(count);
    return first_bad == n ? -1 : first_bad;
}
