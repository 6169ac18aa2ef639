// Internal declarations of the fused hash-and-gather forward (lookup.hip).
#pragma once

#include "engram_internal.h"

namespace engram {

// Positions per launch of the fused kernel: one wave each, fewer than 2^31
// work-items.
constexpr int64_t kLookupMaxPositions = (int64_t)1 << 25;

// Whether one kernel both hashes and gathers: the released head layout (3-gram,
// 8 heads per order: 16 rows per position), a 160-wide bf16 table and at most
// kLookupMaxPositions positions.  Otherwise the forward runs the hash into
// rows_out and then the gather.
bool hash_gather_fused(const HashParams& p, int elem_bytes, int dim, int64_t positions);

// Columns [seq_begin, seq_end) of every batch row, hashed with the columns
// before them (seq_begin = 0, seq_end = seq_len: the whole sequence).
hipError_t launch_hash_gather(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                              int64_t seq_end, const HashParams& p, const void* table, int elem_bytes,
                              int64_t row_begin, int64_t num_rows, int dim, void* out, int64_t* rows_out,
                              int64_t* status, hipStream_t stream);

// Backward phase 1 from tokens: the plan of engram_scatter_add_plan for the
// rows the released head layout hashes from columns [seq_begin, seq_end) of
// `tokens` [batch][seq_len] (16 per position, the columns before seq_begin
// read as history), hashed inside the plan's first kernel (scatter.hip).
hipError_t launch_scatter_plan_tokens(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                                      int64_t seq_end, const HashParams& p, int64_t row_begin, int64_t num_rows,
                                      int dim, int64_t* uniq_rows, int64_t* num_uniq, void* workspace,
                                      int64_t* status, hipStream_t stream);

}  // namespace engram
