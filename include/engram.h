/*
 * engram.h — C ABI of the Engram n-gram embedding hot path on MI355X (gfx950).
 *
 * Three calls carry the lookup path: raw token IDs -> hashed head rows
 * (engram_hash), head rows -> table values (engram_gather), and output
 * gradients -> per-row gradient sums (engram_scatter_add).  Around them: the
 * single-GPU half of the row-owner exchange (engram_route_*, pack/unpack,
 * permute, and one-pass forms of the requester's copies) and the PLE layer's
 * causal short convolution and grouped RMSNorm
 * (engram_short_conv*, engram_grouped_rms_norm*), each declared with the
 * passage that defines it.  From raw tokens, engram_hash_gather and
 * engram_scatter_add_plan_from_tokens (and their context-parallel slice forms)
 * run the forward and the backward's sort without a rows array.
 *
 * Passages defining the operations ("engram API page" = the page titled
 * nemo_automodel.components.models.qwen3_8_flash_next.engram; "model-coverage
 * page" = the page titled Qwen3.8-Flash-Next):
 *   - hash: engram API page, Qwen3_8_FlashNextNGramEmbedding (class
 *     description, _hash_input_ids, _shift_right_after_eos);
 *   - gather: engram API page, Qwen3_8_FlashNextNGramEmbedding._lookup_ngram_ids
 *     and Qwen3_8_FlashNextOwnerShardedEmbedding (class description, forward):
 *     an owner looks up only its contiguous rows [row_begin, row_begin+num_rows);
 *   - scatter-add: the same class description and the model-coverage page,
 *     Validated Configuration: the backward pass routes gradients back so that
 *     only the owner accumulates each row's gradient;
 *   - errors: engram API page, _validate_global_ids / _validate_received_ids:
 *     an ID outside the owned range is an error reported with a diagnostic,
 *     never clamped; the model-coverage page, Current Scope: GPU paths never
 *     fall back silently.
 *
 * Conventions for every call:
 *   - Pointers named "device" point to GPU memory owned by the caller; the
 *     library allocates nothing and keeps no mutable global state, so calls on
 *     different streams are independent and the library is thread-safe.  The
 *     one exception is engram_scatter_add_noalloc, whose workspace is a fixed
 *     device array that its calls on one GPU share (see its declaration).
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); a
 *     returned ENGRAM_OK means "launched", results are ready when the stream is.
 *   - Host-checkable argument errors return a negative engram_status at once
 *     and enqueue nothing.
 *   - Data errors (a row outside the owned range) never cause an out-of-bounds
 *     access: gather writes a zero row for it, scatter-add drops it, and when
 *     `status` is non-NULL the lowest offending lookup index is stored there
 *     (-1 when every row is in range).  The library itself first sets
 *     *status = -1 on the stream, so the caller needs no initialisation.
 *   - Sizes are int64; all arrays are dense and row-major.
 *   - Device arrays are aligned to their access width: 16 bytes for arrays
 *     of rows (tables, gathered values, gradients, PLE activations) and for
 *     the hash's output rows (stored as pairs of int64), 8 bytes for other
 *     int64 arrays and status words, 4 bytes for fp32 weights and for the
 *     opaque rows of the routing calls.  A misaligned pointer returns
 *     ENGRAM_EINVAL.  Memory from hipMalloc (or torch) is always aligned.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ENGRAM_OK = 0,
    ENGRAM_EINVAL = -1,     /* null or misaligned pointer, negative or too large size, unsupported dim */
    ENGRAM_EDTYPE = -2,     /* unknown element type */
    ENGRAM_EWORKSPACE = -3, /* workspace missing, not 256-byte aligned or smaller than required */
    ENGRAM_ELAUNCH = -4,    /* the HIP runtime refused a kernel launch */
    ENGRAM_ESPEC = -5       /* hash spec outside the supported range */
} engram_status;

typedef enum { ENGRAM_F32 = 0, ENGRAM_BF16 = 1 } engram_dtype;

#define ENGRAM_MAX_NGRAM 8
#define ENGRAM_MAX_HEADS 64

/* Hash configuration: the constructor arguments of Qwen3_8_FlashNextNGramEmbedding
 * (engram API page).  H = (ngram_size - 1) * heads_per_ngram heads; heads
 * [0, heads_per_ngram) hash bigrams, the next heads_per_ngram trigrams, and so on.
 *   ngram_size       largest n-gram order including the current token, 2..8 (released: 3)
 *   heads_per_ngram  heads per order, >= 1, H <= 64 (released: 8)
 *   eos_id           raw ID after which the context resets (released: 248044)
 *   fill_id          value of a missing history token (before the sequence start
 *                    or across an EOS); the page's description of it is cut off,
 *                    0 is the value this project uses
 *   multipliers[k]   signed int64 multiplier of the token k positions back, k < ngram_size
 *   head_mod[h]      positive modulus of head h, 2 <= head_mod[h] <= 2^62
 *   head_offset[h]   global row offset of head h, >= 0, head_offset[h] + head_mod[h] - 1
 *                    must not overflow int64
 * Each position's order-n mix is the 64-bit XOR of the wrapped products of the
 * current token and its n-1 predecessors; row = mix mod head_mod (positive
 * remainder) + head_offset. */
typedef struct {
    int32_t ngram_size;
    int32_t heads_per_ngram;
    int64_t eos_id;
    int64_t fill_id;
    int64_t multipliers[ENGRAM_MAX_NGRAM];
    int64_t head_mod[ENGRAM_MAX_HEADS];
    int64_t head_offset[ENGRAM_MAX_HEADS];
} engram_hash_spec;

/* Hash raw token IDs into global table rows (engram API page,
 * Qwen3_8_FlashNextNGramEmbedding._hash_input_ids).
 *   tokens    device int64 [batch][seq_len], raw tokenizer IDs (any int64 value)
 *   spec      host pointer, read during the call only
 *   rows_out  device int64 [batch][seq_len][H], 16-byte aligned
 * Batch rows are independent; a packed (THD) stream is batch = 1 whose
 * documents are separated by EOS.  batch * seq_len == 0 is a no-op;
 * batch * seq_len <= 2^32 - 64 (one work-item per position).
 * Returns ENGRAM_OK, ENGRAM_EINVAL or ENGRAM_ESPEC. */
int engram_hash(const int64_t* tokens, int64_t batch, int64_t seq_len, const engram_hash_spec* spec,
                int64_t* rows_out, hipStream_t stream);

/* Hash the whole raw sequence but emit rows only for positions [seq_begin, seq_end)
 * of every batch row (engram API page, _forward_global_slice): the two (in general
 * ngram_size - 1) preceding tokens and EOS resets before seq_begin are honoured,
 * so the slice equals columns [seq_begin, seq_end) of engram_hash on the full row.
 *   tokens    device int64 [batch][seq_len]
 *   rows_out  device int64 [batch][seq_end - seq_begin][H], 16-byte aligned
 * Requires 0 <= seq_begin <= seq_end <= seq_len and batch * (seq_end - seq_begin)
 * <= 2^32 - 64. */
int engram_hash_slice(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                      int64_t seq_end, const engram_hash_spec* spec, int64_t* rows_out,
                      hipStream_t stream);

/* Owner-local row gather (engram API page, Qwen3_8_FlashNextOwnerShardedEmbedding.forward
 * on the owner's shard; _lookup_ngram_ids concatenates the H heads of a position,
 * which is this output viewed as [..., H * dim]).
 *   table     device [num_rows][dim] of `dtype`: global rows [row_begin, row_begin + num_rows)
 *   rows      device int64 [n] global row IDs
 *   out       device [n][dim] of `dtype`; out[i] = table[rows[i] - row_begin], bit for bit
 *   status    device int64 scalar or NULL (see conventions)
 * dim * element size must be a multiple of 16 bytes and at most 1024 bytes;
 * n <= 2^40 (any count that fits in memory).
 * Returns ENGRAM_OK, ENGRAM_EINVAL or ENGRAM_EDTYPE. */
int engram_gather(const void* table, int32_t dtype, int64_t row_begin, int64_t num_rows, int32_t dim,
                  const int64_t* rows, int64_t n, void* out, int64_t* status, hipStream_t stream);

/* The forward in one call: engram_hash of every position, then engram_gather of
 * its H rows (engram API page, Qwen3_8_FlashNextNGramEmbedding: the input IDs are
 * hashed (_hash_input_ids) and the head rows looked up (_lookup_ngram_ids), on
 * the owner's shard as Qwen3_8_FlashNextOwnerShardedEmbedding does).
 *   tokens    device int64 [batch][seq_len]
 *   table, dtype, row_begin, num_rows, dim, status: as for engram_gather
 *   out       device [batch][seq_len][H][dim] of `dtype`, 16-byte aligned:
 *             out[b][t][h] = table[row(b, t, h) - row_begin], bit for bit what
 *             engram_hash followed by engram_gather gives
 *   rows_out  device int64 [batch][seq_len][H], 16-byte aligned, or NULL: the
 *             hashed rows, as engram_hash writes them
 * For the released layout (ngram_size 3, 8 heads per order), a 160-wide bf16
 * table and at most 2^25 positions, one kernel hashes and gathers, and rows_out
 * may be NULL (the rows are then neither written nor read).  Any other call runs
 * the hash into rows_out and the gather from it, and rows_out is required.
 * Lookup index i = (b * seq_len + t) * H + h in `status`.  Requires batch *
 * seq_len <= 2^32 - 64.
 * Returns ENGRAM_OK, ENGRAM_EINVAL, ENGRAM_EDTYPE or ENGRAM_ESPEC. */
int engram_hash_gather(const int64_t* tokens, int64_t batch, int64_t seq_len, const engram_hash_spec* spec,
                       const void* table, int32_t dtype, int64_t row_begin, int64_t num_rows, int32_t dim,
                       void* out, int64_t* rows_out, int64_t* status, hipStream_t stream);

/* engram_hash_gather for columns [seq_begin, seq_end) of every batch row, each
 * hashed with the two tokens before it even where they lie before seq_begin
 * (engram API page, Qwen3_8_FlashNextNGramEmbedding._forward_global_slice:
 * hash the complete sequence, look up only one local slice; a
 * context-parallel rank's forward).  out: device [batch][seq_end -
 * seq_begin][H][dim]; rows_out (or NULL, as for engram_hash_gather): device
 * int64 [batch][seq_end - seq_begin][H].  Equals engram_hash_slice followed by
 * engram_gather bit for bit.  Lookup index i = (b * width + (t - seq_begin)) *
 * H + h in `status`.  0 <= seq_begin <= seq_end <= seq_len; batch * width <=
 * 2^32 - 64.  Returns ENGRAM_OK, ENGRAM_EINVAL, ENGRAM_EDTYPE or ENGRAM_ESPEC. */
int engram_hash_gather_slice(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                             int64_t seq_end, const engram_hash_spec* spec, const void* table, int32_t dtype,
                             int64_t row_begin, int64_t num_rows, int32_t dim, void* out, int64_t* rows_out,
                             int64_t* status, hipStream_t stream);

/* Bytes of device workspace engram_scatter_add needs for n lookups into a
 * num_rows-row shard with rows of dim values (256-byte aligned start). */
size_t engram_scatter_add_workspace(int64_t n, int64_t num_rows, int32_t dim);

/* Owner-local gradient scatter-add: the backward of engram_gather.  For every
 * distinct in-range row r, S[r] = sum of grad_out[i] over the lookups i with
 * rows[i] == r, accumulated in fp64 in a fixed order (deterministic run to run)
 * and rounded once to fp32.  Exactly one output form:
 *   dense    grad_dense device fp32 [num_rows][dim]: grad_dense[r] = fp32(grad_dense[r] + S[r])
 *            (the caller zeroes it, or passes an existing gradient to add to);
 *            uniq_rows, uniq_grad, num_uniq must be NULL;
 *   compact  uniq_rows device int64 [n], uniq_grad device fp32 [n][dim], num_uniq device
 *            int64 scalar: the U distinct rows in ascending order (global IDs) and
 *            their S; *num_uniq = U; entries past U are left untouched;
 *            grad_dense must be NULL.
 *   rows      device int64 [n] global row IDs (as given to engram_gather)
 *   grad_out  device [n][dim] of `dtype` (the gradient of engram_gather's output)
 *   workspace device, at least engram_scatter_add_workspace(n, num_rows, dim) bytes,
 *             256-byte aligned; contents need no initialisation and are scratch
 * Limits: n < 2^31, num_rows < 2^32 - 1, dim as for engram_gather.
 * Returns ENGRAM_OK, ENGRAM_EINVAL, ENGRAM_EDTYPE or ENGRAM_EWORKSPACE. */
int engram_scatter_add(const int64_t* rows, int64_t n, const void* grad_out, int32_t dtype, int32_t dim,
                       int64_t row_begin, int64_t num_rows, float* grad_dense, int64_t* uniq_rows,
                       float* uniq_grad, int64_t* num_uniq, void* workspace, size_t workspace_bytes,
                       int64_t* status, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): engram_scatter_add with
 * its workspace taken from a fixed device array inside the library, of
 * ENGRAM_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it runs on, held until the
 * process ends.  The call allocates nothing.  Arguments, output forms, limits
 * and results are those of engram_scatter_add; sizes whose workspace
 * (engram_scatter_add_workspace) exceeds the array return ENGRAM_EWORKSPACE
 * before anything is enqueued: at dim 160, up to about 1.18 M lookups.  Every
 * call on one GPU shares that GPU's array, so calls that overlap on one GPU
 * (other streams, other host threads) race and give undefined results;
 * calls ordered on one stream are safe, each starting from scratch contents
 * it initialises itself.  Returns ENGRAM_ELAUNCH when the array's device
 * address cannot be obtained. */
#define ENGRAM_NOALLOC_SCRATCH_BYTES (64u << 20)
int engram_scatter_add_noalloc(const int64_t* rows, int64_t n, const void* grad_out, int32_t dtype, int32_t dim,
                               int64_t row_begin, int64_t num_rows, float* grad_dense, int64_t* uniq_rows,
                               float* uniq_grad, int64_t* num_uniq, int64_t* status, hipStream_t stream);

/* The two phases of engram_scatter_add, for callers that reuse one set of row ids
 * (several gradients over the same lookups) or time the phases apart.
 *
 * engram_scatter_add_plan: sorts the lookups by row (stable, so each row's lookups
 * keep ascending index order) and records the runs of equal rows in `workspace`.
 *   rows       device int64 [n] global row IDs
 *   uniq_rows  device int64 [n] or NULL: when given, the U distinct in-range rows in
 *              ascending order (global IDs) are written to uniq_rows[0, U)
 *   num_uniq   device int64 scalar or NULL: receives U
 *   status     as for engram_gather (out-of-range rows are left out of the plan)
 * engram_scatter_add_apply: the per-row fp64 sums of grad_out along the plan in
 * `workspace`, in exactly one output form (dense grad_dense += S, or compact
 * uniq_grad[u] = S of the u-th distinct row).  n, row_begin, num_rows and dim must
 * be those of the plan call, and the workspace must not have been reused since;
 * mismatched use gives unspecified sums but no access outside the buffers sized
 * by these arguments.
 * engram_scatter_add(rows, ...) is exactly plan followed by apply on one stream.
 * Same limits and return codes as engram_scatter_add. */
int engram_scatter_add_plan(const int64_t* rows, int64_t n, int64_t row_begin, int64_t num_rows, int32_t dim,
                            int64_t* uniq_rows, int64_t* num_uniq, void* workspace, size_t workspace_bytes,
                            int64_t* status, hipStream_t stream);

int engram_scatter_add_apply(const void* grad_out, int32_t dtype, int32_t dim, int64_t n, int64_t row_begin,
                             int64_t num_rows, float* grad_dense, float* uniq_grad, const void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* engram_scatter_add_plan for rows as the owner receives them from the
 * exchange (engram API page, _FixedCapacityAllToAll.backward routes each
 * gradient row back to the owner of its ID; Qwen3_8_FlashNextOwnerShardedEmbedding:
 * only the owner accumulates a row's gradient): ids [world][capacity] as
 * received (the first split_sizes[w] entries of block w are IDs, all of them
 * for a count above capacity, none for a negative count; the rest is padding,
 * never checked).  The plan covers n = world * capacity entries, padding as
 * dropped lookups, so engram_scatter_add_apply then reads the gradient rows
 * straight from the received padded gradient blocks [world][capacity][dim]
 * with that n; no unpack of the IDs or the gradients is needed.  *status =
 * lowest padded index holding an ID outside [row_begin, row_begin + num_rows),
 * else -1.  Workspace: engram_scatter_add_workspace(world * capacity, ...).
 * world * capacity < 2^31.  Returns ENGRAM_OK, ENGRAM_EINVAL or ENGRAM_EWORKSPACE. */
int engram_scatter_add_plan_padded(const int64_t* ids, const int64_t* split_sizes, int32_t world, int64_t capacity,
                                   int64_t row_begin, int64_t num_rows, int32_t dim, int64_t* uniq_rows,
                                   int64_t* num_uniq, void* workspace, size_t workspace_bytes, int64_t* status,
                                   hipStream_t stream);

/* engram_scatter_add_plan for the rows engram_hash would write from `tokens`, hashed
 * inside the plan (engram API page, Qwen3_8_FlashNextNGramEmbedding: the backward of
 * _lookup_ngram_ids reaches the rows _hash_input_ids gives; the hash depends on the
 * tokens alone, so the backward may hash again instead of keeping the rows).  The
 * released layout only (ngram_size 3, 8 heads per order: n = batch * seq_len * 16
 * lookups, lookup (b * seq_len + t) * 16 + h); the plan, its outputs and the apply
 * that follows (with this n) are exactly those of engram_scatter_add_plan on the
 * hashed rows.  Every position has exactly one lookup per head, so when every
 * head's range [offset, offset + vocab size) lies in [row_begin, row_begin +
 * num_rows) and the ranges are disjoint and ascending in head order (the released
 * module data: the bigram heads, then the trigram heads, one after another), the
 * sort runs per head over the bits of the largest vocab size (three passes instead
 * of four for the released table); the result is the same.
 *   tokens    device int64 [batch][seq_len]
 *   other arguments as for engram_scatter_add_plan; the workspace is
 *   engram_scatter_add_workspace(n, num_rows, dim) bytes
 * Requires n < 2^31.  Returns ENGRAM_OK, ENGRAM_EINVAL (also for another head
 * layout), ENGRAM_ESPEC or ENGRAM_EWORKSPACE. */
int engram_scatter_add_plan_from_tokens(const int64_t* tokens, int64_t batch, int64_t seq_len,
                                        const engram_hash_spec* spec, int64_t row_begin, int64_t num_rows, int32_t dim,
                                        int64_t* uniq_rows, int64_t* num_uniq, void* workspace,
                                        size_t workspace_bytes, int64_t* status, hipStream_t stream);

/* engram_scatter_add_plan_from_tokens for one context-parallel slice: the rows
 * engram_hash_slice would write for columns [seq_begin, seq_end) of every batch
 * row, hashed inside the plan with the columns before seq_begin as history
 * (engram API page, Qwen3_8_FlashNextNGramEmbedding._forward_global_slice: the two
 * preceding raw tokens and the EOS resets carry across the slice boundary).  So a
 * rank's backward re-hashes its slice without keeping a rows array.  n = batch *
 * (seq_end - seq_begin) * 16 lookups, lookup (b * (seq_end - seq_begin) + t -
 * seq_begin) * 16 + h, exactly as engram_hash_slice lays out rows_out; the plan,
 * its outputs and the apply that follows (with this n) are those of
 * engram_scatter_add_plan on those rows.  The sort splits by head under the same
 * conditions as engram_scatter_add_plan_from_tokens.
 *   tokens    device int64 [batch][seq_len], the whole sequence of every row
 *   seq_begin, seq_end   0 <= seq_begin <= seq_end <= seq_len < 2^32
 *   other arguments as for engram_scatter_add_plan_from_tokens; the workspace is
 *   engram_scatter_add_workspace(n, num_rows, dim) bytes
 * Requires n < 2^31.  Returns ENGRAM_OK, ENGRAM_EINVAL (also for another head
 * layout or a bad column range), ENGRAM_ESPEC or ENGRAM_EWORKSPACE. */
int engram_scatter_add_plan_from_tokens_slice(const int64_t* tokens, int64_t batch, int64_t seq_len,
                                              int64_t seq_begin, int64_t seq_end, const engram_hash_spec* spec,
                                              int64_t row_begin, int64_t num_rows, int32_t dim, int64_t* uniq_rows,
                                              int64_t* num_uniq, void* workspace, size_t workspace_bytes,
                                              int64_t* status, hipStream_t stream);

/* ---- Owner routing: the single-GPU half of the row-owner exchange ----------
 * Engram API page, Qwen3_8_FlashNextOwnerShardedEmbedding: with `world` owners,
 * rank r owns global rows [r * local_rows, (r + 1) * local_rows), local_rows =
 * num_embeddings / world (num_embeddings must divide by world); a request rank
 * groups its IDs by owner before the first All-to-All (_exchange_ids), checks
 * the destination segments (_validate_sorted_send_ids), and exchanges segments
 * padded to one agreed capacity (_fixed_capacity_all_to_all).  The collective
 * itself is not part of this library.  1 <= world <= 255.  Rows handled by pack,
 * unpack and permute are opaque: row_bytes is a multiple of 4, at most 1 MiB. */

/* Bytes of device workspace engram_route_plan needs for n IDs. */
size_t engram_route_workspace(int64_t n);

/* Group IDs by owner, keeping request order inside each owner's segment.
 *   global_ids   device int64 [n]
 *   sorted_ids   device int64 [n]: segment of owner 0, then owner 1, ...; IDs
 *                outside [0, num_embeddings) come last, after every segment
 *   order        device int64 [n]: request position of each sorted entry
 *   send_counts  device int64 [world]: segment lengths (out-of-range IDs excluded)
 *   status       device int64 or NULL: lowest request index holding an ID
 *                outside the table, else -1
 * n < 2^31.  Returns ENGRAM_OK, ENGRAM_EINVAL or ENGRAM_EWORKSPACE. */
int engram_route_plan(const int64_t* global_ids, int64_t n, int64_t num_embeddings, int32_t world,
                      int64_t* sorted_ids, int64_t* order, int64_t* send_counts, void* workspace,
                      size_t workspace_bytes, int64_t* status, hipStream_t stream);

/* _validate_sorted_send_ids: every ID of segment w (send_counts, device int64
 * [world]) lies in owner w's rows.  *status (device, required) = lowest sorted
 * index that breaks this, n if a count is negative or the counts exceed n, else -1. */
int engram_route_validate(const int64_t* sorted_ids, int64_t n, const int64_t* send_counts, int32_t world,
                          int64_t num_embeddings, int64_t* status, hipStream_t stream);

/* Send side of _fixed_capacity_all_to_all: compact rows src [src_rows][row],
 * segments ordered by rank -> dst [world][capacity][row], segment w in block w,
 * the rest of each block filled with the element `fill` (host pointer to
 * fill_bytes = 1, 2, 4 or 8 bytes, repeated over the row).  Segment w is the
 * next max(split_sizes[w], 0) source rows: a count above capacity keeps its
 * first `capacity` rows but still consumes all of them, a negative count is
 * an empty segment.  Source rows at or past src_rows are never read; a block
 * row whose source lies there takes the fill.  *status (device or NULL) =
 * lowest rank whose split size is negative or above capacity, else world if
 * some segment reaches past src_rows, else -1. */
int engram_pack_fixed_capacity(const void* src, int64_t src_rows, int64_t row_bytes, const int64_t* split_sizes,
                               int32_t world, int64_t capacity, const void* fill, int32_t fill_bytes, void* dst,
                               int64_t* status, hipStream_t stream);

/* Receive side: src [world][capacity][row] -> compact dst [sum(split_sizes)][row] in
 * rank order: the first min(split_sizes[w], capacity) rows of block w (none for a
 * negative count); dst has room for dst_rows rows and rows that would land past
 * them are dropped.  *status = lowest rank whose split size is negative or above
 * capacity, world if the compact rows exceed dst_rows, else -1. */
int engram_unpack_fixed_capacity(const void* src, int64_t row_bytes, const int64_t* split_sizes, int32_t world,
                                 int64_t capacity, void* dst, int64_t dst_rows, int64_t* status, hipStream_t stream);

/* The requester's return path in one pass (engram API page,
 * _fixed_capacity_all_to_all restores the compact source-ordered rows after the
 * collective, and Qwen3_8_FlashNextOwnerShardedEmbedding.forward returns values
 * in the original request order): compact row k, the k-th row that
 * engram_unpack_fixed_capacity would write (block w's first
 * min(split_sizes[w], capacity) rows, in rank order), is written to dst row
 * order[k], as engram_unpermute_rows would move it; order is the request
 * position of each grouped entry (engram_route_plan), dst has n rows.  Equals
 * engram_unpack_fixed_capacity into an n-row buffer followed by
 * engram_unpermute_rows, except that a dst row whose compact row does not exist
 * (counts summing below n) is left as it was.  Compact rows at or past n are
 * dropped; order entries outside [0, n) are skipped.  *status (device or NULL)
 * = lowest rank whose split size is negative or above capacity, world if the
 * compact rows exceed n, else -1. */
int engram_unpack_unpermute_rows(const void* src, int64_t row_bytes, const int64_t* split_sizes, int32_t world,
                                 int64_t capacity, const int64_t* order, int64_t n, void* dst, int64_t* status,
                                 hipStream_t stream);

/* The requester's send in the backward in one pass (engram API page,
 * _FixedCapacityAllToAll.backward routes gradient rows back along the value
 * route, and _fixed_capacity_all_to_all pads every segment to the agreed
 * capacity with a fill): the gradient rows src [n][row], in request order, are
 * taken in grouped order (grouped row k = src row order[k], as
 * engram_permute_rows) and packed as engram_pack_fixed_capacity packs them:
 * block w holds grouped rows offset(w) .. offset(w) + min(split_sizes[w],
 * capacity) - 1 and the fill after them.  Equals engram_permute_rows followed
 * by engram_pack_fixed_capacity with src_rows = n, except that a block row
 * whose order entry lies outside [0, n) takes the fill.  *status as
 * engram_pack_fixed_capacity with src_rows = n. */
int engram_permute_pack_rows(const void* src, int64_t row_bytes, const int64_t* order, int64_t n,
                             const int64_t* split_sizes, int32_t world, int64_t capacity, const void* fill,
                             int32_t fill_bytes, void* dst, int64_t* status, hipStream_t stream);

/* The owner's lookup on the exchange's padded blocks in one pass (engram API
 * page, Qwen3_8_FlashNextOwnerShardedEmbedding: owners look up the received
 * IDs in their local rows and return the values through the same fixed-capacity
 * exchange, _fixed_capacity_all_to_all).  ids: device int64 [world][capacity]
 * as received; the first split_sizes[w] entries of block w are IDs (all of
 * them for a count above capacity, none for a negative count), the rest is
 * padding.  out: device [world][capacity][dim] of the table's dtype; an ID's
 * row is looked up as engram_gather does (a zero row for an ID outside
 * [row_begin, row_begin + num_rows)), padding rows are zero.  *status (device
 * or NULL) = lowest padded index w * capacity + r holding an ID outside the
 * shard, else -1.  Equals engram_unpack_fixed_capacity of the IDs,
 * engram_gather and engram_pack_fixed_capacity of the values with a zero fill.
 * Row sizes as engram_gather; 1 <= world <= 255. */
int engram_gather_padded(const void* table, int32_t dtype, int64_t row_begin, int64_t num_rows, int32_t dim,
                         const int64_t* ids, const int64_t* split_sizes, int32_t world, int64_t capacity, void* out,
                         int64_t* status, hipStream_t stream);

/* dst[i] = src[order[i]] (into grouped order) and dst[order[i]] = src[i] (back to
 * request order), rows of row_bytes; an order entry outside [0, n) is skipped. */
int engram_permute_rows(const void* src, int64_t row_bytes, const int64_t* order, int64_t n, void* dst,
                        hipStream_t stream);
int engram_unpermute_rows(const void* src, int64_t row_bytes, const int64_t* order, int64_t n, void* dst,
                          hipStream_t stream);

/* ---- PLE: causal short convolution and grouped RMSNorm ----------------------
 * Engram API page, Qwen3_8_FlashNextPLELayer (_causal_short_conv, init_weights):
 * a causal depthwise convolution over the sequence of x [batch][seq][channels]
 * with kernel width K = conv_kernel_size (4) and dilation d = ngram_size (3):
 *     y[b][t][c] = bias[c] + sum_k weight[c][k] * x[b][t - (K - 1 - k) * d][c]
 * (tap K - 1 is the current token); positions before 0 read the halo when one
 * is given, else zero ("left zero history").  The halo [batch][(K-1)*d][channels]
 * holds the (K-1)*d tokens that precede position 0 (9 for the released
 * settings), as a context-parallel shard receives them.
 * Layers API page, Qwen3_8_FlashNextGroupedRMSNorm and _grouped_rms_norm_fp32:
 * each run of group_size features of a row is scaled by
 * 1 / sqrt(mean(x^2) + eps) and then by (1 + weight[feature]), in fp32.
 *
 * Activations are ENGRAM_BF16 or ENGRAM_F32 (x, dy, y, dx, halo, dhalo all of
 * that type); weights, biases and their gradients are fp32.  channels (conv)
 * and group_size (norm) times the element size must be a multiple of 16 bytes;
 * group_size * element size <= 10240 bytes (5120 bf16, 2560 fp32 features);
 * hidden % group_size == 0.  At most 2^36 elements per tensor, and for the
 * norm at most 2^25 (row, group) pairs, so that every launch fits; a
 * convolution call whose launches would hold 2^32 work-items or more (short
 * sequences over very many batch rows reach that first) gets ENGRAM_EINVAL.
 * 1 <= K <= 4, d >= 1.  Gradients of weight and bias are sums over every batch
 * row and position, reduced in a fixed order (deterministic), and overwrite
 * dweight / dbias.  The backward calls need a device workspace (256-byte
 * aligned) of the size returned by the *_workspace call; it holds fp64
 * partial sums and is not read after the call completes.
 * Returns ENGRAM_OK, ENGRAM_EINVAL, ENGRAM_EDTYPE, ENGRAM_EWORKSPACE or
 * ENGRAM_ELAUNCH. */

/* Bytes of workspace engram_short_conv_backward needs (0 for bad sizes). */
size_t engram_short_conv_workspace(int64_t batch, int64_t seq, int64_t channels, int32_t kernel);

/* y = conv(x) as above.  weight device fp32 [channels][K]; bias device fp32
 * [channels] or NULL; halo device or NULL (zero history); y device, same
 * shape and type as x, must not overlap x or halo. */
int engram_short_conv(const void* x, int32_t dtype, int64_t batch, int64_t seq, int64_t channels,
                      const float* weight, const float* bias, int32_t kernel, int32_t dilation, const void* halo,
                      void* y, hipStream_t stream);

/* Gradients of engram_short_conv given dy (same shape as x): dx (same shape),
 * dweight [channels][K], dbias [channels] or NULL (not wanted), dhalo
 * [batch][(K-1)*d][channels] or NULL (not wanted).  x and halo are those of
 * the forward call (halo NULL = zero history). */
int engram_short_conv_backward(const void* x, const void* dy, int32_t dtype, int64_t batch, int64_t seq,
                               int64_t channels, const float* weight, int32_t kernel, int32_t dilation,
                               const void* halo, void* dx, float* dweight, float* dbias, void* dhalo, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace engram_grouped_rms_norm_backward needs (0 for bad sizes). */
size_t engram_grouped_rms_norm_workspace(int64_t rows, int64_t hidden);

/* y = grouped RMSNorm of x [rows][hidden], weight device fp32 [hidden], eps >= 0. */
int engram_grouped_rms_norm(const void* x, int32_t dtype, int64_t rows, int64_t hidden, int64_t group_size,
                            const float* weight, float eps, void* y, hipStream_t stream);

/* dx [rows][hidden] and dweight [hidden] of engram_grouped_rms_norm given dy. */
int engram_grouped_rms_norm_backward(const void* x, const void* dy, int32_t dtype, int64_t rows, int64_t hidden,
                                     int64_t group_size, const float* weight, float eps, void* dx, float* dweight,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static English text for an engram_status code. */
const char* engram_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
