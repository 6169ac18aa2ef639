// Owner-local gradient scatter-add for gfx950: the backward of the row gather.
//
// Engram API page ("nemo_automodel.components.models.qwen3_8_flash_next.engram"),
// Qwen3_8_FlashNextOwnerShardedEmbedding: the backward route brings each
// lookup's output gradient back to the row's owner, which alone accumulates
// the row's gradient (also the model-coverage page "Qwen3.8-Flash-Next",
// Validated Configuration).  For every distinct owned row r the result is
// the sum of grad_out[i] over the lookups i of r.
//
// Hot rows (Zipf token streams repeat the same n-grams thousands of times)
// must not serialise on atomics, and the sums must not depend on scheduling.
// So the path sorts instead of atomically adding, in two phases:
// plan (depends on the row ids only)
//   1. keys     key = row - row_begin (or the sentinel num_rows for a row out
//               of range), value = lookup index; per-tile histogram of the
//               first digit in the same pass.
//   2. sort     stable LSD radix sort of (key, index), 8-bit digits, as many
//               passes as the bit length of num_rows needs (29 bits -> 4).
//               Per pass: tile histograms (also summed per chunk of tiles),
//               then a stable scatter that derives its digit offsets from
//               those counts, ranks digits inside each wave with ballots (no
//               atomics) and writes each tile digit-grouped through LDS.
//               From tokens, when the heads' row ranges are disjoint,
//               ascending and inside the shard, the sort is split by head
//               instead: every position has exactly one lookup per head, so
//               head h's lookups take entries [h * npos, (h + 1) * npos) with
//               no counting pass, and each head sorts only row - offset[h]
//               (below its modulus: 25 bits for the released table, three
//               passes of 8, 8 and 9 bits).  Disjoint ascending ranges make
//               the head-major order the global row order, so the result is
//               the same as the whole sort's.
//   3. runs     run starts per slice of S sorted entries, their prefix sum
//               (the distinct-row index of every run) and, for the compact
//               form, the distinct rows themselves.
// apply (once per gradient)
//   4. reduce   one worker (cpr lanes, one 16-byte chunk of the row each)
//               per slice walks its S entries in order, accumulating the
//               gradient rows in fp64.  A run that ends inside the slice is
//               written once; a run cut by a slice edge leaves an fp64 partial.
//   5. fix-up   the slice where a cut run starts adds the partials of the
//               following slices in slice order and writes the run.
// Every step has a fixed order, so two calls give bit-identical results.
#include <algorithm>

#include "radix_sort.h"
#include "hash_math.h"
#include "lookup.h"

namespace engram {
namespace {

// Build-time tuning parameters of the reduce, at the values measured best on
// the long-context and owner-shard workloads: entries per worker slice (32 and
// 128 were slower), non-temporal sum stores (plain stores were slower),
// non-temporal gradient loads (slower: off), gradient rows in flight per lane
// (8, 12 and 24 were no better).
#ifndef ENGRAM_REDUCE_SLICE
#define ENGRAM_REDUCE_SLICE 64
#endif
#ifndef ENGRAM_REDUCE_NT
#define ENGRAM_REDUCE_NT 1
#endif
#ifndef ENGRAM_REDUCE_NT_LOAD
#define ENGRAM_REDUCE_NT_LOAD 0
#endif
#ifndef ENGRAM_REDUCE_BATCH
#define ENGRAM_REDUCE_BATCH 16
#endif
constexpr uint32_t kSlice = ENGRAM_REDUCE_SLICE;  // sorted entries per reduce worker
static_assert((kSlice & (kSlice - 1)) == 0 && kSlice >= 32, "slices are powers of two, at least 32 entries");
// Blocks of the slice bookkeeping kernels cover `span` sorted entries: a power
// of two from kBlock (and at least one slice) to kRunSpanMax, the smallest that
// keeps the block count at most about 4,096 (fewer, fuller blocks for large n;
// enough blocks to fill the chip for small n).
constexpr uint32_t kRunSpanMax = 4096;
constexpr uint32_t kRunSpanMin = kSlice > (uint32_t)kBlock ? kSlice : (uint32_t)kBlock;
constexpr uint32_t kRunSlicesMax = kRunSpanMax / kSlice;  // slices per bookkeeping block, at most
static_assert(kRunSpanMax % kSlice == 0 && kRunSlicesMax <= (uint32_t)kBlock, "whole slices per bookkeeping block");

uint32_t run_span(int64_t n) {
    uint32_t span = kRunSpanMin;
    while (span < kRunSpanMax && (n + span - 1) / span > 4096) span *= 2;
    return span;
}

// Index of the first run starting in slice j among all runs: the runs before
// it in its bookkeeping block plus the runs of the blocks before.
struct RunBase {
    const uint32_t* slice;  // per slice, within its block
    const uint32_t* block;  // per block, exclusive prefix over blocks
    uint32_t shift;         // log2(slices per block)
    __device__ __forceinline__ uint32_t operator()(uint32_t j) const { return slice[j] + block[j >> shift]; }
};
constexpr uint32_t kFlagHead = 1, kFlagWhole = 2, kFlagTail = 4;

struct Layout {
    size_t sorted_keys, spare_keys, sorted_vals, spare_vals, hist, count_totals, counters, slice_runs, slice_base,
        slice_first, slice_flags, long_runs, long_done, carry_head, carry_tail, block_runs, block_base, total;
    int64_t num_tiles, num_slices, num_run_blocks;
};
constexpr int kMaxPasses = 4;  // 32-bit keys, 8-bit digits
constexpr int kRadixWide = 512;  // the 9-bit last pass of a sort split by head
constexpr int kTokenHeads = 16;  // rows per position of the released head layout

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Keys per thread of the plan's sort tiles, by lookup count.  Small tiles
// suit small sorts (more blocks; the plan's dependent launches finish
// sooner); large tiles suit large ones, where the plan runs beside the
// gather: each digit run a tile writes is longer, so fewer lines are written
// in part, and fewer blocks compete with the gather for wave slots.
#ifndef ENGRAM_SORT_ITEMS_LARGE
#define ENGRAM_SORT_ITEMS_LARGE 24  // keys per thread from 2^21 lookups (16 or 24)
#endif
static_assert(ENGRAM_SORT_ITEMS_LARGE == 16 || ENGRAM_SORT_ITEMS_LARGE == 24, "the plan's sort takes 16 or 24");
int sort_items(int64_t n) {
    return n <= ((int64_t)1 << 20) ? 8 : n >= ((int64_t)1 << 21) ? ENGRAM_SORT_ITEMS_LARGE : 16;
}

// Tiles per head of a sort split by head (0 when n is not 16 rows per position).
int64_t head_tiles(int64_t n) {
    const int64_t tile = (int64_t)kBlock * sort_items(n);
    return n > 0 && n % kTokenHeads == 0 ? (n / kTokenHeads + tile - 1) / tile : 0;
}

Layout make_layout(int64_t n, int dim) {
    Layout L;
    const int64_t tile = (int64_t)kBlock * sort_items(n);
    L.num_tiles = (n + tile - 1) / tile;
    const int64_t ht = head_tiles(n);
    // room for either form of the sort: whole, or split by head with 512-digit counts
    const size_t hist_words = std::max((size_t)kRadix * (size_t)L.num_tiles,
                                       (size_t)kRadixWide * (size_t)(kTokenHeads * ht));
    const size_t pass_words = std::max(count_words(L.num_tiles),
                                       ht ? (size_t)kTokenHeads * count_words(ht, kRadixWide) : (size_t)0);
    L.num_slices = (n + kSlice - 1) / kSlice;
    L.num_run_blocks = (n + run_span(n) - 1) / run_span(n);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
    L.sorted_keys = take(4 * (size_t)n);
    L.spare_keys = take(4 * (size_t)n);
    L.sorted_vals = take(4 * (size_t)n);
    L.spare_vals = take(4 * (size_t)n);
    L.hist = take(4 * hist_words);
    L.count_totals = take(4 * pass_words * kMaxPasses);  // one set per pass
    L.counters = take(16);
    L.slice_runs = take(4 * (size_t)L.num_slices);
    L.slice_base = take(4 * (size_t)L.num_slices);
    L.slice_first = take(4 * (size_t)L.num_slices);
    L.slice_flags = take(4 * (size_t)L.num_slices);
    L.long_runs = take(8 * (size_t)L.num_slices);
    L.long_done = take(4 * (size_t)L.num_slices);
    L.carry_head = take(8 * (size_t)L.num_slices * (size_t)dim);
    L.carry_tail = take(8 * (size_t)L.num_slices * (size_t)dim);
    L.block_runs = take(4 * (size_t)L.num_run_blocks);
    L.block_base = take(4 * (size_t)L.num_run_blocks);
    L.total = off;
    return L;
}

__global__ __launch_bounds__(kBlock) void scatter_init_kernel(int64_t* status, uint32_t* counters,
                                                              int64_t* num_uniq, uint32_t* count_totals,
                                                              uint32_t total_words) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (status) *status = -1;
        counters[0] = 0;  // number of in-range lookups
        if (num_uniq) *num_uniq = 0;
    }
    for (uint32_t i = blockIdx.x * kBlock + threadIdx.x; i < total_words; i += gridDim.x * kBlock)
        count_totals[i] = 0;
}

// Tile histograms count with LDS atomics into one sub-histogram per wave
// (summed at the end), which keeps same-address conflicts inside a wave.
// Where the plan's rows come from when it starts from tokens: the token batch
// they hash from, for the released head layout (3-gram, 8 heads per order:
// lookup e is head e % 16 of flattened position e / 16; engram API page,
// Qwen3_8_FlashNextNGramEmbedding: _hash_input_ids with the context of
// _shift_right_after_eos).
struct TokenRows {
    const int64_t* tokens;  // [batch * seq_len], flattened
    uint32_t seq_len;
    HashParams p;
    // A context-parallel slice: positions [seq_begin, seq_begin + width) of
    // every batch row, flattened over [batch][width]; their context is read
    // from the columns before seq_begin (engram API page,
    // Qwen3_8_FlashNextNGramEmbedding._forward_global_slice).  The whole
    // sequence is seq_begin 0 and width seq_len.
    uint32_t seq_begin, width;
};

// The three tokens of one position of a slice, read straight from the batch
// row (the columns before the slice are its history): flattened position pos
// is batch row b = pos / width, column t = seq_begin + pos % width.  Missing
// context (t < s, or an EOS in [t - s, t - 1]) takes the fill value.
__device__ __forceinline__ void slice_context(const TokenRows& tr, uint32_t b, uint32_t col, int64_t* x0,
                                              int64_t* ctx1, int64_t* ctx2) {
    const uint32_t t = tr.seq_begin + col;
    const int64_t* row = tr.tokens + (size_t)b * tr.seq_len;
    const int64_t a = row[t], b1 = row[t >= 1 ? t - 1 : t], b2 = row[t >= 2 ? t - 2 : t];
    const bool valid1 = t >= 1 && b1 != tr.p.eos;
    const bool valid2 = valid1 && t >= 2 && b2 != tr.p.eos;
    *x0 = a;
    *ctx1 = valid1 ? b1 : tr.p.fill;
    *ctx2 = valid2 ? b2 : tr.p.fill;
}
// Rows as the exchange delivers them: [world][capacity] blocks whose first
// counts[w] entries are rows and the rest padding (counts == nullptr: every
// entry is a row).  Padding takes the sentinel key without a report.
struct Padding {
    const int64_t* counts;
    uint32_t capacity;
};

// Step 1: keys, digit-0 tile histograms, in-range count.  A key's lookup
// index is its position, so the first sort pass reads no value array.  With
// TOKENS the rows are hashed here: the tile's positions (and the two before
// them) are staged in LDS, and lane l computes head l % 16 of its lookups'
// positions (the context of shift s is the token s back unless that lies
// before the batch row's start or an EOS sits in [t - s, t - 1]; missing
// context takes the fill value).
template <int ITEMS, bool TOKENS, bool SLICE = false>
__global__ __launch_bounds__(kBlock) void keys_kernel(const int64_t* __restrict__ rows, TokenRows tr, uint32_t n,
                                                      int64_t row_begin, uint64_t num_rows,
                                                      uint32_t* __restrict__ keys, DigitCounts dc,
                                                      int64_t* __restrict__ status,
                                                      uint32_t* __restrict__ counters, Padding pad) {
    constexpr int TILE = kBlock * ITEMS, TILE_POS = TILE / kTokenHeads;
    __shared__ uint32_t s_cnt[kBlock / 64][kRadix];
    __shared__ uint32_t s_valid;
    __shared__ int64_t s_tok[TOKENS ? TILE_POS + 2 : 1];  // positions p0 - 2 .. p0 + TILE_POS - 1
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) s_cnt[k][tid] = 0;
    if (tid == 0) s_valid = 0;
    const uint32_t p0 = blockIdx.x * (uint32_t)TILE_POS;  // the tile's first position (TOKENS)
    if (TOKENS && !SLICE) {
        const uint32_t npos = n / kTokenHeads;
        for (int i = tid; i < TILE_POS + 2; i += kBlock) {
            const int64_t q = (int64_t)p0 - 2 + i;
            s_tok[i] = q >= 0 && q < (int64_t)npos ? tr.tokens[q] : 0;
        }
    }
    __syncthreads();
    const uint32_t base = blockIdx.x * (uint32_t)TILE + (uint32_t)w * (64 * ITEMS);
    const uint32_t sentinel = (uint32_t)num_rows;
    uint32_t my_valid = 0;
    int64_t r[ITEMS];
    if (TOKENS) {
        // This lane's head: modulus, reciprocal and offset selected with
        // compile-time indices (the parameters stay kernel arguments).
        const int h = lane & (kTokenHeads - 1);
        uint64_t mod = tr.p.mod[0], magic = tr.p.magic[0];
        int64_t off = tr.p.off[0];
#pragma unroll
        for (int j = 1; j < kTokenHeads; ++j)
            if (h == j) {
                mod = tr.p.mod[j];
                magic = tr.p.magic[j];
                off = tr.p.off[j];
            }
        // Item it of this lane is position pos0 + 4 it; its column t advances
        // by 4 a step, wrapping at the row length (the slice's width).
        const uint32_t npos = n / kTokenHeads;
        const uint32_t pos0 = (base + (uint32_t)lane) / kTokenHeads;
        const uint32_t wrap = SLICE ? tr.width : tr.seq_len;
        uint32_t t = pos0 % wrap, b = pos0 / wrap;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            int64_t x0, ctx1, ctx2;
            if (SLICE) {
                const bool in = pos0 + 4u * (uint32_t)it < npos;
                slice_context(tr, in ? b : 0u, in ? t : 0u, &x0, &ctx1, &ctx2);  // past the end: position 0, unused
            } else {
                const int li = (int)(pos0 + 4u * (uint32_t)it - p0) + 2;
                const int64_t x1 = s_tok[li - 1], x2 = s_tok[li - 2];
                x0 = s_tok[li];
                const bool valid1 = t >= 1 && x1 != tr.p.eos;
                const bool valid2 = valid1 && t >= 2 && x2 != tr.p.eos;
                ctx1 = valid1 ? x1 : tr.p.fill;
                ctx2 = valid2 ? x2 : tr.p.fill;
            }
            const uint64_t mix2 = (uint64_t)x0 * (uint64_t)tr.p.mult[0] ^ (uint64_t)ctx1 * (uint64_t)tr.p.mult[1];
            const uint64_t mix = h < 8 ? mix2 : mix2 ^ (uint64_t)ctx2 * (uint64_t)tr.p.mult[2];
            r[it] = (int64_t)floor_mod((int64_t)mix, mod, magic) + off;
            t += 4;
            while (t >= wrap) {
                t -= wrap;
                ++b;
            }
        }
    } else {
        // Loads are clamped rather than guarded, so all of a thread's loads are
        // in flight together (a guarded load becomes a branch that waits for it).
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) r[it] = rows[min(base + (uint32_t)it * 64 + (uint32_t)lane, n - 1)];
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const uint32_t e = base + (uint32_t)it * 64 + (uint32_t)lane;
        if (e < n) {
            uint32_t key = sentinel;
            bool real = true;
            if (!TOKENS && pad.counts) {
                const uint32_t seg = e / pad.capacity;
                real = (int64_t)(e - seg * pad.capacity) < pad.counts[seg];
            }
            const uint64_t local = (uint64_t)r[it] - (uint64_t)row_begin;
            if (real && local < num_rows) {
                key = (uint32_t)local;
                ++my_valid;
            } else if (real) {
                report_bad(status, e);
            }
            keys[e] = key;
            atomicAdd(&s_cnt[w][key & 0xFFu], 1u);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) my_valid += __shfl_xor(my_valid, o, 64);
    if (lane == 0 && my_valid) atomicAdd(&s_valid, my_valid);
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) c += s_cnt[k][tid];
    publish_tile_counts(dc, blockIdx.x, tid, c);
    if (tid == 0 && s_valid) atomicAdd(&counters[0], s_valid);
}

// Step 1 of the plan from tokens, split by head (see step 2 above): block
// (h, tile) hashes head h of the tile's positions, so position pos's head-h
// lookup (lookup index 16 pos + h) becomes entry pos of segment h, with the
// histogram of the digit-0 of row - offset[h].  The host has checked that
// every head's range lies in the shard, so every lookup is in range.  Lane
// l's item it is position base + 64 it + l: each lane loads its own tokens,
// and the two before each position come from the lanes below it (lanes 0 and
// 1 take them from the previous item's lanes 62 and 63, or, for the first
// item, from the two positions before the wave's span).  With DIRECT (short
// segments, whose first pass takes its counts from the tile histograms alone)
// the kernel also does what the plan's init kernel would: block 0 sets the
// status word and the in-range count (every lookup), and the grid clears the
// later passes' chunk and group totals (`zero_words`), which are first added
// to after this kernel.
// With SLICE (a context-parallel slice) each position reads its three tokens
// from its batch row (slice_context): the lanes below may hold another row.
template <int ITEMS, bool DIRECT, bool SLICE = false>
__global__ __launch_bounds__(kBlock) void head_keys_kernel(TokenRows tr, int64_t row_begin, Segments sg,
                                                           uint32_t* __restrict__ keys, DigitCounts dc,
                                                           uint32_t* __restrict__ counters,
                                                           int64_t* __restrict__ status,
                                                           uint32_t* __restrict__ zero_words, uint32_t zero_count) {
    if (DIRECT) {
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            if (status) *status = -1;
            counters[0] = sg.len * (uint32_t)kTokenHeads;
        }
        for (uint32_t i = blockIdx.x * kBlock + threadIdx.x; i < zero_count; i += gridDim.x * kBlock)
            zero_words[i] = 0;
    }
    __shared__ uint32_t s_cnt[kBlock / 64][kRadix];
    __shared__ uint32_t s_valid;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint32_t h = blockIdx.x / sg.tiles, tile = blockIdx.x - h * sg.tiles;
    const uint32_t npos = sg.len, sb = segment_base(sg, h);
    dc = segment_counts(dc, sg, h);
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) s_cnt[k][tid] = 0;
    if (tid == 0) s_valid = 0;
    __syncthreads();
    // Head h's modulus, reciprocal and offset (block-uniform), selected with
    // compile-time indices so the parameters stay kernel arguments.
    uint64_t mod = tr.p.mod[0], magic = tr.p.magic[0];
    int64_t off = tr.p.off[0];
#pragma unroll
    for (int j = 1; j < kTokenHeads; ++j)
        if (h == (uint32_t)j) {
            mod = tr.p.mod[j];
            magic = tr.p.magic[j];
            off = tr.p.off[j];
        }
    const bool trigram = h >= (uint32_t)(kTokenHeads / 2);
    const uint32_t wbase = tile * (uint32_t)(kBlock * ITEMS) + (uint32_t)w * (64 * ITEMS);
    const uint32_t pos0 = wbase + (uint32_t)lane;
    const uint32_t wrap = SLICE ? tr.width : tr.seq_len;
    uint32_t t = pos0 % wrap, b = pos0 / wrap;  // item 0's column and row; the column advances by 64 an item
    uint32_t my_valid = 0;
    uint32_t* const seg_keys = keys + (size_t)h * npos;
    int64_t tok[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) tok[it] = SLICE ? 0 : tr.tokens[min(pos0 + 64u * (uint32_t)it, npos - 1)];
    // the two positions before the span (only read where the column says they
    // belong to the same batch row)
    int64_t last1 = SLICE ? 0 : tr.tokens[min(wbase >= 1 ? wbase - 1 : 0u, npos - 1)];
    int64_t last2 = SLICE ? 0 : tr.tokens[min(wbase >= 2 ? wbase - 2 : 0u, npos - 1)];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const uint32_t pos = pos0 + 64u * (uint32_t)it;
        int64_t x0, ctx1, ctx2;
        if (SLICE) {
            const bool in = pos < npos;
            slice_context(tr, in ? b : 0u, in ? t : 0u, &x0, &ctx1, &ctx2);  // past the end: position 0, unused
        } else {
            x0 = tok[it];
            const int64_t up1 = __shfl_up(x0, 1, 64), up2 = __shfl_up(x0, 2, 64);
            const int64_t x1 = lane >= 1 ? up1 : last1;
            const int64_t x2 = lane >= 2 ? up2 : lane == 1 ? last1 : last2;
            last1 = __shfl(x0, 63, 64);  // for the next item: the positions before its lanes 0 and 1
            last2 = __shfl(x0, 62, 64);
            const bool valid1 = t >= 1 && x1 != tr.p.eos;
            const bool valid2 = valid1 && t >= 2 && x2 != tr.p.eos;
            ctx1 = valid1 ? x1 : tr.p.fill;
            ctx2 = valid2 ? x2 : tr.p.fill;
        }
        const uint64_t mix2 = (uint64_t)x0 * (uint64_t)tr.p.mult[0] ^ (uint64_t)ctx1 * (uint64_t)tr.p.mult[1];
        const uint64_t mix = trigram ? mix2 ^ (uint64_t)ctx2 * (uint64_t)tr.p.mult[2] : mix2;
        const int64_t row = (int64_t)floor_mod((int64_t)mix, mod, magic) + off;
        if (pos < npos) {
            const uint32_t key = (uint32_t)((uint64_t)row - (uint64_t)row_begin);
            seg_keys[pos] = key;
            atomicAdd(&s_cnt[w][(key - sb) & 0xFFu], 1u);
            ++my_valid;
        }
        t += 64;
        if (SLICE) {
            while (t >= wrap) {
                t -= wrap;
                ++b;
            }
        } else if (t >= wrap) {
            t = wrap >= 64 ? t - wrap : t % wrap;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) my_valid += __shfl_xor(my_valid, o, 64);
    if (lane == 0 && my_valid) atomicAdd(&s_valid, my_valid);
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) c += s_cnt[k][tid];
    if (DIRECT) {
        dc.hist[(size_t)tile * kRadix + tid] = c;
    } else {
        publish_tile_counts(dc, tile, tid, c);
        if (tid == 0 && s_valid) atomicAdd(&counters[0], s_valid);
    }
}

// Step 3a: per slice, the number of runs that start in it, the index of the
// first such start (0xFFFFFFFF when a run covers the whole slice) and the
// runs starting before it inside its block of `span` entries; per block, the
// runs starting in it.
constexpr uint32_t kNoStart = 0xFFFFFFFFu;
__global__ __launch_bounds__(kBlock) void run_count_kernel(const uint32_t* __restrict__ keys, uint32_t n,
                                                           const uint32_t* __restrict__ counters,
                                                           uint32_t* __restrict__ slice_runs,
                                                           uint32_t* __restrict__ slice_first,
                                                           uint32_t* __restrict__ slice_base, uint32_t num_slices,
                                                           uint32_t* __restrict__ block_runs, uint32_t span) {
    __shared__ uint32_t s_cnt[kRunSlicesMax], s_first[kRunSlicesMax];
    __shared__ uint32_t s_tmp[kBlock / 64];
    const uint32_t nv = min(counters[0], n);
    const uint32_t slices = span / kSlice;
    if (threadIdx.x < slices) {
        s_cnt[threadIdx.x] = 0;
        s_first[threadIdx.x] = kNoStart;
    }
    __syncthreads();
    for (uint32_t off = 0; off < span; off += kBlock) {
        const uint32_t t = off + threadIdx.x;
        const uint32_t i = blockIdx.x * span + t;
        const uint32_t kc = keys[min(i, n - 1)], kp = keys[i == 0 ? 0u : min(i - 1, n - 1)];
        const bool start = i < nv && (i == 0 || kc != kp);
        const uint64_t b = __ballot(start);
        const uint32_t q = t / kSlice;
        if (kSlice >= 64) {  // a wave lies inside one slice: one LDS update per wave
            if ((threadIdx.x & 63) == 0 && b) {
                atomicAdd(&s_cnt[q], (uint32_t)__popcll(b));
                atomicMin(&s_first[q], i + (uint32_t)(__ffsll((unsigned long long)b) - 1));
            }
        } else if (start) {
            atomicAdd(&s_cnt[q], 1u);
            atomicMin(&s_first[q], i);
        }
    }
    __syncthreads();
    const uint32_t c = threadIdx.x < slices ? s_cnt[threadIdx.x] : 0u;
    uint32_t total;
    const uint32_t before = block_exclusive_scan_n<kBlock>(c, &total, s_tmp);
    if (threadIdx.x < slices) {
        const uint32_t j = blockIdx.x * slices + threadIdx.x;
        if (j < num_slices) {
            slice_runs[j] = c;
            slice_first[j] = s_first[threadIdx.x];
            slice_base[j] = before;  // within the block; RunBase adds the block's base
        }
    }
    if (threadIdx.x == 0) block_runs[blockIdx.x] = total;
}

// Step 3b: exclusive prefix of the blocks' run counts in one 256-thread block
// (a small block starts quickly beside the gather).  Rounds of 4,096 counts:
// a coalesced load into LDS, a serial scan of 16 contiguous counts per
// thread, one block scan of the thread totals, and a coalesced store.  The
// total is the number of distinct rows.
constexpr int kScanBlock = 256;
constexpr int kScanPer = 16;
constexpr int kScanRound = kScanBlock * kScanPer;
__device__ __forceinline__ int scan_pad(int e) { return e + (e >> 4); }  // one spare word per 16: no bank conflicts

__global__ __launch_bounds__(kScanBlock) void block_scan_kernel(const uint32_t* __restrict__ counts,
                                                                uint32_t count, uint32_t* __restrict__ prefix,
                                                                int64_t* __restrict__ num_uniq) {
    __shared__ uint32_t s_val[kScanRound + kScanRound / 16];
    __shared__ uint32_t s_tmp[kScanBlock / 64];
    const int tid = threadIdx.x;
    uint32_t carry = 0;
    for (uint32_t base = 0; base < count; base += kScanRound) {
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            const uint32_t i = base + (uint32_t)(k * kScanBlock + tid);
            const uint32_t raw = counts[min(i, count - 1)];
            s_val[scan_pad(k * kScanBlock + tid)] = i < count ? raw : 0u;
        }
        __syncthreads();
        uint32_t loc[kScanPer], sum = 0;
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            loc[k] = s_val[scan_pad(tid * kScanPer + k)];
            sum += loc[k];
        }
        uint32_t tot;
        uint32_t run = carry + block_exclusive_scan_n<kScanBlock>(sum, &tot, s_tmp);
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            s_val[scan_pad(tid * kScanPer + k)] = run;
            run += loc[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            const uint32_t i = base + (uint32_t)(k * kScanBlock + tid);
            if (i < count) prefix[i] = s_val[scan_pad(k * kScanBlock + tid)];
        }
        carry += tot;
        __syncthreads();
    }
    if (tid == 0 && num_uniq) *num_uniq = carry;
}

// Step 3c (compact form): the distinct rows in ascending order, written by
// the thread that holds each run's first entry (consecutive runs ->
// consecutive addresses).  One block per bookkeeping block.
__global__ __launch_bounds__(kBlock) void uniq_rows_kernel(const uint32_t* __restrict__ keys, uint32_t n,
                                                           const uint32_t* __restrict__ counters,
                                                           const uint32_t* __restrict__ block_base, int64_t row_begin,
                                                           int64_t* __restrict__ uniq_rows, uint32_t span) {
    __shared__ uint32_t s_cnt[kBlock / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t base = block_base[blockIdx.x];
    const uint32_t nv = min(counters[0], n);
    uint32_t carried = base;  // runs starting in this block before the current round
    for (uint32_t off = 0; off < span; off += kBlock) {
        const uint32_t i = blockIdx.x * span + off + threadIdx.x;
        const uint32_t key = keys[min(i, n - 1)], kp = keys[i == 0 ? 0u : min(i - 1, n - 1)];
        const bool start = i < nv && (i == 0 || key != kp);
        const uint64_t b = __ballot(start);
        if (lane == 0) s_cnt[w] = (uint32_t)__popcll(b);
        __syncthreads();
        uint32_t before = 0, round = 0;
#pragma unroll
        for (int k = 0; k < kBlock / 64; ++k) {
            const uint32_t c = s_cnt[k];
            before += k < w ? c : 0u;
            round += c;
        }
        if (start) {
            const uint32_t u = carried + before + (uint32_t)__popcll(b & lanemask_lt(lane));
            if (u < n) uniq_rows[u] = (int64_t)key + row_begin;
        }
        carried += round;
        __syncthreads();
    }
}

// Read by lanes with nothing to load, so gradient loads never need a branch.
__device__ u32x4 kZeroChunk = {0u, 0u, 0u, 0u};  // never written

// 16 bytes of gradient -> EPC fp64 addends (bf16 = upper half of a binary32).
template <bool BF16>
__device__ __forceinline__ void accumulate(double* acc, u32x4 x) {
    if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] += (double)__uint_as_float(x[q] << 16);
            acc[2 * q + 1] += (double)__uint_as_float(x[q] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += (double)__uint_as_float(x[q]);
    }
}

template <int EPC>
__device__ __forceinline__ void store_partial(double* dst, const double* acc) {
#pragma unroll
    for (int e = 0; e < EPC; e += 2) {
        double __attribute__((ext_vector_type(2))) v;
        v.x = acc[e];
        v.y = acc[e + 1];
        *(double __attribute__((ext_vector_type(2)))*)(dst + e) = v;
    }
}

template <int EPC>
__device__ __forceinline__ void add_partial(double* acc, const double* src) {
#pragma unroll
    for (int e = 0; e < EPC; e += 2) {
        const double __attribute__((ext_vector_type(2))) v = *(const double __attribute__((ext_vector_type(2)))*)(src + e);
        acc[e] += v.x;
        acc[e + 1] += v.y;
    }
}

// acc += the partials of slices k0 .. k1-1 (rows `dim` doubles apart), added in
// slice order.  AHEAD slices' loads are issued before any of their adds: the
// partials come from HBM, and a walk with only a few loads in flight is bound
// by their latency.
template <int EPC, int AHEAD>
__device__ __forceinline__ void add_partials(double* acc, const double* src, int64_t k0, int64_t k1, int dim) {
    typedef double __attribute__((ext_vector_type(2))) d2;
    constexpr int kAhead = AHEAD;
    int64_t k = k0;
    for (; k + kAhead <= k1; k += kAhead) {
        d2 v[kAhead][EPC / 2];
#pragma unroll
        for (int q = 0; q < kAhead; ++q)
#pragma unroll
            for (int e = 0; e < EPC / 2; ++e) v[q][e] = *(const d2*)(src + (size_t)(k + q) * dim + 2 * e);
        __builtin_amdgcn_sched_barrier(0);  // keep the scheduler from interleaving the adds into the loads
#pragma unroll
        for (int q = 0; q < kAhead; ++q)
#pragma unroll
            for (int e = 0; e < EPC / 2; ++e) {
                acc[2 * e] += v[q][e].x;
                acc[2 * e + 1] += v[q][e].y;
            }
    }
    for (; k < k1; ++k) add_partial<EPC>(acc, src + (size_t)k * dim);
}

// The same sum with the lanes of a cpr-lane worker reading interleaved 16-byte
// pairs: lane c adds pairs c, c + cpr, c + 2 cpr, ... of each row into
// acc2[0], acc2[1], ..., so one load instruction of the worker covers
// consecutive bytes of a row (a lane reading its own contiguous EPC doubles
// makes every instruction touch a line per lane).  Each element's additions
// stay in slice order.
template <int EPC, int AHEAD>
__device__ __forceinline__ void add_partials_interleaved(double __attribute__((ext_vector_type(2)))* acc2,
                                                         const double* rows, int64_t k0, int64_t k1, int dim,
                                                         int cpr, int c) {
    typedef double __attribute__((ext_vector_type(2))) d2;
    int64_t k = k0;
    for (; k + AHEAD <= k1; k += AHEAD) {
        d2 v[AHEAD][EPC / 2];
#pragma unroll
        for (int q = 0; q < AHEAD; ++q) {
            const d2* row = (const d2*)(rows + (size_t)(k + q) * dim) + c;
#pragma unroll
            for (int e = 0; e < EPC / 2; ++e) v[q][e] = row[e * cpr];
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the scheduler from interleaving the adds into the loads
#pragma unroll
        for (int q = 0; q < AHEAD; ++q)
#pragma unroll
            for (int e = 0; e < EPC / 2; ++e) acc2[e] += v[q][e];
    }
    for (; k < k1; ++k)
#pragma unroll
        for (int e = 0; e < EPC / 2; ++e) acc2[e] += *(const d2*)(rows + (size_t)k * dim + 2 * (e * cpr + c));
}

// Final write of one run: dense RMW (fp64 add, one rounding) or the compact
// sum.  key < num_rows and u < n hold for every run of a correct plan; the
// checks keep each store in bounds regardless.  Compact form with bf16
// gradients: a lane holds 8 sums = fp32 output chunks 2c and 2c+1 (16 B
// each); the worker's lanes exchange them so that store q writes chunks
// [q*cpr, (q+1)*cpr), one contiguous span per store instruction (whole
// cache lines, no half-written lines).  All lanes of the worker call this
// together.
template <int EPC, bool DENSE>
__device__ __forceinline__ void write_run(const double* acc, uint32_t key, uint32_t u, int c, int dim, uint32_t n,
                                          uint32_t num_rows, float* grad_dense, float* uniq_grad) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    if (DENSE ? key >= num_rows : u >= n) return;
    f32x4* g = (f32x4*)(DENSE ? grad_dense + (size_t)key * dim : uniq_grad + (size_t)u * dim);
    f32x4 v[EPC / 4];
    int chunk[EPC / 4];
    if (EPC == 8 && !DENSE) {
        const int cpr = dim / EPC;
        const int wl0 = (int)(threadIdx.x & 63) - c;
        float h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (float)acc[e];
#pragma unroll
        for (int q = 0; q < EPC / 4; ++q) {
            chunk[q] = q * cpr + c;
            const int src = wl0 + chunk[q] / 2, half = chunk[q] & 1;
            const float a0 = __shfl(h[0], src, 64), a1 = __shfl(h[1], src, 64), a2 = __shfl(h[2], src, 64),
                        a3 = __shfl(h[3], src, 64), b0 = __shfl(h[4], src, 64), b1 = __shfl(h[5], src, 64),
                        b2 = __shfl(h[6], src, 64), b3 = __shfl(h[7], src, 64);
            v[q].x = half ? b0 : a0;
            v[q].y = half ? b1 : a1;
            v[q].z = half ? b2 : a2;
            v[q].w = half ? b3 : a3;
        }
    } else {
        // Dense (a read-modify-write keeps the lines in L2, so lane order does
        // not matter there) and fp32 gradients (4 sums = one chunk per lane).
#pragma unroll
        for (int q = 0; q < EPC / 4; ++q) {
            chunk[q] = c * (EPC / 4) + q;
            if (DENSE) {
                const f32x4 old = g[chunk[q]];
                v[q].x = (float)((double)old.x + acc[4 * q]);
                v[q].y = (float)((double)old.y + acc[4 * q + 1]);
                v[q].z = (float)((double)old.z + acc[4 * q + 2]);
                v[q].w = (float)((double)old.w + acc[4 * q + 3]);
            } else {
                v[q].x = (float)acc[4 * q];
                v[q].y = (float)acc[4 * q + 1];
                v[q].z = (float)acc[4 * q + 2];
                v[q].w = (float)acc[4 * q + 3];
            }
        }
    }
#pragma unroll
    for (int q = 0; q < EPC / 4; ++q) {
        if (DENSE) {
            g[chunk[q]] = v[q];
        } else {
#if ENGRAM_REDUCE_NT
            __builtin_nontemporal_store(v[q], g + chunk[q]);
#else
            g[chunk[q]] = v[q];
#endif
        }
    }
}

constexpr int kReduceBatch = ENGRAM_REDUCE_BATCH;  // sorted entries in flight per lane

// Step 4.  Worker = cpr consecutive lanes, lane c owning 16-byte chunk c of
// the row; 64 / cpr workers per wave (bf16 x 160: 3 workers of 20 lanes).
// Per batch of bb <= 8 sorted entries, lanes c < bb load entry c's key, the
// key after it and its lookup index; one ballot marks where runs end, and the
// lookup indices reach the other lanes by shuffle.  The next batch's keys are
// fetched while the current batch's gradient chunks are summed.
template <int CPR_T, bool BF16, bool DENSE>
__global__ __launch_bounds__(kBlock) void segment_reduce_kernel(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ vals, uint32_t* __restrict__ counters,
    const u32x4* __restrict__ dy, uint32_t n, uint32_t num_rows, int cpr_rt, int dim, uint32_t num_slices,
    RunBase slice_base, const uint32_t* __restrict__ slice_first,
    float* __restrict__ grad_dense, float* __restrict__ uniq_grad,
    double* __restrict__ carry_head, double* __restrict__ carry_tail, uint32_t* __restrict__ slice_flags,
    uint32_t* __restrict__ long_done) {
    constexpr int EPC = BF16 ? 8 : 4;
    constexpr int B = kReduceBatch;
    const int cpr = CPR_T ? CPR_T : cpr_rt;
    const int wpw = 64 / cpr;
    const int lane = threadIdx.x & 63;
    const int sub = lane / cpr;
    const int c = lane - sub * cpr;
    const int wl0 = sub * cpr;
    const int bb = cpr < B ? cpr : B;
    const int64_t wave = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    const int64_t j = wave * wpw + sub;
    if (blockIdx.x == 0 && threadIdx.x == 0) {  // long-run list of the fix-up that follows, its most parts
        counters[1] = 0;
        counters[2] = 0;
    }
    // finished-part counts of the long-run sums two kernels on
    for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < num_slices; i += (uint64_t)gridDim.x * kBlock)
        long_done[i] = 0;
    if (sub >= wpw || j >= num_slices) return;
    const uint32_t nv = min(counters[0], n);
    // Worker j covers [first run start in slice j, first run start in slice
    // j+1): runs are cut only where a slice holds no run start at all (inside
    // a run longer than a slice); there the cut falls on the slice edge.
    const uint32_t f0 = slice_first[j];
    const uint32_t f1 = j + 1 < num_slices ? slice_first[j + 1] : kNoStart;
    const uint32_t s0 = min(f0 != kNoStart ? f0 : (uint32_t)j * kSlice, nv);
    const uint32_t s1 = j + 1 < num_slices ? min(f1 != kNoStart ? f1 : (uint32_t)(j + 1) * kSlice, nv) : nv;
    if (s0 >= s1) {
        if (c == 0) slice_flags[j] = 0;
        return;
    }
    bool head_open = f0 == kNoStart && s0 > 0 && keys[s0 - 1] == keys[s0];
    uint32_t u = slice_base(j);
    uint32_t flags = 0;
    double acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0;

    // Entry i + c of a batch: key, next key (0xFFFFFFFF past the end), lookup index.
    // Indices are clamped so every load is in bounds and unconditional.
    uint32_t k_cur, k_nxt, v_cur;
    {
        const uint32_t p = s0 + (uint32_t)c;
        const uint32_t kc = keys[min(p, nv - 1)], kn = keys[min(p + 1, nv - 1)], vc = vals[min(p, s1 - 1)];
        k_cur = p < nv ? kc : 0xFFFFFFFFu;
        k_nxt = p + 1 < nv ? kn : 0xFFFFFFFFu;
        v_cur = vc;
    }
    for (uint32_t i = s0; i < s1; i += bb) {
        const uint32_t mk = k_cur, mv = v_cur;
        const bool ends = c < bb && i + c < s1 && k_cur != k_nxt;
        const uint32_t emask = (uint32_t)(__ballot(ends) >> wl0);
        u32x4 x[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint32_t vb = __shfl(mv, wl0 + b, 64);
            const u32x4* src = (b < bb && i + b < s1 && vb < n) ? dy + ((size_t)vb * cpr + c) : &kZeroChunk;
#if ENGRAM_REDUCE_NT_LOAD
            x[b] = __builtin_nontemporal_load(src);
#else
            x[b] = *src;
#endif
        }
        if (i + bb < s1) {
            const uint32_t p = i + bb + (uint32_t)c;
            const uint32_t kc = keys[min(p, nv - 1)], kn = keys[min(p + 1, nv - 1)], vc = vals[min(p, s1 - 1)];
            k_cur = p < nv ? kc : 0xFFFFFFFFu;
            k_nxt = p + 1 < nv ? kn : 0xFFFFFFFFu;
            v_cur = vc;
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint32_t p = i + b;
            if (b >= bb || p >= s1) break;
            accumulate<BF16>(acc, x[b]);
            const bool run_end = (emask >> b) & 1u;
            if (!run_end && p + 1 < s1) continue;
            // Flush: the run ends at p, or the slice ends at p inside a run.
            const uint32_t key = __shfl(mk, wl0 + b, 64);
            if (head_open) {
                // first run of the slice, begun in an earlier slice
                store_partial<EPC>(carry_head + (size_t)j * dim + c * EPC, acc);
                flags |= kFlagHead | (run_end ? 0u : kFlagWhole);
                head_open = false;
            } else if (!run_end) {
                // begins here and runs on into the next slice
                store_partial<EPC>(carry_tail + (size_t)j * dim + c * EPC, acc);
                flags |= kFlagTail;
                ++u;
            } else {
                write_run<EPC, DENSE>(acc, key, u, c, dim, n, num_rows, grad_dense, uniq_grad);
                ++u;
            }
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
        }
    }
    if (c == 0) slice_flags[j] = flags;
}

// Step 5: runs cut by slice edges, summed in slice order by the slice j where
// they begin.  The run's last slice m comes from its last entry, found by a
// galloping then binary search over the sorted keys (about 2 log2(run / S)
// dependent loads).  A run over at most kLongRun slices is summed here by
// one worker; a longer one (a hot row) is listed for long_run_kernel, which
// splits its sum over a whole block, in parts of about kPartSlices slices
// (at most kMaxParts); the list's largest part count bounds that kernel's
// work items.
constexpr int64_t kLongRun = 32;
constexpr int64_t kPartSlices = 128;  // 64 was slower (more fences), 256 no faster
constexpr int64_t kMaxParts = 32;
__device__ __forceinline__ int64_t long_run_parts(int64_t head_partials) {
    return min(kMaxParts, (head_partials + kPartSlices - 1) / kPartSlices);
}

template <int CPR_T, bool BF16, bool DENSE>
__global__ __launch_bounds__(kBlock) void carry_fixup_kernel(
    const uint32_t* __restrict__ keys, uint32_t* __restrict__ counters, uint32_t n, uint32_t num_rows,
    int cpr_rt, int dim, uint32_t num_slices, const uint32_t* __restrict__ slice_runs,
    RunBase slice_base, const uint32_t* __restrict__ slice_first,
    const uint32_t* __restrict__ slice_flags, const double* __restrict__ carry_head,
    const double* __restrict__ carry_tail, uint32_t* __restrict__ long_runs,
    float* __restrict__ grad_dense, float* __restrict__ uniq_grad) {
    constexpr int EPC = BF16 ? 8 : 4;
    const int cpr = CPR_T ? CPR_T : cpr_rt;
    const int wpw = 64 / cpr;
    const int lane = threadIdx.x & 63;
    const int sub = lane / cpr;
    const int c = lane - sub * cpr;
    const int64_t wave = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    const int64_t j = wave * wpw + sub;
    if (sub >= wpw || j >= num_slices) return;
    if (!(slice_flags[j] & kFlagTail)) return;
    const uint32_t nv = min(counters[0], n);
    // A tail run continues past the slice, so (j + 1) * kSlice < nv.
    uint32_t lo = (uint32_t)(j + 1) * kSlice - 1;
    if (lo + 1 >= nv) return;
    const uint32_t key = keys[lo];
    int64_t m = j + 1;
    if (slice_flags[j + 1] & kFlagWhole) {
        // The run covers slice j+1 entirely.  Its last worker is the one just
        // before the first later slice holding a run start (or the last slice
        // with entries): scan slice_first, 4 * cpr slices per step.
        const int wl0 = sub * cpr;
        const int64_t last = (int64_t)(nv - 1) / kSlice;
        int64_t kstar = last + 1;
        for (int64_t b0 = j + 2; b0 <= last; b0 += 4 * cpr) {
            int q_first = 4;
#pragma unroll
            for (int q = 3; q >= 0; --q) {
                const int64_t idx = b0 + 4 * c + q;
                const uint32_t f = slice_first[min(idx, last)];
                if (idx <= last && f != kNoStart) q_first = q;
            }
            const uint64_t worker_lanes = cpr >= 64 ? ~0ull : ((1ull << cpr) - 1ull);
            const uint64_t any = (__ballot(q_first < 4) >> wl0) & worker_lanes;
            if (any) {
                const int l = __ffsll((unsigned long long)any) - 1;
                const int qf = __shfl(q_first, wl0 + l, 64);
                kstar = b0 + 4 * l + qf;
                break;
            }
        }
        m = min(kstar - 1, (int64_t)num_slices - 1);
    }
    if (m - j > kLongRun) {
        if (c == 0) {
            const uint32_t at = atomicAdd(&counters[1], 1u);
            atomicMax(&counters[2], (uint32_t)long_run_parts(m - j));
            if (at < num_slices) {
                long_runs[2 * at] = (uint32_t)j;
                long_runs[2 * at + 1] = (uint32_t)m;
            }
        }
        return;
    }
    double acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
    add_partial<EPC>(acc, carry_tail + (size_t)j * dim + c * EPC);
    add_partials<EPC, 4>(acc, carry_head + c * EPC, j + 1, m + 1, dim);
    const uint32_t u = slice_base(j) + slice_runs[j] - 1;
    write_run<EPC, DENSE>(acc, key, u, c, dim, n, num_rows, grad_dense, uniq_grad);
}

// Long runs.  A run's head partials j+1 .. m are cut into parts of about
// kPartSlices slices (at most kMaxParts), each summed by one block: the
// block's sub-workers (cpr lanes each) sum equal contiguous shares of the
// part, and the shares are added in sub-worker order.  A one-part run is
// finished by its block: tail partial plus the shares.  Otherwise each block
// leaves its part's sum in place of the part's first partial and counts
// itself done; the block that counts last (a fence before the count releases
// its sum, a fence after it acquires the others') adds the tail partial and
// the part sums in part order.  The sum of a run does not depend on
// scheduling; the list order may vary.  Work items are (part, run) pairs,
// part below the list's largest part count, with the first parts of all runs
// first, so every run's first part goes to a different block.  A block has 8 waves, each lane holding 512 bytes of loads
// in flight.
constexpr int kLongBlock = 512;

template <int CPR_T, bool BF16, bool DENSE>
__global__ __launch_bounds__(kLongBlock) void long_run_kernel(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ counters, uint32_t n, uint32_t num_rows,
    int cpr_rt, int dim, uint32_t num_slices, const uint32_t* __restrict__ slice_runs,
    RunBase slice_base, double* __restrict__ carry_head,
    const double* __restrict__ carry_tail, const uint32_t* __restrict__ long_runs,
    uint32_t* __restrict__ long_done, float* __restrict__ grad_dense, float* __restrict__ uniq_grad) {
    constexpr int EPC = BF16 ? 8 : 4;
    extern __shared__ double s_share[];  // [sub-workers][dim]
    __shared__ uint32_t s_last;
    const int cpr = CPR_T ? CPR_T : cpr_rt;
    const int wpw = 64 / cpr;
    const int lane = threadIdx.x & 63;
    const int sub = lane / cpr;
    const int c = lane - sub * cpr;
    const int nsub = wpw * (kLongBlock / 64);
    const int w = (threadIdx.x >> 6) * wpw + sub;  // sub-worker index in the block
    const bool active = sub < wpw;
    const uint32_t count = min(counters[1], num_slices);
    const uint64_t items = (uint64_t)count * min((uint64_t)counters[2], (uint64_t)kMaxParts);
    for (uint64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const uint32_t r = (uint32_t)(it % count);
        const int64_t p = (int64_t)(it / count);
        const int64_t j = long_runs[2 * r], m = long_runs[2 * r + 1];
        const int64_t total = m - j;  // head partials j+1 .. m
        const int64_t parts = long_run_parts(total);
        if (p >= parts) continue;  // uniform over the block
        const int64_t per_part = (total + parts - 1) / parts;
        const int64_t p0 = j + 1 + p * per_part, p1 = min(p0 + per_part, m + 1);
        const int64_t per = (p1 - p0 + nsub - 1) / nsub;
        if (active) {
            double __attribute__((ext_vector_type(2))) acc2[EPC / 2];
#pragma unroll
            for (int e = 0; e < EPC / 2; ++e) acc2[e] = 0.0;
            const int64_t b = min(p0 + (int64_t)w * per, p1), end = min(b + per, p1);
            add_partials_interleaved<EPC, 64 / EPC>(acc2, carry_head, b, end, dim, cpr, c);  // 512 B per lane in flight
#pragma unroll
            for (int e = 0; e < EPC / 2; ++e) {
                s_share[(size_t)w * dim + 2 * (e * cpr + c)] = acc2[e].x;
                s_share[(size_t)w * dim + 2 * (e * cpr + c) + 1] = acc2[e].y;
            }
        }
        __syncthreads();
        double acc[EPC];
        if (w == 0 && active) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
            if (parts == 1) add_partial<EPC>(acc, carry_tail + (size_t)j * dim + c * EPC);
#pragma unroll 2
            for (int q = 0; q < nsub; ++q)
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[e] += s_share[(size_t)q * dim + c * EPC + e];
            if (parts > 1) store_partial<EPC>(carry_head + (size_t)p0 * dim + c * EPC, acc);
        }
        bool finish = parts == 1;
        if (parts > 1) {
            // Only wave 0 (sub-worker 0) writes and reads part sums, so only
            // it fences: each fence writes back or invalidates a whole L2.
            if (threadIdx.x < 64) __threadfence();
            __syncthreads();
            if (threadIdx.x == 0) s_last = atomicAdd(&long_done[r], 1u) == (uint32_t)(parts - 1) ? 1u : 0u;
            __syncthreads();
            finish = s_last != 0;
            if (finish && threadIdx.x < 64) {
                __threadfence();
                if (w == 0 && active) {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
                    add_partial<EPC>(acc, carry_tail + (size_t)j * dim + c * EPC);
                    // the part sums, eight loads at a time (indices clamped, so always in bounds)
                    typedef double __attribute__((ext_vector_type(2))) d2;
                    for (int64_t q0 = 0; q0 < parts; q0 += 8) {
                        d2 v[8][EPC / 2];
#pragma unroll
                        for (int qq = 0; qq < 8; ++qq) {
                            const int64_t q = min(q0 + qq, parts - 1);
                            const d2* src = (const d2*)(carry_head + (size_t)(j + 1 + q * per_part) * dim + c * EPC);
#pragma unroll
                            for (int e = 0; e < EPC / 2; ++e) v[qq][e] = src[e];
                        }
#pragma unroll
                        for (int qq = 0; qq < 8; ++qq)
                            if (q0 + qq < parts)
#pragma unroll
                                for (int e = 0; e < EPC / 2; ++e) {
                                    acc[2 * e] += v[qq][e].x;
                                    acc[2 * e + 1] += v[qq][e].y;
                                }
                    }
                }
            }
        }
        if (finish && w == 0 && active) {
            const uint32_t key = keys[min((uint32_t)(j + 1) * kSlice - 1, n - 1)];
            const uint32_t u = slice_base(j) + slice_runs[j] - 1;
            write_run<EPC, DENSE>(acc, key, u, c, dim, n, num_rows, grad_dense, uniq_grad);
        }
        __syncthreads();
    }
}

template <int CPR_T, bool BF16, bool DENSE>
hipError_t launch_reduce(const Layout& L, const char* ws, const void* grad_out, uint32_t n, uint32_t num_rows,
                         int cpr, int dim, float* grad_dense, float* uniq_grad, hipStream_t stream) {
    const int wpw = 64 / cpr;
    const int64_t waves = (L.num_slices + wpw - 1) / wpw;
    const int64_t grid = (waves + (kBlock / 64) - 1) / (kBlock / 64);
    const uint32_t ns = (uint32_t)L.num_slices;
    const uint32_t* sorted_keys = (const uint32_t*)(ws + L.sorted_keys);
    const uint32_t* sorted_vals = (const uint32_t*)(ws + L.sorted_vals);
    double* carry_head = (double*)(ws + L.carry_head);
    double* carry_tail = (double*)(ws + L.carry_tail);
    uint32_t* flags = (uint32_t*)(ws + L.slice_flags);
    uint32_t* counters = (uint32_t*)(ws + L.counters);
    uint32_t* long_runs = (uint32_t*)(ws + L.long_runs);
    uint32_t* long_done = (uint32_t*)(ws + L.long_done);
    uint32_t shift = 0;
    while ((kSlice << shift) < run_span(n)) ++shift;
    const RunBase base{(const uint32_t*)(ws + L.slice_base), (const uint32_t*)(ws + L.block_base), shift};
    hipLaunchKernelGGL((segment_reduce_kernel<CPR_T, BF16, DENSE>), dim3((unsigned)grid), dim3(kBlock), 0, stream,
                       sorted_keys, sorted_vals, counters, (const u32x4*)grad_out, n, num_rows, cpr, dim, ns,
                       base, (const uint32_t*)(ws + L.slice_first), grad_dense, uniq_grad, carry_head, carry_tail,
                       flags, long_done);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((carry_fixup_kernel<CPR_T, BF16, DENSE>), dim3((unsigned)grid), dim3(kBlock), 0, stream,
                       sorted_keys, counters, n, num_rows, cpr, dim, ns, (const uint32_t*)(ws + L.slice_runs), base,
                       (const uint32_t*)(ws + L.slice_first),
                       (const uint32_t*)flags, (const double*)carry_head,
                       (const double*)carry_tail, long_runs, grad_dense, uniq_grad);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const size_t share_bytes = (size_t)wpw * (kLongBlock / 64) * dim * sizeof(double);
    hipLaunchKernelGGL((long_run_kernel<CPR_T, BF16, DENSE>), dim3(256), dim3(kLongBlock), share_bytes, stream,
                       sorted_keys, (const uint32_t*)counters, n, num_rows, cpr, dim, ns,
                       (const uint32_t*)(ws + L.slice_runs), base, carry_head, (const double*)carry_tail,
                       (const uint32_t*)long_runs, long_done, grad_dense, uniq_grad);
    return hipGetLastError();
}

template <bool BF16, bool DENSE>
hipError_t dispatch_reduce(const Layout& L, const char* ws, const void* grad_out, uint32_t n, uint32_t num_rows,
                           int cpr, int dim, float* grad_dense, float* uniq_grad, hipStream_t stream) {
    if (BF16 && cpr == 20)
        return launch_reduce<20, BF16, DENSE>(L, ws, grad_out, n, num_rows, cpr, dim, grad_dense, uniq_grad, stream);
    if (!BF16 && cpr == 40)
        return launch_reduce<40, BF16, DENSE>(L, ws, grad_out, n, num_rows, cpr, dim, grad_dense, uniq_grad, stream);
    return launch_reduce<0, BF16, DENSE>(L, ws, grad_out, n, num_rows, cpr, dim, grad_dense, uniq_grad, stream);
}

// Steps 1-2: keys and the radix passes, ending in the sorted slots.
// The shape of one sort: its segments (one for the whole sort, kTokenHeads
// when split by head), the tiles per segment, the number of passes and the
// digit width of the last one.
struct SortShape {
    Segments sg;
    uint32_t num_segs;
    int passes, last_bits;
    size_t pass_words;  // chunk and group totals of one pass, all segments
    bool direct;        // split by head into short segments: no init kernel, first pass from tile counts
};

// One digit pass: the histogram (unless the keys kernel made it), then the scatter.
template <int ITEMS, int BITS>
hipError_t sort_pass(const SortShape& S, char* ws, const Layout& L, uint32_t* totals, bool first, int shift,
                     const uint32_t* k_cur, const uint32_t* v_cur, uint32_t* k_nxt, uint32_t* v_nxt,
                     hipStream_t stream) {
    static_assert(BITS == 8 || BITS == 9, "8- or 9-bit digits");
    constexpr int R = 1 << BITS;
    Segments sg = S.sg;
    sg.hist_words = sg.tiles * (uint32_t)R;
    sg.total_words = (uint32_t)count_words(sg.tiles, R);
    const DigitCounts dc = make_digit_counts(ws + L.hist, totals, sg.tiles, R);
    const uint32_t grid = sg.tiles * S.num_segs;
    if (!first) {
        hipLaunchKernelGGL((upsweep_kernel<ITEMS, BITS>), dim3(grid), dim3(kBlock), 0, stream, k_cur, shift, dc, sg);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const uint32_t* v_in = first ? nullptr : v_cur;
    if (BITS == 8 && first && S.direct)
        hipLaunchKernelGGL((downsweep_kernel<false, ITEMS, false, 8, true>), dim3(grid), dim3(kBlock), 0, stream,
                           k_cur, v_in, k_nxt, v_nxt, shift, dc, sg, GroupedOut{});
    else if (small_counts(dc))
        hipLaunchKernelGGL((downsweep_kernel<true, ITEMS, false, BITS>), dim3(grid), dim3(kBlock), 0, stream, k_cur,
                           v_in, k_nxt, v_nxt, shift, dc, sg, GroupedOut{});
    else
        hipLaunchKernelGGL((downsweep_kernel<false, ITEMS, false, BITS>), dim3(grid), dim3(kBlock), 0, stream, k_cur,
                           v_in, k_nxt, v_nxt, shift, dc, sg, GroupedOut{});
    return hipGetLastError();
}

template <int ITEMS>
hipError_t run_sort(const Layout& L, char* ws, const int64_t* rows, const TokenRows* tr, Padding pad, int64_t n,
                    int64_t row_begin, int64_t num_rows, const SortShape& S, int64_t* status, hipStream_t stream) {
    uint32_t* counters = (uint32_t*)(ws + L.counters);
    uint32_t* count_totals = (uint32_t*)(ws + L.count_totals);
    const uint32_t nn = (uint32_t)n, tiles = (uint32_t)L.num_tiles;
    const int passes = S.passes;
    hipError_t err;
    // Passes ping-pong between the two buffers and must end in the sorted slots.
    uint32_t *k_cur, *k_nxt, *v_cur, *v_nxt;
    if (passes % 2 == 0) {
        k_cur = (uint32_t*)(ws + L.sorted_keys); k_nxt = (uint32_t*)(ws + L.spare_keys);
        v_cur = (uint32_t*)(ws + L.sorted_vals); v_nxt = (uint32_t*)(ws + L.spare_vals);
    } else {
        k_cur = (uint32_t*)(ws + L.spare_keys); k_nxt = (uint32_t*)(ws + L.sorted_keys);
        v_cur = (uint32_t*)(ws + L.spare_vals); v_nxt = (uint32_t*)(ws + L.sorted_vals);
    }
    if (S.num_segs > 1) {
        Segments sg = S.sg;
        sg.hist_words = sg.tiles * (uint32_t)kRadix;
        sg.total_words = (uint32_t)count_words(sg.tiles);
        const DigitCounts dc0 = make_digit_counts(ws + L.hist, count_totals, sg.tiles);
        const dim3 grid(sg.tiles * S.num_segs);
        uint32_t* const zero_words = S.direct ? count_totals + S.pass_words : nullptr;
        const uint32_t zero_count = S.direct ? (uint32_t)(S.pass_words * (size_t)(passes - 1)) : 0u;
        const bool slice = tr->seq_begin != 0 || tr->width != tr->seq_len;
        if (S.direct && !slice)
            hipLaunchKernelGGL((head_keys_kernel<ITEMS, true, false>), grid, dim3(kBlock), 0, stream, *tr, row_begin,
                               sg, k_cur, dc0, counters, status, zero_words, zero_count);
        else if (S.direct)
            hipLaunchKernelGGL((head_keys_kernel<ITEMS, true, true>), grid, dim3(kBlock), 0, stream, *tr, row_begin,
                               sg, k_cur, dc0, counters, status, zero_words, zero_count);
        else if (!slice)
            hipLaunchKernelGGL((head_keys_kernel<ITEMS, false, false>), grid, dim3(kBlock), 0, stream, *tr,
                               row_begin, sg, k_cur, dc0, counters, status, zero_words, zero_count);
        else
            hipLaunchKernelGGL((head_keys_kernel<ITEMS, false, true>), grid, dim3(kBlock), 0, stream, *tr, row_begin,
                               sg, k_cur, dc0, counters, status, zero_words, zero_count);
    } else if (tr) {
        const DigitCounts dc0 = make_digit_counts(ws + L.hist, count_totals, tiles);
        if (tr->seq_begin != 0 || tr->width != tr->seq_len)
            hipLaunchKernelGGL((keys_kernel<ITEMS, true, true>), dim3(tiles), dim3(kBlock), 0, stream, nullptr, *tr,
                               nn, row_begin, (uint64_t)num_rows, k_cur, dc0, status, counters, Padding{});
        else
            hipLaunchKernelGGL((keys_kernel<ITEMS, true, false>), dim3(tiles), dim3(kBlock), 0, stream, nullptr, *tr,
                               nn, row_begin, (uint64_t)num_rows, k_cur, dc0, status, counters, Padding{});
    } else {
        hipLaunchKernelGGL((keys_kernel<ITEMS, false>), dim3(tiles), dim3(kBlock), 0, stream, rows, TokenRows{}, nn,
                           row_begin, (uint64_t)num_rows, k_cur, make_digit_counts(ws + L.hist, count_totals, tiles),
                           status, counters, pad);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    for (int p = 0; p < passes; ++p) {
        uint32_t* totals = count_totals + p * S.pass_words;
        if (p == passes - 1 && S.last_bits == 9)
            err = sort_pass<ITEMS, 9>(S, ws, L, totals, p == 0, 8 * p, k_cur, v_cur, k_nxt, v_nxt, stream);
        else
            err = sort_pass<ITEMS, 8>(S, ws, L, totals, p == 0, 8 * p, k_cur, v_cur, k_nxt, v_nxt, stream);
        if (err != hipSuccess) return err;
        uint32_t* t = k_cur; k_cur = k_nxt; k_nxt = t;
        t = v_cur; v_cur = v_nxt; v_nxt = t;
    }
    return hipSuccess;
}

// Whether the plan from tokens can split its sort by head, and with how many
// passes: every head's range [offset, offset + modulus) inside the shard,
// each starting at or after the previous one's end, and fewer passes over
// the bits of the largest modulus than over those of num_rows.
bool head_split(const TokenRows* tr, int64_t n, int64_t row_begin, int64_t num_rows, int whole_passes,
                int* passes, int* last_bits) {
    if (!tr || head_tiles(n) == 0) return false;
    uint64_t prev_end = 0, max_mod = 0;
    for (int h = 0; h < kTokenHeads; ++h) {
        const int64_t off = tr->p.off[h];
        const uint64_t mod = tr->p.mod[h];
        if (off < row_begin) return false;
        const uint64_t lo = (uint64_t)(off - row_begin);  // shard-relative start
        if (lo > (uint64_t)num_rows || mod > (uint64_t)num_rows - lo || lo < prev_end) return false;
        prev_end = lo + mod;
        max_mod = std::max(max_mod, mod);
    }
    int bits = 0;
    while (bits < 64 && ((max_mod - 1) >> bits) != 0) ++bits;  // keys below max_mod
    int p = bits <= 8 ? 1 : std::max(2, (bits - 1 + 7) / 8);
    if (p >= whole_passes) return false;
    *passes = p;
    *last_bits = 8 * p >= bits ? 8 : 9;
    return true;
}

}  // namespace

size_t scatter_workspace_bytes(int64_t n, int64_t num_rows, int dim) {
    (void)num_rows;
    return make_layout(n, dim).total;
}

namespace {

hipError_t scatter_plan(const int64_t* rows, const TokenRows* tr, Padding pad, int64_t n, int64_t row_begin,
                        int64_t num_rows,
                        int dim, int64_t* uniq_rows, int64_t* num_uniq, void* workspace, int64_t* status,
                        hipStream_t stream) {
    const Layout L = make_layout(n, dim);
    char* ws = (char*)workspace;
    uint32_t* counters = (uint32_t*)(ws + L.counters);
    int bits = 0;
    while (bits < 32 && ((uint64_t)num_rows >> bits) != 0) ++bits;  // the sentinel num_rows sorts last
    SortShape S;
    S.passes = (bits + 7) / 8;
    S.last_bits = 8;
    S.num_segs = 1;
    S.sg = one_segment((uint32_t)n, (uint32_t)L.num_tiles);
    S.pass_words = count_words(L.num_tiles);
    S.direct = false;
    int seg_passes, seg_last_bits;
    if (head_split(tr, n, row_begin, num_rows, S.passes, &seg_passes, &seg_last_bits)) {
        const int64_t ht = head_tiles(n);
        S.passes = seg_passes;
        S.last_bits = seg_last_bits;
        S.num_segs = kTokenHeads;
        S.sg.len = (uint32_t)(n / kTokenHeads);
        S.sg.tiles = (uint32_t)ht;
        S.sg.val_mul = kTokenHeads;  // entry pos of head h is lookup 16 pos + h
        for (int h = 0; h < kTokenHeads; ++h) S.sg.base[h] = (uint32_t)(tr->p.off[h] - row_begin);
        S.pass_words = (size_t)kTokenHeads * count_words(ht, kRadixWide);
        S.direct = ht <= (int64_t)kDirectTiles;
    }
    uint32_t* count_totals = (uint32_t*)(ws + L.count_totals);
    const uint32_t total_words = (uint32_t)(S.pass_words * S.passes);
    hipError_t err = hipSuccess;
    if (!S.direct) {  // the direct form's keys kernel does this itself
        const uint32_t init_grid = std::max(1u, std::min(64u, (total_words + kBlock - 1) / kBlock));
        hipLaunchKernelGGL(scatter_init_kernel, dim3(init_grid), dim3(kBlock), 0, stream, status, counters, num_uniq,
                           count_totals, total_words);
        err = hipGetLastError();
    }
    if (err != hipSuccess || n == 0) return err;
    const int items = sort_items(n);
    if (items == 8) err = run_sort<8>(L, ws, rows, tr, pad, n, row_begin, num_rows, S, status, stream);
    else if (items == 16) err = run_sort<16>(L, ws, rows, tr, pad, n, row_begin, num_rows, S, status, stream);
    else err = run_sort<24>(L, ws, rows, tr, pad, n, row_begin, num_rows, S, status, stream);
    if (err != hipSuccess) return err;

    const uint32_t nn = (uint32_t)n;
    const uint32_t* k_cur = (const uint32_t*)(ws + L.sorted_keys);
    const uint32_t ns = (uint32_t)L.num_slices;
    const uint32_t run_blocks = (uint32_t)L.num_run_blocks, span = run_span(n);
    hipLaunchKernelGGL(run_count_kernel, dim3(run_blocks), dim3(kBlock), 0, stream, k_cur, nn, counters,
                       (uint32_t*)(ws + L.slice_runs), (uint32_t*)(ws + L.slice_first),
                       (uint32_t*)(ws + L.slice_base), ns, (uint32_t*)(ws + L.block_runs), span);
    hipLaunchKernelGGL(block_scan_kernel, dim3(1), dim3(kScanBlock), 0, stream, (const uint32_t*)(ws + L.block_runs),
                       run_blocks, (uint32_t*)(ws + L.block_base), num_uniq);
    if (uniq_rows)
        hipLaunchKernelGGL(uniq_rows_kernel, dim3(run_blocks), dim3(kBlock), 0, stream, k_cur, nn, counters,
                           (const uint32_t*)(ws + L.block_base), row_begin, uniq_rows, span);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scatter_plan(const int64_t* rows, int64_t n, int64_t row_begin, int64_t num_rows, int dim,
                               int64_t* uniq_rows, int64_t* num_uniq, void* workspace, int64_t* status,
                               hipStream_t stream) {
    return scatter_plan(rows, nullptr, Padding{}, n, row_begin, num_rows, dim, uniq_rows, num_uniq, workspace, status,
                        stream);
}

hipError_t launch_scatter_plan_padded(const int64_t* ids, const int64_t* counts, int world, int64_t capacity,
                                      int64_t row_begin, int64_t num_rows, int dim, int64_t* uniq_rows,
                                      int64_t* num_uniq, void* workspace, int64_t* status, hipStream_t stream) {
    return scatter_plan(ids, nullptr, Padding{counts, (uint32_t)capacity}, (int64_t)world * capacity, row_begin,
                        num_rows, dim, uniq_rows, num_uniq, workspace, status, stream);
}

hipError_t launch_scatter_plan_tokens(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                                      int64_t seq_end, const HashParams& p, int64_t row_begin, int64_t num_rows,
                                      int dim, int64_t* uniq_rows, int64_t* num_uniq, void* workspace,
                                      int64_t* status, hipStream_t stream) {
    const TokenRows tr{tokens, (uint32_t)seq_len, p, (uint32_t)seq_begin, (uint32_t)(seq_end - seq_begin)};
    return scatter_plan(nullptr, &tr, Padding{}, batch * (seq_end - seq_begin) * kTokenHeads, row_begin, num_rows,
                        dim, uniq_rows,
                        num_uniq, workspace, status, stream);
}

hipError_t launch_scatter_apply(const void* grad_out, int elem_bytes, int dim, int64_t n, int64_t num_rows,
                                float* grad_dense, float* uniq_grad, const void* workspace, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const Layout L = make_layout(n, dim);
    const char* ws = (const char*)workspace;
    const int cpr = dim * elem_bytes / 16;
    const uint32_t nn = (uint32_t)n, nr = (uint32_t)num_rows;
    const bool bf16 = elem_bytes == 2, dense = grad_dense != nullptr;
    if (bf16 && dense) return dispatch_reduce<true, true>(L, ws, grad_out, nn, nr, cpr, dim, grad_dense, uniq_grad, stream);
    if (bf16) return dispatch_reduce<true, false>(L, ws, grad_out, nn, nr, cpr, dim, grad_dense, uniq_grad, stream);
    if (dense) return dispatch_reduce<false, true>(L, ws, grad_out, nn, nr, cpr, dim, grad_dense, uniq_grad, stream);
    return dispatch_reduce<false, false>(L, ws, grad_out, nn, nr, cpr, dim, grad_dense, uniq_grad, stream);
}

}  // namespace engram
