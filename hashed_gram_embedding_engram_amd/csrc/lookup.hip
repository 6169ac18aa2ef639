// Fused forward of the n-gram embedding for gfx950: the rows of a position are
// hashed and gathered by the wave that copies them, so the forward neither
// writes nor reads a rows array (engram API page,
// "nemo_automodel.components.models.qwen3_8_flash_next.engram":
// Qwen3_8_FlashNextNGramEmbedding hashes the input IDs (_hash_input_ids, with
// the context of _shift_right_after_eos) and looks the head rows up
// (_lookup_ngram_ids); Qwen3_8_FlashNextOwnerShardedEmbedding reads only the
// owner's rows and reports the others).
//
// One wave per position, for the released layout: 3-gram, 8 heads per order,
// so the position's 16 rows of a 160-wide bf16 table are one gather wave's
// work (gather.hip).  Lanes 0-2 load the tokens t, t-1 and t-2 of the
// position's batch row and the wave shares them; the context of shift s is
// the token s back unless it lies before the row start or an EOS sits in
// [t - s, t - 1], and missing context takes the fill value.  Lane h < 16
// computes head h's row (bigram heads 0-7 from the order-2 mix, trigram heads
// 8-15 from the order-3 mix, each the XOR of 64-bit wrapped products), checks
// it against the shard, and optionally stores it.  The rows then go to
// copy_wave_rows as the gather's do.
#include "hash_math.h"
#include "lookup.h"
#include "row_copy.h"

namespace engram {
namespace {

constexpr int kLookupBlock = 256;
constexpr int kLookupHeads = 16;

// Read by lanes that have no row to copy, so loads never need a branch.
__device__ u32x4 kLookupZero = {0u, 0u, 0u, 0u};  // never written

// Same occupancy cap as the gather kernel (four waves per SIMD): the copy is
// the same, and the backward's plan runs beside it on another stream.
// Positions [seq_begin, seq_begin + width) of every batch row (the whole row
// when seq_begin = 0 and width = seq_len): position pos of the output is batch
// row pos / width, column seq_begin + pos % width, hashed with the columns
// before it (a context-parallel rank's slice of a global sequence).
template <bool ROW32, bool ROWS_OUT>
__global__ __launch_bounds__(kLookupBlock) __attribute__((amdgpu_waves_per_eu(1, 4))) void hash_gather_kernel(
    const int64_t* __restrict__ tokens, int64_t seq_len, int64_t seq_begin, int64_t width, int64_t positions,
    HashParams p, const u32x4* __restrict__ table, int64_t row_begin, uint64_t num_rows, u32x4* __restrict__ out,
    int64_t* __restrict__ rows_out, int64_t* __restrict__ status) {
    const int lane = threadIdx.x & 63;
    const int64_t pos = (int64_t)blockIdx.x * (kLookupBlock / 64) + (threadIdx.x >> 6);
    if (pos >= positions) return;
    const int64_t b = pos / width, t = seq_begin + (pos - b * width);
    int64_t tok = 0;
    if (lane < 3 && t >= lane) tok = tokens[b * seq_len + t - lane];
    const int64_t x0 = __shfl(tok, 0, 64), x1 = __shfl(tok, 1, 64), x2 = __shfl(tok, 2, 64);
    const bool valid1 = t >= 1 && x1 != p.eos;
    const bool valid2 = valid1 && t >= 2 && x2 != p.eos;
    const int64_t ctx1 = valid1 ? x1 : p.fill, ctx2 = valid2 ? x2 : p.fill;
    const uint64_t mix2 = (uint64_t)x0 * (uint64_t)p.mult[0] ^ (uint64_t)ctx1 * (uint64_t)p.mult[1];
    const uint64_t mix3 = mix2 ^ (uint64_t)ctx2 * (uint64_t)p.mult[2];
    // Head h's modulus, reciprocal and offset for lane h (selected with
    // compile-time indices: the parameters stay kernel arguments).
    uint64_t mod = p.mod[0], magic = p.magic[0];
    int64_t off = p.off[0];
#pragma unroll
    for (int j = 1; j < kLookupHeads; ++j)
        if (lane == j) {
            mod = p.mod[j];
            magic = p.magic[j];
            off = p.off[j];
        }
    const int64_t n0 = pos * kLookupHeads;
    uint64_t local = ~0ull;
    if (lane < kLookupHeads) {
        const int64_t row = (int64_t)floor_mod((int64_t)(lane < 8 ? mix2 : mix3), mod, magic) + off;
        if (ROWS_OUT) rows_out[n0 + lane] = row;
        local = (uint64_t)row - (uint64_t)row_begin;
        if (local >= num_rows) {
            if (status) atomicMin((unsigned long long*)status, (unsigned long long)(n0 + lane));
            local = ~0ull;
        }
    }
    copy_wave_rows<20, kLookupHeads, ROW32, false>(table, local, n0, n0 + kLookupHeads, out, lane, &kLookupZero);
}

}  // namespace

bool hash_gather_fused(const HashParams& p, int elem_bytes, int dim, int64_t positions) {
    return p.ngram_size == 3 && p.heads_per_ngram == 8 && elem_bytes == 2 && dim == 160 &&
           positions <= kLookupMaxPositions;
}

hipError_t launch_hash_gather(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                              int64_t seq_end, const HashParams& p, const void* table, int elem_bytes,
                              int64_t row_begin, int64_t num_rows, int dim, void* out, int64_t* rows_out,
                              int64_t* status, hipStream_t stream) {
    const int64_t width = seq_end - seq_begin;
    const int64_t positions = batch * width;
    if (!hash_gather_fused(p, elem_bytes, dim, positions)) {
        // Two kernels through the caller's rows array.
        hipError_t err = launch_hash(tokens, batch, seq_len, seq_begin, seq_end, p, rows_out, stream);
        if (err != hipSuccess) return err;
        const int64_t heads = (int64_t)(p.ngram_size - 1) * p.heads_per_ngram;
        return launch_gather(table, elem_bytes, row_begin, num_rows, dim, rows_out, positions * heads, out, status,
                             stream);
    }
    hipError_t err = launch_status_init(status, stream);
    if (err != hipSuccess || positions == 0) return err;
    const dim3 grid((unsigned)((positions + kLookupBlock / 64 - 1) / (kLookupBlock / 64)));
    const bool row32 = (uint64_t)num_rows < 0xFFFFFFFFull;
    const u32x4* t = (const u32x4*)table;
    u32x4* o = (u32x4*)out;
    if (row32 && rows_out)
        hipLaunchKernelGGL((hash_gather_kernel<true, true>), grid, dim3(kLookupBlock), 0, stream, tokens, seq_len,
                           seq_begin, width, positions, p, t, row_begin, (uint64_t)num_rows, o, rows_out, status);
    else if (row32)
        hipLaunchKernelGGL((hash_gather_kernel<true, false>), grid, dim3(kLookupBlock), 0, stream, tokens, seq_len,
                           seq_begin, width, positions, p, t, row_begin, (uint64_t)num_rows, o, rows_out, status);
    else if (rows_out)
        hipLaunchKernelGGL((hash_gather_kernel<false, true>), grid, dim3(kLookupBlock), 0, stream, tokens, seq_len,
                           seq_begin, width, positions, p, t, row_begin, (uint64_t)num_rows, o, rows_out, status);
    else
        hipLaunchKernelGGL((hash_gather_kernel<false, false>), grid, dim3(kLookupBlock), 0, stream, tokens, seq_len,
                           seq_begin, width, positions, p, t, row_begin, (uint64_t)num_rows, o, rows_out, status);
    return hipGetLastError();
}

}  // namespace engram
