// Engram n-gram hash kernel for gfx950.
//
// Computes, for every position of every batch row, the global table row of
// each of the H = (ngram_size-1) * heads_per_ngram hash heads (engram API page
// "nemo_automodel.components.models.qwen3_8_flash_next.engram",
// Qwen3_8_FlashNextNGramEmbedding: class description, _shift_right_after_eos,
// _hash_input_ids):
//   * the token s positions back is the context of shift s unless it lies
//     before the row start or an EOS sits in [t-s, t-1] (context resets after
//     EOS); missing context takes the fill value;
//   * the order-n mix is the XOR of the 64-bit wrapped products
//     token[t-k] * multiplier[k], k < n;
//   * head h of order n: row = mix mod head_mod[h] (positive remainder) +
//     head_offset[h]; bigram heads come first, then trigram heads, ...
//
// One lane per position.  The wave shares its tokens through cross-lane
// shuffles: lane l reads position t-s from lane l-s, so only the first s
// lanes of a wave (and lanes right after a slice start) load history from
// memory.  The modulus uses a Barrett reduction with per-head reciprocals
// computed on the host: no 64-bit division on the GPU.
#include "engram_internal.h"
#include "hash_math.h"

namespace engram {
namespace {

// One wave per block: a wave's positions share nothing with other waves (its
// LDS rows are its own), and small token batches then spread over every
// compute unit instead of a few four-wave blocks.
constexpr int kHashBlock = 64;

template <int NG, int HPN>
__global__ __launch_bounds__(kHashBlock) void hash_kernel(const int64_t* __restrict__ tokens, int64_t seq_len,
                                                   int64_t seq_begin, int64_t width, int64_t total,
                                                   HashParams p, int64_t* __restrict__ rows_out) {
    const int ng = NG ? NG : p.ngram_size;
    const int hpn = HPN ? HPN : p.heads_per_ngram;
    const int heads = (ng - 1) * hpn;
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = g < total;
    int64_t b = 0, col = 0;
    if (live) {
        b = g / width;
        col = g - b * width;
    }
    const int64_t t = seq_begin + col;
    const int64_t* row = tokens + b * seq_len;
    const int64_t x = live ? row[t] : 0;

    // prod[k] = wrapped product of the shift-k context with multiplier k.
    uint64_t prod[kMaxNgram];
    prod[0] = (uint64_t)x * (uint64_t)p.mult[0];
    bool valid = true;  // no EOS in [t-s, t-1] and t-s >= 0
#pragma unroll
    for (int s = 1; s < kMaxNgram; ++s) {
        if (s >= ng) break;
        // Every lane takes part in the shuffle, live or not.
        int64_t prev = __shfl_up(x, s, 64);
        if (lane < s || col < s) prev = (live && t >= s) ? row[t - s] : 0;
        valid = valid && (t >= s) && (prev != p.eos);
        const int64_t ctx = valid ? prev : p.fill;
        prod[s] = (uint64_t)ctx * (uint64_t)p.mult[s];
    }
    uint64_t mix = prod[0];
    if (NG == 3 && HPN == 8) {
        // 16 rows per position.  A wave's 64 positions own one contiguous
        // 8 KiB span of the output; the rows go through LDS so that every
        // store instruction writes 1 KiB of consecutive 16-byte chunks.
        typedef long long i64x2 __attribute__((ext_vector_type(2)));
        constexpr int kPad = 18;  // int64 per position in LDS: 16 rows + 16 bytes against bank conflicts
        __shared__ int64_t s_rows[kHashBlock / 64][64 * kPad];
        int64_t* mine = &s_rows[threadIdx.x >> 6][lane * kPad];
        if (live) {
#pragma unroll
            for (int o = 2; o <= 3; ++o) {
                mix ^= prod[o - 1];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int h = (o - 2) * 8 + j;
                    mine[h] = (int64_t)floor_mod((int64_t)mix, p.mod[h], p.magic[h]) + p.off[h];
                }
            }
        }
        __syncthreads();  // every thread of the block reaches this barrier (none has returned)
        const int64_t wave_first = g - lane;                                // first position of this wave
        const int live_pos = (int)min((int64_t)64, total - wave_first);    // positions of the wave in range
        const int64_t* src = s_rows[threadIdx.x >> 6];
        i64x2* dst = (i64x2*)(rows_out + wave_first * 16);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int c = it * 64 + lane;  // 16-byte chunk of the wave's span: position c / 8, rows 2 (c % 8)
            const int pos = c >> 3;
            if (pos < live_pos) {
                const int64_t* q = src + pos * kPad + (c & 7) * 2;
                i64x2 v;
                v.x = q[0];
                v.y = q[1];
                dst[c] = v;
            }
        }
        return;
    }
    if (!live) return;
    int64_t* out = rows_out + g * heads;
    if (HPN == 8) {
#pragma unroll
        for (int o = 2; o <= kMaxNgram; ++o) {
            if (o > ng) break;
            mix ^= prod[o - 1];
            int64_t r[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int h = (o - 2) * 8 + j;
                r[j] = (int64_t)floor_mod((int64_t)mix, p.mod[h], p.magic[h]) + p.off[h];
            }
            // 4 x 16-byte stores per order.
            long long __attribute__((ext_vector_type(2)))* dst =
                (long long __attribute__((ext_vector_type(2)))*)(out + (o - 2) * 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                long long __attribute__((ext_vector_type(2))) v;
                v.x = r[2 * j];
                v.y = r[2 * j + 1];
                dst[j] = v;
            }
        }
    } else {
        for (int o = 2; o <= ng; ++o) {
            mix ^= prod[o - 1];
            for (int j = 0; j < hpn; ++j) {
                const int h = (o - 2) * hpn + j;
                out[h] = (int64_t)floor_mod((int64_t)mix, p.mod[h], p.magic[h]) + p.off[h];
            }
        }
    }
    (void)heads;
}

}  // namespace

hipError_t launch_hash(const int64_t* tokens, int64_t batch, int64_t seq_len, int64_t seq_begin,
                       int64_t seq_end, const HashParams& p, int64_t* rows_out, hipStream_t stream) {
    const int64_t width = seq_end - seq_begin;
    const int64_t total = batch * width;
    if (total == 0) return hipSuccess;
    const int block = kHashBlock;
    const int64_t grid = (total + block - 1) / block;
    if (p.ngram_size == 3 && p.heads_per_ngram == 8)
        hipLaunchKernelGGL((hash_kernel<3, 8>), dim3((unsigned)grid), dim3(block), 0, stream, tokens, seq_len,
                           seq_begin, width, total, p, rows_out);
    else if (p.heads_per_ngram == 8)
        hipLaunchKernelGGL((hash_kernel<0, 8>), dim3((unsigned)grid), dim3(block), 0, stream, tokens, seq_len,
                           seq_begin, width, total, p, rows_out);
    else
        hipLaunchKernelGGL((hash_kernel<0, 0>), dim3((unsigned)grid), dim3(block), 0, stream, tokens, seq_len,
                           seq_begin, width, total, p, rows_out);
    return hipGetLastError();
}

}  // namespace engram
