// PLE causal short convolution and grouped Gemma RMSNorm for gfx950.
//
// Engram API page ("nemo_automodel.components.models.qwen3_8_flash_next.engram"),
// Qwen3_8_FlashNextPLELayer._causal_short_conv: causal depthwise convolution
// over the sequence of [batch, sequence, channels], kernel width K (4) and
// dilation d (ngram_size = 3), left zero history; under context parallelism a
// shard receives the preceding (K - 1) * d = 9 tokens as a halo.  Tap k
// multiplies the input (K - 1 - k) * d positions back.
// Layers API page ("nemo_automodel.components.models.qwen3_8_flash_next.layers"),
// Qwen3_8_FlashNextGroupedRMSNorm / _grouped_rms_norm_fp32: each group of
// `group` features is scaled by 1 / sqrt(mean(x^2) + eps) and by (1 + weight),
// in fp32.
//
// All of these are HBM-bound streams: one read of each input and one write of
// each output per element.  Arithmetic is fp32 per element; the weight
// gradients (sums over every batch row and position) are accumulated per tile
// and then reduced over the tiles in a fixed order in fp64, so they are
// deterministic.
#include <algorithm>
#include <type_traits>

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kPleBlock = 256;

// 16-byte chunk of VEC elements: bf16 (VEC 8) or fp32 (VEC 4), as fp32 values.
template <bool BF16>
__device__ __forceinline__ void unpack16(u32x4 v, float* f) {
    if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = __uint_as_float(v[q] << 16);
            f[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) f[q] = __uint_as_float(v[q]);
    }
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack16(const float* f) {
    u32x4 v;
    if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = bf16_bits(f[2 * q]) | (bf16_bits(f[2 * q + 1]) << 16);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __float_as_uint(f[q]);
    }
    return v;
}

__device__ u32x4 kPleZero = {0u, 0u, 0u, 0u};  // never written

// Four channels per thread: 8 bytes in bf16, 16 bytes in fp32.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <bool BF16>
using Quad = typename std::conditional<BF16, u32x2, u32x4>::type;

template <bool BF16>
__device__ __forceinline__ void unpack4(Quad<BF16> v, float* f) {
    if constexpr (BF16) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            f[2 * q] = __uint_as_float(v[q] << 16);
            f[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) f[q] = __uint_as_float(v[q]);
    }
}

template <bool BF16>
__device__ __forceinline__ Quad<BF16> pack4(const float* f) {
    Quad<BF16> v;
    if constexpr (BF16) {
        v[0] = bf16_bits(f[0]) | (bf16_bits(f[1]) << 16);
        v[1] = bf16_bits(f[2]) | (bf16_bits(f[3]) << 16);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __float_as_uint(f[q]);
    }
    return v;
}

// ---------------------------------------------------------------- convolution

// Input chunk at sequence position ts of batch row b: x when ts >= 0, the halo
// when -H <= ts < 0 and a halo is given, else zero (left zero history).
__device__ __forceinline__ const u32x4* conv_src(const u32x4* x, const u32x4* halo, int64_t b, int64_t S, int64_t H,
                                                  int64_t chunks, int64_t ch, int64_t ts) {
    if (ts >= 0) return x + ((b * S + ts) * chunks + ch);
    if (halo && ts >= -H) return halo + ((b * H + H + ts) * chunks + ch);
    return &kPleZero;
}

template <bool BF16, int K>
__global__ __launch_bounds__(kPleBlock) void short_conv_fwd_kernel(const u32x4* __restrict__ x,
                                                                   const u32x4* __restrict__ halo,
                                                                   const float* __restrict__ w,
                                                                   const float* __restrict__ bias, int64_t B,
                                                                   int64_t S, int64_t C, int d, int tile,
                                                                   u32x4* __restrict__ y) {
    constexpr int VEC = BF16 ? 8 : 4;
    const int64_t chunks = C / VEC, tiles = (S + tile - 1) / tile;
    const int64_t idx = (int64_t)blockIdx.x * kPleBlock + threadIdx.x;
    if (idx >= B * tiles * chunks) return;
    const int64_t ch = idx % chunks, rest = idx / chunks, tt = rest % tiles, b = rest / tiles;
    const int64_t H = (int64_t)(K - 1) * d;
    float wv[VEC][K], bv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
#pragma unroll
        for (int k = 0; k < K; ++k) wv[e][k] = w[(ch * VEC + e) * K + k];
        bv[e] = bias ? bias[ch * VEC + e] : 0.0f;
    }
    const int64_t t1 = min(S, (tt + 1) * tile);
    for (int64_t t = tt * tile; t < t1; ++t) {
        u32x4 raw[K];
#pragma unroll
        for (int k = 0; k < K; ++k) raw[k] = *conv_src(x, halo, b, S, H, chunks, ch, t - (int64_t)(K - 1 - k) * d);
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = bv[e];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float f[VEC];
            unpack16<BF16>(raw[k], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = fmaf(wv[e][k], f[e], acc[e]);
        }
        y[(b * S + t) * chunks + ch] = pack16<BF16>(acc);
    }
}

// dx (and the halo's gradient for the first tile) plus per-tile fp64 partial
// sums of dweight and dbias.  partial: [B * tiles][C][K + 1].
template <bool BF16, int K>
__global__ __launch_bounds__(kPleBlock) void short_conv_bwd_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ dy, const u32x4* __restrict__ halo,
    const float* __restrict__ w, int64_t B, int64_t S, int64_t C, int d, int tile, u32x4* __restrict__ dx,
    u32x4* __restrict__ dhalo, double* __restrict__ partial) {
    constexpr int VEC = BF16 ? 8 : 4;
    const int64_t chunks = C / VEC, tiles = (S + tile - 1) / tile;
    const int64_t idx = (int64_t)blockIdx.x * kPleBlock + threadIdx.x;
    if (idx >= B * tiles * chunks) return;
    const int64_t ch = idx % chunks, rest = idx / chunks, tt = rest % tiles, b = rest / tiles;
    const int64_t H = (int64_t)(K - 1) * d;
    float wv[VEC][K];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int k = 0; k < K; ++k) wv[e][k] = w[(ch * VEC + e) * K + k];
    float pw[VEC][K + 1];  // fp32 within a tile, fp64 across tiles
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int k = 0; k <= K; ++k) pw[e][k] = 0.0f;
    // dy at positions past the end is zero: it reads the zero chunk
    auto dy_src = [&](int64_t ts) -> const u32x4* {
        return ts < S ? dy + ((b * S + ts) * chunks + ch) : &kPleZero;
    };
    const int64_t t0 = tt * tile, t1 = min(S, t0 + tile);
    for (int64_t t = t0; t < t1; ++t) {
        u32x4 g[K], xs[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            g[k] = *dy_src(t + (int64_t)(K - 1 - k) * d);
            xs[k] = *conv_src(x, halo, b, S, H, chunks, ch, t - (int64_t)(K - 1 - k) * d);
        }
        float acc[VEC], gt[VEC];
        unpack16<BF16>(g[K - 1], gt);  // dy at t itself
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float f[VEC], xf[VEC];
            unpack16<BF16>(g[k], f);
            unpack16<BF16>(xs[k], xf);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                acc[e] = fmaf(wv[e][k], f[e], acc[e]);
                pw[e][k] = fmaf(gt[e], xf[e], pw[e][k]);
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) pw[e][K] += gt[e];
        dx[(b * S + t) * chunks + ch] = pack16<BF16>(acc);
    }
    if (dhalo && tt == 0) {
        for (int64_t j = 0; j < H; ++j) {  // halo position j is sequence position j - H
            float acc[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int64_t ts = j - H + (int64_t)(K - 1 - k) * d;
                float f[VEC];
                unpack16<BF16>(ts >= 0 ? *dy_src(ts) : kPleZero, f);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] = fmaf(wv[e][k], f[e], acc[e]);
            }
            dhalo[(b * H + j) * chunks + ch] = pack16<BF16>(acc);
        }
    }
    double* p = partial + ((b * tiles + tt) * C + ch * VEC) * (K + 1);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int k = 0; k <= K; ++k) p[e * (K + 1) + k] = (double)pw[e][k];
}

// ---- dilation 3 (the released layer): sliding register windows
//
// One thread owns four channels of one batch row over a tile of positions
// (kConvTile in the backward, kConvTileUp in the forward) and walks them
// kConvStep positions at a time.  Its window holds the inputs from
// HIST = (K - 1) * 3 positions back up to the current step, so every input is
// loaded once per tile (plus the HIST-position overlap with the previous tile)
// instead of once per tap.  Window indices are compile-time constants: the
// window lives in registers.
//
// A block is four waves over four consecutive tiles of the same 64 quads
// (wave w takes tile 4 * tile_group + w), and consecutive tile groups of the
// same quads are qgroups blocks apart, which lands them on the same XCD when
// qgroups is a multiple of 8 (40 at 10,240 channels).  Odd waves walk their
// tile from its end down: the rows on both sides of every tile edge are then
// read by the two neighbouring waves at about the same time (both at the end
// of their walks, or both at the start), so the overlap rows come from L2
// instead of being fetched twice.

// Build-time tuning parameters (positions per step, positions per tile of the
// backward and of the forward), at the measured best of steps 3, 6, 9, of
// backward tiles 48, 72, 96, 144, 192, and of forward tiles 24 to 96.  The streaming
// outputs of the norm kernels and of the convolution backward are stored
// non-temporally (each 3-5% faster at [8, 4096, 10240]); the convolution
// forward keeps plain stores (1.7% slower with them).
#ifndef ENGRAM_CONV_STEP
#define ENGRAM_CONV_STEP 3
#endif
#ifndef ENGRAM_CONV_TILE
#define ENGRAM_CONV_TILE 96
#endif
#ifndef ENGRAM_CONV_TILE_UP
#define ENGRAM_CONV_TILE_UP 48
#endif
constexpr int kConvD = 3;
constexpr int kConvStep = ENGRAM_CONV_STEP;
constexpr int kConvTile = ENGRAM_CONV_TILE;      // backward: positions per thread (multiple of kConvStep)
constexpr int kConvTileUp = ENGRAM_CONV_TILE_UP;  // forward: positions per thread (multiple of kConvStep)
constexpr int kConvWavesPerBlock = kPleBlock / 64;

template <bool BF16, int K>
__global__ __launch_bounds__(kPleBlock) void short_conv_fwd_d3_kernel(const void* __restrict__ xp,
                                                                      const void* __restrict__ halop,
                                                                      const float* __restrict__ w,
                                                                      const float* __restrict__ bias, int64_t B,
                                                                      int64_t S, int64_t C, void* __restrict__ yp) {
    using Q = Quad<BF16>;
    constexpr int HIST = (K - 1) * kConvD, P = kConvStep;
    const Q* halo = (const Q*)halop;
    const Q* zero = (const Q*)&kPleZero;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t quads = C / 4, tiles = (S + kConvTileUp - 1) / kConvTileUp;
    const int64_t tgroups = (tiles + kConvWavesPerBlock - 1) / kConvWavesPerBlock, qgroups = (quads + 63) / 64;
    const int64_t qg = blockIdx.x % qgroups, rest = blockIdx.x / qgroups, tg = rest % tgroups, b = rest / tgroups;
    const int64_t q = qg * 64 + lane, tt = tg * kConvWavesPerBlock + wave;
    const int64_t t0 = min(S, tt * kConvTileUp), t1 = min(S, t0 + kConvTileUp);
    if (q >= quads || t1 <= t0) return;  // no barrier or cross-lane step below
    float wv[4][K], bv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int k = 0; k < K; ++k) wv[e][k] = w[(q * 4 + e) * K + k];
        bv[e] = bias ? bias[q * 4 + e] : 0.0f;
    }
    const Q* xb = (const Q*)xp + b * S * quads + q;
    auto xsrc = [&](int64_t tx) -> const Q* {
        return tx >= S ? zero : tx >= 0 ? xb + tx * quads : (halo ? halo + ((b * HIST + HIST + tx) * quads + q) : zero);
    };
    Q* yb = (Q*)yp + b * S * quads + q;
    auto step = [&](int64_t t, const Q (&win)[HIST + P]) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            if (t + j >= t1) break;  // wave-uniform
            float acc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = bv[e];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float f[4];
                unpack4<BF16>(win[HIST + j - (K - 1 - k) * kConvD], f);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(wv[e][k], f[e], acc[e]);
            }
            yb[(t + j) * quads] = pack4<BF16>(acc);
        }
    };
    if ((wave & 1) == 0) {  // up from t0
        Q win[HIST + P];  // x at t - HIST .. t + P - 1
#pragma unroll
        for (int i = 0; i < HIST; ++i) win[i] = *xsrc(t0 - HIST + i);
        for (int64_t t = t0; t < t1; t += P) {
#pragma unroll
            for (int j = 0; j < P; ++j) win[HIST + j] = *xsrc(t + j);
            step(t, win);
#pragma unroll
            for (int i = 0; i < HIST; ++i) win[i] = win[i + P];
        }
    } else {  // down from the last step; the step below reuses the window's lowest HIST rows as its highest
        Q win[HIST + P];
        int64_t t = t0 + ((t1 - t0 - 1) / P) * P;
#pragma unroll
        for (int i = 0; i < HIST; ++i) win[P + i] = *xsrc(t - HIST + P + i);
        for (; t >= t0; t -= P) {
#pragma unroll
            for (int j = 0; j < P; ++j) win[j] = *xsrc(t - HIST + j);
            step(t, win);
#pragma unroll
            for (int i = HIST - 1; i >= 0; --i) win[P + i] = win[i];
        }
    }
}

// Backward, dilation 3.  A block is four waves over four consecutive tiles of
// the same 64 quads; wave w takes tile 4 * tile_group + w, odd waves walking
// down as in the forward.  Every wave keeps
// fp32 sums of dweight / dbias over its tile; the four are added in wave order
// in fp64 and written as one partial per (batch row, tile group):
// partial [B * tile_groups][C][K + 1].
template <bool BF16, int K>
__global__ __launch_bounds__(kPleBlock) void short_conv_bwd_d3_kernel(
    const void* __restrict__ xp, const void* __restrict__ dyp, const void* __restrict__ halop,
    const float* __restrict__ w, int64_t B, int64_t S, int64_t C, void* __restrict__ dxp, void* __restrict__ dhalop,
    double* __restrict__ partial) {
    using Q = Quad<BF16>;
    constexpr int HIST = (K - 1) * kConvD, P = kConvStep;
    __shared__ float s_part[kConvWavesPerBlock][K + 1][4][64];
    const Q* zero = (const Q*)&kPleZero;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t quads = C / 4, tiles = (S + kConvTile - 1) / kConvTile;
    const int64_t tgroups = (tiles + kConvWavesPerBlock - 1) / kConvWavesPerBlock, qgroups = (quads + 63) / 64;
    const int64_t qg = blockIdx.x % qgroups, rest = blockIdx.x / qgroups, tg = rest % tgroups, b = rest / tgroups;
    const int64_t q = qg * 64 + lane, tt = tg * kConvWavesPerBlock + wave;
    const bool live = q < quads;
    const int64_t qc = live ? q : quads - 1;  // clamped: loads stay in bounds, nothing is stored
    float wv[4][K], pw[4][K + 1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int k = 0; k < K; ++k) wv[e][k] = w[(qc * 4 + e) * K + k];
#pragma unroll
        for (int k = 0; k <= K; ++k) pw[e][k] = 0.0f;
    }
    const Q* xb = (const Q*)xp + b * S * quads + qc;
    const Q* gb = (const Q*)dyp + b * S * quads + qc;
    const Q* halo = (const Q*)halop;
    const int64_t t0 = min(S, tt * kConvTile), t1 = min(S, t0 + kConvTile);  // empty for a tile past the end
    Q* dxb = (Q*)dxp + b * S * quads + q;
    // x at position tx (halo before 0, zero from S on)
    auto xsrc = [&](int64_t tx) -> const Q* {
        return tx >= S ? zero : tx >= 0 ? xb + tx * quads : (halo ? halo + ((b * HIST + HIST + tx) * quads + qc) : zero);
    };
    auto gsrc = [&](int64_t tg) -> const Q* { return tg < S ? gb + tg * quads : zero; };
    auto step = [&](int64_t t, const Q (&xw)[HIST + P], const Q (&gw)[HIST + P]) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            if (t + j >= t1) break;  // wave-uniform
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, g[4];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float f[4];
                unpack4<BF16>(gw[j + (K - 1 - k) * kConvD], f);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(wv[e][k], f[e], acc[e]);
            }
            if (live) __builtin_nontemporal_store(pack4<BF16>(acc), dxb + (t + j) * quads);
            unpack4<BF16>(gw[j], g);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float xf[4];
                unpack4<BF16>(xw[HIST + j - (K - 1 - k) * kConvD], xf);
#pragma unroll
                for (int e = 0; e < 4; ++e) pw[e][k] = fmaf(g[e], xf[e], pw[e][k]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) pw[e][K] += g[e];
        }
    };
    if ((wave & 1) == 0 || t1 <= t0) {  // up from t0
        Q xw[HIST + P];  // x at t - HIST .. t + P - 1
        Q gw[HIST + P];  // dy at t .. t + HIST + P - 1
#pragma unroll
        for (int i = 0; i < HIST; ++i) {
            xw[i] = *xsrc(t0 - HIST + i);
            gw[i] = *gsrc(t0 + i);
        }
        if (dhalop && tt == 0 && t1 > t0 && live) {
#pragma unroll
            for (int i = 0; i < HIST; ++i) {
                float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int off = i - HIST + (K - 1 - k) * kConvD;
                    if (off >= 0) {
                        float f[4];
                        unpack4<BF16>(gw[off], f);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[e] = fmaf(wv[e][k], f[e], acc[e]);
                    }
                }
                ((Q*)dhalop)[(b * HIST + i) * quads + q] = pack4<BF16>(acc);
            }
        }
        // Each step's inputs are loaded one step ahead, so two steps of loads
        // are in flight; past the tile's last step the current one is loaded
        // again (in bounds, unused).
        Q xn[P], gn[P];
#pragma unroll
        for (int j = 0; j < P; ++j) {
            xn[j] = *xsrc(t0 + j);
            gn[j] = *gsrc(t0 + HIST + j);
        }
        for (int64_t t = t0; t < t1; t += P) {
#pragma unroll
            for (int j = 0; j < P; ++j) {
                xw[HIST + j] = xn[j];
                gw[HIST + j] = gn[j];
            }
            const int64_t tn = t + P < t1 ? t + P : t;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                xn[j] = *xsrc(tn + j);
                gn[j] = *gsrc(tn + HIST + j);
            }
            step(t, xw, gw);
#pragma unroll
            for (int i = 0; i < HIST; ++i) {
                xw[i] = xw[i + P];
                gw[i] = gw[i + P];
            }
        }
    } else {  // down from the last step, the windows shifting up
        Q xw[HIST + P];
        Q gw[HIST + P];
        int64_t t = t0 + ((t1 - t0 - 1) / P) * P;
#pragma unroll
        for (int i = 0; i < HIST; ++i) {
            xw[P + i] = *xsrc(t - HIST + P + i);
            gw[P + i] = *gsrc(t + P + i);
        }
        Q xn[P], gn[P];  // one step ahead, as in the walk up
#pragma unroll
        for (int j = 0; j < P; ++j) {
            xn[j] = *xsrc(t - HIST + j);
            gn[j] = *gsrc(t + j);
        }
        for (; t >= t0; t -= P) {
#pragma unroll
            for (int j = 0; j < P; ++j) {
                xw[j] = xn[j];
                gw[j] = gn[j];
            }
            const int64_t tn = t - P >= t0 ? t - P : t;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                xn[j] = *xsrc(tn - HIST + j);
                gn[j] = *gsrc(tn + j);
            }
            step(t, xw, gw);
#pragma unroll
            for (int i = HIST - 1; i >= 0; --i) {
                xw[P + i] = xw[i];
                gw[P + i] = gw[i];
            }
        }
    }
#pragma unroll
    for (int k = 0; k <= K; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_part[wave][k][e][lane] = pw[e][k];
    __syncthreads();
    if (wave == 0 && live) {
        double* out = partial + ((b * tgroups + tg) * C + q * 4) * (K + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int k = 0; k <= K; ++k) {
                double sum = 0.0;
#pragma unroll
                for (int v = 0; v < kConvWavesPerBlock; ++v) sum += (double)s_part[v][k][e][lane];
                out[e * (K + 1) + k] = sum;
            }
    }
}

// Column sums of partial [parts][cols] in fp64: each of the block's
// kSumWaves waves sums one contiguous slice of the parts in part order, and
// the slice sums are then added in slice order (deterministic).  With
// K1 = K + 1 > 0 the columns are (channel, tap or bias) of the convolution:
// column c * K1 + k goes to dw[c * K + k] for k < K and to db[c] for k == K;
// with K1 == 0 column i goes to dw[i].
constexpr int kSumWaves = 16;

__global__ __launch_bounds__(64 * kSumWaves) void column_sum_kernel(const double* __restrict__ partial, int64_t parts,
                                                                    int64_t cols, int K1, float* __restrict__ dw,
                                                                    float* __restrict__ db) {
    __shared__ double s_sum[kSumWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t col = (int64_t)blockIdx.x * 64 + lane;
    const int64_t cc = col < cols ? col : cols - 1;
    const int64_t per = (parts + kSumWaves - 1) / kSumWaves, p0 = min(parts, wave * per), p1 = min(parts, p0 + per);
    double s = 0.0;
    for (int64_t p = p0; p < p1; ++p) s += partial[p * cols + cc];
    s_sum[wave][lane] = s;
    __syncthreads();
    if (wave != 0 || col >= cols) return;
    double total = 0.0;
#pragma unroll
    for (int v = 0; v < kSumWaves; ++v) total += s_sum[v][lane];
    if (K1 == 0) {
        dw[col] = (float)total;
    } else {
        const int64_t c = col / K1, k = col % K1;
        if (k < K1 - 1)
            dw[c * (K1 - 1) + k] = (float)total;
        else if (db)
            db[c] = (float)total;
    }
}

// ---------------------------------------------------------------- grouped RMSNorm

constexpr int kNormMaxChunks = 10;  // 16-byte chunks per lane: group * elem_bytes <= 10240

// One wave per (row, group); lanes own chunks lane, lane + 64, ...; CH is the
// number of chunks per lane, ceil(group / VEC / 64).
template <bool BF16, int CH>
__global__ __launch_bounds__(kPleBlock) void rms_norm_fwd_kernel(const u32x4* __restrict__ x,
                                                                 const float* __restrict__ w, int64_t rows,
                                                                 int64_t hidden, int64_t group, float eps,
                                                                 u32x4* __restrict__ y) {
    constexpr int VEC = BF16 ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int64_t groups = hidden / group, gchunks = group / VEC, hchunks = hidden / VEC;
    const int64_t wave = (int64_t)blockIdx.x * (kPleBlock / 64) + (threadIdx.x >> 6);
    if (wave >= rows * groups) return;
    const int64_t r = wave / groups, g = wave - r * groups;
    const u32x4* xr = x + r * hchunks + g * gchunks;
    u32x4 v[CH];
    float ss = 0.0f;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int64_t c = lane + 64 * q;
        v[q] = *(c < gchunks ? xr + c : &kPleZero);  // unconditional load
        float f[VEC];
        unpack16<BF16>(v[q], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss = fmaf(f[e], f[e], ss);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float inv = 1.0f / sqrtf(ss / (float)group + eps);
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int64_t c = lane + 64 * q;
        if (c >= gchunks) break;
        float f[VEC];
        unpack16<BF16>(v[q], f);
        const float* wg = w + g * group + c * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) f[e] = f[e] * inv * (1.0f + wg[e]);
        __builtin_nontemporal_store(pack16<BF16>(f), y + r * hchunks + g * gchunks + c);
    }
}

// dx per row, and the weight gradient's sums.  A block's four waves share
// one group g (its 1 + weight is staged once in LDS) and take four
// consecutive blocks of rows_per_wave rows.  Each wave keeps fp32 sums over
// its rows in LDS (each lane owns its features' slots, so no atomics); the
// four are added in wave order in fp64 and written as one partial per block:
// partial [ceil(rows / (4 * rows_per_wave))][hidden].  The next row's loads
// are issued before the current row's reductions.
template <bool BF16, int CH>
__global__ __launch_bounds__(kPleBlock) void rms_norm_bwd_kernel(const u32x4* __restrict__ x,
                                                                 const u32x4* __restrict__ dy,
                                                                 const float* __restrict__ w, int64_t rows,
                                                                 int64_t hidden, int64_t group, float eps,
                                                                 int rows_per_wave, u32x4* __restrict__ dx,
                                                                 double* __restrict__ partial) {
    constexpr int VEC = BF16 ? 8 : 4, H4 = VEC / 4, WAVES = kPleBlock / 64;
    __shared__ float4 s_pw[WAVES][CH * H4][64];
    __shared__ float4 s_wp[CH * H4][64];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t groups = hidden / group, gchunks = group / VEC, hchunks = hidden / VEC;
    const int64_t g = blockIdx.x % groups, bb = blockIdx.x / groups;
    for (int i = threadIdx.x; i < CH * H4 * 64; i += kPleBlock) {
        const int ln = i & 63, qh = i >> 6, q = qh / H4, h = qh % H4;
        const int64_t c = ln + 64 * q;
        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (c < gchunks) {
            const float* wg = w + g * group + c * VEC + 4 * h;
            v = make_float4(1.0f + wg[0], 1.0f + wg[1], 1.0f + wg[2], 1.0f + wg[3]);
        }
        s_wp[qh][ln] = v;
        s_pw[0][qh][ln] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        s_pw[1][qh][ln] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        s_pw[2][qh][ln] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        s_pw[3][qh][ln] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    __syncthreads();
    const int64_t r0 = min(rows, (bb * WAVES + wid) * rows_per_wave), r1 = min(rows, r0 + rows_per_wave);
    u32x4 xa[CH], ga[CH];
    auto load_row = [&](int64_t r, u32x4* xv, u32x4* gv) {
        const int64_t base = r * hchunks + g * gchunks;
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            const int64_t c = lane + 64 * q;
            xv[q] = *(c < gchunks ? x + base + c : &kPleZero);  // unconditional loads
            gv[q] = *(c < gchunks ? dy + base + c : &kPleZero);
        }
    };
    if (r0 < r1) load_row(r0, xa, ga);
    for (int64_t r = r0; r < r1; ++r) {
        u32x4 xn[CH], gn[CH];
        load_row(min(r + 1, r1 - 1), xn, gn);  // the last row reloads itself: in bounds, unused
        float ss = 0.0f, sdx = 0.0f;             // sum x^2, sum (dy * (1 + w)) * x
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            float xf[VEC], gf[VEC];
            unpack16<BF16>(xa[q], xf);
            unpack16<BF16>(ga[q], gf);
#pragma unroll
            for (int h = 0; h < H4; ++h) {
                const float4 wp = s_wp[q * H4 + h][lane];
                const float wv[4] = {wp.x, wp.y, wp.z, wp.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ss = fmaf(xf[4 * h + e], xf[4 * h + e], ss);
                    sdx = fmaf(gf[4 * h + e] * wv[e], xf[4 * h + e], sdx);
                }
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            ss += __shfl_xor(ss, o, 64);
            sdx += __shfl_xor(sdx, o, 64);
        }
        const float inv = 1.0f / sqrtf(ss / (float)group + eps);
        const float coef = inv * inv * inv * sdx / (float)group;
        const int64_t base = r * hchunks + g * gchunks;
        // Unpack again below rather than keep 2 * CH * VEC unpacked floats live
        // across the reductions (an empty asm the compiler cannot see through).
#pragma unroll
        for (int q = 0; q < CH; ++q) asm volatile("" : "+v"(xa[q]), "+v"(ga[q]));
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            const int64_t c = lane + 64 * q;
            if (c >= gchunks) break;
            float xf[VEC], gf[VEC], out[VEC];
            unpack16<BF16>(xa[q], xf);
            unpack16<BF16>(ga[q], gf);
#pragma unroll
            for (int h = 0; h < H4; ++h) {
                const float4 wp = s_wp[q * H4 + h][lane];
                const float wv[4] = {wp.x, wp.y, wp.z, wp.w};
                float4 a = s_pw[wid][q * H4 + h][lane];
                float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    out[4 * h + e] = inv * gf[4 * h + e] * wv[e] - coef * xf[4 * h + e];
                    av[e] = fmaf(gf[4 * h + e], xf[4 * h + e] * inv, av[e]);
                }
                s_pw[wid][q * H4 + h][lane] = make_float4(av[0], av[1], av[2], av[3]);
            }
            __builtin_nontemporal_store(pack16<BF16>(out), dx + base + c);
        }
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            xa[q] = xn[q];
            ga[q] = gn[q];
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < CH * H4 * 64; i += kPleBlock) {
        const int ln = i & 63, qh = i >> 6, q = qh / H4, h = qh % H4;
        const int64_t c = ln + 64 * q;
        if (c >= gchunks) continue;
        double sum[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int v = 0; v < WAVES; ++v) {
            const float4 a = s_pw[v][qh][ln];
            sum[0] += (double)a.x;
            sum[1] += (double)a.y;
            sum[2] += (double)a.z;
            sum[3] += (double)a.w;
        }
        double* out = partial + bb * hidden + g * group + c * VEC + 4 * h;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = sum[e];
    }
}

__global__ __launch_bounds__(kPleBlock) void ple_zero_kernel(u32x4* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kPleBlock + threadIdx.x;
    if (i < n) p[i] = u32x4{0u, 0u, 0u, 0u};
}

constexpr int kConvTileFwd = 16;
constexpr int kConvTileBwd = 64;
// Rows per wave of the norm backward: enough waves to fill the chip (about
// 2,048 row blocks per group), at most 64 rows so the LDS sums stay short.
int norm_rows_per_wave(int64_t rows) { return (int)std::min<int64_t>(64, std::max<int64_t>(4, rows / 2048)); }
int64_t norm_partials(int64_t rows) {
    const int64_t rpw = norm_rows_per_wave(rows);
    return (rows + 4 * rpw - 1) / (4 * rpw);
}

unsigned blocks_for(int64_t threads) { return (unsigned)((threads + kPleBlock - 1) / kPleBlock); }

}  // namespace

// Work-items of the largest launch a convolution call (forward or backward)
// makes; saturates at INT64_MAX.  Arguments are non-negative.
static int64_t mul_sat(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

int64_t short_conv_launch_items(int64_t batch, int64_t seq, int64_t channels, int kernel, int dilation,
                                int elem_bytes) {
    const int64_t vec = 16 / elem_bytes;
    // the halo's gradient zeroed when there are no positions
    const int64_t halo = mul_sat(mul_sat(batch, (int64_t)(kernel - 1) * dilation), channels / vec);
    if (dilation == kConvD) {
        const int64_t tile = std::min(kConvTile, kConvTileUp);  // the larger grid of the two
        const int64_t tiles = (seq + tile - 1) / tile;
        const int64_t blocks = mul_sat(mul_sat(batch, (tiles + kConvWavesPerBlock - 1) / kConvWavesPerBlock),
                                       (channels / 4 + 63) / 64);
        return std::max(mul_sat(blocks, kPleBlock), halo);
    }
    const int64_t fwd = mul_sat(mul_sat(batch, (seq + kConvTileFwd - 1) / kConvTileFwd), channels / vec);
    const int64_t bwd = mul_sat(mul_sat(batch, (seq + kConvTileBwd - 1) / kConvTileBwd), channels / vec);
    return std::max({fwd, bwd, halo});
}

size_t short_conv_workspace_bytes(int64_t batch, int64_t seq, int64_t channels, int kernel) {
    const int64_t tiles = (seq + kConvTileBwd - 1) / kConvTileBwd;
    return (size_t)batch * (size_t)tiles * (size_t)channels * (size_t)(kernel + 1) * sizeof(double);
}

size_t rms_norm_workspace_bytes(int64_t rows, int64_t hidden) {
    return (size_t)norm_partials(rows) * (size_t)hidden * sizeof(double);
}

bool rms_norm_group_ok(int elem_bytes, int64_t group) {
    const int vec = 16 / elem_bytes;
    return group % vec == 0 && group / vec <= 64 * kNormMaxChunks;
}

#define ENGRAM_CONV_DISPATCH(KERNEL, ...)                                                              \
    switch (K * 4 + elem_bytes) {                                                                     \
        case 1 * 4 + 2: hipLaunchKernelGGL((KERNEL<true, 1>), grid, block, 0, stream, __VA_ARGS__); break;  \
        case 2 * 4 + 2: hipLaunchKernelGGL((KERNEL<true, 2>), grid, block, 0, stream, __VA_ARGS__); break;  \
        case 3 * 4 + 2: hipLaunchKernelGGL((KERNEL<true, 3>), grid, block, 0, stream, __VA_ARGS__); break;  \
        case 4 * 4 + 2: hipLaunchKernelGGL((KERNEL<true, 4>), grid, block, 0, stream, __VA_ARGS__); break;  \
        case 1 * 4 + 4: hipLaunchKernelGGL((KERNEL<false, 1>), grid, block, 0, stream, __VA_ARGS__); break; \
        case 2 * 4 + 4: hipLaunchKernelGGL((KERNEL<false, 2>), grid, block, 0, stream, __VA_ARGS__); break; \
        case 3 * 4 + 4: hipLaunchKernelGGL((KERNEL<false, 3>), grid, block, 0, stream, __VA_ARGS__); break; \
        default: hipLaunchKernelGGL((KERNEL<false, 4>), grid, block, 0, stream, __VA_ARGS__); break;        \
    }

hipError_t launch_short_conv(const void* x, int elem_bytes, int64_t B, int64_t S, int64_t C, const float* w,
                             const float* bias, int K, int d, const void* halo, void* y, hipStream_t stream) {
    if (B * S == 0) return hipSuccess;
    if (d == kConvD) {
        const int64_t tiles = (S + kConvTileUp - 1) / kConvTileUp;
        const int64_t blocks = B * ((tiles + kConvWavesPerBlock - 1) / kConvWavesPerBlock) * ((C / 4 + 63) / 64);
        const dim3 grid((unsigned)blocks), block(kPleBlock);
        ENGRAM_CONV_DISPATCH(short_conv_fwd_d3_kernel, x, halo, w, bias, B, S, C, y)
    } else {
        const int vec = 16 / elem_bytes;
        const int64_t threads = B * ((S + kConvTileFwd - 1) / kConvTileFwd) * (C / vec);
        const dim3 grid(blocks_for(threads)), block(kPleBlock);
        ENGRAM_CONV_DISPATCH(short_conv_fwd_kernel, (const u32x4*)x, (const u32x4*)halo, w, bias, B, S, C, d,
                             kConvTileFwd, (u32x4*)y)
    }
    return hipGetLastError();
}

hipError_t launch_short_conv_backward(const void* x, const void* dy, int elem_bytes, int64_t B, int64_t S, int64_t C,
                                      const float* w, int K, int d, const void* halo, void* dx, float* dw, float* db,
                                      void* dhalo, void* workspace, hipStream_t stream) {
    const int vec = 16 / elem_bytes;
    double* partial = (double*)workspace;
    int64_t parts = 0;
    if (B * S > 0 && d == kConvD) {
        const int64_t tiles = (S + kConvTile - 1) / kConvTile;
        const int64_t tgroups = (tiles + kConvWavesPerBlock - 1) / kConvWavesPerBlock;
        const int64_t blocks = B * tgroups * ((C / 4 + 63) / 64);
        parts = B * tgroups;
        const dim3 grid((unsigned)blocks), block(kPleBlock);
        ENGRAM_CONV_DISPATCH(short_conv_bwd_d3_kernel, x, dy, halo, w, B, S, C, dx, dhalo, partial)
    } else if (B * S > 0) {
        const int64_t tiles = (S + kConvTileBwd - 1) / kConvTileBwd;
        parts = B * tiles;
        const dim3 grid(blocks_for(B * tiles * (C / vec))), block(kPleBlock);
        ENGRAM_CONV_DISPATCH(short_conv_bwd_kernel, (const u32x4*)x, (const u32x4*)dy, (const u32x4*)halo, w, B, S,
                             C, d, kConvTileBwd, (u32x4*)dx, (u32x4*)dhalo, partial)
    } else if (dhalo && B > 0) {  // no positions: the halo's gradient is zero
        const int64_t n = B * (int64_t)(K - 1) * d * (C / vec);
        if (n > 0)
            hipLaunchKernelGGL(ple_zero_kernel, dim3(blocks_for(n)), dim3(kPleBlock), 0, stream, (u32x4*)dhalo, n);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t cols = C * (K + 1);
    hipLaunchKernelGGL(column_sum_kernel, dim3((unsigned)((cols + 63) / 64)), dim3(64 * kSumWaves), 0, stream,
                       (const double*)partial, parts, cols, K + 1, dw, db);
    return hipGetLastError();
}

#define ENGRAM_NORM_CASE(KERNEL, BF, CHN, ...) \
    case CHN: hipLaunchKernelGGL((KERNEL<BF, CHN>), grid, block, 0, stream, __VA_ARGS__); break;
#define ENGRAM_NORM_DISPATCH(KERNEL, ...)                                                               \
    if (elem_bytes == 2) {                                                                             \
        switch (ch) {                                                                                  \
            ENGRAM_NORM_CASE(KERNEL, true, 1, __VA_ARGS__) ENGRAM_NORM_CASE(KERNEL, true, 2, __VA_ARGS__)   \
            ENGRAM_NORM_CASE(KERNEL, true, 3, __VA_ARGS__) ENGRAM_NORM_CASE(KERNEL, true, 4, __VA_ARGS__)   \
            ENGRAM_NORM_CASE(KERNEL, true, 5, __VA_ARGS__) ENGRAM_NORM_CASE(KERNEL, true, 6, __VA_ARGS__)   \
            ENGRAM_NORM_CASE(KERNEL, true, 7, __VA_ARGS__) ENGRAM_NORM_CASE(KERNEL, true, 8, __VA_ARGS__)   \
            ENGRAM_NORM_CASE(KERNEL, true, 9, __VA_ARGS__) default: ENGRAM_NORM_CASE(KERNEL, true, 10, __VA_ARGS__) \
        }                                                                                              \
    } else {                                                                                           \
        switch (ch) {                                                                                  \
            ENGRAM_NORM_CASE(KERNEL, false, 1, __VA_ARGS__) ENGRAM_NORM_CASE(KERNEL, false, 2, __VA_ARGS__) \
            ENGRAM_NORM_CASE(KERNEL, false, 3, __VA_ARGS__) ENGRAM_NORM_CASE(KERNEL, false, 4, __VA_ARGS__) \
            ENGRAM_NORM_CASE(KERNEL, false, 5, __VA_ARGS__) ENGRAM_NORM_CASE(KERNEL, false, 6, __VA_ARGS__) \
            ENGRAM_NORM_CASE(KERNEL, false, 7, __VA_ARGS__) ENGRAM_NORM_CASE(KERNEL, false, 8, __VA_ARGS__)   \
            ENGRAM_NORM_CASE(KERNEL, false, 9, __VA_ARGS__) default: ENGRAM_NORM_CASE(KERNEL, false, 10, __VA_ARGS__) \
        }                                                                                              \
    }

// Chunks per lane for a group: ceil(group / VEC / 64), at most kNormMaxChunks.
int norm_chunks_per_lane(int elem_bytes, int64_t group) {
    const int64_t gchunks = group / (16 / elem_bytes);
    return (int)((gchunks + 63) / 64);
}

hipError_t launch_rms_norm(const void* x, int elem_bytes, int64_t rows, int64_t hidden, int64_t group, const float* w,
                           float eps, void* y, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int ch = norm_chunks_per_lane(elem_bytes, group);
    const int64_t waves = rows * (hidden / group);
    const dim3 grid(blocks_for(waves * 64)), block(kPleBlock);
    ENGRAM_NORM_DISPATCH(rms_norm_fwd_kernel, (const u32x4*)x, w, rows, hidden, group, eps, (u32x4*)y)
    return hipGetLastError();
}

hipError_t launch_rms_norm_backward(const void* x, const void* dy, int elem_bytes, int64_t rows, int64_t hidden,
                                    int64_t group, const float* w, float eps, void* dx, float* dw, void* workspace,
                                    hipStream_t stream) {
    const int64_t parts = rows > 0 ? norm_partials(rows) : 0;
    double* partial = (double*)workspace;
    if (rows > 0) {
        const int ch = norm_chunks_per_lane(elem_bytes, group);
        const dim3 grid((unsigned)(parts * (hidden / group))), block(kPleBlock);
        ENGRAM_NORM_DISPATCH(rms_norm_bwd_kernel, (const u32x4*)x, (const u32x4*)dy, w, rows, hidden, group, eps,
                             norm_rows_per_wave(rows), (u32x4*)dx, partial)
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(column_sum_kernel, dim3((unsigned)((hidden + 63) / 64)), dim3(64 * kSumWaves), 0, stream,
                       (const double*)partial, parts, hidden, 0, dw, (float*)nullptr);
    return hipGetLastError();
}

}  // namespace engram
