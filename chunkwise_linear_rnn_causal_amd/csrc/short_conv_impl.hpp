// short_conv_impl.hpp -- causal depthwise short convolution over tokens (gfx950),
// HBM-bound; one launch covers any of q, k and v.
//
// The token-mixing step that recent linear-attention layers (DeltaNet: kernel
// size 4) put after the q/k/v projections (wln20 "LLM注意力优化：线性注意力",
// DeltaNet section): per batch b, head h and channel c, with a separate set of K
// taps per channel,
//     y_t[c] = sum_{tau=0}^{K-1} w[h][c][tau] * x_{t-tau}[c],
// where inputs before the first token come from the caller's window of the K-1
// previous inputs (or are zero). The window after the last token is returned, so
// a sequence can be processed in pieces and a decode step is the case L = 1.
//
// Mapping. A thread owns 8 consecutive channels (one 16-byte bf16 segment) of
// one head over a tile of TT tokens. Consecutive lanes take consecutive channel
// segments, then consecutive tiles, so each load instruction reads whole rows.
// The thread issues the loads of its K-1 window rows (the tail of the previous
// tile, served from cache) and of its TT rows before any arithmetic, then slides
// along the tile in fp32 with the taps in registers. The tile's rows are read and
// the outputs written with non-temporal accesses (each is touched once); 8-token
// tiles (bf16) keep 4 waves per SIMD resident, which measured fastest. Only the tile-0 thread of a
// column reads the incoming window and writes the outgoing one, so the window
// may be updated in place.
#pragma once

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

template <typename T, int K, int TT>
__global__ void __launch_bounds__(256) short_conv_kernel(ConvArgs a) {
    const unsigned blk = blockIdx.x;
    const int ti = blk >= a.blk2 ? 2 : (blk >= a.blk1 ? 1 : 0);
    const ConvTensor t = ti == 2 ? a.t2 : (ti == 1 ? a.t1 : a.t0);
    const unsigned blk0 = ti == 2 ? a.blk2 : (ti == 1 ? a.blk1 : 0u);
    const int d = t.d, G = d / 8, L = a.L, NT = a.NT;
    const size_t item = (size_t)(blk - blk0) * 256 + threadIdx.x;
    if (item >= (size_t)a.BH * NT * G) return;
    const int cg = (int)(item % G);
    const size_t r = item / G;
    const int tile = (int)(r % NT);
    const size_t bh = r / NT;
    const int h = (int)(bh % a.H);
    const int c0 = cg * 8;
    constexpr int W = K - 1;

    // taps of the 8 channels: w[h][c0 + j][tau], 8 * K consecutive floats
    float w[8][K];
    {
        const f32x4 *wp = reinterpret_cast<const f32x4 *>(t.w + ((size_t)h * d + c0) * K);
#pragma unroll
        for (int i = 0; i < 2 * K; ++i) {
            const f32x4 q4 = wp[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[(4 * i + e) / K][(4 * i + e) % K] = q4[e];
        }
    }

    const T *x = (const T *)t.x + bh * (size_t)a.ldx * d + c0;
    const T *s_in = t.s_in ? (const T *)t.s_in + bh * (size_t)W * d + c0 : nullptr;
    const int t0 = tile * TT;

    // the window rows t0-W .. t0-1 and the tile's rows, all loads first
    Raw8<T> win[W > 0 ? W : 1];
#pragma unroll
    for (int m = 0; m < W; ++m) {
        const int row = t0 - W + m;
        if (row >= 0) win[m] = ld_raw8<T>(x + (size_t)row * d);
        else if (s_in) win[m] = ld_raw8<T>(s_in + (size_t)(W + row) * d);
        else win[m] = zero_raw8<T>();
    }
    Raw8<T> raw[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i)
        raw[i] = (t0 + i < L) ? ld_raw8_nt<T>(x + (size_t)(t0 + i) * d) : zero_raw8<T>();

    // slide: hist[0] = x_{t-1}, hist[1] = x_{t-2}, ...
    float hist[W > 0 ? W : 1][8];
#pragma unroll
    for (int m = 0; m < W; ++m) unpack8<T>(win[W - 1 - m], hist[m]);
    T *y = (T *)t.y + bh * (size_t)L * d + c0;
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        float cur[8], out[8];
        unpack8<T>(raw[i], cur);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float acc = w[j][0] * cur[j];
#pragma unroll
            for (int tau = 1; tau < K; ++tau) acc = __builtin_fmaf(w[j][tau], hist[tau - 1][j], acc);
            out[j] = acc;
        }
        if (t0 + i < L) st8_nt<T>(y + (size_t)(t0 + i) * d, out);
#pragma unroll
        for (int m = W - 1; m > 0; --m)
#pragma unroll
            for (int j = 0; j < 8; ++j) hist[m][j] = hist[m - 1][j];
        if constexpr (W > 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) hist[0][j] = cur[j];
        }
    }

    // outgoing window: the W most recent inputs, oldest first (raw copies). The
    // incoming window was read above by this same thread, so s_out may be s_in.
    if (tile == 0 && t.s_out) {
        T *s_out = (T *)t.s_out + bh * (size_t)W * d + c0;
#pragma unroll
        for (int m = 0; m < W; ++m) {
            const int idx = L - W + m;
            Raw8<T> v = win[0];
            if (idx >= 0) {
                v = ld_raw8<T>(x + (size_t)idx * d);
            } else {  // idx in [-W, -1]: incoming window row W + idx (selected, not indexed)
#pragma unroll
                for (int m2 = 1; m2 < W; ++m2)
                    if (m2 == W + idx) v = win[m2];
            }
#pragma unroll
            for (int u = 0; u < (int)(sizeof(T) / 2); ++u)
                reinterpret_cast<uint4 *>(s_out + (size_t)m * d)[u] = v.v[u];
        }
    }
}

template <typename T, int K>
hipError_t launch_short_conv(const ConvArgs &a, unsigned blocks, hipStream_t st) {
    constexpr int TT = conv_tile<T>();
    hipLaunchKernelGGL((short_conv_kernel<T, K, TT>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
