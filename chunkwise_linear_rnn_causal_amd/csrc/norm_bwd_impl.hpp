// norm_bwd_impl.hpp -- backward pass of the normalized variant (gfx950) on top
// of the plain one.
//
// Forward (proig-chaa "线性注意力：从 Softmax Attention 到 Kernel Attention 的本质
// 变化", sections 13-14): n_t = S_t^T q_t with S_t = S_0 + sum_{j<=t} k_j v_j^T,
// den_t = q_t . z_t with z_t = z_0 + sum_{j<=t} k_j, o_t = n_t / den_t. With
// rho_t = 1 / den_t and g_t = -(do_t . o_t) / den_t the output gradient splits
// into the plain backward with output gradient rho_t do_t (the plain kernels
// scale the dO rows they stage) and a rank-one normalizer term:
//   dq_t += g_t z_t,   dk_j += sum_{t>=j} g_t q_t + dz_L,   dz_0 = sum_t g_t q_t + dz_L.
// The denominators come from the forward pass itself (den_out), so the backward
// uses the values the forward divided by. Everything runs on fp32 operands (bf16
// inputs are upcast first): at the first tokens of a sequence the plain term and
// the normalizer term of dq cancel to a fraction of their sizes, and the
// gradients there are several times the tensor's RMS, so fp16 rounding of the
// rescaled dO rows alone left 1.5e-2 of RMS (emulated at B8 H16 L2048 d64), and of
// the score gradients 3.2e-2.
//
// Kernels:
//   norm_prep_kernel  one workgroup per (head, chunk): rho_t, g_t per token and
//       the chunk's sums of k and of g q.
//   norm_scan_kernel  one workgroup per head: exclusive prefix of the k sums
//       from z_0 and exclusive suffix of the g q sums from dz_L, over chunks (in
//       place), and dz_0.
//   norm_apply_kernel one workgroup per (head, chunk): the normalizer terms into
//       dq and dk (after the plain backward wrote them).
#pragma once

#include <algorithm>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

struct NormArgs {
    const void *q, *k, *dout;  // [BH, L, DK], [BH, L, DK], [BH, L, DV] (input type)
    const float *o, *den;      // forward output [BH, L, DV] and denominators [BH, L] (fp32)
    const float *z_in;         // [BH, DK] or nullptr
    const float *dz_out;       // [BH, DK] or nullptr
    float *rho, *g;            // [BH, L]
    float *ksum, *gqsum;       // [BH, nchunks, DK]: chunk sums, then (after the scan) the
                               // normalizer before the chunk / the g q sum after it
    float *gq, *gk;            // the gradients of q and k (updated)
    float *dz_in;              // [BH, DK] or nullptr
    int BH, L, nchunks;
};

template <typename TI, int DK, int DV>
__global__ void __launch_bounds__(256) norm_prep_kernel(NormArgs a) {
    constexpr int C = 64;
    __shared__ float gs[C];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / a.nchunks, c = blockIdx.x - bh * a.nchunks;
    const int L = a.L, t0 = c * C;
    // do_t . o_t: four threads per token, DV / 4 columns each
    {
        const int r = tid >> 2, qq = tid & 3, t = t0 + r;
        float dot = 0.f;
        if (t < L) {
            const TI *dor = (const TI *)a.dout + ((size_t)bh * L + t) * DV + qq * (DV / 4);
            const float *orow = a.o + ((size_t)bh * L + t) * DV + qq * (DV / 4);
#pragma unroll
            for (int j = 0; j < DV / 4; j += 8) {
                float x[8], y[8];
                ld8<TI>(dor + j, x);
                ld8<float>(orow + j, y);
#pragma unroll
                for (int e = 0; e < 8; ++e) dot = fmaf(x[e], y[e], dot);
            }
        }
        dot += __shfl_xor(dot, 1, 64);
        dot += __shfl_xor(dot, 2, 64);
        if (qq == 0) {
            float gt = 0.f;
            if (t < L) {
                const float inv = 1.f / a.den[(size_t)bh * L + t];
                gt = -dot * inv;
                a.rho[(size_t)bh * L + t] = inv;
                a.g[(size_t)bh * L + t] = gt;
            }
            gs[r] = gt;
        }
    }
    __syncthreads();
    // chunk sums of k and g q, one channel per thread
    if (tid < DK) {
        const TI *kg = (const TI *)a.k + (size_t)bh * L * DK + tid;
        const TI *qg = (const TI *)a.q + (size_t)bh * L * DK + tid;
        float ks = 0.f, gq = 0.f;
        const int n = min(C, L - t0);
#pragma unroll 8
        for (int r = 0; r < n; ++r) {
            ks += to_f32<TI>(kg[(size_t)(t0 + r) * DK]);
            gq = fmaf(gs[r], to_f32<TI>(qg[(size_t)(t0 + r) * DK]), gq);
        }
        a.ksum[((size_t)bh * a.nchunks + c) * DK + tid] = ks;
        a.gqsum[((size_t)bh * a.nchunks + c) * DK + tid] = gq;
    }
}

template <int DK>
__global__ void __launch_bounds__(DK) norm_scan_kernel(NormArgs a) {
    const int i = threadIdx.x, bh = blockIdx.x, nch = a.nchunks;
    float *ks = a.ksum + (size_t)bh * nch * DK + i, *gq = a.gqsum + (size_t)bh * nch * DK + i;
    float z = a.z_in ? a.z_in[(size_t)bh * DK + i] : 0.f;
    for (int c = 0; c < nch; ++c) {
        const float x = ks[(size_t)c * DK];
        ks[(size_t)c * DK] = z;  // the normalizer before chunk c
        z += x;
    }
    float r = a.dz_out ? a.dz_out[(size_t)bh * DK + i] : 0.f;
    for (int c = nch - 1; c >= 0; --c) {
        const float x = gq[(size_t)c * DK];
        gq[(size_t)c * DK] = r;  // dz_L plus the g q sums of the chunks after c
        r += x;
    }
    if (a.dz_in) a.dz_in[(size_t)bh * DK + i] = r;
}

template <typename TI, int DK>
__global__ void __launch_bounds__(DK) norm_apply_kernel(NormArgs a) {
    constexpr int C = 64;
    __shared__ float gs[C];
    const int i = threadIdx.x;
    const int bh = blockIdx.x / a.nchunks, c = blockIdx.x - bh * a.nchunks;
    const int L = a.L, t0 = c * C, n = min(C, L - t0);
    for (int r = i; r < C; r += DK) gs[r] = r < n ? a.g[(size_t)bh * L + t0 + r] : 0.f;
    __syncthreads();
    const size_t base = ((size_t)bh * L + t0) * DK + i;
    const TI *kg = (const TI *)a.k + base, *qg = (const TI *)a.q + base;
    float *dq = a.gq + base, *dk = a.gk + base;
    float z = a.ksum[((size_t)bh * a.nchunks + c) * DK + i];
#pragma unroll 8
    for (int r = 0; r < n; ++r) {
        z += to_f32<TI>(kg[(size_t)r * DK]);
        dq[(size_t)r * DK] += gs[r] * z;
    }
    float s = a.gqsum[((size_t)bh * a.nchunks + c) * DK + i];
#pragma unroll 8
    for (int r = n - 1; r >= 0; --r) {
        s = fmaf(gs[r], to_f32<TI>(qg[(size_t)r * DK]), s);
        dk[(size_t)r * DK] += s;
    }
}

// bf16 -> fp32 copy (the normalized backward computes on fp32 operands)
// q, k, v and dO widened to fp32 in one launch: blockIdx.y picks the tensor.
// Each thread takes U groups of 8 elements a grid stride apart and issues all
// its loads before its stores.
struct UpcastArgs {
    const bf16 *x[4];
    float *y[4];
    size_t n8[4];
};

template <int UNUSED = 0>
__global__ void __launch_bounds__(256) upcast_bf16_kernel(UpcastArgs a) {
    constexpr int U = 4;
    const int t = blockIdx.y;
    const bf16 *x = a.x[t];
    float *y = a.y[t];
    const size_t n8 = a.n8[t], stride = (size_t)gridDim.x * 256;
    for (size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x; i0 < n8; i0 += U * stride) {
        float v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * stride < n8) ld8<bf16>(x + (i0 + u * stride) * 8, v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * stride < n8) st8<float>(y + (i0 + u * stride) * 8, v[u]);
    }
}

// nq elements each of q and k, nv each of v and dO (multiples of 8: d_k and d_v are)
inline hipError_t launch_upcast4(const void *q, const void *k, const void *v, const void *d_o, float *q32,
                                 float *k32, float *v32, float *o32, size_t nq, size_t nv, hipStream_t st) {
    UpcastArgs a{{(const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (const bf16 *)d_o},
                 {q32, k32, v32, o32},
                 {nq / 8, nq / 8, nv / 8, nv / 8}};
    const size_t n8 = std::max(nq, nv) / 8;
    if (n8 == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<size_t>((n8 + 255) / 256, 2048);
    hipLaunchKernelGGL(upcast_bf16_kernel<>, dim3(blocks, 4), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename TI, int DK, int DV>
hipError_t launch_norm_bwd_pre(const NormArgs &a, hipStream_t st) {
    if (a.nchunks > 0)
        hipLaunchKernelGGL((norm_prep_kernel<TI, DK, DV>), dim3(a.BH * a.nchunks), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename TI, int DK>
hipError_t launch_norm_bwd_post(const NormArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((norm_scan_kernel<DK>), dim3(a.BH), dim3(DK), 0, st, a);
    if (a.nchunks > 0)
        hipLaunchKernelGGL((norm_apply_kernel<TI, DK>), dim3(a.BH * a.nchunks), dim3(DK), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
