// decode_impl.hpp -- one-token recurrent decode step (gfx950), HBM-bound.
//
// Per sequence-head, in place on the state, then o = S^T q with the updated
// state (tensorplay "Talk Linear Attention", sections 2.1-2.2: the constant-size
// state is all that is carried between tokens):
//   decay (plain: gamma = 1)  S <- gamma S + k v^T   (wln20 "LLM注意力优化：线性注意力",
//                                                     data-dependent decay)
//   per-key-channel decay     S <- Diag(alpha) S + k v^T (tensorplay section 5.1,
//                                                     the GLA gate; one gate per row)
//   gated delta rule          r = S^T k;  S <- alpha S + k (beta (v - alpha r))^T
//                             (wln20, Gated DeltaNet section, d_k x d_v orientation:
//                             alpha (S - beta k r^T) + beta k v^T regrouped)
//   KDA                       r = (Diag(alpha) S)^T k;  S <- Diag(alpha) S + k (beta (v - r))^T
//                             (wln20, Kimi Delta Attention section: the delta rule
//                             with one gate per key channel)
// The delta rule needs the retrieval r over all rows before any row is updated:
// the state stays in registers between the two reductions. The fp32 state dominates the
// traffic (2 x d_k x d_v x 4 bytes per head and step), so the kernel is a
// streaming read-modify-write: one 256-thread workgroup per head (or head and
// value-column slice), each thread
// owning d_k / RG consecutive rows of one 16-byte column group, all of its state
// loads issued before any arithmetic, non-temporal loads and stores for the state
// (it is touched once per step), and a shuffle + LDS reduction of o over rows.
// The delta rules run two workgroups per head, each on half of the value columns.
#pragma once

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

// Value columns per workgroup. The retrieval r = S^T k of the delta rule is per
// value column, so a head's columns split over workgroups with no exchange; the
// delta rule holds its state slice across the retrieval barrier, and halving the
// slice halves the registers that holds (64 columns at d_v = 128: 8 rows of
// 16 bytes per thread instead of 16).
template <int VAR, int DV>
constexpr int decode_cols() {
    return ((VAR == V_GDN || VAR == V_KDA) && DV > 32) ? DV / 2 : DV;
}

// Occupancy: the state in flight is what keeps HBM busy. Without the retrieval
// pass a wave needs 65 registers when the compiler may use up to 72, which gives
// 7 waves per SIMD (6 at its own choice of 74; 8 at 64 was no faster). The delta
// rule on half-width slices fits the same bound. The per-channel gate with fp32
// rows is left to the compiler (a cap at 7 waves spills).
template <int VAR, typename TI>
constexpr int decode_min_waves() {
    return (VAR == V_VDECAY && sizeof(TI) == 4) ? 1 : 7;
}

template <int VAR, typename TI, typename TO, int DK, int DV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(decode_min_waves<VAR, TI>(), 8)))
decode_kernel(DecodeArgs a) {
    constexpr int CW = decode_cols<VAR, DV>();  // value columns of this workgroup
    constexpr int NSL = DV / CW;
    constexpr int CG = CW / 4;        // 16-byte column groups per row
    constexpr int RG = 256 / CG;      // row groups
    constexpr int RPT = DK / RG;      // rows per thread
    static_assert(RPT >= 1 && DK % RG == 0, "shape");

    __shared__ f32x4 red[4][CG];

    const int tid = threadIdx.x, rg = tid / CG;
    const size_t h = blockIdx.x / NSL;
    const int cg = tid % CG + (int)(blockIdx.x % NSL) * CG;  // column group within the head's row
    float *S = a.S + h * DK * DV + (size_t)rg * RPT * DV + 4 * cg;

    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (size_t)m * DV));

    const TI *qp = (const TI *)a.q + h * DK + rg * RPT;
    const TI *kp = (const TI *)a.k + h * DK + rg * RPT;
    float qr[RPT], kr[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        qr[m] = to_f32<TI>(qp[m]);
        kr[m] = to_f32<TI>(kp[m]);
    }
    const f32x4 vv = ld4<TI>((const TI *)a.v + h * DV + 4 * cg);
    const int wv = tid >> 6;
    // sum of a per-thread partial over all row groups, returned to every thread
    // of the column group: shuffles inside the wave, then the four waves'
    // partials through LDS
    auto rows_total = [&](f32x4 acc, f32x4 (&buf)[4][CG]) __attribute__((always_inline)) {
#pragma unroll
        for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
        }
        const int lc = tid % CG;
        if ((tid & 63) < CG) buf[wv][lc] = acc;
        __syncthreads();
        return buf[0][lc] + buf[1][lc] + buf[2][lc] + buf[3][lc];
    };

    // new state column group: ns = al * s + kr * u (u per column group)
    float al = 1.f;
    f32x4 u = vv;
    float alr[(VAR == V_VDECAY || VAR == V_KDA) ? RPT : 1];  // per-row (key channel) gates
    if constexpr (VAR == V_VDECAY || VAR == V_KDA) {
        const float *lp = a.lg + h * DK + rg * RPT;
#pragma unroll
        for (int m = 0; m < RPT; ++m) alr[m] = __expf(lp[m]);
    } else if constexpr (VAR == V_DECAY) {
        al = __expf(a.lg[h]);
    } else if constexpr (VAR == V_GDN) {
        __shared__ f32x4 rred[4][CG];
        al = a.lg ? __expf(a.lg[h]) : 1.f;
        const float be = a.beta[h];
        f32x4 racc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) racc += kr[m] * s[m];
        const f32x4 r = rows_total(racc, rred);  // r = S^T k for this column group
        u = be * (vv - al * r);
    }
    if constexpr (VAR == V_KDA) {
        // r = (Diag(alpha) S)^T k: the retrieval reads the decayed state
        __shared__ f32x4 rred[4][CG];
        const float be = a.beta[h];
        f32x4 racc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) racc += (kr[m] * alr[m]) * s[m];
        const f32x4 r = rows_total(racc, rred);
        u = be * (vv - r);
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const f32x4 ns = ((VAR == V_VDECAY || VAR == V_KDA) ? alr[m] : al) * s[m] + kr[m] * u;
        __builtin_nontemporal_store(ns, reinterpret_cast<f32x4 *>(S + (size_t)m * DV));
        acc += qr[m] * ns;
    }
    // reduce over the row groups of this wave, then over the four waves
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
    }
    if ((tid & 63) < CG) red[wv][tid % CG] = acc;
    __syncthreads();
    if (tid < CG) {
        const f32x4 o = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
        st4<TO>((TO *)a.o + h * DV + 4 * cg, o);
    }
}

template <int VAR, typename TI, typename TO, int DK, int DV>
hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
    constexpr int NSL = DV / decode_cols<VAR, DV>();
    hipLaunchKernelGGL((decode_kernel<VAR, TI, TO, DK, DV>), dim3(a.NH * NSL), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
