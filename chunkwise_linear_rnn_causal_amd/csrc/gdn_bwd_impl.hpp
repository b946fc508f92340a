// gdn_bwd_impl.hpp -- backward pass of the gated delta rule (gfx950), bf16
// inputs, fp16 MFMA operands with fp32 accumulation, C = 64.
//
// Forward, per chunk (wln20 "LLM注意力优化：线性注意力", Gated DeltaNet section;
// tensorplay "Talk Linear Attention", section 6.2, WY / UT chunk form), with
// chunk-local cumulative log-gate G_r, a_r = e^{G_r}, Gamma_rs = e^{G_r - G_s},
// the state S_0 before the chunk, K^ = diag(a_C / a) K and Q^ = diag(a) Q:
//   B_k = Gamma (.) K K^T, strictly lower;  P = diag(beta) B_k;  T = (I + P)^-1
//   R = V - diag(a) K S_0;  U = T diag(beta) R  (= U~ - W S_0)
//   A_m = Gamma (.) Q K^T, lower with the diagonal
//   O = Q^ S_0 + A_m U;  S_C = a_C S_0 + K^^T U.
// Reverse mode, given dO and dS_C = dLoss/dS_C:
//   dU   = A_m^T dO + K^ dS_C
//   dS_0 = a_C dS_C + Q^^T dO - W^T dU        (the reverse serial step)
//   dY   = T^T dU;  dv = diag(beta) dY
//   X    = dY S_0^T
//   dA'  = Gamma (.) (dO U^T), lower with the diagonal
//   dB'  = -diag(beta) Gamma (.) (dY U^T), strictly lower;  Bsym = dB' + dB'^T
//   dq   = diag(a) dO S_0^T + dA' K
//   dk   = dA'^T Q + diag(a_C / a) U dS_C^T - diag(a beta) X + Bsym K
//   dbeta_r = dY_r . v_r - a_r (k_r . X_r) - sum_s (dY U^T)_rs (B_k)_rs
// (the last from U = diag(beta) (R - B_k U)). The loss depends on the gates only
// through q_t e^{G_t}, v_t e^{-G_t} and the final state e^{G_L} S'_L of the
// gate-free recurrence in the variables S'_t = S_t e^{-G_t}, so
//   dl_t = sum_{u >= t} (q_u . dq_u - v_u . dv_u) + <dS_L, S_L>.
// The gate of token t + 1 multiplies only the state S_t, so the same sum from
// the first token after a chunk on is <dS_end, S_end> of the state at the end
// of the chunk and its gradient: inside chunk c
//   dl_t = sum_{u = t}^{end of c} (q_u . dq_u - v_u . dv_u) + <dS_end(c), S_end(c)>,
// which keeps the sum to at most 64 terms (a sum over the whole sequence would
// add up the rounding of L terms whose total is much smaller than their sizes).
// The per-chunk states are recomputed (tensorplay section 4.1.2: stored per
// chunk for back-propagation) by two serial scans over the chunks that share
// one form: X' = a_C X + M^T Z (+ E), Z = Y~ + sigma N X, with
//   forward: X = S,  N = W,  sigma = -1, Y~ = U~,       M = K^,  E = 0       (Z = U)
//   reverse: X = dS, N = K^, sigma = +1, Y~ = A_m^T dO, M = -W,  E = Q^^T dO (Z = dU)
//
// Launches (launch_gdn_bwd):
//   gdn_prep_kernel<bf16, DK, 64, true>  W, U~ (row-major) and T per chunk.
//   gdn_bwd_dut_kernel  A_m^T dO per chunk.
//   gdn_bwd_scan_kernel  forward and reverse scans in one launch, one workgroup
//       per (direction, head, 32-column value slice); each stores X per chunk
//       (S before the chunk / dS after it) and overwrites U~ with U (A_m^T dO
//       with dU) in place.
//   gdn_bwd_grad_kernel  one workgroup (8 waves) per (head, chunk): dq, dk, dv,
//       dbeta and the log-gate gradient.
#pragma once

#include "gdn_prep_impl.hpp"
#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

namespace gdnb {

constexpr int C = 64;

// 16 bytes as a native vector (copies of HIP's uint4 struct can become memory
// copies that keep a register array in scratch)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Operand fragment with the "natural" K-slot map: slot e of lane group g holds
// k0 + 8g + e (one 16-byte read of a row whose K index runs along it).
template <int P> __device__ inline f16x8 nat_frag(const f16 *X, int row, int k0, int g) {
    return *reinterpret_cast<const f16x8 *>(X + row * P + k0 + 8 * g);
}
// Operand fragment with the "paired" K-slot map of tr_frag: slots 0..3 of group
// g hold k0 + 4g + e, slots 4..7 hold k0 + 16 + 4g + e (two 8-byte reads).
template <int P> __device__ inline f16x8 pair_frag(const f16 *X, int row, int k0, int g) {
    const f16x4 a = *reinterpret_cast<const f16x4 *>(X + row * P + k0 + 4 * g);
    const f16x4 b = *reinterpret_cast<const f16x4 *>(X + row * P + k0 + 16 + 4 * g);
    return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// Paired-map fragment whose K index runs down the columns of a row-major tile:
// X[k0 + map][col0 + n].
template <int P> __device__ inline f16x8 col_frag(const f16 *X, int k0, int col0, int lane) {
    return tr_frag<P>(X, k0 + 4 * ((lane >> 4) & 3), col0, lane);
}

__device__ inline u32x4 bf16x8_to_f16x8(u32x4 w) {
    // packed round-toward-zero conversion: exact for bf16 values in fp16's
    // normal range; below it the error stays under 2^-24
    u32x4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        h[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(w[i]), bf16_hi(w[i])));
    return h;
}
// eight bf16 values times f, rounded to fp16
__device__ inline u32x4 bf16x8_scaled_f16(u32x4 w, float f) {
    u32x4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f16 lo = (f16)(bf16_lo(w[i]) * f), hi = (f16)(bf16_hi(w[i]) * f);
        h[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return h;
}

// sum over the 16 lanes of a lane group (n = 0..15)
__device__ inline float group16_sum(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

// Rows [t0, t0 + C) of a bf16 [L][D] head into a fp16 LDS tile of pitch P
// (rows past L zero), NT threads; all loads are issued before any store.
template <int D, int P, int NT>
__device__ inline void stage_bf16(f16 *dst, const bf16 *src, int t0, int L, int tid) {
    constexpr int SEG = D / 8, TOT = C * SEG, N = (TOT + NT - 1) / NT;
    u32x4 r[N];
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const int idx = tid + NT * m, row = idx / SEG, seg = idx % SEG;
        if (TOT % NT == 0 || idx < TOT)
            r[m] = *reinterpret_cast<const u32x4 *>(src + (size_t)min(t0 + row, L - 1) * D + seg * 8);
    }
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const int idx = tid + NT * m, row = idx / SEG, seg = idx % SEG;
        if (TOT % NT == 0 || idx < TOT)
            *reinterpret_cast<u32x4 *>(dst + row * P + seg * 8) =
                t0 + row < L ? bf16x8_to_f16x8(r[m]) : u32x4{0u, 0u, 0u, 0u};
    }
}
// C rows of an fp16 [.][D] array (row stride D) into an LDS tile of pitch P.
template <int D, int P, int NT>
__device__ inline void stage_f16(f16 *dst, const f16 *src, int tid) {
    constexpr int SEG = D / 8, TOT = C * SEG, N = (TOT + NT - 1) / NT;
    u32x4 r[N];
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const int idx = tid + NT * m, row = idx / SEG, seg = idx % SEG;
        if (TOT % NT == 0 || idx < TOT) r[m] = *reinterpret_cast<const u32x4 *>(src + (size_t)row * D + seg * 8);
    }
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const int idx = tid + NT * m, row = idx / SEG, seg = idx % SEG;
        if (TOT % NT == 0 || idx < TOT) *reinterpret_cast<u32x4 *>(dst + row * P + seg * 8) = r[m];
    }
}

}  // namespace gdnb

// ---------------------------------------------------------------------------
// A_m^T dO per chunk: [BH, Lp, DV] fp16 into a.du. One workgroup (4 waves) per
// (head, chunk).
template <int DK, int DV>
__global__ void __launch_bounds__(256) gdn_bwd_dut_kernel(BwdArgs a) {
    using namespace gdnb;
    using MF = Mfma<f16>;
    constexpr int KP = DK + 16, VP = DV + 16, AP = C + 16;
    __shared__ __attribute__((aligned(16))) f16 Qs[C * KP];
    __shared__ __attribute__((aligned(16))) f16 Ks[C * KP];
    __shared__ __attribute__((aligned(16))) f16 Os[C * VP];
    __shared__ __attribute__((aligned(16))) f16 At[C * AP];  // A_m^T: [s][r]
    __shared__ float Gs[C];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int bh = blockIdx.x / a.nchunks, c = blockIdx.x - bh * a.nchunks;
    const int L = a.L, t0 = c * C;
    stage_bf16<DK, KP, 256>(Qs, (const bf16 *)a.q + (size_t)bh * L * DK, t0, L, tid);
    stage_bf16<DK, KP, 256>(Ks, (const bf16 *)a.k + (size_t)bh * L * DK, t0, L, tid);
    stage_bf16<DV, VP, 256>(Os, (const bf16 *)a.dout + (size_t)bh * L * DV, t0, L, tid);
    if (wv == 0) {
        const float l = (a.lg && t0 + lane < L) ? a.lg[(size_t)bh * L + t0 + lane] : 0.f;
        Gs[lane] = wave_inclusive_sum(l);
    }
    __syncthreads();

    // A_m^T tiles D[s][r] = k_s . q_r, masked (s <= r) and decayed
    for (int tile = wv; tile < 16; tile += 4) {
        const int sb = tile >> 2, rb = tile & 3;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        if (sb <= rb) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                d = MF::mma(nat_frag<KP>(Ks, sb * 16 + n, ks * 32, g), nat_frag<KP>(Qs, rb * 16 + n, ks * 32, g), d);
        }
        const int r = rb * 16 + n;
        const float Gr = Gs[r];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = sb * 16 + 4 * g + e;
            At[s * AP + r] = (f16)(s <= r ? d[e] * __expf(Gr - Gs[s]) : 0.f);
        }
    }
    __syncthreads();

    // (A_m^T dO)^T tiles D[j][s] = sum_r dO[r][j] A_m^T[s][r]; lane holds
    // j = jb*16 + 4g + e, s = sb*16 + n: four consecutive columns of row s
    f16 *du = (f16 *)a.du + ((size_t)bh * a.Lp + t0) * DV;
    for (int tile = wv; tile < (DV / 16) * 4; tile += 4) {
        const int jb = tile >> 2, sb = tile & 3;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk * 32 + 31 < sb * 16) continue;  // rows r < s only
            d = MF::mma(col_frag<VP>(Os, kk * 32, jb * 16, lane), pair_frag<AP>(At, sb * 16 + n, kk * 32, g), d);
        }
        st4<f16>(du + (size_t)(sb * 16 + n) * DV + jb * 16 + 4 * g, d);
    }
}

// ---------------------------------------------------------------------------
// The two serial scans. Workgroup b < BH * NS runs the forward scan of head
// b / NS, value columns [32 (b % NS), +32); the others the reverse scan. Eight
// waves: waves 0-3 run the serial chain (the Z and X products), waves 4-7 store
// X and Z to the workspace and stage the next chunk (loads one chunk ahead), so
// the chain does not wait on memory. Two barriers per chunk.
template <int DK, int DV>
struct GdnScanCfg {
    static constexpr int DVT = 32, NS = DV / DVT;
    static constexpr int C = gdnb::C, KP = DK + 16, YP = DVT + 16, XP = DVT + 16;
    // per buffer: W, K^, Q^ (reverse), Y~, dO (reverse)
    static constexpr int OW = 0, OK = C * KP, OQ = 2 * C * KP, OY = 3 * C * KP, OO = OY + C * YP,
                         SET = OO + C * YP;
    static constexpr int XS = 2 * SET, ZS = XS + DK * XP, TOTAL = ZS + C * YP;  // fp16 elements
    static constexpr int NKL = C * DK / 8 / 256;  // 16-byte loads per staging thread per C x DK tile
    static_assert(NKL >= 1 && NKL * 256 * 8 == C * DK, "scan staging geometry");
};

template <int DK, int DV, bool REV>
__device__ __attribute__((always_inline)) inline void gdn_scan(const BwdArgs &a, int b, f16 *lds, float *Eg) {
    using namespace gdnb;
    using MF = Mfma<f16>;
    using Cfg = GdnScanCfg<DK, DV>;
    constexpr int DVT = Cfg::DVT, NS = Cfg::NS, KP = Cfg::KP, YP = Cfg::YP, XP = Cfg::XP;
    constexpr int NKL = Cfg::NKL, SEGK = DK / 8, SEGY = DVT / 8;
    constexpr int NTI = DK / 16, RT = (NTI + 3) / 4;  // state row tiles; per chain wave
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int bh = b / NS, j0 = (b % NS) * DVT;
    const int L = a.L, nch = a.nchunks;
    f16 *yg = (f16 *)(REV ? a.du : a.u) + (size_t)bh * a.Lp * DV + j0;
    f16 *xg = (f16 *)(REV ? a.dhs : a.hs) + (size_t)bh * nch * DK * DV + j0;
    f16 *Xs = lds + Cfg::XS, *Zs = lds + Cfg::ZS;

    if (wv < 4) {
        // ===== chain waves: X row tiles wv + 4m, both 16-column tiles; lane holds
        // rows i = 16 ti + 4g + e, column j = 16 tj + n of the slice
        f32x4 X[RT][2];
        const float *x0 = REV ? a.ds_out : a.s_in;
#pragma unroll
        for (int m = 0; m < RT; ++m) {
            const int ti = wv + 4 * m;
#pragma unroll
            for (int tj = 0; tj < 2; ++tj) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    X[m][tj][e] = (x0 && ti < NTI)
                        ? x0[(size_t)bh * DK * DV + (size_t)(ti * 16 + 4 * g + e) * DV + j0 + tj * 16 + n] : 0.f;
            }
        }
        auto write_x = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < RT; ++m) {
                const int ti = wv + 4 * m;
                if (NTI % 4 != 0 && ti >= NTI) continue;
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) Xs[(ti * 16 + 4 * g + e) * XP + tj * 16 + n] = (f16)X[m][tj][e];
                }
            }
        };
        write_x();
        __syncthreads();  // prologue
        for (int i = 0; i < nch; ++i) {
            const f16 *S = lds + (i & 1) * Cfg::SET;
            // Z = Y~ + sigma N X, row block wv
            {
                const f16 *N = S + (REV ? Cfg::OK : Cfg::OW);
                f32x4 z[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
                f16x8 nf[DK / 32], xf[DK / 32][2];
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    nf[ks] = pair_frag<KP>(N, wv * 16 + n, ks * 32, g);
                    xf[ks][0] = col_frag<XP>(Xs, ks * 32, 0, lane);
                    xf[ks][1] = col_frag<XP>(Xs, ks * 32, 16, lane);
                }
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    z[0] = MF::mma(nf[ks], xf[ks][0], z[0]);
                    z[1] = MF::mma(nf[ks], xf[ks][1], z[1]);
                }
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = wv * 16 + 4 * g + e, j = tj * 16 + n;
                        const float y = (float)S[Cfg::OY + r * YP + j];
                        Zs[r * YP + j] = (f16)(REV ? y + z[tj][e] : y - z[tj][e]);
                    }
                }
            }
            __syncthreads();
            // X' = a_C X + M^T Z (+ Q^^T dO)
            {
                const float eg = Eg[i & 1];
                const f16 *M = S + (REV ? Cfg::OW : Cfg::OK);
#pragma unroll
                for (int m = 0; m < RT; ++m) {
                    X[m][0] *= eg;
                    X[m][1] *= eg;
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const f16x8 z0 = col_frag<YP>(Zs, kk * 32, 0, lane), z1 = col_frag<YP>(Zs, kk * 32, 16, lane);
                    f16x8 o0, o1;
                    if constexpr (REV) {
                        o0 = col_frag<YP>(S + Cfg::OO, kk * 32, 0, lane);
                        o1 = col_frag<YP>(S + Cfg::OO, kk * 32, 16, lane);
                    }
#pragma unroll
                    for (int m = 0; m < RT; ++m) {
                        const int ti = wv + 4 * m;
                        if (NTI % 4 != 0 && ti >= NTI) continue;
                        f16x8 mf = col_frag<KP>(M, kk * 32, ti * 16, lane);
                        if constexpr (REV) {
                            mf = neg_frag<f16>(mf);
                            const f16x8 qf = col_frag<KP>(S + Cfg::OQ, kk * 32, ti * 16, lane);
                            X[m][0] = MF::mma(qf, o0, X[m][0]);
                            X[m][1] = MF::mma(qf, o1, X[m][1]);
                        }
                        X[m][0] = MF::mma(mf, z0, X[m][0]);
                        X[m][1] = MF::mma(mf, z1, X[m][1]);
                    }
                }
            }
            write_x();
            __syncthreads();
        }
        // final X: the forward scan's S_L, the reverse scan's dS_0
        float *xo = REV ? a.gs_in : a.s_last;
        if (xo) {
#pragma unroll
            for (int m = 0; m < RT; ++m) {
                const int ti = wv + 4 * m;
                if (ti >= NTI) continue;
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        xo[(size_t)bh * DK * DV + (size_t)(ti * 16 + 4 * g + e) * DV + j0 + tj * 16 + n] = X[m][tj][e];
                }
            }
        }
    } else {
        // ===== staging waves (256 threads): loads one chunk ahead, staging,
        // stores of X and Z
        const int st = tid - 256;
        const bf16 *kg = (const bf16 *)a.k + (size_t)bh * L * DK;
        const bf16 *qg = (const bf16 *)a.q + (size_t)bh * L * DK;
        const bf16 *og = (const bf16 *)a.dout + (size_t)bh * L * DV + j0;
        const f16 *wg = (const f16 *)a.w + (size_t)bh * a.Lp * DK;
        // Every load is unconditional and every masking an arithmetic select, so
        // no branch separates a load from its use and the waits stay exact:
        // without a gate the (finite) beta row is read and multiplied by zero.
        const float *lgg = (a.lg ? a.lg : a.beta) + (size_t)bh * L;
        const float lsc = a.lg ? 1.f : 0.f;
        u32x4 pw[NKL], pk[NKL], pq[NKL], py, po;
        float pl;
        auto load = [&](int c) __attribute__((always_inline)) {
            const int t0 = c * C;
#pragma unroll
            for (int m = 0; m < NKL; ++m) {
                const int idx = st + 256 * m, row = idx / SEGK, seg = idx % SEGK;
                pw[m] = *reinterpret_cast<const u32x4 *>(wg + (size_t)(t0 + row) * DK + seg * 8);
                pk[m] = *reinterpret_cast<const u32x4 *>(kg + (size_t)min(t0 + row, L - 1) * DK + seg * 8);
                if constexpr (REV)
                    pq[m] = *reinterpret_cast<const u32x4 *>(qg + (size_t)min(t0 + row, L - 1) * DK + seg * 8);
            }
            {
                const int row = st / SEGY, seg = st % SEGY;
                py = *reinterpret_cast<const u32x4 *>(yg + (size_t)(t0 + row) * DV + seg * 8);
                if constexpr (REV)
                    po = *reinterpret_cast<const u32x4 *>(og + (size_t)min(t0 + row, L - 1) * DV + seg * 8);
            }
            pl = lgg[min(t0 + lane, L - 1)];
        };
        auto stage = [&](int c, int buf) __attribute__((always_inline)) {
            f16 *S = lds + buf * Cfg::SET;
            const int t0 = c * C;
            const float G = wave_inclusive_sum(t0 + lane < L ? pl * lsc : 0.f);
            const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
#pragma unroll
            for (int m = 0; m < NKL; ++m) {
                const int idx = st + 256 * m, row = idx / SEGK, seg = idx % SEGK;
                const float Gr = __shfl(G, row, 64);
                const float vz = t0 + row < L ? 1.f : 0.f;  // rows past the end: zero
                *reinterpret_cast<u32x4 *>(S + Cfg::OW + row * KP + seg * 8) = pw[m];
                *reinterpret_cast<u32x4 *>(S + Cfg::OK + row * KP + seg * 8) =
                    bf16x8_scaled_f16(pk[m], vz * __expf(gC - Gr));
                if constexpr (REV)
                    *reinterpret_cast<u32x4 *>(S + Cfg::OQ + row * KP + seg * 8) =
                        bf16x8_scaled_f16(pq[m], vz * __expf(Gr));
            }
            {
                const int row = st / SEGY, seg = st % SEGY;
                *reinterpret_cast<u32x4 *>(S + Cfg::OY + row * YP + seg * 8) = py;
                if constexpr (REV) {
                    const uint32_t msk = t0 + row < L ? 0xffffffffu : 0u;
                    *reinterpret_cast<u32x4 *>(S + Cfg::OO + row * YP + seg * 8) = bf16x8_to_f16x8(po) & msk;
                }
            }
            if (st == 0) Eg[buf] = __expf(gC);
        };
        // chunk of step i; steps past the end repeat the last chunk, so the loads
        // and the staging of the step after the last are unconditional (into the
        // buffer no wave reads any more)
        auto cidx = [&](int i) { i = min(i, nch - 1); return REV ? nch - 1 - i : i; };
        if (nch > 0) {
            load(cidx(0));
            stage(cidx(0), 0);
            load(cidx(1));
        }
        __syncthreads();  // prologue
        for (int i = 0; i < nch; ++i) {
            const int c = cidx(i);
            // X (S before chunk c, or dS after it) to the workspace
#pragma unroll
            for (int m = 0; m < (DK * SEGY + 255) / 256; ++m) {
                const int idx = st + 256 * m, row = idx / SEGY, seg = idx % SEGY;
                if ((DK * SEGY) % 256 == 0 || idx < DK * SEGY)
                    *reinterpret_cast<u32x4 *>(xg + ((size_t)c * DK + row) * DV + seg * 8) =
                        *reinterpret_cast<const u32x4 *>(Xs + row * XP + seg * 8);
            }
            stage(cidx(i + 1), (i + 1) & 1);
            load(cidx(i + 2));
            __syncthreads();
            // Z (U or dU) to the workspace, over Y~
            {
                const int row = st / SEGY, seg = st % SEGY;
                *reinterpret_cast<u32x4 *>(yg + (size_t)(c * C + row) * DV + seg * 8) =
                    *reinterpret_cast<const u32x4 *>(Zs + row * YP + seg * 8);
            }
            __syncthreads();
        }
    }
}

template <int DK, int DV>
__global__ void __launch_bounds__(512) gdn_bwd_scan_kernel(BwdArgs a) {
    using Cfg = GdnScanCfg<DK, DV>;
    __shared__ __attribute__((aligned(16))) f16 lds[Cfg::TOTAL];
    __shared__ float Eg[2];
    // value slices of one head on one XCD: they share its rows through that L2
    const int vid = xcd_virtual_block();
    if (vid < a.BH * Cfg::NS)
        gdn_scan<DK, DV, false>(a, vid, lds, Eg);
    else
        gdn_scan<DK, DV, true>(a, vid - a.BH * Cfg::NS, lds, Eg);
}

// ---------------------------------------------------------------------------
// Per-chunk gradients: one workgroup (8 waves) per (head, chunk).
template <int DK, int DV>
struct GdnGradCfg {
    static constexpr int KP = DK + 16, VP = DV + 16, AP = gdnb::C + 16, C = gdnb::C;
    static constexpr int OQ = 0, OK = OQ + C * KP, OO = OK + C * KP, OU = OO + C * VP, ODU = OU + C * VP,
                         OY = ODU + C * VP, OT = OY + C * VP, OA = OT + C * AP, OB = OA + C * AP,
                         TOTAL = OB + C * AP;  // fp16 elements
};

template <int DK, int DV>
__global__ void __launch_bounds__(512) gdn_bwd_grad_kernel(BwdArgs a) {
    using namespace gdnb;
    using MF = Mfma<f16>;
    using Cfg = GdnGradCfg<DK, DV>;
    constexpr int KP = Cfg::KP, VP = Cfg::VP, AP = Cfg::AP;
    constexpr int NIB = DK / 16, RPW = NIB / 2;  // column blocks of dq / dk; row blocks per wave
    __shared__ __attribute__((aligned(16))) f16 lds[Cfg::TOTAL];
    // per-token partial sums, each slot written once (a fixed summation order):
    // dY . v per pair of waves, (dY U^T) . B_k per key block, k . X and q . dq
    // per column block; then q . dq - v . dv per token, and per-wave partials of
    // <dS_end, S_end>
    __shared__ float Gs[C], Bt[C], rYV[2][C], rYB[4][C], rKX[NIB][C], rQD[NIB][C], dGs[C], bpart[8];

    f16 *Qs = lds + Cfg::OQ, *Ks = lds + Cfg::OK, *Os = lds + Cfg::OO, *Us = lds + Cfg::OU;
    f16 *dUs = lds + Cfg::ODU, *dYs = lds + Cfg::OY, *Ts = lds + Cfg::OT, *dAs = lds + Cfg::OA,
        *Bss = lds + Cfg::OB;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int nch = a.nchunks, bh = blockIdx.x / nch, c = blockIdx.x - bh * nch;
    const int L = a.L, t0 = c * C;
    const int ib = wv % NIB, rb0 = (wv / NIB) * RPW;

    // B fragments of S_0 and dS_C for this wave's column block (natural map over j)
    f16x8 sf[DV / 32], df[DV / 32];
    {
        const size_t off = ((size_t)bh * nch + c) * DK * DV + (size_t)(ib * 16 + n) * DV + 8 * g;
#pragma unroll
        for (int ks = 0; ks < DV / 32; ++ks) {
            sf[ks] = *reinterpret_cast<const f16x8 *>((const f16 *)a.hs + off + ks * 32);
            df[ks] = *reinterpret_cast<const f16x8 *>((const f16 *)a.dhs + off + ks * 32);
        }
    }
    // <dS_end, S_end> of this chunk: dS after it (the reverse scan's) and S
    // before the next chunk (the last chunk: the final state and d_state_out, in fp32)
    const bool last = c == nch - 1;
    float bdot = 0.f;
    {
        constexpr int NP = (DK * DV / 8 + 511) / 512;
        if (!last) {
            const f16 *dh = (const f16 *)a.dhs + ((size_t)bh * nch + c) * DK * DV;
            const f16 *hn = (const f16 *)a.hs + ((size_t)bh * nch + c + 1) * DK * DV;
            f16x8 x[NP], y[NP];
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                const int idx = tid + 512 * m;
                if (idx < DK * DV / 8) {
                    x[m] = *reinterpret_cast<const f16x8 *>(dh + idx * 8);
                    y[m] = *reinterpret_cast<const f16x8 *>(hn + idx * 8);
                }
            }
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                if (tid + 512 * m < DK * DV / 8) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) bdot = fmaf((float)x[m][e], (float)y[m][e], bdot);
                }
            }
        } else if (a.ds_out) {
            const float *dh = a.ds_out + (size_t)bh * DK * DV, *hn = a.s_last + (size_t)bh * DK * DV;
            for (int idx = tid; idx < DK * DV / 4; idx += 512) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(dh + idx * 4);
                const f32x4 y = *reinterpret_cast<const f32x4 *>(hn + idx * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) bdot = fmaf(x[e], y[e], bdot);
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) bdot += __shfl_xor(bdot, off, 64);
    }
    stage_bf16<DK, KP, 512>(Qs, (const bf16 *)a.q + (size_t)bh * L * DK, t0, L, tid);
    stage_bf16<DK, KP, 512>(Ks, (const bf16 *)a.k + (size_t)bh * L * DK, t0, L, tid);
    stage_bf16<DV, VP, 512>(Os, (const bf16 *)a.dout + (size_t)bh * L * DV, t0, L, tid);
    stage_f16<DV, VP, 512>(Us, (const f16 *)a.u + ((size_t)bh * a.Lp + t0) * DV, tid);
    stage_f16<DV, VP, 512>(dUs, (const f16 *)a.du + ((size_t)bh * a.Lp + t0) * DV, tid);
    stage_f16<C, AP, 512>(Ts, (const f16 *)a.t + ((size_t)bh * nch + c) * C * C, tid);
    if (wv == 0) {
        const bool valid = t0 + lane < L;
        const float l = (a.lg && valid) ? a.lg[(size_t)bh * L + t0 + lane] : 0.f;
        Gs[lane] = wave_inclusive_sum(l);
        Bt[lane] = valid ? a.beta[(size_t)bh * L + t0 + lane] : 0.f;
    }
    if (lane == 0) bpart[wv] = bdot;
    __syncthreads();
    const float gC = Gs[C - 1];
    const bf16 *vg = (const bf16 *)a.v + (size_t)bh * L * DV;

    // (1a) dY = T^T dU; dv = diag(beta) dY; dY . v. Wave w's tiles all lie in row
    // block w % 4.
    float yv[4] = {0.f, 0.f, 0.f, 0.f};
    for (int tile = wv; tile < 4 * (DV / 16); tile += 8) {
        const int rb = tile & 3, jb = tile >> 2;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk * 32 + 31 < rb * 16) continue;  // T^T[r][s] = 0 for s < r
            d = MF::mma(col_frag<AP>(Ts, kk * 32, rb * 16, lane), col_frag<VP>(dUs, kk * 32, jb * 16, lane), d);
        }
        const int j = jb * 16 + n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rb * 16 + 4 * g + e, t = t0 + r;
            dYs[r * VP + j] = (f16)d[e];
            if (t < L) {
                a.gv[((size_t)bh * L + t) * DV + j] = Bt[r] * d[e];
                yv[e] = fmaf(d[e], (float)vg[(size_t)t * DV + j], yv[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float x = group16_sum(yv[e]);
        if (n == 0) rYV[wv >> 2][(wv & 3) * 16 + 4 * g + e] = x;
    }
    // (1b) dA' = Gamma (.) (dO U^T), lower with the diagonal
    for (int tile = wv; tile < 16; tile += 8) {
        const int rb = tile >> 2, sb = tile & 3;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        if (sb <= rb) {
#pragma unroll
            for (int ks = 0; ks < DV / 32; ++ks)
                d = MF::mma(nat_frag<VP>(Os, rb * 16 + n, ks * 32, g), nat_frag<VP>(Us, sb * 16 + n, ks * 32, g), d);
        }
        const int s = sb * 16 + n;
        const float Gsv = Gs[s];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rb * 16 + 4 * g + e;
            dAs[r * AP + s] = (f16)(s <= r ? d[e] * __expf(Gs[r] - Gsv) : 0.f);
        }
    }
    __syncthreads();

    // (2) dY U^T and B_k on the lower tiles: (dY U^T) . B_k per row and key
    // block, Bsym = dB' + dB'^T
    for (int tile = wv; tile < 16; tile += 8) {
        const int rb = tile >> 2, sb = tile & 3;
        if (sb > rb) continue;
        f32x4 yu = {0.f, 0.f, 0.f, 0.f}, kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DV / 32; ++ks)
            yu = MF::mma(nat_frag<VP>(dYs, rb * 16 + n, ks * 32, g), nat_frag<VP>(Us, sb * 16 + n, ks * 32, g), yu);
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
            kk = MF::mma(nat_frag<KP>(Ks, rb * 16 + n, ks * 32, g), nat_frag<KP>(Ks, sb * 16 + n, ks * 32, g), kk);
        const int s = sb * 16 + n;
        const float Gsv = Gs[s];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rb * 16 + 4 * g + e;
            const bool strict = s < r;
            const float gam = strict ? __expf(Gs[r] - Gsv) : 0.f;
            const float part = group16_sum(yu[e] * gam * kk[e]);
            if (n == 0) rYB[sb][r] = part;
            const f16 db = (f16)(-Bt[r] * gam * yu[e]);
            if (s <= r) Bss[r * AP + s] = db;
            if (strict) Bss[s * AP + r] = db;
        }
    }
    __syncthreads();

    // (3) dq and dk for column block ib, row blocks rb0 .. rb0 + RPW - 1
    for (int u = 0; u < RPW; ++u) {
        const int rb = rb0 + u;
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, dq = {0.f, 0.f, 0.f, 0.f}, dk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DV / 32; ++ks) {
            x = MF::mma(nat_frag<VP>(dYs, rb * 16 + n, ks * 32, g), sf[ks], x);
            dq = MF::mma(nat_frag<VP>(Os, rb * 16 + n, ks * 32, g), sf[ks], dq);
            dk = MF::mma(nat_frag<VP>(Us, rb * 16 + n, ks * 32, g), df[ks], dk);
        }
        // rows r = rb*16 + 4g + e (tokens), column i = ib*16 + n
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rb * 16 + 4 * g + e;
            const float Gr = Gs[r], ar = __expf(Gr);
            dq[e] *= ar;
            dk[e] = dk[e] * __expf(gC - Gr) - ar * Bt[r] * x[e];
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const f16x8 kcol = col_frag<KP>(Ks, kk * 32, ib * 16, lane);
            dq = MF::mma(pair_frag<AP>(dAs, rb * 16 + n, kk * 32, g), kcol, dq);
            dk = MF::mma(col_frag<AP>(dAs, kk * 32, rb * 16, lane), col_frag<KP>(Qs, kk * 32, ib * 16, lane), dk);
            dk = MF::mma(pair_frag<AP>(Bss, rb * 16 + n, kk * 32, g), kcol, dk);
        }
        const int i = ib * 16 + n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rb * 16 + 4 * g + e, t = t0 + r;
            if (t < L) {
                a.gq[((size_t)bh * L + t) * DK + i] = dq[e];
                a.gk[((size_t)bh * L + t) * DK + i] = dk[e];
            }
            const float qd = group16_sum(dq[e] * (float)Qs[r * KP + i]);
            const float kx = group16_sum(x[e] * (float)Ks[r * KP + i]);
            if (n == 0) {
                rQD[ib][r] = qd;
                rKX[ib][r] = kx;
            }
        }
    }
    __syncthreads();

    // (4) per token: dbeta, then the log-gate gradient (suffix sum within the chunk)
    if (tid < C) {
        const int r = tid, t = t0 + r;
        const float yv = rYV[0][r] + rYV[1][r];
        float yb = 0.f, kx = 0.f, qd = 0.f;
        for (int sb = 0; sb <= r / 16; ++sb) yb += rYB[sb][r];
#pragma unroll
        for (int i = 0; i < NIB; ++i) {
            kx += rKX[i][r];
            qd += rQD[i][r];
        }
        if (a.gbeta && t < L) a.gbeta[(size_t)bh * L + t] = yv - __expf(Gs[r]) * kx - yb;
        dGs[r] = t < L ? qd - Bt[r] * yv : 0.f;
    }
    if (!a.glg) return;
    __syncthreads();
    if (tid < C && t0 + tid < L) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += bpart[i];
        for (int u = C - 1; u >= tid; --u) acc += dGs[u];
        a.glg[(size_t)bh * L + t0 + tid] = acc;
    }
}

template <int DK, int DV>
hipError_t launch_gdn_bwd(const BwdArgs &a, hipStream_t st) {
    using Cfg = GdnScanCfg<DK, DV>;
    const int nch = a.nchunks;
    if (nch > 0) {
        PrepArgs p{};
        p.k = a.k; p.v = a.v; p.lg = a.lg; p.beta = a.beta;
        p.w = a.w; p.ut = a.u; p.t = a.t;
        p.BH = a.BH; p.L = a.L; p.Lp = a.Lp; p.dv = DV; p.nchunks = nch; p.ld = a.L;
        hipLaunchKernelGGL((gdn_prep_kernel<bf16, DK, 64, true>), dim3(a.BH * nch), dim3(256), 0, st, p);
        hipLaunchKernelGGL((gdn_bwd_dut_kernel<DK, DV>), dim3(a.BH * nch), dim3(256), 0, st, a);
    }
    hipLaunchKernelGGL((gdn_bwd_scan_kernel<DK, DV>), dim3(2 * a.BH * Cfg::NS), dim3(512), 0, st, a);
    if (nch > 0) {
        hipLaunchKernelGGL((gdn_bwd_grad_kernel<DK, DV>), dim3(a.BH * nch), dim3(512), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace la
