// vdecay_fwd_impl.hpp -- chunkwise forward with one decay gate per key channel
// (gfx950).
//
// Method. The update S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t
// (tensorplay "Talk Linear Attention", section 5.1: the GLA gate matrix G_t (.)
// S_{t-1} with alpha_t broadcast over the value columns; wln20 "LLM注意力优化：
// 线性注意力", Kimi Delta Attention section, the diagonal gate Diag(alpha_t)).
// With the chunk-local cumulative log-gate G_r[c] = sum_{u<=r} l_u[c], the
// chunk form is the per-channel version of the scalar one (tensorplay section
// 5.2, (Q (.) B)(K / B)^T with B the cumulative product):
//   O_c    = (Q (.) e^G) S_prev + A V,   A_rs = sum_c q_r[c] k_s[c] e^{G_r[c] - G_s[c]}  (s <= r)
//   S_next = Diag(e^{G_end}) S_prev + (K (.) e^{G_end - G})^T V
// The decay no longer factors out of A, and e^{-G} alone overflows, so A is
// formed per 16-token block pair around each block's middle token m_i:
//   q_r e^{G_r - G_{m_i}}  and  k_s e^{G_{m_j} - G_s}   (row r in block i, key s in block j)
// are each within 8 tokens of their reference, and the pair is joined by the
// per-channel factor D_ij = e^{G_{m_i} - G_{m_j}} <= 1, applied to the key
// operand in registers. Every factor is bounded by e^{8 max|l|}; with l >= -10
// (the documented domain) all of them stay below e^80 and fit the fp32 range of
// the score operands (bf16 for bf16 inputs, fp32 for fp32 inputs). One exp per
// element per chunk plus 15 per channel, instead of one per (row, key, channel).
// The diagonal score q_t . k_t carries no decay; it is taken in fp32 from the
// inputs, so bf16's rounding only touches terms damped by at least one gate.
// When a chunk's rebased operands all stay below 2^14 (the common case for
// moderate gates), they are stored and multiplied as fp16 instead, with 8x
// finer rounding; a workgroup vote picks the type per chunk.
//
// Mapping. One workgroup (8 waves) owns one (batch*head, DVT-column value
// slice) and walks the chunks in order with its d_k x DVT slice of S in fp32
// MFMA accumulators. Per chunk:
//  1. each wave loads the gates of d_k/8 channels with the chunk's rows in its
//     lanes, takes the per-channel prefix with a DPP wave scan, writes G, and
//     forms those channels' 15 reference factors from the rows it wrote;
//  2. every thread derives its q and k segments' operand rows (one exp each);
//  3. the chunk's 10 score tiles are spread over the waves and written, as
//     A[r][s] in the operand type, over the dead gate tile; after a barrier
//     each wave computes the output tiles of one query row block and one half
//     of the slice's columns (inter term, intra term V^T A^T) and its share of
//     the state tiles.
// Four barriers per chunk. The next chunk's gates and V are loaded as soon as
// this chunk's are consumed (step 1), its q and k after step 2.
#pragma once

#include <type_traits>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

// Per-channel log-gates below this are taken as this value: the chunk form
// rebases the decay around the middle of each 16-token block, and with every
// gate in [-10, 0] each rebased factor stays below e^80, inside fp32. A gate of
// e^-10 already damps the channel's history to 4.5e-5 per token, so the clamp
// moves the result by at most that fraction of the damped history.
constexpr float kMinChannelLogGate = -10.0f;

// Score operand type: bf16 for bf16 inputs (the exponent range of fp32), fp32
// for fp32 inputs.
template <typename TI> struct ScoreOp;
template <> struct ScoreOp<bf16> { using type = bf16; };
template <> struct ScoreOp<float> { using type = float; };

template <typename TI, int DK, int DVT> struct VdCfg {
    using TM = typename OpOf<TI>::type;
    using TS = typename ScoreOp<TI>::type;
    static constexpr int C = 64, NT = 512, NRB = 4;
    static constexpr bool H = sizeof(TM) == 2;
    static constexpr int PG = DK + 4;                  // gate tile pitch (fp32)
    static constexpr int PQ = H ? DK + 8 : DK + 4;     // Qh, Qe, Kb, St pitch
    static constexpr int PK = H ? DK + 16 : DK + 4;    // Kt pitch (transpose reads)
    static constexpr int PV = H ? DVT + 16 : DVT + 4;  // V pitch (transpose reads)
    static constexpr int GW = DK / 8;                  // gate channels per wave
    // factor rows: e^{G_m_i} (4), e^{G_end - G_m_j} (4), D_ij (6), e^{G_end} (1)
    static constexpr int NF = 15, FQ = 0, FKT = 4, FD = 8, FEND = 14;
    static constexpr int PSB = H ? C + 8 : C + 4;      // score buffer pitch
    static constexpr size_t GBYTES = (size_t)C * PG * 4, SBYTES = (size_t)C * PSB * sizeof(TM);
    static constexpr size_t oG = 0;                    // gates; the scores reuse it in step 3
    static constexpr size_t oF = oG + (GBYTES > SBYTES ? GBYTES : SBYTES);
    static constexpr size_t oQh = oF + (size_t)NF * DK * 4;
    static constexpr size_t oQe = oQh + (size_t)C * PQ * sizeof(TS);
    static constexpr size_t oKb = oQe + (size_t)C * PQ * sizeof(TM);
    static constexpr size_t oKt = oKb + (size_t)C * PQ * sizeof(TS);
    static constexpr size_t oV = oKt + (size_t)C * PK * sizeof(TM);
    static constexpr size_t oSt = oV + (size_t)C * PV * sizeof(TM);
    static constexpr size_t oQK = oSt + 2 * (size_t)DVT * PQ * sizeof(TM);
    static constexpr size_t BYTES = oQK + (size_t)C * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <typename T> struct type_tag { using type = T; };

// factor row of D_ij, i > j
__device__ constexpr int d_row(int i, int j) { return j == 0 ? i - 1 : (j == 1 ? i + 1 : 5); }

template <typename TI, typename TO, int DK, int DVT>
__global__ void __launch_bounds__(512) vdecay_fwd_kernel(ChunkArgs a) {
    using Cfg = VdCfg<TI, DK, DVT>;
    using TM = typename Cfg::TM;
    using TS = typename Cfg::TS;
    using MF = Mfma<TM>;
    using MS = Mfma<TS>;
    using frag = typename MF::frag;
    using sfrag = typename MS::frag;
    constexpr int C = Cfg::C, NRB = Cfg::NRB, PG = Cfg::PG, PQ = Cfg::PQ, PK = Cfg::PK, PV = Cfg::PV;
    constexpr int GW = Cfg::GW;
    constexpr bool H = Cfg::H;
    constexpr int E = MF::E;
    static_assert(MS::E == E, "operand shapes");
    constexpr int NKS = DK / (4 * E);       // k-steps over channels
    constexpr int NTK = C / (4 * E);        // k-steps over tokens (state update)
    constexpr int NTJ = DVT / 16, NTI = DK / 16, NTILE = NTI * NTJ;
    constexpr int NTJW = NTJ / 2;           // output tiles per wave (half the slice)
    constexpr int TPW = (NTILE + 7) / 8;    // state tiles per wave
    constexpr int SEGQ = DK / 8, SEGV = DVT / 8;
    constexpr int NQS = (C * SEGQ + 511) / 512;
    constexpr int NVS = (C * SEGV + 511) / 512;
    static_assert(DVT == 32 || DVT == 64, "value slice");

    __shared__ __align__(16) unsigned char smem[Cfg::BYTES];
    float *Gs = reinterpret_cast<float *>(smem + Cfg::oG);
    float *F = reinterpret_cast<float *>(smem + Cfg::oF);
    TS *Qh = reinterpret_cast<TS *>(smem + Cfg::oQh);
    TM *Qe = reinterpret_cast<TM *>(smem + Cfg::oQe);
    TS *Kb = reinterpret_cast<TS *>(smem + Cfg::oKb);
    TM *Kt = reinterpret_cast<TM *>(smem + Cfg::oKt);
    TM *Vs = reinterpret_cast<TM *>(smem + Cfg::oV);
    TM *St = reinterpret_cast<TM *>(smem + Cfg::oSt);
    float *QK = reinterpret_cast<float *>(smem + Cfg::oQK);  // q_t . k_t per row
    __shared__ float Vote[8];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int vid = xcd_virtual_block();
    const int bh = vid / a.nsplit, split = vid % a.nsplit;
    const int L = a.L, dv = a.dv, j0 = split * DVT;
    const TI *qg = (const TI *)a.q + (size_t)bh * a.ld * DK;
    const TI *kg = (const TI *)a.k + (size_t)bh * a.ld * DK;
    const TI *vg = (const TI *)a.v + (size_t)bh * a.ld * dv + j0;
    const float *lgg = a.lg + (size_t)bh * a.ld * DK + wv * GW;  // this wave's gate channels
    TO *og = (TO *)a.o + (size_t)bh * a.ld * dv + j0;
    const int nchunks = (L + C - 1) / C;
    const int rb = wv < 4 ? wv : 7 - wv;  // query row block (waves w, w+4 share a SIMD)
    const int hh = wv >> 2;               // half of the value slice

    // ---- carried state: tile wv + 8 m covers rows 16 ci + 4g + e, columns 16 cj + n
    f32x4 Sacc[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        Sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile = wv + 8 * m;
        if (tile < NTILE && a.s_in) {
            const int ci = tile / NTJ, cj = tile % NTJ;
            const float *sp = a.s_in + (size_t)bh * DK * dv + (size_t)(ci * 16 + 4 * g) * dv + j0 + cj * 16 + n;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[m][e] = sp[(size_t)e * dv];
        }
    }
    auto write_st = [&](TM *Sdst) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int tile = wv + 8 * m;
            if (tile < NTILE) {
                const int ci = tile / NTJ, cj = tile % NTJ;
                st4<TM>(&Sdst[(cj * 16 + n) * PQ + ci * 16 + 4 * g], Sacc[m]);
            }
        }
    };
    write_st(St);

    // ---- chunk registers: q, k segments tid + 512 m of the [C][DK/8] grid, v of
    // the [C][DVT/8] grid, and this wave's GW gate channels of row `lane`
    Raw8<TI> rq[NQS], rk[NQS], rv[NVS];
    f32x4 gl[GW / 4];
    auto load_qk = [&](int c) __attribute__((always_inline)) {
        const int t0 = c * C, nv = min(C, L - t0);
#pragma unroll
        for (int m = 0; m < NQS; ++m) {
            const int sid = tid + 512 * m, row = sid / SEGQ, cs = sid % SEGQ;
            if (sid < C * SEGQ && row < nv) {
                const size_t off = (size_t)(t0 + row) * DK + 8 * cs;
                rq[m] = ld_raw8<TI>(qg + off);
                rk[m] = ld_raw8<TI>(kg + off);
            } else {
                rq[m] = zero_raw8<TI>();
                rk[m] = zero_raw8<TI>();
            }
        }
    };
    auto load_gv = [&](int c) __attribute__((always_inline)) {
        const int t0 = c * C, nv = min(C, L - t0);
#pragma unroll
        for (int m = 0; m < NVS; ++m) {
            const int sid = tid + 512 * m, row = sid / SEGV, cs = sid % SEGV;
            rv[m] = (sid < C * SEGV && row < nv) ? ld_raw8<TI>(vg + (size_t)(t0 + row) * dv + 8 * cs)
                                                 : zero_raw8<TI>();
        }
#pragma unroll
        for (int u = 0; u < GW / 4; ++u)
            gl[u] = lane < nv ? *reinterpret_cast<const f32x4 *>(lgg + (size_t)(t0 + lane) * DK + 4 * u)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    if (nchunks > 0) {
        load_gv(0);
        load_qk(0);
    }

    // reference rows of the 15 factors (fr = lane % 16): e^{G[ra] - G[rb]}, rb < 0: none
    const int fr = lane & 15;
    const int ra = fr < 4 ? 16 * fr + 8 : fr < 8 ? C - 1 : fr == 8 ? 24 : fr == 9 ? 40 : fr == 10 ? 56
                 : fr == 11 ? 40 : fr < 14 ? 56 : C - 1;
    const int rbf = fr < 4 ? -1 : fr < 8 ? 16 * (fr - 4) + 8 : fr < 11 ? 8 : fr < 13 ? 24 : fr == 13 ? 40 : -1;

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C, nv = min(C, L - t0);
        __syncthreads();  // previous chunk's readers are done; S^T of chunk c-1 visible

        // ---- 1. V into LDS; gates: per-channel prefix over the rows (lanes), G
        // and the reference factors of this wave's channels
#pragma unroll
        for (int m = 0; m < NVS; ++m) {
            const int sid = tid + 512 * m;
            if (sid < C * SEGV) {
                float x[8];
                unpack8<TI>(rv[m], x);
                st8<TM>(&Vs[(sid / SEGV) * PV + 8 * (sid % SEGV)], x);
            }
        }
#pragma unroll
        for (int u = 0; u < GW / 4; ++u) {
            f32x4 gsum;
#pragma unroll
            for (int e = 0; e < 4; ++e) gsum[e] = wave_inclusive_sum(fmaxf(gl[u][e], kMinChannelLogGate));
            *reinterpret_cast<f32x4 *>(&Gs[lane * PG + wv * GW + 4 * u]) = gsum;
        }
        // the wave reads back the rows it just wrote (one wave's LDS operations
        // complete in order): factor fr of channel (lane >> 4) + 4 it
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < GW / 4; ++it) {
            const int ch = wv * GW + (lane >> 4) + 4 * it;
            if (fr < Cfg::NF) {
                const float xa = Gs[ra * PG + ch];
                const float xb = rbf < 0 ? 0.f : Gs[rbf * PG + ch];
                F[fr * DK + ch] = __expf(xa - xb);
            }
        }
        if (c + 1 < nchunks) load_gv(c + 1);  // a whole chunk of cover for the gates
        __syncthreads();

        // ---- 2. operand rows from this thread's q and k segments
        float qh[NQS][8], kb[NQS][8], big = 0.f;
#pragma unroll
        for (int m = 0; m < NQS; ++m) {
            const int sid = tid + 512 * m;
            if (sid < C * SEGQ) {
                const int row = sid / SEGQ, c0 = 8 * (sid % SEGQ);
                const int blk = row >> 4, mid = 16 * blk + 8;
                float q8[8], k8[8], gr[8], gm[8], fq[8], fk[8];
                unpack8<TI>(rq[m], q8);
                unpack8<TI>(rk[m], k8);
#pragma unroll
                for (int h4 = 0; h4 < 2; ++h4) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&Gs[row * PG + c0 + 4 * h4]);
                    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&Gs[mid * PG + c0 + 4 * h4]);
                    const f32x4 c4 = *reinterpret_cast<const f32x4 *>(&F[(Cfg::FQ + blk) * DK + c0 + 4 * h4]);
                    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&F[(Cfg::FKT + blk) * DK + c0 + 4 * h4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        gr[4 * h4 + e] = a4[e];
                        gm[4 * h4 + e] = b4[e];
                        fq[4 * h4 + e] = c4[e];
                        fk[4 * h4 + e] = d4[e];
                    }
                }
                // the undecayed diagonal score q_t . k_t from the inputs themselves,
                // reduced over the row's SEGQ consecutive lanes
                float qk = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) qk += q8[e] * k8[e];
#pragma unroll
                for (int off = 1; off < SEGQ; off <<= 1) qk += __shfl_xor(qk, off, 64);
                if (c0 == 0) QK[row] = qk;
                float qe[8], kt[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    qh[m][e] = q8[e] * __expf(gr[e] - gm[e]);
                    qe[e] = qh[m][e] * fq[e];
                    kb[m][e] = k8[e] * __expf(gm[e] - gr[e]);
                    kt[e] = kb[m][e] * fk[e];
                    big = fmaxf(big, fmaxf(fabsf(qh[m][e]), fabsf(kb[m][e])));
                }
                st8<TM>(&Qe[row * PQ + c0], qe);
                st8<TM>(&Kt[row * PK + c0], kt);
            }
        }
        // fp16 score operands when every rebased value of the chunk fits fp16 with
        // headroom (then 8x finer rounding than bf16), else bf16: a workgroup vote
        bool sf16 = false;
        if constexpr (H) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) big = fmaxf(big, __shfl_xor(big, off, 64));
            if (lane == 0) Vote[wv] = big;
            __syncthreads();
            float all = Vote[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) all = fmaxf(all, Vote[i]);
            sf16 = all < 16384.f;
        }
#pragma unroll
        for (int m = 0; m < NQS; ++m) {
            const int sid = tid + 512 * m;
            if (sid < C * SEGQ) {
                const int row = sid / SEGQ, c0 = 8 * (sid % SEGQ);
                if (sf16) {
                    st8<f16>(reinterpret_cast<f16 *>(&Qh[row * PQ + c0]), qh[m]);
                    st8<f16>(reinterpret_cast<f16 *>(&Kb[row * PQ + c0]), kb[m]);
                } else {
                    st8<TS>(&Qh[row * PQ + c0], qh[m]);
                    st8<TS>(&Kb[row * PQ + c0], kb[m]);
                }
            }
        }
        if (c + 1 < nchunks) load_qk(c + 1);
        __syncthreads();

        // ---- 3a. the chunk's 10 score tiles D[s][r] (key block sb <= query block
        // rb), spread over the waves, into the score buffer as A[r][s]; off the
        // diagonal block the key operand takes the factor D_{rb,sb} of its channels
        TM *SB = reinterpret_cast<TM *>(smem + Cfg::oG);
        constexpr int PSB = Cfg::PSB;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int tix = wv + 8 * m;
            if (tix < NRB * (NRB + 1) / 2) {
                const int trb = tix < 1 ? 0 : tix < 3 ? 1 : tix < 6 ? 2 : 3;
                const int tsb = tix - trb * (trb + 1) / 2;
                const float *Dr = &F[(Cfg::FD + (tsb < trb ? d_row(trb, tsb) : 0)) * DK];
                // the tile in score operand type T (stored in the 2- or 4-byte tiles)
                auto score = [&](auto t_tag) __attribute__((always_inline)) -> f32x4 {
                    using T = typename decltype(t_tag)::type;
                    using M = Mfma<T>;
                    const T *Kbt = reinterpret_cast<const T *>(Kb);
                    const T *Qht = reinterpret_cast<const T *>(Qh);
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int col = g * (DK / 4) + ks * E;
                        typename M::frag kf = ld_frag<T>(&Kbt[(tsb * 16 + n) * PQ + col]);
                        if (tsb < trb) {
                            if constexpr (E == 8) {
                                const f32x4 d0 = *reinterpret_cast<const f32x4 *>(&Dr[col]);
                                const f32x4 d1 = *reinterpret_cast<const f32x4 *>(&Dr[col + 4]);
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    kf[e] = from_f32<T>(to_f32<T>(kf[e]) * d0[e]);
                                    kf[4 + e] = from_f32<T>(to_f32<T>(kf[4 + e]) * d1[e]);
                                }
                            } else {
                                kf = kf * Dr[col];
                            }
                        }
                        acc = M::mma(kf, ld_frag<T>(&Qht[(trb * 16 + n) * PQ + col]), acc);
                    }
                    return acc;
                };
                f32x4 sc;
                if constexpr (H) {
                    sc = sf16 ? score(type_tag<f16>{}) : score(type_tag<TS>{});
                } else {
                    sc = score(type_tag<TS>{});
                }
                if (tsb == trb) {  // causal mask; the diagonal itself is exact
                    const float qk = QK[trb * 16 + n];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (4 * g + e > n) sc[e] = 0.f;
                        if (4 * g + e == n) sc[e] = qk;
                    }
                }
                st4<TM>(&SB[(trb * 16 + n) * PSB + tsb * 16 + 4 * g], sc);
            }
        }
        __syncthreads();

        // ---- 3b. this wave's output tiles (query block rb, half hh of the slice)
        const TM *Stc = St + (c & 1) * DVT * PQ;
        TM *Stn = St + ((c + 1) & 1) * DVT * PQ;
        const int rl_ = rb * 16 + n;    // chunk-local query row of this lane (B operand column)
        const int jw = hh * (DVT / 2);  // first value column of this wave
        frag qe[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qe[ks] = ld_frag<TM>(&Qe[rl_ * PQ + g * (DK / 4) + ks * E]);
        // inter: D[j][r] = sum_c S[c][j] q_r[c] e^{G_r[c]}
        f32x4 oacc[NTJW];
#pragma unroll
        for (int jt = 0; jt < NTJW; ++jt) {
            oacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                oacc[jt] = MF::mma(ld_frag<TM>(&Stc[(jw + jt * 16 + n) * PQ + g * (DK / 4) + ks * E]), qe[ks],
                                   oacc[jt]);
        }
        // intra: D[j][r] += sum_s V[s][j] A[r][s], the scores read back with the
        // token slots of the V^T operand: s = 32p + 4g + (0..3), 32p + 16 + 4g + (0..3)
        if constexpr (H) {
#pragma unroll
            for (int p = 0; p < NRB / 2; ++p) {
                if (2 * p <= rb) {
                    frag bop;
                    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
                    const h4 lo = *reinterpret_cast<const h4 *>(&SB[rl_ * PSB + 32 * p + 4 * g]);
                    h4 hi = {0, 0, 0, 0};
                    if (2 * p + 1 <= rb) hi = *reinterpret_cast<const h4 *>(&SB[rl_ * PSB + 32 * p + 16 + 4 * g]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bop[e] = lo[e];
                        bop[4 + e] = hi[e];
                    }
#pragma unroll
                    for (int jt = 0; jt < NTJW; ++jt)
                        oacc[jt] = MF::mma(tr_frag<PV>(Vs, 32 * p + 4 * g, jw + jt * 16, lane), bop, oacc[jt]);
                }
            }
        } else {
#pragma unroll
            for (int sb = 0; sb < NRB; ++sb) {
                if (sb <= rb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float a_ = SB[rl_ * PSB + sb * 16 + 4 * g + e];
#pragma unroll
                        for (int jt = 0; jt < NTJW; ++jt)
                            oacc[jt] = MF::mma(Vs[(sb * 16 + 4 * g + e) * PV + jw + jt * 16 + n], a_, oacc[jt]);
                    }
                }
            }
        }
        if (rl_ < nv) {
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt)
                st4<TO>(og + (size_t)(t0 + rl_) * dv + jw + jt * 16 + 4 * g, oacc[jt]);
        }

        // state: S <- Diag(e^{G_end}) S + (K (.) e^{G_end - G})^T V
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int tile = wv + 8 * m;
            if (tile < NTILE) {
                const int ci = tile / NTJ, cj = tile % NTJ;
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(&F[Cfg::FEND * DK + ci * 16 + 4 * g]);
                Sacc[m] *= eg;
#pragma unroll
                for (int ks = 0; ks < NTK; ++ks) {
                    frag ka, vb;
                    if constexpr (H) {
                        ka = tr_frag<PK>(Kt, 32 * ks + 4 * g, ci * 16, lane);
                        vb = tr_frag<PV>(Vs, 32 * ks + 4 * g, cj * 16, lane);
                    } else {
                        ka = Kt[(4 * ks + g) * PK + ci * 16 + n];
                        vb = Vs[(4 * ks + g) * PV + cj * 16 + n];
                    }
                    Sacc[m] = MF::mma(ka, vb, Sacc[m]);
                }
            }
        }
        write_st(Stn);
    }

    if (a.s_out) {
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int tile = wv + 8 * m;
            if (tile < NTILE) {
                const int ci = tile / NTJ, cj = tile % NTJ;
                float *sp = a.s_out + (size_t)bh * DK * dv + (size_t)(ci * 16 + 4 * g) * dv + j0 + cj * 16 + n;
#pragma unroll
                for (int e = 0; e < 4; ++e) sp[(size_t)e * dv] = Sacc[m][e];
            }
        }
    }
}

template <typename TI, typename TO, int DK>
hipError_t launch_vdecay(const ChunkArgs &a, hipStream_t st) {
    // 64-column slices halve the per-head gate and operand work against 32
    ChunkArgs b = a;
    if (a.dv % 64 == 0) {
        b.nsplit = a.dv / 64;
        hipLaunchKernelGGL((vdecay_fwd_kernel<TI, TO, DK, 64>), dim3(b.BH * b.nsplit), dim3(512), 0, st, b);
    } else {
        b.nsplit = a.dv / 32;
        hipLaunchKernelGGL((vdecay_fwd_kernel<TI, TO, DK, 32>), dim3(b.BH * b.nsplit), dim3(512), 0, st, b);
    }
    return hipGetLastError();
}

}  // namespace la
