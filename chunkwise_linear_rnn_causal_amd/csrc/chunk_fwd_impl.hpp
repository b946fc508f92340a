// chunk_fwd_impl.hpp -- fused chunkwise causal linear-attention forward (gfx950).
//
// Method (tensorplay "Talk Linear Attention", section 3.2, chunkwise parallel
// form; section 5.2 for the decayed variant): for chunk c of C tokens with
// chunk-local cumulative log-gate G_r and a_r = exp(G_r),
//   O_c    = diag(a) Q_c S_prev  +  (Gamma (.) Q_c K_c^T (.) M) V_c
//   S_next = a_C S_prev + (diag(a_C / a) K_c)^T V_c,   Gamma_rs = exp(G_r - G_s)
// with M the inclusive causal mask. Without gates a = 1. The normalized variant
// divides each output row by rowsum(Q_c K_c^T (.) M) + q_r . z_prev and carries
// z_next = z_prev + sum_s k_s (proig-chaa notes, sections 13-14). The gated delta
// rule replaces V_c by U_c = U~_c - W_c S_prev, with W and U~ prepared per chunk
// by gdn_prep (see gdn_prep_impl.hpp for the derivation).
//
// Mapping. One workgroup (4 waves) owns one (batch*head, 32-column value slice)
// and walks the chunks in order, keeping its d_k x 32 slice of S in fp32 MFMA
// accumulators for the whole sequence (nothing but Q, K, V, gates and O crosses
// HBM). Value slices of one head are placed on one XCD so Q and K are shared
// through that XCD's L2. Per chunk:
//   1. Q and K staged to LDS row-major (score / inter operands), K also
//      transposed + scaled by exp(g_C - G_s) (state-update operand), V
//      transposed; S_prev written to LDS transposed in the operand type. The
//      global loads of chunk c+1 are issued right after chunk c is staged, into
//      registers, so their latency hides behind chunk c's math.
//   2. Wave w owns query rows 16w..16w+15 (and the mirrored block for C = 128).
//      It computes the inter term (S^T Q^T on MFMA), the score tiles
//      K_sb Q_rb^T for sb <= rb, masks/decays/rounds them in registers and feeds
//      them straight back as the B operand of the intra term V^T A^T: the D
//      layout of a score tile is exactly the B-operand layout of the next MFMA
//      with the key index in the K slots. Output rows are lane-indexed, so the
//      per-row scales (exp(G_r), 1/den_r) are per-lane scalars and each lane
//      stores four consecutive output columns.
//   3. S <- exp(g_C) S + K~^T V on MFMA into the accumulators.
#pragma once

#include <type_traits>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

template <typename T> __device__ inline float frag_elem(const typename Mfma<T>::frag &f, int i);
template <> __device__ inline float frag_elem<f16>(const f16x8 &f, int i) { return (float)f[i]; }
template <> __device__ inline float frag_elem<float>(const float &f, int) { return f; }

template <int VAR, typename TM, int DK, int DVT, int C>
struct ChunkCfg {
    static constexpr int NW = 4;
    static constexpr int PAD = 16 / (int)sizeof(TM);
    static constexpr int KP = DK + PAD;  // row pitch of Ks / STs (elements)
    static constexpr size_t lds_bytes =
        sizeof(TM) * (2 * (size_t)C * KP + (size_t)DK * C + (size_t)DVT * C + (size_t)DVT * KP) +
        sizeof(float) * (C + (VAR == V_NORM ? 2 * DK : 1));
};

// TI: input storage type (bf16 or fp32); TO: output type (fp32 or bf16); the
// tensor-core operand type TM is fp16 for bf16 inputs and fp32 for fp32 inputs.
template <int VAR, typename TI, typename TO, int DK, int DVT, int C>
__global__ void __launch_bounds__(256) chunk_fwd_kernel(ChunkArgs a) {
    using TM = typename OpOf<TI>::type;
    using MF = Mfma<TM>;
    using frag = typename MF::frag;
    using Cfg = ChunkCfg<VAR, TM, DK, DVT, C>;
    constexpr int E = MF::E;
    constexpr int NW = Cfg::NW;
    constexpr int NRB = C / 16;          // 16-row blocks per chunk
    constexpr int RBW = NRB / NW;        // row blocks per wave (1 or 2)
    constexpr bool DECAYED = (VAR == V_DECAY || VAR == V_GDN);
    constexpr int KP = Cfg::KP;
    constexpr int NTI = DK / 16, NTJ = DVT / 16;
    constexpr int NTS = (NTI * NTJ + NW - 1) / NW;  // state tiles per wave
    constexpr int NKS = DK / (4 * E);    // k-steps over channels
    constexpr int NTK = C / (4 * E);     // k-steps over tokens
    constexpr int PER = C / 64;          // tokens per lane in the gate scan
    constexpr int NQR = DK / 32;         // 8-element runs of one lane's channels (DK/4)
    // K / V staging units of 4 tokens x 8 channels
    constexpr int KCB = DK / 8, KCBL = KCB < 4 ? KCB : 4, KTQL = 16 / KCBL, KNCBG = KCB / KCBL;
    constexpr int KUNITS = (C / 4) * KCB, NUK = (KUNITS + 255) / 256;
    constexpr int VCB = DVT / 8, VCBL = VCB < 4 ? VCB : 4, VTQL = 16 / VCBL, VNCBG = VCB / VCBL;
    constexpr int VUNITS = (C / 4) * VCB, NUV = (VUNITS + 255) / 256;
    static_assert(NRB % NW == 0 && (RBW == 1 || RBW == 2), "C must be 64 or 128");
    static_assert(DVT % 16 == 0 && DK % 32 == 0, "tile sizes");
    static_assert(KUNITS % 64 == 0, "K staging must be wave-uniform (it shuffles gates)");
    static_assert(VAR != V_GDN || NRB == NW, "one U row block per wave");

    __shared__ __attribute__((aligned(16))) TM Qs[C * KP];
    __shared__ __attribute__((aligned(16))) TM Ks[C * KP];
    __shared__ __attribute__((aligned(16))) TM KTs[DK * C];
    __shared__ __attribute__((aligned(16))) TM VTs[DVT * C];
    __shared__ __attribute__((aligned(16))) TM STs[DVT * KP];
    __shared__ float Gs[C];
    __shared__ float Zs[VAR == V_NORM ? 2 * DK : 1];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int vid = xcd_virtual_block();
    const int bh = vid / a.nsplit, split = vid - bh * a.nsplit;
    const int j0 = split * DVT;
    const int L = a.L, dv = a.dv;

    const TI *qg = (const TI *)a.q + (size_t)bh * L * DK;
    const TI *kg = (const TI *)a.k + (size_t)bh * L * DK;
    const TI *vg = (VAR == V_GDN) ? nullptr : (const TI *)a.v + (size_t)bh * L * dv + j0;
    TO *og = (TO *)a.o + (size_t)bh * L * dv + j0;
    const float *lgg = (DECAYED && a.lg) ? a.lg + (size_t)bh * L : nullptr;
    const TM *wg = (VAR == V_GDN) ? (const TM *)a.w + (size_t)bh * a.Lp * DK : nullptr;
    const TM *utg = (VAR == V_GDN) ? (const TM *)a.ut + ((size_t)bh * dv + j0) * a.Lp : nullptr;

    // ---- initial state slice in accumulator layout: lane (g, n) of tile (ti, tj)
    // holds S[ti*16 + 4g + e][j0 + tj*16 + n].
    f32x4 Sacc[NTS];
#pragma unroll
    for (int m = 0; m < NTS; ++m) {
        const int tile = wv + NW * m;
        Sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tile < NTI * NTJ && a.s_in) {
            const int ti = tile / NTJ, tj = tile % NTJ;
            const float *sp = a.s_in + (size_t)bh * DK * dv + (size_t)(ti * 16 + 4 * g) * dv + j0 +
                              tj * 16 + n;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[m][e] = sp[(size_t)e * dv];
        }
    }
    if constexpr (VAR == V_NORM) {
        for (int i = tid; i < DK; i += 256) Zs[i] = a.z_in ? a.z_in[(size_t)bh * DK + i] : 0.f;
    }
    // Settle the prologue's loads here, so that no load is pending at the loop
    // head and the per-chunk waits can be exact (leaving output stores in flight).
    __builtin_amdgcn_s_waitcnt(0);

    // ---- registers of the next chunk, loaded one chunk ahead so that global
    // latency overlaps the current chunk's math. Loads are unconditional from
    // clamped (always valid) rows; rows past L are zeroed when the registers are
    // consumed, so no load waits on a branch.
    Raw8<TI> kpre[NUK][4];
    Raw8<TI> qpre[NUK][4];
    Raw8<TI> vpre[NUV][4];
    float gpre[PER];
    Raw8<TM> wpre[NQR];           // gated delta: W row of this wave's U row block
    f32x4 upre[NTJ];              // gated delta: U~ of this wave's U row block

    // Every memory operation of a full chunk is unconditional (threads without a
    // staging unit load a duplicate address), so the compiler's wait counts stay
    // exact; only the ragged last chunk clamps rows.
    const float *gsrc = lgg ? lgg : reinterpret_cast<const float *>(qg);
    auto load_chunk = [&](int c, auto ragged_tag) {
        constexpr bool RAGGED = decltype(ragged_tag)::value;
        const int t0 = c * C;
        auto row = [&](int t) { return RAGGED ? min(t, L - 1) : t; };
#pragma unroll
        for (int i = 0; i < NUK; ++i) {
            const int u = (tid + 256 * i) % KUNITS;
            const int gi = u >> 4, l16 = u & 15;
            const int tq = (gi / KNCBG) * KTQL + (l16 % KTQL);
            const int cb = (gi % KNCBG) * KCBL + (l16 / KTQL);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = row(t0 + 4 * tq + r);
                kpre[i][r] = ld_raw8<TI>(kg + (size_t)t * DK + 8 * cb);
                qpre[i][r] = ld_raw8<TI>(qg + (size_t)t * DK + 8 * cb);
            }
        }
        if constexpr (VAR != V_GDN) {
#pragma unroll
            for (int i = 0; i < NUV; ++i) {
                const int u = (tid + 256 * i) % VUNITS;
                const int gi = u >> 4, l16 = u & 15;
                const int tq = (gi / VNCBG) * VTQL + (l16 % VTQL);
                const int cb = (gi % VNCBG) * VCBL + (l16 / VTQL);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = row(t0 + 4 * tq + r);
                    vpre[i][r] = ld_raw8<TI>(vg + (size_t)t * dv + 8 * cb);
                }
            }
        }
        if constexpr (DECAYED) {
#pragma unroll
            for (int p = 0; p < PER; ++p) gpre[p] = gsrc[row(t0 + lane * PER + p)];
        }
        if constexpr (VAR == V_GDN) {
            const int srow = t0 + wv * 16 + n;  // W and U~ have Lp rows: always in range
#pragma unroll
            for (int i = 0; i < NQR; ++i) wpre[i] = ld_raw8<TM>(wg + (size_t)srow * DK + g * (DK / 4) + 8 * i);
#pragma unroll
            for (int tj = 0; tj < NTJ; ++tj)
                upre[tj] = ld4<TM>(utg + (size_t)(tj * 16 + n) * a.Lp + t0 + wv * 16 + 4 * g);
        }
    };

    const int nchunks = (L + C - 1) / C;
    const int nfull = L / C;  // chunks with all C rows valid
    const std::true_type ragged_t{};
    const std::false_type full_t{};
    using NextNone = std::integral_constant<int, 0>;
    using NextFull = std::integral_constant<int, 1>;
    using NextTail = std::integral_constant<int, 2>;  // ragged next chunk if L % C != 0

    // One chunk. ragged_tag: this chunk has rows past L. next_tag: which loads to
    // issue for chunk c + 1.
    auto chunk_body = [&](int c, auto ragged_tag, auto next_tag) {
        constexpr bool RAGGED = decltype(ragged_tag)::value;
        constexpr int NEXT = decltype(next_tag)::value;
        const int t0 = c * C;
        __syncthreads();  // the previous chunk is done with every LDS tile

        // S_prev, transposed, in the operand type: STs[j][i].
#pragma unroll
        for (int m = 0; m < NTS; ++m) {
            const int tile = wv + NW * m;
            if (tile < NTI * NTJ) {
                const int ti = tile / NTJ, tj = tile % NTJ;
                st4<TM>(&STs[(tj * 16 + n) * KP + ti * 16 + 4 * g], Sacc[m]);
            }
        }

        // Chunk-local inclusive cumulative log-gate, computed by every wave.
        float gl[PER];
        float gC = 0.f;
        if constexpr (DECAYED) {
            float run = 0.f;
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                run += (lgg && (!RAGGED || t0 + lane * PER + p < L)) ? gpre[p] : 0.f;
                gl[p] = run;
            }
            float incl = run;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(incl, off, 64);
                if (lane >= off) incl += y;
            }
            float excl = __shfl_up(incl, 1, 64);
            if (lane == 0) excl = 0.f;
#pragma unroll
            for (int p = 0; p < PER; ++p) gl[p] += excl;
            gC = __shfl(incl, 63, 64);
            if (wv == 0) {
#pragma unroll
                for (int p = 0; p < PER; ++p) Gs[lane * PER + p] = gl[p];
            }
        }

        // ---- stage K row-major and transposed (scaled by exp(g_C - G_s)).
#pragma unroll
        for (int i = 0; i < NUK; ++i) {
            const int u = tid + 256 * i;
            if (KUNITS % 256 == 0 || u < KUNITS) {
                const int gi = u >> 4, l16 = u & 15;
                const int tq = (gi / KNCBG) * KTQL + (l16 % KTQL);
                const int cb = (gi % KNCBG) * KCBL + (l16 / KTQL);
                float x[4][8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool valid = !RAGGED || t0 + 4 * tq + r < L;
                    float y[8];
                    unpack8<TI>(qpre[i][r], y);
                    unpack8<TI>(kpre[i][r], x[r]);
                    if (!valid) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[r][e] = y[e] = 0.f;
                    }
                    st8<TM>(&Qs[(4 * tq + r) * KP + 8 * cb], y);
                    st8<TM>(&Ks[(4 * tq + r) * KP + 8 * cb], x[r]);
                }
                float wsc[4] = {1.f, 1.f, 1.f, 1.f};
                if constexpr (DECAYED) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int s = 4 * tq + r;
                        float Gsv;
                        if constexpr (PER == 1) {
                            Gsv = __shfl(gl[0], s, 64);
                        } else {
                            const float x0 = __shfl(gl[0], s >> 1, 64), x1 = __shfl(gl[1], s >> 1, 64);
                            Gsv = (s & 1) ? x1 : x0;
                        }
                        wsc[r] = __expf(gC - Gsv);
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    f32x4 col = {x[0][e] * wsc[0], x[1][e] * wsc[1], x[2][e] * wsc[2], x[3][e] * wsc[3]};
                    st4<TM>(&KTs[tidx<C>(8 * cb + e, 4 * tq)], col);
                }
            }
        }
        // ---- stage V (transposed) for the value slice.
        if constexpr (VAR != V_GDN) {
#pragma unroll
            for (int i = 0; i < NUV; ++i) {
                const int u = tid + 256 * i;
                if (VUNITS % 256 == 0 || u < VUNITS) {
                    const int gi = u >> 4, l16 = u & 15;
                    const int tq = (gi / VNCBG) * VTQL + (l16 % VTQL);
                    const int cb = (gi % VNCBG) * VCBL + (l16 / VTQL);
                    float x[4][8];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        unpack8<TI>(vpre[i][r], x[r]);
                        if (RAGGED && t0 + 4 * tq + r >= L) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) x[r][e] = 0.f;
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        f32x4 col = {x[0][e], x[1][e], x[2][e], x[3][e]};
                        st4<TM>(&VTs[tidx<C>(8 * cb + e, 4 * tq)], col);
                    }
                }
            }
        }

        // Delta rule: this chunk's W row and U~ as operands (the prefetch
        // registers are refilled right after the barrier).
        frag wf[VAR == V_GDN ? NKS : 1];
        f32x4 ucur[VAR == V_GDN ? NTJ : 1];
        if constexpr (VAR == V_GDN) {
#pragma unroll
            for (int i = 0; i < NQR; ++i) {
                if constexpr (E == 8) {
                    wf[i] = neg_frag<TM>(*reinterpret_cast<const frag *>(&wpre[i].v[0]));
                } else {
                    float x[8];
                    unpack8<TM>(wpre[i], x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) wf[8 * i + e] = -x[e];
                }
            }
#pragma unroll
            for (int tj = 0; tj < NTJ; ++tj) ucur[tj] = upre[tj];
        }
        __syncthreads();  // staged tiles, STs and Gs visible

        if constexpr (NEXT == 1) {
            load_chunk(c + 1, full_t);
        } else if constexpr (NEXT == 2) {
            if (c + 1 < nchunks) load_chunk(c + 1, ragged_t);
        }
        // Keep the prefetch here: the scheduler would otherwise sink the loads
        // towards their use in the next chunk and expose their latency.
        __builtin_amdgcn_sched_barrier(0);

        // ---- gated delta rule: U = U~ - W S_prev for this wave's 16 rows,
        // written transposed into VTs. D[s][j]: lane (g, n) holds s = wv*16 + 4g + e.
        if constexpr (VAR == V_GDN) {
#pragma unroll
            for (int tj = 0; tj < NTJ; ++tj) {
                const int jj = tj * 16 + n;
                f32x4 acc = ucur[tj];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = MF::mma(wf[ks], ld_frag<TM>(&STs[jj * KP + g * (DK / 4) + ks * E]), acc);
                st4<TM>(&VTs[tidx<C>(jj, wv * 16 + 4 * g)], acc);
            }
            __syncthreads();
        }

        // ---- normalizer carry: z_next = z_prev + sum_s k_s (fp32), from the
        // transposed K tile (unscaled for this variant).
        const int zc = (c & 1) * DK, zn = ((c + 1) & 1) * DK;
        if constexpr (VAR == V_NORM) {
            for (int i = tid; i < DK; i += 256) {
                float sacc = 0.f;
#pragma unroll
                for (int s0 = 0; s0 < C; s0 += 8) {
                    float x[8];
                    ld8<TM>(&KTs[tidx<C>(i, s0)], x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) sacc += x[e];
                }
                Zs[zn + i] = Zs[zc + i] + sacc;
            }
        }

        // ---- outputs for the row blocks this wave owns.
#pragma unroll
        for (int rr = 0; rr < RBW; ++rr) {
            const int rb = (rr == 0) ? wv : (NRB - 1 - wv);
            const int rl = rb * 16 + n;   // chunk-local query row of this lane
            const int rrow = t0 + rl;
            const float Gr = DECAYED ? Gs[rl] : 0.f;
            frag qf[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qf[ks] = ld_frag<TM>(&Qs[rl * KP + g * (DK / 4) + ks * E]);

            // inter-chunk term: D[j][r] = sum_i S[i][j] q_r[i]
            f32x4 oacc[NTJ];
#pragma unroll
            for (int tj = 0; tj < NTJ; ++tj) {
                oacc[tj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    oacc[tj] = MF::mma(ld_frag<TM>(&STs[(tj * 16 + n) * KP + g * (DK / 4) + ks * E]),
                                       qf[ks], oacc[tj]);
            }
            if constexpr (DECAYED) {
                const float er = __expf(Gr);
#pragma unroll
                for (int tj = 0; tj < NTJ; ++tj) oacc[tj] *= er;
            }

            // score tiles D[s][r] = k_s . q_r for key blocks sb <= rb.
            f32x4 sc[NRB];
            float rowsum = 0.f;
#pragma unroll
            for (int sb = 0; sb < NRB; ++sb) {
                sc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (sb <= rb) {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        sc[sb] = MF::mma(ld_frag<TM>(&Ks[(sb * 16 + n) * KP + g * (DK / 4) + ks * E]),
                                         qf[ks], sc[sb]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int sl = sb * 16 + 4 * g + e;
                        float x = sc[sb][e];
                        if (sl > rl) {
                            x = 0.f;
                        } else if constexpr (DECAYED) {
                            x *= __expf(Gr - Gs[sl]);
                        }
                        x = to_f32<TM>(from_f32<TM>(x));
                        sc[sb][e] = x;
                        if constexpr (VAR == V_NORM) rowsum += x;
                    }
                }
            }

            // intra-chunk term: D[j][r] += sum_s V[s][j] A[r][s]
            if constexpr (E == 8) {
                using V4 = typename Vec4<TM>::type;
#pragma unroll
                for (int p = 0; p < NRB / 2; ++p) {
                    if (2 * p <= rb) {
                        frag bop;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            bop[e] = from_f32<TM>(sc[2 * p][e]);
                            bop[4 + e] = from_f32<TM>(sc[2 * p + 1][e]);
                        }
                        const bool hi = (2 * p + 1 <= rb);
#pragma unroll
                        for (int tj = 0; tj < NTJ; ++tj) {
                            const int jj = tj * 16 + n;
                            const V4 lo4 = *reinterpret_cast<const V4 *>(&VTs[tidx<C>(jj, 32 * p + 4 * g)]);
                            V4 hi4 = *reinterpret_cast<const V4 *>(&VTs[tidx<C>(jj, 32 * p + 16 + 4 * g)]);
                            if (!hi) {
#pragma unroll
                                for (int e = 0; e < 4; ++e) hi4[e] = from_f32<TM>(0.0f);
                            }
                            frag aop;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                aop[e] = lo4[e];
                                aop[4 + e] = hi4[e];
                            }
                            oacc[tj] = MF::mma(aop, bop, oacc[tj]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int sb = 0; sb < NRB; ++sb) {
                    if (sb <= rb) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
#pragma unroll
                            for (int tj = 0; tj < NTJ; ++tj)
                                oacc[tj] = MF::mma(VTs[tidx<C>(tj * 16 + n, sb * 16 + 4 * g + e)],
                                                   sc[sb][e], oacc[tj]);
                        }
                    }
                }
            }

            if constexpr (VAR == V_NORM) {
                float qz = 0.f;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int el = 0; el < E; ++el)
                        qz += frag_elem<TM>(qf[ks], el) * Zs[zc + g * (DK / 4) + ks * E + el];
                float den = rowsum + qz;
                den += __shfl_xor(den, 16, 64);
                den += __shfl_xor(den, 32, 64);
                const float inv = 1.0f / den;
#pragma unroll
                for (int tj = 0; tj < NTJ; ++tj) oacc[tj] *= inv;
            }

            if (!RAGGED || rrow < L) {
#pragma unroll
                for (int tj = 0; tj < NTJ; ++tj) st4<TO>(og + (size_t)rrow * dv + tj * 16 + 4 * g, oacc[tj]);
            }
        }

        // ---- state update: S <- exp(g_C) S + K~^T V
        if constexpr (DECAYED) {
            const float eg = __expf(gC);
#pragma unroll
            for (int m = 0; m < NTS; ++m) Sacc[m] *= eg;
        }
#pragma unroll
        for (int m = 0; m < NTS; ++m) {
            const int tile = wv + NW * m;
            if (tile < NTI * NTJ) {
                const int ti = tile / NTJ, tj = tile % NTJ;
#pragma unroll
                for (int ks = 0; ks < NTK; ++ks) {
                    const int s0 = g * (C / 4) + ks * E;
                    Sacc[m] = MF::mma(ld_frag<TM>(&KTs[tidx<C>(ti * 16 + n, s0)]),
                                      ld_frag<TM>(&VTs[tidx<C>(tj * 16 + n, s0)]), Sacc[m]);
                }
            }
        }
    };

    // Schedule: the first full chunk is peeled so that both edges into the
    // steady-state loop leave the same memory operations in flight (the wait
    // counts inside the loop are then exact and let output stores drain in the
    // background); the last full chunk prefetches the ragged tail, if any.
    if (nfull > 0) {
        load_chunk(0, full_t);
    } else if (nchunks > 0) {
        load_chunk(0, ragged_t);
    }
    if (nfull >= 2) {
        chunk_body(0, full_t, NextFull{});
        for (int c = 1; c < nfull - 1; ++c) chunk_body(c, full_t, NextFull{});
    }
    if (nfull >= 1) chunk_body(nfull - 1, full_t, NextTail{});
    if (nfull < nchunks) chunk_body(nfull, ragged_t, NextNone{});

    if (a.s_out) {
#pragma unroll
        for (int m = 0; m < NTS; ++m) {
            const int tile = wv + NW * m;
            if (tile < NTI * NTJ) {
                const int ti = tile / NTJ, tj = tile % NTJ;
                float *sp = a.s_out + (size_t)bh * DK * dv + (size_t)(ti * 16 + 4 * g) * dv + j0 + tj * 16 + n;
#pragma unroll
                for (int e = 0; e < 4; ++e) sp[(size_t)e * dv] = Sacc[m][e];
            }
        }
    }
    if constexpr (VAR == V_NORM) {
        // The threads that wrote the last z update read it back: no barrier needed.
        if (a.z_out && split == 0)
            for (int i = tid; i < DK; i += 256) a.z_out[(size_t)bh * DK + i] = Zs[(nchunks & 1) * DK + i];
    }
}

template <int VAR, typename TI, typename TO, int DK, int DVT, int C>
hipError_t launch_chunk(const ChunkArgs &a, hipStream_t st) {
    const int blocks = a.BH * a.nsplit;
    hipLaunchKernelGGL((chunk_fwd_kernel<VAR, TI, TO, DK, DVT, C>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
