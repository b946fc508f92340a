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
// Mapping. One workgroup (NW waves) owns one (batch*head, DVT-column value
// slice) and walks the chunks in order, keeping its d_k x DVT slice of S in fp32
// MFMA accumulators for the whole sequence (nothing but Q, K, V, gates and O
// crosses HBM). Value slices of one head are placed on one XCD so Q and K are
// shared through that XCD's L2. Per chunk:
//   1. Wave 0 has built the gate tables (G, exp(G), exp(g_C - G), exp(g_C)) one
//      chunk ahead with a DPP prefix scan. All waves stage Q and K to LDS
//      row-major (score / inter operands), K also transposed and scaled by
//      exp(g_C - G_s) (state-update operand), V transposed, and S_prev
//      transposed in the operand type; transposed tiles are XOR-swizzled in
//      16-byte units. The global loads of chunk c+1 are issued right after chunk
//      c is staged, into registers, so their latency hides behind chunk c's math.
//   2. Query row blocks of 16 rows are assigned to waves by Roles: with C/8
//      waves, wave pairs split the value columns of one row block; with C/32
//      waves, each wave takes a row block and its mirror so the triangular score
//      work balances. A wave computes the inter term (S^T Q^T on MFMA), the score
//      tiles K_sb Q_rb^T for sb <= rb, masks/decays/rounds them in registers and
//      feeds them straight back as the B operand of the intra term V^T A^T: the D
//      layout of a score tile is exactly the B-operand layout of the next MFMA
//      with the key index in the K slots. Output rows are lane-indexed, so the
//      per-row scales (exp(G_r), 1/den_r) are per-lane scalars and each lane
//      stores four consecutive output columns.
//   3. S <- exp(g_C) S + K~^T V on MFMA into the accumulators; the state tiles
//      are split greedily so waves with fewer score tiles take more of them.
#pragma once

#include <type_traits>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

template <typename T> __device__ inline float frag_elem(const typename Mfma<T>::frag &f, int i);
template <> __device__ inline float frag_elem<f16>(const f16x8 &f, int i) { return (float)f[i]; }
template <> __device__ inline float frag_elem<float>(const float &f, int) { return f; }

// N dwords from global memory (N in {1, 2, 4, 8}; p aligned to the load size).
template <int N> __device__ inline void ld_dwords(const void *p, uint32_t (&d)[N]) {
    if constexpr (N == 1) {
        d[0] = *reinterpret_cast<const uint32_t *>(p);
    } else if constexpr (N == 2) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        d[0] = v.x; d[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
            d[4 * i] = v.x; d[4 * i + 1] = v.y; d[4 * i + 2] = v.z; d[4 * i + 3] = v.w;
        }
    }
}
// Dwords holding elements of type T, widened to fp32.
template <typename T, int N> __device__ inline float dw_elem(const uint32_t (&d)[N], int i) {
    if constexpr (sizeof(T) == 2) {
        return (i & 1) ? bf16_hi(d[i >> 1]) : bf16_lo(d[i >> 1]);
    } else {
        return __uint_as_float(d[i]);
    }
}

// Staging geometry: units of 4 tokens x X channels of a [C][D] tile. A 16-lane
// group covers 4 token quads x 4 channel groups, which keeps the transposed
// 4-token writes of a group on distinct LDS slots and loads rows in runs of
// 4 * X elements.
template <int C, int D, int X> struct Units {
    static constexpr int NCG = D / X;              // channel groups per token row
    static constexpr int CGL = NCG < 4 ? NCG : 4;  // channel groups per 16-lane group
    static constexpr int TQL = 16 / CGL;           // token quads per 16-lane group
    static constexpr int NCGG = NCG / CGL;
    static constexpr int N = (C / 4) * NCG;        // number of units
    static_assert(N % 16 == 0 && NCG % CGL == 0, "unit geometry");
    __device__ static inline void pos(int u, int &tq, int &cg) {
        const int gi = u >> 4, l16 = u & 15;
        tq = (gi / NCGG) * TQL + (l16 % TQL);
        cg = (gi % NCGG) * CGL + (l16 / TQL);
    }
};

// Channels per staging unit so that nthreads threads get one unit each when the
// tile allows (2 <= X <= 8).
constexpr int unit_width(int C, int D, int nthreads) {
    const int x = C * D / (4 * nthreads);
    return x < 2 ? 2 : (x > 8 ? 8 : x);
}

// X consecutive elements (as fp32) stored in type T.
template <typename T, int X> __device__ inline void st_row(T *p, const float *x) {
    if constexpr (X == 8) {
        f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
        st4<T>(p, a);
        st4<T>(p + 4, b);
    } else if constexpr (X == 4) {
        f32x4 a = {x[0], x[1], x[2], x[3]};
        st4<T>(p, a);
    } else {
        static_assert(X == 2, "row width");
        if constexpr (sizeof(T) == 2) {
            typedef T T2 __attribute__((ext_vector_type(2)));
            T2 v = {from_f32<T>(x[0]), from_f32<T>(x[1])};
            *reinterpret_cast<T2 *>(p) = v;
        } else {
            *reinterpret_cast<float2 *>(p) = make_float2(x[0], x[1]);
        }
    }
}

// Output-phase roles of wave w. Mode 0: NW == NRB, wave w owns row block w and
// every value column. Mode 1: NW == 2 NRB, waves w and w + NRB share row block w
// and take one half of the value columns each. Mode 2: NW == NRB / 2, wave w owns
// row blocks w and NRB - 1 - w (balanced triangle).
template <int NW, int NRB> struct Roles {
    static constexpr int MODE = (NW == NRB) ? 0 : (NW == 2 * NRB) ? 1 : (2 * NW == NRB) ? 2 : -1;
    static_assert(MODE >= 0, "wave count must be C/16, C/8 or C/32");
    static constexpr int RBW = MODE == 2 ? 2 : 1;
    static constexpr int rb(int w, int i) { return MODE == 2 ? (i == 0 ? w : NRB - 1 - w) : (w % NRB); }
    static constexpr int half(int w) { return MODE == 1 ? w / NRB : 0; }
    // relative score work of wave w (16 x 16 score tiles)
    static constexpr int score_tiles(int w) { return MODE == 2 ? NRB + 1 : (w % NRB) + 1; }
};

// Contiguous ranges of state tiles per wave, filled greedily so that waves with
// fewer score tiles take more state tiles.
template <int NTT, int NW> struct TileSplit {
    int start[NW];
    int cnt[NW];
    int maxcnt;
};
template <int NTT, int NW, int NRB>
constexpr TileSplit<NTT, NW> make_tile_split() {
    TileSplit<NTT, NW> t{};
    for (int w = 0; w < NW; ++w) t.cnt[w] = 0;
    for (int i = 0; i < NTT; ++i) {
        int best = 0;
        for (int w = 1; w < NW; ++w)
            if (Roles<NW, NRB>::score_tiles(w) + t.cnt[w] < Roles<NW, NRB>::score_tiles(best) + t.cnt[best]) best = w;
        ++t.cnt[best];
    }
    int acc = 0;
    t.maxcnt = 0;
    for (int w = 0; w < NW; ++w) {
        t.start[w] = acc;
        acc += t.cnt[w];
        if (t.cnt[w] > t.maxcnt) t.maxcnt = t.cnt[w];
    }
    return t;
}

template <int VAR, typename TM, int DK, int DVT, int C>
struct ChunkCfg {
    static constexpr bool DECAYED = (VAR == V_DECAY || VAR == V_GDN);
    static constexpr int PAD = 16 / (int)sizeof(TM);
    static constexpr int KP = DK + PAD;  // row pitch of Qs / Ks / STs (elements)
    static constexpr size_t lds_bytes =
        sizeof(TM) * (2 * (size_t)C * KP + (size_t)DK * C + (DECAYED ? 2 : 1) * (size_t)DVT * C +
                      (size_t)DVT * KP) +
        sizeof(float) * ((DECAYED ? 8 * C + 2 : 0) + (VAR == V_NORM ? 2 * DK : 0));
};

// TI: input storage type (bf16 or fp32); TO: output type (fp32 or bf16); the
// tensor-core operand type TM is fp16 for bf16 inputs and fp32 for fp32 inputs.
// NW: waves per workgroup; DVT: value columns per workgroup.
template <int VAR, typename TI, typename TO, int DK, int DVT, int C, int NW>
__global__ void __launch_bounds__(NW * 64) chunk_fwd_kernel(ChunkArgs a) {
    using TM = typename OpOf<TI>::type;
    using MF = Mfma<TM>;
    using frag = typename MF::frag;
    using Cfg = ChunkCfg<VAR, TM, DK, DVT, C>;
    constexpr int NT = NW * 64;          // threads
    constexpr int E = MF::E;
    constexpr int NRB = C / 16;          // 16-row blocks per chunk
    using R = Roles<NW, NRB>;
    constexpr bool DECAYED = Cfg::DECAYED;
    constexpr int KP = Cfg::KP;
    constexpr int NTI = DK / 16, NTJ = DVT / 16;
    constexpr int NTJW = R::MODE == 1 ? NTJ / 2 : NTJ;  // output column tiles per wave
    constexpr int NKS = DK / (4 * E);    // k-steps over channels
    constexpr int NTK = C / (4 * E);     // k-steps over tokens
    constexpr int PER = C / 64;          // tokens per lane in the gate scan
    constexpr int NQR = DK / 32;         // 8-element runs of one lane's channels (DK/4)
    constexpr int XK = unit_width(C, DK, NT), XV = unit_width(C, DVT, NT);
    using UK = Units<C, DK, XK>;
    using UV = Units<C, DVT, XV>;
    constexpr int NUK = (UK::N + NT - 1) / NT, NUV = (UV::N + NT - 1) / NT;
    constexpr int KRAW = XK * (int)sizeof(TI) / 4, VRAW = XV * (int)sizeof(TI) / 4;
    constexpr auto TS = make_tile_split<NTI * NTJ, NW, NRB>();
    constexpr int NTS = TS.maxcnt;       // state tiles per wave (at most)
    static_assert(NTJW >= 1 && (R::MODE != 1 || NTJ % 2 == 0), "value slice too narrow for the roles");
    static_assert(VAR != V_GDN || (R::MODE <= 1 && NRB == 4), "delta rule: one U row block per wave (pair)");

    __shared__ __attribute__((aligned(16))) TM Qs[C * KP];
    __shared__ __attribute__((aligned(16))) TM Ks[C * KP];
    __shared__ __attribute__((aligned(16))) TM KTs[DK * C];
    __shared__ __attribute__((aligned(16))) TM VTs[DVT * C];
    __shared__ __attribute__((aligned(16))) TM VWs[DECAYED ? DVT * C : 1];  // V (or U) scaled by w_s
    __shared__ __attribute__((aligned(16))) TM STs[DVT * KP];
    // Gate tables per buffer: [0] G_s, [1] exp(G_s), [2] w_s = exp(g_C - G_s),
    // [3] exp(G_{end of s's 16-block} - G_s); Tsc = exp(g_C).
    __shared__ __attribute__((aligned(16))) float Tg[DECAYED ? 2 * 4 * C : 1];
    __shared__ float Tsc[DECAYED ? 2 : 1];
    __shared__ float Zs[VAR == V_NORM ? 2 * DK : 1];
    TM *VW = DECAYED ? VWs : VTs;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int vid = xcd_virtual_block();
    const int bh = vid / a.nsplit, split = vid - bh * a.nsplit;
    const int j0 = split * DVT;
    const int L = a.L, dv = a.dv;
    int ts0 = 0, tsn = 0;  // this wave's state tiles (selected without indexing a table)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (wv == w) {
            ts0 = TS.start[w];
            tsn = TS.cnt[w];
        }
    }

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
        Sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m < tsn && a.s_in) {
            const int tile = ts0 + m, ti = tile / NTJ, tj = tile % NTJ;
            const float *sp = a.s_in + (size_t)bh * DK * dv + (size_t)(ti * 16 + 4 * g) * dv + j0 +
                              tj * 16 + n;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[m][e] = sp[(size_t)e * dv];
        }
    }
    if constexpr (VAR == V_NORM) {
        for (int i = tid; i < DK; i += NT) Zs[i] = a.z_in ? a.z_in[(size_t)bh * DK + i] : 0.f;
    }
    // Settle the prologue's loads here, so that no load is pending at the loop
    // head and the per-chunk waits can be exact (leaving output stores in flight).
    __builtin_amdgcn_s_waitcnt(0);

    // ---- registers of the next chunk, loaded one chunk ahead so that global
    // latency overlaps the current chunk's math. Every memory operation of a full
    // chunk is unconditional (threads without a staging unit load a duplicate
    // address), so the compiler's wait counts stay exact; only the ragged last
    // chunk clamps rows, which are zeroed when the registers are consumed.
    uint32_t kpre[NUK][4][KRAW];
    uint32_t qpre[NUK][4][KRAW];
    uint32_t vpre[NUV][4][VRAW];
    float gpre[PER];
    Raw8<TM> wpre[NQR];           // gated delta: W row of this wave's U row block
    f32x4 upre[NTJW];             // gated delta: U~ of this wave's U tiles
    const float *gsrc = lgg ? lgg : reinterpret_cast<const float *>(qg);

    auto load_chunk = [&](int c, auto ragged_tag) {
        constexpr bool RAGGED = decltype(ragged_tag)::value;
        const int t0 = c * C;
        auto row = [&](int t) { return RAGGED ? min(t, L - 1) : t; };
        if constexpr (DECAYED) {  // first: the gate tables wait only for these
#pragma unroll
            for (int p = 0; p < PER; ++p) gpre[p] = gsrc[row(t0 + lane * PER + p)];
        }
#pragma unroll
        for (int i = 0; i < NUK; ++i) {
            int tq, cg;
            UK::pos((tid + NT * i) % UK::N, tq, cg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = row(t0 + 4 * tq + r);
                ld_dwords<KRAW>(kg + (size_t)t * DK + cg * XK, kpre[i][r]);
                ld_dwords<KRAW>(qg + (size_t)t * DK + cg * XK, qpre[i][r]);
            }
        }
        if constexpr (VAR != V_GDN) {
#pragma unroll
            for (int i = 0; i < NUV; ++i) {
                int tq, cg;
                UV::pos((tid + NT * i) % UV::N, tq, cg);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = row(t0 + 4 * tq + r);
                    ld_dwords<VRAW>(vg + (size_t)t * dv + cg * XV, vpre[i][r]);
                }
            }
        }
        if constexpr (VAR == V_GDN) {
            const int srow = t0 + (wv % NRB) * 16 + n;  // W and U~ have Lp rows: always in range
#pragma unroll
            for (int i = 0; i < NQR; ++i) wpre[i] = ld_raw8<TM>(wg + (size_t)srow * DK + g * (DK / 4) + 8 * i);
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) {
                const int tj = R::half(wv) * NTJW + jt;
                upre[jt] = ld4<TM>(utg + (size_t)(tj * 16 + n) * a.Lp + t0 + (wv % NRB) * 16 + 4 * g);
            }
        }
    };

    // Gate tables of chunk c into buffer buf, from the prefetched log-gates.
    // Called by wave 0 only (wave-uniform), one chunk ahead of its use.
    auto gate_tables = [&](int c, int buf) {
        const int t0 = c * C;
        float *T = Tg + buf * 4 * C;
        if constexpr (PER == 1) {
            const float x = (lgg && t0 + lane < L) ? gpre[0] : 0.f;
            const float G = wave_inclusive_sum(x);
            const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
            // G at the last token of this lane's 16-token block (lanes 15, 31, 47, 63)
            const float e0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 15));
            const float e1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 31));
            const float e2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 47));
            const float Ge = (lane < 16) ? e0 : (lane < 32) ? e1 : (lane < 48) ? e2 : gC;
            T[lane] = G;
            T[C + lane] = __expf(G);
            T[2 * C + lane] = __expf(gC - G);
            T[3 * C + lane] = __expf(Ge - G);
            if (lane == 0) Tsc[buf] = __expf(gC);
        } else {
            float gl[PER];
            float run = 0.f;
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                run += (lgg && t0 + lane * PER + p < L) ? gpre[p] : 0.f;
                gl[p] = run;
            }
            const float incl = wave_inclusive_sum(run);
            const float excl = incl - run;
            const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
#pragma unroll
            for (int p = 0; p < PER; ++p) gl[p] += excl;
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int s = lane * PER + p, se = s | 15;
                const float x0 = __shfl(gl[0], se >> 1, 64), x1 = __shfl(gl[1], se >> 1, 64);
                const float Ge = (se & 1) ? x1 : x0;
                T[s] = gl[p];
                T[C + s] = __expf(gl[p]);
                T[2 * C + s] = __expf(gC - gl[p]);
                T[3 * C + s] = __expf(Ge - gl[p]);
            }
            if (lane == 0) Tsc[buf] = __expf(gC);
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
        const int buf = c & 1;
        const float *T = Tg + buf * 4 * C;
        __syncthreads();  // previous chunk done with every tile; gate tables visible

        // S_prev, transposed, in the operand type: STs[j][i].
#pragma unroll
        for (int m = 0; m < NTS; ++m) {
            if (m < tsn) {
                const int tile = ts0 + m, ti = tile / NTJ, tj = tile % NTJ;
                st4<TM>(&STs[(tj * 16 + n) * KP + ti * 16 + 4 * g], Sacc[m]);
            }
        }

        // ---- stage Q and K row-major, K transposed.
#pragma unroll
        for (int i = 0; i < NUK; ++i) {
            const int u = tid + NT * i;
            if (UK::N % NT == 0 || u < UK::N) {
                int tq, cg;
                UK::pos(u, tq, cg);
                float x[4][XK];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool valid = !RAGGED || t0 + 4 * tq + r < L;
                    float y[XK];
#pragma unroll
                    for (int e = 0; e < XK; ++e) {
                        y[e] = valid ? dw_elem<TI, KRAW>(qpre[i][r], e) : 0.f;
                        x[r][e] = valid ? dw_elem<TI, KRAW>(kpre[i][r], e) : 0.f;
                    }
                    st_row<TM, XK>(&Qs[(4 * tq + r) * KP + cg * XK], y);
                    st_row<TM, XK>(&Ks[(4 * tq + r) * KP + cg * XK], x[r]);
                }
#pragma unroll
                for (int e = 0; e < XK; ++e) {
                    f32x4 col = {x[0][e], x[1][e], x[2][e], x[3][e]};
                    st4<TM>(&KTs[tidx<C, TM>(cg * XK + e, 4 * tq)], col);
                }
            }
        }
        // ---- stage V transposed, and V scaled by w_s for the state update.
        if constexpr (VAR != V_GDN) {
#pragma unroll
            for (int i = 0; i < NUV; ++i) {
                const int u = tid + NT * i;
                if (UV::N % NT == 0 || u < UV::N) {
                    int tq, cg;
                    UV::pos(u, tq, cg);
                    f32x4 w4 = {1.f, 1.f, 1.f, 1.f};
                    if constexpr (DECAYED) w4 = *reinterpret_cast<const f32x4 *>(&T[2 * C + 4 * tq]);
#pragma unroll
                    for (int e = 0; e < XV; ++e) {
                        f32x4 col;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool valid = !RAGGED || t0 + 4 * tq + r < L;
                            col[r] = valid ? dw_elem<TI, VRAW>(vpre[i][r], e) : 0.f;
                        }
                        st4<TM>(&VTs[tidx<C, TM>(cg * XV + e, 4 * tq)], col);
                        if constexpr (DECAYED) st4<TM>(&VWs[tidx<C, TM>(cg * XV + e, 4 * tq)], col * w4);
                    }
                }
            }
        }

        // Delta rule: this chunk's W row and U~ as operands (the prefetch
        // registers are refilled right after the barrier).
        frag wf[VAR == V_GDN ? NKS : 1];
        f32x4 ucur[VAR == V_GDN ? NTJW : 1];
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
            for (int jt = 0; jt < NTJW; ++jt) ucur[jt] = upre[jt];
        }
        __syncthreads();  // staged tiles and STs visible

        if constexpr (NEXT == 1) {
            load_chunk(c + 1, full_t);
        } else if constexpr (NEXT == 2) {
            if (c + 1 < nchunks) load_chunk(c + 1, ragged_t);
        }
        // Keep the prefetch here: the scheduler would otherwise sink the loads
        // towards their use in the next chunk and expose their latency.
        __builtin_amdgcn_sched_barrier(0);

        // ---- gated delta rule: U = U~ - W S_prev for this wave's 16 rows and
        // column tiles, written transposed into VTs (intra operand) and scaled by
        // w_s into VWs (state operand). D[s][j]: lane (g, n) holds s = ub*16 + 4g + e.
        if constexpr (VAR == V_GDN) {
            const int ub = wv % NRB;
            const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&T[2 * C + ub * 16 + 4 * g]);
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) {
                const int jj = (R::half(wv) * NTJW + jt) * 16 + n;
                f32x4 acc = ucur[jt];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = MF::mma(wf[ks], ld_frag<TM>(&STs[jj * KP + g * (DK / 4) + ks * E]), acc);
                st4<TM>(&VTs[tidx<C, TM>(jj, ub * 16 + 4 * g)], acc);
                st4<TM>(&VWs[tidx<C, TM>(jj, ub * 16 + 4 * g)], acc * w4);
            }
            __syncthreads();
        }

        // ---- normalizer carry: z_next = z_prev + sum_s k_s (fp32), from the
        // transposed K tile.
        const int zc = (c & 1) * DK, zn = ((c + 1) & 1) * DK;
        if constexpr (VAR == V_NORM) {
            for (int i = tid; i < DK; i += NT) {
                float sacc = 0.f;
#pragma unroll
                for (int s0 = 0; s0 < C; s0 += 4) {  // 4 tokens never cross a swizzle unit
                    const f32x4 x = ld4<TM>(&KTs[tidx<C, TM>(i, s0)]);
                    sacc += (x[0] + x[1]) + (x[2] + x[3]);
                }
                Zs[zn + i] = Zs[zc + i] + sacc;
            }
        }

        // ---- outputs for one 16-row block and one range of value tiles; both
        // are compile-time constants so every score tile is straight-line code.
        auto row_block = [&](auto rb_tag, auto tj_tag) {
            constexpr int rb = decltype(rb_tag)::value;
            constexpr int tj0 = decltype(tj_tag)::value;
            const int rl = rb * 16 + n;   // chunk-local query row of this lane
            const int rrow = t0 + rl;
            frag qf[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qf[ks] = ld_frag<TM>(&Qs[rl * KP + g * (DK / 4) + ks * E]);
            const float Gr = DECAYED ? T[rl] : 0.f;

            // inter-chunk term: D[j][r] = exp(G_r) sum_i S[i][j] q_r[i]
            f32x4 oacc[NTJW];
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) {
                const int tj = tj0 + jt;
                oacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    oacc[jt] = MF::mma(ld_frag<TM>(&STs[(tj * 16 + n) * KP + g * (DK / 4) + ks * E]),
                                       qf[ks], oacc[jt]);
            }
            if constexpr (DECAYED) {
                const float er = T[C + rl];
#pragma unroll
                for (int jt = 0; jt < NTJW; ++jt) oacc[jt] *= er;
            }

            // score tiles D[s][r] = k_s . q_r for key blocks sb <= rb. Off the
            // diagonal, exp(G_r - G_s) = exp(G_r - G_e) exp(G_e - G_s) with e the
            // last token of block sb: both factors <= 1, so no overflow for any
            // gates, and one exp per tile.
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
                    if (sb == rb) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int sl = sb * 16 + 4 * g + e;
                            float x = sc[sb][e];
                            if constexpr (DECAYED) x *= __expf(Gr - T[sl]);
                            sc[sb][e] = (sl > rl) ? 0.f : x;
                        }
                    } else if constexpr (DECAYED) {
                        const float fr = __expf(Gr - T[sb * 16 + 15]);
                        const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&T[3 * C + sb * 16 + 4 * g]);
                        sc[sb] *= fr * b4;
                    }
                    if constexpr (VAR == V_NORM) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            sc[sb][e] = to_f32<TM>(from_f32<TM>(sc[sb][e]));
                            rowsum += sc[sb][e];
                        }
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
                        for (int jt = 0; jt < NTJW; ++jt) {
                            const int jj = (tj0 + jt) * 16 + n;
                            const V4 lo4 = *reinterpret_cast<const V4 *>(&VTs[tidx<C, TM>(jj, 32 * p + 4 * g)]);
                            V4 hi4 = *reinterpret_cast<const V4 *>(&VTs[tidx<C, TM>(jj, 32 * p + 16 + 4 * g)]);
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
                            oacc[jt] = MF::mma(aop, bop, oacc[jt]);
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
                            for (int jt = 0; jt < NTJW; ++jt)
                                oacc[jt] = MF::mma(VTs[tidx<C, TM>((tj0 + jt) * 16 + n, sb * 16 + 4 * g + e)],
                                                   sc[sb][e], oacc[jt]);
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
                for (int jt = 0; jt < NTJW; ++jt) oacc[jt] *= inv;
            }

            if (!RAGGED || rrow < L) {
#pragma unroll
                for (int jt = 0; jt < NTJW; ++jt)
                    st4<TO>(og + (size_t)rrow * dv + (tj0 + jt) * 16 + 4 * g, oacc[jt]);
            }
        };
        auto wave_role = [&](auto w_tag) {
            constexpr int W = decltype(w_tag)::value;
            row_block(std::integral_constant<int, R::rb(W, 0)>{},
                      std::integral_constant<int, R::half(W) * NTJW>{});
            if constexpr (R::RBW == 2)
                row_block(std::integral_constant<int, R::rb(W, 1)>{}, std::integral_constant<int, 0>{});
        };
        switch (wv) {
            case 0: wave_role(std::integral_constant<int, 0>{}); break;
            case 1: wave_role(std::integral_constant<int, 1>{}); break;
            case 2: wave_role(std::integral_constant<int, 2>{}); break;
            case 3: wave_role(std::integral_constant<int, 3>{}); break;
            default:
                if constexpr (NW == 8) {
                    switch (wv) {
                        case 4: wave_role(std::integral_constant<int, 4 % NW>{}); break;
                        case 5: wave_role(std::integral_constant<int, 5 % NW>{}); break;
                        case 6: wave_role(std::integral_constant<int, 6 % NW>{}); break;
                        default: wave_role(std::integral_constant<int, 7 % NW>{}); break;
                    }
                }
                break;
        }

        // ---- state update: S <- exp(g_C) S + K^T (w (.) V)
        if constexpr (DECAYED) {
            const float eg = Tsc[buf];
#pragma unroll
            for (int m = 0; m < NTS; ++m) Sacc[m] *= eg;
        }
#pragma unroll
        for (int m = 0; m < NTS; ++m) {
            if (m < tsn) {
                const int tile = ts0 + m, ti = tile / NTJ, tj = tile % NTJ;
#pragma unroll
                for (int ks = 0; ks < NTK; ++ks) {
                    const int s0 = g * (C / 4) + ks * E;
                    Sacc[m] = MF::mma(ld_frag<TM>(&KTs[tidx<C, TM>(ti * 16 + n, s0)]),
                                      ld_frag<TM>(&VW[tidx<C, TM>(tj * 16 + n, s0)]), Sacc[m]);
                }
            }
        }

        // ---- wave 0 prepares the next chunk's gate tables (its loads arrived
        // during this chunk's math).
        if constexpr (DECAYED) {
            if (NEXT != 0 && wv == 0 && c + 1 < nchunks) gate_tables(c + 1, buf ^ 1);
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
    if constexpr (DECAYED) {
        if (nchunks > 0 && wv == 0) gate_tables(0, 0);
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
            if (m < tsn) {
                const int tile = ts0 + m, ti = tile / NTJ, tj = tile % NTJ;
                float *sp = a.s_out + (size_t)bh * DK * dv + (size_t)(ti * 16 + 4 * g) * dv + j0 + tj * 16 + n;
#pragma unroll
                for (int e = 0; e < 4; ++e) sp[(size_t)e * dv] = Sacc[m][e];
            }
        }
    }
    if constexpr (VAR == V_NORM) {
        // The threads that wrote the last z update read it back: no barrier needed.
        if (a.z_out && split == 0)
            for (int i = tid; i < DK; i += NT) a.z_out[(size_t)bh * DK + i] = Zs[(nchunks & 1) * DK + i];
    }
}

template <int VAR, typename TI, typename TO, int DK, int DVT, int C, int NW>
hipError_t launch_chunk(const ChunkArgs &a, hipStream_t st) {
    const int blocks = a.BH * a.nsplit;
    hipLaunchKernelGGL((chunk_fwd_kernel<VAR, TI, TO, DK, DVT, C, NW>), dim3(blocks), dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
