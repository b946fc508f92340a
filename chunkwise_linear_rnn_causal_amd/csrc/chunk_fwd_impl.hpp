// chunk_fwd_impl.hpp -- fused chunkwise causal linear-attention forward (gfx950).
//
// Method (tensorplay "Talk Linear Attention", section 3.2, chunkwise parallel
// form; section 5.2 for the decayed variant): for chunk c of C tokens with
// chunk-local cumulative log-gate G_r and a_r = exp(G_r),
//   O_c    = diag(a) Q_c S_prev  +  (Gamma (.) Q_c K_c^T (.) M) V_c
//   S_next = a_C S_prev + K_c^T diag(a_C / a) V_c,   Gamma_rs = exp(G_r - G_s)
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
//   1. Q, K and V arrive as whole 16-byte row segments (every wave load covers
//      complete rows), are converted to the operand type and written row-major
//      into XOR-swizzled LDS tiles; V is also written scaled by exp(g_C - G_s)
//      for the state update. Operands that need the token index in the K slots
//      (K^T and V^T) are read from the row-major tiles with the gfx950
//      transpose load. The loads of chunk c+1 are issued right after chunk c is
//      staged, so their latency hides behind chunk c's math. Wave 0 has built
//      the gate tables (G, exp(G), exp(g_C - G), exp(g_C)) one chunk ahead.
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
//   3. S <- exp(g_C) S + K^T (w V) on MFMA into the accumulators; the state
//      tiles are split greedily so waves with fewer score tiles take more.
#pragma once

#include <type_traits>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

template <typename T> __device__ inline float frag_elem(const typename Mfma<T>::frag &f, int i);
template <> __device__ inline float frag_elem<f16>(const f16x8 &f, int i) { return (float)f[i]; }
template <> __device__ inline float frag_elem<float>(const float &f, int) { return f; }

// ---------------------------------------------------------------------------
// Row-major LDS tiles [rows][W] of the operand type, padded by PAD elements per
// row (fp16; fp32 tiles pad by 4). Padding rather than an XOR swizzle keeps
// every address a per-lane base plus a compile-time offset. The pads are chosen
// for gfx950's LDS (64 banks; 8-byte reads served 32 lanes at a time): with a
// 32-byte pad the transpose loads below (16 consecutive rows x 32 bytes per
// half-wave) are conflict-free, 16-byte staging writes of whole rows are too,
// and 16-byte operand reads of 16 rows see at most 2-way conflicts; the Q tile,
// which only sees operand reads, pads by 16 bytes (conflict-free).
template <typename TM, int W, int PAD> struct RowTile {
    static constexpr int P = sizeof(TM) == 2 ? W + PAD : W + 4;  // row pitch (elements)
    static constexpr int SIZE_ROWS(int rows) { return rows * P; }
    __device__ static constexpr int at(int row, int col) { return row * P + col; }
};

// Operand fragment X[k][col0 + n] for the K-slots {r0 .. r0+3, r0+16 .. r0+19}
// of this lane's group, from a row-major fp16 tile of pitch P, with two
// transpose loads. In a 16-lane group the transpose load hands lane i element e
// of the 8-byte row piece addressed by lane 4e + i/4, column i % 4; so lane j
// addresses row r + (j >> 2), columns col0 + 4 (j & 3).
template <int P>
__device__ inline f16x8 tr_frag(const f16 *X, int r0, int col0, int lane) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const int j = lane & 15;
    const f16 *p0 = X + (r0 + (j >> 2)) * P + col0 + 4 * (j & 3);
    const f16 *p1 = p0 + 16 * P;
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(p0));
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(p1));
    const f16x4 ha = __builtin_bit_cast(f16x4, a), hb = __builtin_bit_cast(f16x4, b);
    return f16x8{ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
}

// ---------------------------------------------------------------------------
// Contiguous ranges of state tiles per wave, filled greedily so that waves with
// fewer score tiles take more state tiles.
template <int NW, int NRB> struct Roles {
    static constexpr int MODE = (NW == NRB) ? 0 : (NW == 2 * NRB) ? 1 : (2 * NW == NRB) ? 2 : -1;
    static_assert(MODE >= 0, "wave count must be C/16, C/8 or C/32");
    static constexpr int RBW = MODE == 2 ? 2 : 1;
    static constexpr int rb(int w, int i) { return MODE == 2 ? (i == 0 ? w : NRB - 1 - w) : (w % NRB); }
    static constexpr int half(int w) { return MODE == 1 ? w / NRB : 0; }
    // relative score work of wave w (16 x 16 score tiles)
    static constexpr int score_tiles(int w) { return MODE == 2 ? NRB + 1 : (w % NRB) + 1; }
};

template <int NTT, int NW> struct TileSplit {
    int start[NW];
    int cnt[NW];
    int maxcnt;
};
template <int NTT, int NW, int NRB>
constexpr TileSplit<NTT, NW> make_tile_split(int extra0) {
    TileSplit<NTT, NW> t{};
    for (int w = 0; w < NW; ++w) t.cnt[w] = 0;
    auto load = [&](int w) { return Roles<NW, NRB>::score_tiles(w) + t.cnt[w] + (w == 0 ? extra0 : 0); };
    for (int i = 0; i < NTT; ++i) {
        int best = 0;
        for (int w = 1; w < NW; ++w)
            if (load(w) < load(best)) best = w;
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
    static constexpr int KP = DK + PAD;  // row pitch of STs (elements)
    using QT = RowTile<TM, DK, 8>;                        // Q: operand reads only
    using KT = RowTile<TM, DK, 16>;                       // K: operand and transpose reads
    using VT = RowTile<TM, DVT, DVT == 16 ? 0 : 16>;      // V, wV: transpose reads
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
    using QT = typename Cfg::QT;          // Q tile
    using KT = typename Cfg::KT;          // K tile
    using VT = typename Cfg::VT;          // V (or U) tiles
    constexpr bool H = sizeof(TM) == 2;
    constexpr int NT = NW * 64;           // threads
    constexpr int E = MF::E;
    constexpr int NRB = C / 16;           // 16-row blocks per chunk
    using R = Roles<NW, NRB>;
    constexpr bool DECAYED = Cfg::DECAYED;
    constexpr int KP = Cfg::KP;
    constexpr int NTI = DK / 16, NTJ = DVT / 16;
    constexpr int NTJW = R::MODE == 1 ? NTJ / 2 : NTJ;  // output column tiles per wave
    constexpr int NKS = DK / (4 * E);     // k-steps over channels
    constexpr int NTK = C / (4 * E);      // k-steps over tokens
    constexpr int PER = C / 64;           // tokens per lane in the gate scan
    constexpr int NQR = DK / 32;          // 8-element runs of one lane's channels (DK/4)
    // Staging: 16-byte row segments; one wave load covers 64/SEG whole rows.
    constexpr int EPS = 16 / (int)sizeof(TI);              // input elements per segment
    constexpr int SEGQ = DK / EPS, SEGV = DVT / EPS;        // segments per row
    constexpr int NIQ = C * SEGQ / 64;                      // wave loads per chunk for Q (and K)
    constexpr int NIV = (VAR == V_GDN) ? 0 : C * SEGV / 64;
    constexpr int NI = 2 * NIQ + NIV;
    constexpr int NSLOT = (NI + NW - 1) / NW;
    static_assert(64 % SEGQ == 0 && (VAR == V_GDN || 64 % SEGV == 0) && C * SEGQ % 64 == 0 &&
                  C * SEGV % 64 == 0, "staging geometry");
    constexpr int ZW = 0;                 // wave that carries the normalizer
    constexpr auto TS = make_tile_split<NTI * NTJ, NW, NRB>(VAR == V_NORM ? NTI : 0);
    constexpr int NTS = TS.maxcnt;        // state tiles per wave (at most)
    static_assert(NTJW >= 1 && (R::MODE != 1 || NTJ % 2 == 0), "value slice too narrow for the roles");
    static_assert(VAR != V_GDN || (R::MODE <= 1 && NRB == 4), "delta rule: one U row block per wave (pair)");

    __shared__ __attribute__((aligned(16))) TM Qs[C * QT::P];
    __shared__ __attribute__((aligned(16))) TM Ks[C * KT::P];
    __shared__ __attribute__((aligned(16))) TM Vs[C * VT::P];
    __shared__ __attribute__((aligned(16))) TM VWs[DECAYED ? C * VT::P : 1];  // V (or U) scaled by w_s
    __shared__ __attribute__((aligned(16))) TM STs[DVT * KP];
    // Gate tables per buffer: [0] G_s, [1] exp(G_s), [2] w_s = exp(g_C - G_s),
    // [3] exp(G_{end of s's 16-block} - G_s); Tsc = exp(g_C).
    __shared__ __attribute__((aligned(16))) float Tg[DECAYED ? 2 * 4 * C : 1];
    __shared__ float Tsc[DECAYED ? 2 : 1];
    __shared__ __attribute__((aligned(16))) float Zs[VAR == V_NORM ? 2 * DK : 1];
    TM *VW = DECAYED ? VWs : Vs;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // Per-head bases; offsets inside a head are 32-bit (L * d < 2^31 is checked
    // by the ABI layer).
    const TI *qg = (const TI *)a.q + (size_t)bh * L * DK;
    const TI *kg = (const TI *)a.k + (size_t)bh * L * DK;
    const TI *vg = (VAR == V_GDN) ? nullptr : (const TI *)a.v + (size_t)bh * L * dv + j0;
    TO *og = (TO *)a.o + (size_t)bh * L * dv + j0;
    const float *lgg = (DECAYED && a.lg) ? a.lg + (size_t)bh * L : nullptr;
    const TM *wg = (VAR == V_GDN) ? (const TM *)a.w + (size_t)bh * a.Lp * DK : nullptr;
    const TM *utg = (VAR == V_GDN) ? (const TM *)a.ut + (size_t)bh * a.Lp * dv + j0 : nullptr;

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
    // Normalizer z in accumulator layout (wave ZW): lane (g, n) of tile ti holds
    // z[ti*16 + 4g + e] (every column n alike).
    f32x4 zacc[VAR == V_NORM ? NTI : 1];
    if constexpr (VAR == V_NORM) {
#pragma unroll
        for (int ti = 0; ti < NTI; ++ti) {
#pragma unroll
            for (int e = 0; e < 4; ++e) zacc[ti][e] = a.z_in ? a.z_in[(size_t)bh * DK + ti * 16 + 4 * g + e] : 0.f;
        }
        for (int i = tid; i < DK; i += NT) Zs[i] = a.z_in ? a.z_in[(size_t)bh * DK + i] : 0.f;
    }
    // Settle the prologue's loads here, so that no load is pending at the loop
    // head and the per-chunk waits can be exact (leaving output stores in flight).
    __builtin_amdgcn_s_waitcnt(0);

    // ---- registers of the next chunk, loaded one chunk ahead so that global
    // latency overlaps the current chunk's math. Wave load i (i < NI) covers
    // rows i*64/SEG .. of Q, K or V; wave w issues loads w, w + NW, ... and waves
    // past the end repeat the last load, so every memory operation of a full
    // chunk is unconditional and the compiler's wait counts stay exact. Only the
    // ragged last chunk clamps rows, which are zeroed when staged.
    uint4 pre[NSLOT];
    float gpre[PER];
    Raw8<TM> wpre[NQR];           // gated delta: W row of this wave's U row block
    f32x4 upre[NTJW];             // gated delta: U~ of this wave's U tiles (transposed layout)
    const float *gsrc = lgg ? lgg : reinterpret_cast<const float *>(qg);

    // Geometry of slot m of this wave: tensor (0 Q, 1 K, 2 V), chunk row, segment.
    auto slot_geom = [&](int m, int &kind, int &row, int &seg) {
        int i = wv + NW * m;
        i = i < NI ? i : NI - 1;
        if (i < NIQ) {
            kind = 0;
            row = i * (64 / SEGQ) + lane / SEGQ;
            seg = lane % SEGQ;
        } else if (i < 2 * NIQ) {
            kind = 1;
            row = (i - NIQ) * (64 / SEGQ) + lane / SEGQ;
            seg = lane % SEGQ;
        } else {
            kind = 2;
            row = (i - 2 * NIQ) * (64 / SEGV) + lane / SEGV;
            seg = lane % SEGV;
        }
    };

    // Loads of chunk c: the log-gates (first, so that the gate tables wait only
    // for them), the Q/K/V segments of slot m, and the delta-rule W row and U~.
    auto load_gates = [&](int c, auto ragged_tag) {
        constexpr bool RAGGED = decltype(ragged_tag)::value;
        const int t0 = c * C;
        if constexpr (DECAYED) {
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int t = t0 + lane * PER + p;
                gpre[p] = gsrc[RAGGED ? min(t, L - 1) : t];
            }
        }
    };
    auto load_slot = [&](int c, int m, auto ragged_tag) {
        constexpr bool RAGGED = decltype(ragged_tag)::value;
        int kind, r, seg;
        slot_geom(m, kind, r, seg);
        const int t = RAGGED ? min(c * C + r, L - 1) : c * C + r;
        const TI *p = kind == 0 ? qg + t * DK : kind == 1 ? kg + t * DK : vg + t * dv;
        pre[m] = *reinterpret_cast<const uint4 *>(p + seg * EPS);
    };
    auto load_wu = [&](int c) {
        if constexpr (VAR == V_GDN) {
            const int srow = c * C + (wv % NRB) * 16 + n;  // W and U~ have Lp rows: always in range
#pragma unroll
            for (int i = 0; i < NQR; ++i) wpre[i] = ld_raw8<TM>(wg + srow * DK + g * (DK / 4) + 8 * i);
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) {
                const int tj = R::half(wv) * NTJW + jt;
                upre[jt] = ld4<TM>(utg + srow * dv + tj * 16 + 4 * g);
            }
        }
    };
    auto load_chunk = [&](int c, auto ragged_tag) {
        load_gates(c, ragged_tag);
#pragma unroll
        for (int m = 0; m < NSLOT; ++m) load_slot(c, m, ragged_tag);
        load_wu(c);
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

    // Token-slot operand of a row-major tile: X[k][col0 + n] for the K-slots of
    // k-step ks over tokens. fp16: lane group g carries tokens 32 ks + 4g + (0..3)
    // and 32 ks + 16 + 4g + (0..3), the same slots as the score tiles 2 ks and
    // 2 ks + 1 hold in accumulator layout; fp32: token 4 ks + g.
    auto tok_frag = [&](const TM *X, auto p_tag, int ks, int col0) -> frag {
        constexpr int P = decltype(p_tag)::value;
        if constexpr (H) {
            return tr_frag<P>(X, 32 * ks + 4 * g, col0, lane);
        } else {
            return X[(4 * ks + g) * P + col0 + n];
        }
    };

    const int nchunks = (L + C - 1) / C;
    const int nfull = L / C;  // chunks with all C rows valid
    const std::true_type ragged_t{};
    const std::false_type full_t{};
    using NextNone = std::integral_constant<int, 0>;
    using NextFull = std::integral_constant<int, 1>;
    using NextTail = std::integral_constant<int, 2>;  // ragged next chunk if L % C != 0
    using PK = std::integral_constant<int, KT::P>;
    using PV = std::integral_constant<int, VT::P>;

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

        // ---- stage this chunk's Q, K, V segments row-major (V also scaled by w_s),
        // refilling each slot with chunk c+1 as soon as it is consumed: the load
        // issue (bounded by the per-CU address rate) then overlaps the staging
        // of the other slots instead of stalling every wave after the barrier.
        auto load_next_slot = [&](int m) {
            if constexpr (NEXT == 1) {
                load_slot(c + 1, m, full_t);
            } else if constexpr (NEXT == 2) {
                if (c + 1 < nchunks) load_slot(c + 1, m, ragged_t);
            }
        };
        if constexpr (NEXT == 1) {
            load_gates(c + 1, full_t);
        } else if constexpr (NEXT == 2) {
            if (c + 1 < nchunks) load_gates(c + 1, ragged_t);
        }
#pragma unroll
        for (int m = 0; m < NSLOT; ++m) {
            if (NW * m + NW <= NI || wv + NW * m < NI) {
                int kind, r, seg;
                slot_geom(m, kind, r, seg);
                const bool valid = !RAGGED || t0 + r < L;
                const uint32_t w4[4] = {pre[m].x, pre[m].y, pre[m].z, pre[m].w};
                if constexpr (H) {
                    f16x8 h;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        h[2 * i] = (f16)(valid ? bf16_lo(w4[i]) : 0.f);
                        h[2 * i + 1] = (f16)(valid ? bf16_hi(w4[i]) : 0.f);
                    }
                    if (kind == 2) {
                        *reinterpret_cast<f16x8 *>(&Vs[VT::at(r, seg * 8)]) = h;
                        if constexpr (DECAYED) {
                            const f16 w = (f16)T[2 * C + r];
                            *reinterpret_cast<f16x8 *>(&VWs[VT::at(r, seg * 8)]) = h * w;
                        }
                    } else if (kind == 1) {
                        *reinterpret_cast<f16x8 *>(&Ks[KT::at(r, seg * 8)]) = h;
                    } else {
                        *reinterpret_cast<f16x8 *>(&Qs[QT::at(r, seg * 8)]) = h;
                    }
                } else {
                    f32x4 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = valid ? __uint_as_float(w4[i]) : 0.f;
                    if (kind == 2) {
                        *reinterpret_cast<f32x4 *>(&Vs[VT::at(r, seg * 4)]) = x;
                        if constexpr (DECAYED)
                            *reinterpret_cast<f32x4 *>(&VWs[VT::at(r, seg * 4)]) = x * T[2 * C + r];
                    } else if (kind == 1) {
                        *reinterpret_cast<f32x4 *>(&Ks[KT::at(r, seg * 4)]) = x;
                    } else {
                        *reinterpret_cast<f32x4 *>(&Qs[QT::at(r, seg * 4)]) = x;
                    }
                }
            }
            load_next_slot(m);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Delta rule: this chunk's W row and U~ as operands; their prefetch
        // registers are then refilled with chunk c+1.
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
            if constexpr (NEXT == 1) {
                load_wu(c + 1);
            } else if constexpr (NEXT == 2) {
                if (c + 1 < nchunks) load_wu(c + 1);
            }
        }
        // Keep the prefetch here: the scheduler would otherwise sink the loads
        // towards their use in the next chunk and expose their latency.
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // staged tiles and STs visible

        // ---- gated delta rule: U = U~ - W S_prev for this wave's 16 rows and
        // column tiles, computed transposed, D[j][s] = sum_i S[i][j] (-W[s][i]),
        // so that lane (g, n) holds U[s = ub*16 + n][j = jj + 4g + e] and writes
        // four consecutive columns of the row-major V tile (and of the w_s-scaled
        // copy for the state update).
        if constexpr (VAR == V_GDN) {
            const int ub = wv % NRB;
            const int s = ub * 16 + n;
            const float ws = T[2 * C + s];
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) {
                const int jj = (R::half(wv) * NTJW + jt) * 16;
                f32x4 acc = ucur[jt];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = MF::mma(ld_frag<TM>(&STs[(jj + n) * KP + g * (DK / 4) + ks * E]), wf[ks], acc);
                st4<TM>(&Vs[VT::at(s, jj + 4 * g)], acc);
                st4<TM>(&VWs[VT::at(s, jj + 4 * g)], acc * ws);
            }
            __syncthreads();
        }

        const int zc = (c & 1) * DK, zn = ((c + 1) & 1) * DK;

        // ---- outputs for one 16-row block and one range of value tiles; both
        // are compile-time constants so every score tile is straight-line code.
        auto row_block = [&](auto rb_tag, auto tj_tag) {
            constexpr int rb = decltype(rb_tag)::value;
            constexpr int tj0 = decltype(tj_tag)::value;
            const int rl = rb * 16 + n;   // chunk-local query row of this lane
            const int rrow = t0 + rl;
            frag qf[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qf[ks] = ld_frag<TM>(&Qs[QT::at(rl, g * (DK / 4) + ks * E)]);
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
                        sc[sb] = MF::mma(ld_frag<TM>(&Ks[KT::at(sb * 16 + n, g * (DK / 4) + ks * E)]),
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

            // intra-chunk term: D[j][r] += sum_s V[s][j] A[r][s]; the V^T operand
            // holds the tokens of the two score tiles 2p, 2p+1 that lane group g
            // carries: s = 32p + 4g + (0..3) and 32p + 16 + 4g + (0..3).
            if constexpr (E == 8) {
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
                            frag aop = tok_frag(Vs, PV{}, p, (tj0 + jt) * 16);
                            if (!hi) {
#pragma unroll
                                for (int e = 0; e < 4; ++e) aop[4 + e] = from_f32<TM>(0.0f);
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
                                oacc[jt] = MF::mma(Vs[VT::at(sb * 16 + 4 * g + e, (tj0 + jt) * 16 + n)],
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
                    st4<TO>(og + rrow * dv + (tj0 + jt) * 16 + 4 * g, oacc[jt]);
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

        // ---- state update: S <- exp(g_C) S + K^T (w (.) V), both operands read
        // from the row-major tiles with the token index in the K slots.
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
                for (int ks = 0; ks < NTK; ++ks)
                    Sacc[m] = MF::mma(tok_frag(Ks, PK{}, ks, ti * 16), tok_frag(VW, PV{}, ks, tj * 16), Sacc[m]);
            }
        }
        // ---- normalizer carry: z_next = z_prev + K^T 1 (fp32 accumulators).
        if constexpr (VAR == V_NORM) {
            if (wv == ZW) {
                frag ones;
                if constexpr (E == 8) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) ones[e] = from_f32<TM>(1.0f);
                } else {
                    ones = 1.0f;
                }
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) {
#pragma unroll
                    for (int ks = 0; ks < NTK; ++ks) zacc[ti] = MF::mma(tok_frag(Ks, PK{}, ks, ti * 16), ones, zacc[ti]);
                    if (n == 0) *reinterpret_cast<f32x4 *>(&Zs[zn + ti * 16 + 4 * g]) = zacc[ti];
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
        if (a.z_out && split == 0 && wv == ZW && n == 0) {
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) a.z_out[(size_t)bh * DK + ti * 16 + 4 * g + e] = zacc[ti][e];
        }
    }
}

template <int VAR, typename TI, typename TO, int DK, int DVT, int C, int NW>
hipError_t launch_chunk(const ChunkArgs &a, hipStream_t st) {
    const int blocks = a.BH * a.nsplit;
    hipLaunchKernelGGL((chunk_fwd_kernel<VAR, TI, TO, DK, DVT, C, NW>), dim3(blocks), dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
