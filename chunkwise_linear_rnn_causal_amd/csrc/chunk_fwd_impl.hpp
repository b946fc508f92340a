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
//      into padded LDS tiles; V is also written scaled by exp(g_C - G_s) for
//      the state update. Operands that need the token index in the K slots
//      (K^T and V^T) are read from the row-major tiles with the gfx950
//      transpose load. When two chunks' tiles fit in LDS they are double
//      buffered: chunk c+1 is staged while chunk c is computed, with the loads
//      one or two chunks ahead in registers and one barrier per chunk;
//      otherwise a single buffer is staged between two barriers. The gate
//      tables (G, exp(G), exp(g_C - G), exp(g_C)) are built ahead of the chunk
//      that uses them.
//   2. 16-row query blocks are assigned to waves by Roles. With C/8 waves and
//      double buffering the roles split: four row waves compute the outputs,
//      four staging waves stage, prefetch and carry the state. A row wave
//      computes the inter term (S^T Q^T on MFMA), the score tiles K_sb Q_rb^T
//      for sb <= rb, masks/decays/rounds them in registers and feeds them
//      straight back as the B operand of the intra term V^T A^T: the D layout
//      of a score tile is exactly the B-operand layout of the next MFMA with
//      the key index in the K slots. Output rows are lane-indexed, so the
//      per-row scales (exp(G_r), 1/den_r) are per-lane scalars and each lane
//      holds four consecutive output columns.
//   3. S <- exp(g_C) S + K^T (w V) on MFMA into the accumulators; the state
//      tiles are split greedily over the waves with the least other work.
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

// ---------------------------------------------------------------------------
// Wave roles. Modes 0 and 2 give every wave output rows, state tiles and
// staging:
//   0: C/16 waves, one 16-row block each;
//   2: C/32 waves, each with a row block and its mirror.
// Mode 3 (SPLIT: C/8 waves, double-buffered tiles) separates the two chains of
// a chunk: waves 0..NRB-1 each compute all value columns of one row block,
// while waves NRB.. stage the tiles, prefetch, update the state and the
// normalizer and build the gate tables, so the state work runs beside the rows
// instead of after them.
template <int NW, int NRB, bool SPLIT = false> struct Roles {
    static constexpr int MODE = SPLIT ? 3 : (NW == NRB) ? 0 : (2 * NW == NRB) ? 2 : -1;
    static_assert(MODE >= 0 && (MODE != 3 || NW == 2 * NRB),
                  "wave count must be C/16 or C/32, or C/8 with double-buffered tiles");
    static constexpr int RBW = MODE == 2 ? 2 : 1;
    static constexpr bool rows(int w) { return MODE != 3 || w < NRB; }    // computes output rows
    static constexpr bool stages(int w) { return MODE != 3 || w >= NRB; } // stages tiles, owns state tiles
    static constexpr int rb(int w, int i) {
        return MODE == 2 ? (i == 0 ? w : NRB - 1 - w) : MODE == 3 ? (w < NRB ? w : 0) : w;
    }
    // relative score work of wave w (16 x 16 score tiles); mode 3 keeps state
    // tiles off the row waves
    static constexpr int score_tiles(int w) {
        return MODE == 3 ? (w < NRB ? 1 << 20 : 0) : MODE == 2 ? NRB + 1 : rb(w, 0) + 1;
    }
    static constexpr int NWS = MODE == 3 ? NW - NRB : NW;  // staging waves
    static constexpr int WS0 = MODE == 3 ? NRB : 0;        // first staging wave
    static constexpr int ZW = WS0;                         // wave that carries the normalizer
    // owner of the normalizer's 16-channel block ti (mode 3 spreads the blocks
    // over the staging waves), and the number of blocks wave w owns
    static constexpr int zowner(int ti) { return MODE == 3 ? WS0 + ti % NWS : ZW; }
    static constexpr int zunits(int w, int nti) {
        int u = 0;
        for (int ti = 0; ti < nti; ++ti) u += zowner(ti) == w;
        return u;
    }
    static constexpr int GW = MODE == 3 ? NW - 1 : 0;      // wave that builds the gate tables
};

// Contiguous ranges of state tiles per wave, filled greedily so that waves with
// less other work take more state tiles.

template <int NTT, int NW> struct TileSplit {
    int start[NW];
    int cnt[NW];
    int maxcnt;
};
// extraz: normalizer channel blocks (each weighs one state tile); gates: the
// gate-table wave's extra work in state tiles (split roles only).
template <int NTT, int NW, int NRB, bool SPLIT>
constexpr TileSplit<NTT, NW> make_tile_split(int extraz, int gates) {
    using R = Roles<NW, NRB, SPLIT>;
    TileSplit<NTT, NW> t{};
    for (int w = 0; w < NW; ++w) t.cnt[w] = 0;
    auto load = [&](int w) {
        return R::score_tiles(w) + t.cnt[w] + R::zunits(w, extraz) + (R::MODE == 3 && w == R::GW ? gates : 0);
    };
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

// Compile-time helpers: iterate an integer range, and the staging geometry.
template <typename F, int... I>
__device__ __attribute__((always_inline)) inline void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __attribute__((always_inline)) inline void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Staging of one chunk: Q, K (and V) arrive as 16-byte row segments; wave load
// i covers 64/SEG whole rows of one tensor. Wave w issues loads w, w + NW, ...;
// waves past the end repeat the last load (so every wave issues the same
// memory operations and the wait counts stay exact) without staging it.
template <typename TI, int DK, int DVT, int C, int NW, bool HAS_V, bool HAS_Q = true>
struct StageGeo {
    static constexpr int EPS = 16 / (int)sizeof(TI);   // input elements per segment
    static constexpr int SEGQ = DK / EPS, SEGV = DVT / EPS;
    static constexpr int NIQ = C * SEGQ / 64;           // wave loads per chunk for Q (and for K)
    static constexpr int NIV = HAS_V ? C * SEGV / 64 : 0;
    static constexpr int NQK = HAS_Q ? 2 : 1;           // staged tensors of width DK
    static constexpr int NI = NQK * NIQ + NIV;
    // first wave load of tensor kind (0 Q, 1 K, 2 V)
    static constexpr int base(int kind) { return kind == 2 ? NQK * NIQ : (kind == 1 && HAS_Q ? NIQ : 0); }
    static constexpr int NSLOT = (NI + NW - 1) / NW;
    static_assert(64 % SEGQ == 0 && (!HAS_V || 64 % SEGV == 0) && NIQ * 64 == C * SEGQ &&
                  NIV * 64 == (HAS_V ? C * SEGV : 0), "staging geometry");
    struct Slot {
        bool real;  // staged (false: a repeated load only)
        int kind;   // 0 Q, 1 K, 2 V
        int ii;     // wave load index within the tensor
        int seg;    // segments per row
        int rpi;    // rows per wave load
    };
    static constexpr Slot slot(int w, int m) {
        int i = w + NW * m;
        const bool real = i < NI;
        if (!real) i = NI - 1;
        const int kind = HAS_Q ? (i < NIQ ? 0 : (i < 2 * NIQ ? 1 : 2)) : (i < NIQ ? 1 : 2);
        const int ii = i - base(kind);
        const int seg = kind == 2 ? SEGV : SEGQ;
        return Slot{real, kind, ii, seg, 64 / seg};
    }
};

template <int VAR, typename TM, int DK, int DVT, int C, bool QD = false>
struct ChunkCfg {
    static constexpr bool DECAYED = (VAR == V_DECAY || VAR == V_GDN);
    static constexpr int PAD = 16 / (int)sizeof(TM);
    static constexpr int KP = DK + PAD;  // row pitch of STs (elements)
    using QT = RowTile<TM, DK, 8>;                        // Q: operand reads only
    using KT = RowTile<TM, DK, 16>;                       // K: operand and transpose reads
    using VT = RowTile<TM, DVT, DVT == 16 ? 0 : 16>;      // V, wV: transpose reads
    // one set of tiles (Q unless QD, K, V, wV, S_prev^T), in elements
    static constexpr int OQ = 0;
    static constexpr int OK = OQ + (QD ? 0 : C * QT::P);  // QD: Q is not staged
    static constexpr int OV = OK + C * KT::P;
    static constexpr int OVW = OV + C * VT::P;
    static constexpr int OS = OVW + (DECAYED ? C * VT::P : 0);
    static constexpr int SET = OS + DVT * KP;
    // Double buffering: chunk c+1 is staged into a second set of tiles while
    // chunk c is computed, with one barrier per chunk; used when both sets fit
    // in LDS (otherwise chunk c is staged between two barriers).
    static constexpr bool DB = 2 * SET * sizeof(TM) + 4096 <= 160 * 1024;
    static constexpr int NB = DB ? 2 : 1;   // tile sets
    static constexpr int NTB = DB ? 3 : 2;  // gate-table buffers (chunk c uses buffer c % NTB)
};

// TI: input storage type (bf16 or fp32); TO: output type (fp32 or bf16); the
// tensor-core operand type TM is fp16 for bf16 inputs and fp32 for fp32 inputs.
// NW: waves per workgroup; DVT: value columns per workgroup.
template <int VAR, typename TI, typename TO, int DK, int DVT, int C, int NW>
__global__ void __launch_bounds__(NW * 64) chunk_fwd_kernel(ChunkArgs a) {
    using TM = typename OpOf<TI>::type;
    using MF = Mfma<TM>;
    using frag = typename MF::frag;
    // C/8 waves with double-buffered tiles split the roles (mode 3). When the
    // staging waves would otherwise carry many loads per chunk, the row waves
    // load Q straight into operand registers (QD): each row block's queries are
    // read by one wave only, so Q need not pass through LDS. (The delta rule's
    // row waves also form U and stay on the staged path.)
    constexpr bool SPLIT = NW == 2 * (C / 16) && ChunkCfg<VAR, TM, DK, DVT, C, true>::DB;
    constexpr bool QD = SPLIT && sizeof(TM) == 2 && VAR != V_GDN &&
                        StageGeo<TI, DK, DVT, C, (NW > C / 16 ? NW - C / 16 : 1), true>::NSLOT > 6;
    using Cfg = ChunkCfg<VAR, TM, DK, DVT, C, QD>;
    using QT = typename Cfg::QT;
    using KT = typename Cfg::KT;
    using VT = typename Cfg::VT;
    constexpr bool H = sizeof(TM) == 2;
    constexpr int NT = NW * 64;           // threads
    constexpr int E = MF::E;
    constexpr int NRB = C / 16;           // 16-row blocks per chunk
    using R = Roles<NW, NRB, SPLIT>;
    using Geo = StageGeo<TI, DK, DVT, C, R::NWS, VAR != V_GDN, !QD>;
    constexpr bool DECAYED = Cfg::DECAYED;
    constexpr bool DB = Cfg::DB;
    constexpr int NTB = Cfg::NTB;
    constexpr int KP = Cfg::KP;
    constexpr int NTI = DK / 16, NTJ = DVT / 16;
    constexpr int NTJW = NTJ;             // output column tiles per row wave
    constexpr int NKS = DK / (4 * E);     // k-steps over channels
    constexpr int NTK = C / (4 * E);      // k-steps over tokens
    constexpr int PER = C / 64;           // tokens per lane in the gate scan
    constexpr int NQR = DK / 32;          // 8-element runs of one lane's channels (DK/4)
    constexpr int EPS = Geo::EPS;
    constexpr int NSLOT = Geo::NSLOT;
    constexpr int GW = R::GW;             // wave that builds the gate tables
    constexpr int WS0 = R::WS0, NWS = R::NWS;
    // the gate tables weigh about six state tiles (measured per role with cycle counters)
    constexpr auto TS = make_tile_split<NTI * NTJ, NW, NRB, R::MODE == 3>(VAR == V_NORM ? NTI : 0, DECAYED ? 6 : 0);
    constexpr int NTS = TS.maxcnt;        // state tiles per wave (at most)
    static_assert(NTJW >= 1, "value slice narrower than one tile");
    static_assert(VAR != V_GDN || ((R::MODE == 0 || R::MODE == 3) && NRB == 4),
                  "delta rule: one U row block per wave");

    // Tile sets: [set][Q | K | V | wV | S_prev^T]. Gate tables per buffer:
    // [0] G_s, [1] exp(G_s), [2] w_s = exp(g_C - G_s), [3] exp(G_{end of s's
    // 16-block} - G_s); Tsc = exp(g_C).
    __shared__ __attribute__((aligned(16))) TM Tiles[Cfg::NB * Cfg::SET];
    __shared__ __attribute__((aligned(16))) float Tg[DECAYED ? NTB * 4 * C : 1];
    __shared__ float Tsc[DECAYED ? NTB : 1];
    // Normalizer z of the previous chunk in fp32, double-buffered. q . z is taken
    // on the VALU in fp32: z is a running sum that grows with the sequence and
    // would leave the fp16 operand range.
    __shared__ __attribute__((aligned(16))) float Zs[VAR == V_NORM ? 2 * DK : 1];
    // fp16 operands: the carried state S_prev^T (and the delta rule's U) enter
    // the MFMAs scaled by 2^-s, with s chosen per chunk from the largest |S| of
    // the previous chunk's state (carry_shift), and the products are scaled back
    // in fp32. Slot j % 3 holds each state-holding wave's max |S_j| (the state
    // before chunk j); slots rotate over three chunks, so every slot is read
    // only between barriers that order it after its writes and before its reuse.
    constexpr bool SCALE = H;
    __shared__ __attribute__((aligned(16))) float Smx[SCALE ? 3 * NW : 1];
    // OSTG (split roles, fp32 output, 32-column slices): each row wave passes
    // its 16-row output block through a private LDS tile, so that every store
    // instruction writes whole 128-byte lines (8 lanes x 16 bytes per row)
    // instead of 16 half lines. With 64-column slices the row waves are the
    // longer chain and the extra LDS round trip cost more than it saved; with
    // 16 columns a row is only 64 bytes.
    constexpr bool OSTG = R::MODE == 3 && sizeof(TO) == 4 && DVT == 32;
    constexpr int OP = DVT + 4;  // row pitch of the output tile (floats)
    __shared__ __attribute__((aligned(16))) float Ost[OSTG ? NRB * 16 * OP : 1];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int vid = xcd_virtual_block();
    const int bh = vid / a.nsplit, split = vid - bh * a.nsplit;
    const int j0 = split * DVT;
    const int L = a.L, dv = a.dv;

    // Per-head bases; offsets inside a head are 32-bit (the ABI layer refuses
    // ceil(L / C) * C * max(d_k, d_v) >= 2^31).
    const TI *qg = (const TI *)a.q + (size_t)bh * a.ld * DK;
    const TI *kg = (const TI *)a.k + (size_t)bh * a.ld * DK;
    const TI *vg = (VAR == V_GDN) ? nullptr : (const TI *)a.v + (size_t)bh * a.ld * dv + j0;
    TO *og = (TO *)a.o + (size_t)bh * a.ld * dv + j0;
    const float *lgg = (DECAYED && a.lg) ? a.lg + (size_t)bh * a.ld : nullptr;
    const TM *wg = (VAR == V_GDN) ? (const TM *)a.w + (size_t)bh * a.Lp * DK : nullptr;
    const TM *utg = (VAR == V_GDN) ? (const TM *)a.ut + (size_t)bh * a.Lp * dv + j0 : nullptr;

    // ---- this wave's state tiles (a contiguous range of tile ids ti*NTJ + tj),
    // in accumulator layout: lane (g, n) of tile (ti, tj) holds
    // S[ti*16 + 4g + e][j0 + tj*16 + n].
    int ts0 = 0, tsn = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (wv == w) {
            ts0 = TS.start[w];
            tsn = TS.cnt[w];
        }
    }
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
    // Normalizer z in accumulator layout (block ti in wave R::zowner(ti)): lane (g, n) of tile ti holds
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

    // ---- registers of the next chunk(s): loads are issued one chunk ahead of
    // the staging that consumes them, so global latency overlaps the math.
    // Register sets of prefetched chunks. Double-buffered kernels with few
    // loads per wave keep two: the loads of chunk c+3 are issued while chunk c
    // is computed, two chunks ahead of their staging (short chunks need the
    // deeper window to cover the memory latency). Otherwise one: chunk c+2.
    constexpr int NPS = (DB && NSLOT <= 6) ? 2 : 1;
    constexpr int AHEAD = NPS + 1;  // chunks between a load and the chunk being computed
    uint4 pre[NPS][NSLOT];
    float gpre[NPS][PER];
    Raw8<TM> wpre[NQR];           // gated delta: W row of this wave's U row block
    f32x4 upre[NTJW];             // gated delta: U~ of this wave's U tiles (transposed layout)
    const float *gsrc = lgg ? lgg : reinterpret_cast<const float *>(qg);
    // per-lane byte offsets of a slot's segment within its row block (the row
    // block's start is uniform, so full-chunk loads use a scalar base)
    const uint32_t off_qk = ((lane / Geo::SEGQ) * DK + (lane % Geo::SEGQ) * EPS) * (uint32_t)sizeof(TI);
    const uint32_t off_v = ((lane / Geo::SEGV) * dv + (lane % Geo::SEGV) * EPS) * (uint32_t)sizeof(TI);
    // QD (row waves): lane (g, n) holds q[rb*16 + n][g*DK/4 + 8ks + (0..7)] for
    // k-step ks, as raw input two chunks ahead and as operands of this chunk.
    uint4 qraw[QD ? 2 : 1][QD ? NKS : 1];
    frag qcur[QD ? NKS : 1];

    const int nchunks = (L + C - 1) / C;
    const int nfull = L / C;  // chunks with all C rows valid
    using PK = std::integral_constant<int, KT::P>;
    using PV = std::integral_constant<int, VT::P>;

    // Loads of chunk c: the log-gates, slot M of wave W, and the delta-rule W row
    // and U~. FULL: all rows of chunk c are valid (scalar base + lane offset);
    // otherwise rows are clamped to L - 1 and zeroed when staged.
    auto load_gates = [&](int c, auto full_tag, auto set_tag) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_tag)::value;
        constexpr int PS = decltype(set_tag)::value;
        if constexpr (DECAYED) {
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int t = c * C + lane * PER + p;
                gpre[PS][p] = gsrc[FULL ? t : min(t, L - 1)];
            }
        }
    };
    auto load_slot = [&](auto w_tag, auto m_tag, int c, auto full_tag, auto set_tag) __attribute__((always_inline)) {
        constexpr int W = decltype(w_tag)::value;
        constexpr int PS = decltype(set_tag)::value;
        if constexpr (R::stages(W)) {
        constexpr auto S = Geo::slot(W - WS0, decltype(m_tag)::value);
        constexpr int M = decltype(m_tag)::value;
        constexpr bool FULL = decltype(full_tag)::value;
        const TI *tb = S.kind == 0 ? qg : (S.kind == 1 ? kg : vg);
        const int pitch = S.kind == 2 ? dv : DK;
        if constexpr (FULL) {
            const char *base = reinterpret_cast<const char *>(tb + (size_t)(c * C + S.ii * S.rpi) * pitch);
            pre[PS][M] = *reinterpret_cast<const uint4 *>(base + (S.kind == 2 ? off_v : off_qk));
        } else {
            const int t = min(c * C + S.ii * S.rpi + lane / S.seg, L - 1);
            pre[PS][M] = *reinterpret_cast<const uint4 *>(tb + t * pitch + (lane % S.seg) * EPS);
        }
        }
    };
    auto load_wu = [&](int c) __attribute__((always_inline)) {
        if constexpr (VAR == V_GDN) {
            if (!R::rows(wv)) return;
            const int srow = c * C + (wv % NRB) * 16 + n;  // W and U~ have Lp rows: always in range
#pragma unroll
            for (int i = 0; i < NQR; ++i) wpre[i] = ld_raw8<TM>(wg + srow * DK + g * (DK / 4) + 8 * i);
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) {
                const int tj = jt;
                upre[jt] = ld4<TM>(utg + srow * dv + tj * 16 + 4 * g);
            }
        }
    };

    // QD: queries of chunk c for this row wave's block into raw set QS; rows
    // past L read row L - 1 (they only feed outputs that are not stored).
    auto load_q = [&](int c, auto set_tag) __attribute__((always_inline)) {
        if constexpr (QD) {
            constexpr int QS = decltype(set_tag)::value;
            const int t = min(c * C + R::rb(wv, 0) * 16 + n, L - 1);
            const TI *p = qg + t * DK + g * (DK / 4);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qraw[QS][ks] = *reinterpret_cast<const uint4 *>(p + ks * EPS);
        }
    };
    auto cvt_q = [&](auto set_tag) __attribute__((always_inline)) {
        if constexpr (QD) {
            constexpr int QS = decltype(set_tag)::value;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const uint32_t w4[4] = {qraw[QS][ks].x, qraw[QS][ks].y, qraw[QS][ks].z, qraw[QS][ks].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qcur[ks][2 * i] = (f16)bf16_lo(w4[i]);
                    qcur[ks][2 * i + 1] = (f16)bf16_hi(w4[i]);
                }
            }
        }
    };

    // Gate tables of chunk c into buffer buf, from the prefetched log-gates.
    // Called by the gate-table wave GW only (wave-uniform), ahead of the chunk's staging.
    auto gate_tables = [&](int c, int buf, auto set_tag) __attribute__((always_inline)) {
        constexpr int PS = decltype(set_tag)::value;
        const int t0 = c * C;
        float *T = Tg + buf * 4 * C;
        if constexpr (PER == 1) {
            const float x = (lgg && t0 + lane < L) ? gpre[PS][0] : 0.f;
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
                run += (lgg && t0 + lane * PER + p < L) ? gpre[PS][p] : 0.f;
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
    auto tok_frag = [&](const TM *X, auto p_tag, int ks, int col0) __attribute__((always_inline)) -> frag {
        constexpr int P = decltype(p_tag)::value;
        if constexpr (H) {
            return tr_frag<P>(X, 32 * ks + 4 * g, col0, lane);
        } else {
            return X[(4 * ks + g) * P + col0 + n];
        }
    };

    // Run fn(W) with W = this wave's index as a compile-time constant.
    auto for_wave = [&](auto &&fn) __attribute__((always_inline)) {
        switch (wv) {
            case 0: fn(std::integral_constant<int, 0>{}); break;
            case 1: fn(std::integral_constant<int, 1 % NW>{}); break;
            case 2: fn(std::integral_constant<int, 2 % NW>{}); break;
            case 3: fn(std::integral_constant<int, 3 % NW>{}); break;
            default:
                if constexpr (NW == 8) {
                    switch (wv) {
                        case 4: fn(std::integral_constant<int, 4>{}); break;
                        case 5: fn(std::integral_constant<int, 5>{}); break;
                        case 6: fn(std::integral_constant<int, 6>{}); break;
                        default: fn(std::integral_constant<int, 7>{}); break;
                    }
                }
                break;
        }
    };

    // ---- per-wave pieces of a chunk; W (the wave) is a compile-time constant, so
    // every tile, slot and row index below folds into address immediates.

    // Stage slot M of chunk cs (in registers) into tile set X: convert to the
    // operand type and write row-major; V also scaled by w_s of chunk cs.
    // CHECK: rows past L are zeroed.
    auto stage_slot = [&](auto w_tag, auto m_tag, int cs, TM *X, auto check_tag, auto set_tag) __attribute__((always_inline)) {
        constexpr int W = decltype(w_tag)::value;
        constexpr int PS = decltype(set_tag)::value;
        constexpr auto S = Geo::slot(R::stages(W) ? W - WS0 : 0, decltype(m_tag)::value);
        constexpr int M = decltype(m_tag)::value;
        constexpr bool CHECK = decltype(check_tag)::value;
        if constexpr (R::stages(W) && S.real) {
            const int r = S.ii * S.rpi + lane / S.seg, seg = lane % S.seg;
            const bool valid = !CHECK || cs * C + r < L;
            const uint32_t w4[4] = {pre[PS][M].x, pre[PS][M].y, pre[PS][M].z, pre[PS][M].w};
            if constexpr (H) {
                f16x8 h;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h[2 * i] = (f16)(valid ? bf16_lo(w4[i]) : 0.f);
                    h[2 * i + 1] = (f16)(valid ? bf16_hi(w4[i]) : 0.f);
                }
                if constexpr (S.kind == 2) {
                    *reinterpret_cast<f16x8 *>(&X[Cfg::OV + VT::at(r, seg * 8)]) = h;
                    if constexpr (DECAYED) {
                        const f16 w = (f16)Tg[(cs % NTB) * 4 * C + 2 * C + r];
                        *reinterpret_cast<f16x8 *>(&X[Cfg::OVW + VT::at(r, seg * 8)]) = h * w;
                    }
                } else if constexpr (S.kind == 1) {
                    *reinterpret_cast<f16x8 *>(&X[Cfg::OK + KT::at(r, seg * 8)]) = h;
                } else {
                    *reinterpret_cast<f16x8 *>(&X[Cfg::OQ + QT::at(r, seg * 8)]) = h;
                }
            } else {
                f32x4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = valid ? __uint_as_float(w4[i]) : 0.f;
                if constexpr (S.kind == 2) {
                    *reinterpret_cast<f32x4 *>(&X[Cfg::OV + VT::at(r, seg * 4)]) = x;
                    if constexpr (DECAYED)
                        *reinterpret_cast<f32x4 *>(&X[Cfg::OVW + VT::at(r, seg * 4)]) =
                            x * Tg[(cs % NTB) * 4 * C + 2 * C + r];
                } else if constexpr (S.kind == 1) {
                    *reinterpret_cast<f32x4 *>(&X[Cfg::OK + KT::at(r, seg * 4)]) = x;
                } else {
                    *reinterpret_cast<f32x4 *>(&X[Cfg::OQ + QT::at(r, seg * 4)]) = x;
                }
            }
        }
    };

    // Slot M of this wave in common code (one code path for all waves): the
    // slot's tensor must be the same for every wave; the wave's row offset is
    // then a scalar. Otherwise the per-wave versions above are dispatched.
    auto slot_uniform = [&](auto m_tag) __attribute__((always_inline)) {
        constexpr int M = decltype(m_tag)::value;
        constexpr auto S0 = Geo::slot(0, M);
        constexpr auto S1 = Geo::slot(NWS - 1, M);
        return std::bool_constant<S0.kind == S1.kind>{};
    };
    auto stage_any = [&](auto m_tag, int cs, TM *X, auto check_tag, auto set_tag) __attribute__((always_inline)) {
        constexpr int M = decltype(m_tag)::value;
        constexpr int PS = decltype(set_tag)::value;
        constexpr bool CHECK = decltype(check_tag)::value;
        if constexpr (decltype(slot_uniform(m_tag))::value) {
            constexpr auto S = Geo::slot(0, M);
            const int i = (wv - WS0) + NWS * M;
            if (wv >= WS0 && i < Geo::NI) {
                const int ii = i - Geo::base(S.kind);
                const int r = ii * S.rpi + lane / S.seg, seg = lane % S.seg;
                const bool valid = !CHECK || cs * C + r < L;
                const uint32_t w4[4] = {pre[PS][M].x, pre[PS][M].y, pre[PS][M].z, pre[PS][M].w};
                if constexpr (H) {
                    f16x8 h;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        h[2 * q] = (f16)(valid ? bf16_lo(w4[q]) : 0.f);
                        h[2 * q + 1] = (f16)(valid ? bf16_hi(w4[q]) : 0.f);
                    }
                    if constexpr (S.kind == 2) {
                        *reinterpret_cast<f16x8 *>(&X[Cfg::OV + VT::at(r, seg * 8)]) = h;
                        if constexpr (DECAYED) {
                            const f16 w = (f16)Tg[(cs % NTB) * 4 * C + 2 * C + r];
                            *reinterpret_cast<f16x8 *>(&X[Cfg::OVW + VT::at(r, seg * 8)]) = h * w;
                        }
                    } else if constexpr (S.kind == 1) {
                        *reinterpret_cast<f16x8 *>(&X[Cfg::OK + KT::at(r, seg * 8)]) = h;
                    } else {
                        *reinterpret_cast<f16x8 *>(&X[Cfg::OQ + QT::at(r, seg * 8)]) = h;
                    }
                } else {
                    f32x4 x;
#pragma unroll
                    for (int q = 0; q < 4; ++q) x[q] = valid ? __uint_as_float(w4[q]) : 0.f;
                    if constexpr (S.kind == 2) {
                        *reinterpret_cast<f32x4 *>(&X[Cfg::OV + VT::at(r, seg * 4)]) = x;
                        if constexpr (DECAYED)
                            *reinterpret_cast<f32x4 *>(&X[Cfg::OVW + VT::at(r, seg * 4)]) =
                                x * Tg[(cs % NTB) * 4 * C + 2 * C + r];
                    } else if constexpr (S.kind == 1) {
                        *reinterpret_cast<f32x4 *>(&X[Cfg::OK + KT::at(r, seg * 4)]) = x;
                    } else {
                        *reinterpret_cast<f32x4 *>(&X[Cfg::OQ + QT::at(r, seg * 4)]) = x;
                    }
                }
            }
        } else {
            for_wave([&](auto w_tag) __attribute__((always_inline)) { stage_slot(w_tag, m_tag, cs, X, check_tag, set_tag); });
        }
    };
    auto load_any = [&](auto m_tag, int c, auto full_tag, auto set_tag) __attribute__((always_inline)) {
        constexpr int M = decltype(m_tag)::value;
        constexpr int PS = decltype(set_tag)::value;
        constexpr bool FULL = decltype(full_tag)::value;
        if constexpr (decltype(slot_uniform(m_tag))::value) {
            if (wv < WS0) return;
            constexpr auto S = Geo::slot(0, M);
            int i = (wv - WS0) + NWS * M;
            i = i < Geo::NI ? i : Geo::NI - 1;  // repeat the last load past the end
            const int ii = i - Geo::base(S.kind);
            const TI *tb = S.kind == 0 ? qg : (S.kind == 1 ? kg : vg);
            const int pitch = S.kind == 2 ? dv : DK;
            if constexpr (FULL) {
                const char *base = reinterpret_cast<const char *>(tb + (size_t)(c * C + ii * S.rpi) * pitch);
                pre[PS][M] = *reinterpret_cast<const uint4 *>(base + (S.kind == 2 ? off_v : off_qk));
            } else {
                const int t = min(c * C + ii * S.rpi + lane / S.seg, L - 1);
                pre[PS][M] = *reinterpret_cast<const uint4 *>(tb + t * pitch + (lane % S.seg) * EPS);
            }
        } else {
            for_wave([&](auto w_tag) __attribute__((always_inline)) { load_slot(w_tag, m_tag, c, full_tag, set_tag); });
        }
    };

    // S_prev, transposed, in the operand type and scaled by 2^-sh:
    // X[OS + j*KP + i].
    auto write_sts = [&](auto w_tag, TM *X, int sh) __attribute__((always_inline)) {
        constexpr int W = decltype(w_tag)::value;
        auto put = [&](auto scaled) __attribute__((always_inline)) {
            const float sc = decltype(scaled)::value ? pow2i(-sh) : 1.f;
#pragma unroll
            for (int m = 0; m < TS.cnt[W]; ++m) {
                const int tile = TS.start[W] + m, ti = tile / NTJ, tj = tile % NTJ;
                st4<TM>(&X[Cfg::OS + (tj * 16 + n) * KP + ti * 16 + 4 * g],
                        decltype(scaled)::value ? Sacc[m] * sc : Sacc[m]);
            }
        };
        // the shift is wave-uniform and usually zero: skip the multiplies then
        if (SCALE && sh != 0) put(std::true_type{});
        else put(std::false_type{});
    };
    // max |S| over wave W's state tiles (the state before chunk j) into slot j % 3.
    auto put_smax = [&](auto w_tag, int j) __attribute__((always_inline)) {
        constexpr int W = decltype(w_tag)::value;
        if constexpr (SCALE && TS.cnt[W] > 0) {
            float m = 0.f;
#pragma unroll
            for (int t = 0; t < TS.cnt[W]; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(Sacc[t][e]));
            m = wave_max_nonneg(m);
            if (lane == 0) Smx[(j % 3) * NW + W] = m;
        }
    };
    // Operand shift for a state whose magnitude is bounded by slot j's max
    // (wave-uniform).
    auto get_shift = [&](int j) __attribute__((always_inline)) -> int {
        if constexpr (SCALE) {
            const float *M = Smx + (j % 3) * NW;
            float m = 0.f;
            static_for<NW>([&](auto w_tag) __attribute__((always_inline)) {
                if constexpr (TS.cnt[decltype(w_tag)::value] > 0) m = fmaxf(m, M[decltype(w_tag)::value]);
            });
            return __builtin_amdgcn_readfirstlane(carry_shift(m));
        } else {
            return 0;
        }
    };

    // Delta rule: this chunk's W row and U~ as operands, from the prefetch
    // registers (which are then free for the next chunk).
    auto take_wu = [&](frag (&wf)[VAR == V_GDN ? NKS : 1],
                       f32x4 (&ucur)[VAR == V_GDN ? NTJW : 1]) __attribute__((always_inline)) {
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
    };

    // Gated delta rule: U = U~ - W S_prev for this wave's 16 rows and column
    // tiles, computed transposed, D[j][s] = sum_i S[i][j] (-W[s][i]), so that lane
    // (g, n) holds U[s = ub*16 + n][j = jj + 4g + e] and writes four consecutive
    // columns of the row-major V tile (and of the w_s-scaled copy).
    // U is formed in the scale of S_prev^T (2^-sh): U 2^-sh = U~ 2^-sh - W (S_prev 2^-sh).
    auto gdn_u = [&](TM *X, const float *T, const frag (&wf)[VAR == V_GDN ? NKS : 1],
                     const f32x4 (&ucur)[VAR == V_GDN ? NTJW : 1], int sh) __attribute__((always_inline)) {
        if constexpr (VAR == V_GDN) {
            if (!R::rows(wv)) return;
            const int ub = wv % NRB;
            const int s = ub * 16 + n;
            const float ws = T[2 * C + s];
            const float sc = SCALE ? pow2i(-sh) : 1.f;
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) {
                const int jj = jt * 16;
                f32x4 acc = SCALE ? ucur[jt] * sc : ucur[jt];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = MF::mma(ld_frag<TM>(&X[Cfg::OS + (jj + n) * KP + g * (DK / 4) + ks * E]), wf[ks], acc);
                st4<TM>(&X[Cfg::OV + VT::at(s, jj + 4 * g)], acc);
                st4<TM>(&X[Cfg::OVW + VT::at(s, jj + 4 * g)], acc * ws);
            }
        }
    };

    // Outputs of one 16-row block rb and one range of value tiles (from tj0) of
    // chunk c, from tile set X. CHECK: rows past L are not stored.
    // Every LDS operand of the block is read before the math when the fragments
    // fit in registers (HOIST), so the reads overlap instead of each waiting.
    // sh: shift of the S_prev^T operand (and of U for the delta rule).
    auto row_block = [&](auto rb_tag, auto tj_tag, int c, const TM *X, const float *T,
                         auto check_tag, int sh) __attribute__((always_inline)) {
        constexpr int rb = decltype(rb_tag)::value;
        constexpr int tj0 = decltype(tj_tag)::value;
        constexpr bool CHECK = decltype(check_tag)::value;
        constexpr int FR = (int)sizeof(frag) / 4;  // VGPRs per fragment
        constexpr bool HOIST = H && FR * (NKS * (1 + NTJW + rb + 1) + NTJW * (rb / 2 + 1)) <= 80;
        constexpr bool NZ = H && VAR == V_NORM;   // rowsums of the rounded scores on MFMA (fp16 path)
        const TM *Qs = X + Cfg::OQ, *Ks = X + Cfg::OK, *Vs = X + Cfg::OV, *STs = X + Cfg::OS;
        const int t0 = c * C;
        const int rl = rb * 16 + n;   // chunk-local query row of this lane

        // ---- operands
        frag qf[NKS], sf[NTJW][NKS], kf[rb + 1][NKS], vf[rb / 2 + 1][NTJW];
        auto load_k = [&](int sb) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) kf[sb][ks] = ld_frag<TM>(&Ks[KT::at(sb * 16 + n, g * (DK / 4) + ks * E)]);
        };
        auto load_v = [&](int p) __attribute__((always_inline)) {
            if constexpr (E == 8) {
#pragma unroll
                for (int jt = 0; jt < NTJW; ++jt) vf[p][jt] = tok_frag(Vs, PV{}, p, (tj0 + jt) * 16);
            }
        };
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (QD) {
                qf[ks] = qcur[ks];
            } else {
                qf[ks] = ld_frag<TM>(&Qs[QT::at(rl, g * (DK / 4) + ks * E)]);
            }
        }
#pragma unroll
        for (int jt = 0; jt < NTJW; ++jt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                sf[jt][ks] = ld_frag<TM>(&STs[((tj0 + jt) * 16 + n) * KP + g * (DK / 4) + ks * E]);
        if constexpr (HOIST) {
#pragma unroll
            for (int sb = 0; sb <= rb; ++sb) load_k(sb);
#pragma unroll
            for (int p = 0; p <= rb / 2; ++p) load_v(p);
            __builtin_amdgcn_sched_barrier(0);
        }
        const float Gr = DECAYED ? T[rl] : 0.f;

        // inter-chunk term: D[j][r] = exp(G_r) sum_i S[i][j] q_r[i]
        f32x4 oacc[NTJW];
#pragma unroll
        for (int jt = 0; jt < NTJW; ++jt) {
            oacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) oacc[jt] = MF::mma(sf[jt][ks], qf[ks], oacc[jt]);
        }
        // undo the operand scale of S_prev^T (the delta rule's U carries the same
        // scale, so there the whole output is scaled back at the end)
        const float us = (SCALE && VAR != V_GDN) ? pow2i(sh) : 1.f;
        if constexpr (DECAYED) {
            const float er = T[C + rl] * us;
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) oacc[jt] *= er;
        } else if constexpr (SCALE) {
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) oacc[jt] *= us;
        }
        // normalizer, fp16 path: the rowsums of the rounded scores, accumulated
        // below in a tile whose rows are all alike (every lane gets its row's value).
        f32x4 dacc = {0.f, 0.f, 0.f, 0.f};

        // score tiles D[s][r] = k_s . q_r for key blocks sb <= rb. Off the
        // diagonal, exp(G_r - G_s) = exp(G_r - G_e) exp(G_e - G_s) with e the
        // last token of block sb: both factors <= 1, so no overflow for any
        // gates, and one exp per tile.
        f32x4 sc[NRB];
        float rowsum = 0.f;  // fp32 path only
#pragma unroll
        for (int sb = 0; sb < NRB; ++sb) {
            sc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (sb <= rb) {
                if constexpr (!HOIST) load_k(sb);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) sc[sb] = MF::mma(kf[sb][ks], qf[ks], sc[sb]);
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
                if constexpr (VAR == V_NORM && !NZ) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) rowsum += sc[sb][e];
                }
            }
        }

        // intra-chunk term: D[j][r] += sum_s V[s][j] A[r][s]; the V^T operand
        // holds the tokens of the two score tiles 2p, 2p+1 that lane group g
        // carries: s = 32p + 4g + (0..3) and 32p + 16 + 4g + (0..3).
        if constexpr (E == 8) {
            frag ones;
            if constexpr (NZ) {
#pragma unroll
                for (int e = 0; e < 8; ++e) ones[e] = from_f32<TM>(1.0f);
            }
#pragma unroll
            for (int p = 0; p < NRB / 2; ++p) {
                if (2 * p <= rb) {
                    // normalized: scores as fp16 high + low parts (A = hi + lo to
                    // about 2^-22), because the normalized output is a weighted
                    // average whose weights would otherwise carry fp16's 2^-12
                    // rounding into every output
                    frag bop, blo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bop[e] = from_f32<TM>(sc[2 * p][e]);
                        bop[4 + e] = from_f32<TM>(sc[2 * p + 1][e]);
                        if constexpr (NZ) {
                            blo[e] = from_f32<TM>(sc[2 * p][e] - to_f32<TM>(bop[e]));
                            blo[4 + e] = from_f32<TM>(sc[2 * p + 1][e] - to_f32<TM>(bop[4 + e]));
                        }
                    }
                    if constexpr (!HOIST) load_v(p);
                    const bool hi = (2 * p + 1 <= rb);
#pragma unroll
                    for (int jt = 0; jt < NTJW; ++jt) {
                        frag aop = vf[p][jt];
                        if (!hi) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) aop[4 + e] = from_f32<TM>(0.0f);
                        }
                        oacc[jt] = MF::mma(aop, bop, oacc[jt]);
                        if constexpr (NZ) oacc[jt] = MF::mma(aop, blo, oacc[jt]);
                    }
                    if constexpr (NZ) {  // rowsums of the same split scores
                        dacc = MF::mma(ones, bop, dacc);
                        dacc = MF::mma(ones, blo, dacc);
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
                            oacc[jt] = MF::mma(Vs[VT::at(sb * 16 + 4 * g + e, (tj0 + jt) * 16 + n)], sc[sb][e], oacc[jt]);
                    }
                }
            }
        }

        if constexpr (VAR == V_GDN && SCALE) {
            const float ug = pow2i(sh);
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) oacc[jt] *= ug;
        }
        if constexpr (VAR == V_NORM) {
            // den[r] = q_r . z_prev + rowsum_r: q . z in fp32 over this lane's
            // channels, summed over the four lane groups
            const int zc = (c & 1) * DK;
            float qz = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int el = 0; el < E; ++el)
                    qz += frag_elem<TM>(qf[ks], el) * Zs[zc + g * (DK / 4) + ks * E + el];
            float den = NZ ? qz : rowsum + qz;
            den += __shfl_xor(den, 16, 64);
            den += __shfl_xor(den, 32, 64);
            if constexpr (NZ) den += dacc[0];
            const float inv = 1.0f / den;
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) oacc[jt] *= inv;
            // the denominators, for the backward pass (one value slice writes them)
            if (a.den_out && split == 0 && g == 0 && (!CHECK || t0 + rl < L))
                a.den_out[(size_t)bh * a.ld + t0 + rl] = den;
        }

        // rows of this block start at a uniform offset: scalar base + lane offset
        TO *ob = og + (size_t)(t0 + rb * 16) * dv + tj0 * 16;
        if constexpr (OSTG) {
            // the wave's tile: written in accumulator layout, read back with
            // LPR lanes per row (LDS operations of one wave complete in order)
            float *Ow = Ost + rb * 16 * OP;
#pragma unroll
            for (int jt = 0; jt < NTJW; ++jt) *reinterpret_cast<f32x4 *>(&Ow[n * OP + jt * 16 + 4 * g]) = oacc[jt];
            __builtin_amdgcn_wave_barrier();
            constexpr int LPR = NTJW * 4;     // lanes per output row (16 bytes each)
            constexpr int RPI = 64 / LPR;     // rows per store instruction
#pragma unroll
            for (int h = 0; h < 16 / RPI; ++h) {
                const int r = h * RPI + lane / LPR, cq = lane % LPR;
                const f32x4 v = *reinterpret_cast<const f32x4 *>(&Ow[r * OP + 4 * cq]);
                if (!CHECK || t0 + rb * 16 + r < L) st4<TO>(ob + (uint32_t)(r * dv + 4 * cq), v);
            }
            __builtin_amdgcn_wave_barrier();
        } else {
            if (!CHECK || t0 + rl < L) {
#pragma unroll
                for (int jt = 0; jt < NTJW; ++jt) st4<TO>(ob + (uint32_t)(n * dv + jt * 16 + 4 * g), oacc[jt]);
            }
        }
    };

    // The rows of wave W.
    auto rows_of = [&](auto w_tag, int c, const TM *X, const float *T, auto check_tag, int sh) __attribute__((always_inline)) {
        constexpr int W = decltype(w_tag)::value;
        if constexpr (!R::rows(W)) return;
        row_block(std::integral_constant<int, R::rb(W, 0)>{}, std::integral_constant<int, 0>{}, c,
                  X, T, check_tag, sh);
        if constexpr (R::RBW == 2)
            row_block(std::integral_constant<int, R::rb(W, 1)>{}, std::integral_constant<int, 0>{}, c, X, T,
                      check_tag, sh);
    };

    // State update S <- exp(g_C) S + K^T (w (.) V) of wave W's tiles from tile set
    // X, both operands read from the row-major tiles with the token index in the
    // K slots; then the normalizer carry z_next = z_prev + K^T 1 (each channel
    // block in its owner wave). sh: the delta rule's U tile is held at 2^-sh,
    // so S is brought to that scale for the update and back afterwards.
    auto state_update = [&](auto w_tag, int c, const TM *X, float eg, int sh) __attribute__((always_inline)) {
        constexpr int W = decltype(w_tag)::value;
        constexpr bool USC = SCALE && VAR == V_GDN;
        if constexpr (DECAYED) {
            const float f = USC ? eg * pow2i(-sh) : eg;
#pragma unroll
            for (int m = 0; m < TS.cnt[W]; ++m) Sacc[m] *= f;
        }
        const TM *Ks = X + Cfg::OK;
        const TM *VW = X + (DECAYED ? Cfg::OVW : Cfg::OV);
#pragma unroll
        for (int m = 0; m < TS.cnt[W]; ++m) {
            const int tile = TS.start[W] + m, ti = tile / NTJ, tj = tile % NTJ;
#pragma unroll
            for (int ks = 0; ks < NTK; ++ks)
                Sacc[m] = MF::mma(tok_frag(Ks, PK{}, ks, ti * 16), tok_frag(VW, PV{}, ks, tj * 16), Sacc[m]);
        }
        if constexpr (USC) {
            const float f = pow2i(sh);
#pragma unroll
            for (int m = 0; m < TS.cnt[W]; ++m) Sacc[m] *= f;
        }
        if constexpr (VAR == V_NORM && R::zunits(W, NTI) > 0) {
            const int zn = ((c + 1) & 1) * DK;
            frag ones;
            if constexpr (E == 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) ones[e] = from_f32<TM>(1.0f);
            } else {
                ones = 1.0f;
            }
            static_for<NTI>([&](auto ti_tag) __attribute__((always_inline)) {
                constexpr int ti = decltype(ti_tag)::value;
                if constexpr (R::zowner(ti) == W) {
#pragma unroll
                    for (int ks = 0; ks < NTK; ++ks) zacc[ti] = MF::mma(tok_frag(Ks, PK{}, ks, ti * 16), ones, zacc[ti]);
                    if (n == 0) *reinterpret_cast<f32x4 *>(&Zs[zn + ti * 16 + 4 * g]) = zacc[ti];
                }
            });
        }
    };

    // ---- double-buffered chunk: tile set b = c & 1 holds chunk c; chunk c+1 is
    // staged into set b ^ 1 right after this wave's rows are done (no barrier in
    // between) from its register set, which is then refilled with chunk
    // c+AHEAD (and the log-gates likewise). P = c & 1 at compile time. FAST:
    // chunks c .. c+AHEAD are all full.
    auto chunk_db = [&](int c, auto fast_tag, auto par_tag) __attribute__((always_inline)) {
        constexpr bool FAST = decltype(fast_tag)::value;
        constexpr int P = decltype(par_tag)::value;
        using Cur = std::integral_constant<int, P % NPS>;        // register set of chunk c+2
        using Nxt = std::integral_constant<int, (P ^ 1) % NPS>;  // register set of chunks c+1, c+AHEAD
        using Check = std::bool_constant<!FAST>;
        TM *X = Tiles + P * Cfg::SET, *Xn = Tiles + (P ^ 1) * Cfg::SET;
        const float *T = Tg + (c % NTB) * 4 * C;
        __syncthreads();  // chunk c staged, its gate tables and S_prev visible; chunk c-1 done
        // shifts of S_c^T (bounded by max |S_{c-1}|) and of S_{c+1}^T (by max |S_c|)
        const int sh = get_shift(c > 0 ? c - 1 : 0), shn = get_shift(c);
        if constexpr (FAST) {
            load_gates(c + AHEAD, std::true_type{}, Nxt{});
        } else {
            if (c + AHEAD < nchunks) load_gates(c + AHEAD, std::false_type{}, Nxt{});
        }
        frag wf[VAR == V_GDN ? NKS : 1];
        f32x4 ucur[VAR == V_GDN ? NTJW : 1];
        if constexpr (VAR == V_GDN) {
            take_wu(wf, ucur);
            if (FAST || c + 1 < nchunks) load_wu(c + 1);
        }
        // Keep the prefetch here: the scheduler would otherwise sink the loads
        // towards their use and expose their latency.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (VAR == V_GDN) {
            gdn_u(X, T, wf, ucur, sh);
            __syncthreads();  // U rows of every wave visible
        }
        const bool next = FAST || c + 1 < nchunks;
        const float eg = DECAYED ? Tsc[c % NTB] : 1.f;
        for_wave([&](auto w_tag) __attribute__((always_inline)) { rows_of(w_tag, c, X, T, Check{}, sh); });
        if (next) {
            static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
                stage_any(m_tag, c + 1, Xn, Check{}, Nxt{});
                if constexpr (FAST) {
                    load_any(m_tag, c + AHEAD, std::true_type{}, Nxt{});
                } else {
                    if (c + AHEAD < nchunks) load_any(m_tag, c + AHEAD, std::false_type{}, Nxt{});
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        for_wave([&](auto w_tag) __attribute__((always_inline)) {
            state_update(w_tag, c, X, eg, sh);
            put_smax(w_tag, c + 1);
            if (next) write_sts(w_tag, Xn, shn);
        });
        if constexpr (DECAYED) {
            if (wv == GW && (FAST || c + 2 < nchunks)) gate_tables(c + 2, (c + 2) % NTB, Cur{});
        }
    };

    // ---- single-buffered chunk: chunk c is staged between two barriers and
    // each slot is refilled with chunk c+1. FAST: chunks c and c+1 are full.
    auto chunk_sb = [&](int c, auto fast_tag) __attribute__((always_inline)) {
        constexpr bool FAST = decltype(fast_tag)::value;
        using Check = std::bool_constant<!FAST>;
        TM *X = Tiles;
        const float *T = Tg + (c % NTB) * 4 * C;
        __syncthreads();  // previous chunk done with every tile; gate tables visible
        using S0 = std::integral_constant<int, 0>;
        if constexpr (FAST) {
            load_gates(c + 1, std::true_type{}, S0{});
        } else {
            if (c + 1 < nchunks) load_gates(c + 1, std::false_type{}, S0{});
        }
        const int sh = get_shift(c);  // exact: max |S_c| was written before the barrier
        for_wave([&](auto w_tag) __attribute__((always_inline)) { write_sts(w_tag, X, sh); });
        static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
            stage_any(m_tag, c, X, Check{}, S0{});
            if constexpr (FAST) {
                load_any(m_tag, c + 1, std::true_type{}, S0{});
            } else {
                if (c + 1 < nchunks) load_any(m_tag, c + 1, std::false_type{}, S0{});
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        frag wf[VAR == V_GDN ? NKS : 1];
        f32x4 ucur[VAR == V_GDN ? NTJW : 1];
        if constexpr (VAR == V_GDN) {
            take_wu(wf, ucur);
            if (FAST || c + 1 < nchunks) load_wu(c + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // staged tiles and STs visible
        if constexpr (VAR == V_GDN) {
            gdn_u(X, T, wf, ucur, sh);
            __syncthreads();
        }
        const float eg = DECAYED ? Tsc[c % NTB] : 1.f;
        for_wave([&](auto w_tag) __attribute__((always_inline)) {
            rows_of(w_tag, c, X, T, Check{}, sh);
            state_update(w_tag, c, X, eg, sh);
            put_smax(w_tag, c + 1);
        });
        if constexpr (DECAYED) {
            if (wv == GW && (FAST || c + 1 < nchunks)) gate_tables(c + 1, (c + 1) % NTB, S0{});
        }
    };

    // ---- split roles (mode 3). Each role runs its own straight-line loop over
    // the chunks (one dispatch on the wave index outside the loop), so every
    // wait count stays exact; both roles execute the same barriers: one in the
    // prologue and one per chunk (two for the delta rule).
    // Row wave, chunk c: the outputs of its row block (delta rule: first its
    // U rows, then a barrier).
    auto row_iter = [&](auto w_tag, int c, auto check_tag, auto par_tag) __attribute__((always_inline)) {
        constexpr int P = decltype(par_tag)::value;  // c & 1
        const TM *X = Tiles + P * Cfg::SET;
        const float *T = Tg + (c % NTB) * 4 * C;
        __syncthreads();  // chunk c staged, its gate tables and S_prev visible
        const int sh = get_shift(c > 0 ? c - 1 : 0);  // S_c^T is bounded by max |S_{c-1}|
        if constexpr (QD) {
            cvt_q(par_tag);  // chunk c's queries, loaded two chunks ago
            if (c + 2 < nchunks) load_q(c + 2, par_tag);
        }
        if constexpr (VAR == V_GDN) {
            frag wf[NKS];
            f32x4 ucur[NTJW];
            take_wu(wf, ucur);
            if (c + 1 < nchunks) load_wu(c + 1);
            __builtin_amdgcn_sched_barrier(0);
            gdn_u(const_cast<TM *>(X), T, wf, ucur, sh);
            __syncthreads();  // U rows visible to the state waves
        }
        rows_of(w_tag, c, X, T, check_tag, sh);
    };
    // State wave, chunk c (P = c & 1 at compile time): stage chunk c+1 into the
    // other tile set from its register set and refill that set with chunk
    // c+AHEAD; then S <- update with chunk c, S_next^T into the other set, and
    // the gate tables of chunk c+2 (log-gates of chunk c+AHEAD prefetched).
    // FAST: chunks c .. c+AHEAD are full. The other tile set was last read by the rows of chunk
    // c-1, which the barrier has retired.
    auto state_iter = [&](auto w_tag, int c, auto fast_tag, auto par_tag) __attribute__((always_inline)) {
        constexpr int W = decltype(w_tag)::value;
        constexpr bool FAST = decltype(fast_tag)::value;
        constexpr int P = decltype(par_tag)::value;
        using Cur = std::integral_constant<int, P % NPS>;
        using Nxt = std::integral_constant<int, (P ^ 1) % NPS>;
        using Check = std::bool_constant<!FAST>;
        const TM *X = Tiles + P * Cfg::SET;
        TM *Xn = Tiles + (P ^ 1) * Cfg::SET;
        __syncthreads();  // chunk c staged and visible; chunk c-1 done everywhere
        const int sh = VAR == V_GDN ? get_shift(c > 0 ? c - 1 : 0) : 0;  // U of chunk c
        const int shn = get_shift(c);  // S_{c+1}^T, bounded by max |S_c|
        if constexpr (FAST) {
            load_gates(c + AHEAD, std::true_type{}, Nxt{});
        } else {
            if (c + AHEAD < nchunks) load_gates(c + AHEAD, std::false_type{}, Nxt{});
        }
        const bool next = FAST || c + 1 < nchunks;
        // slots [M0, M1) of chunk c+1
        auto stage_range = [&](auto m0_tag, auto m1_tag) __attribute__((always_inline)) {
            if (next) {
                static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
                    constexpr int M = decltype(m_tag)::value;
                    if constexpr (M >= decltype(m0_tag)::value && M < decltype(m1_tag)::value) {
                        stage_slot(w_tag, m_tag, c + 1, Xn, Check{}, Nxt{});
                        if constexpr (FAST) {
                            load_slot(w_tag, m_tag, c + AHEAD, std::true_type{}, Nxt{});
                        } else {
                            if (c + AHEAD < nchunks) load_slot(w_tag, m_tag, c + AHEAD, std::false_type{}, Nxt{});
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                });
            }
        };
        // The delta rule's mid-chunk barrier waits for the row waves' U rows:
        // half the staging goes before it (beside U), half after (beside the
        // rows).
        constexpr int MH = VAR == V_GDN ? NSLOT / 2 : NSLOT;
        stage_range(std::integral_constant<int, 0>{}, std::integral_constant<int, MH>{});
        if constexpr (VAR == V_GDN) __syncthreads();  // U of chunk c visible
        stage_range(std::integral_constant<int, MH>{}, std::integral_constant<int, NSLOT>{});
        const float eg = DECAYED ? Tsc[c % NTB] : 1.f;
        state_update(w_tag, c, X, eg, sh);
        put_smax(w_tag, c + 1);
        if (next) write_sts(w_tag, Xn, shn);
        if constexpr (DECAYED) {
            if (W == GW && (FAST || c + 2 < nchunks)) gate_tables(c + 2, (c + 2) % NTB, Cur{});
        }
    };

    // Schedule. The first FAST chunk is peeled so that both edges into the
    // steady-state loop leave the same memory operations in flight (the wait
    // counts inside the loop are then exact and let output stores drain in the
    // background); the last chunks take the checked path.
    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, 1 % NPS>;
    if constexpr (R::MODE == 3) {
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        for_wave([&](auto w_tag) __attribute__((always_inline)) {
            constexpr int W = decltype(w_tag)::value;
            if constexpr (R::rows(W)) {
                if (nchunks > 0) {
                    load_q(0, P0{});
                    if (nchunks > 1) load_q(1, P1{});
                    load_wu(0);
                    __syncthreads();  // prologue (the state waves' gate tables)
                }
                int c = 0;
                for (; c + 1 < nfull; c += 2) {
                    row_iter(w_tag, c, std::false_type{}, P0{});
                    row_iter(w_tag, c + 1, std::false_type{}, P1{});
                }
                for (; c < nchunks; ++c) {
                    if (c < nfull) {
                        if (c & 1) {
                            row_iter(w_tag, c, std::false_type{}, P1{});
                        } else {
                            row_iter(w_tag, c, std::false_type{}, P0{});
                        }
                    } else {
                        if (c & 1) {
                            row_iter(w_tag, c, std::true_type{}, P1{});
                        } else {
                            row_iter(w_tag, c, std::true_type{}, P0{});
                        }
                    }
                }
            } else {
                // The staging waves issue ahead of the row waves that share their
                // SIMDs: their loads and the state update feed the next chunk.
                __builtin_amdgcn_s_setprio(1);
                // chunks 0 .. NPS-1 into register sets 0 .. NPS-1; gate tables
                // of chunks 0 and 1; chunk 0 staged and chunk NPS into set 0
                if (nchunks > 0) {
                    load_gates(0, std::false_type{}, Set0{});
                    static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
                        load_slot(w_tag, m_tag, 0, std::false_type{}, Set0{});
                    });
                    if constexpr (NPS == 2) {
                        if (nchunks > 1) {
                            load_gates(1, std::false_type{}, Set1{});
                            static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
                                load_slot(w_tag, m_tag, 1, std::false_type{}, Set1{});
                            });
                        }
                    }
                    if constexpr (DECAYED) {
                        if (W == GW) gate_tables(0, 0, Set0{});
                        if constexpr (NPS == 2) {
                            if (W == GW && nchunks > 1) gate_tables(1, 1, Set1{});
                            if (nchunks > 2) load_gates(2, std::false_type{}, Set0{});
                        } else {
                            if (nchunks > 1) {
                                load_gates(1, std::false_type{}, Set0{});
                                if (W == GW) gate_tables(1, 1, Set0{});
                            }
                        }
                    }
                    put_smax(w_tag, 0);
                    __syncthreads();  // gate tables of chunk 0 and max |S_0| visible
                    static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
                        stage_slot(w_tag, m_tag, 0, Tiles, std::true_type{}, Set0{});
                        if (nchunks > NPS) load_slot(w_tag, m_tag, NPS, std::false_type{}, Set0{});
                    });
                    write_sts(w_tag, Tiles, get_shift(0));
                }
                int c = 0;
                if (nfull >= AHEAD + 1) {
                    state_iter(w_tag, 0, std::true_type{}, P0{});
                    for (c = 1; c + 1 <= nfull - AHEAD - 1; c += 2) {
                        state_iter(w_tag, c, std::true_type{}, P1{});
                        state_iter(w_tag, c + 1, std::true_type{}, P0{});
                    }
                }
                for (; c < nchunks; ++c) {
                    if (c & 1) {
                        state_iter(w_tag, c, std::false_type{}, P1{});
                    } else {
                        state_iter(w_tag, c, std::false_type{}, P0{});
                    }
                }
            }
        });
    } else if constexpr (DB) {
        // chunks 0 .. NPS-1 into register sets 0 .. NPS-1; gate tables of
        // chunks 0 and 1; chunk 0 staged and chunk NPS into set 0
        if (nchunks > 0) {
            load_gates(0, std::false_type{}, Set0{});
            static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
                load_any(m_tag, 0, std::false_type{}, Set0{});
            });
            if constexpr (NPS == 2) {
                if (nchunks > 1) {
                    load_gates(1, std::false_type{}, Set1{});
                    static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
                        load_any(m_tag, 1, std::false_type{}, Set1{});
                    });
                }
            }
            load_wu(0);
            if constexpr (DECAYED) {
                if (wv == GW) gate_tables(0, 0, Set0{});
                if constexpr (NPS == 2) {
                    if (wv == GW && nchunks > 1) gate_tables(1, 1, Set1{});
                    if (nchunks > 2) load_gates(2, std::false_type{}, Set0{});
                } else {
                    if (nchunks > 1) {
                        load_gates(1, std::false_type{}, Set0{});
                        if (wv == GW) gate_tables(1, 1, Set0{});
                    }
                }
            }
            for_wave([&](auto w_tag) __attribute__((always_inline)) { put_smax(w_tag, 0); });
            __syncthreads();  // gate tables of chunk 0 and max |S_0| visible
            static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
                stage_any(m_tag, 0, Tiles, std::true_type{}, Set0{});
                if (nchunks > NPS) load_any(m_tag, NPS, std::false_type{}, Set0{});
            });
            const int sh0 = get_shift(0);
            for_wave([&](auto w_tag) __attribute__((always_inline)) { write_sts(w_tag, Tiles, sh0); });
        }
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        int c = 0;
        if (nfull >= AHEAD + 1) {
            chunk_db(0, std::true_type{}, P0{});
            for (c = 1; c + 1 <= nfull - AHEAD - 1; c += 2) {
                chunk_db(c, std::true_type{}, P1{});
                chunk_db(c + 1, std::true_type{}, P0{});
            }
        }
        for (; c < nchunks; ++c) {
            if (c & 1) {
                chunk_db(c, std::false_type{}, P1{});
            } else {
                chunk_db(c, std::false_type{}, P0{});
            }
        }
    } else {
        if (nchunks > 0) {
            load_gates(0, std::false_type{}, Set0{});
            static_for<NSLOT>([&](auto m_tag) __attribute__((always_inline)) {
                load_any(m_tag, 0, std::false_type{}, Set0{});
            });
            load_wu(0);
            if constexpr (DECAYED) {
                if (wv == GW) gate_tables(0, 0, Set0{});
            }
            for_wave([&](auto w_tag) __attribute__((always_inline)) { put_smax(w_tag, 0); });
        }
        int c = 0;
        if (nfull >= 2) {
            chunk_sb(0, std::true_type{});
            for (c = 1; c < nfull - 1; ++c) chunk_sb(c, std::true_type{});
        }
        for (; c < nchunks; ++c) chunk_sb(c, std::false_type{});
    }

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
        if (a.z_out && split == 0 && n == 0) {
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti) {
                if (wv == R::zowner(ti)) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) a.z_out[(size_t)bh * DK + ti * 16 + 4 * g + e] = zacc[ti][e];
                }
            }
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
