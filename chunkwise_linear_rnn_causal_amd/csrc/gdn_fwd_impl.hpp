// gdn_fwd_impl.hpp -- serial chunk pass of the gated delta rule (gfx950, bf16 inputs).
//
// Method (wln20 "LLM注意力优化：线性注意力", Gated DeltaNet section; tensorplay
// "Talk Linear Attention", section 6.2, WY / UT chunk form). For chunk c with
// chunk-local cumulative log-gate G_r, a_r = exp(G_r), Gamma_rs = exp(G_r - G_s)
// and the per-chunk products of the chunk-parallel preparation
// (gdn_prep_impl.hpp): W = T diag(beta a) K, U~ = T diag(beta) V and the masked
// decayed scores Gamma (.) Q K^T (.) M:
//   U      = U~ - W S                      (the serial correction)
//   O      = diag(a) Q S + (Gamma (.) Q K^T (.) M) U
//   S_next = a_C S + K^T diag(a_C / a) U
// with S the d_k x d_v state before the chunk and M the inclusive causal mask.
//
// Mapping. One workgroup owns one (batch*head, 16-column value slice) and walks
// the chunks in order. The columns of S are independent in the serial chain
// (U's columns need only S's columns), so the chain needs nothing from other
// workgroups. Eight waves in three roles:
//  - wave 0, the chain wave, holds the state slice in fp32 MFMA accumulators
//    for the whole sequence and runs U = U~ - W S and the state update. The D
//    layout of a 16 x 16 accumulator tile (lane (g, n): rows 4g + e, column n)
//    is, for two row-adjacent tiles, exactly an MFMA operand fragment with the
//    tile row index in the K slots {32p + 4g + e, 32p + 16 + 4g + e}: S's tiles
//    are the B operand of W S (channels in the K slots), U's tiles the B
//    operand of K^T U (tokens in the K slots). The chain therefore never
//    passes through LDS and has no barrier inside a chunk. It also owns the
//    whole slice of S, so the fp16 operand scale (a power of two keeping the
//    carried state inside fp16's range) comes from an exact wave maximum.
//  - waves 1-3 stage K and W of chunk c+1 into the other half of
//    double-buffered LDS tiles (loads issued two chunks ahead).
//  - waves 4-7, one per 16-row block, form the outputs: the inter term of
//    chunk c in iteration c, and the intra term (scores times U) of chunk c in
//    iteration c+1, when the chain wave has left U's fragments in LDS; the
//    fragment of S^T they need is the chain wave's B operand of S, written
//    once per chunk. Their query rows and score fragments come straight from
//    global memory into registers (two chunks ahead), so the only LDS reads of
//    these waves are S^T and U. The first of them, whose block has the fewest
//    scores, also builds the gate tables of the next chunk (cycle counters per
//    role showed the gate tables making their staging wave the longest role).
// One barrier per chunk. Operand K slots of Q and W rows follow the channel
// order {32p + 4g + e, 32p + 16 + 4g + e} of S's fragments (two 8-byte pieces
// per fragment). The per-workgroup LDS traffic is what bounds the chunk period
// (the serial chain's own MFMA work is 32 instructions per chunk), which is why
// the scores, identical in every value slice of a head, are formed once by the
// preparation instead of here.
#pragma once

#include <type_traits>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

template <int DK> struct GdnCfg {
    static constexpr int C = 64;        // chunk
    static constexpr int DVT = 16;      // value columns per workgroup
    static constexpr int NW = 8;        // waves
    static constexpr int NTI = DK / 16; // 16-channel tiles of the state slice
    static constexpr int NKS = DK / 32; // k-steps over channels
    static constexpr int NRB = C / 16;  // 16-row blocks
    static constexpr int WP = DK + 8;   // row pitch of the W tile (fp16 elements)
    static constexpr int KP = DK + 16;  // row pitch of the K tile (also read transposed)
    static constexpr int OK = 0, OW = OK + C * KP, SET = OW + C * WP;
    // staging: wave loads of 1 KB (64 lanes x 16 bytes) per tensor and chunk
    static constexpr int SEG = DK / 8;            // 16-byte segments per row
    static constexpr int RPL = 64 / SEG;          // rows per wave load
    static constexpr int NI1 = C / RPL;           // wave loads per tensor
    static constexpr int NSW = 3;                 // staging waves
    static constexpr int NLD = 2 * NI1;           // wave loads per chunk (K and W)
    static constexpr int NSL = (NLD + NSW - 1) / NSW;  // slots per staging wave
    static_assert(64 % SEG == 0 && NI1 * RPL == C, "staging geometry");
};

// Two 8-byte reads: row `row` of a row-major fp16 tile, channels
// {32p + 4g + (0..3), 32p + 16 + 4g + (0..3)} -- an operand fragment in the
// channel order of the state's accumulator tiles.
template <int P>
__device__ inline f16x8 chan_frag(const f16 *X, int row, int p, int g) {
    const f16 *r = X + row * P + 32 * p + 4 * g;
    const f16x4 a = *reinterpret_cast<const f16x4 *>(r);
    const f16x4 b = *reinterpret_cast<const f16x4 *>(r + 16);
    return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// QK16: q and k come as fp16 rows of the workspace (a.qc, a.kc, [BH, Lp, DK];
// the short convolution fused into the preparation writes them) instead of bf16
// inputs.
// VEC: Kimi Delta Attention (kda_prep_impl.hpp). The preparation folds the
// per-channel gates into q, k, W and the scores, and the state's rows decay by
// the chunk's Gam_C (a.cdec) instead of a scalar exp(g_C); there is no scalar gate.
template <typename TO, int DK, bool QK16, bool VEC = false>
__global__ void __launch_bounds__(512) gdn_fwd_kernel(ChunkArgs a) {
    using Cfg = GdnCfg<DK>;
    using MF = Mfma<f16>;
    constexpr int C = Cfg::C, NTI = Cfg::NTI, NKS = Cfg::NKS, NRB = Cfg::NRB;
    constexpr int WP = Cfg::WP, KP = Cfg::KP, SET = Cfg::SET;
    constexpr int NSL = Cfg::NSL, SEG = Cfg::SEG, RPL = Cfg::RPL, NI1 = Cfg::NI1;

    __shared__ __attribute__((aligned(16))) f16 Tiles[2 * SET];
    // gate tables per buffer: [0] exp(G_s), [1] exp(g_C - G_s); Tsc: exp(g_C)
    __shared__ __attribute__((aligned(16))) float Tg[2 * 2 * C];
    __shared__ float Tsc[2];
    // VEC: the state's per-channel decay of chunk c (buffer c & 1)
    __shared__ __attribute__((aligned(16))) float Cd[2][VEC ? DK : 4];
    // chain -> output waves: S^T fragments of the state before chunk c (buffer
    // c & 1) with their shift, and U fragments of chunk c (buffer c & 1)
    __shared__ __attribute__((aligned(16))) f16x8 Sf[2][NKS][64];
    __shared__ __attribute__((aligned(16))) f16x8 Uf[2][2][64];
    __shared__ int Ssh[2];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int vid = xcd_virtual_block();
    const int bh = vid / a.nsplit, split = vid - bh * a.nsplit;
    const int j0 = split * Cfg::DVT;
    const int L = a.L, dv = a.dv;
    const int nchunks = (L + C - 1) / C;

    // q and k as raw 16-bit words: bf16 inputs, or fp16 rows of the workspace
    const uint16_t *qg = QK16 ? (const uint16_t *)a.qc + (size_t)bh * a.Lp * DK
                              : (const uint16_t *)a.q + (size_t)bh * a.ld * DK;
    // two packed 16-bit values to two packed fp16 values: bf16 with the packed
    // round-toward-zero conversion (exact for every bf16 value in fp16's normal
    // range); fp16 as they are
    auto to_h2 = [](uint32_t u) __attribute__((always_inline)) {
        return QK16 ? u : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(u), bf16_hi(u)));
    };
    const f16 *mg = (const f16 *)a.mf + (size_t)bh * nchunks * (6 * 512);
    const uint16_t *kg = QK16 ? (const uint16_t *)a.kc + (size_t)bh * a.Lp * DK
                              : (const uint16_t *)a.k + (size_t)bh * a.ld * DK;
    const float *lgg = a.lg ? a.lg + (size_t)bh * a.ld : nullptr;
    const f16 *wg = (const f16 *)a.w + (size_t)bh * a.Lp * DK;
    TO *og = (TO *)a.o + (size_t)bh * a.ld * dv + j0;

    if (wv == 0) {
        // ================= chain wave =================
        // The slice is carried at its operand scale: St = S 2^-sh, with the shift
        // sh >= 0 chosen from the exact max |S| (carry_shift) and changed only when
        // that max moves to another power-of-two band, by an exact rescale. The
        // products U 2^-sh = U~ 2^-sh - W St and St_next = exp(g_C) St + K^T (w U 2^-sh)
        // then need no scaling of their own.
        f32x4 St[NTI];
        int sh = 0;
#pragma unroll
        for (int ti = 0; ti < NTI; ++ti) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                St[ti][e] = a.s_in ? a.s_in[(size_t)bh * DK * dv + (size_t)(ti * 16 + 4 * g + e) * dv + j0 + n] : 0.f;
        }
        // rescale St when the band of its max moves (uniform branch; rare)
        auto rescale = [&]() __attribute__((always_inline)) {
            float m = 0.f;
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(St[ti][e]));
            m = wave_max_nonneg(m);
            // exponent of the true max |S| = m 2^sh, then the shift it calls for
            const int eb = (int)((__float_as_uint(m) >> 23) & 0xffu);
            const int want = __builtin_amdgcn_readfirstlane(eb == 0 ? 0 : min(max(eb + sh - 134, 0), 120));
            if (want != sh) {
                const float f = pow2i(sh - want);
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) St[ti] *= f;
                sh = want;
            }
        };
        // U~ of chunk c in accumulator layout (the preparation writes it so): lane
        // (g, n) holds rows 16 rb + 4g + e, column j0 + n; two register sets,
        // loaded two chunks ahead
        const f16 *utl = (const f16 *)a.ut + (size_t)bh * (a.Lp / C) * (dv / 16) * (NRB * 256) +
                         (size_t)split * (NRB * 256) + lane * 4;
        const size_t ut_chunk = (size_t)(dv / 16) * (NRB * 256);
        f16x4 ut[2][NRB];
        auto load_ut = [&](int c, int set) __attribute__((always_inline)) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
                ut[set][rb] = *reinterpret_cast<const f16x4 *>(utl + c * ut_chunk + rb * 256);
        };
        // fragments of -St: the B operand of -W St, and (as -St^T) the A operand of the
        // output waves' inter term (they flip the sign back)
        f16x8 nsb[NKS];
        auto make_nsb = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int p = 0; p < NKS; ++p)
                nsb[p] = f16x8{(f16)(-St[2 * p][0]), (f16)(-St[2 * p][1]), (f16)(-St[2 * p][2]),
                               (f16)(-St[2 * p][3]), (f16)(-St[2 * p + 1][0]), (f16)(-St[2 * p + 1][1]),
                               (f16)(-St[2 * p + 1][2]), (f16)(-St[2 * p + 1][3])};
        };
        auto publish = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int p = 0; p < NKS; ++p) Sf[buf][p][lane] = nsb[p];
            if (lane == 0) Ssh[buf] = sh;
        };
        rescale();
        make_nsb();
        publish(0);
        if (nchunks > 0) {
            load_ut(0, 0);
            load_ut(min(1, nchunks - 1), 1);
        }
        __syncthreads();  // prologue: chunk 0 staged, S_0 fragments visible

        auto iter = [&](int c, auto par) __attribute__((always_inline)) {
            constexpr int P = decltype(par)::value;
            const f16 *X = Tiles + P * SET;
            const float *T = Tg + P * 2 * C;
            const f16 *Ks = X + Cfg::OK, *Ws = X + Cfg::OW;
            // Every LDS operand of the chunk's chain is read up front (W for U, K^T
            // and the state-update weights), so the reads overlap each other and the
            // MFMAs instead of each waiting its own round trip.
            // (K^T is read once half of W has been used, which bounds the live registers)
            f16x8 wf[NRB][NKS], kt[NTI][2];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int p = 0; p < NKS; ++p) wf[rb][p] = chan_frag<WP>(Ws, rb * 16 + n, p, g);
            // the scalar gate's weights and decay; VEC has no scalar gate (both are 1)
            // and reads the per-channel decay of its state rows instead
            f32x4 wlo[2], whi[2];
            float eg = 1.f;
            f32x4 cd[VEC ? NTI : 1];
            if constexpr (VEC) {
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) cd[ti] = *reinterpret_cast<const f32x4 *>(&Cd[P][ti * 16 + 4 * g]);
            } else {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    wlo[q] = *reinterpret_cast<const f32x4 *>(&T[C + 32 * q + 4 * g]);
                    whi[q] = *reinterpret_cast<const f32x4 *>(&T[C + 32 * q + 16 + 4 * g]);
                }
                eg = Tsc[P];
            }
            __builtin_amdgcn_sched_barrier(0);
            // U 2^-sh = U~ 2^-sh + W (-St)
            f32x4 U[NRB];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e) U[rb][e] = (float)ut[P][rb][e];
            if (sh != 0) {
                const float us = pow2i(-sh);
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) U[rb] *= us;
            }
            constexpr int PH = (NKS + 1) / 2;
#pragma unroll
            for (int p = 0; p < PH; ++p)
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) U[rb] = MF::mma(wf[rb][p], nsb[p], U[rb]);
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti)
#pragma unroll
                for (int q = 0; q < 2; ++q) kt[ti][q] = tr_frag<KP>(Ks, 32 * q + 4 * g, ti * 16, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = PH; p < NKS; ++p)
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) U[rb] = MF::mma(wf[rb][p], nsb[p], U[rb]);
            // unconditional (the last chunk again near the end): every path through
            // the loop leaves the same loads in flight, so the wait counts are exact
            load_ut(min(c + 2, nchunks - 1), P);
            // U fragments: weighted by w_s = exp(g_C - G_s) for the state update;
            // as they are for the output waves
            f16x8 ub[2];
#pragma unroll
            for (int q = 0; q < 2; ++q)
                ub[q] = VEC ? pack_tiles(U[2 * q], U[2 * q + 1], 1.f)
                            : pack_tiles(U[2 * q] * wlo[q], U[2 * q + 1] * whi[q], 1.f);
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti) {
                if constexpr (VEC) St[ti] *= cd[ti];
                else St[ti] *= eg;
            }
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) St[ti] = MF::mma(kt[ti][q], ub[q], St[ti]);
#pragma unroll
            for (int q = 0; q < 2; ++q) Uf[P][q][lane] = pack_tiles(U[2 * q], U[2 * q + 1], 1.f);
            rescale();
            make_nsb();
            publish(P ^ 1);
            __syncthreads();  // chunk c+1 staged; S_{c+1} and U_c fragments visible
        };
        int c = 0;
        for (; c + 1 < nchunks; c += 2) {
            iter(c, std::integral_constant<int, 0>{});
            iter(c + 1, std::integral_constant<int, 1>{});
        }
        if (c < nchunks) iter(c, std::integral_constant<int, 0>{});
        __syncthreads();  // epilogue: the output waves finish the last chunk
        if (a.s_out) {
            const float f = pow2i(sh);
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.s_out[(size_t)bh * DK * dv + (size_t)(ti * 16 + 4 * g + e) * dv + j0 + n] = St[ti][e] * f;
        }
    } else if (wv < 4) {
        // ================= staging waves (wave index a compile-time constant) =================
        auto stage_role = [&](auto sw_tag) __attribute__((always_inline)) {
        constexpr int sw = decltype(sw_tag)::value;
        uint4 pre[2][NSL];
        // slot m of this wave: wave load i = sw + 3 m (the last wave load again past
        // the end, so every staging wave has the same loads in flight); tensor
        // i / NI1 (0 K, 1 W)
        auto slot = [](int m) { return min(sw + Cfg::NSW * m, Cfg::NLD - 1); };
        auto load_chunk = [&](int c, int set) __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < NSL; ++m) {
                const int i = slot(m), kind = i / NI1, ii = i % NI1;  // compile-time after unrolling
                const int row = ii * RPL + lane / SEG, seg = lane % SEG;
                const int t = c * C + row;
                if (kind == 1)
                    pre[set][m] = *reinterpret_cast<const uint4 *>(wg + (size_t)t * DK + seg * 8);
                else
                    pre[set][m] = *reinterpret_cast<const uint4 *>(kg + (size_t)min(t, L - 1) * DK + seg * 8);
            }
        };
        auto stage_chunk = [&](int c, int set, int buf) __attribute__((always_inline)) {
            f16 *X = Tiles + buf * SET;
#pragma unroll
            for (int m = 0; m < NSL; ++m) {
                const int i = slot(m), kind = i / NI1, ii = i % NI1;
                const int row = ii * RPL + lane / SEG, seg = lane % SEG;
                const uint4 w4 = pre[set][m];
                if (kind == 1) {
                    *reinterpret_cast<uint4 *>(&X[Cfg::OW + row * WP + seg * 8]) = w4;
                } else {
                    // bf16 -> fp16 with the packed round-toward-zero conversion: every
                    // bf16 value in fp16's normal range converts exactly
                    const bool valid = c * C + row < L;
                    const uint32_t u[4] = {w4.x, w4.y, w4.z, w4.w};
                    uint4 h;
                    uint32_t *hw = reinterpret_cast<uint32_t *>(&h);
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        hw[k] = valid ? to_h2(u[k]) : 0u;
                    *reinterpret_cast<uint4 *>(&X[Cfg::OK + row * KP + seg * 8]) = h;
                }
            }
        };

        // Loads are issued unconditionally (chunk indices past the end repeat the
        // last chunk), so every path leaves the same loads in flight and the wait
        // before each staged slot is exact: two chunks of loads stay in flight.
        // (the fences keep the prologue's loads in this order, the one the loop
        // assumes on entry: chunk 1 older than chunk 2)
        if (nchunks > 0) {
            load_chunk(0, 0);
            load_chunk(min(1, nchunks - 1), 1);
            __builtin_amdgcn_sched_barrier(0);
            stage_chunk(0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            load_chunk(min(2, nchunks - 1), 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();  // prologue
        // iteration c: stage chunk c+1 (register set (c+1) & 1) into buffer (c+1) & 1,
        // then load chunk c+3 into that register set. In the last iteration the
        // staged chunk is a repeat of the last one, in the buffer no wave reads
        // any more: staging stays unconditional, which keeps the wait counts exact.
        auto iter = [&](int c, auto par) __attribute__((always_inline)) {
            constexpr int P = decltype(par)::value;  // c & 1
            stage_chunk(c + 1, P ^ 1, P ^ 1);
            load_chunk(min(c + 3, nchunks - 1), P ^ 1);
            // no instruction crosses the barrier: a conversion hoisted above it
            // would need the next register set a chunk early (a full wait)
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        // The first two iterations are peeled: the loop is then entered with its
        // register sets in flight in the same order as at its back edge, which the
        // compiler needs to keep the waits at one set (not every load) per chunk.
        int c = 0;
        if (nchunks >= 2) {
            iter(0, std::integral_constant<int, 0>{});
            iter(1, std::integral_constant<int, 1>{});
            c = 2;
        }
        for (; c + 1 < nchunks; c += 2) {
            iter(c, std::integral_constant<int, 0>{});
            iter(c + 1, std::integral_constant<int, 1>{});
        }
        if (c < nchunks) iter(c, std::integral_constant<int, 0>{});
        __syncthreads();  // epilogue
        };
        if (wv == 1) stage_role(std::integral_constant<int, 0>{});
        else if (wv == 2) stage_role(std::integral_constant<int, 1>{});
        else stage_role(std::integral_constant<int, 2>{});
    } else {
        // ================= output waves: row block rb (a compile-time constant) =================
        auto out_role = [&](auto rb_tag) __attribute__((always_inline)) {
        constexpr int rb = decltype(rb_tag)::value;
        constexpr int NP = rb / 2 + 1;                  // score fragments (rb, p), 2p <= rb
        constexpr int F0 = rb + (rb > 2 ? rb - 2 : 0);  // index of fragment (rb, 0)
        const int r = rb * 16 + n;  // this lane's query row within the chunk
        // Query row r in S's channel order (channels 32p + 4g .. + 3 and
        // 32p + 16 + 4g .. + 3, raw bf16) and the score fragments, two register
        // sets loaded two chunks ahead; chunk indices past the end repeat the
        // last chunk, so every iteration leaves the same loads in flight.
        uint2 qraw[2][NKS][2];
        uint4 mraw[2][NP];
        // The first output wave (the one with the least work) also builds the gate
        // tables: in iteration c those of chunk c+1, from log-gates loaded with
        // that chunk's queries (and, for VEC, the chunk's per-channel state decay).
        constexpr bool GT = rb == 0;
        constexpr int NCD = (DK + 63) / 64;
        float gpre[2];
        float cpre[2][NCD];
        const float *gsrc = lgg ? lgg : reinterpret_cast<const float *>(kg);  // kg: at least L floats
        auto load = [&](int c, int set) __attribute__((always_inline)) {
            const uint16_t *qrow = qg + (size_t)min(c * C + r, L - 1) * DK + 4 * g;
#pragma unroll
            for (int p = 0; p < NKS; ++p) {
                qraw[set][p][0] = *reinterpret_cast<const uint2 *>(qrow + 32 * p);
                qraw[set][p][1] = *reinterpret_cast<const uint2 *>(qrow + 32 * p + 16);
            }
            const f16 *mrow = mg + (size_t)c * (6 * 512) + F0 * 512 + lane * 8;
#pragma unroll
            for (int p = 0; p < NP; ++p) mraw[set][p] = *reinterpret_cast<const uint4 *>(mrow + p * 512);
            if constexpr (GT) {
                // unconditional, from a valid address when there is no gate; the value
                // is masked where it is used (masking it here would wait for it here)
                gpre[set] = gsrc[min(c * C + lane, L - 1)];
                if constexpr (VEC) {
#pragma unroll
                    for (int i = 0; i < NCD; ++i)
                        cpre[set][i] = a.cdec[((size_t)bh * nchunks + c) * DK + min(lane + 64 * i, DK - 1)];
                }
            }
        };
        // gate tables of chunk c from register set `set` into buffer `buf`: the
        // chunk-local inclusive prefix G of the log-gates (rows past L: 0), exp(G),
        // exp(g_C - G) and exp(g_C)
        auto gate_tables = [&](int c, int set, int buf) __attribute__((always_inline)) {
            float *T = Tg + buf * 2 * C;
            const float G = wave_inclusive_sum((lgg && c * C + lane < L) ? gpre[set] : 0.f);
            const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
            T[lane] = __expf(G);
            T[C + lane] = __expf(gC - G);
            if (lane == 0) Tsc[buf] = __expf(gC);
            if constexpr (VEC) {
#pragma unroll
                for (int i = 0; i < NCD; ++i)
                    if (lane + 64 * i < DK) Cd[buf][lane + 64 * i] = cpre[set][i];
            }
        };
        f32x4 oprev = {0.f, 0.f, 0.f, 0.f};
        f16x8 bprev[NP];
        int shprev = 0;
        // intra term of the previous chunk from U's fragments, then its store
        auto finish_prev = [&](int cp, const f16x8 (&uf)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int p = 0; p < NP; ++p) oprev = MF::mma(uf[p], bprev[p], oprev);
            oprev *= pow2i(shprev);
            const int t = cp * C + r;
            if (t < L) st4<TO>(og + (size_t)t * dv + 4 * g, oprev);
        };
        if (nchunks > 0) {
            load(0, 0);
            load(min(1, nchunks - 1), 1);
            if constexpr (GT) gate_tables(0, 0, 0);
        }
        __syncthreads();  // prologue
        auto iter = [&](int c, auto par) __attribute__((always_inline)) {
            constexpr int P = decltype(par)::value;
            const float *T = Tg + P * 2 * C;
            // this chunk's operands: queries converted to fp16 (round toward zero:
            // exact for every bf16 value in fp16's normal range), score fragments,
            // then S^T and U from LDS
            f16x8 qf[NKS], mf[NP], sf[NKS], uf[2];
#pragma unroll
            for (int p = 0; p < NKS; ++p) {
                const uint32_t u[4] = {qraw[P][p][0].x, qraw[P][p][0].y, qraw[P][p][1].x, qraw[P][p][1].y};
                uint32_t h[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    h[k] = to_h2(u[k]);
                qf[p] = __builtin_bit_cast(f16x8, make_uint4(h[0], h[1], h[2], h[3]));
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) mf[p] = __builtin_bit_cast(f16x8, mraw[P][p]);
            load(min(c + 2, nchunks - 1), P);
#pragma unroll
            for (int p = 0; p < NKS; ++p) sf[p] = Sf[P][p][lane];
#pragma unroll
            for (int p = 0; p < 2; ++p) uf[p] = Uf[P ^ 1][p][lane];
            const int sh = Ssh[P];
            const float er = -T[r];  // -: the fragments hold -S^T
            if (c > 0) finish_prev(c - 1, uf);
            // inter term: O^T = S^T (a Q)^T at scale 2^-sh
            f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < NKS; ++p) oacc = MF::mma(sf[p], qf[p], oacc);
            oprev = oacc * er;
#pragma unroll
            for (int p = 0; p < NP; ++p) bprev[p] = mf[p];
            shprev = sh;
            // chunk c+1's tables into the other buffer, last read in iteration c-1
            // (past the end: a repeat of the last chunk that no wave reads)
            if constexpr (GT) gate_tables(c + 1, P ^ 1, P ^ 1);
            __syncthreads();
        };
        int c = 0;
        for (; c + 1 < nchunks; c += 2) {
            iter(c, std::integral_constant<int, 0>{});
            iter(c + 1, std::integral_constant<int, 1>{});
        }
        if (c < nchunks) iter(c, std::integral_constant<int, 0>{});
        __syncthreads();  // epilogue: U of the last chunk visible
        if (nchunks > 0) {
            f16x8 uf[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) uf[p] = Uf[(nchunks - 1) & 1][p][lane];
            finish_prev(nchunks - 1, uf);
        }
        };
        switch (wv) {
            case 4: out_role(std::integral_constant<int, 0>{}); break;
            case 5: out_role(std::integral_constant<int, 1>{}); break;
            case 6: out_role(std::integral_constant<int, 2>{}); break;
            default: out_role(std::integral_constant<int, 3>{}); break;
        }
    }
}

template <typename TO, int DK>
hipError_t launch_gdn_fwd(const ChunkArgs &a, hipStream_t st) {
    const int blocks = a.BH * a.nsplit;
    if (a.cdec)
        hipLaunchKernelGGL((gdn_fwd_kernel<TO, DK, true, true>), dim3(blocks), dim3(512), 0, st, a);
    else if (a.qc)
        hipLaunchKernelGGL((gdn_fwd_kernel<TO, DK, true>), dim3(blocks), dim3(512), 0, st, a);
    else
        hipLaunchKernelGGL((gdn_fwd_kernel<TO, DK, false>), dim3(blocks), dim3(512), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
