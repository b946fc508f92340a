// gdn_prep_impl.hpp -- chunk-parallel preparation for the gated delta rule.
//
// The delta rule S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
// (wln20 "LLM注意力优化：线性注意力", Gated DeltaNet section, written in the d_k x d_v
// orientation) can be rewritten as S_t = alpha_t S_{t-1} + k_t u_t^T with the
// pseudo-value u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t). tensorplay "Talk Linear
// Attention" section 6.2 names the obstacle (u_t depends on S_{t-1}) and the cure
// (a WY / Householder-product representation that makes it chunk-parallel) without
// spelling it out; worked out for one chunk with a_r = exp(G_r), G the chunk-local
// cumulative log-gate:
//   (I + P) U = diag(beta) V - diag(beta a) K S_0,
//   P_rs = beta_r exp(G_r - G_s) (k_r . k_s) for s < r, 0 otherwise,
// so with T = (I + P)^-1:  W = T diag(beta a) K,  U~ = T diag(beta) V,  U = U~ - W S_0.
// W and U~ do not depend on the state, so this kernel computes them for every
// chunk in parallel (one workgroup per chunk); the serial chunk pass then only
// forms U = U~ - W S_prev.
//
// Layout of the results, in the tensor-core operand type (fp16 for bf16
// inputs, fp32 for fp32 inputs): W row-major [BH, Lp, DK]; U~ [BH, Lp, dv]
// elements, row-major for fp32 inputs (the serial pass reads four consecutive
// columns per lane), and for bf16 inputs in the accumulator layout of the
// serial pass (see the store below). Padded tokens (t >= L) have beta = 0 and
// k = v = 0, which makes their rows of W and U~ zero.
//
// For bf16 inputs the kernel also forms the chunk's masked decayed scores,
// M_rs = exp(G_r - G_s) (q_r . k_s) for s <= r and 0 above the diagonal, which
// the serial pass needs in every value slice of a head: here they are formed
// once per chunk. They come out of the same 16 x 16 tile loop as P (a tile of
// M^T and the matching tile of P share the key fragment) and are stored as the
// serial pass's MFMA operand fragments, [BH][chunk][6][64 lanes][8] fp16:
// fragment (rb, p) holds, for lane (g, n), the scores of query row 16 rb + n
// against keys {32p + 4g + e, 32p + 16 + 4g + e} (e = 0..3), for the six pairs
// (rb, p) with 2p <= rb (fragment index rb + max(rb - 2, 0) + p).
#pragma once

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

template <typename TM, int DK, int C, bool CONV = false>
struct PrepCfg {
    static constexpr int DVMAX = 128;
    static constexpr int PAD = 16 / (int)sizeof(TM);
    static constexpr int KP = DK + PAD;   // row pitch of K
    static constexpr int TP = C + 1;      // fp32 row pitch of P and T
    static constexpr int OP = C + PAD;    // row pitch of T in the operand type
    static constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }
    static constexpr size_t up16(size_t x) { return (x + 15) / 16 * 16; }
    // Three regions, each reused as lifetimes end (about 38 KB at d_k = 128,
    // so four workgroups fit on a CU):
    //   A: K row-major (until P is formed), then T in fp32 (until it is
    //      converted), then K^T scaled by beta a (for W), then V^T scaled by
    //      beta (for U~);
    //   B: P in fp32 (until T is complete), then T in the operand type;
    //   C: the per-wave scratch of the off-diagonal blocks.
    // K and V stay in registers from their load until their scaled transposes
    // are staged, after T is converted.
    static constexpr size_t o_a = 0;
    // With the fused short convolution, region B first holds each tensor's raw
    // rows with a halo of HALO rows before the chunk (bf16, pitch RP); still four
    // workgroups per CU at d_k = 128.
    static constexpr int HALO = 3, RP = (DK > DVMAX ? DK : DVMAX) + 8;
    static constexpr size_t o_p = o_a + up16(cmax(cmax(sizeof(TM) * C * KP, 4 * C * TP),
                                                  sizeof(TM) * (DK > DVMAX ? DK : DVMAX) * C));
    static constexpr size_t o_c = o_p + up16(cmax(cmax(4 * C * TP, sizeof(TM) * C * OP),
                                                  CONV ? 2 * (C + HALO) * RP : 0));
    static constexpr size_t o_g = o_c + 4 * 4 * 256;
    static constexpr size_t lds_bytes = o_g + 4 * 2 * C;
};

// The fused short convolution (wln20 "LLM注意力优化：线性注意力", DeltaNet
// section: a kernel-4 causal depthwise convolution in front of the delta rule):
// y_t = sum_{tau < K} w_tau x_{t - tau} per channel, for 4 consecutive tokens
// s0 .. s0 + 3 of the chunk and the 8 channels [8 cb, 8 cb + 8), from a raw bf16
// tile whose row j is token t0 - 3 + j (7 packed rows read once). tv: the 8
// channels' taps, 8 K consecutive floats (tap tau of channel e at e K + tau).
// Rows whose bit in `valid` is clear (at or past L) come out zero. fp16 results.
template <int K>
__device__ inline void conv4_rows(const bf16 *raw, int RP, int s0, int cb,
                                  const float __attribute__((ext_vector_type(4))) (&tv)[2 * K], unsigned valid,
                                  Raw8<f16> (&out)[4]) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 xr[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) xr[j] = *reinterpret_cast<const u32x4 *>(raw + (s0 + j) * RP + cb * 8);
    auto xval = [&](int j, int e) __attribute__((always_inline)) {
        const uint32_t w = xr[j][e >> 1];
        return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = 0.f;
#pragma unroll
            for (int tau = 0; tau < K; ++tau) acc = fmaf(tv[(e * K + tau) / 4][(e * K + tau) % 4], xval(r + 3 - tau, e), acc);
            h[e] = (f16)((valid >> r) & 1u ? acc : 0.f);
        }
        out[r].v[0] = __builtin_bit_cast(uint4, h);
    }
}

// BWD: the backward pass's preparation (gdn_bwd_impl.hpp): U~ row-major for
// every input type, no score fragments, and T stored as well.
// KT > 0: the short convolution with KT taps fused in front (bf16 forward only;
// q, k, v are raw inputs, see PrepArgs).
template <typename TI, int DK, int C, bool BWD = false, int KT = 0>
__global__ void __launch_bounds__(256, KT > 0 ? 3 : 4) gdn_prep_kernel(PrepArgs a) {
    constexpr bool CONV = KT > 0;
    using TM = typename OpOf<TI>::type;
    using MF = Mfma<TM>;
    using Cfg = PrepCfg<TM, DK, C, CONV>;
    static_assert(!CONV || (sizeof(TI) == 2 && !BWD), "the fused convolution: bf16 forward");
    constexpr int E = MF::E;
    constexpr int NW = 4;
    constexpr int NRB = C / 16;
    constexpr int KP = Cfg::KP, TP = Cfg::TP, OP = Cfg::OP;
    constexpr int NKS = DK / (4 * E);
    constexpr int NTK = C / (4 * E);
    static_assert(C == 64 && NRB == NW, "one 16-row diagonal block of T per wave: C = 64");
    // score fragments and U~ in the serial pass's accumulator layout: bf16 forward
    constexpr bool SC = sizeof(TI) == 2 && !BWD;

    __shared__ __attribute__((aligned(16))) char lds[Cfg::lds_bytes];
    TM *Ks = reinterpret_cast<TM *>(lds + Cfg::o_a);
    float *Tm = reinterpret_cast<float *>(lds + Cfg::o_a);   // after P is formed
    TM *KTs = reinterpret_cast<TM *>(lds + Cfg::o_a);        // after T is converted
    float *Pm = reinterpret_cast<float *>(lds + Cfg::o_p);
    TM *To = reinterpret_cast<TM *>(lds + Cfg::o_p);         // after T is complete
    float *Ysc = reinterpret_cast<float *>(lds + Cfg::o_c);
    TM *VTs = reinterpret_cast<TM *>(lds + Cfg::o_a);        // after W is formed
    float *Gs = reinterpret_cast<float *>(lds + Cfg::o_g);
    float *Bs = Gs + C;
    bf16 *Raw = reinterpret_cast<bf16 *>(lds + Cfg::o_p);    // CONV: raw rows, before P

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int bh = blockIdx.x / a.nchunks, c = blockIdx.x - bh * a.nchunks;
    const int t0 = c * C, L = a.L, dv = a.dv;
    const TI *kg = (const TI *)a.k + (size_t)bh * a.ld * DK;
    const TI *vg = (const TI *)a.v + (size_t)bh * a.ld * dv;
    const float *lgg = a.lg ? a.lg + (size_t)bh * a.ld : nullptr;
    const float *bg = a.beta + (size_t)bh * a.ld;

    // Every global load of the chunk is issued first (log-gate, beta, K and V
    // rows), so their latencies overlap. Staging unit u (one per thread) covers
    // four consecutive tokens of one 8-channel column block. Rows past the end
    // of the sequence are read from the last token (so every load is
    // unconditional) and then zeroed.
    const int tl = t0 + lane;
    const float lgv = (lgg && tl < L) ? lgg[tl] : 0.f;
    const float bv = (tl < L) ? bg[tl] : 0.f;
    constexpr int KCB = DK / 8, KCBL = KCB < 4 ? KCB : 4, KTQL = 16 / KCBL, KNCBG = KCB / KCBL;
    constexpr int KUNITS = (C / 4) * KCB;
    static_assert(KUNITS % 64 == 0 && KUNITS <= 256, "one K staging unit per thread, wave-uniform");
    const int VCB = dv / 8;
    const int VCBL = VCB < 4 ? VCB : 4, VTQL = 16 / VCBL, VNCBG = VCB / VCBL;
    const int VUNITS = (C / 4) * VCB;  // multiple of 64, at most 256, for dv in {32, 64, 128}
    const int gi = tid >> 4, l16 = tid & 15;
    const int ktq = (gi / KNCBG) * KTQL + (l16 % KTQL), kcb = (gi % KNCBG) * KCBL + (l16 / KTQL);
    const int vtq = (gi / VNCBG) * VTQL + (l16 % VTQL), vcb = (gi % VNCBG) * VCBL + (l16 / VTQL);
    // Score jobs of this wave (bf16 inputs): fragment (wv, 0), and on even waves
    // (3, 1) or (2, 1); their query rows are loaded here with the rest.
    const bool job1 = (wv & 1) == 0;
    const int jrb1 = wv == 0 ? 3 : 2;
    uint4 qx[2][NKS];
    if constexpr (SC && !CONV) {
        const TI *qg = (const TI *)a.q + (size_t)bh * a.ld * DK;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (j == 1 && !job1) break;
            const int t = t0 + (j ? jrb1 : wv) * 16 + n;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                qx[j][ks] = *reinterpret_cast<const uint4 *>(qg + (size_t)(t < L ? t : L - 1) * DK + g * (DK / 4) + ks * E);
        }
    }
    // K and V stay in their storage format until they are staged (fewer registers)
    Raw8<TI> kr[4], vr[4];
    // CONV: the convolved K and V rows of this thread's units, in fp16
    Raw8<f16> kc[4], vc[4];
    if constexpr (CONV) {
        // Each tensor's C rows plus HALO rows before the chunk pass through region
        // B as raw bf16 (rows before the sequence from the window, or zero; rows
        // at or past L are never used by a kept output); each thread then
        // convolves its staging unit's 4 rows x 8 channels from there.
        constexpr int HALO = Cfg::HALO, RP = Cfg::RP, RROWS = C + HALO;
        const int h = bh % a.H;
        constexpr int K = KT;
        // the raw rows of q, k and v are all loaded up front (their latencies
        // overlap); each tensor then passes through region B in turn
        constexpr int NMAX = (RROWS * 16 + 255) / 256;  // d <= 128
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        u32x4 rq[NMAX], rk[NMAX], rv[NMAX];
        auto load_raw = [&](int which, int d, u32x4 (&r)[NMAX]) __attribute__((always_inline)) {
            const bf16 *x = (const bf16 *)(which == 0 ? a.q : which == 1 ? a.k : a.v) + (size_t)bh * a.ld * d;
            const int seg = d / 8;
#pragma unroll
            for (int m = 0; m < NMAX; ++m) {
                const int idx = tid + 256 * m, row = idx / seg, sg = idx % seg, t = t0 - HALO + row;
                r[m] = *reinterpret_cast<const u32x4 *>(x + (size_t)min(max(t, 0), L - 1) * d + sg * 8);
            }
        };
        // rows before the sequence (chunk 0 only) come from the window, or are zero
        auto stage_raw = [&](int which, int d, const u32x4 (&r)[NMAX]) __attribute__((always_inline)) {
            const bf16 *win = (const bf16 *)a.cwin[which];
            const int seg = d / 8, tot = RROWS * seg;
#pragma unroll
            for (int m = 0; m < NMAX; ++m) {
                const int idx = tid + 256 * m, row = idx / seg, sg = idx % seg, t = t0 - HALO + row;
                if (idx >= tot) continue;
                u32x4 val = r[m];
                if (t < 0) {
                    val = u32x4{0u, 0u, 0u, 0u};
                    if (win && t >= -(K - 1))
                        val = *reinterpret_cast<const u32x4 *>(win + ((size_t)bh * (K - 1) + (K - 1) + t) * d + sg * 8);
                }
                *reinterpret_cast<u32x4 *>(Raw + row * RP + sg * 8) = val;
            }
        };
        // taps of a unit's 8 channels: 8 K consecutive floats, loaded as vectors
        // up front with the raw rows
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        auto load_taps = [&](int which, int d, int cb, f32x4v (&tv)[2 * K]) __attribute__((always_inline)) {
            const f32x4v *w = reinterpret_cast<const f32x4v *>(a.cw[which] + ((size_t)h * d + cb * 8) * K);
#pragma unroll
            for (int i = 0; i < 2 * K; ++i) tv[i] = w[i];
        };
        // loads run ahead of the convolution: the raw rows one tensor ahead, the
        // taps just before they are needed (registers)
        f32x4v tq[2 * K], tk[2 * K], tvv[2 * K];
        load_raw(1, DK, rk);
        if (tid < KUNITS) load_taps(1, DK, kcb, tk);
        load_raw(2, dv, rv);
        // K: convolved into kc, the workspace copy (fp16) and, below, the LDS tile
        stage_raw(1, DK, rk);
        __syncthreads();
        // bit r: token 4 tq + r of the chunk lies before L
        auto valid4 = [&](int tq) { return (unsigned)((1 << max(0, min(4, L - t0 - 4 * tq))) - 1); };
        if (tid < KUNITS) {
            conv4_rows<K>(Raw, RP, 4 * ktq, kcb, tk, valid4(ktq), kc);
            f16 *ko = (f16 *)a.kc + ((size_t)bh * a.Lp + t0) * DK;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<uint4 *>(ko + (size_t)(4 * ktq + r) * DK + 8 * kcb) = kc[r].v[0];
        }
        load_raw(0, DK, rq);
        if (tid < VUNITS) load_taps(2, dv, vcb, tvv);
        __syncthreads();
        // V: convolved into vc
        stage_raw(2, dv, rv);
        __syncthreads();
        if (tid < VUNITS) conv4_rows<K>(Raw, RP, 4 * vtq, vcb, tvv, valid4(vtq), vc);
        if (tid < KUNITS) load_taps(0, DK, kcb, tq);
        __syncthreads();
        // Q: convolved into the workspace copy, which the score jobs read back
        // after the next barrier
        stage_raw(0, DK, rq);
        __syncthreads();
        if (tid < KUNITS) {
            Raw8<f16> y[4];
            conv4_rows<K>(Raw, RP, 4 * ktq, kcb, tq, valid4(ktq), y);
            f16 *qo = (f16 *)a.qc + ((size_t)bh * a.Lp + t0) * DK;
#pragma unroll
            for (int r = 0; r < 4; ++r) *reinterpret_cast<uint4 *>(qo + (size_t)(4 * ktq + r) * DK + 8 * kcb) = y[r].v[0];
        }
        // (the barrier before the scores follows the K staging below)
    } else {
    if (tid < KUNITS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * ktq + r;
            kr[r] = ld_raw8<TI>(kg + (size_t)(t < L ? t : L - 1) * DK + 8 * kcb);
        }
    }
    if (tid < VUNITS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * vtq + r;
            vr[r] = ld_raw8<TI>(vg + (size_t)(t < L ? t : L - 1) * dv + 8 * vcb);
        }
    }
    }

    // Gates: inclusive scan of the chunk's log-gates (one token per lane).
    float G = lgv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(G, off, 64);
        if (lane >= off) G += y;
    }
    if (wv == 0) {
        Gs[lane] = G;
        Bs[lane] = bv;
    }

    // Stage K row-major (zero past the end of the sequence).
    if (CONV && tid < KUNITS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) *reinterpret_cast<uint4 *>(&Ks[(4 * ktq + r) * KP + 8 * kcb]) = kc[r].v[0];
    } else if (tid < KUNITS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = 4 * ktq + r;
            if (t0 + s >= L) {
#pragma unroll
                for (int i = 0; i < (int)(sizeof(TI) / 2); ++i) kr[r].v[i] = make_uint4(0u, 0u, 0u, 0u);
            }
            float kx[8];
            unpack8<TI>(kr[r], kx);
            st8<TM>(&Ks[s * KP + 8 * kcb], kx);
        }
    }
    __syncthreads();

    // P = strict_lower(diag(beta) (Gamma (.) K K^T)) from the 16x16 tiles rb >= sb,
    // taken as score jobs (rb, p): the tiles (rb, 2p) and (rb, 2p + 1) that lie on
    // or below the diagonal. Wave 0 takes (0, 0) and (3, 1), wave 1 (1, 0), wave 2
    // (2, 0) and (2, 1), wave 3 (3, 0): three, two, three and two tiles.
    // P tile D[r][s]: lane (g, n) holds r = rb*16 + 4g + e, s = sb*16 + n.
    // Score tile (bf16) D[s][r] = k_s . q_r: s = sb*16 + 4g + e, r = rb*16 + n; off
    // the diagonal block exp(G_r - G_s) = exp(G_r - G_e) exp(G_e - G_s), e the last
    // token of block sb (both factors <= 1).
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (j == 1 && !job1) break;
        const int rb = j ? jrb1 : wv, p = j;
        typename MF::frag qf[NKS];
        if constexpr (CONV) {
            const f16 *qrow = (const f16 *)a.qc + ((size_t)bh * a.Lp + t0 + rb * 16 + n) * DK + g * (DK / 4);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qf[ks] = ld_frag<TM>(qrow + ks * E);
        } else if constexpr (SC) {
            // bf16 -> fp16 with the packed round-toward-zero conversion (exact for
            // every bf16 value in fp16's normal range); rows past L are zero
            const bool valid = t0 + rb * 16 + n < L;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const uint32_t u[4] = {qx[j][ks].x, qx[j][ks].y, qx[j][ks].z, qx[j][ks].w};
                uint32_t h[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    h[i] = valid ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(u[i]), bf16_hi(u[i]))) : 0u;
                qf[ks] = __builtin_bit_cast(f16x8, make_uint4(h[0], h[1], h[2], h[3]));
            }
        }
        f32x4 ms[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int sb = 2 * p + hb;
            ms[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (sb > rb) continue;
            f32x4 d = {0.f, 0.f, 0.f, 0.f}, e4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const typename MF::frag kb = ld_frag<TM>(&Ks[(sb * 16 + n) * KP + g * (DK / 4) + ks * E]);
                d = MF::mma(ld_frag<TM>(&Ks[(rb * 16 + n) * KP + g * (DK / 4) + ks * E]), kb, d);
                if constexpr (SC) e4 = MF::mma(kb, qf[ks], e4);
            }
            {
                const int s = sb * 16 + n;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = rb * 16 + 4 * g + e;
                    Pm[r * TP + s] = (s < r) ? Bs[r] * __expf(Gs[r] - Gs[s]) * d[e] : 0.f;
                }
            }
            if constexpr (SC) {
                const int r = rb * 16 + n;
                const float Gr = Gs[r];
                if (sb == rb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = sb * 16 + 4 * g + e;
                        ms[hb][e] = (s > r) ? 0.f : e4[e] * __expf(Gr - Gs[s]);
                    }
                } else {
                    const float Ge = Gs[sb * 16 + 15];
                    const float fr = __expf(Gr - Ge);
#pragma unroll
                    for (int e = 0; e < 4; ++e) ms[hb][e] = e4[e] * (fr * __expf(Ge - Gs[sb * 16 + 4 * g + e]));
                }
            }
        }
        if constexpr (SC) {
            const int f = rb + (rb > 2 ? rb - 2 : 0) + p;
            f16 *mo = (f16 *)a.mf + (((size_t)bh * a.nchunks + c) * 6 + f) * 512 + lane * 8;
            *reinterpret_cast<f16x8 *>(mo) = pack_tiles(ms[0], ms[1], 1.f);
        }
    }
    __syncthreads();  // P complete; K row-major is dead from here (Tm reuses it)

    // T = (I + P)^-1, blocked by 16 rows. T is unit lower triangular, and so are
    // its diagonal blocks T_ii = (I + P_ii)^-1; the blocks below the diagonal
    // follow from (I + P) T = I as T_ij = -T_ii sum_{j <= k < i} P_ik T_kj.
    //
    // Diagonal blocks: wave w inverts block w by forward substitution, lane n
    // holding column n of the block in registers (the four lane groups compute
    // the same column; group 0 writes it).
    {
        // column by column: once T[s][n] is known it enters every later row's
        // sum, so the serial chain is one fma per row (each row's sum still
        // adds its terms in the order s = 0, 1, ...)
        const int base = 16 * wv;
        float tc[16], acc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            tc[s] = (s == n) ? 1.f : ((s < n) ? 0.f : -acc[s]);
#pragma unroll
            for (int r = s + 1; r < 16; ++r) acc[r] = fmaf(Pm[(base + r) * TP + base + s], tc[s], acc[r]);
        }
        if (g == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) Tm[(base + r) * TP + base + n] = tc[r];
        }
    }
    __syncthreads();

    // Below-diagonal block (i, j) on fp32 MFMA (16x16x4): Y = sum_k P_ik T_kj,
    // then T_ij = -T_ii Y. Y passes through a per-wave LDS tile to move from the
    // accumulator layout to the B-operand layout; LDS operations of one wave
    // complete in order, so the wave needs no barrier for it.
    auto below_block = [&](int i, int j) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int kb = j; kb < i; ++kb) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(Pm[(16 * i + n) * TP + 16 * kb + 4 * q + g],
                                                         Tm[(16 * kb + 4 * q + g) * TP + 16 * j + n], y,
                                                         0, 0, 0);
        }
        float *Y = Ysc + wv * 256;
#pragma unroll
        for (int e = 0; e < 4; ++e) Y[(4 * g + e) * 16 + n] = y[e];
        __builtin_amdgcn_wave_barrier();
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            t = __builtin_amdgcn_mfma_f32_16x16x4f32(Tm[(16 * i + n) * TP + 16 * i + 4 * q + g],
                                                     Y[(4 * q + g) * 16 + n], t, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Tm[(16 * i + 4 * g + e) * TP + 16 * j + n] = -t[e];
    };
    // Blocks one, two and three below the diagonal, each group after the last.
    if (wv < 3) below_block(wv + 1, wv);
    __syncthreads();
    if (wv < 2) below_block(wv + 2, wv);
    __syncthreads();
    if (wv == 0) below_block(3, 0);
    __syncthreads();  // T complete; P is dead from here (To reuses it)

    // T in the operand type, zero above the diagonal blocks (unrolled so that
    // the reads of a thread go out together).
#pragma unroll
    for (int i = 0; i < C * C / 256; ++i) {
        const int idx = tid + 256 * i;
        const int r = idx / C, s = idx % C;
        To[r * OP + s] = from_f32<TM>((s >> 4) > (r >> 4) ? 0.f : Tm[r * TP + s]);
    }
    __syncthreads();  // T converted: region A (T in fp32) is free
    if constexpr (BWD) {
        // T row-major, [bh][chunk][C][C] in the operand type (16 bytes per piece)
        constexpr int EP = 16 / (int)sizeof(TM);
        TM *tout = (TM *)a.t + ((size_t)bh * a.nchunks + c) * C * C;
#pragma unroll
        for (int i = 0; i < C * C / EP / 256; ++i) {
            const int idx = tid + 256 * i, r = idx / (C / EP), s0 = (idx % (C / EP)) * EP;
            *reinterpret_cast<uint4 *>(tout + r * C + s0) = *reinterpret_cast<const uint4 *>(&To[r * OP + s0]);
        }
    }

    // Stage K transposed scaled by beta_s a_s (zero past the end of the
    // sequence, where beta is zero too).
    if (tid < KUNITS) {
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = 4 * ktq + r;
            sc[r] = __shfl(bv, s, 64) * __expf(__shfl(G, s, 64));
        }
        float kx[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (CONV)
                unpack8<f16>(kc[r], kx[r]);
            else
                unpack8<TI>(kr[r], kx[r]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f32x4 col = {kx[0][e] * sc[0], kx[1][e] * sc[1], kx[2][e] * sc[2], kx[3][e] * sc[3]};
            st4<TM>(&KTs[tidx<C, TM>(8 * kcb + e, 4 * ktq)], col);
        }
    }
    __syncthreads();

    // W^T tiles D[ch][r] = sum_s (beta a K)[s][ch] T[r][s]; lane holds ch = cbk*16 + 4g + e.
    TM *wout = (TM *)a.w + ((size_t)bh * a.Lp + t0) * DK;
    for (int tile = wv; tile < (DK / 16) * NRB; tile += NW) {
        const int cbk = tile / NRB, rb = tile % NRB;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NTK; ++ks) {
            const int s0 = g * (C / 4) + ks * E;
            d = MF::mma(ld_frag<TM>(&KTs[tidx<C, TM>(cbk * 16 + n, s0)]),
                        ld_frag<TM>(&To[(rb * 16 + n) * OP + s0]), d);
        }
        st4<TM>(wout + (size_t)(rb * 16 + n) * DK + cbk * 16 + 4 * g, d);
    }
    __syncthreads();  // W formed: region A is free

    // Stage V transposed scaled by beta_s (zero past the end, where beta is zero).
    if (tid < VUNITS) {
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = __shfl(bv, 4 * vtq + r, 64);
        float vx[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (CONV)
                unpack8<f16>(vc[r], vx[r]);
            else
                unpack8<TI>(vr[r], vx[r]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f32x4 col = {vx[0][e] * sc[0], vx[1][e] * sc[1], vx[2][e] * sc[2], vx[3][e] * sc[3]};
            st4<TM>(&VTs[tidx<C, TM>(8 * vcb + e, 4 * vtq)], col);
        }
    }
    __syncthreads();

    const int NJB = dv / 16;
    if constexpr (SC) {
        // bf16 inputs: U~ in the accumulator layout of the serial pass
        // (gdn_fwd_impl.hpp), tiles D[r][j] = sum_s T[r][s] (beta V)[s][j]: lane
        // (g, n) holds rows r = rb*16 + 4g + e of column j = jb*16 + n, stored as
        // [bh][chunk][jb][rb][lane][4] so that the serial pass loads 8 bytes per
        // lane per row block.
        TM *uout = (TM *)a.ut + ((size_t)bh * a.nchunks + c) * NJB * (NRB * 256);
        for (int tile = wv; tile < NRB * NJB; tile += NW) {
            const int rb = tile / NJB, jb = tile % NJB;
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NTK; ++ks) {
                const int s0 = g * (C / 4) + ks * E;
                d = MF::mma(ld_frag<TM>(&To[(rb * 16 + n) * OP + s0]),
                            ld_frag<TM>(&VTs[tidx<C, TM>(jb * 16 + n, s0)]), d);
            }
            st4<TM>(uout + (size_t)(jb * NRB + rb) * 256 + lane * 4, d);
        }
    } else {
        // U~ row-major, from transposed tiles D[j][r] = sum_s (beta V)[s][j] T[r][s];
        // lane holds r = rb*16 + n and four consecutive columns j = jb*16 + 4g + e.
        TM *uout = (TM *)a.ut + ((size_t)bh * a.Lp + t0) * dv;
        for (int tile = wv; tile < NRB * NJB; tile += NW) {
            const int rb = tile / NJB, jb = tile % NJB;
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NTK; ++ks) {
                const int s0 = g * (C / 4) + ks * E;
                d = MF::mma(ld_frag<TM>(&VTs[tidx<C, TM>(jb * 16 + n, s0)]),
                            ld_frag<TM>(&To[(rb * 16 + n) * OP + s0]), d);
            }
            st4<TM>(uout + (size_t)(rb * 16 + n) * dv + jb * 16 + 4 * g, d);
        }
    }
}

template <typename TI, int DK, int C>
hipError_t launch_gdn_prep(const PrepArgs &a, hipStream_t st) {
    const int blocks = a.BH * a.nchunks;
    if constexpr (sizeof(TI) == 2) {
        if (a.cw[0]) {
            switch (a.K) {
                case 1: hipLaunchKernelGGL((gdn_prep_kernel<TI, DK, C, false, 1>), dim3(blocks), dim3(256), 0, st, a); break;
                case 2: hipLaunchKernelGGL((gdn_prep_kernel<TI, DK, C, false, 2>), dim3(blocks), dim3(256), 0, st, a); break;
                case 3: hipLaunchKernelGGL((gdn_prep_kernel<TI, DK, C, false, 3>), dim3(blocks), dim3(256), 0, st, a); break;
                case 4: hipLaunchKernelGGL((gdn_prep_kernel<TI, DK, C, false, 4>), dim3(blocks), dim3(256), 0, st, a); break;
                default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gdn_prep_kernel<TI, DK, C>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
