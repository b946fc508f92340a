// vdecay_bwd_impl.hpp -- backward pass of the per-key-channel decay (gfx950):
// bf16 inputs, fp16 MFMA operands (fp32 on the diagonal blocks), fp32
// accumulation and gradients.
//
// Method. Reverse mode of S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t
// (tensorplay "Talk Linear Attention", sections 5.1-5.2, the GLA gate; wln20
// "LLM注意力优化：线性注意力", Kimi Delta Attention section, the diagonal gate
// Diag(alpha_t)), in the chunk form of the forward kernel. For chunk c with the
// chunk-local per-channel cumulative log-gates G_r, the state H_c at its start
// and dH_c = dLoss/d(state at its end):
//   dq_r = e^{G_r} (.) H_c do_r + sum_{s<=r} (do_r . v_s) k_s (.) e^{G_r - G_s}
//   dk_s = sum_{r>=s} (do_r . v_s) q_r (.) e^{G_r - G_s} + e^{G_end - G_s} (.) dH_c v_s
//   dv_s = sum_{r>=s} A_rs do_r + dH_c^T (k_s (.) e^{G_end - G_s}),
//          A_rs = sum_c q_r[c] k_s[c] e^{G_r[c] - G_s[c]}
//   dH_{c-1} = Diag(e^{G_end}) dH_c + (Q (.) e^G)^T dO.
// The loss sees a chunk's gates only through q_r e^{G_r}, k_s e^{-G_s} and the
// factor Diag(e^{G_end}) of the state the chunk hands on, so, per channel,
//   dl_t = sum_{r>=t in the chunk} (q_r dq_r - k_r dk_r) + sum_j dH_c[.][j] H_{c+1}[.][j],
// H_{c+1} being the state at the chunk's end: the sum restarts at every chunk.
// The intra-chunk products split the chunk into four 16-token blocks. For a
// query block i after a key block j the decay factors as
//   e^{G_r - G_s} = e^{G_r - B_i} D_ij e^{E_j - G_s},  D_ij = e^{B_i - E_j},
// with B_i the cumulative gate just before block i and E_j the one at the last
// token of block j: every factor is at most 1, so fp16 operands
//   Qb_r = q_r e^{G_r - B_i},  Kb_s = k_s e^{E_j - G_s}  (D_ij applied per channel)
// hold them for any gate, and whatever underflows is negligible against the
// terms that matter. Then, with dP = dO V^T,
//   dq_r = e^{G_r - B_i} (.) [sum_{j<i} D_ij (.) sum_{s in j} dP_rs Kb_s + e^{B_i} (.) H_c do_r] + diag_r
//   dk_s = e^{E_j - G_s} (.) [sum_{i>j} D_ij (.) sum_{r in i} dP_rs Qb_r + e^{G_end - E_j} (.) dH_c v_s] + diag_s
// The diagonal blocks (r, s in the same block) carry factors of both signs; they
// are taken in fp32 on the MFMA (16x16x4), rebased around the block's middle
// token, whose factors stay below e^80 for gates >= -10 (the forward's
// argument), inside fp32's range: a reduced-precision operand there loses
// the accuracy of the large local terms (an emulation of bf16 operands gave
// 2.5e-2 of RMS on dq with gates spread over [-10, 0]).
// Gates below kMinChannelLogGate are taken at that value, as in the forward; the
// gradient reported for them is the one at the clamped value.
//
// Kernels:
//   vd_scans_kernel  the forward scan (H_c per chunk in fp16, transposed, and
//       the final state) and the reverse scan (dH_c per chunk, dS_0) in one
//       launch, one workgroup (4 waves) per (direction, head, value slice). Each
//       wave takes d_k / 4 channels of the chunk's rows (rows in lanes), scans
//       their gates and writes those channels of the scaled operand.
//   vd_bwd_grad_kernel  one workgroup (8 waves) per (head, chunk): waves w and
//       w + 4 own query block w (dq) and key block w (dk, dv), each for one half
//       of the output columns, and the gate gradient of block w over their dq
//       and dk channels.
#pragma once

#include <stdint.h>

#include "la_common.hpp"
#include "la_kernels.hpp"
#include "vdecay_fwd_impl.hpp"

namespace la {

// ---------------------------------------------------------------------------
// state scan over the chunks: S <- Diag(e^{G_end}) S + X^T Y with
// X = k (.) e^{G_end - G}, Y = v (forward) or X = q (.) e^{G}, Y = dO (backward).
template <int DK, int DVT, bool FWD>
__device__ __attribute__((always_inline)) inline void vd_scan(const BwdArgs &a, int blk, f16 *lds) {
    using MF = Mfma<f16>;
    using frag = MF::frag;
    constexpr int C = 64;
    constexpr int PX = DK + 16, PY = DVT + 16;
    constexpr int NTI = DK / 16, NTJ = DVT / 16, NTILE = NTI * NTJ, TPW = (NTILE + 3) / 4;
    constexpr int NTK = C / 32;
    constexpr int CW = DK / 4, NXU = CW / 8;  // channels per wave; 16-byte units of a row's share
    constexpr int SEGY = DVT / 8, NYS = (C * SEGY + 255) / 256;
    static_assert(CW % 8 == 0, "channel share");
    // double-buffered operand tiles: chunk it is staged into buffer it & 1, whose
    // last reader (chunk it - 2) is behind the barrier of chunk it - 1
    f16(*Xs)[C * PX] = reinterpret_cast<f16(*)[C * PX]>(lds);
    f16(*Ys)[C * PY] = reinterpret_cast<f16(*)[C * PY]>(lds + 2 * C * PX);
    float(*Eend)[DK] = reinterpret_cast<float(*)[DK]>(lds + 2 * C * (PX + PY));

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int bh = blk / a.nsplit, split = blk % a.nsplit;
    const int L = a.L, dv = a.dv, j0 = split * DVT, nchunks = (L + C - 1) / C;
    const bf16 *xg = (const bf16 *)(FWD ? a.k : a.q) + (size_t)bh * L * DK + wv * CW;
    const bf16 *yg = (const bf16 *)(FWD ? a.v : a.dout) + (size_t)bh * L * dv + j0;
    const float *lg = a.lg + (size_t)bh * L * DK + wv * CW;
    f16 *hs = (f16 *)(FWD ? a.hs : a.dhs) + (size_t)bh * nchunks * DK * dv;

    f32x4 Sacc[TPW];
    const float *s0 = FWD ? a.s_in : a.ds_out;
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        Sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile = wv + 4 * m;
        if (tile < NTILE && s0) {
            const int ti = tile / NTJ, tj = tile % NTJ;
            const float *sp = s0 + (size_t)bh * DK * dv + (size_t)(ti * 16 + 4 * g) * dv + j0 + tj * 16 + n;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[m][e] = sp[(size_t)e * dv];
        }
    }

    // Prefetch registers: chunk it + NSET is loaded while chunk it is folded in.
    // Every load is
    // unconditional (rows past the end re-read the last row; the masks kx, ky
    // zero them where the registers are used; chunks past the end re-read the
    // last one, unused), so the compiler counts the loads in flight exactly and
    // waits for a set only where it is used.
    constexpr int NSET = 1;  // register sets (two need more than 256 VGPRs)
    u32x4 rx[NSET][NXU];     // row `lane`: this wave's CW channels (bf16)
    u32x4 rg[NSET][CW / 4];  // their log-gates (fp32 bits)
    u32x4 ry[NSET][NYS];
    uint32_t kx[NSET], ky[NSET][NYS];
    auto chunk_of = [&](int it) __attribute__((always_inline)) {
        it = min(it, nchunks - 1);
        return FWD ? it : nchunks - 1 - it;
    };
    auto load = [&](auto set_tag, int it) __attribute__((always_inline)) {
        constexpr int P = decltype(set_tag)::value % NSET;
        const int t0 = chunk_of(it) * C, nv = min(C, L - t0);
        kx[P] = lane < nv ? 0xffffffffu : 0u;
        const size_t row = (size_t)(t0 + min(lane, nv - 1)) * DK;
        const u32x4 *py[NYS];
#pragma unroll
        for (int m = 0; m < NYS; ++m) {
            const int sid = min(tid + 256 * m, C * SEGY - 1), r = sid / SEGY;
            ky[P][m] = (tid + 256 * m < C * SEGY && r < nv) ? 0xffffffffu : 0u;
            py[m] = reinterpret_cast<const u32x4 *>(yg + (size_t)(t0 + min(r, nv - 1)) * dv + 8 * (sid % SEGY));
        }
        const u32x4 *px = reinterpret_cast<const u32x4 *>(xg + row);
        const u32x4 *pg = reinterpret_cast<const u32x4 *>(lg + row);
#pragma unroll
        for (int m = 0; m < NYS; ++m) ry[P][m] = *py[m];
#pragma unroll
        for (int u = 0; u < NXU; ++u) rx[P][u] = px[u];
#pragma unroll
        for (int u = 0; u < CW / 4; ++u) rg[P][u] = pg[u];
    };

    // chunk `it` of the scan from tile buffer B and register set B % NSET
    auto step = [&](auto set_tag, int it) __attribute__((always_inline)) {
        constexpr int B = decltype(set_tag)::value;  // tile buffer
        constexpr int P = B % NSET;                  // register set
        const int c = chunk_of(it);
        // the state this chunk starts from (forward) / ends at (backward), transposed
        f16 *hc = hs + (size_t)c * DK * dv;
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int tile = wv + 4 * m;
            if (NTILE % 4 == 0 || tile < NTILE) {
                const int ti = tile / NTJ, tj = tile % NTJ;
                st4<f16>(hc + (size_t)(j0 + tj * 16 + n) * DK + ti * 16 + 4 * g, Sacc[m]);
            }
        }
        // per channel: gate prefix over the rows (lanes), the chunk's total, and the
        // scaled operand row, staged 8 channels at a time
#pragma unroll
        for (int u = 0; u < NXU; ++u) {
            Raw8<bf16> r8;
            const u32x4 w = rx[P][u] & kx[P];
            r8.v[0] = make_uint4(w[0], w[1], w[2], w[3]);
            float x[8];
            unpack8<bf16>(r8, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = 8 * u + e;
                const float G =
                    wave_inclusive_sum(fmaxf(__uint_as_float(rg[P][i / 4][i % 4] & kx[P]), kMinChannelLogGate));
                const float gend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
                x[e] *= __expf(FWD ? gend - G : G);
                if (lane == 0) Eend[B][wv * CW + i] = __expf(gend);
            }
            st8<f16>(&Xs[B][lane * PX + wv * CW + 8 * u], x);
        }
#pragma unroll
        for (int m = 0; m < NYS; ++m) {
            const int sid = tid + 256 * m;
            if (sid < C * SEGY) {
                float y[8];
                Raw8<bf16> r8;
                const u32x4 w = ry[P][m] & ky[P][m];
                r8.v[0] = make_uint4(w[0], w[1], w[2], w[3]);
                unpack8<bf16>(r8, y);
                st8<f16>(&Ys[B][(sid / SEGY) * PY + 8 * (sid % SEGY)], y);
            }
        }
        // keep the loads after the last reads of this set: hoisted above them they
        // would need fresh registers, copied back at the loop head after a wait
        __builtin_amdgcn_sched_barrier(0);
        load(set_tag, it + NSET);
        __syncthreads();  // buffer B staged
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int tile = wv + 4 * m;
            if (NTILE % 4 == 0 || tile < NTILE) {
                const int ti = tile / NTJ, tj = tile % NTJ;
                Sacc[m] *= *reinterpret_cast<const f32x4 *>(&Eend[B][ti * 16 + 4 * g]);
#pragma unroll
                for (int ks = 0; ks < NTK; ++ks) {
                    const frag xa = tr_frag<PX>(Xs[B], 32 * ks + 4 * g, ti * 16, lane);
                    const frag yb = tr_frag<PY>(Ys[B], 32 * ks + 4 * g, tj * 16, lane);
                    Sacc[m] = MF::mma(xa, yb, Sacc[m]);
                }
            }
        }
    };

    // settle the initial state's loads, so that no load of the prologue is pending
    // at the loop head and the waits inside the loop count only the prefetch
    __builtin_amdgcn_s_waitcnt(0);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    if (nchunks > 0) {
        load(S0{}, 0);
        if constexpr (NSET == 2) load(S1{}, 1);
        int it = 0;
        for (; it + 1 < nchunks; it += 2) {
            step(S0{}, it);
            step(S1{}, it + 1);
        }
        if (it < nchunks) step(S0{}, it);
    }
    // forward: the final state S_L; backward: dLoss/dS_0
    float *out = FWD ? a.s_last : a.gs_in;
    if (out) {
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int tile = wv + 4 * m;
            if (tile < NTILE) {
                const int ti = tile / NTJ, tj = tile % NTJ;
                float *sp = out + (size_t)bh * DK * dv + (size_t)(ti * 16 + 4 * g) * dv + j0 + tj * 16 + n;
#pragma unroll
                for (int e = 0; e < 4; ++e) sp[(size_t)e * dv] = Sacc[m][e];
            }
        }
    }
}

// The two scans are independent; the forward one runs on the first BH * nsplit
// workgroups.
template <int DK, int DVT>
__global__ void __launch_bounds__(256) vd_scans_kernel(BwdArgs a) {
    // both directions' tiles: two buffers of X (C x (DK + 16)) and Y (C x (DVT + 16))
    // in fp16, then two rows of DK gate factors
    __shared__ __align__(16) f16 lds[2 * 64 * (DK + 16 + DVT + 16) + 4 * DK];
    // value slices of one head on one XCD: they share its rows and gates through that L2
    const int per = a.BH * a.nsplit, vid = xcd_virtual_block();
    if (vid < per)
        vd_scan<DK, DVT, true>(a, vid, lds);
    else
        vd_scan<DK, DVT, false>(a, vid - per, lds);
}

// ---------------------------------------------------------------------------
template <int DK, int DV> struct VdBwdCfg {
    static constexpr int C = 64;
    static constexpr int PK = DK + 16, PV = DV + 16, PG = DK + 4;
    static constexpr int NG = 512 / DK;  // thread groups of the <dH_c, H_{c+1}> sums
    static constexpr int NF = 14;        // factor rows
    static constexpr size_t GB = (size_t)C * PG * 4, HB = (size_t)DV * PK * 2;
    static constexpr size_t oRG = 0;  // G (fp32), later H_c^T (fp16)
    static constexpr size_t oDs = oRG + (GB > HB ? GB : HB);
    static constexpr size_t oQh = oDs + HB;  // raw q (bf16), later Qb (fp16)
    static constexpr size_t oKh = oQh + (size_t)C * PK * 2;
    static constexpr size_t oVs = oKh + (size_t)C * PK * 2;
    static constexpr size_t oOs = oVs + (size_t)C * PV * 2;
    static constexpr size_t oF = oOs + (size_t)C * PV * 2;
    static constexpr size_t oQK = oF + (size_t)NF * DK * 4;
    static constexpr size_t oBS = oQK + (size_t)C * 4;       // block totals of the gate gradient [4][DK]
    static constexpr size_t oBP = oBS + (size_t)4 * DK * 4;  // partial <dH_c, H_{c+1}> [NG][DK]
    static constexpr size_t oBD = oBP + (size_t)NG * DK * 4;
    static constexpr size_t BYTES = oBD + (size_t)DK * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Factor rows, per channel: e^{B_i} (FB + i), e^{G_end - E_j} (FE + j) and
// D_ij = e^{B_i - E_j} (FD + d_row(i, j), i > j), with B_i = G just before block i
// (0 for i = 0) and E_j = G at the last token of block j. Row fr is
// e^{G[ra] - G[rb]} with these rows (-1: 0).
__device__ constexpr int vdb_ra(int fr) {
    return fr == 0 ? -1 : fr < 4 ? 16 * fr - 1 : fr < 8 ? 63 : fr == 8 ? 15 : fr == 9 ? 31 : fr == 10 ? 47
         : fr == 11 ? 31 : 47;
}
__device__ constexpr int vdb_rb(int fr) {
    return fr < 4 ? -1 : fr < 8 ? 16 * (fr - 4) + 15 : fr < 11 ? 15 : fr < 13 ? 31 : 47;
}

// One workgroup per (head, chunk). Cross-block pairs (query block i > key block
// j) are taken with references at the block boundaries: Qb_r = q_r e^{G_r - B_i},
// Kb_s = k_s e^{E_j - G_s} and D_ij are all at most 1, so fp16 operands hold them
// for any gate (values that underflow are negligible against the terms that
// matter). The diagonal 16 x 16 blocks are taken in fp32 on the MFMA (16x16x4),
// rebased around the block's middle token m: its factors stay below e^80 for
// gates >= -10, inside fp32. Everything else is fp16 x fp16 -> fp32.
template <int DK, int DV>
__global__ void __launch_bounds__(512) vd_bwd_grad_kernel(BwdArgs a) {
    using Cfg = VdBwdCfg<DK, DV>;
    using MH = Mfma<f16>;
    using MS = Mfma<float>;
    using hfrag = MH::frag;
    constexpr int C = 64, NRB = 4, PK = Cfg::PK, PV = Cfg::PV, PG = Cfg::PG, NG = Cfg::NG, NF = Cfg::NF;
    constexpr int GW = DK / 8, SEGK = DK / 8, SEGV = DV / 8;
    constexpr int NKS_K = DK / 32, NKS_V = DV / 32;  // k-steps over d_k, d_v
    constexpr int NCW = DK / 32, NJW = DV / 32;      // 16-wide output tiles per half
    constexpr int NQ = (C * SEGK + 511) / 512, NVV = (C * SEGV + 511) / 512, NS = (DV * SEGK + 511) / 512;
    constexpr int RPG = DV / NG;
    constexpr int FB = 0, FE = 4, FD = 8;
    static_assert(RPG >= 1 && GW % 4 == 0, "shapes");

    __shared__ __align__(16) unsigned char smem[Cfg::BYTES];
    float *Gs = reinterpret_cast<float *>(smem + Cfg::oRG);
    f16 *Hs = reinterpret_cast<f16 *>(smem + Cfg::oRG);
    f16 *Ds = reinterpret_cast<f16 *>(smem + Cfg::oDs);
    uint16_t *Qr = reinterpret_cast<uint16_t *>(smem + Cfg::oQh);  // raw bf16 bits, then Qb
    uint16_t *Kr = reinterpret_cast<uint16_t *>(smem + Cfg::oKh);
    f16 *Qb = reinterpret_cast<f16 *>(smem + Cfg::oQh);
    f16 *Kb = reinterpret_cast<f16 *>(smem + Cfg::oKh);
    f16 *Vs = reinterpret_cast<f16 *>(smem + Cfg::oVs);
    f16 *Os = reinterpret_cast<f16 *>(smem + Cfg::oOs);
    float *F = reinterpret_cast<float *>(smem + Cfg::oF);
    float *QK = reinterpret_cast<float *>(smem + Cfg::oQK);
    float *BS = reinterpret_cast<float *>(smem + Cfg::oBS);
    float *BP = reinterpret_cast<float *>(smem + Cfg::oBP);
    float *BD = reinterpret_cast<float *>(smem + Cfg::oBD);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int L = a.L, nchunks = (L + C - 1) / C;
    const int bh = blockIdx.x / nchunks, c = blockIdx.x - bh * nchunks;
    const int t0 = c * C, nv = min(C, L - t0);
    const bf16 *qg = (const bf16 *)a.q + ((size_t)bh * L + t0) * DK;
    const bf16 *kg = (const bf16 *)a.k + ((size_t)bh * L + t0) * DK;
    const bf16 *vg = (const bf16 *)a.v + ((size_t)bh * L + t0) * DV;
    const bf16 *og = (const bf16 *)a.dout + ((size_t)bh * L + t0) * DV;
    const f16 *hg = (const f16 *)a.hs + ((size_t)bh * nchunks + c) * DK * DV;
    const f16 *dhg = (const f16 *)a.dhs + ((size_t)bh * nchunks + c) * DK * DV;

    // ---- 1. loads: q, k, v, dO rows, H_c^T, dH_c^T, and this wave's GW gate
    // channels of row `lane`
    Raw8<bf16> rq[NQ], rk[NQ], rv[NVV], ro[NVV];
    Raw8<f16> rh[NS], rd[NS];
    f32x4 gl[GW / 4];
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
        const int sid = tid + 512 * m, row = sid / SEGK, off = row * DK + 8 * (sid % SEGK);
        const bool ok = sid < C * SEGK && row < nv;
        rq[m] = ok ? ld_raw8<bf16>(qg + off) : zero_raw8<bf16>();
        rk[m] = ok ? ld_raw8<bf16>(kg + off) : zero_raw8<bf16>();
    }
#pragma unroll
    for (int m = 0; m < NVV; ++m) {
        const int sid = tid + 512 * m, row = sid / SEGV, off = row * DV + 8 * (sid % SEGV);
        const bool ok = sid < C * SEGV && row < nv;
        rv[m] = ok ? ld_raw8<bf16>(vg + off) : zero_raw8<bf16>();
        ro[m] = ok ? ld_raw8<bf16>(og + off) : zero_raw8<bf16>();
    }
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int sid = tid + 512 * m;
        if (sid < DV * SEGK) {
            const int off = (sid / SEGK) * DK + 8 * (sid % SEGK);
            rh[m] = ld_raw8<f16>(hg + off);
            rd[m] = ld_raw8<f16>(dhg + off);
        }
    }
#pragma unroll
    for (int u = 0; u < GW / 4; ++u)
        gl[u] = lane < nv ? *reinterpret_cast<const f32x4 *>(a.lg + ((size_t)bh * L + t0 + lane) * DK + wv * GW + 4 * u)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
    // <dH_c, H_{c+1}> per channel: thread (channel tid % DK) over RPG state rows;
    // H_{c+1} is the next chunk's stored start state, or the final state
    {
        const int ch = tid % DK, grp = tid / DK;
        float acc = 0.f;
        if (c + 1 < nchunks) {
            const f16 *hn = hg + (size_t)DK * DV;
#pragma unroll
            for (int i = 0; i < RPG; ++i) {
                const int j = grp * RPG + i;
                acc += (float)dhg[j * DK + ch] * (float)hn[j * DK + ch];
            }
        } else {
            const float *sl = a.s_last + (size_t)bh * DK * DV + (size_t)ch * DV;
#pragma unroll
            for (int i = 0; i < RPG; ++i) {
                const int j = grp * RPG + i;
                acc += (float)dhg[j * DK + ch] * sl[j];
            }
        }
        BP[grp * DK + ch] = acc;
    }

    // ---- 2. V, dO, dH_c^T and the raw q, k rows into LDS; the exact diagonal
    // scores q_t . k_t; the gate prefix of this wave's channels (rows in lanes)
    // and their factor rows
    auto put = [&](const Raw8<bf16> &r, f16 *dst) __attribute__((always_inline)) {
        float x[8];
        unpack8<bf16>(r, x);
        st8<f16>(dst, x);
    };
#pragma unroll
    for (int m = 0; m < NVV; ++m) {
        const int sid = tid + 512 * m;
        if (sid < C * SEGV) {
            const int o = (sid / SEGV) * PV + 8 * (sid % SEGV);
            put(rv[m], &Vs[o]);
            put(ro[m], &Os[o]);
        }
    }
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int sid = tid + 512 * m;
        if (sid < DV * SEGK) *reinterpret_cast<uint4 *>(&Ds[(sid / SEGK) * PK + 8 * (sid % SEGK)]) = rd[m].v[0];
    }
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
        const int sid = tid + 512 * m;
        if (sid < C * SEGK) {
            const int row = sid / SEGK, o = row * PK + 8 * (sid % SEGK);
            *reinterpret_cast<uint4 *>(&Qr[o]) = rq[m].v[0];
            *reinterpret_cast<uint4 *>(&Kr[o]) = rk[m].v[0];
            float q8[8], k8[8];
            unpack8<bf16>(rq[m], q8);
            unpack8<bf16>(rk[m], k8);
            float qk = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) qk += q8[e] * k8[e];
#pragma unroll
            for (int off = 1; off < SEGK; off <<= 1) qk += __shfl_xor(qk, off, 64);
            if (sid % SEGK == 0) QK[row] = qk;
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
    {
        const int fr = lane & 15, ra = vdb_ra(fr), rb = vdb_rb(fr);
#pragma unroll
        for (int it = 0; it < GW / 4; ++it) {
            const int ch = wv * GW + (lane >> 4) + 4 * it;
            if (fr < NF) {
                const float xa = ra < 0 ? 0.f : Gs[ra * PG + ch];
                const float xb = rb < 0 ? 0.f : Gs[rb * PG + ch];
                F[fr * DK + ch] = __expf(xa - xb);
            }
        }
    }
    __syncthreads();

    // ---- 3. the diagonal blocks in fp32, the per-position factors, and the
    // boundary-referenced operands (staging layout, into registers)
    const int w = wv & 3, half = wv >> 2;
    const int r = 16 * w + n;  // this lane's token: query row of dq, key row of dk and dv
    const int mid = 16 * w + 8;
    auto rawf = [&](const uint16_t *X, int idx) __attribute__((always_inline)) -> float {
        return __uint_as_float((uint32_t)X[idx] << 16);
    };
    auto nat16 = [&](const f16 *X, int P, int row, int ks, int KW) __attribute__((always_inline)) -> hfrag {
        return ld_frag<f16>(&X[row * P + g * (KW / 4) + ks * 8]);
    };
    auto trn16 = [&](const f16 *X, int P, int row, int ks) __attribute__((always_inline)) -> hfrag {
        const f16x4 lo = *reinterpret_cast<const f16x4 *>(&X[row * P + 32 * ks + 4 * g]);
        const f16x4 hi = *reinterpret_cast<const f16x4 *>(&X[row * P + 32 * ks + 16 + 4 * g]);
        return hfrag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    f32x4 dqD[NCW], dkD[NCW], atD;
    float E1[NCW][4], E2[NCW][4];
    {
        // dP of the diagonal block both ways: pt[e] = dP[r][16w + 4g + e] (rows s),
        // pk[e] = dP[16w + 4g + e][r] (rows r'), column r = 16w + n
        f32x4 pt = {0.f, 0.f, 0.f, 0.f}, pk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS_V; ++ks) {
            const hfrag vr = nat16(Vs, PV, r, ks, DV), orow = nat16(Os, PV, r, ks, DV);
            pt = MH::mma(vr, orow, pt);
            pk = MH::mma(orow, vr, pk);
        }
        // B operands of the 16x16x4 steps t: lane (g, n) takes element g of lane (t, n)
        float bq[4], bk[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float xq[4], xk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xq[e] = __shfl(pt[e], t * 16 + n, 64);
                xk[e] = __shfl(pk[e], t * 16 + n, 64);
            }
            const float vq = g == 0 ? xq[0] : g == 1 ? xq[1] : g == 2 ? xq[2] : xq[3];
            const float vk = g == 0 ? xk[0] : g == 1 ? xk[1] : g == 2 ? xk[2] : xk[3];
            bq[t] = (4 * t + g <= n) ? vq : 0.f;  // dP[r][s], s = 16w + 4t + g <= r
            bk[t] = (4 * t + g >= n) ? vk : 0.f;  // dP[r'][s], r' = 16w + 4t + g >= s = r
        }
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int ct = half * NCW + q_, ch = ct * 16 + n, c4 = ct * 16 + 4 * g;
            const float gm = Gs[mid * PG + ch];
            f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int u = 16 * w + 4 * t + g;
                const float d = Gs[u * PG + ch] - gm;
                aq = MS::mma(rawf(Kr, u * PK + ch) * __expf(-d), bq[t], aq);  // k_u e^{G_m - G_u}
                ak = MS::mma(rawf(Qr, u * PK + ch) * __expf(d), bk[t], ak);   // q_u e^{G_u - G_m}
            }
            const f32x4 gr = *reinterpret_cast<const f32x4 *>(&Gs[r * PG + c4]);
            const f32x4 gmv = *reinterpret_cast<const f32x4 *>(&Gs[mid * PG + c4]);
            const f32x4 gb = w > 0 ? *reinterpret_cast<const f32x4 *>(&Gs[(16 * w - 1) * PG + c4])
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
            const f32x4 ge = *reinterpret_cast<const f32x4 *>(&Gs[(16 * w + 15) * PG + c4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dqD[q_][e] = aq[e] * __expf(gr[e] - gmv[e]);
                dkD[q_][e] = ak[e] * __expf(gmv[e] - gr[e]);
                E1[q_][e] = __expf(gr[e] - gb[e]);
                E2[q_][e] = __expf(ge[e] - gr[e]);
            }
        }
        // A of the diagonal block: rows r' = 16w + 4g + e, column s = r, over all
        // channels c = 4t + g: q_{16w+n}[c] x and k_{16w+n}[c] / x, x = e^{G - G_m}
        atD = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int t = 0; t < DK / 4; ++t) {
            const int ch = 4 * t + g;
            const float x = __expf(Gs[r * PG + ch] - Gs[mid * PG + ch]);
            // a hardware reciprocal: a correctly rounded divide costs ten instructions
            atD = MS::mma(rawf(Qr, r * PK + ch) * x, rawf(Kr, r * PK + ch) * __builtin_amdgcn_rcpf(x), atD);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rr = 16 * w + 4 * g + e;
            if (rr < r) atD[e] = 0.f;
            if (rr == r) atD[e] = QK[r];  // the undecayed diagonal, exact
        }
    }
    float qb[NQ][8], kb[NQ][8];
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
        const int sid = tid + 512 * m;
        if (sid < C * SEGK) {
            const int row = sid / SEGK, c0 = 8 * (sid % SEGK), blk = row >> 4;
            float q8[8], k8[8];
            unpack8<bf16>(rq[m], q8);
            unpack8<bf16>(rk[m], k8);
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                const f32x4 gr = *reinterpret_cast<const f32x4 *>(&Gs[row * PG + c0 + 4 * h4]);
                const f32x4 gb = blk > 0 ? *reinterpret_cast<const f32x4 *>(&Gs[(16 * blk - 1) * PG + c0 + 4 * h4])
                                         : f32x4{0.f, 0.f, 0.f, 0.f};
                const f32x4 ge = *reinterpret_cast<const f32x4 *>(&Gs[(16 * blk + 15) * PG + c0 + 4 * h4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qb[m][4 * h4 + e] = q8[4 * h4 + e] * __expf(gr[e] - gb[e]);
                    kb[m][4 * h4 + e] = k8[4 * h4 + e] * __expf(ge[e] - gr[e]);
                }
            }
        }
    }
    __syncthreads();  // every read of G and of the raw rows is done

    // ---- 4. Qb, Kb over the raw rows; H_c^T over G; <dH_c, H_{c+1}>
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
        const int sid = tid + 512 * m;
        if (sid < C * SEGK) {
            const int o = (sid / SEGK) * PK + 8 * (sid % SEGK);
            st8<f16>(&Qb[o], qb[m]);
            st8<f16>(&Kb[o], kb[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int sid = tid + 512 * m;
        if (sid < DV * SEGK) *reinterpret_cast<uint4 *>(&Hs[(sid / SEGK) * PK + 8 * (sid % SEGK)]) = rh[m].v[0];
    }
    if (tid < DK) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NG; ++i) s += BP[i * DK + tid];
        BD[tid] = s;
    }
    __syncthreads();

    // ---- 5. cross-block pairs and the state terms (fp16 operands)
    auto tok16 = [&](const f16 *X, int ks, int col0) __attribute__((always_inline)) -> hfrag {
        return tr_frag<PK>(X, 32 * ks + 4 * g, col0, lane);
    };
    // elements 0..3 scaled by f0, 4..7 by f1
    auto scl2 = [&](hfrag x, float f0, float f1) __attribute__((always_inline)) -> hfrag {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = (f16)((float)x[e] * f0);
            x[4 + e] = (f16)((float)x[4 + e] * f1);
        }
        return x;
    };
    float dG[NCW][4];
    const bool live = r < nv;

    // dq, query block w: dQ^T[c][r] = E1 (aI + e^{B_w} aH) + diagonal block
    {
        f32x4 aI[NCW], aH[NCW];
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int ct = half * NCW + q_;
            aH[q_] = f32x4{0.f, 0.f, 0.f, 0.f};
            aI[q_] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS_V; ++ks)
                aH[q_] = MH::mma(tr_frag<PK>(Hs, 32 * ks + 4 * g, ct * 16, lane), trn16(Os, PV, r, ks), aH[q_]);
        }
        // dP^T tiles D[s][r] = sum_j V[s][j] dO[r][j] for key blocks sb < w
        f32x4 dpt[NRB];
#pragma unroll
        for (int sb = 0; sb < NRB; ++sb) {
            dpt[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (sb < w) {
#pragma unroll
                for (int ks = 0; ks < NKS_V; ++ks)
                    dpt[sb] = MH::mma(nat16(Vs, PV, sb * 16 + n, ks, DV), nat16(Os, PV, r, ks, DV), dpt[sb]);
            }
        }
#pragma unroll
        for (int p = 0; p < NRB / 2; ++p) {
            if (2 * p < w) {
                const hfrag b = pack_tiles(dpt[2 * p], dpt[2 * p + 1], 1.f);
#pragma unroll
                for (int q_ = 0; q_ < NCW; ++q_) {
                    const int ct = half * NCW + q_, ch = ct * 16 + n;
                    const float f0 = F[(FD + d_row(w, 2 * p)) * DK + ch];
                    const float f1 = 2 * p + 1 < w ? F[(FD + d_row(w, 2 * p + 1)) * DK + ch] : 0.f;
                    aI[q_] = MH::mma(scl2(tok16(Kb, p, ct * 16), f0, f1), b, aI[q_]);
                }
            }
        }
        float *dqg = a.gq + ((size_t)bh * L + t0 + r) * DK;
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int c4 = (half * NCW + q_) * 16 + 4 * g;
            const f32x4 fb = *reinterpret_cast<const f32x4 *>(&F[(FB + w) * DK + c4]);
            const f32x4 qv = live ? ld4<bf16>(qg + (size_t)r * DK + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = E1[q_][e] * (aI[q_][e] + fb[e] * aH[q_][e]) + dqD[q_][e];
                dG[q_][e] = qv[e] * x[e];
            }
            if (live) *reinterpret_cast<f32x4 *>(dqg + c4) = x;
        }
    }

    // dk, key block w: dK^T[c][s] = E2 (aI + e^{G_end - E_w} aH) + diagonal block
    {
        f32x4 aI[NCW], aH[NCW];
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int ct = half * NCW + q_;
            aH[q_] = f32x4{0.f, 0.f, 0.f, 0.f};
            aI[q_] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS_V; ++ks)
                aH[q_] = MH::mma(tr_frag<PK>(Ds, 32 * ks + 4 * g, ct * 16, lane), trn16(Vs, PV, r, ks), aH[q_]);
        }
        // dP tiles D[r'][s] = sum_j dO[r'][j] V[s][j] for query blocks rbk > w
        f32x4 dp[NRB];
#pragma unroll
        for (int rbk = 0; rbk < NRB; ++rbk) {
            dp[rbk] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (rbk > w) {
#pragma unroll
                for (int ks = 0; ks < NKS_V; ++ks)
                    dp[rbk] = MH::mma(nat16(Os, PV, rbk * 16 + n, ks, DV), nat16(Vs, PV, r, ks, DV), dp[rbk]);
            }
        }
#pragma unroll
        for (int p = 0; p < NRB / 2; ++p) {
            if (2 * p + 1 > w) {
                const hfrag b = pack_tiles(dp[2 * p], dp[2 * p + 1], 1.f);
#pragma unroll
                for (int q_ = 0; q_ < NCW; ++q_) {
                    const int ct = half * NCW + q_, ch = ct * 16 + n;
                    const float f0 = 2 * p > w ? F[(FD + d_row(2 * p, w)) * DK + ch] : 0.f;
                    const float f1 = F[(FD + d_row(2 * p + 1, w)) * DK + ch];
                    aI[q_] = MH::mma(scl2(tok16(Qb, p, ct * 16), f0, f1), b, aI[q_]);
                }
            }
        }
        float *dkg = a.gk + ((size_t)bh * L + t0 + r) * DK;
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int c4 = (half * NCW + q_) * 16 + 4 * g;
            const f32x4 fe = *reinterpret_cast<const f32x4 *>(&F[(FE + w) * DK + c4]);
            const f32x4 kv = live ? ld4<bf16>(kg + (size_t)r * DK + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = E2[q_][e] * (aI[q_][e] + fe[e] * aH[q_][e]) + dkD[q_][e];
                dG[q_][e] -= kv[e] * x[e];
            }
            if (live) *reinterpret_cast<f32x4 *>(dkg + c4) = x;
        }
    }

    // dv, key block w: dV^T[j][s] = sum_c dH[c][j] Kb[s][c] e^{G_end - E_w}[c]
    //                              + sum_r' dO[r'][j] A[r'][s]
    {
        hfrag kw[NKS_K];
#pragma unroll
        for (int ks = 0; ks < NKS_K; ++ks) {
            const int cb = g * (DK / 4) + 8 * ks;
            const hfrag kr = nat16(Kb, PK, r, ks, DK);
            const f32x4 fa = *reinterpret_cast<const f32x4 *>(&F[(FE + w) * DK + cb]);
            const f32x4 fc = *reinterpret_cast<const f32x4 *>(&F[(FE + w) * DK + cb + 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kw[ks][e] = (f16)((float)kr[e] * fa[e]);
                kw[ks][4 + e] = (f16)((float)kr[4 + e] * fc[e]);
            }
        }
        f32x4 acc[NJW];
#pragma unroll
        for (int q_ = 0; q_ < NJW; ++q_) {
            const int jt = half * NJW + q_;
            acc[q_] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS_K; ++ks) acc[q_] = MH::mma(nat16(Ds, PK, jt * 16 + n, ks, DK), kw[ks], acc[q_]);
        }
        // A tiles D[r'][s] = sum_c Qb[r'][c] Kb[s][c] D_{rbk,w}[c] for query blocks rbk > w
        f32x4 at[NRB];
#pragma unroll
        for (int rbk = 0; rbk < NRB; ++rbk) {
            at[rbk] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (rbk > w) {
#pragma unroll
                for (int ks = 0; ks < NKS_K; ++ks) {
                    const int cb = g * (DK / 4) + 8 * ks;
                    const float *Dr = &F[(FD + d_row(rbk, w)) * DK + cb];
                    const f32x4 da = *reinterpret_cast<const f32x4 *>(Dr);
                    const f32x4 db = *reinterpret_cast<const f32x4 *>(Dr + 4);
                    hfrag kd = nat16(Kb, PK, r, ks, DK);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kd[e] = (f16)((float)kd[e] * da[e]);
                        kd[4 + e] = (f16)((float)kd[4 + e] * db[e]);
                    }
                    at[rbk] = MH::mma(nat16(Qb, PK, rbk * 16 + n, ks, DK), kd, at[rbk]);
                }
            } else if (rbk == w) {
                at[rbk] = atD;
            }
        }
#pragma unroll
        for (int p = 0; p < NRB / 2; ++p) {
            if (2 * p + 1 >= w) {
                const hfrag b = pack_tiles(at[2 * p], at[2 * p + 1], 1.f);
#pragma unroll
                for (int q_ = 0; q_ < NJW; ++q_)
                    acc[q_] = MH::mma(tr_frag<PV>(Os, 32 * p + 4 * g, (half * NJW + q_) * 16, lane), b, acc[q_]);
            }
        }
        float *dvg = a.gv + ((size_t)bh * L + t0 + r) * DV;
        if (live) {
#pragma unroll
            for (int q_ = 0; q_ < NJW; ++q_)
                *reinterpret_cast<f32x4 *>(dvg + (half * NJW + q_) * 16 + 4 * g) = acc[q_];
        }
    }

    // ---- 6. gate gradient: suffix over the block's tokens (the 16 lanes of each
    // lane group), then the later blocks' totals and <dH_c, H_{c+1}>
#pragma unroll
    for (int q_ = 0; q_ < NCW; ++q_) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = dG[q_][e];
            x += dpp_f32<0x101>(0.f, x);
            x += dpp_f32<0x102>(0.f, x);
            x += dpp_f32<0x104>(0.f, x);
            x += dpp_f32<0x108>(0.f, x);
            dG[q_][e] = x;
        }
        if (n == 0) {
            const int c4 = (half * NCW + q_) * 16 + 4 * g;
            *reinterpret_cast<f32x4 *>(&BS[w * DK + c4]) = f32x4{dG[q_][0], dG[q_][1], dG[q_][2], dG[q_][3]};
        }
    }
    __syncthreads();
    if (a.glg && live) {
        float *dlg = a.glg + ((size_t)bh * L + t0 + r) * DK;
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int c4 = (half * NCW + q_) * 16 + 4 * g;
            f32x4 x = *reinterpret_cast<const f32x4 *>(&BD[c4]);
            for (int b2 = w + 1; b2 < NRB; ++b2) x += *reinterpret_cast<const f32x4 *>(&BS[b2 * DK + c4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] += dG[q_][e];
            *reinterpret_cast<f32x4 *>(dlg + c4) = x;
        }
    }
}

template <int DK, int DV>
hipError_t launch_vdecay_bwd(const BwdArgs &a, hipStream_t st) {
    constexpr int DVT = DV >= 64 ? 64 : DV;  // value slices of the state scans
    const int nchunks = (a.L + 63) / 64;
    BwdArgs b = a;
    b.nsplit = DV / DVT;
    hipLaunchKernelGGL((vd_scans_kernel<DK, DVT>), dim3(2 * a.BH * b.nsplit), dim3(256), 0, st, b);
    if (nchunks > 0)
        hipLaunchKernelGGL((vd_bwd_grad_kernel<DK, DV>), dim3(a.BH * nchunks), dim3(512), 0, st, b);
    return hipGetLastError();
}

}  // namespace la
