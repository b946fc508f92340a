// kda_prep_impl.hpp -- chunk-parallel preparation for Kimi Delta Attention
// (gfx950, bf16 inputs).
//
// Method. KDA is the gated delta rule with the scalar gate widened to one gate
// per key channel (wln20 "LLM注意力优化：线性注意力", Kimi Delta Attention section):
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
// in the d_k x d_v orientation. It rewrites as S_t = Diag(alpha_t) S_{t-1} + k_t u_t^T
// with u_t = beta_t (v_t - S_{t-1}^T (alpha_t (.) k_t)). Within a chunk with the
// per-channel cumulative log-gates G_r and Gam_r = exp(G_r), unrolling S_{t-1}
// from the chunk's initial state S_0 gives
//   S_{t-1}^T (alpha_t (.) k_t) = S_0^T (Gam_t (.) k_t) + sum_{s<t} u_s A_ts,
//   A_ts = sum_c k_t[c] k_s[c] exp(G_t[c] - G_s[c]),
// so, as for the scalar gate (tensorplay "Talk Linear Attention", section 6.2,
// the WY / UT form), with P = strict_lower(diag(beta) A) and T = (I + P)^-1:
//   W = T diag(beta) (K (.) Gam),  U~ = T diag(beta) V,  U = U~ - W S_0,
//   O = (Q (.) Gam) S_0 + M U,      M_rs = sum_c q_r[c] k_s[c] exp(G_r[c] - G_s[c]) (s <= r),
//   S_C = Diag(Gam_C) S_0 + (K (.) Gam_C / Gam)^T U.
// This kernel computes everything that does not depend on S_0, one workgroup
// per chunk: W, U~ and the score fragments M in the layouts of the delta rule's
// serial pass (gdn_fwd_impl.hpp), the pre-scaled queries Q (.) Gam and keys
// K (.) Gam_C / Gam (fp16, [BH, Lp, DK]), and the chunk's state decay Gam_C
// ([BH, nchunks, DK]). The serial pass then runs as for the delta rule without
// a scalar gate, with the state's rows decayed by Gam_C.
//
// The decay inside A and M no longer factors out of the dot products. The
// chunk's four 16-token blocks are taken as in the per-channel decay's backward
// (vdecay_bwd_impl.hpp): for a query block i after a key block j,
//   exp(G_t - G_s) = exp(G_t - B_i) D_ij exp(E_j - G_s),  D_ij = exp(B_i - E_j),
// B_i the gate sum just before block i and E_j the one at block j's last token;
// every factor is at most 1, so fp16 operands hold them for any gate. The
// diagonal blocks carry factors of both signs; they are taken in fp32 on the
// MFMA (16x16x4), rebased around the block's middle token m (factors below
// e^80 for gates >= -10; gates below are taken as -10, as in the forward of
// the per-channel decay).
//
// Mapping. 256 threads; wave w owns tokens 16w .. 16w + 15 of the chunk, lane
// (g, n) token 16w + n and the quarter g of its key channels and value columns,
// which it loads, rebases, writes and feeds to the MFMA itself. The gate prefix
// takes the chunk's tokens in lanes instead (wave w: a quarter of the channels).
#pragma once

#include "la_common.hpp"
#include "la_kernels.hpp"
#include "vdecay_fwd_impl.hpp"

namespace la {

template <int DK> struct KdaPrepCfg {
    static constexpr int C = 64;
    static constexpr int PG = DK + 4;   // fp32 G pitch
    static constexpr int TP = C + 1;    // fp32 P and T pitch
    static constexpr int OP = C + 8;    // fp16 T pitch
    static constexpr int PK = DK + 16;  // fp16 rebased keys / (beta Gam K) pitch
    static constexpr int PV = 128 + 16; // fp16 beta V pitch (any d_v <= 128)
    static constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }
    static constexpr size_t up16(size_t x) { return (x + 15) / 16 * 16; }
    // R_G: G (fp32), then T (fp32); R_A: K (.) exp(E - G), then beta Gam K, then
    // beta V (fp16); R_P: P (fp32), then T (fp16); factor rows D_ij; scratch of
    // the off-diagonal blocks of T.
    static constexpr size_t o_g = 0;
    static constexpr size_t o_a = o_g + up16(cmax((size_t)C * PG * 4, (size_t)C * TP * 4));
    static constexpr size_t o_p = o_a + up16(cmax((size_t)C * PK * 2, (size_t)C * PV * 2));
    static constexpr size_t o_f = o_p + up16(cmax((size_t)C * TP * 4, (size_t)C * OP * 2));
    static constexpr size_t o_y = o_f + (size_t)6 * DK * 4;
    static constexpr size_t bytes = o_y + 4 * 256 * 4;
    static_assert(bytes <= 80 * 1024, "two workgroups per CU");
};

template <int DK>
__global__ void __launch_bounds__(256, 2) kda_prep_kernel(PrepArgs a) {
    using Cfg = KdaPrepCfg<DK>;
    using MF = Mfma<f16>;
    using frag = MF::frag;
    constexpr int C = 64, NRB = 4;
    constexpr int PG = Cfg::PG, TP = Cfg::TP, OP = Cfg::OP, PK = Cfg::PK, PV = Cfg::PV;
    constexpr int CQ = DK / 4, NU = CQ / 8;  // channels per lane; 8-channel units
    constexpr int GW = DK / 4;               // gate channels per wave (prefix)
    static_assert(NU >= 1, "d_k >= 32");

    __shared__ __attribute__((aligned(16))) char lds[Cfg::bytes];
    float *Gs = reinterpret_cast<float *>(lds + Cfg::o_g);
    float *Tm = reinterpret_cast<float *>(lds + Cfg::o_g);   // after P is formed
    f16 *Ra = reinterpret_cast<f16 *>(lds + Cfg::o_a);
    float *Pm = reinterpret_cast<float *>(lds + Cfg::o_p);
    f16 *To = reinterpret_cast<f16 *>(lds + Cfg::o_p);       // after T is complete
    float *F = reinterpret_cast<float *>(lds + Cfg::o_f);
    float *Ysc = reinterpret_cast<float *>(lds + Cfg::o_y);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int bh = blockIdx.x / a.nchunks, c = blockIdx.x - bh * a.nchunks;
    const int t0 = c * C, L = a.L, dv = a.dv, VQ = dv / 4;
    const int tr = 16 * wv + n, t = t0 + tr;  // this lane's token
    const bool valid = t < L;
    const size_t row = (size_t)bh * a.ld + (valid ? t : L - 1);
    const bf16 *qp = (const bf16 *)a.q + row * DK + g * CQ;
    const bf16 *kp = (const bf16 *)a.k + row * DK + g * CQ;
    const bf16 *vp = (const bf16 *)a.v + row * dv + g * VQ;

    // ---- loads: this lane's q, k and v slices, its beta, and (tokens in lanes)
    // the gates of this wave's channel quarter; rows past L read the last token
    // and are zeroed
    uint4 qr[NU], kr[NU], vr[4];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        qr[u] = reinterpret_cast<const uint4 *>(qp)[u];
        kr[u] = reinterpret_cast<const uint4 *>(kp)[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (8 * u < VQ) vr[u] = reinterpret_cast<const uint4 *>(vp)[u];
    const float bv = valid ? a.beta[row] : 0.f;
    const int tg = t0 + lane;
    const float *gp = a.lg + ((size_t)bh * a.ld + (tg < L ? tg : L - 1)) * DK + wv * GW;
    f32x4 gl[GW / 4];
#pragma unroll
    for (int i = 0; i < GW / 4; ++i) gl[i] = *reinterpret_cast<const f32x4 *>(gp + 4 * i);
    if (!valid) {
#pragma unroll
        for (int u = 0; u < NU; ++u) qr[u] = kr[u] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int u = 0; u < 4; ++u) vr[u] = make_uint4(0u, 0u, 0u, 0u);
    }

    // ---- 1. per-channel gate prefix (tokens in lanes; rows past L add 0)
#pragma unroll
    for (int i = 0; i < GW / 4; ++i) {
        f32x4 gs;
#pragma unroll
        for (int e = 0; e < 4; ++e) gs[e] = wave_inclusive_sum(tg < L ? fmaxf(gl[i][e], kMinChannelLogGate) : 0.f);
        *reinterpret_cast<f32x4 *>(&Gs[lane * PG + wv * GW + 4 * i]) = gs;
    }
    __syncthreads();
    // D_ij = exp(B_i - E_j) (row d_row(i, j)) and the chunk's state decay exp(G_C)
    for (int idx = tid; idx < 6 * DK; idx += 256) {
        const int fr = idx / DK, ch = idx - fr * DK;
        const int i = fr < 3 ? fr + 1 : fr < 5 ? fr - 1 : 3, j = fr < 3 ? 0 : fr < 5 ? 1 : 2;
        F[fr * DK + ch] = __expf(Gs[(16 * i - 1) * PG + ch] - Gs[(16 * j + 15) * PG + ch]);
    }
    if (tid < DK) a.cdec[((size_t)bh * a.nchunks + c) * DK + tid] = __expf(Gs[(C - 1) * PG + tid]);

    // ---- 2. this lane's rebased rows, the pre-scaled q and k for the serial
    // pass, the diagonal block's products in fp32, and beta-scaled operands
    const int mid = 16 * wv + 8;
    uint4 kq[NU], qb[NU], bgk[NU];  // fp16: k e^{G - B}, q e^{G - B}, beta k e^{G}
    f32x4 pd = {0.f, 0.f, 0.f, 0.f}, md = {0.f, 0.f, 0.f, 0.f};
    f16 *qcp = (f16 *)a.qc + ((size_t)bh * a.Lp + t) * DK + g * CQ;
    f16 *kcp = (f16 *)a.kc + ((size_t)bh * a.Lp + t) * DK + g * CQ;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int c0 = g * CQ + 8 * u;
        float q8[8], k8[8];
        {
            Raw8<bf16> rq, rk;
            rq.v[0] = qr[u];
            rk.v[0] = kr[u];
            unpack8<bf16>(rq, q8);
            unpack8<bf16>(rk, k8);
        }
        float gr[8], gb[8], ge[8], gm[8], gc[8];
        ld8<float>(&Gs[tr * PG + c0], gr);
        ld8<float>(&Gs[(16 * wv + 15) * PG + c0], ge);
        ld8<float>(&Gs[mid * PG + c0], gm);
        ld8<float>(&Gs[(C - 1) * PG + c0], gc);
        if (wv > 0) {
            ld8<float>(&Gs[(16 * wv - 1) * PG + c0], gb);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gb[e] = 0.f;
        }
        float xq[8], xb[8], xk[8], xc[8], xg[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float fb = __expf(gr[e] - gb[e]);  // <= 1
            xq[e] = q8[e] * fb;
            xb[e] = k8[e] * fb;
            xk[e] = k8[e] * __expf(ge[e] - gr[e]);   // <= 1
            const float fg = __expf(gr[e]);
            xc[e] = q8[e] * fg;
            xg[e] = bv * k8[e] * fg;
            // diagonal block, rebased around its middle token (the K slot of step
            // 8u + e is channel c0 + e of this lane's token, in A and B alike)
            const float x = __expf(gr[e] - gm[e]);
            const float kx = k8[e] * __builtin_amdgcn_rcpf(x);  // a correctly rounded divide costs ten instructions
            pd = __builtin_amdgcn_mfma_f32_16x16x4f32(k8[e] * x, kx, pd, 0, 0, 0);
            md = __builtin_amdgcn_mfma_f32_16x16x4f32(kx, q8[e] * x, md, 0, 0, 0);
        }
        float kcv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kcv[e] = k8[e] * __expf(gc[e] - gr[e]);  // <= 1
        auto pk = [](const float (&x)[8]) __attribute__((always_inline)) {
            f16x8 h;
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (f16)x[e];
            return __builtin_bit_cast(uint4, h);
        };
        qb[u] = pk(xq);
        kq[u] = pk(xb);
        bgk[u] = pk(xg);
        *reinterpret_cast<uint4 *>(&Ra[tr * PK + c0]) = pk(xk);
        *reinterpret_cast<uint4 *>(qcp + 8 * u) = pk(xc);
        *reinterpret_cast<uint4 *>(kcp + 8 * u) = pk(kcv);
    }
    __syncthreads();  // the rebased keys and the factor rows are visible; G is dead

    // ---- 3. P and the score fragments. P tile D[t][s] (t in block wv, lane (g, n):
    // t = 16 wv + 4g + e, s = 16 sb + n); score tile D[s][r] (s = 16 sb + 4g + e,
    // r = 16 wv + n). Cross blocks on fp16 operands, channels in the K slots
    // g CQ + 8 ks + (0..7); the diagonal block from the fp32 products.
    {
        const int w = wv;
        f32x4 ms[NRB];
#pragma unroll
        for (int sb = 0; sb < NRB; ++sb) {
            ms[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (sb >= w) continue;
            f32x4 p4 = {0.f, 0.f, 0.f, 0.f};
            const float *Dr = &F[d_row(w, sb) * DK];
#pragma unroll
            for (int ks = 0; ks < NU; ++ks) {
                const int c0 = g * CQ + 8 * ks;
                f16x8 kk = *reinterpret_cast<const f16x8 *>(&Ra[(16 * sb + n) * PK + c0]);
                const f32x4 d0 = *reinterpret_cast<const f32x4 *>(Dr + c0);
                const f32x4 d1 = *reinterpret_cast<const f32x4 *>(Dr + c0 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kk[e] = (f16)((float)kk[e] * d0[e]);
                    kk[4 + e] = (f16)((float)kk[4 + e] * d1[e]);
                }
                p4 = MF::mma(__builtin_bit_cast(frag, kq[ks]), kk, p4);
                ms[sb] = MF::mma(kk, __builtin_bit_cast(frag, qb[ks]), ms[sb]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tt = 16 * w + 4 * g + e;
                Pm[tt * TP + 16 * sb + n] = __shfl(bv, 4 * g + e, 64) * p4[e];
            }
        }
        // the diagonal block: P strictly lower, scores on and below the diagonal
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ii = 4 * g + e;  // row within the block
            // every lane takes part in the shuffle (an inactive source lane reads 0)
            const float bt = __shfl(bv, ii, 64);
            Pm[(16 * w + ii) * TP + 16 * w + n] = n < ii ? bt * pd[e] : 0.f;
            ms[w][e] = ii > n ? 0.f : md[e];
        }
        f16 *mo = (f16 *)a.mf + ((size_t)bh * a.nchunks + c) * 6 * 512 + lane * 8;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (2 * p <= w) {
                const int f = w + (w > 2 ? w - 2 : 0) + p;
                *reinterpret_cast<f16x8 *>(mo + f * 512) = pack_tiles(ms[2 * p], ms[2 * p + 1], 1.f);
            }
        }
    }
    __syncthreads();  // P complete; the rebased keys are dead

    // ---- 4. T = (I + P)^-1 by 16-row blocks: the diagonal blocks by forward
    // substitution (wave w, lane n holding column n), the blocks below as
    // T_ij = -T_ii sum_{j <= k < i} P_ik T_kj on fp32 MFMA
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
    auto below_block = [&](int i, int j) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int kb = j; kb < i; ++kb) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(Pm[(16 * i + n) * TP + 16 * kb + 4 * q + g],
                                                         Tm[(16 * kb + 4 * q + g) * TP + 16 * j + n], y, 0, 0, 0);
        }
        float *Y = Ysc + wv * 256;
#pragma unroll
        for (int e = 0; e < 4; ++e) Y[(4 * g + e) * 16 + n] = y[e];
        __builtin_amdgcn_wave_barrier();
        f32x4 tt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            tt = __builtin_amdgcn_mfma_f32_16x16x4f32(Tm[(16 * i + n) * TP + 16 * i + 4 * q + g], Y[(4 * q + g) * 16 + n],
                                                      tt, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Tm[(16 * i + 4 * g + e) * TP + 16 * j + n] = -tt[e];
    };
    if (wv < 3) below_block(wv + 1, wv);
    __syncthreads();
    if (wv < 2) below_block(wv + 2, wv);
    __syncthreads();
    if (wv == 0) below_block(3, 0);
    __syncthreads();  // T complete; P is dead
#pragma unroll
    for (int i = 0; i < C * C / 256; ++i) {
        const int idx = tid + 256 * i, r = idx / C, s = idx % C;
        To[r * OP + s] = (f16)((s >> 4) > (r >> 4) ? 0.f : Tm[r * TP + s]);
    }
    // beta Gam K, row-major (this lane's row and channel quarter)
#pragma unroll
    for (int u = 0; u < NU; ++u) *reinterpret_cast<uint4 *>(&Ra[tr * PK + g * CQ + 8 * u]) = bgk[u];
    __syncthreads();

    // T rows as an operand with the token K slots of the transpose loads
    auto trow = [&](int r, int ks) __attribute__((always_inline)) -> frag {
        const f16x4 lo = *reinterpret_cast<const f16x4 *>(&To[r * OP + 32 * ks + 4 * g]);
        const f16x4 hi = *reinterpret_cast<const f16x4 *>(&To[r * OP + 32 * ks + 16 + 4 * g]);
        return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    // ---- 5. W^T tiles D[ch][r] = sum_s (beta Gam K)[s][ch] T[r][s], row-major W
    f16 *wout = (f16 *)a.w + ((size_t)bh * a.Lp + t0) * DK;
    for (int tile = wv; tile < (DK / 16) * NRB; tile += 4) {
        const int cbk = tile / NRB, rb = tile % NRB;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) d = MF::mma(tr_frag<PK>(Ra, 32 * ks + 4 * g, cbk * 16, lane), trow(rb * 16 + n, ks), d);
        st4<f16>(wout + (size_t)(rb * 16 + n) * DK + cbk * 16 + 4 * g, d);
    }
    __syncthreads();  // W formed
    // beta V, row-major (this lane's row and column quarter)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (8 * u < VQ) {
            Raw8<bf16> r8;
            r8.v[0] = vr[u];
            float x[8];
            unpack8<bf16>(r8, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= bv;
            st8<f16>(&Ra[tr * PV + g * VQ + 8 * u], x);
        }
    }
    __syncthreads();
    // ---- 6. U~ tiles D[r][j] = sum_s T[r][s] (beta V)[s][j] in the serial pass's
    // accumulator layout [bh][chunk][jb][rb][lane][4]
    const int NJB = dv / 16;
    f16 *uout = (f16 *)a.ut + ((size_t)bh * a.nchunks + c) * NJB * (NRB * 256);
    for (int tile = wv; tile < NRB * NJB; tile += 4) {
        const int rb = tile / NJB, jb = tile % NJB;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) d = MF::mma(trow(rb * 16 + n, ks), tr_frag<PV>(Ra, 32 * ks + 4 * g, jb * 16, lane), d);
        st4<f16>(uout + (size_t)(jb * NRB + rb) * 256 + lane * 4, d);
    }
}

template <int DK>
hipError_t launch_kda_prep(const PrepArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((kda_prep_kernel<DK>), dim3(a.BH * a.nchunks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
