// bwd_impl.hpp -- backward pass of the chunkwise forward (gfx950): gradients of
// a loss with respect to q, k, v, the log-gates and the initial state, given
// the output gradient dO and optionally the final-state gradient.
//
// Reverse-mode of S_t = g_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t (tensorplay
// "Talk Linear Attention", section 2.1; the decay of wln20 "LLM注意力优化：线性注意力",
// data-dependent decay equation), in the chunk form of tensorplay section 3.2.
// For chunk c with chunk-local cumulative log-gate G_r, a_r = e^{G_r}, the
// state H_c at its start and dH_c = dLoss/d(state at its end):
//   dq_r = a_r H_c do_r + sum_{s<=r} e^{G_r - G_s} (do_r . v_s) k_s
//   dk_s = sum_{r>=s} e^{G_r - G_s} (do_r . v_s) q_r + e^{G_end - G_s} dH_c v_s
//   dv_s = sum_{r>=s} e^{G_r - G_s} (q_r . k_s) do_r + e^{G_end - G_s} dH_c^T k_s
//   dH_{c-1} = e^{G_end} dH_c + sum_r a_r q_r do_r^T
// and, since the loss sees the cumulative gates only through differences,
//   dl_t = sum_{u>=t} (q_u . dq_u - k_u . dk_u) + <dS_L, S_L>.
//
// Kernels:
//   state_scans_kernel  one workgroup per (head, value slice) walks the chunks
//       forward, storing each H_c (operand type, transposed) and the final state S_L; with
//       FWD = false it walks them backward with (q (.) a, dO) in place of
//       (k (.) e^{G_end - G}, v), storing each dH_c and returning dS_0. Both
//       scans run in one launch.
//   bwd_dqkv_kernel  one workgroup (8 waves) per (head, chunk), fully parallel:
//       waves w, w+4 own query block w (dq) and key block w (dk, dv), each for
//       half of the output columns. Products are
//       taken transposed (dQ^T = K^T dP^T, ...) so that the 16 x 16 score-like
//       tiles dP = dO V^T, A = Q K^T leave the MFMA in exactly the B-operand
//       layout of the next product, as in the forward kernel. It also writes
//       q_t . dq_t - k_t . dk_t per token and, for the scalar decay,
//       <dH_c, H_{c+1}> per chunk.
//   dgate_kernel  one workgroup per head: per chunk, the reverse prefix sum of
//       those terms within the chunk, started from <dH_c, H_{c+1}>.
#pragma once

#include <type_traits>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

// ---------------------------------------------------------------------------
// state scan: S <- e^{G_end} S + sum_s f_s X_s^T Y_s over chunks, forward
// (X = k, Y = v, f_s = e^{G_end - G_s}) or backward (X = q, Y = dO, f_s = e^{G_s}).
// The per-chunk states are stored transposed, [d_v][d_k] per chunk, so each lane
// writes four consecutive d_k entries at once. The next chunk's rows and gates
// are loaded into registers while the current chunk is folded in; every wave
// scans the chunk's gates itself (rows in lanes), so no barrier guards them.
template <typename TI, int DK, int DVT, bool FWD, bool DECAY>
__device__ __attribute__((always_inline)) inline void state_scan(const BwdArgs &a, int blk, void *lds) {
    using TM = typename OpOf<TI>::type;
    using MF = Mfma<TM>;
    using frag = typename MF::frag;
    constexpr int C = 64, E = MF::E;
    constexpr bool H = E == 8;
    constexpr int PX = H ? DK + 16 : DK + 4, PY = H ? DVT + 16 : DVT + 4;
    constexpr int NTI = DK / 16, NTJ = DVT / 16, NTILE = NTI * NTJ, TPW = (NTILE + 3) / 4;
    constexpr int NTK = C / (4 * E);
    constexpr int SEGX = DK / 8, SEGY = DVT / 8;
    constexpr int NXS = (C * SEGX + 255) / 256, NYS = (C * SEGY + 255) / 256;
    // double-buffered operand tiles: chunk it is staged into buffer it & 1, whose
    // last reader (chunk it - 2) is behind the barrier of chunk it - 1
    TM(*Xs)[C * PX] = reinterpret_cast<TM(*)[C * PX]>(lds);
    TM(*Ys)[C * PY] = reinterpret_cast<TM(*)[C * PY]>(static_cast<TM *>(lds) + 2 * C * PX);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int bh = blk / a.nsplit, split = blk % a.nsplit;
    const int L = a.L, dv = a.dv, j0 = split * DVT, nchunks = (L + C - 1) / C;
    const TI *xg = (const TI *)(FWD ? a.k : a.q) + (size_t)bh * L * DK;
    const TI *yg = (const TI *)(FWD ? a.v : a.dout) + (size_t)bh * L * dv + j0;
    const float *lg = DECAY ? a.lg + (size_t)bh * L : nullptr;
    TM *hs = (TM *)(FWD ? a.hs : a.dhs) + (size_t)bh * nchunks * DK * dv;

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

    // Prefetch registers, NSET sets: chunk it + NSET is loaded while chunk it is
    // folded in (with two, a load has a whole chunk of work to arrive). Every load is
    // unconditional (rows past the end re-read the last row; masks zero them
    // where the registers are used; chunks past the end re-read the last one,
    // unused), so the compiler counts the loads in flight exactly and waits for
    // a set only where it is used.
    constexpr int NSET = 2;                  // register sets
    constexpr int NU = (int)sizeof(TI) / 2;  // 16-byte words per 8 elements
    u32x4 rx[NSET][NXS][NU], ry[NSET][NYS][NU];
    uint32_t kxm[NSET][NXS], kym[NSET][NYS], kg[NSET];
    float rg[NSET];
    // reverse scan of the normalized variant: dO rows scaled by rho (1 / den)
    const float *rho = FWD ? nullptr : (a.rho ? a.rho + (size_t)bh * L : nullptr);
    float rr[NSET][NYS];
    auto chunk_of = [&](int it) __attribute__((always_inline)) {
        it = min(it, nchunks - 1);
        return FWD ? it : nchunks - 1 - it;
    };
    auto load = [&](auto set_tag, int it) __attribute__((always_inline)) {
        constexpr int P = decltype(set_tag)::value % NSET;
        const int t0 = chunk_of(it) * C, nv = min(C, L - t0);
        const TI *px[NXS], *py[NYS];
#pragma unroll
        for (int m = 0; m < NXS; ++m) {
            const int sid = min(tid + 256 * m, C * SEGX - 1), row = sid / SEGX;
            kxm[P][m] = (tid + 256 * m < C * SEGX && row < nv) ? 0xffffffffu : 0u;
            px[m] = xg + (size_t)(t0 + min(row, nv - 1)) * DK + 8 * (sid % SEGX);
        }
#pragma unroll
        for (int m = 0; m < NYS; ++m) {
            const int sid = min(tid + 256 * m, C * SEGY - 1), row = sid / SEGY;
            kym[P][m] = (tid + 256 * m < C * SEGY && row < nv) ? 0xffffffffu : 0u;
            py[m] = yg + (size_t)(t0 + min(row, nv - 1)) * dv + 8 * (sid % SEGY);
            rr[P][m] = rho ? rho[t0 + min(row, nv - 1)] : 1.f;
        }
#pragma unroll
        for (int m = 0; m < NXS; ++m)
#pragma unroll
            for (int i = 0; i < NU; ++i) rx[P][m][i] = reinterpret_cast<const u32x4 *>(px[m])[i];
#pragma unroll
        for (int m = 0; m < NYS; ++m)
#pragma unroll
            for (int i = 0; i < NU; ++i) ry[P][m][i] = reinterpret_cast<const u32x4 *>(py[m])[i];
        if constexpr (DECAY) {
            kg[P] = lane < nv ? 0xffffffffu : 0u;
            rg[P] = lg[t0 + min(lane, nv - 1)];
        }
    };
    // eight prefetched elements, masked, as Raw8
    auto take = [&](const u32x4 (&r)[NU], uint32_t k) __attribute__((always_inline)) -> Raw8<TI> {
        Raw8<TI> o;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const u32x4 w = r[i] & k;
            o.v[i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
        return o;
    };

    // chunk `it` of the scan from tile buffer B and register set B % NSET
    auto step = [&](auto set_tag, int it) __attribute__((always_inline)) {
        constexpr int B = decltype(set_tag)::value;  // tile buffer
        constexpr int P = B % NSET;                  // register set
        const int c = chunk_of(it);
        // store the state this chunk starts from (forward) / ends at (backward), transposed
        TM *hc = hs + (size_t)c * DK * dv;
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int tile = wv + 4 * m;
            if (NTILE % 4 == 0 || tile < NTILE) {
                const int ti = tile / NTJ, tj = tile % NTJ;
                st4<TM>(hc + (size_t)(j0 + tj * 16 + n) * DK + ti * 16 + 4 * g, Sacc[m]);
            }
        }
        // the chunk's gate prefix, rows in lanes (every wave)
        float G = 0.f, gend = 0.f;
        if constexpr (DECAY) {
            G = wave_inclusive_sum(__uint_as_float(__float_as_uint(rg[P]) & kg[P]));
            gend = __shfl(G, 63, 64);
        }
#pragma unroll
        for (int m = 0; m < NXS; ++m) {
            const int sid = tid + 256 * m;
            if (sid < C * SEGX) {
                const int row = sid / SEGX;
                float x[8];
                unpack8<TI>(take(rx[P][m], kxm[P][m]), x);
                if constexpr (DECAY) {
                    const float Gr = __shfl(G, row, 64);
                    const float f = FWD ? __expf(gend - Gr) : __expf(Gr);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] *= f;
                }
                st8<TM>(&Xs[B][row * PX + 8 * (sid % SEGX)], x);
            }
        }
#pragma unroll
        for (int m = 0; m < NYS; ++m) {
            const int sid = tid + 256 * m;
            if (sid < C * SEGY) {
                float y[8];
                unpack8<TI>(take(ry[P][m], kym[P][m]), y);
                if (rho) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] *= rr[P][m];
                }
                st8<TM>(&Ys[B][(sid / SEGY) * PY + 8 * (sid % SEGY)], y);
            }
        }
        // keep the loads after the last reads of this set: hoisted above them they
        // would need fresh registers, copied back at the loop head after a wait
        __builtin_amdgcn_sched_barrier(0);
        load(set_tag, it + NSET);
        __syncthreads();  // buffer B staged
        const float eg = DECAY ? __expf(gend) : 1.f;
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int tile = wv + 4 * m;
            if (NTILE % 4 == 0 || tile < NTILE) {
                const int ti = tile / NTJ, tj = tile % NTJ;
                Sacc[m] *= eg;
#pragma unroll
                for (int ks = 0; ks < NTK; ++ks) {
                    frag xa, yb;
                    if constexpr (H) {
                        xa = tr_frag<PX>(Xs[B], 32 * ks + 4 * g, ti * 16, lane);
                        yb = tr_frag<PY>(Ys[B], 32 * ks + 4 * g, tj * 16, lane);
                    } else {
                        xa = Xs[B][(4 * ks + g) * PX + ti * 16 + n];
                        yb = Ys[B][(4 * ks + g) * PY + tj * 16 + n];
                    }
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

// The two scans are independent; one launch runs both, the forward one on the
// first BH * nsplit workgroups.
template <typename TI, int DK, int DVT, bool DECAY>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) state_scans_kernel(BwdArgs a) {
    // both directions' tiles: two buffers of X (C x PX) and Y (C x PY) in the operand type
    using TM = typename OpOf<TI>::type;
    constexpr int PAD = sizeof(TM) == 2 ? 16 : 4;
    __shared__ __align__(16) TM lds[2 * 64 * (DK + PAD + DVT + PAD)];
    // value slices of one head on one XCD: they share its rows through that L2
    const int per = a.BH * a.nsplit, vid = xcd_virtual_block();
    if (vid < per)
        state_scan<TI, DK, DVT, true, DECAY>(a, vid, lds);
    else
        state_scan<TI, DK, DVT, false, DECAY>(a, vid - per, lds);
}

// ---------------------------------------------------------------------------
// dq, dk, dv of one chunk (C = 64, 8 waves): wave w takes query block w & 3 (dq)
// and key block w & 3 (dk, dv) for half w >> 2 of the output columns; the two
// waves of a block compute its score-like tiles each.
template <typename TI, int DK, int DV, bool DECAY>
__global__ void __launch_bounds__(512) bwd_dqkv_kernel(BwdArgs a) {
    using TM = typename OpOf<TI>::type;
    using MF = Mfma<TM>;
    using frag = typename MF::frag;
    constexpr int C = 64, E = MF::E, NRB = 4;
    constexpr bool H = E == 8;
    constexpr int PK = H ? DK + 16 : DK + 4;  // q, k and the transposed states (d_k columns)
    constexpr int PV = H ? DV + 16 : DV + 4;  // v, dO
    constexpr int NKS_K = DK / (4 * E), NKS_V = DV / (4 * E);  // k-steps over d_k, d_v
    constexpr int NCT = DK / 16, NJT = DV / 16, NCW = NCT / 2, NJW = NJT / 2;
    constexpr int SEGK = DK / 8, SEGV = DV / 8;
    __shared__ __align__(16) TM Qs[C * PK];
    __shared__ __align__(16) TM Ks[C * PK];
    __shared__ __align__(16) TM Vs[C * PV];
    __shared__ __align__(16) TM Os[C * PV];   // dO
    __shared__ __align__(16) TM Hs[DV * PK];  // H_c^T  [dv][dk]
    __shared__ __align__(16) TM Ds[DV * PK];  // dH_c^T [dv][dk]
    __shared__ float Gt[C];
    __shared__ float RT[2][C];
    __shared__ float XP[8];  // per wave: its share of <dH_c, H_{c+1}>
    __shared__ float Gend;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, n = lane & 15;
    const int L = a.L, nchunks = (L + C - 1) / C;
    // Persistent: each workgroup takes chunks (batch-head, chunk) = item in
    // steps of the grid size; the next item's rows and states are loaded into
    // registers while the current one is computed.
    const int items = a.BH * nchunks;
    constexpr int NQ = (C * SEGK + 511) / 512, NVV = (C * SEGV + 511) / 512, NS = (DV * SEGK + 511) / 512;
    Raw8<TI> rq[NQ], rk[NQ], rv[NVV], ro[NVV];
    float rro[NVV];  // normalized variant: the dO rows' scale rho (1 / den)
    Raw8<TM> rh[NS], rd[NS];
    float rgl = 0.f;  // wave 0: the log-gate of token `lane`
    auto fetch = [&](int item) __attribute__((always_inline)) {
        const int bh = item / nchunks, c = item % nchunks;
        const int t0 = c * C, nv = min(C, L - t0);
        const TI *qg = (const TI *)a.q + ((size_t)bh * L + t0) * DK;
        const TI *kg = (const TI *)a.k + ((size_t)bh * L + t0) * DK;
        const TI *vg = (const TI *)a.v + ((size_t)bh * L + t0) * DV;
        const TI *og = (const TI *)a.dout + ((size_t)bh * L + t0) * DV;
        const TM *hg = (const TM *)a.hs + ((size_t)bh * nchunks + c) * DK * DV;
        const TM *dhg = (const TM *)a.dhs + ((size_t)bh * nchunks + c) * DK * DV;
        if constexpr (DECAY) {
            if (wv == 0) rgl = lane < nv ? a.lg[(size_t)bh * L + t0 + lane] : 0.f;
        }
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int sid = tid + 512 * m, row = sid / SEGK, off = row * DK + 8 * (sid % SEGK);
            const bool ok = sid < C * SEGK && row < nv;
            rq[m] = ok ? ld_raw8<TI>(qg + off) : zero_raw8<TI>();
            rk[m] = ok ? ld_raw8<TI>(kg + off) : zero_raw8<TI>();
        }
#pragma unroll
        for (int m = 0; m < NVV; ++m) {
            const int sid = tid + 512 * m, row = sid / SEGV, off = row * DV + 8 * (sid % SEGV);
            const bool ok = sid < C * SEGV && row < nv;
            rv[m] = ok ? ld_raw8<TI>(vg + off) : zero_raw8<TI>();
            ro[m] = ok ? ld_raw8<TI>(og + off) : zero_raw8<TI>();
            if constexpr (!DECAY) rro[m] = (a.rho && ok) ? a.rho[(size_t)bh * L + t0 + row] : 1.f;
        }
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int sid = tid + 512 * m;
            if (sid < DV * SEGK) {
                const int off = (sid / SEGK) * DK + 8 * (sid % SEGK);
                rh[m] = ld_raw8<TM>(hg + off);
                rd[m] = ld_raw8<TM>(dhg + off);
            }
        }
    };

    auto process = [&](int item, auto &&prefetch_next) __attribute__((always_inline)) {
    const int bh = item / nchunks, c = item % nchunks;
    const int t0 = c * C, nv = min(C, L - t0);
    (void)c;
    // ---- stage the chunk (its loads were issued one item ago)
    if constexpr (DECAY) {
        if (wv == 0) {
            const float G = wave_inclusive_sum(rgl);
            Gt[lane] = G;
            if (lane == 63) Gend = G;
        }
    }
    auto put = [&](const Raw8<TI> &r, TM *dst) __attribute__((always_inline)) {
        float x[8];
        unpack8<TI>(r, x);
        st8<TM>(dst, x);
    };
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
        const int sid = tid + 512 * m;
        if (sid < C * SEGK) {
            const int o = (sid / SEGK) * PK + 8 * (sid % SEGK);
            put(rq[m], &Qs[o]);
            put(rk[m], &Ks[o]);
        }
    }
#pragma unroll
    for (int m = 0; m < NVV; ++m) {
        const int sid = tid + 512 * m;
        if (sid < C * SEGV) {
            const int o = (sid / SEGV) * PV + 8 * (sid % SEGV);
            put(rv[m], &Vs[o]);
            if (!DECAY && a.rho) {  // the normalized variant (no gates)
                float x[8];
                unpack8<TI>(ro[m], x);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] *= rro[m];
                st8<TM>(&Os[o], x);
            } else {
                put(ro[m], &Os[o]);
            }
        }
    }
    float xterm = 0.f;  // this thread's share of <dH_c, H_c> (scalar decay)
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int sid = tid + 512 * m;
        if (sid < DV * SEGK) {
            const int o = (sid / SEGK) * PK + 8 * (sid % SEGK);
#pragma unroll
            for (int u = 0; u < (int)(sizeof(TM) / 2); ++u) {
                reinterpret_cast<uint4 *>(&Hs[o])[u] = rh[m].v[u];
                reinterpret_cast<uint4 *>(&Ds[o])[u] = rd[m].v[u];
            }
            if constexpr (DECAY) {
                if constexpr (H) {  // fp16 pairs, products exact, sums in fp32
                    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                    const uint32_t wh[4] = {rh[m].v[0].x, rh[m].v[0].y, rh[m].v[0].z, rh[m].v[0].w};
                    const uint32_t wd[4] = {rd[m].v[0].x, rd[m].v[0].y, rd[m].v[0].z, rd[m].v[0].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xterm = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, wh[i]), __builtin_bit_cast(h2, wd[i]),
                                                       xterm, false);
                } else {
                    float xh[8], xd[8];
                    unpack8<TM>(rh[m], xh);
                    unpack8<TM>(rd[m], xd);
#pragma unroll
                    for (int e = 0; e < 8; ++e) xterm += xh[e] * xd[e];
                }
            }
        }
    }
    __syncthreads();
    prefetch_next();  // the registers are free: the next item's loads fly during the math

    const int w = wv & 3, half = wv >> 2;
    const float gend = DECAY ? Gend : 0.f;
    // natural-layout operand: row `row` of X, k-step ks of a K-dim of width KW
    auto nat = [&](const TM *X, int P, int row, int ks, int KW) __attribute__((always_inline)) -> frag {
        return ld_frag<TM>(&X[row * P + g * (KW / 4) + ks * E]);
    };
    // natural-layout operand whose K-slots follow the transpose-load pattern:
    // elements 32 ks + 4g + (0..3) and 32 ks + 16 + 4g + (0..3) of row `row`
    auto trn = [&](const TM *X, int P, int row, int ks) __attribute__((always_inline)) -> frag {
        if constexpr (H) {
            typedef _Float16 h4 __attribute__((ext_vector_type(4)));
            const h4 lo = *reinterpret_cast<const h4 *>(&X[row * P + 32 * ks + 4 * g]);
            const h4 hi = *reinterpret_cast<const h4 *>(&X[row * P + 32 * ks + 16 + 4 * g]);
            return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
            return X[row * P + 4 * ks + g];
        }
    };
    // row-slot operand of a row-major tile (rows in the K-slots, column col0 + n per lane)
    auto tok = [&](const TM *X, auto p_tag, int ks, int col0) __attribute__((always_inline)) -> frag {
        constexpr int P = decltype(p_tag)::value;
        if constexpr (H) return tr_frag<P>(X, 32 * ks + 4 * g, col0, lane);
        else return X[(4 * ks + g) * P + col0 + n];
    };
    using PKt = std::integral_constant<int, PK>;
    using PVt = std::integral_constant<int, PV>;
    auto decay_of = [&](int r, int s) __attribute__((always_inline)) -> float {
        if constexpr (DECAY) return __expf(Gt[r] - Gt[s]);
        else return 1.f;
    };
    // score-like tile pairs -> B operand over 32 tokens (tiles 2p, 2p+1)
    auto bop_of = [&](const f32x4 &t0_, const f32x4 &t1_) __attribute__((always_inline)) -> frag {
        frag b{};
        if constexpr (H) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                b[e] = from_f32<TM>(t0_[e]);
                b[4 + e] = from_f32<TM>(t1_[e]);
            }
        }
        return b;
    };

    float rterm = 0.f;  // (q . dq - k . dk) of token 16 w + n over this wave's columns

    // ---- dq for query block w: dQ^T[c][r] = a_r sum_j H[c][j] dO[r][j] + sum_s K[s][c] dP[r][s]
    {
        f32x4 acc[NCW];
        const int r = 16 * w + n;
        const float ar = DECAY ? __expf(Gt[r]) : 1.f;
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int ct = half * NCW + q_;
            acc[q_] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS_V; ++ks)
                acc[q_] = MF::mma(tok(Hs, PKt{}, ks, ct * 16), trn(Os, PV, r, ks), acc[q_]);
            acc[q_] *= ar;
        }
        // dP^T tiles D[s][r] = sum_j V[s][j] dO[r][j] for key blocks sb <= w
        f32x4 dpt[NRB];
#pragma unroll
        for (int sb = 0; sb < NRB; ++sb) {
            dpt[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (sb <= w) {
#pragma unroll
                for (int ks = 0; ks < NKS_V; ++ks)
                    dpt[sb] = MF::mma(nat(Vs, PV, sb * 16 + n, ks, DV), nat(Os, PV, r, ks, DV), dpt[sb]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s_ = sb * 16 + 4 * g + e;
                    dpt[sb][e] = (s_ > r) ? 0.f : dpt[sb][e] * decay_of(r, s_);
                }
            }
        }
        if constexpr (H) {
#pragma unroll
            for (int p = 0; p < NRB / 2; ++p) {
                if (2 * p <= w) {
                    const frag bop = bop_of(dpt[2 * p], dpt[2 * p + 1]);
#pragma unroll
                    for (int q_ = 0; q_ < NCW; ++q_)
                        acc[q_] = MF::mma(tok(Ks, PKt{}, p, (half * NCW + q_) * 16), bop, acc[q_]);
                }
            }
        } else {
#pragma unroll
            for (int sb = 0; sb < NRB; ++sb) {
                if (sb <= w) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int q_ = 0; q_ < NCW; ++q_)
                            acc[q_] = MF::mma(Ks[(sb * 16 + 4 * g + e) * PK + (half * NCW + q_) * 16 + n], dpt[sb][e],
                                              acc[q_]);
                }
            }
        }
        float *dqg = a.gq + ((size_t)bh * L + t0 + r) * DK;
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int ct = half * NCW + q_;
            if (r < nv) *reinterpret_cast<f32x4 *>(dqg + ct * 16 + 4 * g) = acc[q_];
#pragma unroll
            for (int e = 0; e < 4; ++e) rterm += acc[q_][e] * to_f32<TM>(Qs[r * PK + ct * 16 + 4 * g + e]);
        }
    }

    // ---- dk for key block w: dK^T[c][s] = e^{G_end - G_s} sum_j dH[c][j] V[s][j] + sum_r Q[r][c] dP[r][s]
    // ---- dv for key block w: dV^T[j][s] = e^{G_end - G_s} sum_c dH[c][j] K[s][c] + sum_r dO[r][j] A[r][s]
    const int s = 16 * w + n;
    const float ws = DECAY ? __expf(gend - Gt[s]) : 1.f;
    {
        f32x4 acc[NCW];
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int ct = half * NCW + q_;
            acc[q_] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS_V; ++ks)
                acc[q_] = MF::mma(tok(Ds, PKt{}, ks, ct * 16), trn(Vs, PV, s, ks), acc[q_]);
            acc[q_] *= ws;
        }

        // dP tiles D[r][s] = sum_j dO[r][j] V[s][j] for query blocks rbk >= w
        f32x4 dp[NRB];
#pragma unroll
        for (int rbk = 0; rbk < NRB; ++rbk) {
            dp[rbk] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (rbk >= w) {
#pragma unroll
                for (int ks = 0; ks < NKS_V; ++ks)
                    dp[rbk] = MF::mma(nat(Os, PV, rbk * 16 + n, ks, DV), nat(Vs, PV, s, ks, DV), dp[rbk]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rr = rbk * 16 + 4 * g + e;
                    dp[rbk][e] = (rr < s) ? 0.f : dp[rbk][e] * decay_of(rr, s);
                }
            }
        }
        if constexpr (H) {
#pragma unroll
            for (int p = 0; p < NRB / 2; ++p) {
                if (2 * p + 1 >= w) {
                    const frag bop = bop_of(dp[2 * p], dp[2 * p + 1]);
#pragma unroll
                    for (int q_ = 0; q_ < NCW; ++q_)
                        acc[q_] = MF::mma(tok(Qs, PKt{}, p, (half * NCW + q_) * 16), bop, acc[q_]);
                }
            }
        } else {
#pragma unroll
            for (int rbk = 0; rbk < NRB; ++rbk) {
                if (rbk >= w) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int q_ = 0; q_ < NCW; ++q_)
                            acc[q_] = MF::mma(Qs[(rbk * 16 + 4 * g + e) * PK + (half * NCW + q_) * 16 + n], dp[rbk][e],
                                              acc[q_]);
                }
            }
        }
        float *dkg = a.gk + ((size_t)bh * L + t0 + s) * DK;
#pragma unroll
        for (int q_ = 0; q_ < NCW; ++q_) {
            const int ct = half * NCW + q_;
            if (s < nv) *reinterpret_cast<f32x4 *>(dkg + ct * 16 + 4 * g) = acc[q_];
#pragma unroll
            for (int e = 0; e < 4; ++e) rterm -= acc[q_][e] * to_f32<TM>(Ks[s * PK + ct * 16 + 4 * g + e]);
        }
    }
    {
        f32x4 acc[NJW];
#pragma unroll
        for (int q_ = 0; q_ < NJW; ++q_) {
            const int jt = half * NJW + q_;
            acc[q_] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS_K; ++ks)
                acc[q_] = MF::mma(nat(Ds, PK, jt * 16 + n, ks, DK), nat(Ks, PK, s, ks, DK), acc[q_]);
            acc[q_] *= ws;
        }
        // <dH_c, H_{c+1}> = e^{g_C} <dH_c, H_c> + sum_s v_s . (the state term of dv_s),
        // since H_{c+1} = e^{g_C} H_c + sum_s e^{g_C - G_s} k_s v_s^T
        if constexpr (DECAY) {
            xterm *= __expf(gend);
#pragma unroll
            for (int q_ = 0; q_ < NJW; ++q_) {
                const int jt = half * NJW + q_;
                const f32x4 vr = ld4<TM>(&Vs[s * PV + jt * 16 + 4 * g]);
#pragma unroll
                for (int e = 0; e < 4; ++e) xterm += acc[q_][e] * vr[e];
            }
        }
        // A tiles D[r][s] = sum_c Q[r][c] K[s][c] for query blocks rbk >= w
        f32x4 at[NRB];
#pragma unroll
        for (int rbk = 0; rbk < NRB; ++rbk) {
            at[rbk] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (rbk >= w) {
#pragma unroll
                for (int ks = 0; ks < NKS_K; ++ks)
                    at[rbk] = MF::mma(nat(Qs, PK, rbk * 16 + n, ks, DK), nat(Ks, PK, s, ks, DK), at[rbk]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rr = rbk * 16 + 4 * g + e;
                    at[rbk][e] = (rr < s) ? 0.f : at[rbk][e] * decay_of(rr, s);
                }
            }
        }
        if constexpr (H) {
#pragma unroll
            for (int p = 0; p < NRB / 2; ++p) {
                if (2 * p + 1 >= w) {
                    const frag bop = bop_of(at[2 * p], at[2 * p + 1]);
#pragma unroll
                    for (int q_ = 0; q_ < NJW; ++q_)
                        acc[q_] = MF::mma(tok(Os, PVt{}, p, (half * NJW + q_) * 16), bop, acc[q_]);
                }
            }
        } else {
#pragma unroll
            for (int rbk = 0; rbk < NRB; ++rbk) {
                if (rbk >= w) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int q_ = 0; q_ < NJW; ++q_)
                            acc[q_] = MF::mma(Os[(rbk * 16 + 4 * g + e) * PV + (half * NJW + q_) * 16 + n], at[rbk][e],
                                              acc[q_]);
                }
            }
        }
        float *dvg = a.gv + ((size_t)bh * L + t0 + s) * DV;
        if (s < nv) {
#pragma unroll
            for (int q_ = 0; q_ < NJW; ++q_)
                *reinterpret_cast<f32x4 *>(dvg + (half * NJW + q_) * 16 + 4 * g) = acc[q_];
        }
    }
    // q . dq - k . dk of token 16 w + n: sum over the lane groups, then the halves
    rterm += __shfl_xor(rterm, 16, 64);
    rterm += __shfl_xor(rterm, 32, 64);
    if (g == 0) RT[half][s] = rterm;
    if constexpr (DECAY) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) xterm += __shfl_xor(xterm, off, 64);
        if (lane == 0) XP[wv] = xterm;
    }
    __syncthreads();  // also: every wave is done with this item's tiles
    if (DECAY && tid < C && tid < nv) a.rterm[(size_t)bh * L + t0 + tid] = RT[0][tid] + RT[1][tid];
    if (DECAY && tid == 0) {
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) x += XP[i];
        a.xterm[(size_t)bh * nchunks + c] = x;
    }
    };

    int item = blockIdx.x;
    if (item < items) fetch(item);
    for (; item < items; item += gridDim.x) {
        const int nxt = item + gridDim.x;
        process(item, [&]() __attribute__((always_inline)) {
            if (nxt < items) fetch(nxt);
        });
    }
}

// ---------------------------------------------------------------------------
// dl_t = sum_{u >= t in t's chunk} rterm_u + <dH_c, H_{c+1}>: the gates of chunk c
// reach the loss only through q_t e^{G_t}, k_t e^{-G_t} and the factor e^{g_C} of
// the state the chunk hands on, so the suffix restarts at every chunk end (a
// suffix over the whole sequence adds up the rounding of every later token's
// term). One workgroup (256 threads) per head, one chunk per thread.
template <int DK>
__global__ void __launch_bounds__(256) dgate_kernel(BwdArgs a) {
    const int bh = blockIdx.x, L = a.L, nchunks = (L + 63) / 64;
    const float *rt = a.rterm + (size_t)bh * L;
    float *dl = a.glg + (size_t)bh * L;
    for (int c = threadIdx.x; c < nchunks; c += 256) {
        float run = a.xterm[(size_t)bh * nchunks + c];
        for (int t = min(L, 64 * c + 64) - 1; t >= 64 * c; --t) {
            run += rt[t];
            dl[t] = run;
        }
    }
}

// Workgroups of the persistent dq/dk/dv kernel: one per CU (its tiles take
// most of a CU's LDS).
constexpr int kBwdGrid = 256;

template <typename TI, int DK, int DV, bool DECAY>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t st) {
    constexpr int DVT = DV >= 64 ? 64 : DV;  // value slices of the state scans
    const int nchunks = (a.L + 63) / 64;
    BwdArgs b = a;
    b.nsplit = DV / DVT;
    hipLaunchKernelGGL((state_scans_kernel<TI, DK, DVT, DECAY>), dim3(2 * a.BH * b.nsplit), dim3(256), 0, st, b);
    if (nchunks > 0)
        hipLaunchKernelGGL((bwd_dqkv_kernel<TI, DK, DV, DECAY>), dim3(min(a.BH * nchunks, kBwdGrid)), dim3(512), 0, st, b);
    if (DECAY && nchunks > 0 && a.glg) hipLaunchKernelGGL((dgate_kernel<DK>), dim3(a.BH), dim3(256), 0, st, b);
    return hipGetLastError();
}

}  // namespace la
