/*
 * oracle.c -- fp64 CPU oracle for causal linear attention (TEST INFRASTRUCTURE).
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
 * may load this library. It shares no code with the GPU path. It is deliberately
 * plain and slow: the naive per-token recurrence, in float64, with sequential
 * summation over t, exactly as the pages state the method.
 *
 * Canonical orientation: the state S is d_k x d_v (row = key channel), S_t =
 * S_{t-1} + k_t v_t^T and o_t = S_t^T q_t  (tensorplay "Talk Linear Attention",
 * section 2.1, the recurrence and output equations). Pages that write the state
 * as v k^T (wln20 "LLM注意力优化：线性注意力", RNN form; tensorplay section 6)
 * describe its transpose; outputs are identical.
 *
 * Variants (per batch-head, independently):
 *   PLAIN        S <- S + k v^T;                      o = S^T q
 *                (tensorplay section 2.1)
 *   NORMALIZED   S <- S + k v^T;  z <- z + k;         o = S^T q / (q . z)
 *                q and k arrive already feature-mapped (proig-chaa notes
 *                sections 13-14: causal recurrence of S and z)
 *   DECAY        S <- gamma S + k v^T, gamma = exp(l); o = S^T q
 *                (wln20, data-dependent decay equation; proig-chaa section 20)
 *   VECTOR_DECAY S <- Diag(exp(l)) S + k v^T, l in R^{dk}; o = S^T q. One
 *                log-gate per key channel: tensorplay section 5.1 writes the GLA
 *                update as G_t (.) S_{t-1} + k_t v_t^T with G_t the gate alpha_t
 *                (a projection output) broadcast over the value columns, whose
 *                parallel form in section 5.2 scales Q and K per channel by the
 *                cumulative product B; wln20's Kimi Delta Attention section uses
 *                the same diagonal gate Diag(alpha_t) (here without the delta rule)
 *   GATED_DELTA  r = S^T k (retrieve); S <- alpha (S - beta k r^T) + beta k v^T;
 *                o = S^T q, alpha = exp(l) (alpha = 1 when no log-gate is given)
 *                This is the transpose of S'_t = S'_{t-1} alpha_t (I - beta_t k_t
 *                k_t^T) + beta_t v_t k_t^T, o_t = S'_t q_t (wln20, Gated DeltaNet
 *                section; tensorplay section 6.2 reparameterised delta rule).
 *   KDA          S <- Diag(exp(l)) S, l in R^{dk}; r = S^T k; S <- S + beta k (v - r)^T;
 *                o = S^T q. That is S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 *                + beta_t k_t v_t^T (wln20, Kimi Delta Attention section: the
 *                gated delta rule with the scalar gate widened to a diagonal one,
 *                read in the d_k x d_v orientation, where the diagonal acts on
 *                the key channels and the delta-rule factor multiplies from the
 *                left, as the page writes it).
 *
 * Inputs are float64 copies of exactly the values the GPU reads (bf16 or fp32
 * widened without rounding). Gates are log-gates l = log(gamma) or log(alpha);
 * the oracle forms gamma = exp(l) in float64.
 *
 * Layouts (all row-major, contiguous):
 *   q, k  [BH, L, dk]     v, o  [BH, L, dv]     log_gate, beta  [BH, L]
 *   (VECTOR_DECAY, KDA: log_gate [BH, L, dk])
 *   state_in, state_out  [BH, dk, dv]          z_in, z_out  [BH, dk]
 * NULL state_in / z_in mean zero; NULL state_out / z_out mean "not returned".
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_PLAIN 0
#define OR_NORMALIZED 1
#define OR_DECAY 2
#define OR_GATED_DELTA 3
#define OR_VECTOR_DECAY 4
#define OR_KDA 5

#define OR_OK 0
#define OR_BAD_ARG 1
#define OR_NO_MEM 2

int oracle_abi_version(void) { return 1; }

/* One batch-head: the whole sequence, token by token. */
static int run_head(int variant, const double *q, const double *k, const double *v,
                    const double *lg, const double *beta, const double *s_in,
                    const double *z_in, double *o, double *s_out, double *z_out,
                    long L, long dk, long dv)
{
    double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
    double *z = (double *)malloc(sizeof(double) * (size_t)dk);
    double *r = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !z || !r) {
        free(S); free(z); free(r);
        return OR_NO_MEM;
    }
    for (long i = 0; i < dk * dv; ++i) S[i] = s_in ? s_in[i] : 0.0;
    for (long i = 0; i < dk; ++i) z[i] = z_in ? z_in[i] : 0.0;

    for (long t = 0; t < L; ++t) {
        const double *qt = q + t * dk;
        const double *kt = k + t * dk;
        const double *vt = v + t * dv;
        double *ot = o + t * dv;

        if (variant == OR_PLAIN || variant == OR_NORMALIZED) {
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    S[i * dv + j] += kt[i] * vt[j];
            if (variant == OR_NORMALIZED)
                for (long i = 0; i < dk; ++i) z[i] += kt[i];
        } else if (variant == OR_DECAY) {
            double g = exp(lg[t]);
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    S[i * dv + j] = g * S[i * dv + j] + kt[i] * vt[j];
        } else if (variant == OR_VECTOR_DECAY) {
            for (long i = 0; i < dk; ++i) {
                double g = exp(lg[t * dk + i]);
                for (long j = 0; j < dv; ++j)
                    S[i * dv + j] = g * S[i * dv + j] + kt[i] * vt[j];
            }
        } else if (variant == OR_KDA) {
            /* the per-channel decay first, then the delta rule on the decayed state */
            const double bk = beta[t];
            for (long i = 0; i < dk; ++i) {
                const double ai = exp(lg[t * dk + i]);
                for (long j = 0; j < dv; ++j) S[i * dv + j] *= ai;
            }
            for (long j = 0; j < dv; ++j) {
                double rj = 0.0;
                for (long i = 0; i < dk; ++i) rj += kt[i] * S[i * dv + j];
                r[j] = rj;
            }
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    S[i * dv + j] += bk * kt[i] * (vt[j] - r[j]);
        } else { /* OR_GATED_DELTA */
            double a = lg ? exp(lg[t]) : 1.0;
            double b = beta[t];
            for (long j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * kt[i];
                r[j] = acc;
            }
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    S[i * dv + j] = a * (S[i * dv + j] - b * kt[i] * r[j]) + b * kt[i] * vt[j];
        }

        for (long j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i];
            ot[j] = acc;
        }
        if (variant == OR_NORMALIZED) {
            double den = 0.0;
            for (long i = 0; i < dk; ++i) den += qt[i] * z[i];
            for (long j = 0; j < dv; ++j) ot[j] /= den;
        }
    }
    if (s_out) memcpy(s_out, S, sizeof(double) * (size_t)(dk * dv));
    if (z_out) memcpy(z_out, z, sizeof(double) * (size_t)dk);
    free(S); free(z); free(r);
    return OR_OK;
}

/*
 * Full forward over BH independent batch-heads. nthreads <= 0 uses the OpenMP
 * default. Returns OR_OK, OR_BAD_ARG or OR_NO_MEM.
 */
int oracle_forward(int variant, const double *q, const double *k, const double *v,
                   const double *log_gate, const double *beta, const double *state_in,
                   const double *z_in, double *o, double *state_out, double *z_out,
                   long BH, long L, long dk, long dv, int nthreads)
{
    if (variant < OR_PLAIN || variant > OR_KDA) return OR_BAD_ARG;
    if (BH < 0 || L < 0 || dk <= 0 || dv <= 0) return OR_BAD_ARG;
    if ((BH > 0 && L > 0) && (!q || !k || !v || !o)) return OR_BAD_ARG;
    if ((variant == OR_DECAY || variant == OR_VECTOR_DECAY || variant == OR_KDA) && L > 0 && !log_gate)
        return OR_BAD_ARG;
    const long gstride = (variant == OR_VECTOR_DECAY || variant == OR_KDA) ? L * dk : L;
    if ((variant == OR_GATED_DELTA || variant == OR_KDA) && L > 0 && !beta) return OR_BAD_ARG;

    int status = OR_OK;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) reduction(max : status)
#endif
    for (long h = 0; h < BH; ++h) {
        int st = run_head(variant, q + h * L * dk, k + h * L * dk, v + h * L * dv,
                          log_gate ? log_gate + h * gstride : NULL, beta ? beta + h * L : NULL,
                          state_in ? state_in + h * dk * dv : NULL, z_in ? z_in + h * dk : NULL,
                          o + h * L * dv, state_out ? state_out + h * dk * dv : NULL,
                          z_out ? z_out + h * dk : NULL, L, dk, dv);
        if (st > status) status = st;
    }
    return status;
}

/*
 * One-token decode step, in place on the state (tensorplay section 2.2:
 * constant-size state carried from token to token), with the same per-token
 * update as the forward pass:
 *   DECAY (PLAIN: log_gate NULL)  S <- exp(l) S + k v^T            (wln20 decay equation)
 *   VECTOR_DECAY                  S <- Diag(exp(l)) S + k v^T, l [dk] per head
 *   GATED_DELTA                   r = S^T k; S <- a (S - b k r^T) + b k v^T,
 *                                 a = exp(l) (1 when log_gate is NULL), b = beta
 *                                 (wln20 Gated DeltaNet section)
 *   KDA                           S <- Diag(exp(l)) S; r = S^T k; S <- S + b k (v - r)^T,
 *                                 l [dk] per head (wln20 Kimi Delta Attention section)
 * then o = S^T q. Layouts: q, k [NH, dk]; v, o [NH, dv]; log_gate, beta [NH];
 * state [NH, dk, dv] (VECTOR_DECAY, KDA: log_gate [NH, dk]).
 */
int oracle_decode_step(int variant, const double *q, const double *k, const double *v,
                       const double *log_gate, const double *beta, double *state, double *o,
                       long NH, long dk, long dv, int nthreads)
{
    if (variant != OR_PLAIN && variant != OR_DECAY && variant != OR_GATED_DELTA &&
        variant != OR_VECTOR_DECAY && variant != OR_KDA)
        return OR_BAD_ARG;
    if ((variant == OR_DECAY || variant == OR_VECTOR_DECAY || variant == OR_KDA) && !log_gate) return OR_BAD_ARG;
    const long gstride = (variant == OR_VECTOR_DECAY || variant == OR_KDA) ? dk : 1;
    if ((variant == OR_GATED_DELTA || variant == OR_KDA) && !beta) return OR_BAD_ARG;
    if (NH < 0 || dk <= 0 || dv <= 0 || !state) return OR_BAD_ARG;
    int status = OR_OK;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) reduction(max : status)
#endif
    for (long h = 0; h < NH; ++h) {
        int st = run_head(variant, q + h * dk, k + h * dk, v + h * dv,
                          log_gate ? log_gate + h * gstride : NULL, beta ? beta + h : NULL,
                          state + h * dk * dv, NULL, o + h * dv, state + h * dk * dv, NULL, 1, dk, dv);
        if (st > status) status = st;
    }
    return status;
}

/*
 * Causal depthwise short convolution over the token axis, applied to one of the
 * projected q, k or v (wln20 "LLM注意力优化：线性注意力", DeltaNet section: a
 * short convolution after the q/k/v projections mixes each token with its
 * nearest predecessors, kernel size 4 in DeltaNet). Per batch b, head h and
 * channel c, independently ("depthwise"), with tap tau multiplying the input
 * tau tokens back:
 *     y_t[c] = sum_{tau=0}^{K-1} w[h][c][tau] * x_{t-tau}[c]
 * The page writes the taps as w_tau; one set per channel is the depthwise
 * reading. Inputs before the first token come from the sliding window of the K-1
 * previous inputs (state_in, oldest first) or are zero when state_in is NULL.
 * state_out receives the window after the last token: the K-1 most recent
 * inputs, oldest first. No activation is applied.
 * Layouts: x, y [B, H, L, d]; w [H, d, K]; state_in, state_out [B, H, K-1, d].
 * Summation is sequential in tau, in float64.
 */
int oracle_short_conv(const double *x, const double *w, const double *state_in, double *y,
                      double *state_out, long B, long H, long L, long d, long K, int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || d <= 0 || K < 1) return OR_BAD_ARG;
    if (B * H > 0 && L > 0 && (!x || !y || !w)) return OR_BAD_ARG;
    const long W = K - 1;
    int status = OR_OK;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) reduction(max : status)
#endif
    for (long bh = 0; bh < B * H; ++bh) {
        const long h = bh % H;
        /* the whole history of this head: W window values, then the L inputs */
        double *hist = (double *)malloc(sizeof(double) * (size_t)((W + L) * d + 1));
        if (!hist) {
            status = OR_NO_MEM;
            continue;
        }
        for (long j = 0; j < W; ++j)
            for (long c = 0; c < d; ++c)
                hist[j * d + c] = state_in ? state_in[(bh * W + j) * d + c] : 0.0;
        for (long t = 0; t < L; ++t)
            for (long c = 0; c < d; ++c) hist[(W + t) * d + c] = x[(bh * L + t) * d + c];
        for (long t = 0; t < L; ++t)
            for (long c = 0; c < d; ++c) {
                double acc = 0.0;
                for (long tau = 0; tau < K; ++tau)
                    acc += w[(h * d + c) * K + tau] * hist[(W + t - tau) * d + c];
                y[(bh * L + t) * d + c] = acc;
            }
        if (state_out)
            for (long j = 0; j < W; ++j)
                for (long c = 0; c < d; ++c) state_out[(bh * W + j) * d + c] = hist[(L + j) * d + c];
        free(hist);
    }
    return status;
}

/*
 * Backward pass: gradients of a scalar loss through the forward recurrence,
 * given do = dLoss/do_t for every token and (optionally) d_state_out =
 * dLoss/dS_L for the final state. Reverse-mode differentiation of the per-token
 * update, written out step by step (the forward states are kept):
 *   S_t = g_t S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t     (g_t = exp(l_t); PLAIN: 1;
 *                                                        VECTOR_DECAY: Diag(exp(l_t)))
 * Walking t = L .. 1 with dS the gradient of the state after step t:
 *   dS   += q_t do_t^T          (o_t reads S_t)
 *   dq_t  = S_t do_t
 *   dk_t  = dS v_t,   dv_t = dS^T k_t
 *   dl_t  = g_t <dS, S_{t-1}>   (VECTOR_DECAY: per key channel, row by row)
 *   dS    = g_t dS              (gradient of the state before step t)
 * and d_state_in = dS at the end. Variants: PLAIN, DECAY, VECTOR_DECAY.
 * Layouts as in oracle_forward; do like o, d_state_out like state_out;
 * dq, dk like q; dv like v; d_log_gate like log_gate (may be NULL for PLAIN);
 * d_state_in like state_in (NULL = not returned). The recurrence is the one of
 * tensorplay section 2.1 (with the decay of wln20's data-dependent equation and
 * the per-channel gate of tensorplay section 5.1); the derivative rules are
 * those of the products above.
 */
static int bwd_head(int variant, const double *q, const double *k, const double *v,
                    const double *lg, const double *s_in, const double *dout, const double *ds_out,
                    double *dq, double *dk, double *dv, double *dlg, double *ds_in, long L, long dk_,
                    long dv_)
{
    const long D = dk_ * dv_;
    double *S = (double *)malloc(sizeof(double) * (size_t)((L + 1) * D));
    double *dS = (double *)malloc(sizeof(double) * (size_t)D);
    if (!S || !dS) {
        free(S); free(dS);
        return OR_NO_MEM;
    }
    for (long i = 0; i < D; ++i) S[i] = s_in ? s_in[i] : 0.0;
    for (long t = 0; t < L; ++t) {
        const double *Sp = S + t * D;
        double *Sn = S + (t + 1) * D;
        for (long i = 0; i < dk_; ++i) {
            double g = 1.0;
            if (variant == OR_DECAY) g = exp(lg[t]);
            if (variant == OR_VECTOR_DECAY) g = exp(lg[t * dk_ + i]);
            for (long j = 0; j < dv_; ++j)
                Sn[i * dv_ + j] = g * Sp[i * dv_ + j] + k[t * dk_ + i] * v[t * dv_ + j];
        }
    }
    for (long i = 0; i < D; ++i) dS[i] = ds_out ? ds_out[i] : 0.0;
    for (long t = L - 1; t >= 0; --t) {
        const double *qt = q + t * dk_, *kt = k + t * dk_, *vt = v + t * dv_, *dot = dout + t * dv_;
        const double *Sa = S + (t + 1) * D, *Sb = S + t * D;
        for (long i = 0; i < dk_; ++i)
            for (long j = 0; j < dv_; ++j) dS[i * dv_ + j] += qt[i] * dot[j];
        for (long i = 0; i < dk_; ++i) {
            double acc = 0.0;
            for (long j = 0; j < dv_; ++j) acc += Sa[i * dv_ + j] * dot[j];
            dq[t * dk_ + i] = acc;
        }
        for (long i = 0; i < dk_; ++i) {
            double acc = 0.0;
            for (long j = 0; j < dv_; ++j) acc += dS[i * dv_ + j] * vt[j];
            dk[t * dk_ + i] = acc;
        }
        for (long j = 0; j < dv_; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk_; ++i) acc += dS[i * dv_ + j] * kt[i];
            dv[t * dv_ + j] = acc;
        }
        if (variant == OR_DECAY) {
            const double g = exp(lg[t]);
            double acc = 0.0;
            for (long i = 0; i < D; ++i) acc += dS[i] * Sb[i];
            if (dlg) dlg[t] = g * acc;
            for (long i = 0; i < D; ++i) dS[i] *= g;
        } else if (variant == OR_VECTOR_DECAY) {
            for (long i = 0; i < dk_; ++i) {
                const double g = exp(lg[t * dk_ + i]);
                double acc = 0.0;
                for (long j = 0; j < dv_; ++j) acc += dS[i * dv_ + j] * Sb[i * dv_ + j];
                if (dlg) dlg[t * dk_ + i] = g * acc;
                for (long j = 0; j < dv_; ++j) dS[i * dv_ + j] *= g;
            }
        }
    }
    if (ds_in) memcpy(ds_in, dS, sizeof(double) * (size_t)D);
    free(S); free(dS);
    return OR_OK;
}

int oracle_backward(int variant, const double *q, const double *k, const double *v,
                    const double *log_gate, const double *state_in, const double *dout,
                    const double *d_state_out, double *dq, double *dk, double *dv,
                    double *d_log_gate, double *d_state_in, long BH, long L, long dk_, long dv_,
                    int nthreads)
{
    if (variant != OR_PLAIN && variant != OR_DECAY && variant != OR_VECTOR_DECAY) return OR_BAD_ARG;
    if (BH < 0 || L < 0 || dk_ <= 0 || dv_ <= 0) return OR_BAD_ARG;
    if (BH > 0 && L > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv)) return OR_BAD_ARG;
    if (variant != OR_PLAIN && L > 0 && !log_gate) return OR_BAD_ARG;
    const long gstride = variant == OR_VECTOR_DECAY ? L * dk_ : L;
    int status = OR_OK;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) reduction(max : status)
#endif
    for (long h = 0; h < BH; ++h) {
        int st = bwd_head(variant, q + h * L * dk_, k + h * L * dk_, v + h * L * dv_,
                          log_gate ? log_gate + h * gstride : NULL,
                          state_in ? state_in + h * dk_ * dv_ : NULL, dout + h * L * dv_,
                          d_state_out ? d_state_out + h * dk_ * dv_ : NULL, dq + h * L * dk_,
                          dk + h * L * dk_, dv + h * L * dv_, d_log_gate ? d_log_gate + h * gstride : NULL,
                          d_state_in ? d_state_in + h * dk_ * dv_ : NULL, L, dk_, dv_);
        if (st > status) status = st;
    }
    return status;
}

/*
 * Backward pass of the normalized variant for one batch-head, by reverse mode of
 * the per-token recurrence (proig-chaa "线性注意力：从 Softmax Attention 到 Kernel
 * Attention 的本质变化", sections 13-14: the kernel form with its normalizer):
 *   S_t = S_{t-1} + k_t v_t^T,  z_t = z_{t-1} + k_t,
 *   n_t = S_t^T q_t,  den_t = q_t . z_t,  o_t = n_t / den_t.
 * Every state S_0 .. S_L and normalizer z_0 .. z_L is kept. Walking t = L .. 1
 * with G = dLoss/dS_t and Z = dLoss/dz_t (both carried unchanged to t - 1, since
 * S_{t-1} and z_{t-1} enter with the identity):
 *   dn    = do_t / den_t,  dden = -(do_t . n_t) / den_t^2
 *   G    += q_t dn^T,      Z   += dden q_t
 *   dq_t  = S_t dn + dden z_t
 *   dk_t  = G v_t + Z,     dv_t = G^T k_t
 * and finally dS_0 = G, dz_0 = Z.
 */
static int bwd_head_norm(const double *q, const double *k, const double *v, const double *s_in,
                         const double *z_in, const double *dout, const double *ds_out,
                         const double *dz_out, double *dq, double *dk, double *dv, double *ds_in,
                         double *dz_in, long L, long dk_, long dv_)
{
    const long D = dk_ * dv_;
    double *S = (double *)malloc(sizeof(double) * (size_t)((L + 1) * D));
    double *z = (double *)malloc(sizeof(double) * (size_t)((L + 1) * dk_));
    double *G = (double *)malloc(sizeof(double) * (size_t)D);
    double *Z = (double *)malloc(sizeof(double) * (size_t)dk_);
    double *n = (double *)malloc(sizeof(double) * (size_t)dv_);
    double *dn = (double *)malloc(sizeof(double) * (size_t)dv_);
    if (!S || !z || !G || !Z || !n || !dn) {
        free(S); free(z); free(G); free(Z); free(n); free(dn);
        return OR_NO_MEM;
    }
    for (long i = 0; i < D; ++i) S[i] = s_in ? s_in[i] : 0.0;
    for (long i = 0; i < dk_; ++i) z[i] = z_in ? z_in[i] : 0.0;
    for (long t = 0; t < L; ++t) {
        const double *Sp = S + t * D, *zp = z + t * dk_;
        double *Sn = S + (t + 1) * D, *zn = z + (t + 1) * dk_;
        for (long i = 0; i < dk_; ++i) {
            for (long j = 0; j < dv_; ++j) Sn[i * dv_ + j] = Sp[i * dv_ + j] + k[t * dk_ + i] * v[t * dv_ + j];
            zn[i] = zp[i] + k[t * dk_ + i];
        }
    }
    for (long i = 0; i < D; ++i) G[i] = ds_out ? ds_out[i] : 0.0;
    for (long i = 0; i < dk_; ++i) Z[i] = dz_out ? dz_out[i] : 0.0;
    for (long t = L - 1; t >= 0; --t) {
        const double *qt = q + t * dk_, *kt = k + t * dk_, *vt = v + t * dv_, *dot = dout + t * dv_;
        const double *St = S + (t + 1) * D, *zt = z + (t + 1) * dk_;
        double den = 0.0;
        for (long i = 0; i < dk_; ++i) den += qt[i] * zt[i];
        double don = 0.0;
        for (long j = 0; j < dv_; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk_; ++i) acc += St[i * dv_ + j] * qt[i];
            n[j] = acc;
            dn[j] = dot[j] / den;
            don += dot[j] * acc;
        }
        const double dden = -don / (den * den);
        for (long i = 0; i < dk_; ++i) {
            for (long j = 0; j < dv_; ++j) G[i * dv_ + j] += qt[i] * dn[j];
            Z[i] += dden * qt[i];
        }
        for (long i = 0; i < dk_; ++i) {
            double acc = 0.0;
            for (long j = 0; j < dv_; ++j) acc += St[i * dv_ + j] * dn[j];
            dq[t * dk_ + i] = acc + dden * zt[i];
            double gv = 0.0;
            for (long j = 0; j < dv_; ++j) gv += G[i * dv_ + j] * vt[j];
            dk[t * dk_ + i] = gv + Z[i];
        }
        for (long j = 0; j < dv_; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk_; ++i) acc += G[i * dv_ + j] * kt[i];
            dv[t * dv_ + j] = acc;
        }
    }
    if (ds_in) memcpy(ds_in, G, sizeof(double) * (size_t)D);
    if (dz_in) memcpy(dz_in, Z, sizeof(double) * (size_t)dk_);
    free(S); free(z); free(G); free(Z); free(n); free(dn);
    return OR_OK;
}

int oracle_backward_norm(const double *q, const double *k, const double *v, const double *state_in,
                         const double *z_in, const double *dout, const double *d_state_out,
                         const double *d_z_out, double *dq, double *dk, double *dv, double *d_state_in,
                         double *d_z_in, long BH, long L, long dk_, long dv_, int nthreads)
{
    if (BH < 0 || L < 0 || dk_ <= 0 || dv_ <= 0) return OR_BAD_ARG;
    if (BH > 0 && L > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv)) return OR_BAD_ARG;
    int status = OR_OK;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) reduction(max : status)
#endif
    for (long h = 0; h < BH; ++h) {
        int st = bwd_head_norm(q + h * L * dk_, k + h * L * dk_, v + h * L * dv_,
                               state_in ? state_in + h * dk_ * dv_ : NULL, z_in ? z_in + h * dk_ : NULL,
                               dout + h * L * dv_, d_state_out ? d_state_out + h * dk_ * dv_ : NULL,
                               d_z_out ? d_z_out + h * dk_ : NULL, dq + h * L * dk_, dk + h * L * dk_,
                               dv + h * L * dv_, d_state_in ? d_state_in + h * dk_ * dv_ : NULL,
                               d_z_in ? d_z_in + h * dk_ : NULL, L, dk_, dv_);
        if (st > status) status = st;
    }
    return status;
}

/*
 * Backward pass of the gated delta rule for one batch-head, by reverse mode of
 * the per-token recurrence (canonical orientation, as in run_head):
 *   r_t = S_{t-1}^T k_t
 *   S_t = a_t (S_{t-1} - b_t k_t r_t^T) + b_t k_t v_t^T = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T
 *   o_t = S_t^T q_t,   a_t = exp(l_t) (1 without log-gates), b_t = beta_t
 * (wln20 "LLM注意力优化：线性注意力", Gated DeltaNet section; tensorplay section 6.2).
 * Every state S_0 .. S_L is kept (plain, not memory-lean). Walking t = L .. 1
 * with G the gradient of the loss with respect to S_t:
 *   G    += q_t do_t^T                       (o_t reads S_t)
 *   dq_t  = S_t do_t
 *   dv_t  = b G^T k                          (from b k v^T)
 *   dk_t  = b G v - a b (G r + S_{t-1} G^T k) (from b k v^T and -a b k k^T S_{t-1})
 *   db_t  = k^T G (v - a r)
 *   da_t  = <G, S_{t-1}> - b (k^T G) . r,     dl_t = a da_t
 *   G     = a (G - b k (k^T G))              (gradient of S_{t-1}; I - b k k^T is symmetric)
 * and d_state_in = G at the end.
 */
static int bwd_head_gdn(const double *q, const double *k, const double *v, const double *lg,
                        const double *be, const double *s_in, const double *dout,
                        const double *ds_out, double *dq, double *dk, double *dv, double *dlg,
                        double *dbe, double *ds_in, long L, long dk_, long dv_)
{
    const long D = dk_ * dv_;
    double *S = (double *)malloc(sizeof(double) * (size_t)((L + 1) * D));
    double *G = (double *)malloc(sizeof(double) * (size_t)D);
    double *r = (double *)malloc(sizeof(double) * (size_t)dv_);
    double *Gk = (double *)malloc(sizeof(double) * (size_t)dv_);
    if (!S || !G || !r || !Gk) {
        free(S); free(G); free(r); free(Gk);
        return OR_NO_MEM;
    }
    for (long i = 0; i < D; ++i) S[i] = s_in ? s_in[i] : 0.0;
    for (long t = 0; t < L; ++t) {
        const double *Sp = S + t * D, *kt = k + t * dk_, *vt = v + t * dv_;
        double *Sn = S + (t + 1) * D;
        const double a = lg ? exp(lg[t]) : 1.0, b = be[t];
        for (long j = 0; j < dv_; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk_; ++i) acc += Sp[i * dv_ + j] * kt[i];
            r[j] = acc;
        }
        for (long i = 0; i < dk_; ++i)
            for (long j = 0; j < dv_; ++j)
                Sn[i * dv_ + j] = a * (Sp[i * dv_ + j] - b * kt[i] * r[j]) + kt[i] * b * vt[j];
    }
    for (long i = 0; i < D; ++i) G[i] = ds_out ? ds_out[i] : 0.0;
    for (long t = L - 1; t >= 0; --t) {
        const double *qt = q + t * dk_, *kt = k + t * dk_, *vt = v + t * dv_, *dot = dout + t * dv_;
        const double *St = S + (t + 1) * D, *Sp = S + t * D;
        const double a = lg ? exp(lg[t]) : 1.0, b = be[t];
        for (long i = 0; i < dk_; ++i)
            for (long j = 0; j < dv_; ++j) G[i * dv_ + j] += qt[i] * dot[j];
        for (long i = 0; i < dk_; ++i) {
            double acc = 0.0;
            for (long j = 0; j < dv_; ++j) acc += St[i * dv_ + j] * dot[j];
            dq[t * dk_ + i] = acc;
        }
        for (long j = 0; j < dv_; ++j) {
            double rj = 0.0, gk = 0.0;
            for (long i = 0; i < dk_; ++i) {
                rj += Sp[i * dv_ + j] * kt[i];
                gk += G[i * dv_ + j] * kt[i];
            }
            r[j] = rj;
            Gk[j] = gk;
            dv[t * dv_ + j] = b * gk;
        }
        for (long i = 0; i < dk_; ++i) {
            double gv = 0.0, gr = 0.0, sgk = 0.0;
            for (long j = 0; j < dv_; ++j) {
                gv += G[i * dv_ + j] * vt[j];
                gr += G[i * dv_ + j] * r[j];
                sgk += Sp[i * dv_ + j] * Gk[j];
            }
            dk[t * dk_ + i] = b * gv - a * b * (gr + sgk);
        }
        double db = 0.0, gkr = 0.0, gs = 0.0;
        for (long j = 0; j < dv_; ++j) {
            db += Gk[j] * (vt[j] - a * r[j]);
            gkr += Gk[j] * r[j];
        }
        for (long i = 0; i < D; ++i) gs += G[i] * Sp[i];
        if (dbe) dbe[t] = db;
        if (dlg) dlg[t] = a * (gs - b * gkr);
        for (long i = 0; i < dk_; ++i)
            for (long j = 0; j < dv_; ++j)
                G[i * dv_ + j] = a * (G[i * dv_ + j] - b * kt[i] * Gk[j]);
    }
    if (ds_in) memcpy(ds_in, G, sizeof(double) * (size_t)D);
    free(S); free(G); free(r); free(Gk);
    return OR_OK;
}

/*
 * Backward pass of the gated delta rule over BH batch-heads (see bwd_head_gdn).
 * log_gate may be NULL (alpha = 1, DeltaNet); then d_log_gate is not written.
 * Layouts as in oracle_backward; beta and d_beta [BH, L].
 */
int oracle_backward_gdn(const double *q, const double *k, const double *v, const double *log_gate,
                        const double *beta, const double *state_in, const double *dout,
                        const double *d_state_out, double *dq, double *dk, double *dv,
                        double *d_log_gate, double *d_beta, double *d_state_in, long BH, long L,
                        long dk_, long dv_, int nthreads)
{
    if (BH < 0 || L < 0 || dk_ <= 0 || dv_ <= 0) return OR_BAD_ARG;
    if (BH > 0 && L > 0 && (!q || !k || !v || !beta || !dout || !dq || !dk || !dv)) return OR_BAD_ARG;
    int status = OR_OK;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) reduction(max : status)
#endif
    for (long h = 0; h < BH; ++h) {
        int st = bwd_head_gdn(q + h * L * dk_, k + h * L * dk_, v + h * L * dv_,
                              log_gate ? log_gate + h * L : NULL, beta + h * L,
                              state_in ? state_in + h * dk_ * dv_ : NULL, dout + h * L * dv_,
                              d_state_out ? d_state_out + h * dk_ * dv_ : NULL, dq + h * L * dk_,
                              dk + h * L * dk_, dv + h * L * dv_,
                              (d_log_gate && log_gate) ? d_log_gate + h * L : NULL,
                              d_beta ? d_beta + h * L : NULL,
                              d_state_in ? d_state_in + h * dk_ * dv_ : NULL, L, dk_, dv_);
        if (st > status) status = st;
    }
    return status;
}
