/*
 * Driver for the sanitizer build of the fp64 oracle (test infrastructure): calls
 * every oracle entry point on small seeded inputs, with and without the optional
 * arguments, empty sequences and one-token sequences, so that AddressSanitizer
 * and UndefinedBehaviorSanitizer see every loop of the oracle run. Exits 0 when
 * every call returns its expected status.
 */
#include <stdio.h>
#include <stdlib.h>

int oracle_forward(int variant, const double *q, const double *k, const double *v,
                   const double *log_gate, const double *beta, const double *state_in,
                   const double *z_in, double *o, double *state_out, double *z_out,
                   long BH, long L, long dk, long dv, int nthreads);
int oracle_decode_step(int variant, const double *q, const double *k, const double *v,
                       const double *log_gate, const double *beta, double *state, double *o,
                       long NH, long dk, long dv, int nthreads);
int oracle_short_conv(const double *x, const double *w, const double *state_in, double *y,
                      double *state_out, long B, long H, long L, long d, long K, int nthreads);
int oracle_backward(int variant, const double *q, const double *k, const double *v,
                    const double *log_gate, const double *state_in, const double *dout,
                    const double *d_state_out, double *dq, double *dk, double *dv,
                    double *d_log_gate, double *d_state_in, long BH, long L, long dk_, long dv_,
                    int nthreads);
int oracle_backward_gdn(const double *q, const double *k, const double *v, const double *log_gate,
                        const double *beta, const double *state_in, const double *dout,
                        const double *d_state_out, double *dq, double *dk, double *dv,
                        double *d_log_gate, double *d_beta, double *d_state_in, long BH, long L,
                        long dk_, long dv_, int nthreads);

static unsigned long long seed = 88172645463325252ull;
static double rnd(void) {  /* xorshift64, in [-1, 1) */
    seed ^= seed << 13; seed ^= seed >> 7; seed ^= seed << 17;
    return (double)(seed >> 11) / (double)(1ull << 52) - 1.0;
}
/* exactly n doubles on the heap, so any read or write past them is reported */
static double *arr(long n, double lo, double hi) {
    double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (rnd() + 1.0);
    return p;
}

static int fails = 0;
static void expect(int got, int want, const char *what) {
    if (got != want) {
        fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
        ++fails;
    }
}

int main(void) {
    const long BH = 3, dk = 5, dv = 3;
    const long Ls[] = {0, 1, 7};
    for (int li = 0; li < 3; ++li) {
        const long L = Ls[li];
        double *q = arr(BH * L * dk, -1, 1), *k = arr(BH * L * dk, -1, 1), *v = arr(BH * L * dv, -1, 1);
        double *lg = arr(BH * L, -1, 0), *lgv = arr(BH * L * dk, -1, 0), *be = arr(BH * L, 0, 1);
        double *s0 = arr(BH * dk * dv, -1, 1), *z0 = arr(BH * dk, 1, 2), *pos = arr(BH * L * dk, 0.1, 1);
        double *o = arr(BH * L * dv, 0, 0), *s1 = arr(BH * dk * dv, 0, 0), *z1 = arr(BH * dk, 0, 0);
        double *dO = arr(BH * L * dv, -1, 1), *dso = arr(BH * dk * dv, -1, 1);
        double *gq = arr(BH * L * dk, 0, 0), *gk = arr(BH * L * dk, 0, 0), *gv = arr(BH * L * dv, 0, 0);
        double *gl = arr(BH * L * dk, 0, 0), *gb = arr(BH * L, 0, 0), *gs = arr(BH * dk * dv, 0, 0);
        for (int var = 0; var <= 4; ++var) {
            const double *g = var == 4 ? lgv : (var == 2 || var == 3 ? lg : NULL);
            const double *qq = var == 1 ? pos : q, *kk = var == 1 ? pos : k;
            expect(oracle_forward(var, qq, kk, v, g, var == 3 ? be : NULL, s0, var == 1 ? z0 : NULL, o, s1,
                                  var == 1 ? z1 : NULL, BH, L, dk, dv, 1), 0, "forward");
            expect(oracle_forward(var, qq, kk, v, g, var == 3 ? be : NULL, NULL, NULL, o, NULL, NULL,
                                  BH, L, dk, dv, 1), 0, "forward, no state");
        }
        expect(oracle_forward(2, q, k, v, NULL, NULL, NULL, NULL, o, NULL, NULL, BH, L, dk, dv, 1),
               L > 0 ? 1 : 0, "decay without gates");
        for (int var = 0; var <= 4; ++var) {
            if (var == 1) continue;  /* the normalized variant has no decode step */
            const double *g = var == 4 ? lgv : (var == 0 ? NULL : lg);
            if (L > 0) expect(oracle_decode_step(var, q, k, v, g, var == 3 ? be : NULL, s1, o, BH, dk, dv, 1),
                              0, "decode");
        }
        for (long K = 1; K <= 4; ++K) {
            double *w = arr(BH * dk * K, -1, 1), *win = arr(BH * (K - 1) * dk, -1, 1);
            double *wout = arr(BH * (K - 1) * dk, 0, 0);
            expect(oracle_short_conv(q, w, win, gq, wout, 1, BH, L, dk, K, 1), 0, "short conv");
            expect(oracle_short_conv(q, w, NULL, gq, NULL, 1, BH, L, dk, K, 1), 0, "short conv, no window");
            free(w); free(win); free(wout);
        }
        expect(oracle_backward(0, q, k, v, NULL, s0, dO, dso, gq, gk, gv, NULL, gs, BH, L, dk, dv, 1), 0, "bwd plain");
        expect(oracle_backward(2, q, k, v, lg, NULL, dO, NULL, gq, gk, gv, gl, NULL, BH, L, dk, dv, 1), 0, "bwd decay");
        expect(oracle_backward(4, q, k, v, lgv, s0, dO, dso, gq, gk, gv, gl, gs, BH, L, dk, dv, 1), 0, "bwd vector");
        expect(oracle_backward_gdn(q, k, v, lg, be, s0, dO, dso, gq, gk, gv, gl, gb, gs, BH, L, dk, dv, 1), 0,
               "bwd gated delta");
        expect(oracle_backward_gdn(q, k, v, NULL, be, NULL, dO, NULL, gq, gk, gv, gl, NULL, NULL, BH, L, dk, dv, 1),
               0, "bwd deltanet");
        free(q); free(k); free(v); free(lg); free(lgv); free(be); free(s0); free(z0); free(pos);
        free(o); free(s1); free(z1); free(dO); free(dso); free(gq); free(gk); free(gv); free(gl);
        free(gb); free(gs);
    }
    if (fails) return 1;
    puts("sanitized oracle: every call ok");
    return 0;
}
