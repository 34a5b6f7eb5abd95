/*
 * Oracle for the gated linear recurrence of Entangled State Attention (ESA).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, sequential fp64 statement of what
 * the GPU library computes.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg load it; the product path never does.  It shares no source, header, table or
 * helper with the HIP library, and it includes nothing from it.
 *
 * What it follows (the ESA web pages):
 *   - page "entangled-state-attention 0.1.0" (PyPI project page), section "Core idea":
 *       direct form      A_t = sigma(x_t W_A),  V_t = x_t W_V,  E_t = A_t (.) E_{t-1} + V_t
 *       readout          q_t = x_t W_Q,  y_t = W_O (q_t (.) Norm(E_t))
 *       controlled form  g_t = sigma(x_t W_g),  E_t = g_t (.) E_{t-1} + (1 - g_t) (.) V_t
 *   - page "Entangled State Attention v2.1" (PKG-INFO of the 2.1.0 sdist), introduction:
 *       the general elementwise recurrence E_t = A_t (.) E_{t-1} + B_t.
 *   - page "Entangled State Attention" (mlbricks-web.pages.dev/esa), section
 *       "[ ARCHITECTURE ]": the recurrence is composed over the sequence to a compact final
 *       state, then carried one token at a time ("One-token update").
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - "Norm" is a per-head RMSNorm over the Dh channels of one (b, t, h):
 *       n = E / sqrt(mean_d(E^2) + 1e-6), with no learnable gain.
 *   - the readout uses the post-update state E_t (the state that already includes token t).
 *   - the inputs are the projected quantities: gate logits a (= x W_A or x W_g), values V
 *     and queries q, each laid out [B, T, H, Dh] with Dh fastest; W_O is outside.
 *   - the initial state E_{-1} is zero unless an initial state is given.
 *   - the backward pass is the chain rule applied to the forward definition; no page
 *     states it.
 *
 * Everything is fp64 with no blocking, fusion or reordering: one sequential loop over t
 * per lane.  Build with floating-point contraction off so that every multiply and add is
 * rounded as written.
 *
 * Parity pins (tests/test_oracle_*.py): O(T^2) closed form, A = 0, A = 1 (prefix sum),
 * constant-A geometric series, bracketing invariance of the pair combine, library RMSNorm,
 * library logistic function, central finite differences and the adjoint identity for the
 * backward, scan/step equivalence, causality and resume.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EPS 1e-6 /* RMSNorm epsilon (a fixed reading: the pages leave Norm undefined) */

/* Logistic function sigma(x) = 1 / (1 + exp(-x)), evaluated on the side where exp()
 * cannot overflow.  1 - sigma(x) is always taken as sigma(-x). */
static double sigmoid(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

double oracle_sigmoid(double x) { return sigmoid(x); }

/* Core recurrence E_t = A_t * E_{t-1} + B_t ("Entangled State Attention v2.1", introduction;
 * "Entangled State Attention", "[ ARCHITECTURE ]" core recurrence), run over nl independent
 * lanes.  A, Bt, E are [T][nl]; E0 is [nl] or NULL for a zero initial state. */
void oracle_recurrence(int64_t T, int64_t nl, const double *A, const double *Bt,
                       const double *E0, double *E)
{
    for (int64_t l = 0; l < nl; ++l) {
        double e = E0 ? E0[l] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            e = A[t * nl + l] * e + Bt[t * nl + l];
            E[t * nl + l] = e;
        }
    }
}

/* Gate coefficients ("entangled-state-attention 0.1.0", "Core idea"):
 *   mode 0, direct:      A = sigma(a), B = v
 *   mode 1, controlled:  A = g = sigma(a), B = (1 - g) * v with 1 - g = sigma(-a). */
void oracle_gates(int64_t n, int mode, const double *a, const double *v, double *A, double *Bt)
{
    for (int64_t i = 0; i < n; ++i) {
        A[i] = sigmoid(a[i]);
        Bt[i] = (mode == 0) ? v[i] : sigmoid(-a[i]) * v[i];
    }
}

/* Readout y = q * Norm(E) ("entangled-state-attention 0.1.0", "Core idea", readout equation,
 * without W_O), with Norm read as RMSNorm over each group of Dh consecutive channels. */
void oracle_readout(int64_t ngroups, int64_t Dh, const double *E, const double *q, double *y)
{
    for (int64_t g = 0; g < ngroups; ++g) {
        const double *e = E + g * Dh;
        double ss = 0.0;
        for (int64_t d = 0; d < Dh; ++d)
            ss += e[d] * e[d];
        double r = 1.0 / sqrt(ss / (double)Dh + ORACLE_EPS);
        for (int64_t d = 0; d < Dh; ++d)
            y[g * Dh + d] = q[g * Dh + d] * (e[d] * r);
    }
}

/* Forward scan of one batch row: a, v, q, y are [T][C] (C = H*Dh), e0 and eT are [C].
 * E_all, if not NULL, receives every state E_t ([T][C]). */
static int scan_fwd_row(int64_t T, int64_t H, int64_t Dh, int mode, const double *a,
                        const double *v, const double *q, const double *e0, double *y,
                        double *eT, double *E_all)
{
    const int64_t C = H * Dh;
    const int64_t n = T * C;
    double *A = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *Bt = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *E = E_all ? E_all : (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!A || !Bt || !E) {
        free(A);
        free(Bt);
        if (!E_all)
            free(E);
        return -1;
    }
    oracle_gates(n, mode, a, v, A, Bt);
    oracle_recurrence(T, C, A, Bt, e0, E);
    if (y)
        oracle_readout(T * H, Dh, E, q, y);
    if (eT) {
        for (int64_t c = 0; c < C; ++c)
            eT[c] = (T > 0) ? E[(T - 1) * C + c] : (e0 ? e0[c] : 0.0);
    }
    free(A);
    free(Bt);
    if (!E_all)
        free(E);
    return 0;
}

/* Forward over batch rows [b0, b1) of a [B, T, H, Dh] problem.  Pointers address the full
 * tensors; e0 / eT / E_all may be NULL.  Returns 0, or -1 if memory ran out. */
int oracle_scan_fwd(int64_t b0, int64_t b1, int64_t T, int64_t H, int64_t Dh, int mode,
                    const double *a, const double *v, const double *q, const double *e0,
                    double *y, double *eT, double *E_all)
{
    const int64_t C = H * Dh;
    for (int64_t b = b0; b < b1; ++b) {
        const int64_t o = b * T * C;
        int rc = scan_fwd_row(T, H, Dh, mode, a + o, v + o, q ? q + o : NULL,
                              e0 ? e0 + b * C : NULL, y ? y + o : NULL, eT ? eT + b * C : NULL,
                              E_all ? E_all + o : NULL);
        if (rc)
            return rc;
    }
    return 0;
}

/* Backward of the forward scan over batch rows [b0, b1): the chain rule taken through
 * gates, recurrence and readout, in reverse time order.
 *   inputs : a, v, q, dy  [B,T,H,Dh];  e0, dET  [B,H,Dh] or NULL (zero)
 *   outputs: da, dv, dq   [B,T,H,Dh];  de0      [B,H,Dh] or NULL
 * Per (b, t, h), with n = E_t * r, r = (mean_d E_t^2 + eps)^(-1/2):
 *   dq = dy * n,  dn = dy * q,  gE = r * (dn - n * mean_d(dn * n))
 * Reverse recurrence, lam entering at t = T-1 equal to dET:
 *   dE_t = gE_t + lam,  lam <- A_t * dE_t;  de0 = lam after t = 0.
 *   direct:     da_t = dE_t * E_{t-1} * s_t * (1 - s_t),          dv_t = dE_t
 *   controlled: da_t = dE_t * (E_{t-1} - v_t) * s_t * (1 - s_t),  dv_t = dE_t * (1 - s_t)
 * with s_t = sigma(a_t) and 1 - s_t = sigma(-a_t).  Returns 0, or -1 if memory ran out. */
int oracle_scan_bwd(int64_t b0, int64_t b1, int64_t T, int64_t H, int64_t Dh, int mode,
                    const double *a, const double *v, const double *q, const double *e0,
                    const double *dy, const double *dET, double *da, double *dv, double *dq,
                    double *de0)
{
    const int64_t C = H * Dh;
    const int64_t n = T * C;
    double *E = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *gE = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *lam = (double *)malloc(sizeof(double) * (size_t)C);
    if (!E || !gE || !lam) {
        free(E);
        free(gE);
        free(lam);
        return -1;
    }
    for (int64_t b = b0; b < b1; ++b) {
        const int64_t o = b * T * C;
        const double *ab = a + o, *vb = v + o, *qb = q + o, *dyb = dy + o;
        const double *e0b = e0 ? e0 + b * C : NULL;
        int rc = scan_fwd_row(T, H, Dh, mode, ab, vb, qb, e0b, NULL, NULL, E);
        if (rc) {
            free(E);
            free(gE);
            free(lam);
            return rc;
        }
        /* readout backward, one (t, h) group at a time */
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t h = 0; h < H; ++h) {
                const int64_t g = t * C + h * Dh;
                double ss = 0.0;
                for (int64_t d = 0; d < Dh; ++d)
                    ss += E[g + d] * E[g + d];
                const double r = 1.0 / sqrt(ss / (double)Dh + ORACLE_EPS);
                double dnn = 0.0;
                for (int64_t d = 0; d < Dh; ++d) {
                    const double nd = E[g + d] * r;
                    dq[o + g + d] = dyb[g + d] * nd;
                    dnn += (dyb[g + d] * qb[g + d]) * nd;
                }
                const double mu = dnn / (double)Dh;
                for (int64_t d = 0; d < Dh; ++d) {
                    const double nd = E[g + d] * r;
                    const double dn = dyb[g + d] * qb[g + d];
                    gE[g + d] = r * (dn - nd * mu);
                }
            }
        }
        /* reverse recurrence */
        for (int64_t c = 0; c < C; ++c)
            lam[c] = dET ? dET[b * C + c] : 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            for (int64_t c = 0; c < C; ++c) {
                const int64_t i = t * C + c;
                const double dE = gE[i] + lam[c];
                const double s = sigmoid(ab[i]);
                const double u = sigmoid(-ab[i]);
                const double Eprev = (t > 0) ? E[i - C] : (e0b ? e0b[c] : 0.0);
                if (mode == 0) {
                    da[o + i] = dE * Eprev * s * u;
                    dv[o + i] = dE;
                } else {
                    da[o + i] = dE * (Eprev - vb[i]) * s * u;
                    dv[o + i] = dE * u;
                }
                lam[c] = s * dE;
            }
        }
        if (de0)
            for (int64_t c = 0; c < C; ++c)
                de0[b * C + c] = lam[c];
    }
    free(E);
    free(gE);
    free(lam);
    return 0;
}

/* One-token recurrent update with readout ("Entangled State Attention", "[ ARCHITECTURE ]",
 * "One-token update"; "Entangled State Attention v2.1", section 5, lightning_step):
 * per lane  E <- A * E + B  with the gates above, then y = q * Norm(E).
 * a, v, q, y are [B, H, Dh]; state is [B, H, Dh], updated in place. */
void oracle_state_step(int64_t B, int64_t H, int64_t Dh, int mode, const double *a,
                       const double *v, const double *q, double *state, double *y)
{
    const int64_t n = B * H * Dh;
    for (int64_t i = 0; i < n; ++i) {
        const double s = sigmoid(a[i]);
        const double bt = (mode == 0) ? v[i] : sigmoid(-a[i]) * v[i];
        state[i] = s * state[i] + bt;
    }
    for (int64_t g = 0; g < B * H; ++g) {
        const double *e = state + g * Dh;
        double ss = 0.0;
        for (int64_t d = 0; d < Dh; ++d)
            ss += e[d] * e[d];
        const double r = 1.0 / sqrt(ss / (double)Dh + ORACLE_EPS);
        for (int64_t d = 0; d < Dh; ++d)
            y[g * Dh + d] = q[g * Dh + d] * (e[d] * r);
    }
}

double oracle_rmsnorm_eps(void) { return ORACLE_EPS; }
