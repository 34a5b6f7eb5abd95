/*
 * libesa.so used from plain C, with no Python or torch: device buffers from hipMalloc, a
 * stream from hipStreamCreate, the workspace zeroed with esa_workspace_init, then
 * esa_scan_fwd, esa_scan_bwd and esa_state_step on fp32 problems.  Every result is checked
 * against the oracle's C entry points (liboracle_esa.so, test infrastructure) with the fp32
 * parity bar: max |x - r| / max(|r|, rms(r)) <= 1e-5.
 *
 * Inputs are seeded N(mu, sigma) draws (xorshift64 and the Box-Muller transform).  Cases:
 * the 256-step fp32 workload (B=1, T=256, H=2, Dh=16, direct, a, v, q ~ N(0, 1), zero
 * initial state) and a many-tile controlled problem with a ragged tail, an initial state
 * and an upstream state gradient.
 *
 * Exit status: 0 when every check passes, 1 when a result misses the bar, 2 on an error.
 * Built by __graft_entry__.build() into tests/_bin/; run by tests/test_gpu_c_abi.py.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "esa.h"

int oracle_scan_fwd(int64_t, int64_t, int64_t, int64_t, int64_t, int, const double *,
                    const double *, const double *, const double *, double *, double *,
                    double *);
int oracle_scan_bwd(int64_t, int64_t, int64_t, int64_t, int64_t, int, const double *,
                    const double *, const double *, const double *, const double *,
                    const double *, double *, double *, double *, double *);
void oracle_state_step(int64_t, int64_t, int64_t, int, const double *, const double *,
                       const double *, double *, double *);

#define HIP_OK(x)                                                                          \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                \
            exit(2);                                                                       \
        }                                                                                  \
    } while (0)
#define ESA_OK_(x)                                                                         \
    do {                                                                                   \
        int s_ = (x);                                                                      \
        if (s_ != ESA_OK) {                                                                \
            fprintf(stderr, "%s failed: %s\n", #x, esa_status_string(s_));                \
            exit(2);                                                                       \
        }                                                                                  \
    } while (0)

static uint64_t rng;

static double uniform01(void) /* xorshift64, in (0, 1) */
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return ((double)(rng >> 11) + 0.5) / 9007199254740992.0;
}

static double normal(double mu, double sigma) /* Box-Muller */
{
    const double u1 = uniform01(), u2 = uniform01();
    return mu + sigma * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static float *draws(int64_t n, double mu, double sigma)
{
    float *p = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!p)
        exit(2);
    for (int64_t i = 0; i < n; ++i)
        p[i] = (float)normal(mu, sigma);
    return p;
}

static double *widen(const float *x, int64_t n)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!p)
        exit(2);
    for (int64_t i = 0; i < n; ++i)
        p[i] = x ? (double)x[i] : 0.0;
    return p;
}

static float *to_device(const float *h, int64_t n)
{
    float *d = NULL;
    HIP_OK(hipMalloc((void **)&d, sizeof(float) * (size_t)(n > 0 ? n : 1)));
    if (h)
        HIP_OK(hipMemcpy(d, h, sizeof(float) * (size_t)n, hipMemcpyHostToDevice));
    return d;
}

static double compare(const char *name, const float *dev, const double *ref, int64_t n)
{
    float *h = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!h)
        exit(2);
    HIP_OK(hipMemcpy(h, dev, sizeof(float) * (size_t)n, hipMemcpyDeviceToHost));
    double ss = 0.0, worst = 0.0;
    for (int64_t i = 0; i < n; ++i)
        ss += ref[i] * ref[i];
    const double rms = sqrt(ss / (double)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        const double den = fabs(ref[i]) > rms ? fabs(ref[i]) : rms;
        const double e = den > 0.0 ? fabs((double)h[i] - ref[i]) / den : fabs((double)h[i]);
        if (!(e <= worst))
            worst = e; /* a NaN result makes worst NaN, which fails the bar below */
    }
    printf("  %-12s max err %.3e\n", name, worst);
    free(h);
    return worst;
}

/* One fp32 problem: forward, backward and a decode step from its final state.  Returns the
 * largest error of any output. */
static double run_case(int64_t B, int64_t T, int64_t H, int64_t Dh, int mode, int with_states,
                       double a_mu, uint64_t seed, hipStream_t s)
{
    rng = seed;
    const int64_t C = H * Dh, n = B * T * C, ns = B * C;
    printf("case B=%lld T=%lld H=%lld Dh=%lld %s%s\n", (long long)B, (long long)T, (long long)H,
           (long long)Dh, mode == ESA_DIRECT ? "direct" : "controlled",
           with_states ? ", initial state and upstream state gradient" : "");
    float *a = draws(n, a_mu, 1.0), *v = draws(n, 0.0, 1.0), *q = draws(n, 0.0, 1.0);
    float *dy = draws(n, 0.0, 1.0);
    float *e0 = with_states ? draws(ns, 0.0, 1.0) : NULL;
    float *dET = with_states ? draws(ns, 0.0, 1.0) : NULL;
    float *sa = draws(ns, a_mu, 1.0), *sv = draws(ns, 0.0, 1.0), *sq = draws(ns, 0.0, 1.0);

    float *d_a = to_device(a, n), *d_v = to_device(v, n), *d_q = to_device(q, n);
    float *d_dy = to_device(dy, n);
    float *d_e0 = e0 ? to_device(e0, ns) : NULL, *d_dET = dET ? to_device(dET, ns) : NULL;
    float *d_y = to_device(NULL, n), *d_eT = to_device(NULL, ns);
    float *d_da = to_device(NULL, n), *d_dv = to_device(NULL, n), *d_dq = to_device(NULL, n);
    float *d_de0 = to_device(NULL, ns);
    float *d_sa = to_device(sa, ns), *d_sv = to_device(sv, ns), *d_sq = to_device(sq, ns);
    float *d_sy = to_device(NULL, ns);
    const size_t ckb = esa_scan_ckpt_bytes(B, T, H, Dh);
    const size_t wsb = esa_scan_workspace_bytes(B, T, H, Dh, ESA_F32);
    if (ckb == 0 || wsb == 0) {
        fprintf(stderr, "size query failed\n");
        exit(2);
    }
    float *d_ck = NULL;
    void *d_ws = NULL;
    HIP_OK(hipMalloc((void **)&d_ck, ckb));
    HIP_OK(hipMalloc(&d_ws, wsb));

    ESA_OK_(esa_workspace_init(d_ws, wsb, s));
    ESA_OK_(esa_scan_fwd(B, T, H, Dh, ESA_F32, mode, d_a, d_v, d_q, d_e0, d_y, d_eT, d_ck, d_ws,
                         wsb, s));
    ESA_OK_(esa_scan_bwd(B, T, H, Dh, ESA_F32, mode, d_a, d_v, d_q, d_e0, d_dy, d_dET, d_ck, d_da,
                         d_dv, d_dq, d_de0, d_ws, wsb, s));
    /* the decode step continues from the forward's final state, in place */
    ESA_OK_(esa_state_step(B, H, Dh, ESA_F32, mode, d_sa, d_sv, d_sq, d_eT, d_sy, s));
    HIP_OK(hipStreamSynchronize(s));
    uint32_t abort_word = 0;
    HIP_OK(hipMemcpy(&abort_word, (char *)d_ws + 12, 4, hipMemcpyDeviceToHost));
    if (abort_word != 0) {
        fprintf(stderr, "look-back wait timed out\n");
        exit(2);
    }

    double *xa = widen(a, n), *xv = widen(v, n), *xq = widen(q, n), *xdy = widen(dy, n);
    double *xe0 = e0 ? widen(e0, ns) : NULL, *xdET = dET ? widen(dET, ns) : NULL;
    double *ry = widen(NULL, n), *reT = widen(NULL, ns);
    double *rda = widen(NULL, n), *rdv = widen(NULL, n), *rdq = widen(NULL, n);
    double *rde0 = widen(NULL, ns);
    double *xsa = widen(sa, ns), *xsv = widen(sv, ns), *xsq = widen(sq, ns);
    double *rsy = widen(NULL, ns);
    if (oracle_scan_fwd(0, B, T, H, Dh, mode, xa, xv, xq, xe0, ry, reT, NULL) ||
        oracle_scan_bwd(0, B, T, H, Dh, mode, xa, xv, xq, xe0, xdy, xdET, rda, rdv, rdq, rde0)) {
        fprintf(stderr, "oracle ran out of memory\n");
        exit(2);
    }
    oracle_state_step(B, H, Dh, mode, xsa, xsv, xsq, reT, rsy); /* reT becomes the new state */

    double worst = 0.0, e;
    const char *names[] = {"y", "d_logit", "d_value", "d_query"};
    const float *got[] = {d_y, d_da, d_dv, d_dq};
    const double *ref[] = {ry, rda, rdv, rdq};
    for (int k = 0; k < 4; ++k)
        if (!((e = compare(names[k], got[k], ref[k], n)) <= worst))
            worst = e;
    if (!((e = compare("d_init", d_de0, rde0, ns)) <= worst))
        worst = e;
    if (!((e = compare("step y", d_sy, rsy, ns)) <= worst))
        worst = e;
    if (!((e = compare("step state", d_eT, reT, ns)) <= worst))
        worst = e;

    float *hp[] = {a, v, q, dy, e0, dET, sa, sv, sq};
    for (int k = 0; k < 9; ++k)
        free(hp[k]);
    double *dp[] = {xa, xv, xq, xdy, xe0, xdET, ry, reT, rda, rdv, rdq, rde0, xsa, xsv, xsq, rsy};
    for (int k = 0; k < 16; ++k)
        free(dp[k]);
    void *gp[] = {d_a, d_v, d_q, d_dy, d_e0, d_dET, d_y, d_eT, d_da, d_dv, d_dq,
                  d_de0, d_sa, d_sv, d_sq, d_sy, d_ck, d_ws};
    for (int k = 0; k < 18; ++k)
        if (gp[k])
            HIP_OK(hipFree(gp[k]));
    return worst;
}

int main(void)
{
    if (esa_abi_version() != ESA_ABI_VERSION) {
        fprintf(stderr, "header and library ABI versions differ\n");
        return 2;
    }
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    double worst = run_case(1, 256, 2, 16, ESA_DIRECT, 0, 0.0, 0x9e3779b97f4a7c15ull, s);
    const double w2 = run_case(2, 3001, 2, 64, ESA_CONTROLLED, 1, 1.0, 0xd1b54a32d192ed03ull, s);
    if (!(w2 <= worst))
        worst = w2;
    HIP_OK(hipStreamDestroy(s));
    const int pass = worst <= 1e-5;
    printf("%s: worst error %.3e (bar 1e-5)\n", pass ? "PASS" : "FAIL", worst);
    return pass ? 0 : 1;
}
