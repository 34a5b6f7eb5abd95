"""Address and undefined-behaviour sanitizers over the host-side code, on the CPU.

1. The oracle's C, built with gcc -fsanitize=address,undefined, driven through every entry
   point over small shapes (T = 0 and 1, Dh = 1 and 128, both modes, optional initial
   state and upstream gradient), including pointer sets where the optional outputs are NULL.
2. The library's host code (argument validation, workspace layout, dispatch tables), built
   with the sanitizers on the host pass only (-Xarch_host before each -fsanitize; the
   device code is built as usual) and driven through every entry point with arguments that
   fail validation, which returns before any HIP call, plus every size query.  No kernel is
   launched and no GPU is needed.

Any sanitizer report aborts the driver with a non-zero status.
"""
import os
import shutil
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "esa_oracle.c")
CSRC = os.path.join(ROOT, "gated_linear_recurrence_chunked_amd", "csrc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

ORACLE_DRIVER = textwrap.dedent(r"""
    #include <stdint.h>
    #include <stdio.h>
    #include <stdlib.h>
    int oracle_scan_fwd(int64_t, int64_t, int64_t, int64_t, int64_t, int, const double *,
                        const double *, const double *, const double *, double *, double *,
                        double *);
    int oracle_scan_bwd(int64_t, int64_t, int64_t, int64_t, int64_t, int, const double *,
                        const double *, const double *, const double *, const double *,
                        const double *, double *, double *, double *, double *);
    void oracle_state_step(int64_t, int64_t, int64_t, int, const double *, const double *,
                           const double *, double *, double *);
    void oracle_recurrence(int64_t, int64_t, const double *, const double *, const double *,
                           double *);
    void oracle_gates(int64_t, int, const double *, const double *, double *, double *);
    void oracle_readout(int64_t, int64_t, const double *, const double *, double *);
    static uint64_t st = 88172645463325252ull;
    static double rnd(void) {  /* xorshift64, uniform in [-2, 2) */
        st ^= st << 13; st ^= st >> 7; st ^= st << 17;
        return (double)(st >> 11) / 9007199254740992.0 * 4.0 - 2.0;
    }
    static double *arr(int64_t n) {  /* exactly n elements, so an overrun is reported */
        double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        for (int64_t i = 0; i < n; ++i) p[i] = rnd();
        return p;
    }
    int main(void) {
        const int64_t shapes[][4] = {{1, 0, 1, 16}, {1, 1, 1, 1}, {2, 5, 3, 4},
                                     {3, 17, 2, 16}, {1, 9, 1, 128}};
        for (int s = 0; s < 5; ++s) {
            const int64_t B = shapes[s][0], T = shapes[s][1], H = shapes[s][2], Dh = shapes[s][3];
            const int64_t C = H * Dh, n = B * T * C, ns = B * C;
            for (int mode = 0; mode < 2; ++mode) {
                for (int opt = 0; opt < 2; ++opt) {
                    double *a = arr(n), *v = arr(n), *q = arr(n), *dy = arr(n);
                    double *e0 = opt ? arr(ns) : NULL, *dET = opt ? arr(ns) : NULL;
                    double *y = arr(n), *eT = arr(ns), *E = arr(n);
                    double *da = arr(n), *dv = arr(n), *dq = arr(n), *de0 = arr(ns);
                    if (oracle_scan_fwd(0, B, T, H, Dh, mode, a, v, q, e0, y, eT, E)) return 2;
                    if (oracle_scan_fwd(0, B, T, H, Dh, mode, a, v, NULL, e0, NULL,
                                        opt ? eT : NULL, NULL)) return 3;
                    if (oracle_scan_bwd(0, B, T, H, Dh, mode, a, v, q, e0, dy, dET, da, dv,
                                        dq, opt ? de0 : NULL)) return 4;
                    if (T > 0) {
                        double *st0 = arr(ns), *ys = arr(ns);
                        oracle_state_step(B, H, Dh, mode, a, v, q, st0, ys);
                        free(st0); free(ys);
                        double *A = arr(n), *Bt = arr(n), *R = arr(n);
                        oracle_gates(n, mode, a, v, A, Bt);
                        oracle_recurrence(B * T, C, A, Bt, opt ? e0 : NULL, R);
                        oracle_readout(B * T * H, Dh, R, q, y);
                        free(A); free(Bt); free(R);
                    }
                    free(a); free(v); free(q); free(dy); free(e0); free(dET); free(y);
                    free(eT); free(E); free(da); free(dv); free(dq); free(de0);
                }
            }
        }
        puts("oracle ok");
        return 0;
    }
""")

HOST_DRIVER = textwrap.dedent(r"""
    #include <stdint.h>
    #include <stdio.h>
    #include <string.h>
    #include "esa.h"
    #define CHECK(expr, want) do { int got_ = (expr); if (got_ != (want)) { \
        printf("%s: got %d want %d\n", #expr, got_, (want)); return 1; } } while (0)
    static void *A(int k) { return (void *)(uintptr_t)(0x100000000ull + (uint64_t)k * 0x10000000ull); }
    int main(void) {
        const int INV = ESA_ERR_INVALID_ARG, UNS = ESA_ERR_UNSUPPORTED, WS = ESA_ERR_WORKSPACE;
        if (esa_abi_version() != ESA_ABI_VERSION) return 1;
        for (int s = -2; s < 8; ++s)
            if (!esa_status_string(s) || !strlen(esa_status_string(s))) return 1;
        const int64_t dhs[] = {16, 32, 64, 128, 48, 0};
        for (int dt = -1; dt <= 5; ++dt)
            for (int d = 0; d < 6; ++d) {
                size_t w = esa_scan_workspace_bytes(3, 1000, 2, dhs[d], dt);
                int ok = dt >= 0 && dt <= 4 && d < 4;
                if ((w > 0) != ok) { printf("workspace %d %d\n", dt, d); return 1; }
            }
        if (esa_scan_workspace_bytes((int64_t)1 << 40, (int64_t)1 << 40, 1, 16, 1) != 0) return 1;
        if (esa_scan_ckpt_bytes(2, 65, 3, 16) != 2 * 2 * 3 * 16 * 4) return 1;
        CHECK(esa_workspace_init(NULL, 256, NULL), INV);
        CHECK(esa_workspace_init((char *)A(1) + 8, 256, NULL), INV);
        /* forward */
        CHECK(esa_scan_fwd(2, 100, 2, 16, 1, 1, NULL, A(2), A(3), NULL, A(4), A(5), NULL, A(6), 0, NULL), INV);
        CHECK(esa_scan_fwd(2, 100, 2, 16, 9, 1, A(1), A(2), A(3), NULL, A(4), A(5), NULL, A(6), 0, NULL), INV);
        CHECK(esa_scan_fwd(2, 100, 2, 48, 1, 1, A(1), A(2), A(3), NULL, A(4), A(5), NULL, A(6), 0, NULL), UNS);
        CHECK(esa_scan_fwd(2, 100, 2, 16, 1, 1, A(1), A(2), A(3), NULL, A(1), A(5), NULL, A(6), 0, NULL), INV);
        CHECK(esa_scan_fwd(2, 100, 2, 16, 1, 1, A(1), (char *)A(2) + 4, A(3), NULL, A(4), A(5), NULL, A(6), 0, NULL), INV);
        CHECK(esa_scan_fwd(2, 100, 2, 16, 1, 1, A(1), A(2), A(3), NULL, A(4), A(5), NULL, A(6), 100, NULL), WS);
        CHECK(esa_scan_fwd((int64_t)1 << 40, (int64_t)1 << 40, 2, 16, 1, 1, A(1), A(2), A(3), NULL, A(4), A(5), NULL, A(6), 0, NULL), INV);
        /* backward */
        CHECK(esa_scan_bwd(2, 100, 2, 64, 2, 0, A(1), A(2), A(3), NULL, NULL, NULL, NULL, A(5), A(6), A(7), NULL, A(8), 0, NULL), INV);
        CHECK(esa_scan_bwd(2, 100, 2, 64, 2, 0, A(1), A(2), A(3), NULL, A(4), NULL, NULL, A(4), A(6), A(7), NULL, A(8), 0, NULL), INV);
        CHECK(esa_scan_bwd(2, 100, 2, 64, 2, 0, A(1), A(2), A(3), NULL, A(4), NULL, NULL, A(5), A(6), A(7), NULL, NULL, 0, NULL), WS);
        CHECK(esa_scan_bwd(2, 100, 2, 8, 2, 0, A(1), A(2), A(3), NULL, A(4), NULL, NULL, A(5), A(6), A(7), NULL, A(8), 0, NULL), UNS);
        /* decode step */
        CHECK(esa_state_step(4, 2, 64, 1, 1, A(1), A(2), A(3), NULL, A(5), NULL), INV);
        CHECK(esa_state_step(4, 2, 24, 1, 1, A(1), A(2), A(3), A(4), A(5), NULL), UNS);
        CHECK(esa_state_step(4, 2, 64, 1, 1, A(1), A(2), A(3), A(4), A(2), NULL), INV);
        /* sequence segments */
        CHECK(esa_scan_segment_fwd(2, 100, 2, 64, 3, 1, A(1), A(2), NULL, A(4), A(5), 0, NULL), INV);
        CHECK(esa_scan_segment_fwd(2, 100, 2, 64, 3, 1, A(1), A(2), A(3), A(4), NULL, 0, NULL), WS);
        CHECK(esa_scan_segment_bwd(2, 100, 2, 64, 4, 0, A(1), A(2), A(3), NULL, A(4), NULL, NULL, A(6), 0, NULL), INV);
        CHECK(esa_segment_compose(0, 64, 0, A(1), A(2), NULL, A(3), NULL, NULL), INV);
        CHECK(esa_segment_compose(3, 64, 2, A(1), A(2), NULL, A(3), NULL, NULL), INV);
        CHECK(esa_segment_compose(3, 64, 0, A(1), A(2), NULL, A(1), NULL, NULL), INV);
        CHECK(esa_segment_compose((int64_t)1 << 40, (int64_t)1 << 40, 0, A(1), A(2), NULL, A(3), NULL, NULL), INV);
        puts("host ok");
        return 0;
    }
""")


def run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    drv = tmp_path / "drv.c"
    drv.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_check"
    r = run(["gcc", "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", "-ffp-contract=off",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", ORACLE_C, str(drv),
             "-o", str(exe), "-lm"])
    assert r.returncode == 0, r.stderr[-3000:]
    r = run([str(exe)], env=SAN_ENV)
    assert r.returncode == 0 and "oracle ok" in r.stdout, (r.stdout + r.stderr)[-3000:]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_host_library_under_address_and_ub_sanitizers(tmp_path):
    drv = tmp_path / "drv.c"
    drv.write_text(HOST_DRIVER)
    exe = tmp_path / "host_check"
    srcs = [os.path.join(CSRC, f) for f in ("esa_api.hip", "esa_fwd.hip", "esa_bwd.hip",
                                            "esa_step.hip")]
    # device code built as usual (and never launched here); the sanitizers on the host pass
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    dev = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    objs, procs = [], []
    for src in srcs:
        obj = tmp_path / (os.path.basename(src) + ".o")
        procs.append(subprocess.Popen(["hipcc", *dev, "-std=c++17", "-g", "-O2", *san, *inc,
                                       "-c", src, "-o", str(obj)], stdout=subprocess.PIPE,
                                      stderr=subprocess.PIPE, text=True))
        objs.append(str(obj))
    for pr in procs:
        _, err = pr.communicate(timeout=900)
        assert pr.returncode == 0, err[-3000:]
    obj = tmp_path / "drv.o"
    r = run(["hipcc", "-x", "c", "-std=c11", "-g", "-O1", *san, *inc, "-c", str(drv), "-o",
             str(obj)])
    assert r.returncode == 0, r.stderr[-3000:]
    r = run(["hipcc", *dev, *san, *objs, str(obj), "-o", str(exe)])
    assert r.returncode == 0, r.stderr[-3000:]
    r = run([str(exe)], env=SAN_ENV)
    assert r.returncode == 0 and "host ok" in r.stdout, (r.stdout + r.stderr)[-3000:]
