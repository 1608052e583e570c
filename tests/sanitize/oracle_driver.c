/*
 * Sanitizer driver for the CPU oracle (oracle/gspn_oracle.c): built together
 * with it under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py, it calls every oracle entry point on small grids
 * (single pixels, single lines, odd and even sides, grouped taps, chunked
 * scans, saturated logits) with buffers allocated at exactly the sizes the
 * layouts give, so that any read or write outside them, any signed overflow
 * or any other undefined operation stops the run.  It also checks two facts
 * the pages fix: normalised taps sum to 1 per pixel with dropped taps 0, and
 * the outputs are finite for finite inputs.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

void gspn_oracle_normalize(const double* w_raw, double* w_norm, long P, long NL, long L, double eps);
int gspn_oracle_scan_dir(const double* x, const double* lam, const double* u, const double* w,
                         int w_is_raw, double eps, double* out, long B, long C, long H, long W,
                         int dir);
int gspn_oracle_prop2d(const double* x, const double* lam, const double* u, const double* w4,
                       double eps, double* y, long B, long C, long H, long W);
int gspn_oracle_prop2d_backward(const double* x, const double* lam, const double* u,
                                const double* w4, const double* gy, double eps, double* gx,
                                double* glam, double* gu, double* gw4, long B, long C, long H,
                                long W);
int gspn_oracle_prop2d_ex(const double* x, const double* lam, const double* u, const double* w4,
                          long G, long k_chunk, double eps, double* y, long B, long C, long H,
                          long W);
int gspn_oracle_prop2d_ex_backward(const double* x, const double* lam, const double* u,
                                   const double* w4, const double* gy, long G, long k_chunk,
                                   double eps, double* gx, double* glam, double* gu, double* gw4,
                                   long B, long C, long H, long W);

static unsigned long long g_state = 88172645463325252ull;

static double uniform(void) {   /* xorshift64 in [-1, 1) */
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (double)(g_state >> 11) / 4503599627370496.0 - 1.0;
}

/* exactly n doubles, filled; logits get a share of saturated values */
static double* fill(long n, double scale, int saturate) {
    double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!a) exit(3);
    for (long i = 0; i < n; ++i) {
        a[i] = scale * uniform();
        if (saturate && i % 7 == 3) a[i] = (i % 2) ? 800.0 : -800.0;
    }
    return a;
}

static int finite_all(const double* a, long n) {
    for (long i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

static int fails = 0;
#define CHECK(c, what) do { if (!(c)) { fprintf(stderr, "check failed: %s\n", what); ++fails; } } while (0)

static void one_grid(long B, long C, long H, long W, long G, long k, double eps, int sat) {
    const long n = B * C * H * W;
    const long taps = 12 * B * G * H * W;
    double* x = fill(n, 2.0, 0);
    double* lam = fill(n, 1.0, 0);
    double* u = fill(n, 1.0, 0);
    double* gy = fill(n, 1.0, 0);
    double* w4 = fill(taps, 4.0, sat);
    double* y = fill(n, 0.0, 0);
    double* gx = fill(n, 0.0, 0);
    double* glam = fill(n, 0.0, 0);
    double* gu = fill(n, 0.0, 0);
    double* gw4 = fill(taps, 0.0, 0);

    if (G == C && k == 1) {
        CHECK(gspn_oracle_prop2d(x, lam, u, w4, eps, y, B, C, H, W) == 0, "prop2d");
        CHECK(finite_all(y, n), "prop2d finite");
        CHECK(gspn_oracle_prop2d_backward(x, lam, u, w4, gy, eps, gx, glam, gu, gw4, B, C, H, W) == 0,
              "prop2d_backward");
        CHECK(finite_all(gx, n) && finite_all(gw4, taps), "backward finite");
        for (int d = 0; d < 4; ++d) {
            const long NL = d < 2 ? H : W, L = d < 2 ? W : H;
            const double* wd = w4 + (long)d * 3 * B * C * H * W;
            double* wn = fill(3 * B * C * H * W, 0.0, 0);
            gspn_oracle_normalize(wd, wn, B * C, NL, L, eps);
            /* the three normalised taps of a pixel sum to 1 when the clamp
               does not act, and to less when it does; dropped taps are 0 */
            for (long pl = 0; pl < B * C; ++pl)
                for (long i = 0; i < NL; ++i)
                    for (long p = 0; p < L; ++p) {
                        const double* b = wn + pl * 3 * NL * L + i * L + p;
                        const double s = b[0] + b[NL * L] + b[2 * NL * L];
                        CHECK(s <= 1.0 + 1e-12, "normalised sum <= 1");
                        if (p == 0) CHECK(b[0] == 0.0, "left tap dropped");
                        if (p == L - 1) CHECK(b[2 * NL * L] == 0.0, "right tap dropped");
                    }
            CHECK(gspn_oracle_scan_dir(x, lam, u, wd, 1, eps, y, B, C, H, W, d) == 0, "scan raw");
            CHECK(gspn_oracle_scan_dir(x, lam, u, wn, 0, eps, y, B, C, H, W, d) == 0, "scan norm");
            CHECK(finite_all(y, n), "scan finite");
            free(wn);
        }
    }
    CHECK(gspn_oracle_prop2d_ex(x, lam, u, w4, G, k, eps, y, B, C, H, W) == 0, "prop2d_ex");
    CHECK(finite_all(y, n), "ex finite");
    CHECK(gspn_oracle_prop2d_ex_backward(x, lam, u, w4, gy, G, k, eps, gx, glam, gu, gw4, B, C, H,
                                         W) == 0, "ex_backward");
    CHECK(finite_all(gw4, taps), "ex backward finite");
    free(x); free(lam); free(u); free(gy); free(w4); free(y); free(gx); free(glam); free(gu); free(gw4);
}

int main(void) {
    const long shapes[][2] = {{1, 1}, {1, 2}, {2, 1}, {1, 7}, {7, 1}, {2, 2}, {3, 5}, {5, 3}, {4, 4}, {9, 11}};
    for (unsigned s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const long H = shapes[s][0], W = shapes[s][1];
        one_grid(1, 2, H, W, 2, 1, 1e-6, 0);
        one_grid(2, 3, H, W, 3, 1, 1e-3, 1);
        one_grid(1, 4, H, W, 2, 2, 1e-6, 1);
        one_grid(2, 2, H, W, 1, 3, 1e-6, 0);
    }
    /* invalid options are rejected, not run */
    double v = 0.0;
    CHECK(gspn_oracle_prop2d_ex(&v, &v, &v, &v, 0, 1, 1e-6, &v, 1, 1, 1, 1) != 0, "G = 0 rejected");
    CHECK(gspn_oracle_prop2d_ex(&v, &v, &v, &v, 2, 1, 1e-6, &v, 1, 3, 1, 1) != 0, "G does not divide C");
    CHECK(gspn_oracle_prop2d_ex(&v, &v, &v, &v, 1, 0, 1e-6, &v, 1, 1, 1, 1) != 0, "k = 0 rejected");
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle driver: ok\n");
    return 0;
}
