/*
 * Reference oracle for the GSPN four-direction line-scan propagation.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, single-threaded
 * fp64 restatement of what the operator computes.  It exists so the HIP
 * kernels can be checked against something obviously correct.  Only the
 * tests, the smoke check and the bench's CPU-baseline leg may load it; the
 * product library never links or calls it, and it shares no code, header or
 * table with the HIP path.
 *
 * Sources (the paper "Scaling Parallel Sequence Models to Foundation-Scale
 * Vision Encoders", C-GSPN, and its reading notes):
 *   - paper §3 "Background: 2D Spatial Propagation": feature map B x C x H x W,
 *     line-scan recurrence (display lost in the extraction; the standard GSPN
 *     form is used: h_i = w_i h_{i-1} + lambda_i * x_i, output u_i * h_i).
 *   - reading notes, "method / overall framework": lines are scanned in
 *     order, all positions of a line update in parallel from the previous
 *     line through three coefficients (a tridiagonal neighbourhood); w must
 *     be row-stochastic, made so by sigmoid followed by division by the
 *     neighbourhood sum; four directions (top-down, bottom-up, left-right,
 *     right-left) are each scanned once.
 *   - paper §5.1 "Fused CUDA normalization": sigmoid, local reduction,
 *     clamping, division.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - h before the first line is 0, so the first line in scan order is
 *     lambda * x and its taps are unused.
 *   - tap k (0,1,2) stored at destination position p weights position
 *     p + k - 1 of the previous line, in absolute coordinates for every
 *     direction; taps whose source falls outside the line are dropped from
 *     both the numerator and the neighbourhood sum.
 *   - the clamp bounds the neighbourhood sum from below by eps.
 *   - lambda and u are shared by the four directions; the four directional
 *     outputs u * h_d are summed in the order TD, BU, LR, RL.
 *
 * Memory layouts (row-major, innermost last):
 *   x, lambda, u, y : [B][C][H][W]
 *   taps of one direction : [B][C][3][NL][L], indexed by (line, position)
 *       of that direction: TD/BU lines are rows (NL = H, L = W),
 *       LR/RL lines are columns (NL = W, L = H), i.e. LR/RL tap planes are
 *       stored transposed with respect to the pixel grid.
 *   taps of all four directions : [4][B][C][3][...] in order TD, BU, LR, RL.
 *
 * Build: gcc -O2 -shared -fPIC gspn_oracle.c -o libgspn_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { DIR_TD = 0, DIR_BU = 1, DIR_LR = 2, DIR_RL = 3 };

/* Logistic sigmoid 1 / (1 + e^-z) in fp64. */
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/*
 * Row-stochastic normalisation of the three taps of one destination position
 * (reading notes, normalisation formula; paper §5.1 fused normalisation):
 *   s_k = sigmoid(raw_k) if position p + k - 1 lies on the line, else 0
 *   S   = max(s_0 + s_1 + s_2, eps)          (the clamp)
 *   w_k = s_k / S
 */
static void normalize_three(const double raw[3], long p, long L, double eps,
                            double out[3]) {
    double s[3];
    double sum = 0.0;
    for (int k = 0; k < 3; ++k) {
        long q = p + k - 1;
        s[k] = (q >= 0 && q < L) ? sigmoid(raw[k]) : 0.0;
        sum += s[k];
    }
    double S = sum > eps ? sum : eps;
    for (int k = 0; k < 3; ++k) out[k] = s[k] / S;
}

/*
 * Normalise one direction's tap block w_raw [P][3][NL][L] into w_norm (same
 * layout).  Every position is written, including the first line's, whose
 * taps the scan never uses.
 */
void gspn_oracle_normalize(const double* w_raw, double* w_norm, long P,
                           long NL, long L, double eps) {
    long plane = NL * L;
    for (long pl = 0; pl < P; ++pl) {
        const double* src = w_raw + pl * 3 * plane;
        double* dst = w_norm + pl * 3 * plane;
        for (long i = 0; i < NL; ++i) {
            for (long p = 0; p < L; ++p) {
                double raw[3], out[3];
                for (int k = 0; k < 3; ++k) raw[k] = src[k * plane + i * L + p];
                normalize_three(raw, p, L, eps, out);
                for (int k = 0; k < 3; ++k) dst[k * plane + i * L + p] = out[k];
            }
        }
    }
}

/* Pixel (row, col) visited by direction dir at line i, position p. */
static void pixel_of(int dir, long i, long p, long* row, long* col) {
    if (dir == DIR_TD || dir == DIR_BU) { *row = i; *col = p; }
    else                                { *row = p; *col = i; }
}

/*
 * One directional scan over every (b, c) plane (paper §3 line-scan
 * recurrence; reading notes, top-down example generalised to the other three
 * directions).  For each plane, lines are visited in scan order (TD: rows
 * 0..H-1, BU: rows H-1..0, LR: columns 0..W-1, RL: columns W-1..0):
 *   first line:  h[p] = lambda * x
 *   later lines: h[p] = sum_{in-line k} w_k(i, p) * h_prev[p + k - 1]
 *                       + lambda * x
 * and out = u * h at every pixel.  With w_is_raw the taps are normalised
 * first; otherwise they are used as given (a tap whose source lies outside
 * the line contributes nothing, whatever its value).
 * Returns 0, or -1 if scratch memory could not be obtained.
 */
int gspn_oracle_scan_dir(const double* x, const double* lam, const double* u,
                         const double* w, int w_is_raw, double eps,
                         double* out, long B, long C, long H, long W,
                         int dir) {
    long NL = (dir == DIR_TD || dir == DIR_BU) ? H : W;
    long L  = (dir == DIR_TD || dir == DIR_BU) ? W : H;
    int forward = (dir == DIR_TD || dir == DIR_LR);
    long npix = H * W;
    double* hprev = (double*)malloc(sizeof(double) * (size_t)L);
    double* hnew  = (double*)malloc(sizeof(double) * (size_t)L);
    if (!hprev || !hnew) { free(hprev); free(hnew); return -1; }

    for (long pl = 0; pl < B * C; ++pl) {
        const double* xp = x + pl * npix;
        const double* lp = lam + pl * npix;
        const double* up = u + pl * npix;
        const double* wp = w + pl * 3 * npix;   /* [3][NL][L] */
        double* op = out + pl * npix;
        for (long step = 0; step < NL; ++step) {
            long i = forward ? step : NL - 1 - step;
            for (long p = 0; p < L; ++p) {
                long r, c;
                pixel_of(dir, i, p, &r, &c);
                double bx = lp[r * W + c] * xp[r * W + c];
                double h = bx;
                if (step > 0) {
                    double raw[3], tap[3];
                    for (int k = 0; k < 3; ++k) raw[k] = wp[k * npix + i * L + p];
                    if (w_is_raw) normalize_three(raw, p, L, eps, tap);
                    else memcpy(tap, raw, sizeof tap);
                    double mix = 0.0;
                    for (int k = 0; k < 3; ++k) {
                        long q = p + k - 1;
                        if (q < 0 || q >= L) continue;
                        mix += tap[k] * hprev[q];
                    }
                    h = mix + bx;
                }
                hnew[p] = h;
                op[r * W + c] = up[r * W + c] * h;
            }
            double* t = hprev; hprev = hnew; hnew = t;
        }
    }
    free(hprev);
    free(hnew);
    return 0;
}

/*
 * Four-direction propagation y = sum_d u * h_d, summed in fp64 in the order
 * TD, BU, LR, RL, with the taps of every direction normalised (the operator
 * the latent sublayer applies: y_c = Prop2D(x_c; u, lambda, w), reading
 * notes, key design 1).  w4 is [4][B][C][3][...].
 * Returns 0, or -1 if scratch memory could not be obtained.
 */
int gspn_oracle_prop2d(const double* x, const double* lam, const double* u,
                       const double* w4, double eps, double* y, long B,
                       long C, long H, long W) {
    long n = B * C * H * W;
    double* part = (double*)malloc(sizeof(double) * (size_t)n);
    if (!part) return -1;
    for (long e = 0; e < n; ++e) y[e] = 0.0;
    for (int d = 0; d < 4; ++d) {
        if (gspn_oracle_scan_dir(x, lam, u, w4 + (long)d * 3 * n, 1, eps, part,
                                 B, C, H, W, d) != 0) {
            free(part);
            return -1;
        }
        for (long e = 0; e < n; ++e) y[e] += part[e];
    }
    free(part);
    return 0;
}

/*
 * Gradient of the four-direction propagation (paper §6.1 reports forward and
 * backward kernels; the backward itself is not described on the pages, so
 * this is the exact derivative of the forward definition above).
 *
 * Given gy = dL/dy for y = sum_d u * h_d, per plane and direction d, with
 * scan-order lines i = 0 .. NL-1, normalised taps wn(i, p, k) and
 * b_i = lambda_i * x_i:
 *   adjoint, in reverse scan order:
 *     g_{NL-1} = u * gy
 *     g_i      = u * gy + sum_k wn(i+1, q, k) g_{i+1}[q]   over q = p - k + 1
 *                (the transposed tridiagonal map of line i + 1)
 *   gx     = lambda * sum_d g_d       glambda = x * sum_d g_d
 *   gu     = gy * sum_d h_d
 *   gwn(i, p, k) = g_i[p] * h_{i-1}[p + k - 1]  for i >= 1 and in-line k,
 *                  0 otherwise (the first line's taps are unused)
 *   normalisation: s_k = sigmoid(z_k) (in-line), T = s_0 + s_1 + s_2,
 *     T > eps : gs_m = (gwn_m - sum_k gwn_k wn_k) / T
 *     T <= eps: gs_m = gwn_m / eps        (the clamp holds S at eps)
 *     gz_m = gs_m s_m (1 - s_m) for in-line m, 0 for dropped taps.
 * The branch follows the forward's: the sum is used when it exceeds eps.
 * All outputs are fp64, in the layouts of the corresponding inputs.
 * Returns 0, or -1 if scratch memory could not be obtained.
 */
int gspn_oracle_prop2d_backward(const double* x, const double* lam, const double* u,
                                const double* w4, const double* gy, double eps,
                                double* gx, double* glam, double* gu, double* gw4,
                                long B, long C, long H, long W) {
    long npix = H * W;
    long n = B * C * npix;
    long Lmax = H > W ? H : W;
    double* hs = (double*)malloc(sizeof(double) * (size_t)npix);     /* sum_d h_d */
    double* gs = (double*)malloc(sizeof(double) * (size_t)npix);     /* sum_d g_d */
    double* hl = (double*)malloc(sizeof(double) * (size_t)npix);     /* h_d by (line, pos) */
    double* g  = (double*)malloc(sizeof(double) * (size_t)Lmax);
    double* gn = (double*)malloc(sizeof(double) * (size_t)Lmax);
    double* wn = (double*)malloc(sizeof(double) * (size_t)npix * 3); /* wn by (line, pos, k) */
    if (!hs || !gs || !hl || !g || !gn || !wn) {
        free(hs); free(gs); free(hl); free(g); free(gn); free(wn);
        return -1;
    }
    for (long pl = 0; pl < B * C; ++pl) {
        const double* xp = x + pl * npix;
        const double* lp = lam + pl * npix;
        const double* up = u + pl * npix;
        const double* gyp = gy + pl * npix;
        for (long e = 0; e < npix; ++e) { hs[e] = 0.0; gs[e] = 0.0; }
        for (int d = 0; d < 4; d++) {
            long NL = (d == DIR_TD || d == DIR_BU) ? H : W;
            long L  = (d == DIR_TD || d == DIR_BU) ? W : H;
            int forward = (d == DIR_TD || d == DIR_LR);
            const double* wp = w4 + ((long)d * n + pl * npix) * 3;   /* [3][NL][L] */
            double* gwp = gw4 + ((long)d * n + pl * npix) * 3;
            /* normalised taps of every line */
            for (long i = 0; i < NL; ++i)
                for (long p = 0; p < L; ++p) {
                    double raw[3], t[3];
                    for (int k = 0; k < 3; ++k) raw[k] = wp[k * npix + (i * L + p)];
                    normalize_three(raw, p, L, eps, t);
                    for (int k = 0; k < 3; ++k) wn[(i * L + p) * 3 + k] = t[k];
                }
            /* forward scan, keeping every line of h (indexed by line i) */
            for (long step = 0; step < NL; ++step) {
                long i = forward ? step : NL - 1 - step;
                long iprev = forward ? i - 1 : i + 1;
                for (long p = 0; p < L; ++p) {
                    long r, c;
                    pixel_of(d, i, p, &r, &c);
                    double h = lp[r * W + c] * xp[r * W + c];
                    if (step > 0) {
                        for (int k = 0; k < 3; ++k) {
                            const long q = p + k - 1;
                            if (q < 0 || q >= L) continue;
                            h += wn[(i * L + p) * 3 + k] * hl[iprev * L + q];
                        }
                    }
                    hl[i * L + p] = h;
                    hs[r * W + c] += h;
                }
            }
            /* adjoint scan in reverse order */
            for (long step = NL - 1; step >= 0; --step) {
                long i = forward ? step : NL - 1 - step;
                long inext = forward ? i + 1 : i - 1;      /* the line scanned after i */
                long iprev = forward ? i - 1 : i + 1;      /* the line scanned before i */
                for (long p = 0; p < L; ++p) {
                    long r, c;
                    pixel_of(d, i, p, &r, &c);
                    double v = up[r * W + c] * gyp[r * W + c];
                    if (step < NL - 1) {
                        /* destinations q of line inext whose tap k reads position p */
                        for (int k = 0; k < 3; ++k) {
                            long q = p - k + 1;
                            if (q < 0 || q >= L) continue;
                            v += wn[(inext * L + q) * 3 + k] * g[q];
                        }
                    }
                    gn[p] = v;
                    gs[r * W + c] += v;
                }
                /* tap gradients of line i */
                for (long p = 0; p < L; ++p) {
                    double gwn[3] = {0.0, 0.0, 0.0};
                    if (step > 0) {
                        for (int k = 0; k < 3; ++k) {
                            const long q = p + k - 1;
                            if (q < 0 || q >= L) continue;
                            gwn[k] = gn[p] * hl[iprev * L + q];
                        }
                    }
                    double s[3], T = 0.0, dot = 0.0;
                    for (int k = 0; k < 3; ++k) {
                        const long q = p + k - 1;
                        s[k] = (q >= 0 && q < L) ? sigmoid(wp[k * npix + i * L + p]) : 0.0;
                        T += s[k];
                    }
                    for (int k = 0; k < 3; ++k) dot += gwn[k] * wn[(i * L + p) * 3 + k];
                    for (int k = 0; k < 3; ++k) {
                        const long q = p + k - 1;
                        double gz = 0.0;
                        if (q >= 0 && q < L) {
                            double gsk = T > eps ? (gwn[k] - dot) / T : gwn[k] / eps;
                            gz = gsk * s[k] * (1.0 - s[k]);
                        }
                        gwp[k * npix + i * L + p] = gz;
                    }
                }
                double* t = g; g = gn; gn = t;
            }
        }
        for (long e = 0; e < npix; ++e) {
            gx[pl * npix + e] = lp[e] * gs[e];
            glam[pl * npix + e] = xp[e] * gs[e];
            gu[pl * npix + e] = gyp[e] * hs[e];
        }
    }
    free(hs); free(gs); free(hl); free(g); free(gn); free(wn);
    return 0;
}

/*
 * Extended operator: tap groups and chunked (local) scans.
 *
 * Tap groups (paper §4.2, channel-shared weights; §6.2 shares the weights
 * across channels in every module): the C channels form G contiguous groups
 * of C / G channels, and channel c reads the taps of group c / (C / G).  The
 * taps are then [4][B][G][3][..][..].  G = C is the per-channel operator
 * above; G = 1 shares one set of taps among all channels of an image.
 *
 * Chunked scan (paper §4.1: the grid is indexed by (chunk, b, c), k_chunk
 * chunks per plane): each direction's NL lines are cut into k_chunk
 * contiguous segments of Lc = ceil(NL / k_chunk) lines (the last one may be
 * shorter; with k_chunk > NL some are empty), the same segments for both
 * scan orders of an axis.  Each segment is scanned on its own: the first
 * line of a segment in the direction's scan order restarts from
 * h = lambda * x.  k_chunk = 1 is the global scan above.
 *
 * y = sum over TD, BU, LR, RL of u * h_d, accumulated in that order.
 * Returns 0, -1 if scratch memory could not be obtained, -2 for a bad G or
 * k_chunk.
 */
static int restarts_segment(long i, long NL, long Lc, int fwd) {
    if (fwd) return i % Lc == 0;                 /* top (left) line of its segment */
    return i == NL - 1 || (i + 1) % Lc == 0;     /* bottom (right) line of its segment */
}

int gspn_oracle_prop2d_ex(const double* x, const double* lam, const double* u,
                          const double* w4, long G, long k_chunk, double eps,
                          double* y, long B, long C, long H, long W) {
    if (G < 1 || C % G != 0 || k_chunk < 1) return -2;
    long npix = H * W;
    long cpg = C / G;                              /* channels per group */
    long Lmax = H > W ? H : W;
    double* prev = (double*)malloc(sizeof(double) * (size_t)Lmax);
    double* cur = (double*)malloc(sizeof(double) * (size_t)Lmax);
    if (!prev || !cur) { free(prev); free(cur); return -1; }
    for (long b = 0; b < B; ++b) {
        for (long ch = 0; ch < C; ++ch) {
            long pl = b * C + ch;
            const double* xs = x + pl * npix;
            const double* ls = lam + pl * npix;
            const double* us = u + pl * npix;
            double* ys = y + pl * npix;
            for (long e = 0; e < npix; ++e) ys[e] = 0.0;
            for (int dir = DIR_TD; dir <= DIR_RL; dir++) {
                int along_rows = (dir == DIR_TD || dir == DIR_BU);
                long NL = along_rows ? H : W;
                long L = along_rows ? W : H;
                int fwd = (dir == DIR_TD) || (dir == DIR_LR);
                long Lc = (NL + k_chunk - 1) / k_chunk;
                const double* tg = w4 + (((long)dir * B + b) * G + ch / cpg) * 3 * npix;
                for (long step = 0; step < NL; ++step) {
                    long i = fwd ? step : NL - 1 - step;
                    int restart = restarts_segment(i, NL, Lc, fwd);
                    for (long p = 0; p < L; ++p) {
                        long r, c;
                        pixel_of(dir, i, p, &r, &c);
                        long e = r * W + c;
                        double hv = ls[e] * xs[e];
                        if (!restart) {
                            double z[3], wn[3];
                            for (int k = 0; k < 3; ++k) z[k] = tg[(long)k * npix + i * L + p];
                            normalize_three(z, p, L, eps, wn);
                            for (int k = 0; k < 3; ++k) {
                                long src = p + k - 1;
                                if (src >= 0 && src < L) hv += wn[k] * prev[src];
                            }
                        }
                        cur[p] = hv;
                        ys[e] += us[e] * hv;
                    }
                    double* t = prev; prev = cur; cur = t;
                }
            }
        }
    }
    free(prev);
    free(cur);
    return 0;
}

/*
 * Gradient of the extended operator above (tap groups and chunked scans): the
 * exact derivative of gspn_oracle_prop2d_ex, with the formulas of
 * gspn_oracle_prop2d_backward and two changes that follow from the forward:
 *   - a line that restarts its segment does not read the line before it: its
 *     taps get gradient 0, and the line before it (in scan order) receives no
 *     adjoint term from it, so its g is u * gy alone;
 *   - channel c reads the taps of group c / (C / G), so the tap gradient of a
 *     group is the sum over its channels, accumulated in channel order.
 * gw4 has the layout of w4, [4][B][G][3][..][..].
 * Returns 0, -1 if scratch memory could not be obtained, -2 for a bad G or
 * k_chunk.
 */
int gspn_oracle_prop2d_ex_backward(const double* x, const double* lam, const double* u,
                                   const double* w4, const double* gy, long G, long k_chunk,
                                   double eps, double* gx, double* glam, double* gu,
                                   double* gw4, long B, long C, long H, long W) {
    if (G < 1 || C % G != 0 || k_chunk < 1) return -2;
    long npix = H * W;
    long cpg = C / G;
    long Lmax = H > W ? H : W;
    double* hsum = (double*)malloc(sizeof(double) * (size_t)npix);
    double* gsum = (double*)malloc(sizeof(double) * (size_t)npix);
    double* hline = (double*)malloc(sizeof(double) * (size_t)npix);   /* h by (line, pos) */
    double* wnorm = (double*)malloc(sizeof(double) * (size_t)npix * 3);
    double* gnext = (double*)malloc(sizeof(double) * (size_t)Lmax);   /* g of the line after */
    double* gcur = (double*)malloc(sizeof(double) * (size_t)Lmax);
    if (!hsum || !gsum || !hline || !wnorm || !gnext || !gcur) {
        free(hsum); free(gsum); free(hline); free(wnorm); free(gnext); free(gcur);
        return -1;
    }
    for (long e = 0; e < 4 * B * G * 3 * npix; ++e) gw4[e] = 0.0;
    for (long b = 0; b < B; ++b) {
        for (long ch = 0; ch < C; ++ch) {
            long pl = b * C + ch;
            const double* xs = x + pl * npix;
            const double* ls = lam + pl * npix;
            const double* us = u + pl * npix;
            const double* gys = gy + pl * npix;
            for (long e = 0; e < npix; ++e) { hsum[e] = 0.0; gsum[e] = 0.0; }
            for (int dir = DIR_TD; dir <= DIR_RL; dir++) {
                int along_rows = (dir == DIR_TD || dir == DIR_BU);
                long NL = along_rows ? H : W;
                long L = along_rows ? W : H;
                int fwd = (dir == DIR_TD) || (dir == DIR_LR);
                long seg = (NL + k_chunk - 1) / k_chunk;
                long grp = ch / cpg;                        /* the channel's tap group */
                long tap_off = (((long)dir * B + b) * G + grp) * 3 * npix;
                const double* tg = w4 + tap_off;
                double* gtg = gw4 + tap_off;
                for (long i = 0; i < NL; ++i)
                    for (long p = 0; p < L; ++p) {
                        double z[3], wn[3];
                        for (int k = 0; k < 3; ++k) z[k] = tg[(long)k * npix + i * L + p];
                        normalize_three(z, p, L, eps, wn);
                        for (int k = 0; k < 3; ++k) wnorm[(i * L + p) * 3 + k] = wn[k];
                    }
                /* forward, keeping every line */
                for (long step = 0; step < NL; ++step) {
                    long i = fwd ? step : NL - 1 - step;
                    long before = fwd ? i - 1 : i + 1;
                    int restart = restarts_segment(i, NL, seg, fwd);
                    for (long p = 0; p < L; ++p) {
                        long r, c;
                        pixel_of(dir, i, p, &r, &c);
                        double hv = ls[r * W + c] * xs[r * W + c];
                        if (!restart)
                            for (int k = 0; k < 3; ++k) {
                                long src = p + k - 1;
                                if (src >= 0 && src < L)
                                    hv += wnorm[(i * L + p) * 3 + k] * hline[before * L + src];
                            }
                        hline[i * L + p] = hv;
                        hsum[r * W + c] += hv;
                    }
                }
                /* adjoint, lines in reverse scan order */
                for (long step = NL - 1; step >= 0; --step) {
                    long i = fwd ? step : NL - 1 - step;
                    long after = fwd ? i + 1 : i - 1;
                    long before = fwd ? i - 1 : i + 1;
                    int after_reads_i = step < NL - 1 && !restarts_segment(after, NL, seg, fwd);
                    for (long p = 0; p < L; ++p) {
                        long r, c;
                        pixel_of(dir, i, p, &r, &c);
                        double v = us[r * W + c] * gys[r * W + c];
                        if (after_reads_i)
                            for (int k = 0; k < 3; ++k) {
                                long dst = p - k + 1;   /* position of line `after` whose tap k reads p */
                                if (dst >= 0 && dst < L) v += wnorm[(after * L + dst) * 3 + k] * gnext[dst];
                            }
                        gcur[p] = v;
                        gsum[r * W + c] += v;
                    }
                    int reads_before = !restarts_segment(i, NL, seg, fwd);
                    for (long p = 0; p < L; ++p) {
                        double dwn[3] = {0.0, 0.0, 0.0}, s[3], T = 0.0, wdot = 0.0;
                        for (int k = 0; k < 3; ++k) {
                            long src = p + k - 1;
                            int inl = src >= 0 && src < L;
                            if (reads_before && inl) dwn[k] = gcur[p] * hline[before * L + src];
                            s[k] = inl ? sigmoid(tg[(long)k * npix + i * L + p]) : 0.0;
                            T += s[k];
                        }
                        for (int k = 0; k < 3; ++k) wdot += dwn[k] * wnorm[(i * L + p) * 3 + k];
                        for (int k = 0; k < 3; ++k) {
                            long src = p + k - 1;
                            if (src < 0 || src >= L) continue;
                            double gs_k = T > eps ? (dwn[k] - wdot) / T : dwn[k] / eps;
                            gtg[(long)k * npix + i * L + p] += gs_k * s[k] * (1.0 - s[k]);
                        }
                    }
                    double* t = gnext; gnext = gcur; gcur = t;
                }
            }
            for (long e = 0; e < npix; ++e) {
                gx[pl * npix + e] = ls[e] * gsum[e];
                glam[pl * npix + e] = xs[e] * gsum[e];
                gu[pl * npix + e] = gys[e] * hsum[e];
            }
        }
    }
    free(hsum); free(gsum); free(hline); free(wnorm); free(gnext); free(gcur);
    return 0;
}
