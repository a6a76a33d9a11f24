/*
 * oracle.c -- plain fp64 CPU reference of the differentiable 2D anisotropic
 * Gaussian splatting layer (forward render, analytic backward, tile binning).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes ("Learning Video Dynamics with Predictive Differentiable
 * Rendering", abstract: each Gaussian carries 5 + C learnable values --
 * position, scale, rotation and C channel amplitudes; the reading notes on the
 * same paper, sections "Core Idea" and "Method": the rendered frame is the
 * additive superposition of local Gaussian primitives, no compositing):
 *
 *   p = (x + 1/2, y + 1/2)            pixel centre, x right, y down
 *   d = p - mu,  c = cos(theta), s = sin(theta)
 *   u1 =  c dx + s dy,   u2 = -s dx + c dy,   z1 = u1/s1,  z2 = u2/s2
 *   q  = z1^2 + z2^2
 *   w  = exp(-q/2) if q <= k^2 else 0        (k = truncation radius in sigma)
 *   I[b,y,x,ch] = sum_n a[b,n,ch] * w[b,n](x,y)
 *
 * Backward, with G = dL/dI, h = sum_ch G_ch a_ch, v = h w, sums over pixels:
 *   dL/da_ch  = sum G_ch w
 *   dL/dmu_x  = (c/s1) S1 - (s/s2) S2,   dL/dmu_y = (s/s1) S1 + (c/s2) S2
 *   dL/ds1    = S11/s1,  dL/ds2 = S22/s2,  dL/dtheta = (s1/s2 - s2/s1) S12
 * where S1 = sum v z1, S2 = sum v z2, S11 = sum v z1^2, S22 = sum v z2^2,
 * S12 = sum v z1 z2 (derivation: dz1/dtheta = z2 s2/s1, dz2/dtheta =
 * -z1 s1/s2; the truncation indicator is not differentiated).
 *
 * Truncation ties: a pair with |q - k^2| <= tau k^2 may legitimately fall on
 * either side of the edge in another precision (tau = 1e-4, the stated
 * relative tolerance applied to the truncation test), so every output also
 * gets a "slack" = the summed absolute value of such pairs' terms, and a
 * "magnitude" = the summed absolute value of all its terms (the scale a
 * relative error of a cancelling sum refers to).  Nothing else is allowed
 * for: the slack models no particular arithmetic.
 *
 * Binning: per Gaussian the pixel bounding box of the ellipse q <= k^2,
 *   ex = k sqrt((s1 c)^2 + (s2 s)^2),  ey = k sqrt((s1 s)^2 + (s2 c)^2)
 *   x0 = max(0, ceil(mu_x - ex - 1/2)),  x1 = min(W-1, floor(mu_x + ex - 1/2))
 *   (y likewise); empty if x0 > x1 or y0 > y1; invalid Gaussians (any
 * non-finite value, s1 <= 0 or s2 <= 0) have no box.  A Gaussian is listed
 * for a T x T tile iff its box meets the tile's pixels; lists hold ascending
 * Gaussian indices; tiles are ordered frame-major then row-major.
 *
 * Every loop here is the definition written out: Gaussians in ascending
 * order, pixels of a (1-pixel enlarged) box, fp64 throughout.  Threads only
 * split independent frames.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* per-Gaussian geometry                                                     */

typedef struct {
    int valid;
    double mx, my, s1, s2, c, s;
    int x0, x1, y0, y1; /* pixel box, inclusive; x0 > x1 means empty */
} gauss_geo;

static int all_finite(const double *g, int n) {
    for (int i = 0; i < n; i++)
        if (!isfinite(g[i])) return 0;
    return 1;
}

static double clampd(double v, double lo, double hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

static void geometry(const double *g, int C, int H, int W, double k, gauss_geo *o) {
    memset(o, 0, sizeof(*o));
    o->x0 = 1; o->x1 = 0; o->y0 = 1; o->y1 = 0;
    if (!all_finite(g, 5 + C) || !(g[2] > 0.0) || !(g[3] > 0.0)) return;
    o->valid = 1;
    o->mx = g[0]; o->my = g[1]; o->s1 = g[2]; o->s2 = g[3];
    o->c = cos(g[4]);
    o->s = sin(g[4]);
    double t1 = o->s1 * o->c, t2 = o->s2 * o->s;
    double t3 = o->s1 * o->s, t4 = o->s2 * o->c;
    double ex = k * sqrt(t1 * t1 + t2 * t2);
    double ey = k * sqrt(t3 * t3 + t4 * t4);
    double fx0 = ceil(o->mx - ex - 0.5), fx1 = floor(o->mx + ex - 0.5);
    double fy0 = ceil(o->my - ey - 0.5), fy1 = floor(o->my + ey - 0.5);
    fx0 = clampd(fx0, 0.0, (double)W);      /* W (past the end) => empty */
    fx1 = clampd(fx1, -1.0, (double)W - 1); /* -1 => empty */
    fy0 = clampd(fy0, 0.0, (double)H);
    fy1 = clampd(fy1, -1.0, (double)H - 1);
    o->x0 = (int)fx0; o->x1 = (int)fx1; o->y0 = (int)fy0; o->y1 = (int)fy1;
}

/* whitened coordinates and q of pixel (x, y) for one Gaussian */
static double pixel_q(const gauss_geo *G, int x, int y, double *z1, double *z2) {
    double dx = (x + 0.5) - G->mx;
    double dy = (y + 0.5) - G->my;
    double u1 = G->c * dx + G->s * dy;
    double u2 = -G->s * dx + G->c * dy;
    *z1 = u1 / G->s1;
    *z2 = u2 / G->s2;
    return (*z1) * (*z1) + (*z2) * (*z2);
}

/* the scan box: the pixel box enlarged by one pixel, so that pairs sitting
 * just outside the box with q within the tie band still get slack */
static int scan_box(const gauss_geo *G, int H, int W, int *xa, int *xb, int *ya, int *yb) {
    if (!G->valid || G->x0 > G->x1 || G->y0 > G->y1) return 0;
    *xa = G->x0 > 0 ? G->x0 - 1 : 0;
    *xb = G->x1 < W - 1 ? G->x1 + 1 : W - 1;
    *ya = G->y0 > 0 ? G->y0 - 1 : 0;
    *yb = G->y1 < H - 1 ? G->y1 + 1 : H - 1;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* threading over frames                                                     */

typedef struct {
    void (*fn)(void *ctx, int b);
    void *ctx;
    int B, tid, nthreads;
} worker_arg;

static void *worker(void *p) {
    worker_arg *a = (worker_arg *)p;
    for (int b = a->tid; b < a->B; b += a->nthreads) a->fn(a->ctx, b);
    return NULL;
}

static void for_frames(int B, int nthreads, void (*fn)(void *, int), void *ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B) nthreads = B;
    if (nthreads <= 1) {
        for (int b = 0; b < B; b++) fn(ctx, b);
        return;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    worker_arg *args = (worker_arg *)malloc(sizeof(worker_arg) * nthreads);
    for (int t = 0; t < nthreads; t++) {
        args[t].fn = fn; args[t].ctx = ctx; args[t].B = B;
        args[t].tid = t; args[t].nthreads = nthreads;
        pthread_create(&th[t], NULL, worker, &args[t]);
    }
    for (int t = 0; t < nthreads; t++) pthread_join(th[t], NULL);
    free(th);
    free(args);
}

/* ------------------------------------------------------------------------ */
/* forward                                                                   */

typedef struct {
    const double *params;
    int N, H, W, C, allpairs;
    double k, tau;
    double *image, *slack, *mag;
    long long *pairs;
} fwd_ctx;

static void fwd_pair(const fwd_ctx *F, const double *g, const gauss_geo *G, int x, int y,
                     double *img, double *slk, double *mg, long long *npairs) {
    double z1, z2;
    double q = pixel_q(G, x, y, &z1, &z2);
    double kk = F->k * F->k;
    double e = exp(-0.5 * q);
    size_t pix = ((size_t)y * F->W + x) * F->C;
    if (q <= kk) {
        (*npairs)++;
        for (int ch = 0; ch < F->C; ch++) {
            img[pix + ch] += g[5 + ch] * e;
            if (mg) mg[pix + ch] += fabs(g[5 + ch]) * e;
        }
    }
    if (slk && fabs(q - kk) <= F->tau * kk)
        for (int ch = 0; ch < F->C; ch++) slk[pix + ch] += fabs(g[5 + ch]) * e;
}

static void fwd_frame(void *p, int b) {
    fwd_ctx *F = (fwd_ctx *)p;
    int N = F->N, H = F->H, W = F->W, C = F->C, P = 5 + C;
    size_t fsz = (size_t)H * W * C;
    double *img = F->image + (size_t)b * fsz;
    double *slk = F->slack ? F->slack + (size_t)b * fsz : NULL;
    double *mg = F->mag ? F->mag + (size_t)b * fsz : NULL;
    const double *gp = F->params + (size_t)b * N * P;
    long long npairs = 0;
    memset(img, 0, fsz * sizeof(double));
    if (slk) memset(slk, 0, fsz * sizeof(double));
    if (mg) memset(mg, 0, fsz * sizeof(double));
    gauss_geo *geo = (gauss_geo *)malloc(sizeof(gauss_geo) * (size_t)(N > 0 ? N : 1));
    for (int n = 0; n < N; n++) geometry(gp + (size_t)n * P, C, H, W, F->k, &geo[n]);
    if (F->allpairs) {
        /* the definition with no pruning at all: every pixel, every Gaussian */
        for (int y = 0; y < H; y++)
            for (int x = 0; x < W; x++)
                for (int n = 0; n < N; n++)
                    if (geo[n].valid)
                        fwd_pair(F, gp + (size_t)n * P, &geo[n], x, y, img, slk, mg, &npairs);
    } else {
        for (int n = 0; n < N; n++) {
            int xa, xb, ya, yb;
            if (!scan_box(&geo[n], H, W, &xa, &xb, &ya, &yb)) continue;
            for (int y = ya; y <= yb; y++)
                for (int x = xa; x <= xb; x++)
                    fwd_pair(F, gp + (size_t)n * P, &geo[n], x, y, img, slk, mg, &npairs);
        }
    }
    if (F->pairs) F->pairs[b] = npairs;
    free(geo);
}

/* image/slack/mag: [B][H][W][C] fp64 (slack, mag, pairs may be NULL) */
int orc_render(const double *params, int B, int N, int H, int W, int C, double k, double tau,
               int allpairs, int nthreads, double *image, double *slack, double *mag,
               long long *pairs) {
    if (!params || !image || B < 1 || N < 0 || H < 1 || W < 1 || C < 1) return -1;
    fwd_ctx F = {params, N, H, W, C, allpairs, k, tau, image, slack, mag, pairs};
    for_frames(B, nthreads, fwd_frame, &F);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* backward                                                                  */

typedef struct {
    const double *params, *grad_image;
    int N, H, W, C;
    double k, tau;
    double *grad, *gslack, *gmag;
} bwd_ctx;

/* sum slots: 0..C-1 = A_ch, C = S1, C+1 = S2, C+2 = S11, C+3 = S22, C+4 = S12 */
static void bwd_frame(void *p, int b) {
    bwd_ctx *Bc = (bwd_ctx *)p;
    int N = Bc->N, H = Bc->H, W = Bc->W, C = Bc->C, P = 5 + C;
    double kk = Bc->k * Bc->k;
    const double *gp = Bc->params + (size_t)b * N * P;
    const double *gi = Bc->grad_image + (size_t)b * H * W * C;
    double *S = (double *)malloc(sizeof(double) * 3 * (C + 5));
    double *M = S + (C + 5), *Z = S + 2 * (C + 5);
    for (int n = 0; n < N; n++) {
        const double *g = gp + (size_t)n * P;
        double *out = Bc->grad + ((size_t)b * N + n) * P;
        double *osl = Bc->gslack ? Bc->gslack + ((size_t)b * N + n) * P : NULL;
        double *omg = Bc->gmag ? Bc->gmag + ((size_t)b * N + n) * P : NULL;
        for (int i = 0; i < P; i++) {
            out[i] = 0.0;
            if (osl) osl[i] = 0.0;
            if (omg) omg[i] = 0.0;
        }
        gauss_geo G;
        geometry(g, C, H, W, Bc->k, &G);
        int xa, xb, ya, yb;
        if (!scan_box(&G, H, W, &xa, &xb, &ya, &yb)) continue;
        memset(S, 0, sizeof(double) * 3 * (C + 5));
        for (int y = ya; y <= yb; y++) {
            for (int x = xa; x <= xb; x++) {
                double z1, z2;
                double q = pixel_q(&G, x, y, &z1, &z2);
                int inside = q <= kk;
                int tie = osl && fabs(q - kk) <= Bc->tau * kk;
                if (!inside && !tie) continue;
                double e = exp(-0.5 * q);
                const double *gpx = gi + ((size_t)y * W + x) * C;
                double h = 0.0, habs = 0.0;
                for (int ch = 0; ch < C; ch++) {
                    h += gpx[ch] * g[5 + ch];
                    habs += fabs(gpx[ch] * g[5 + ch]);
                }
                double v = h * e, va = habs * e;
                double term[5] = {v * z1, v * z2, v * z1 * z1, v * z2 * z2, v * z1 * z2};
                double tabs[5] = {va * fabs(z1), va * fabs(z2), va * z1 * z1, va * z2 * z2,
                                  va * fabs(z1 * z2)};
                for (int ch = 0; ch < C; ch++) {
                    double t = gpx[ch] * e;
                    if (inside) { S[ch] += t; M[ch] += fabs(t); }
                    if (tie) Z[ch] += fabs(t);
                }
                for (int j = 0; j < 5; j++) {
                    if (inside) { S[C + j] += term[j]; M[C + j] += tabs[j]; }
                    if (tie) Z[C + j] += tabs[j];
                }
            }
        }
        double c = G.c, s = G.s, s1 = G.s1, s2 = G.s2;
        double rot = s1 / s2 - s2 / s1;
        /* the chain rule, applied to the sums, their magnitudes and slacks */
        for (int which = 0; which < 3; which++) {
            double *src = which == 0 ? S : (which == 1 ? M : Z);
            double *dst = which == 0 ? out : (which == 1 ? omg : osl);
            if (!dst) continue;
            if (which == 0) {
                dst[0] = (c / s1) * src[C] - (s / s2) * src[C + 1];
                dst[1] = (s / s1) * src[C] + (c / s2) * src[C + 1];
                dst[4] = rot * src[C + 4];
            } else {
                dst[0] = fabs(c / s1) * src[C] + fabs(s / s2) * src[C + 1];
                dst[1] = fabs(s / s1) * src[C] + fabs(c / s2) * src[C + 1];
                dst[4] = fabs(rot) * src[C + 4];
            }
            dst[2] = src[C + 2] / s1;
            dst[3] = src[C + 3] / s2;
            for (int ch = 0; ch < C; ch++) dst[5 + ch] = src[ch];
        }
    }
    free(S);
}

/* grad/gslack/gmag: [B][N][5+C] fp64 (gslack, gmag may be NULL) */
int orc_grad(const double *params, const double *grad_image, int B, int N, int H, int W, int C,
             double k, double tau, int nthreads, double *grad, double *gslack,
             double *gmag) {
    if (!params || !grad_image || !grad || B < 1 || N < 0 || H < 1 || W < 1 || C < 1) return -1;
    bwd_ctx Bc = {params, grad_image, N, H, W, C, k, tau, grad, gslack, gmag};
    for_frames(B, nthreads, bwd_frame, &Bc);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* binning: brute force over (tile, Gaussian)                               */

typedef struct {
    const double *params;
    int N, H, W, C, T, nTx, nTy;
    double k;
    int *counts;              /* [B][nT] */
    const long long *tile_off; /* [B*nT + 1] or NULL in the count pass */
    int *list;
    int *rect;                /* [B][N][4] pixel box x0,x1,y0,y1 or NULL */
} bin_ctx;

static int box_meets_tile(const gauss_geo *G, int tx, int ty, int T, int H, int W) {
    if (!G->valid || G->x0 > G->x1 || G->y0 > G->y1) return 0;
    int px0 = tx * T, px1 = tx * T + T - 1, py0 = ty * T, py1 = ty * T + T - 1;
    if (px1 > W - 1) px1 = W - 1;
    if (py1 > H - 1) py1 = H - 1;
    return G->x0 <= px1 && G->x1 >= px0 && G->y0 <= py1 && G->y1 >= py0;
}

static void bin_frame(void *p, int b) {
    bin_ctx *Bn = (bin_ctx *)p;
    int N = Bn->N, P = 5 + Bn->C, nT = Bn->nTx * Bn->nTy;
    const double *gp = Bn->params + (size_t)b * N * P;
    gauss_geo *geo = (gauss_geo *)malloc(sizeof(gauss_geo) * (size_t)(N > 0 ? N : 1));
    for (int n = 0; n < N; n++) {
        geometry(gp + (size_t)n * P, Bn->C, Bn->H, Bn->W, Bn->k, &geo[n]);
        if (Bn->rect) {
            int *r = Bn->rect + ((size_t)b * N + n) * 4;
            int empty = !geo[n].valid || geo[n].x0 > geo[n].x1 || geo[n].y0 > geo[n].y1;
            r[0] = empty ? -1 : geo[n].x0;
            r[1] = empty ? -1 : geo[n].x1;
            r[2] = empty ? -1 : geo[n].y0;
            r[3] = empty ? -1 : geo[n].y1;
        }
    }
    for (int ty = 0; ty < Bn->nTy; ty++) {
        for (int tx = 0; tx < Bn->nTx; tx++) {
            int t = ty * Bn->nTx + tx;
            long long at = Bn->tile_off ? Bn->tile_off[(size_t)b * nT + t] : 0;
            int cnt = 0;
            for (int n = 0; n < N; n++) {
                if (!box_meets_tile(&geo[n], tx, ty, Bn->T, Bn->H, Bn->W)) continue;
                if (Bn->tile_off) Bn->list[at + cnt] = n;
                cnt++;
            }
            if (!Bn->tile_off) Bn->counts[(size_t)b * nT + t] = cnt;
        }
    }
    free(geo);
}

/* counts [B*nT], tile_off [B*nT+1] (exclusive scan, last = total);
 * list may be NULL (then only counts/offsets/rects are produced);
 * returns total pairs, or -1 on bad args, -2 if list is given and cap < total */
long long orc_bin(const double *params, int B, int N, int H, int W, int C, double k, int T,
                  int nthreads, int *counts, long long *tile_off, int *list, long long cap,
                  int *rect) {
    if (!params || !counts || !tile_off || B < 1 || N < 0 || H < 1 || W < 1 || C < 1 || T < 1)
        return -1;
    int nTx = (W + T - 1) / T, nTy = (H + T - 1) / T;
    bin_ctx Bn = {params, N, H, W, C, T, nTx, nTy, k, counts, NULL, list, rect};
    for_frames(B, nthreads, bin_frame, &Bn);
    long long tot = 0, nT = (long long)nTx * nTy;
    for (long long i = 0; i < (long long)B * nT; i++) {
        tile_off[i] = tot;
        tot += counts[i];
    }
    tile_off[(long long)B * nT] = tot;
    if (!list) return tot;
    if (cap < tot) return -2;
    Bn.tile_off = tile_off;
    Bn.rect = NULL;
    for_frames(B, nthreads, bin_frame, &Bn);
    return tot;
}

/* ------------------------------------------------------------------------ */
/* support count: pairs with q <= k^2 per frame (no image, no exp)           */

typedef struct {
    const double *params;
    int N, H, W, C;
    double k;
    long long *pairs;
} cnt_ctx;

static void cnt_frame(void *p, int b) {
    cnt_ctx *X = (cnt_ctx *)p;
    int N = X->N, P = 5 + X->C;
    double kk = X->k * X->k;
    const double *gp = X->params + (size_t)b * N * P;
    long long n_in = 0;
    for (int n = 0; n < N; n++) {
        gauss_geo G;
        geometry(gp + (size_t)n * P, X->C, X->H, X->W, X->k, &G);
        int xa, xb, ya, yb;
        if (!scan_box(&G, X->H, X->W, &xa, &xb, &ya, &yb)) continue;
        for (int y = ya; y <= yb; y++)
            for (int x = xa; x <= xb; x++) {
                double z1, z2;
                if (pixel_q(&G, x, y, &z1, &z2) <= kk) n_in++;
            }
    }
    X->pairs[b] = n_in;
}

/* pairs [B]: number of (Gaussian, pixel) pairs inside the truncation */
int orc_count_support(const double *params, int B, int N, int H, int W, int C, double k,
                      int nthreads, long long *pairs) {
    if (!params || !pairs || B < 1 || N < 0 || H < 1 || W < 1 || C < 1) return -1;
    cnt_ctx X = {params, N, H, W, C, k, pairs};
    for_frames(B, nthreads, cnt_frame, &X);
    return 0;
}
