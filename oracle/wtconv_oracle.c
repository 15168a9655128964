/*
 * WTConv CPU oracle, fp64. TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py
 * may load this library. The product path (the HIP library) never links,
 * loads or calls it, and this file shares no code with it.
 *
 * What it computes
 * ----------------
 * The wavelet-convolution (WTConv) layer named in the abstract of
 * "I/O-aware reformulation of wavelet convolution" (arXiv:2608.10805,
 * tech.sinsc.com page and the layerthelatestinalattice.com summary page,
 * Abstract): a drop-in replacement for a convolution whose receptive field
 * grows exponentially with the number of Haar decomposition levels L while
 * its parameter count grows linearly. The abstract names its parts: a Haar
 * analysis butterfly, per-channel learned scales on the convolution of the
 * subbands, and a multi-level synthesis cascade. The layer, per (b, c) plane:
 *
 *   X_0 = x
 *   for l = 1..L:  (LL_l, B1_l, B2_l, B3_l) = DWT(X_{l-1});  X_l = LL_l
 *   Z_l^s = scale[l][c][s] * corr(band_l^s, w_lvl[l][c][s])     s = 0..3
 *   R_L = 0;  for l = L..1:  R_{l-1} = IWT(Z_l^0 + R_l, Z_l^1, Z_l^2, Z_l^3)
 *   y = corr(x, w_base[c]) + R_0
 *
 * Readings taken where the pages are silent (each is a stated convention):
 *   - DWT is the orthonormal 2x2 Haar butterfly on (a b / c d):
 *       LL = (a+b+c+d)/2, B1 = (a+b-c-d)/2 (top minus bottom row),
 *       B2 = (a-b+c-d)/2 (left minus right column), B3 = (a-b-c+d)/2;
 *     IWT is its inverse (the same matrix: the half-Hadamard is symmetric
 *     and its own inverse).
 *   - corr is a 'same' cross-correlation, stride 1, zero padding k/2 on
 *     each side, at the band grid of its own level:
 *       corr(u, w)[i][j] = sum_{m,n<k} w[m][n] * u[i+m-k/2][j+n-k/2].
 *   - level l+1 analyses the raw LL_l, not the convolved one;
 *   - the coarser result R_l is added to the processed LL band Z_l^0;
 *   - no bias and no scale on the base path;
 *   - an image of odd height or width is zero-padded by one row at the
 *     bottom or one column at the right before its analysis, and the
 *     synthesis output is cropped back to the image's size: level l has a
 *     band grid of ceil(h_{l-1} / 2) x ceil(w_{l-1} / 2). (The pages do not
 *     cover sizes that 2^L does not divide; this is the plainest extension,
 *     and equals running the layer on x zero-padded to multiples of 2^L and
 *     cropping the result.)
 *
 * Layouts (all row-major, fp64 here):
 *   x, y, dy, dx    [B][C][H][W]
 *   w_base          [C][kb][kb]
 *   w_lvl           [L][C][4][k][k]      (level index 0 = level 1)
 *   scale           [L][C][4]
 *
 * Two forward variants are kept so they can be checked against each other:
 *   wto_fwd         the cascade above, step by step (the definition);
 *   wto_fwd_closed  the single-pass form of reformulation (2) of the
 *                   abstract: each subband computed directly from its
 *                   2^l x 2^l block of x, and the synthesis written as one
 *                   sum per output pixel indexed by the bits of the output
 *                   coordinates.
 * Backward:
 *   wto_bwd_data    dx by literal reverse-mode of the cascade;
 *   wto_bwd_weight  dW_base, dW_lvl, dscale by literal reverse-mode;
 *   wto_bwd_weight_gcorr  the same three from the correlation
 *                   G = corr-grad(band(x), band(dy)) with the scale folded
 *                   out: dW = scale * G, dscale = sum(W * G) (the abstract's
 *                   reformulation (3), scales folded into the weights,
 *                   applied to the gradient).
 *
 * Reductions over the batch run in a fixed order, so results do not depend
 * on the number of OpenMP threads.
 */
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ---------------------------------------------------------------- helpers */

static void *xmalloc(size_t n)
{
    void *p = calloc(n ? n : 1, 1);
    if (!p) abort();
    return p;
}

/* sign of band s at intra-block position (u = row bit, v = column bit) */
static double band_sign(int s, int u, int v)
{
    double su = u ? -1.0 : 1.0, sv = v ? -1.0 : 1.0;
    switch (s) {
    case 0: return 1.0;
    case 1: return su;
    case 2: return sv;
    default: return su * sv;
    }
}

/* out[i][j] = sum_{m,n} ker[m][n] * u[i+m-p][j+n-p], zero outside */
static void corr_same(const double *u, int h, int w, const double *ker, int k,
                      double *out)
{
    int p = k / 2;
    for (int i = 0; i < h; i++)
        for (int j = 0; j < w; j++) {
            double acc = 0.0;
            for (int m = 0; m < k; m++) {
                int ii = i + m - p;
                if (ii < 0 || ii >= h) continue;
                for (int n = 0; n < k; n++) {
                    int jj = j + n - p;
                    if (jj < 0 || jj >= w) continue;
                    acc += ker[m * k + n] * u[ii * w + jj];
                }
            }
            out[i * w + j] = acc;
        }
}

/* out += corr_same^T(v): the literal transpose, written as a scatter */
static void corr_same_adjoint_acc(const double *v, int h, int w,
                                  const double *ker, int k, double *out)
{
    int p = k / 2;
    for (int i = 0; i < h; i++)
        for (int j = 0; j < w; j++) {
            double vij = v[i * w + j];
            for (int m = 0; m < k; m++) {
                int ii = i + m - p;
                if (ii < 0 || ii >= h) continue;
                for (int n = 0; n < k; n++) {
                    int jj = j + n - p;
                    if (jj < 0 || jj >= w) continue;
                    out[ii * w + jj] += ker[m * k + n] * vij;
                }
            }
        }
}

/* g[m][n] += sum_{i,j} v[i][j] * u[i+m-p][j+n-p]  (d corr / d ker) */
static void corr_same_wgrad_acc(const double *u, const double *v, int h, int w,
                                int k, double *g)
{
    int p = k / 2;
    for (int m = 0; m < k; m++)
        for (int n = 0; n < k; n++) {
            double acc = 0.0;
            for (int i = 0; i < h; i++) {
                int ii = i + m - p;
                if (ii < 0 || ii >= h) continue;
                for (int j = 0; j < w; j++) {
                    int jj = j + n - p;
                    if (jj < 0 || jj >= w) continue;
                    acc += v[i * w + j] * u[ii * w + jj];
                }
            }
            g[m * k + n] += acc;
        }
}

static int half_up(int v) { return (v + 1) / 2; }

/* one-level Haar analysis of an h x w image into 4 bands of ceil(h/2) x
   ceil(w/2), band-major: bands[s][i][j]; an odd last row or column is
   paired with a zero one */
static void dwt2(const double *X, int h, int w, double *bands)
{
    int h2 = half_up(h), w2 = half_up(w), n2 = h2 * w2;
    for (int i = 0; i < h2; i++)
        for (int j = 0; j < w2; j++) {
            int r0 = 2 * i, r1 = 2 * i + 1, c0 = 2 * j, c1 = 2 * j + 1;
            double a = X[r0 * w + c0];
            double b = c1 < w ? X[r0 * w + c1] : 0.0;
            double c = r1 < h ? X[r1 * w + c0] : 0.0;
            double d = (r1 < h && c1 < w) ? X[r1 * w + c1] : 0.0;
            bands[0 * n2 + i * w2 + j] = (a + b + c + d) / 2.0;
            bands[1 * n2 + i * w2 + j] = (a + b - c - d) / 2.0;
            bands[2 * n2 + i * w2 + j] = (a - b + c - d) / 2.0;
            bands[3 * n2 + i * w2 + j] = (a - b - c + d) / 2.0;
        }
}

/* inverse of dwt2: 4 bands of h2 x w2 -> the image of 2h2 x 2w2, of which
   the top-left h x w (h <= 2h2, w <= 2w2) is written to X (row stride w) */
static void iwt2_crop(const double *bands, int h2, int w2, double *X, int h, int w)
{
    int n2 = h2 * w2;
    for (int i = 0; i < h2; i++)
        for (int j = 0; j < w2; j++) {
            double b0 = bands[0 * n2 + i * w2 + j], b1 = bands[1 * n2 + i * w2 + j];
            double b2 = bands[2 * n2 + i * w2 + j], b3 = bands[3 * n2 + i * w2 + j];
            int r0 = 2 * i, r1 = 2 * i + 1, c0 = 2 * j, c1 = 2 * j + 1;
            if (r0 < h && c0 < w) X[r0 * w + c0] = (b0 + b1 + b2 + b3) / 2.0;
            if (r0 < h && c1 < w) X[r0 * w + c1] = (b0 + b1 - b2 - b3) / 2.0;
            if (r1 < h && c0 < w) X[r1 * w + c0] = (b0 - b1 + b2 - b3) / 2.0;
            if (r1 < h && c1 < w) X[r1 * w + c1] = (b0 - b1 - b2 + b3) / 2.0;
        }
}

static void iwt2(const double *bands, int h2, int w2, double *X)
{
    iwt2_crop(bands, h2, w2, X, 2 * h2, 2 * w2);
}

/* offsets of the parameter blocks of channel c */
static const double *wl_ptr(const double *w_lvl, int C, int k, int l1, int c, int s)
{
    /* l1 is the 1-based level */
    return w_lvl + ((((size_t)(l1 - 1) * C + c) * 4 + s) * k * k);
}
static double sc_val(const double *scale, int C, int l1, int c, int s)
{
    return scale[((size_t)(l1 - 1) * C + c) * 4 + s];
}

/* Haar pyramid of one plane: lvl[l] holds the 4 bands of level l (1-based),
   each h[l] x w[l] = ceil(h[l-1] / 2) x ceil(w[l-1] / 2), h[0] x w[0] the
   plane. lvl[0] is unused. */
typedef struct {
    int L, H, W;
    int h[33], w[33];
    double *lvl[33];
} pyramid;

static void pyramid_sizes(pyramid *P, int H, int W, int L)
{
    P->L = L; P->H = H; P->W = W;
    P->h[0] = H; P->w[0] = W;
    for (int l = 1; l <= L; l++) {
        P->h[l] = half_up(P->h[l - 1]);
        P->w[l] = half_up(P->w[l - 1]);
    }
}

static void pyramid_build(pyramid *P, const double *plane, int H, int W, int L)
{
    pyramid_sizes(P, H, W, L);
    const double *prev = plane;
    for (int l = 1; l <= L; l++) {
        P->lvl[l] = xmalloc(sizeof(double) * 4 * (size_t)P->h[l] * P->w[l]);
        dwt2(prev, P->h[l - 1], P->w[l - 1], P->lvl[l]);
        prev = P->lvl[l];   /* band 0 (LL) is the first h[l] x w[l] block */
    }
}

static void pyramid_free(pyramid *P)
{
    for (int l = 1; l <= P->L; l++) free(P->lvl[l]);
}

/* ------------------------------------------------------ single-level Haar */

/* Exposed for the reconstruction/orthonormality checks. */
void wto_haar_dwt(const double *X, int H, int W, double *bands)
{
    dwt2(X, H, W, bands);
}

void wto_haar_iwt(const double *bands, int H2, int W2, double *X)
{
    iwt2(bands, H2, W2, X);
}

/* ---------------------------------------------------------------- threads */

void wto_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
}

int wto_max_threads(void)
{
    return omp_get_max_threads();
}

/* ----------------------------------------------------- forward (cascade) */

static void fwd_plane(const double *x, int H, int W, int L, int C, int c,
                      int kb, int k, const double *w_base, const double *w_lvl,
                      const double *scale, double *y)
{
    corr_same(x, H, W, w_base + (size_t)c * kb * kb, kb, y);
    if (L == 0) return;

    pyramid P;
    pyramid_build(&P, x, H, W, L);

    /* R holds the result carried up from the coarser levels, at the size
       of the level-l band grid (the synthesis output cropped) */
    double *R = NULL;
    for (int l = L; l >= 1; l--) {
        int h = P.h[l], w = P.w[l], n = h * w;
        double *Z = xmalloc(sizeof(double) * 4 * (size_t)n);
        for (int s = 0; s < 4; s++) {
            corr_same(P.lvl[l] + (size_t)s * n, h, w, wl_ptr(w_lvl, C, k, l, c, s), k,
                      Z + (size_t)s * n);
            double sc = sc_val(scale, C, l, c, s);
            for (int t = 0; t < n; t++) Z[(size_t)s * n + t] *= sc;
        }
        if (R) {
            for (int t = 0; t < n; t++) Z[t] += R[t];
            free(R);
        }
        R = xmalloc(sizeof(double) * (size_t)P.h[l - 1] * P.w[l - 1]);
        iwt2_crop(Z, h, w, R, P.h[l - 1], P.w[l - 1]);
        free(Z);
    }
    for (size_t t = 0; t < (size_t)H * W; t++) y[t] += R[t];
    free(R);
    pyramid_free(&P);
}

void wto_fwd(int B, int C, int H, int W, int L, int kb, int k,
             const double *x, const double *w_base, const double *w_lvl,
             const double *scale, double *y)
{
    long planes = (long)B * C;
    size_t hw = (size_t)H * W;
#pragma omp parallel for schedule(dynamic, 1)
    for (long pl = 0; pl < planes; pl++) {
        int c = (int)(pl % C);
        fwd_plane(x + pl * hw, H, W, L, C, c, kb, k, w_base, w_lvl, scale, y + pl * hw);
    }
}

/* ------------------------------------------------- forward (closed form) */

/* band s of level l at (i, j) straight from its 2^l x 2^l block of x:
   2^-l * sum_{u,v < 2^l} sign_s(bit_{l-1} u, bit_{l-1} v) x[i 2^l + u][j 2^l + v] */
static double band_direct(const double *x, int H, int W, int l, int s, int i, int j)
{
    int side = 1 << l;
    double acc = 0.0;
    for (int u = 0; u < side; u++)
        for (int v = 0; v < side; v++) {
            int r = i * side + u, q = j * side + v;
            if (r >= H || q >= W) continue;   /* x is zero beyond the plane */
            acc += band_sign(s, (u >> (l - 1)) & 1, (v >> (l - 1)) & 1) * x[(size_t)r * W + q];
        }
    return acc / (double)side;
}

static void fwd_closed_plane(const double *x, int H, int W, int L, int C, int c,
                             int kb, int k, const double *w_base,
                             const double *w_lvl, const double *scale, double *y)
{
    corr_same(x, H, W, w_base + (size_t)c * kb * kb, kb, y);
    pyramid S;
    pyramid_sizes(&S, H, W, L);   /* band grid sizes only */
    for (int l = 1; l <= L; l++) {
        int h = S.h[l], w = S.w[l], n = h * w;
        double *band = xmalloc(sizeof(double) * (size_t)n);
        double *Z = xmalloc(sizeof(double) * 4 * (size_t)n);
        for (int s = 0; s < 4; s++) {
            for (int i = 0; i < h; i++)
                for (int j = 0; j < w; j++) band[i * w + j] = band_direct(x, H, W, l, s, i, j);
            corr_same(band, h, w, wl_ptr(w_lvl, C, k, l, c, s), k, Z + (size_t)s * n);
            double sc = sc_val(scale, C, l, c, s);
            for (int t = 0; t < n; t++) Z[(size_t)s * n + t] *= sc;
        }
        double f = 1.0 / (double)(1 << l);
        for (int hh = 0; hh < H; hh++)
            for (int ww = 0; ww < W; ww++) {
                int u = (hh >> (l - 1)) & 1, v = (ww >> (l - 1)) & 1;
                size_t pos = (size_t)(hh >> l) * w + (ww >> l);
                double acc = 0.0;
                for (int s = 0; s < 4; s++) acc += band_sign(s, u, v) * Z[(size_t)s * n + pos];
                y[(size_t)hh * W + ww] += f * acc;
            }
        free(band);
        free(Z);
    }
}

void wto_fwd_closed(int B, int C, int H, int W, int L, int kb, int k,
                    const double *x, const double *w_base, const double *w_lvl,
                    const double *scale, double *y)
{
    long planes = (long)B * C;
    size_t hw = (size_t)H * W;
#pragma omp parallel for schedule(dynamic, 1)
    for (long pl = 0; pl < planes; pl++) {
        int c = (int)(pl % C);
        fwd_closed_plane(x + pl * hw, H, W, L, C, c, kb, k, w_base, w_lvl, scale,
                         y + pl * hw);
    }
}

/* ------------------------------------------ backward data (reverse mode) */

static void bwd_data_plane(const double *dy, int H, int W, int L, int C, int c,
                           int kb, int k, const double *w_base,
                           const double *w_lvl, const double *scale, double *dx)
{
    size_t hw = (size_t)H * W;
    memset(dx, 0, sizeof(double) * hw);
    corr_same_adjoint_acc(dy, H, W, w_base + (size_t)c * kb * kb, kb, dx);
    if (L == 0) return;

    /* Reverse of the synthesis cascade: R_{l-1} = IWT(Z_l^0 + R_l, Z_l^1..3)
       sends dR_{l-1} back through DWT (the adjoint of the orthonormal IWT),
       so dZ_l = DWT(dR_{l-1}) and dR_l = its LL band. Starting from
       dR_0 = dy this is the Haar pyramid of dy. */
    pyramid dZ;
    pyramid_build(&dZ, dy, H, W, L);

    /* Reverse of the analysis chain: d band_l^s from the level-l conv, plus
       dX_l flowing back from level l+1 into the LL band. */
    double *dXl = NULL;   /* gradient w.r.t. X_l (level-l resolution) */
    for (int l = L; l >= 1; l--) {
        int h = dZ.h[l], w = dZ.w[l], n = h * w;
        double *dband = xmalloc(sizeof(double) * 4 * (size_t)n);
        for (int s = 0; s < 4; s++) {
            double sc = sc_val(scale, C, l, c, s);
            double *tmp = xmalloc(sizeof(double) * (size_t)n);
            for (int t = 0; t < n; t++) tmp[t] = sc * dZ.lvl[l][(size_t)s * n + t];
            corr_same_adjoint_acc(tmp, h, w, wl_ptr(w_lvl, C, k, l, c, s), k,
                                  dband + (size_t)s * n);
            free(tmp);
        }
        if (dXl) {
            for (int t = 0; t < n; t++) dband[t] += dXl[t];
            free(dXl);
        }
        /* adjoint of "pad, then analyse": synthesise, then crop */
        dXl = xmalloc(sizeof(double) * (size_t)dZ.h[l - 1] * dZ.w[l - 1]);
        iwt2_crop(dband, h, w, dXl, dZ.h[l - 1], dZ.w[l - 1]);
        free(dband);
    }
    for (size_t t = 0; t < hw; t++) dx[t] += dXl[t];
    free(dXl);
    pyramid_free(&dZ);
}

void wto_bwd_data(int B, int C, int H, int W, int L, int kb, int k,
                  const double *dy, const double *w_base, const double *w_lvl,
                  const double *scale, double *dx)
{
    long planes = (long)B * C;
    size_t hw = (size_t)H * W;
#pragma omp parallel for schedule(dynamic, 1)
    for (long pl = 0; pl < planes; pl++) {
        int c = (int)(pl % C);
        bwd_data_plane(dy + pl * hw, H, W, L, C, c, kb, k, w_base, w_lvl, scale,
                       dx + pl * hw);
    }
}

/* ---------------------------------------- backward weight (reverse mode) */

/* number of gradient values per channel: kb^2 + L * 4 * (k^2 + 1) */
static size_t taps_per_channel(int L, int kb, int k)
{
    return (size_t)kb * kb + (size_t)L * 4 * ((size_t)k * k + 1);
}

/* Per-plane gradient contributions, packed per channel as
   [kb*kb base][L][4][k*k w_lvl][L][4] scale. */
static void bwd_weight_plane(const double *x, const double *dy, int H, int W,
                             int L, int C, int c, int kb, int k,
                             const double *w_lvl, const double *scale, double *g)
{
    corr_same_wgrad_acc(x, dy, H, W, kb, g);
    if (L == 0) return;
    pyramid Px, Pd;
    pyramid_build(&Px, x, H, W, L);
    pyramid_build(&Pd, dy, H, W, L);   /* dZ_l = Haar pyramid of dy */
    double *gw = g + (size_t)kb * kb;
    double *gs = gw + (size_t)L * 4 * k * k;
    for (int l = 1; l <= L; l++) {
        int h = Px.h[l], w = Px.w[l], n = h * w;
        double *T = xmalloc(sizeof(double) * (size_t)n);
        double *tmp = xmalloc(sizeof(double) * (size_t)k * k);
        for (int s = 0; s < 4; s++) {
            const double *band = Px.lvl[l] + (size_t)s * n;
            const double *dZ = Pd.lvl[l] + (size_t)s * n;
            double sc = sc_val(scale, C, l, c, s);
            /* Z = sc * T, T = corr(band, w):  dscale = <dZ, T>,
               dw = corr-grad(band, sc * dZ) */
            corr_same(band, h, w, wl_ptr(w_lvl, C, k, l, c, s), k, T);
            double ds = 0.0;
            for (int t = 0; t < n; t++) ds += dZ[t] * T[t];
            gs[(l - 1) * 4 + s] += ds;
            memset(tmp, 0, sizeof(double) * (size_t)k * k);
            corr_same_wgrad_acc(band, dZ, h, w, k, tmp);
            double *dst = gw + ((size_t)(l - 1) * 4 + s) * k * k;
            for (int t = 0; t < k * k; t++) dst[t] += sc * tmp[t];
        }
        free(T);
        free(tmp);
    }
    pyramid_free(&Px);
    pyramid_free(&Pd);
}

/* Variant from the unscaled correlation G of the two pyramids. */
static void bwd_weight_plane_gcorr(const double *x, const double *dy, int H, int W,
                                   int L, int kb, int k, double *g)
{
    /* g packs [kb*kb base][L][4][k*k] G only; scale folding happens once
       per channel after the batch sum. */
    corr_same_wgrad_acc(x, dy, H, W, kb, g);
    if (L == 0) return;
    pyramid Px, Pd;
    pyramid_build(&Px, x, H, W, L);
    pyramid_build(&Pd, dy, H, W, L);
    double *gw = g + (size_t)kb * kb;
    for (int l = 1; l <= L; l++) {
        int h = Px.h[l], w = Px.w[l], n = h * w;
        for (int s = 0; s < 4; s++)
            corr_same_wgrad_acc(Px.lvl[l] + (size_t)s * n, Pd.lvl[l] + (size_t)s * n,
                                h, w, k, gw + ((size_t)(l - 1) * 4 + s) * k * k);
    }
    pyramid_free(&Px);
    pyramid_free(&Pd);
}

static void unpack_grads(int C, int L, int kb, int k, const double *acc, int c,
                         double *dw_base, double *dw_lvl, double *dscale)
{
    const double *gb = acc;
    const double *gw = gb + (size_t)kb * kb;
    const double *gs = gw + (size_t)L * 4 * k * k;
    memcpy(dw_base + (size_t)c * kb * kb, gb, sizeof(double) * (size_t)kb * kb);
    for (int l = 1; l <= L; l++)
        for (int s = 0; s < 4; s++) {
            memcpy(dw_lvl + ((((size_t)(l - 1) * C + c) * 4 + s) * k * k),
                   gw + ((size_t)(l - 1) * 4 + s) * k * k, sizeof(double) * (size_t)k * k);
            dscale[((size_t)(l - 1) * C + c) * 4 + s] = gs[(l - 1) * 4 + s];
        }
}

void wto_bwd_weight(int B, int C, int H, int W, int L, int kb, int k,
                    const double *x, const double *dy, const double *w_lvl,
                    const double *scale, double *dw_base, double *dw_lvl,
                    double *dscale)
{
    size_t taps = taps_per_channel(L, kb, k);
    size_t hw = (size_t)H * W;
    long planes = (long)B * C;
    /* per-plane partials, then a fixed-order sum over b per channel */
    double *part = xmalloc(sizeof(double) * taps * (size_t)planes);
#pragma omp parallel for schedule(dynamic, 1)
    for (long pl = 0; pl < planes; pl++) {
        int c = (int)(pl % C);
        bwd_weight_plane(x + pl * hw, dy + pl * hw, H, W, L, C, c, kb, k, w_lvl,
                         scale, part + (size_t)pl * taps);
    }
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; c++) {
        double *acc = xmalloc(sizeof(double) * taps);
        for (int b = 0; b < B; b++) {
            const double *src = part + ((size_t)b * C + c) * taps;
            for (size_t t = 0; t < taps; t++) acc[t] += src[t];
        }
        unpack_grads(C, L, kb, k, acc, c, dw_base, dw_lvl, dscale);
        free(acc);
    }
    free(part);
}

void wto_bwd_weight_gcorr(int B, int C, int H, int W, int L, int kb, int k,
                          const double *x, const double *dy, const double *w_lvl,
                          const double *scale, double *dw_base, double *dw_lvl,
                          double *dscale)
{
    size_t gtaps = (size_t)kb * kb + (size_t)L * 4 * k * k;
    size_t taps = taps_per_channel(L, kb, k);
    size_t hw = (size_t)H * W;
    long planes = (long)B * C;
    double *part = xmalloc(sizeof(double) * gtaps * (size_t)planes);
#pragma omp parallel for schedule(dynamic, 1)
    for (long pl = 0; pl < planes; pl++)
        bwd_weight_plane_gcorr(x + pl * hw, dy + pl * hw, H, W, L, kb, k,
                               part + (size_t)pl * gtaps);
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; c++) {
        double *G = xmalloc(sizeof(double) * gtaps);
        double *acc = xmalloc(sizeof(double) * taps);
        for (int b = 0; b < B; b++) {
            const double *src = part + ((size_t)b * C + c) * gtaps;
            for (size_t t = 0; t < gtaps; t++) G[t] += src[t];
        }
        memcpy(acc, G, sizeof(double) * (size_t)kb * kb);
        double *gw = acc + (size_t)kb * kb;
        double *gs = gw + (size_t)L * 4 * k * k;
        for (int l = 1; l <= L; l++)
            for (int s = 0; s < 4; s++) {
                const double *Gls = G + (size_t)kb * kb + ((size_t)(l - 1) * 4 + s) * k * k;
                const double *w = wl_ptr(w_lvl, C, k, l, c, s);
                double sc = sc_val(scale, C, l, c, s), ds = 0.0;
                for (int t = 0; t < k * k; t++) {
                    gw[((size_t)(l - 1) * 4 + s) * k * k + t] = sc * Gls[t];
                    ds += w[t] * Gls[t];
                }
                gs[(l - 1) * 4 + s] = ds;
            }
        unpack_grads(C, L, kb, k, acc, c, dw_base, dw_lvl, dscale);
        free(G);
        free(acc);
    }
    free(part);
}
