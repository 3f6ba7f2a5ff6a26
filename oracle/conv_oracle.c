/*
 * Reference 2-D convolution: a plain, slow, obviously correct CPU model.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table
 * or helper with the HIP path.
 *
 * Every value is carried in double precision.  Inputs stored as fp32 or bf16
 * convert to double exactly, so the only rounding here is the fp64
 * accumulation itself.
 *
 * What is computed (sources are the three pages of the reference set):
 *
 *   - Output extent.  oarust 0.8.6 src/rs/ml/matrix/conv.rs,
 *     `Conv1dGeometry::resolve`: effective kernel (k-1)*d+1, extent
 *     (in + 2p - effective)/s + 1, and an error when the padded input is
 *     shorter than the effective kernel.  Applied per spatial axis.
 *
 *   - Forward.  teeny-kernels 0.2.0 src/nn/conv/conv2d.rs, `conv2d_forward`
 *     doc comment and body: cross-correlation (no kernel flip), input row
 *     oh*stride + kh - pad, zero outside the image, group g = co / (C_out/G)
 *     reading input channels [g*C/G, (g+1)*C/G); dilation enters as kh*dil
 *     as in burn-cubecl 0.22.0-pre.4 src/kernel/conv/im2col.rs, `im2col`
 *     (column formula o*stride + k*dilation - padding).  The bias is added
 *     per output channel as in `conv2d_bias_forward` on the teeny-kernels
 *     page.
 *
 *   - Input gradient.  The adjoint of the bias-free forward.  Computed here
 *     deliberately as the scatter that transposes the forward loop (the
 *     shape of `conv2d_backward_dx` on the teeny-kernels page, without its
 *     atomics because this loop is serial per image), so that it is an
 *     independent formulation from the gather used on the GPU.  A second,
 *     per-element gather (`oracle_conv2d_input_grad_at`) evaluates the
 *     defining sum for sampled elements only; oarust's `conv_2d_backward`
 *     dispatches its input adjoint over input elements in the same way.
 *
 * Layouts.  nhwc == 0: x [N,C,H,W], w [C_out, C/G, KH, KW], y [N,C_out,OH,OW].
 *           nhwc == 1: x [N,H,W,C], w [C_out, KH, KW, C/G], y [N,OH,OW,C_out].
 *
 * Alongside each result the oracle returns a normaliser: |bias| plus the sum
 * of |x*w| over the taps that land inside the image (|dy*w| for the input
 * gradient).  The parity tolerance is relative to it.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Spatial extent after the convolution, or -1 when the dilated kernel does
 * not fit the padded input or an argument is out of its domain. */
long oracle_out_size(long in, long k, long stride, long pad, long dil)
{
    if (in < 1 || k < 1 || stride < 1 || pad < 0 || dil < 1)
        return -1;
    long effective = (k - 1) * dil + 1;
    long padded = in + 2 * pad;
    if (padded < effective)
        return -1;
    return (padded - effective) / stride + 1;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

typedef struct {
    long N, C, H, W, CO, KH, KW, sh, sw, ph, pw, dh, dw, G, OH, OW, Cg, Mg;
    int nhwc;
} geom_t;

static int make_geom(geom_t *g, long N, long C, long H, long W, long CO,
                     long KH, long KW, long sh, long sw, long ph, long pw,
                     long dh, long dw, long G, int nhwc)
{
    if (N < 1 || C < 1 || CO < 1 || G < 1 || C % G || CO % G)
        return -1;
    g->OH = oracle_out_size(H, KH, sh, ph, dh);
    g->OW = oracle_out_size(W, KW, sw, pw, dw);
    if (g->OH < 1 || g->OW < 1)
        return -1;
    g->N = N; g->C = C; g->H = H; g->W = W; g->CO = CO;
    g->KH = KH; g->KW = KW; g->sh = sh; g->sw = sw; g->ph = ph; g->pw = pw;
    g->dh = dh; g->dw = dw; g->G = G; g->Cg = C / G; g->Mg = CO / G;
    g->nhwc = nhwc;
    return 0;
}

/* Flat offsets in the chosen layout. */
static long x_at(const geom_t *g, long n, long c, long h, long w)
{
    return g->nhwc ? ((n * g->H + h) * g->W + w) * g->C + c
                   : ((n * g->C + c) * g->H + h) * g->W + w;
}
static long y_at(const geom_t *g, long n, long co, long oh, long ow)
{
    return g->nhwc ? ((n * g->OH + oh) * g->OW + ow) * g->CO + co
                   : ((n * g->CO + co) * g->OH + oh) * g->OW + ow;
}
static long w_at(const geom_t *g, long co, long c, long kh, long kw)
{
    return g->nhwc ? ((co * g->KH + kh) * g->KW + kw) * g->Cg + c
                   : ((co * g->Cg + c) * g->KH + kh) * g->KW + kw;
}

/* One forward output: the defining sum, in the order c, kh, kw. */
static void fwd_one(const geom_t *g, const double *x, const double *w,
                    const double *bias, long n, long co, long oh, long ow,
                    double *val, double *norm)
{
    long grp = co / g->Mg;
    double acc = bias ? bias[co] : 0.0;
    double nrm = bias ? fabs(bias[co]) : 0.0;
    for (long c = 0; c < g->Cg; ++c)
        for (long kh = 0; kh < g->KH; ++kh) {
            long ih = oh * g->sh - g->ph + kh * g->dh;
            if (ih < 0 || ih >= g->H)
                continue;
            for (long kw = 0; kw < g->KW; ++kw) {
                long iw = ow * g->sw - g->pw + kw * g->dw;
                if (iw < 0 || iw >= g->W)
                    continue;
                double p = x[x_at(g, n, grp * g->Cg + c, ih, iw)] *
                           w[w_at(g, co, c, kh, kw)];
                acc += p;
                nrm += fabs(p);
            }
        }
    *val = acc;
    *norm = nrm;
}

/* Full forward convolution.  bias may be NULL; norm may be NULL. */
int oracle_conv2d_forward(const double *x, const double *w, const double *bias,
                          double *y, double *norm, long N, long C, long H,
                          long W, long CO, long KH, long KW, long sh, long sw,
                          long ph, long pw, long dh, long dw, long G, int nhwc)
{
    geom_t g;
    if (make_geom(&g, N, C, H, W, CO, KH, KW, sh, sw, ph, pw, dh, dw, G, nhwc))
        return -1;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (long n = 0; n < g.N; ++n)
        for (long co = 0; co < g.CO; ++co)
            for (long oh = 0; oh < g.OH; ++oh)
                for (long ow = 0; ow < g.OW; ++ow) {
                    double v, r;
                    fwd_one(&g, x, w, bias, n, co, oh, ow, &v, &r);
                    long o = y_at(&g, n, co, oh, ow);
                    y[o] = v;
                    if (norm)
                        norm[o] = r;
                }
    return 0;
}

/* Forward convolution at selected flat output offsets (layout order). */
int oracle_conv2d_forward_at(const double *x, const double *w,
                             const double *bias, const int64_t *idx,
                             long count, double *out, double *norm, long N,
                             long C, long H, long W, long CO, long KH, long KW,
                             long sh, long sw, long ph, long pw, long dh,
                             long dw, long G, int nhwc)
{
    geom_t g;
    if (make_geom(&g, N, C, H, W, CO, KH, KW, sh, sw, ph, pw, dh, dw, G, nhwc))
        return -1;
    long total = g.N * g.CO * g.OH * g.OW;
    for (long i = 0; i < count; ++i)
        if (idx[i] < 0 || idx[i] >= total)
            return -2;
#pragma omp parallel for schedule(dynamic, 64)
    for (long i = 0; i < count; ++i) {
        long o = idx[i], n, co, oh, ow;
        if (g.nhwc) {
            co = o % g.CO; o /= g.CO;
            ow = o % g.OW; o /= g.OW;
            oh = o % g.OH; n = o / g.OH;
        } else {
            ow = o % g.OW; o /= g.OW;
            oh = o % g.OH; o /= g.OH;
            co = o % g.CO; n = o / g.CO;
        }
        double v, r;
        fwd_one(&g, x, w, bias, n, co, oh, ow, &v, &r);
        out[i] = v;
        if (norm)
            norm[i] = r;
    }
    return 0;
}

/* Input gradient of the bias-free forward, by scattering every product of
 * the forward loop back onto the input element it read.  dy has the output
 * shape, dx the input shape; dx and norm are overwritten. */
int oracle_conv2d_input_grad(const double *dy, const double *w, double *dx,
                             double *norm, long N, long C, long H, long W,
                             long CO, long KH, long KW, long sh, long sw,
                             long ph, long pw, long dh, long dw, long G,
                             int nhwc)
{
    geom_t g;
    if (make_geom(&g, N, C, H, W, CO, KH, KW, sh, sw, ph, pw, dh, dw, G, nhwc))
        return -1;
    long in_count = g.N * g.C * g.H * g.W;
    memset(dx, 0, sizeof(double) * (size_t)in_count);
    if (norm)
        memset(norm, 0, sizeof(double) * (size_t)in_count);
    /* Images write disjoint slices of dx, so they run in parallel. */
#pragma omp parallel for schedule(dynamic)
    for (long n = 0; n < g.N; ++n)
        for (long co = 0; co < g.CO; ++co) {
            long grp = co / g.Mg;
            for (long oh = 0; oh < g.OH; ++oh)
                for (long ow = 0; ow < g.OW; ++ow) {
                    double d = dy[y_at(&g, n, co, oh, ow)];
                    for (long c = 0; c < g.Cg; ++c)
                        for (long kh = 0; kh < g.KH; ++kh) {
                            long ih = oh * g.sh - g.ph + kh * g.dh;
                            if (ih < 0 || ih >= g.H)
                                continue;
                            for (long kw = 0; kw < g.KW; ++kw) {
                                long iw = ow * g.sw - g.pw + kw * g.dw;
                                if (iw < 0 || iw >= g.W)
                                    continue;
                                long xi = x_at(&g, n, grp * g.Cg + c, ih, iw);
                                double p = d * w[w_at(&g, co, c, kh, kw)];
                                dx[xi] += p;
                                if (norm)
                                    norm[xi] += fabs(p);
                            }
                        }
                }
        }
    return 0;
}

/* Input gradient at selected flat input offsets, from the defining sum:
 * dx[n,ci,ih,iw] = sum over co in ci's group and taps (kh,kw) such that
 * ih + ph - kh*dh is a non-negative multiple of sh whose quotient is a
 * valid output row (and likewise for columns) of dy * w. */
int oracle_conv2d_input_grad_at(const double *dy, const double *w,
                                const int64_t *idx, long count, double *out,
                                double *norm, long N, long C, long H, long W,
                                long CO, long KH, long KW, long sh, long sw,
                                long ph, long pw, long dh, long dw, long G,
                                int nhwc)
{
    geom_t g;
    if (make_geom(&g, N, C, H, W, CO, KH, KW, sh, sw, ph, pw, dh, dw, G, nhwc))
        return -1;
    long total = g.N * g.C * g.H * g.W;
    for (long i = 0; i < count; ++i)
        if (idx[i] < 0 || idx[i] >= total)
            return -2;
#pragma omp parallel for schedule(dynamic, 64)
    for (long i = 0; i < count; ++i) {
        long o = idx[i], n, ci, ih, iw;
        if (g.nhwc) {
            ci = o % g.C; o /= g.C;
            iw = o % g.W; o /= g.W;
            ih = o % g.H; n = o / g.H;
        } else {
            iw = o % g.W; o /= g.W;
            ih = o % g.H; o /= g.H;
            ci = o % g.C; n = o / g.C;
        }
        long grp = ci / g.Cg, c = ci % g.Cg;
        double acc = 0.0, nrm = 0.0;
        for (long co = grp * g.Mg; co < (grp + 1) * g.Mg; ++co)
            for (long kh = 0; kh < g.KH; ++kh) {
                long th = ih + g.ph - kh * g.dh;
                if (th < 0 || th % g.sh != 0 || th / g.sh >= g.OH)
                    continue;
                for (long kw = 0; kw < g.KW; ++kw) {
                    long tw = iw + g.pw - kw * g.dw;
                    if (tw < 0 || tw % g.sw != 0 || tw / g.sw >= g.OW)
                        continue;
                    double p = dy[y_at(&g, n, co, th / g.sh, tw / g.sw)] *
                               w[w_at(&g, co, c, kh, kw)];
                    acc += p;
                    nrm += fabs(p);
                }
            }
        out[i] = acc;
        if (norm)
            norm[i] = nrm;
    }
    return 0;
}

/*
 * One-dimensional convolution.  oarust 0.8.6 src/rs/ml/matrix/conv.rs,
 * `conv_1d` and `Conv1dGeometry::resolve`: NCL input, OIK weight, a bias per
 * output channel, stride, symmetric padding and dilation inside the kernel
 * window; output length (L + 2p - ((K-1)d + 1))/s + 1.  The page lowers it
 * to an unfold (im2col) and a GEMM; here it is the defining sum
 *
 *   y[n, co, t] = b[co] + sum_{c < C/G} sum_{k < K}
 *                 x[n, g*C/G + c, t*s - p + k*d] * w[co, c, k],
 *
 * x zero outside [0, L), g = co / (C_out/G).  Groups extend the page's
 * definition the way the 2-D forward has them.  nlc == 0: x [N, C, L],
 * w [C_out, C/G, K], y [N, C_out, OL]; nlc == 1: x [N, L, C],
 * w [C_out, K, C/G], y [N, OL, C_out].  norm as for the 2-D forward.
 */
int oracle_conv1d_forward(const double *x, const double *w, const double *bias,
                          double *y, double *norm, long N, long C, long L,
                          long CO, long K, long s, long p, long d, long G,
                          int nlc)
{
    if (N < 1 || C < 1 || CO < 1 || G < 1 || C % G || CO % G)
        return -1;
    long OL = oracle_out_size(L, K, s, p, d);
    if (OL < 1)
        return -1;
    long Cg = C / G, Mg = CO / G;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (long n = 0; n < N; ++n)
        for (long co = 0; co < CO; ++co)
            for (long t = 0; t < OL; ++t) {
                long grp = co / Mg;
                double acc = bias ? bias[co] : 0.0;
                double nrm = bias ? fabs(bias[co]) : 0.0;
                for (long c = 0; c < Cg; ++c)
                    for (long k = 0; k < K; ++k) {
                        long l = t * s - p + k * d;
                        if (l < 0 || l >= L)
                            continue;
                        long ci = grp * Cg + c;
                        double xv = nlc ? x[(n * L + l) * C + ci] : x[(n * C + ci) * L + l];
                        double wv = nlc ? w[(co * K + k) * Cg + c] : w[(co * Cg + c) * K + k];
                        acc += xv * wv;
                        nrm += fabs(xv * wv);
                    }
                long o = nlc ? (n * OL + t) * CO + co : (n * CO + co) * OL + t;
                y[o] = acc;
                if (norm)
                    norm[o] = nrm;
            }
    return 0;
}

/*
 * Transposed 2-D convolution.  oarust 0.8.6 src/rs/ml/matrix/conv.rs,
 * `conv_transpose_2d` and `ConvTranspose2dGeometry::resolve`: NCHW input,
 * weight [C_in, C_out, K, K] (input channels first), a bias per output
 * channel, stride and padding, output extent (H - 1)*s + K - 2p.  Every
 * input element spreads its value over a K x K window of the output:
 *
 *   y[n, co, ih*sh - ph + kh*dh, iw*sw - pw + kw*dw]
 *       += x[n, ci, ih, iw] * w[ci, co - g*C_out/G, kh, kw]
 *
 * for ci in group g (g = ci / (C_in/G)) and co in the same group, keeping
 * only the output positions inside [0, OH) x [0, OW); then the bias.
 * Written deliberately as this scatter, the literal transpose of the forward
 * loop.  Per axis, dilation, groups and an output padding op (0 <= op < s,
 * extra rows and columns at the far edge) generalise the page's square,
 * undilated, ungrouped case: OH = (H - 1)*sh - 2ph + dh*(KH - 1) + 1 + oph.
 * nhwc == 0: x [N, C_in, H, W], w [C_in, C_out/G, KH, KW],
 * y [N, C_out, OH, OW]; nhwc == 1: x [N, H, W, C_in], w [C_in, KH, KW,
 * C_out/G], y [N, OH, OW, C_out].  norm = |b| + sum of |x*w| landing there.
 * Returns -1 for an invalid geometry (including an empty output).
 */
long oracle_conv_transpose_size(long in, long k, long s, long p, long d, long op)
{
    if (in < 1 || k < 1 || s < 1 || d < 1 || p < 0 || op < 0 || op >= s)
        return -1;
    long out = (in - 1) * s - 2 * p + d * (k - 1) + 1 + op;
    return out >= 1 ? out : -1;
}

int oracle_conv_transpose2d(const double *x, const double *w, const double *bias,
                            double *y, double *norm, long N, long CI, long H,
                            long W, long CO, long KH, long KW, long sh, long sw,
                            long ph, long pw, long oph, long opw, long dh,
                            long dw, long G, int nhwc)
{
    if (N < 1 || CI < 1 || CO < 1 || G < 1 || CI % G || CO % G)
        return -1;
    long OH = oracle_conv_transpose_size(H, KH, sh, ph, dh, oph);
    long OW = oracle_conv_transpose_size(W, KW, sw, pw, dw, opw);
    if (OH < 1 || OW < 1)
        return -1;
    long Cg = CI / G, Mg = CO / G;
    long ysz = N * CO * OH * OW;
    for (long o = 0; o < ysz; ++o) {
        y[o] = 0.0;
        if (norm)
            norm[o] = 0.0;
    }
    /* Images are independent: parallel over n, serial scatter inside. */
#pragma omp parallel for schedule(dynamic)
    for (long n = 0; n < N; ++n)
        for (long ci = 0; ci < CI; ++ci) {
            long grp = ci / Cg;
            for (long ih = 0; ih < H; ++ih)
                for (long iw = 0; iw < W; ++iw) {
                    double xv = nhwc ? x[((n * H + ih) * W + iw) * CI + ci]
                                     : x[((n * CI + ci) * H + ih) * W + iw];
                    for (long m = 0; m < Mg; ++m) {
                        long co = grp * Mg + m;
                        for (long kh = 0; kh < KH; ++kh) {
                            long oh = ih * sh - ph + kh * dh;
                            if (oh < 0 || oh >= OH)
                                continue;
                            for (long kw = 0; kw < KW; ++kw) {
                                long ow = iw * sw - pw + kw * dw;
                                if (ow < 0 || ow >= OW)
                                    continue;
                                double wv = nhwc ? w[((ci * KH + kh) * KW + kw) * Mg + m]
                                                 : w[((ci * Mg + m) * KH + kh) * KW + kw];
                                long o = nhwc ? ((n * OH + oh) * OW + ow) * CO + co
                                              : ((n * CO + co) * OH + oh) * OW + ow;
                                y[o] += xv * wv;
                                if (norm)
                                    norm[o] += fabs(xv * wv);
                            }
                        }
                    }
                }
        }
    if (bias) {
#pragma omp parallel for schedule(static)
        for (long o = 0; o < ysz; ++o) {
            long co = nhwc ? o % CO : (o / (OH * OW)) % CO;
            y[o] += bias[co];
            if (norm)
                norm[o] += fabs(bias[co]);
        }
    }
    return 0;
}

/*
 * Weight gradient of the forward convolution:
 *
 *   dw[co, c, kh, kw] = sum_{n, oh, ow} dy[n, co, oh, ow]
 *                       * x[n, g*C/G + c, oh*sh - ph + kh*dh, ow*sw - pw + kw*dw],
 *
 * g = co / (C_out/G), x zero outside the image.  Sources: burn-cubecl
 * 0.22.0-pre.4 src/kernel/conv/im2col.rs, `wgrad_im2col_1x1` (for a 1x1
 * kernel, the sum over pixels of grad_out[pixel, c_out] * input[pixel, c_in])
 * and `wgrad_im2col` (the same over the im2col columns (kernel..., channel));
 * teeny-kernels 0.2.0 src/nn/conv/conv2d.rs, `conv2d_backward_dw` (the same
 * sum accumulated per (c_in_local, kh, kw) into a zeroed dw).  Written here
 * as the defining sum per weight element, in the order n, oh, ow.  The weight
 * is laid out as in the forward (OIHW or OHWI); dy as the forward's y.
 * norm = sum of |dy * x| over the terms that land inside the image.
 */
int oracle_conv2d_weight_grad(const double *x, const double *dy, double *dw,
                              double *norm, long N, long C, long H, long W,
                              long CO, long KH, long KW, long sh, long sw,
                              long ph, long pw, long dh, long dw_, long G,
                              int nhwc)
{
    geom_t g;
    if (make_geom(&g, N, C, H, W, CO, KH, KW, sh, sw, ph, pw, dh, dw_, G, nhwc))
        return -1;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (long co = 0; co < g.CO; ++co)
        for (long c = 0; c < g.Cg; ++c) {
            long grp = co / g.Mg;
            for (long kh = 0; kh < g.KH; ++kh)
                for (long kw = 0; kw < g.KW; ++kw) {
                    double acc = 0.0, nrm = 0.0;
                    for (long n = 0; n < g.N; ++n)
                        for (long oh = 0; oh < g.OH; ++oh) {
                            long ih = oh * g.sh - g.ph + kh * g.dh;
                            if (ih < 0 || ih >= g.H)
                                continue;
                            for (long ow = 0; ow < g.OW; ++ow) {
                                long iw = ow * g.sw - g.pw + kw * g.dw;
                                if (iw < 0 || iw >= g.W)
                                    continue;
                                double p = dy[y_at(&g, n, co, oh, ow)] *
                                           x[x_at(&g, n, grp * g.Cg + c, ih, iw)];
                                acc += p;
                                nrm += fabs(p);
                            }
                        }
                    long o = w_at(&g, co, c, kh, kw);
                    dw[o] = acc;
                    if (norm)
                        norm[o] = nrm;
                }
        }
    return 0;
}
