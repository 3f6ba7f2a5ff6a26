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
