// Weight gradient of a convolution, split over the pixels and reduced in a
// fixed order (no atomics).
//
// dw[co, c, kh, kw] = sum over n, oh, ow of dy[n, co, oh, ow] *
// x[n, g*C/G + c, oh*sh - ph + kh*dh, ow*sw - pw + kw*dw] (x zero outside),
// g = co / (C_out/G): the contraction over every output pixel of the batch
// that burn-cubecl 0.22.0-pre.4 src/kernel/conv/im2col.rs writes as one
// matmul (`wgrad_im2col_1x1`) or one matmul over the im2col columns
// (`wgrad_im2col`).  That page cuts the contraction into equal pieces and
// sums their partial products in a second step (`wgrad_im2col_1x1_split`,
// `split_count`), because the output is tiny next to the contraction and a
// matmul that gives each output element the whole contraction leaves the
// device idle; teeny-kernels 0.2.0 src/nn/conv/conv2d.rs instead adds every
// partial into a zeroed dw with atomics (`conv2d_backward_dw`).
//
// Here: pass 1 splits the pixels of the batch into S contiguous pieces and
// writes one fp32 partial per (piece, weight element) into the caller's
// workspace; pass 2 sums the S partials of each element in piece order and
// rounds once to the weight's dtype.  The result does not depend on timing.
//
// This file holds the generic path (any layout and dtype): in pass 1 a lane
// owns one weight element of one piece and walks the piece's pixels.
#include "kernels.hpp"

#include <algorithm>

namespace convmi {
namespace {

constexpr int kThreads = 256;

// Weight element e (flat, in the weight's layout) -> (co, c, kh, kw).
__device__ __forceinline__ void weight_coords(const Geom& g, int64_t e, int& co, int& c, int& kh,
                                              int& kw)
{
    if (g.nhwc) {  // OHWI [co][kh][kw][c]
        c = static_cast<int>(e % g.Cg); e /= g.Cg;
        kw = static_cast<int>(e % g.KW); e /= g.KW;
        kh = static_cast<int>(e % g.KH); co = static_cast<int>(e / g.KH);
    } else {       // OIHW [co][c][kh][kw]
        kw = static_cast<int>(e % g.KW); e /= g.KW;
        kh = static_cast<int>(e % g.KH); e /= g.KH;
        c = static_cast<int>(e % g.Cg); co = static_cast<int>(e / g.Cg);
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dw_partial_kernel(
    const T* __restrict__ x, const T* __restrict__ dy, float* __restrict__ part, Geom g,
    int64_t wn, int64_t per)
{
    const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (e >= wn) return;
    const int s = blockIdx.y;
    int co, c, kh, kw;
    weight_coords(g, e, co, c, kh, kw);
    const int ci = (co / g.Mg) * g.Cg + c;
    const int64_t M = static_cast<int64_t>(g.N) * g.OH * g.OW;
    const int64_t m0 = s * per, m1 = min(M, m0 + per);
    float acc = 0.f;
    for (int64_t m = m0; m < m1; ++m) {
        const int ow = static_cast<int>(m % g.OW);
        const int64_t r = m / g.OW;
        const int oh = static_cast<int>(r % g.OH);
        const int n = static_cast<int>(r / g.OH);
        const int ih = oh * g.sh - g.ph + kh * g.dh;
        const int iw = ow * g.sw - g.pw + kw * g.dw;
        if (static_cast<unsigned>(ih) >= static_cast<unsigned>(g.H) ||
            static_cast<unsigned>(iw) >= static_cast<unsigned>(g.W))
            continue;
        const int64_t xo = g.nhwc ? ((static_cast<int64_t>(n) * g.H + ih) * g.W + iw) * g.C + ci
                                  : ((static_cast<int64_t>(n) * g.C + ci) * g.H + ih) * g.W + iw;
        const int64_t yo = g.nhwc ? m * g.CO + co
                                  : ((static_cast<int64_t>(n) * g.CO + co) * g.OH + oh) * g.OW + ow;
        acc = fmaf(load_f(dy + yo), load_f(x + xo), acc);
    }
    part[static_cast<int64_t>(s) * wn + e] = acc;
}

// Pass 2 (shared with the MFMA path): dw[e] = sum over s of part[s][e], in
// piece order, rounded once.
template <typename T>
__global__ __launch_bounds__(kThreads) void dw_reduce_kernel(const float* __restrict__ part,
                                                             T* __restrict__ dw, int64_t wn,
                                                             int pieces)
{
    const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (e >= wn) return;
    float acc = 0.f;
    for (int s = 0; s < pieces; ++s) acc += part[static_cast<int64_t>(s) * wn + e];
    store_f(dw + e, acc);
}

}  // namespace

// Pieces of the generic path: enough (piece, element-block) pairs to fill
// the device twice over, no piece shorter than 64 pixels, at most 256.
DwPlan plan_dw_direct(const Geom& g)
{
    DwPlan p{};
    const int64_t wn = static_cast<int64_t>(g.CO) * g.Cg * g.KH * g.KW;
    const int64_t M = static_cast<int64_t>(g.N) * g.OH * g.OW;
    const int64_t eblocks = (wn + kThreads - 1) / kThreads;
    int64_t S = std::max<int64_t>(1, 2048 / eblocks);
    S = std::min<int64_t>({S, 256, std::max<int64_t>(1, M / 64)});
    p.per = (M + S - 1) / S;
    p.pieces = static_cast<int>((M + p.per - 1) / p.per);
    p.workspace = static_cast<size_t>(p.pieces) * static_cast<size_t>(wn) * sizeof(float);
    return p;
}

hipError_t launch_dw_reduce(const float* part, void* dw, int64_t wn, int pieces, int dtype,
                            hipStream_t s)
{
    const dim3 grid(static_cast<unsigned>((wn + kThreads - 1) / kThreads));
    if (dtype == 0)
        return launch(dw_reduce_kernel<float>, grid, dim3(kThreads), 0, s, part,
                      static_cast<float*>(dw), wn, pieces);
    return launch(dw_reduce_kernel<bf16_t>, grid, dim3(kThreads), 0, s, part,
                  static_cast<bf16_t*>(dw), wn, pieces);
}

hipError_t launch_dw_direct(const void* x, const void* dy, void* dw, void* workspace,
                            const Geom& g, int dtype, hipStream_t s)
{
    const DwPlan p = plan_dw_direct(g);
    const int64_t wn = static_cast<int64_t>(g.CO) * g.Cg * g.KH * g.KW;
    float* part = static_cast<float*>(workspace);
    const dim3 grid(static_cast<unsigned>((wn + kThreads - 1) / kThreads), p.pieces);
    // The start event (if armed) stamps the first pass, the stop event the
    // second, so that together they time the whole gradient.
    const ArmedEvents armed = armed_events();
    armed_events() = ArmedEvents{armed.start, nullptr};
    hipError_t e = dtype == 0
                       ? launch(dw_partial_kernel<float>, grid, dim3(kThreads), 0, s,
                                static_cast<const float*>(x), static_cast<const float*>(dy), part, g,
                                wn, p.per)
                       : launch(dw_partial_kernel<bf16_t>, grid, dim3(kThreads), 0, s,
                                static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(dy), part,
                                g, wn, p.per);
    armed_events() = ArmedEvents{nullptr, armed.stop};
    if (e != hipSuccess) {
        armed_events() = ArmedEvents{nullptr, nullptr};
        return e;
    }
    return launch_dw_reduce(part, dw, wn, p.pieces, dtype, s);
}

}  // namespace convmi
