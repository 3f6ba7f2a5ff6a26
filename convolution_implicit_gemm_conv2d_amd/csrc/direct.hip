// Generic direct kernels: forward convolution and input gradient for any
// geometry, layout (NCHW/OIHW or NHWC/OHWI) and dtype (fp32 or bf16).
//
// These serve every shape the specialised kernels decline.  One lane owns one
// output element and walks its taps, so each element is written exactly once
// and no atomics are needed.  Small problems, where this path is used most,
// are bound by the latency of that walk: when the tensors fit 32-bit byte
// offsets, the forward takes its taps in batches whose loads are all in
// flight at once.
//
// Forward: the per-output loop of teeny-kernels 0.2.0 src/nn/conv/conv2d.rs,
// `conv2d_forward` (tap row oh*stride - pad + kh, group window
// [g*C/G, (g+1)*C/G), zero padding by bounds check), with dilation as in the
// burn-cubecl 0.22.0-pre.4 src/kernel/conv/im2col.rs `im2col` column formula,
// and the fused bias of `conv2d_bias_forward`.
//
// Input gradient: a gather over the taps that read each input element, the
// dispatch-per-input-element form of oarust 0.8.6 src/rs/ml/matrix/conv.rs
// `conv_2d_backward`, instead of the atomic scatter of teeny-kernels'
// `conv2d_backward_dx`.  The same sum is the transposed convolution of the
// oarust page (`conv_transpose_2d`), whose per-channel bias the kernel adds
// when one is given.
#include "kernels.hpp"

namespace convmi {
namespace {

constexpr int kThreads = 256;

template <typename T, int NHWC>
__global__ __launch_bounds__(kThreads) void fwd_direct_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, Geom g, int64_t total)
{
    const int64_t step = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t o = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; o < total;
         o += step) {
        int64_t r = o;
        int n, co, oh, ow;
        if (NHWC) {
            co = static_cast<int>(r % g.CO); r /= g.CO;
            ow = static_cast<int>(r % g.OW); r /= g.OW;
            oh = static_cast<int>(r % g.OH); n = static_cast<int>(r / g.OH);
        } else {
            ow = static_cast<int>(r % g.OW); r /= g.OW;
            oh = static_cast<int>(r % g.OH); r /= g.OH;
            co = static_cast<int>(r % g.CO); n = static_cast<int>(r / g.CO);
        }
        const int c0 = (co / g.Mg) * g.Cg;
        const int ih0 = oh * g.sh - g.ph;
        const int iw0 = ow * g.sw - g.pw;
        float acc = 0.f;
        for (int kh = 0; kh < g.KH; ++kh) {
            const int ih = ih0 + kh * g.dh;
            if (static_cast<unsigned>(ih) >= static_cast<unsigned>(g.H)) continue;
            for (int kw = 0; kw < g.KW; ++kw) {
                const int iw = iw0 + kw * g.dw;
                if (static_cast<unsigned>(iw) >= static_cast<unsigned>(g.W)) continue;
                if (NHWC) {
                    const T* xp = x + ((static_cast<int64_t>(n) * g.H + ih) * g.W + iw) * g.C + c0;
                    const T* wp = w + ((static_cast<int64_t>(co) * g.KH + kh) * g.KW + kw) * g.Cg;
                    for (int c = 0; c < g.Cg; ++c) acc = fmaf(load_f(xp + c), load_f(wp + c), acc);
                } else {
                    const int64_t plane = static_cast<int64_t>(g.H) * g.W;
                    const T* xp = x + (static_cast<int64_t>(n) * g.C + c0) * plane +
                                  static_cast<int64_t>(ih) * g.W + iw;
                    const T* wp = w + (static_cast<int64_t>(co) * g.Cg * g.KH + kh) * g.KW + kw;
                    const int wstep = g.KH * g.KW;
                    for (int c = 0; c < g.Cg; ++c)
                        acc = fmaf(load_f(xp + c * plane), load_f(wp + c * wstep), acc);
                }
            }
        }
        if (bias) acc += load_f(bias + co);
        store_f(y + o, acc);
    }
}

template <typename T, int NHWC>
__global__ __launch_bounds__(kThreads) void dx_gather_kernel(
    const T* __restrict__ dy, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ dx, Geom g, int64_t total)
{
    const int64_t step = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t o = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; o < total;
         o += step) {
        int64_t r = o;
        int n, ci, ih, iw;
        if (NHWC) {
            ci = static_cast<int>(r % g.C); r /= g.C;
            iw = static_cast<int>(r % g.W); r /= g.W;
            ih = static_cast<int>(r % g.H); n = static_cast<int>(r / g.H);
        } else {
            iw = static_cast<int>(r % g.W); r /= g.W;
            ih = static_cast<int>(r % g.H); r /= g.H;
            ci = static_cast<int>(r % g.C); n = static_cast<int>(r / g.C);
        }
        const int grp = ci / g.Cg;
        const int c = ci - grp * g.Cg;
        const int co0 = grp * g.Mg;
        float acc = 0.f;
        for (int kh = 0; kh < g.KH; ++kh) {
            const int th = ih + g.ph - kh * g.dh;
            if (th < 0 || th % g.sh) continue;
            const int oh = th / g.sh;
            if (oh >= g.OH) continue;
            for (int kw = 0; kw < g.KW; ++kw) {
                const int tw = iw + g.pw - kw * g.dw;
                if (tw < 0 || tw % g.sw) continue;
                const int ow = tw / g.sw;
                if (ow >= g.OW) continue;
                if (NHWC) {
                    const T* dp = dy + ((static_cast<int64_t>(n) * g.OH + oh) * g.OW + ow) * g.CO + co0;
                    const T* wp = w + ((static_cast<int64_t>(co0) * g.KH + kh) * g.KW + kw) * g.Cg + c;
                    const int64_t wstep = static_cast<int64_t>(g.KH) * g.KW * g.Cg;
                    for (int m = 0; m < g.Mg; ++m)
                        acc = fmaf(load_f(dp + m), load_f(wp + m * wstep), acc);
                } else {
                    const int64_t plane = static_cast<int64_t>(g.OH) * g.OW;
                    const T* dp = dy + (static_cast<int64_t>(n) * g.CO + co0) * plane +
                                  static_cast<int64_t>(oh) * g.OW + ow;
                    const T* wp = w + ((static_cast<int64_t>(co0) * g.Cg + c) * g.KH + kh) * g.KW + kw;
                    const int64_t wstep = static_cast<int64_t>(g.Cg) * g.KH * g.KW;
                    for (int m = 0; m < g.Mg; ++m)
                        acc = fmaf(load_f(dp + m * plane), load_f(wp + m * wstep), acc);
                }
            }
        }
        if (bias) acc += load_f(bias + ci);
        store_f(dx + o, acc);
    }
}

// Loads of one element through a buffer resource (zero at kOutside).
__device__ __forceinline__ float buffer_load_elem(rsrc_t r, uint32_t off, float*)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ float buffer_load_elem(rsrc_t r, uint32_t off, bf16_t*)
{
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
}

// The forward for tensors below 2 GiB, one output per lane.  The taps
// (c, kh, kw) are walked in the weight's storage order -- kw fastest for
// OIHW, c fastest for OHWI -- so the weight offset of tap r is co K + r.  A
// batch of kBatch taps first forms all its byte offsets (a tap outside the
// image, or past the last, becomes kOutside, which the buffer loads read as
// zero), then issues its loads together: one memory round trip per batch
// instead of one per tap.
constexpr int kBatch = 32;
template <typename T, int NHWC>
__global__ __launch_bounds__(kThreads) void fwd_direct_batched_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, Geom g, int total, uint32_t x_bytes, uint32_t w_bytes)
{
    const rsrc_t xr = make_rsrc(x, x_bytes);
    const rsrc_t wr = make_rsrc(w, w_bytes);
    constexpr uint32_t kElem = sizeof(T);
    const int K = g.Cg * g.KH * g.KW;
    const int step = gridDim.x * kThreads;
    for (int o = blockIdx.x * kThreads + threadIdx.x; o < total; o += step) {
        int r = o;
        int n, co, oh, ow;
        if (NHWC) {
            co = r % g.CO; r /= g.CO;
            ow = r % g.OW; r /= g.OW;
            oh = r % g.OH; n = r / g.OH;
        } else {
            ow = r % g.OW; r /= g.OW;
            oh = r % g.OH; r /= g.OH;
            co = r % g.CO; n = r / g.CO;
        }
        const int c0 = (co / g.Mg) * g.Cg;
        const int ih0 = oh * g.sh - g.ph;
        const int iw0 = ow * g.sw - g.pw;
        // Element offset of (n, c0) at input pixel (0, 0).
        const uint32_t xbase = NHWC ? static_cast<uint32_t>(n) * g.H * g.W * g.C + c0
                                    : (static_cast<uint32_t>(n) * g.C + c0) * g.H * g.W;
        const uint32_t plane = static_cast<uint32_t>(g.H) * g.W;
        const uint32_t wbase = static_cast<uint32_t>(co) * K;
        int c = 0, kh = 0, kw = 0;
        float acc = 0.f;
        for (int r0 = 0; r0 < K; r0 += kBatch) {
            uint32_t xo[kBatch], wo[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const bool live = r0 + j < K;
                const int ih = ih0 + kh * g.dh, iw = iw0 + kw * g.dw;
                const bool in = live && static_cast<unsigned>(ih) < static_cast<unsigned>(g.H) &&
                                static_cast<unsigned>(iw) < static_cast<unsigned>(g.W);
                const uint32_t pix = static_cast<uint32_t>(ih) * g.W + static_cast<uint32_t>(iw);
                const uint32_t xe = NHWC ? xbase + pix * g.C + c : xbase + c * plane + pix;
                xo[j] = in ? xe * kElem : kOutside;
                wo[j] = live ? (wbase + r0 + j) * kElem : kOutside;
                if (NHWC) {
                    const bool wc = ++c == g.Cg;
                    c = wc ? 0 : c;
                    kw += wc;
                    const bool ww = kw == g.KW;
                    kw = ww ? 0 : kw;
                    kh += ww;
                } else {
                    const bool ww = ++kw == g.KW;
                    kw = ww ? 0 : kw;
                    kh += ww;
                    const bool wh = kh == g.KH;
                    kh = wh ? 0 : kh;
                    c += wh;
                }
            }
            float xv[kBatch], wv[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                xv[j] = buffer_load_elem(xr, xo[j], static_cast<T*>(nullptr));
                wv[j] = buffer_load_elem(wr, wo[j], static_cast<T*>(nullptr));
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) acc = fmaf(xv[j], wv[j], acc);
        }
        if (bias) acc += load_f(bias + co);
        store_f(y + o, acc);
    }
}

int grid_for(int64_t total) {
    int64_t blocks = (total + kThreads - 1) / kThreads;
    const int64_t cap = 1 << 20;  // grid-stride beyond this
    return static_cast<int>(blocks < cap ? blocks : cap);
}

template <typename T>
hipError_t fwd_t(const void* x, const void* w, const void* b, void* y, const Geom& g,
                 hipStream_t s)
{
    const int64_t total = static_cast<int64_t>(g.N) * g.CO * g.OH * g.OW;
    const T* xb = static_cast<const T*>(x);
    const T* wb = static_cast<const T*>(w);
    const T* bb = static_cast<const T*>(b);
    T* yb = static_cast<T*>(y);
    const int64_t x_bytes = static_cast<int64_t>(g.N) * g.C * g.H * g.W * sizeof(T);
    const int64_t w_bytes = static_cast<int64_t>(g.CO) * g.Cg * g.KH * g.KW * sizeof(T);
    constexpr int64_t kLimit = int64_t(1) << 31;
    if (total < kLimit && x_bytes < kLimit && w_bytes < kLimit)
        return launch(g.nhwc ? fwd_direct_batched_kernel<T, 1> : fwd_direct_batched_kernel<T, 0>,
                      dim3(grid_for(total)), dim3(kThreads), 0, s, xb, wb, bb, yb, g,
                      static_cast<int>(total), static_cast<uint32_t>(x_bytes), static_cast<uint32_t>(w_bytes));
    return launch(g.nhwc ? fwd_direct_kernel<T, 1> : fwd_direct_kernel<T, 0>,
                  dim3(grid_for(total)), dim3(kThreads), 0, s, xb, wb, bb, yb, g, total);
}

template <typename T>
hipError_t dx_t(const void* dy, const void* w, const void* bias, void* dx, const Geom& g,
                hipStream_t s)
{
    const int64_t total = static_cast<int64_t>(g.N) * g.C * g.H * g.W;
    const T* db = static_cast<const T*>(dy);
    const T* wb = static_cast<const T*>(w);
    const T* bb = static_cast<const T*>(bias);
    T* xb = static_cast<T*>(dx);
    return launch(g.nhwc ? dx_gather_kernel<T, 1> : dx_gather_kernel<T, 0>,
                  dim3(grid_for(total)), dim3(kThreads), 0, s, db, wb, bb, xb, g, total);
}

}  // namespace

hipError_t launch_fwd_direct(const void* x, const void* w, const void* bias, void* y,
                             const Geom& g, int dtype, hipStream_t s)
{
    return dtype == 0 ? fwd_t<float>(x, w, bias, y, g, s) : fwd_t<bf16_t>(x, w, bias, y, g, s);
}

hipError_t launch_dx_gather(const void* dy, const void* w, const void* bias, void* dx,
                            const Geom& g, int dtype, hipStream_t s)
{
    return dtype == 0 ? dx_t<float>(dy, w, bias, dx, g, s) : dx_t<bf16_t>(dy, w, bias, dx, g, s);
}

}  // namespace convmi
