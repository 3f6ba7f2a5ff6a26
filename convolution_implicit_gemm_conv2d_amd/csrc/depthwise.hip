// Depthwise forward convolution (one input channel per group): a direct,
// HBM-bound kernel.
//
// With C/G = 1 each output is a per-channel 2-D cross-correlation,
// y[n, oh, ow, c] = bias[c] + sum_{kh, kw} x[n, oh*sh - ph + kh*dh,
// ow*sw - pw + kw*dw, c] * w[c, kh, kw], so there is no cross-channel
// contraction for a matrix unit to exploit (the grouped case of teeny-kernels
// 0.2.0 src/nn/conv/conv2d.rs, `conv2d_forward`, with G = C).
//
// MI355X design: in NHWC the channels of one pixel are contiguous, so a lane
// owns 16 bytes of channels (8 bf16 or 4 fp32) and a wavefront covers
// 64 x 16 = 1 KB of contiguous channels per load.  A lane computes a strip of
// RH output rows at one output column.  For unit stride and a compile-time
// kernel/dilation the strip walks the input rows it needs once, loading each
// (row, kernel column) vector once and feeding every output row of the strip
// that uses it from registers, which cuts cache traffic from KH*KW to about
// KW*(RH + (KH-1)*dh)/RH loads per output.  Other shapes take a generic strip
// kernel that loads per tap.  Accumulation is fp32, the bias is added in fp32
// and each output is rounded once.
#include "kernels.hpp"

namespace convmi {
namespace {

constexpr int kThreads = 256;
constexpr int kRH = 8;  // output rows per lane

template <typename T>
struct Vec;
template <>
struct Vec<bf16_t> {
    static constexpr int N = 8;
    __device__ static void unpack(const uint4& v, float* f)
    {
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    __device__ static uint4 pack(const float* f)
    {
        return uint4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7])};
    }
};
template <>
struct Vec<float> {
    static constexpr int N = 4;
    __device__ static void unpack(const uint4& v, float* f)
    {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    __device__ static uint4 pack(const float* f)
    {
        return uint4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                     __float_as_uint(f[3])};
    }
};

// Lane -> (channel vector cg, output column ow, first output row oh0, image n).
struct Slot {
    int cg, ow, oh0, n;
    bool live;
};
__device__ __forceinline__ Slot slot_of(const Geom& g, int cgroups, int ohtiles)
{
    Slot s;
    const int f = blockIdx.x * kThreads + threadIdx.x;
    s.live = f < g.OW * cgroups;
    s.cg = f % cgroups;
    s.ow = f / cgroups;
    s.n = blockIdx.y / ohtiles;
    s.oh0 = (blockIdx.y - s.n * ohtiles) * kRH;
    return s;
}

template <typename T>
__device__ __forceinline__ void store_strip(const Geom& g, const Slot& s, const T* bias,
                                            T* y, float (*acc)[Vec<T>::N])
{
    constexpr int V = Vec<T>::N;
    const int c0 = s.cg * V;
    float b[V];
#pragma unroll
    for (int e = 0; e < V; ++e) b[e] = bias ? load_f(bias + c0 + e) : 0.f;
#pragma unroll
    for (int j = 0; j < kRH; ++j) {
        const int oh = s.oh0 + j;
        if (oh >= g.OH) break;
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = acc[j][e] + b[e];
        T* yp = y + ((static_cast<int64_t>(s.n) * g.OH + oh) * g.OW + s.ow) * g.C + c0;
        *reinterpret_cast<uint4*>(yp) = Vec<T>::pack(o);
    }
}

// Unit stride, compile-time kernel extent and dilation: each needed input
// row is read once per kernel column.
template <typename T, int KH, int KW, int DH, int DW>
__global__ __launch_bounds__(kThreads) void depthwise_rows_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, Geom g, int cgroups, int ohtiles)
{
    constexpr int V = Vec<T>::N;
    constexpr int ROWS = kRH + (KH - 1) * DH;
    const Slot s = slot_of(g, cgroups, ohtiles);
    if (!s.live) return;
    const int c0 = s.cg * V;

    float wt[KH * KW][V];
#pragma unroll
    for (int e = 0; e < V; ++e)
#pragma unroll
        for (int t = 0; t < KH * KW; ++t)
            wt[t][e] = load_f(w + static_cast<int64_t>(c0 + e) * (KH * KW) + t);

    float acc[kRH][V];
#pragma unroll
    for (int j = 0; j < kRH; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[j][e] = 0.f;

    const T* ximg = x + static_cast<int64_t>(s.n) * g.H * g.W * g.C + c0;
    const int iw0 = s.ow - g.pw;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int ih = s.oh0 - g.ph + i;
        if (static_cast<unsigned>(ih) >= static_cast<unsigned>(g.H)) continue;
        const T* xrow = ximg + static_cast<int64_t>(ih) * g.W * g.C;
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) {
            const int iw = iw0 + kw * DW;
            if (static_cast<unsigned>(iw) >= static_cast<unsigned>(g.W)) continue;
            float xv[V];
            Vec<T>::unpack(*reinterpret_cast<const uint4*>(xrow + static_cast<int64_t>(iw) * g.C), xv);
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int j = i - kh * DH;  // output row of the strip fed by this tap
                if (j < 0 || j >= kRH) continue;
#pragma unroll
                for (int e = 0; e < V; ++e) acc[j][e] = fmaf(xv[e], wt[kh * KW + kw][e], acc[j][e]);
            }
        }
    }
    store_strip<T>(g, s, bias, y, acc);
}

// Any stride, kernel extent and dilation: per-tap loads.
template <typename T>
__global__ __launch_bounds__(kThreads) void depthwise_generic_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, Geom g, int cgroups, int ohtiles)
{
    constexpr int V = Vec<T>::N;
    const Slot s = slot_of(g, cgroups, ohtiles);
    if (!s.live) return;
    const int c0 = s.cg * V;
    const int taps = g.KH * g.KW;
    float acc[kRH][V];
#pragma unroll
    for (int j = 0; j < kRH; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[j][e] = 0.f;
    const T* ximg = x + static_cast<int64_t>(s.n) * g.H * g.W * g.C + c0;
    for (int kh = 0; kh < g.KH; ++kh) {
        for (int kw = 0; kw < g.KW; ++kw) {
            const int iw = s.ow * g.sw - g.pw + kw * g.dw;
            if (static_cast<unsigned>(iw) >= static_cast<unsigned>(g.W)) continue;
            float wv[V];
#pragma unroll
            for (int e = 0; e < V; ++e)
                wv[e] = load_f(w + static_cast<int64_t>(c0 + e) * taps + kh * g.KW + kw);
#pragma unroll
            for (int j = 0; j < kRH; ++j) {
                const int ih = (s.oh0 + j) * g.sh - g.ph + kh * g.dh;
                if (s.oh0 + j >= g.OH || static_cast<unsigned>(ih) >= static_cast<unsigned>(g.H))
                    continue;
                float xv[V];
                Vec<T>::unpack(*reinterpret_cast<const uint4*>(
                                   ximg + (static_cast<int64_t>(ih) * g.W + iw) * g.C), xv);
#pragma unroll
                for (int e = 0; e < V; ++e) acc[j][e] = fmaf(xv[e], wv[e], acc[j][e]);
            }
        }
    }
    store_strip<T>(g, s, bias, y, acc);
}

template <typename T>
hipError_t launch_t(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                    hipStream_t s)
{
    constexpr int V = Vec<T>::N;
    const int cgroups = g.C / V;
    const int ohtiles = (g.OH + kRH - 1) / kRH;
    const dim3 grid((g.OW * cgroups + kThreads - 1) / kThreads, g.N * ohtiles);
    const T* xb = static_cast<const T*>(x);
    const T* wb = static_cast<const T*>(w);
    const T* bb = static_cast<const T*>(bias);
    T* yb = static_cast<T*>(y);
    const bool unit = g.sh == 1 && g.sw == 1;
    if (unit && g.KH == 3 && g.KW == 3 && g.dh == 1 && g.dw == 1)
        return launch(depthwise_rows_kernel<T, 3, 3, 1, 1>, grid, dim3(kThreads), 0, s, xb, wb, bb,
                      yb, g, cgroups, ohtiles);
    if (unit && g.KH == 3 && g.KW == 3 && g.dh == 2 && g.dw == 2)
        return launch(depthwise_rows_kernel<T, 3, 3, 2, 2>, grid, dim3(kThreads), 0, s, xb, wb, bb,
                      yb, g, cgroups, ohtiles);
    if (unit && g.KH == 5 && g.KW == 5 && g.dh == 1 && g.dw == 1)
        return launch(depthwise_rows_kernel<T, 5, 5, 1, 1>, grid, dim3(kThreads), 0, s, xb, wb, bb,
                      yb, g, cgroups, ohtiles);
    return launch(depthwise_generic_kernel<T>, grid, dim3(kThreads), 0, s, xb, wb, bb, yb, g,
                  cgroups, ohtiles);
}

}  // namespace

bool can_depthwise(const Geom& g, int dtype)
{
    const int vec = dtype == 1 ? 8 : 4;
    return g.nhwc && g.aligned16 && g.Cg == 1 && g.Mg == 1 && g.C % vec == 0 &&
           static_cast<int64_t>(g.OW) * (g.C / vec) < (int64_t(1) << 31) - kThreads &&
           static_cast<int64_t>(g.N) * ((g.OH + kRH - 1) / kRH) < 65536;
}

hipError_t launch_depthwise(const void* x, const void* w, const void* bias, void* y,
                            const Geom& g, int dtype, hipStream_t s)
{
    return dtype == 1 ? launch_t<bf16_t>(x, w, bias, y, g, s) : launch_t<float>(x, w, bias, y, g, s);
}

}  // namespace convmi
