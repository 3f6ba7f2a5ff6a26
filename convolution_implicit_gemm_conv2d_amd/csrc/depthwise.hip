// Depthwise forward convolution (one input channel per group): a direct,
// HBM-bound kernel.
//
// With C/G = 1 each output is a per-channel 2-D cross-correlation,
// y[n, oh, ow, c] = bias[c] + sum_{kh, kw} x[n, oh*sh - ph + kh*dh,
// ow*sw - pw + kw*dw, c] * w[c, kh, kw], so there is no cross-channel
// contraction for a matrix unit to exploit (the grouped case of teeny-kernels
// 0.2.0 src/nn/conv/conv2d.rs, `conv2d_forward`, with G = C).
//
// MI355X design.  In NHWC the channels of one pixel are contiguous, so a lane
// owns 16 bytes of channels (8 bf16 or 4 fp32) and a wavefront covers
// 64 x 16 = 1 KB of contiguous memory per load.
//
// Unit stride with a compile-time kernel and dilation takes the streaming
// kernel: a lane walks down one output column over a segment of rows.  Each
// input row it needs is loaded once per kernel column, several rows ahead of
// use (a register ring), and feeds every output row that reads it; finished
// output rows are stored as the walk passes them.  Input and accumulator rings
// are indexed by compile-time slots (the loop is unrolled by the ring length),
// padding rows and columns load as zero through buffer-resource bounds, so the
// loop has no data-dependent branches.  Workgroups are numbered so that every
// XCD receives a contiguous run of whole images: the halo rows and columns
// that neighbouring workgroups share are then served by the same L2.
//
// Other shapes take a generic strip kernel that loads per tap.  Accumulation
// is fp32, the bias is added in fp32 and each output is rounded once.
#include "kernels.hpp"

#include <algorithm>

namespace convmi {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin over 8 XCDs

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

// Work decomposition shared by both kernels.  Workgroup b covers kThreads
// consecutive (column, channel-vector) slots of one (image, row segment);
// segments are `seg_rows` output rows tall.  The launch order is remapped so
// that XCD k (which receives workgroups k, k+8, ...) gets a contiguous block
// of logical workgroups when the count divides evenly.
struct Slot {
    int cg, ow, n, oh_begin, oh_end;
    bool live;
};
__device__ __forceinline__ Slot slot_of(const Geom& g, int cgroups, int col_blocks, int segs,
                                        int seg_rows)
{
    const int nb = gridDim.x;
    int b = blockIdx.x;
    if (nb % kXcds == 0) b = (b % kXcds) * (nb / kXcds) + b / kXcds;
    const int colb = b % col_blocks;
    const int rest = b / col_blocks;
    const int seg = rest % segs;
    Slot s;
    s.n = rest / segs;
    const int f = colb * kThreads + threadIdx.x;
    s.live = f < g.OW * cgroups;
    s.cg = f % cgroups;
    s.ow = f / cgroups;
    s.oh_begin = seg * seg_rows;
    s.oh_end = min(g.OH, s.oh_begin + seg_rows);
    return s;
}

// Loads the lane's per-channel weights.  With C/G = 1 the V channels of a
// lane keep their taps back to back (w[c][kh][kw]): TAPS 16-byte vectors.
template <typename T, int TAPS>
__device__ __forceinline__ void load_weights(const T* w, int c0, float (&wt)[TAPS][Vec<T>::N])
{
    constexpr int V = Vec<T>::N;
    const uint4* wv = reinterpret_cast<const uint4*>(w + static_cast<int64_t>(c0) * TAPS);
    float flat[TAPS * V];
#pragma unroll
    for (int i = 0; i < TAPS; ++i) Vec<T>::unpack(wv[i], flat + i * V);
#pragma unroll
    for (int e = 0; e < V; ++e)
#pragma unroll
        for (int t = 0; t < TAPS; ++t) wt[t][e] = flat[e * TAPS + t];
}

// The lane's V bias values as one vector load; a null bias is a resource of
// zero bytes, whose loads return zero.
template <typename T>
__device__ __forceinline__ void load_bias(const T* bias, int C, int c0, float (&b)[Vec<T>::N])
{
    const rsrc_t br = make_rsrc(bias, bias ? static_cast<uint32_t>(C) * sizeof(T) : 0u);
    Vec<T>::unpack(buffer_load16(br, static_cast<uint32_t>(c0) * sizeof(T)), b);
}

// Unit stride, compile-time kernel and dilation: the streaming walk.
//   L  = (KH-1)*DH + 1 output rows are live at once (accumulator ring);
//   RS = input ring length (a multiple of L), prefetch depth RS - 1 rows.
template <typename T, int KH, int KW, int DH, int DW>
__global__ __launch_bounds__(kThreads) void depthwise_stream_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, Geom g, int cgroups, int col_blocks, int segs, int seg_rows)
{
    constexpr int V = Vec<T>::N;
    constexpr int L = (KH - 1) * DH + 1;
    constexpr int RS = L >= 5 ? L : 2 * L;
    constexpr int PF = RS - 1;
    const Slot s = slot_of(g, cgroups, col_blocks, segs, seg_rows);
    if (!s.live) return;
    const int c0 = s.cg * V;

    float wt[KH * KW][V];
    load_weights<T, KH * KW>(w, c0, wt);
    float b[V];
    load_bias<T>(bias, g.C, c0, b);

    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * sizeof(T);
    const uint32_t row_bytes = static_cast<uint32_t>(g.W) * pix_bytes;
    const rsrc_t xr =
        make_rsrc(x + static_cast<int64_t>(s.n) * g.H * g.W * g.C, row_bytes * static_cast<uint32_t>(g.H));
    uint32_t col_off[KW];
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) {
        const int iw = s.ow - g.pw + kw * DW;
        col_off[kw] = static_cast<unsigned>(iw) < static_cast<unsigned>(g.W)
                          ? static_cast<uint32_t>(iw) * pix_bytes + static_cast<uint32_t>(c0) * sizeof(T)
                          : kOutside;
    }
    // Input row i of the walk is image row r_start + i.
    const int count = s.oh_end - s.oh_begin;
    const int nrows = count + L - 1;
    const int r_start = s.oh_begin - g.ph;
    auto load_row = [&](int i, uint4 (&dst)[KW]) {
        const int r = r_start + i;
        const bool in = static_cast<unsigned>(r) < static_cast<unsigned>(g.H) && i < nrows;
        const uint32_t roff = static_cast<uint32_t>(r) * row_bytes;
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
            dst[kw] = buffer_load16(xr, (in && col_off[kw] != kOutside) ? roff + col_off[kw] : kOutside);
    };

    uint4 ring[RS][KW];
#pragma unroll
    for (int u = 0; u < PF; ++u) load_row(u, ring[u]);
    float acc[L][V];
#pragma unroll
    for (int j = 0; j < L; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[j][e] = 0.f;

    // Output through a buffer resource over this image: a store for an
    // output row outside the segment gets an offset past the end and is
    // dropped, so the walk needs no branches.
    const uint32_t yrow_bytes = static_cast<uint32_t>(g.OW) * pix_bytes;
    const rsrc_t yr = make_rsrc(y + static_cast<int64_t>(s.n) * g.OH * g.OW * g.C,
                                yrow_bytes * static_cast<uint32_t>(g.OH));
    const uint32_t ycol_off = static_cast<uint32_t>(s.ow) * pix_bytes + static_cast<uint32_t>(c0) * sizeof(T);

    // The walk runs in whole ring periods; rows past nrows load as zero and
    // their stores are dropped.
    for (int it = 0; it < nrows; it += RS) {
#pragma unroll
        for (int u = 0; u < RS; ++u) {
            const int i = it + u;
            load_row(i + PF, ring[(u + PF) % RS]);  // prefetch into the slot just consumed
            float xv[KW][V];
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) Vec<T>::unpack(ring[u][kw], xv[kw]);
            // Row i feeds output j = i - kh*DH of the segment through tap kh;
            // slot (j mod L) is compile-time since `it` is a multiple of L.
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int slot = ((u - kh * DH) % L + L) % L;
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        acc[slot][e] = fmaf(xv[kw][e], wt[kh * KW + kw][e], acc[slot][e]);
            }
            // Output j = i - (L-1) has now received every tap.
            const int jd = i - (L - 1);
            const int sd = (u + 1) % L;
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = acc[sd][e] + b[e];
            const bool keep = jd >= 0 && jd < count;
            buffer_store16(yr, keep ? static_cast<uint32_t>(s.oh_begin + jd) * yrow_bytes + ycol_off : kOutside,
                           Vec<T>::pack(o));
#pragma unroll
            for (int e = 0; e < V; ++e) acc[sd][e] = 0.f;
        }
    }
}

// Any stride, kernel extent and dilation: a strip of kRH rows, per-tap loads.
constexpr int kRH = 8;
template <typename T>
__global__ __launch_bounds__(kThreads) void depthwise_generic_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, Geom g, int cgroups, int col_blocks, int segs, int seg_rows)
{
    constexpr int V = Vec<T>::N;
    const Slot s = slot_of(g, cgroups, col_blocks, segs, seg_rows);
    if (!s.live) return;
    const int c0 = s.cg * V;
    const int taps = g.KH * g.KW;
    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * sizeof(T);
    const rsrc_t xr = make_rsrc(x + static_cast<int64_t>(s.n) * g.H * g.W * g.C,
                                static_cast<uint32_t>(g.H) * g.W * pix_bytes);
    const uint32_t lane_off = static_cast<uint32_t>(c0) * sizeof(T);
    float b[V];
    load_bias<T>(bias, g.C, c0, b);
    for (int oh0 = s.oh_begin; oh0 < s.oh_end; oh0 += kRH) {
        float acc[kRH][V];
#pragma unroll
        for (int j = 0; j < kRH; ++j)
#pragma unroll
            for (int e = 0; e < V; ++e) acc[j][e] = 0.f;
        for (int kh = 0; kh < g.KH; ++kh) {
            for (int kw = 0; kw < g.KW; ++kw) {
                const int iw = s.ow * g.sw - g.pw + kw * g.dw;
                const bool col_in = static_cast<unsigned>(iw) < static_cast<unsigned>(g.W);
                float wv[V];
#pragma unroll
                for (int e = 0; e < V; ++e)
                    wv[e] = load_f(w + static_cast<int64_t>(c0 + e) * taps + kh * g.KW + kw);
#pragma unroll
                for (int j = 0; j < kRH; ++j) {
                    const int ih = (oh0 + j) * g.sh - g.ph + kh * g.dh;
                    const bool in = col_in && static_cast<unsigned>(ih) < static_cast<unsigned>(g.H);
                    const uint32_t off =
                        in ? (static_cast<uint32_t>(ih) * g.W + iw) * pix_bytes + lane_off : kOutside;
                    float xv[V];
                    Vec<T>::unpack(buffer_load16(xr, off), xv);
#pragma unroll
                    for (int e = 0; e < V; ++e) acc[j][e] = fmaf(xv[e], wv[e], acc[j][e]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kRH; ++j) {
            const int oh = oh0 + j;
            if (oh >= s.oh_end) break;
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = acc[j][e] + b[e];
            T* yp = y + ((static_cast<int64_t>(s.n) * g.OH + oh) * g.OW + s.ow) * g.C + c0;
            *reinterpret_cast<uint4*>(yp) = Vec<T>::pack(o);
        }
    }
}

template <typename T>
hipError_t launch_t(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                    hipStream_t s)
{
    constexpr int V = Vec<T>::N;
    const int cgroups = g.C / V;
    const int col_blocks = (g.OW * cgroups + kThreads - 1) / kThreads;
    // Row segments: up to about eight waves per CU on 256 CUs (all resident
    // at once), but segments no shorter than eight rows (each segment
    // re-reads its halo).
    const int64_t waves_per_seg = static_cast<int64_t>(g.N) * col_blocks * (kThreads / 64);
    int segs = static_cast<int>(2048 / waves_per_seg);
    segs = max(1, min(segs, g.OH / 8));
    const int seg_rows = (g.OH + segs - 1) / segs;
    segs = (g.OH + seg_rows - 1) / seg_rows;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(g.N) * segs * col_blocks));
    const T* xb = static_cast<const T*>(x);
    const T* wb = static_cast<const T*>(w);
    const T* bb = static_cast<const T*>(bias);
    T* yb = static_cast<T*>(y);
    const bool unit = g.sh == 1 && g.sw == 1;
    auto go = [&](auto kernel) {
        return launch(kernel, grid, dim3(kThreads), 0, s, xb, wb, bb, yb, g, cgroups, col_blocks,
                      segs, seg_rows);
    };
    if (unit && g.KH == 3 && g.KW == 3 && g.dh == 1 && g.dw == 1)
        return go(depthwise_stream_kernel<T, 3, 3, 1, 1>);
    if (unit && g.KH == 3 && g.KW == 3 && g.dh == 2 && g.dw == 2)
        return go(depthwise_stream_kernel<T, 3, 3, 2, 2>);
    if (unit && g.KH == 5 && g.KW == 5 && g.dh == 1 && g.dw == 1)
        return go(depthwise_stream_kernel<T, 5, 5, 1, 1>);
    return go(depthwise_generic_kernel<T>);
}

}  // namespace

bool can_depthwise(const Geom& g, int dtype)
{
    const int vec = dtype == 1 ? 8 : 4;
    const int64_t esz = dtype == 1 ? 2 : 4;
    const int64_t img_bytes = static_cast<int64_t>(std::max(g.H * g.W, g.OH * g.OW)) * g.C * esz;
    const int64_t col_blocks = (static_cast<int64_t>(g.OW) * (g.C / vec) + kThreads - 1) / kThreads;
    return g.nhwc && g.aligned16 && g.Cg == 1 && g.Mg == 1 && g.C % vec == 0 &&
           img_bytes < (int64_t(1) << 31) && col_blocks * g.N * g.OH < (int64_t(1) << 24);
}

hipError_t launch_depthwise(const void* x, const void* w, const void* bias, void* y,
                            const Geom& g, int dtype, hipStream_t s)
{
    return dtype == 1 ? launch_t<bf16_t>(x, w, bias, y, g, s) : launch_t<float>(x, w, bias, y, g, s);
}

}  // namespace convmi
