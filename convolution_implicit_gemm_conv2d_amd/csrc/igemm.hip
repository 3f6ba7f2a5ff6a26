// Dense forward convolution as an implicit GEMM on the MFMA units.
//
// Per group g the convolution is the matrix product
//   y[m, co] = bias[co] + sum_k A[m, k] * B[co, k],
//   m = (n, oh, ow),  k = (kh, kw, c),
//   A[m, k] = x[n, oh*sh - ph + kh*dh, ow*sw - pw + kw*dw, g*Cg + c] (0 outside),
//   B[co, k] = w[co, kh, kw, c]                           (OHWI, already K-major),
// i.e. the im2col column matrix of burn-cubecl 0.22.0-pre.4
// src/kernel/conv/im2col.rs (`im2col`: column o*stride + k*dilation - padding,
// zero where clipped, columns ordered (kernel..., channel)) times the weight,
// which that page materialises at one copy per tap.  Here the column matrix
// is never built: every A fragment is gathered from x on the fly, straight
// into MFMA operand registers.
//
// MI355X design.  A workgroup owns one 64-wide output-channel tile and keeps
// that tile's whole weight panel [64][K] resident in LDS (rows padded by 16
// bytes so the lanes of an MFMA operand read hit distinct banks).  Each of
// its four waves computes 32*PT pixels x 64 channels with
// v_mfma_f32_32x32x16_bf16, which keeps the matrix pipe near its peak rate
// with only a few independent accumulators (the 16x16x32 form needs many
// more).  Weights are the A operand (rows = channels), pixels the B operand,
// so every lane ends with runs of four consecutive output channels of one
// pixel for 8-byte stores.  One k-step is one kernel tap x 16 channels; a
// lane's pixel fragment is 8 channels = one 16-byte load through a buffer
// resource, so zero padding costs nothing (out-of-image taps use an offset
// past the end and read zero).  Fragments rotate through three register
// buffers so that two k-blocks are in flight while one runs on the MFMA
// units.  The bias is added in fp32 before the single rounding to bf16.
// Workgroups are persistent over pixel tiles, two per CU.
#include "kernels.hpp"

namespace convmi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBN = 64;             // output channels per workgroup (two 32-row MFMA tiles)
constexpr int kLdsBytes = 160 * 1024;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

struct IgemmArgs {
    const bf16_t* x;
    const bf16_t* w;
    const bf16_t* bias;
    bf16_t* y;
    Geom g;
    int64_t M;        // N*OH*OW pixels
    int K;            // KH*KW*Cg
    int co_tiles;     // ceil(Mg / 64) per group
    int px_tiles;     // ceil(M / (32*PT))
};

// v_mfma_f32_32x32x16_bf16 operand layout: lane l supplies row/column
// l % 32 and k-group l / 32 (8 consecutive k); the 16 results of lane l are
// column l % 32, rows 8*(v/4) + 4*(l/32) + v%4.
//
// PT: 32-pixel MFMA tiles per wave.  KB: 16-channel k-steps per k-block; a
// k-block is one kernel tap x KB*16 channels, and KB*16 divides Cg.
template <int PT, int KB>
__global__ __launch_bounds__(kThreads) void igemm_kernel(IgemmArgs a)
{
    extern __shared__ uint4 w_lds[];  // [64][K/8 + 1] 16-byte units
    const Geom& g = a.g;
    const int K = a.K;
    const int row16 = K / 8 + 1;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;  // MFMA row (weights) / column (pixels) of this lane
    const int q = lane >> 5;    // MFMA k-group: 8 consecutive channels of a 16-channel step

    const int grp_id = blockIdx.y / a.co_tiles;  // convolution group
    const int co_in_grp = (blockIdx.y - grp_id * a.co_tiles) * kBN;
    const int co0 = grp_id * g.Mg + co_in_grp;   // first output channel of the tile
    const int co_last = grp_id * g.Mg + g.Mg - 1;

    // Stage this tile's weight panel: 64 rows of K values.  Rows past the
    // group's last channel are clamped onto it; the MFMA rows they feed are
    // never stored.
    {
        const int units = kBN * (K / 8);
        for (int base = 0; base < units; base += 8 * kThreads) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = min(base + u * kThreads + tid, units - 1);
                const int r = i / (K / 8);
                v[u] = reinterpret_cast<const uint4*>(a.w + static_cast<int64_t>(min(co0 + r, co_last)) * K)[i - r * (K / 8)];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = min(base + u * kThreads + tid, units - 1);
                const int r = i / (K / 8);
                w_lds[r * row16 + (i - r * (K / 8))] = v[u];
            }
        }
    }
    __syncthreads();

    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * 2u;
    const rsrc_t xr = make_rsrc(a.x, static_cast<uint32_t>(g.N) * static_cast<uint32_t>(g.H * g.W) * pix_bytes);
    const rsrc_t yr = make_rsrc(a.y, static_cast<uint32_t>(a.M) * static_cast<uint32_t>(g.CO) * 2u);
    const rsrc_t br = make_rsrc(a.bias, a.bias ? static_cast<uint32_t>(g.CO) * 2u : 0u);
    const uint32_t lane_ch = static_cast<uint32_t>(grp_id * g.Cg + q * 8) * 2u;
    const int chunks = g.Cg / (16 * KB);
    const int kblocks = g.KH * g.KW * chunks;

    for (int tile = blockIdx.x * kWaves + wave; tile < a.px_tiles; tile += gridDim.x * kWaves) {
        const int64_t m0 = static_cast<int64_t>(tile) * (32 * PT);
        // Per pixel tile: the lane's pixel, its image offset and the top-left
        // input coordinate of its window.  Pixels past the end are clamped
        // onto the last one (computed, never stored).
        int base_h[PT], base_w[PT];
        uint32_t img_off[PT];
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            int64_t m = m0 + p * 32 + col;
            m = m < a.M ? m : a.M - 1;
            const int64_t per_img = static_cast<int64_t>(g.OH) * g.OW;
            const int n = static_cast<int>(m / per_img);
            const int r = static_cast<int>(m - n * per_img);
            const int oh = r / g.OW;
            const int ow = r - oh * g.OW;
            base_h[p] = oh * g.sh - g.ph;
            base_w[p] = ow * g.sw - g.pw;
            img_off[p] = static_cast<uint32_t>(n) * static_cast<uint32_t>(g.H * g.W) * pix_bytes + lane_ch;
        }
        // k-block kb = (tap t, channel chunk ch); its step s covers channels
        // ch*16*KB + 16*s + 8*q .. +8 of the group for this lane.
        auto load_block = [&](int kb, uint4 (&dst)[KB][PT]) {
            const int t = kb / chunks;
            const int ch = kb - t * chunks;
            const int kh = t / g.KW;
            const int kw = t - kh * g.KW;
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                const int ih = base_h[p] + kh * g.dh;
                const int iw = base_w[p] + kw * g.dw;
                const bool in = kb < kblocks && static_cast<unsigned>(ih) < static_cast<unsigned>(g.H) &&
                                static_cast<unsigned>(iw) < static_cast<unsigned>(g.W);
                const uint32_t off = img_off[p] + (static_cast<uint32_t>(ih) * g.W + iw) * pix_bytes +
                                     static_cast<uint32_t>(ch) * (KB * 32u);
#pragma unroll
                for (int st = 0; st < KB; ++st)
                    dst[st][p] = buffer_load16(xr, in ? off + st * 32u : kOutside);
            }
        };

        f32x16 acc[2][PT];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int p = 0; p < PT; ++p)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[ct][p][v] = 0.f;

        // A weight row is ordered (kh, kw, channel) like the k-blocks, so
        // step st of block kb is k = (kb*KB + st)*16 + 8q: 16-byte unit
        // (kb*KB + st)*2 + q of the row.
        auto run_block = [&](int kb, const uint4 (&frag)[KB][PT]) {
#pragma unroll
            for (int st = 0; st < KB; ++st) {
                const int k16 = (kb * KB + st) * 2 + q;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const bf16x8 wa = as_bf16x8(w_lds[(ct * 32 + col) * row16 + k16]);
#pragma unroll
                    for (int p = 0; p < PT; ++p)
                        acc[ct][p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            wa, as_bf16x8(frag[st][p]), acc[ct][p], 0, 0, 0);
                }
            }
        };

        // Three fragment buffers in rotation: blocks kb+1 and kb+2 are in
        // flight while block kb runs on the MFMA units.
        uint4 f0[KB][PT], f1[KB][PT], f2[KB][PT];
        load_block(0, f0);
        load_block(1, f1);
        for (int kb = 0; kb < kblocks; kb += 3) {
            load_block(kb + 2, f2);
            run_block(kb, f0);
            if (kb + 1 < kblocks) {
                load_block(kb + 3, f0);
                run_block(kb + 1, f1);
            }
            if (kb + 2 < kblocks) {
                load_block(kb + 4, f1);
                run_block(kb + 2, f2);
            }
        }

        // Lane holds, for pixel m0 + 32p + col, channels
        // co0 + 32ct + 8j + 4q + {0..3} in acc[ct][p][4j .. 4j+3].
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int co_rel = co_in_grp + ct * 32 + j * 8 + q * 4;
                const int co = co0 + ct * 32 + j * 8 + q * 4;
                const bool co_ok = co_rel < g.Mg;
                const uint2 bv = __builtin_bit_cast(
                    uint2, __builtin_amdgcn_raw_buffer_load_b64(br, static_cast<uint32_t>(co) * 2u, 0, 0));
                const float b0 = __uint_as_float(bv.x << 16), b1 = __uint_as_float(bv.x & 0xffff0000u);
                const float b2 = __uint_as_float(bv.y << 16), b3 = __uint_as_float(bv.y & 0xffff0000u);
#pragma unroll
                for (int p = 0; p < PT; ++p) {
                    const int64_t m = m0 + p * 32 + col;
                    const uint2 out = {pack_bf16x2(acc[ct][p][4 * j + 0] + b0, acc[ct][p][4 * j + 1] + b1),
                                       pack_bf16x2(acc[ct][p][4 * j + 2] + b2, acc[ct][p][4 * j + 3] + b3)};
                    const uint32_t off = (co_ok && m < a.M)
                                             ? (static_cast<uint32_t>(m) * static_cast<uint32_t>(g.CO) + co) * 2u
                                             : kOutside;
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(yr, 0, 0, 0)), out), yr,
                        off, 0, 0);
                }
            }
        }
    }
}

size_t lds_bytes(const Geom& g)
{
    const int K = g.KH * g.KW * g.Cg;
    return static_cast<size_t>(kBN) * (K / 8 + 1) * 16;
}

int num_cus()
{
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    return cus;
}

// Two 32-pixel tiles per wave: 64 accumulators and three k-blocks of
// fragments in flight fit two waves per SIMD.
template <int KB>
hipError_t launch_kb(IgemmArgs a, hipStream_t s, size_t lds)
{
    constexpr int PT = 2;
    a.px_tiles = static_cast<int>((a.M + 32 * PT - 1) / (32 * PT));
    auto kernel = igemm_kernel<PT, KB>;
    static size_t lds_allowed = 64 * 1024;  // the default dynamic LDS limit
    if (lds > lds_allowed) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
        lds_allowed = lds;
    }
    const int groups_y = a.g.G * a.co_tiles;
    const int per_cu = lds <= static_cast<size_t>(kLdsBytes / 2) ? 2 : 1;
    int gx = (a.px_tiles + kWaves - 1) / kWaves;
    const int cap = max(1, num_cus() * per_cu / groups_y);
    gx = min(gx, cap);
    return launch(kernel, dim3(gx, groups_y), dim3(kThreads), lds, s, a);
}

}  // namespace

bool can_igemm(const Geom& g, int dtype)
{
    if (dtype != 1 || !g.nhwc || !g.aligned16) return false;
    if (g.Cg % 16 != 0 || g.Mg % 4 != 0) return false;
    if (lds_bytes(g) > static_cast<size_t>(kLdsBytes)) return false;
    const int64_t x_bytes = static_cast<int64_t>(g.N) * g.H * g.W * g.C * 2;
    const int64_t y_bytes = static_cast<int64_t>(g.N) * g.OH * g.OW * g.CO * 2;
    return x_bytes < (int64_t(1) << 31) && y_bytes < (int64_t(1) << 31);
}

hipError_t launch_igemm(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                        hipStream_t s)
{
    IgemmArgs a;
    a.x = static_cast<const bf16_t*>(x);
    a.w = static_cast<const bf16_t*>(w);
    a.bias = static_cast<const bf16_t*>(bias);
    a.y = static_cast<bf16_t*>(y);
    a.g = g;
    a.M = static_cast<int64_t>(g.N) * g.OH * g.OW;
    a.K = g.KH * g.KW * g.Cg;
    a.co_tiles = (g.Mg + kBN - 1) / kBN;
    const size_t lds = lds_bytes(g);
    const int steps = g.Cg / 16;  // 16-channel k-steps per tap
    if (steps % 4 == 0) return launch_kb<4>(a, s, lds);
    if (steps % 3 == 0) return launch_kb<3>(a, s, lds);
    if (steps % 2 == 0) return launch_kb<2>(a, s, lds);
    return launch_kb<1>(a, s, lds);
}

}  // namespace convmi
