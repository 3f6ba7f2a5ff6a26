// Pointwise (1x1) forward convolution as one GEMM on the MFMA units.
//
// A 1x1 kernel maps every output pixel to the input pixel
// under it, so the convolution is y[m, co] = bias[co] + sum_c x[m, c] *
// w[co, c] over the M = N*OH*OW pixels, both operands K-major in NHWC/OHWI
// (burn-cubecl 0.22.0-pre.4 src/kernel/conv/im2col.rs, `check_pointwise`,
// `conv_im2col_1x1`, `reshape_weight`).  A stride only selects which input
// pixel row feeds pixel m (`strided_spatial_view` on the same page), which
// the kernel folds into its row addressing instead of a view.  Zero padding
// of a 1x1 kernel puts the input pixel under an output pixel outside the
// image at the border; those output pixels are the bias alone (zero padding
// reads zeros outside the image: teeny-kernels src/nn/conv/conv2d.rs,
// `conv2d_forward`).
//
// MI355X design: at C=256, C_out=64 the GEMM does 51 FLOP per HBM byte, far
// below the bf16 ridge (~312), so the kernel is an HBM stream.  Each block
// stages its 64 output channels' weights in LDS by buffer-to-LDS loads
// (padded rows, conflict-free reads) and each wave pulls 32 pixel rows straight from HBM into MFMA
// operand registers (16-byte loads), runs v_mfma_f32_16x16x32_bf16 with the
// weights as the A operand (rows = output channels) so every lane ends with
// four consecutive output channels of one pixel, adds the bias in fp32 and
// rounds once to bf16.  The wave's output tile is regrouped in LDS so that
// stores write whole 128-byte lines.  Blocks of eight waves (256 pixels)
// share one copy of the weights between twice as many pixels as four-wave
// blocks would, and at 120 registers two of them fit on a CU, so every block
// of the 56x56 x 32 layer is resident at once and the whole input is in
// flight from the start.
#include "kernels.hpp"

namespace convmi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kBN = 64;          // output channels per block (four 16-row MFMA tiles)
constexpr int kWaveM = 32;       // pixels per wave (two 16-column MFMA tiles)
constexpr int kBM = (kThreads / 64) * kWaveM;  // pixels per block
constexpr int kMaxC = 256;       // C = 32*KS with KS <= 8 k-steps held in registers

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// KS = C / 32: the number of 32-wide k-steps, all held in registers.
template <int KS, bool FULL_LINES>
__global__ __launch_bounds__(kThreads) void pointwise_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const bf16_t* __restrict__ bias,
    bf16_t* __restrict__ y, int64_t M, int CO, int H, int W, int OH, int OW, int sh, int sw,
    int ph, int pw)
{
    constexpr int C = 32 * KS;
    constexpr int ROW16 = C / 8 + 1;  // LDS row pitch in 16-byte units: one pad unit
    __shared__ uint4 w_lds[kBN * ROW16];
    __shared__ uint4 out_lds[FULL_LINES ? (kThreads / 64) * kWaveM * 8 : 1];
    const int co0 = blockIdx.y * kBN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;  // MFMA column: the pixel within a 16-pixel tile
    const int grp = lane >> 4;  // MFMA k-group: 8 consecutive channels of a k-step
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kBM + wave * kWaveM;

    // The bias of this lane's output channels co0 + 16t + 4*grp + {0..3}
    // (a null bias, and channels past C_out, read zero through the resource
    // bounds), and the block's 64 weight rows straight into their padded LDS
    // rows by 16-byte buffer-to-LDS loads (wave load j of wave w fills units
    // 64 (8j + w) ..; pad units and rows past C_out load zero; the MFMA rows
    // these feed are never stored).  Both go out before the pixel loads, so
    // one wait for all but those pixel loads covers them.
    const rsrc_t br = make_rsrc(bias, bias ? static_cast<uint32_t>(CO) * 2u : 0u);
    uint2 braw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int co = co0 + t * 16 + grp * 4;
        braw[t] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                br, co < CO ? static_cast<uint32_t>(co) * 2 : kOutside, 0, 0));
    }
    constexpr int kWPadded = kBN * ROW16;  // a multiple of 64 units
    constexpr int kWWaveLoads = kWPadded / 64;
    const uint32x4_t wrs = dma_rsrc(w, static_cast<uint32_t>(CO) * C * 2u);
#pragma unroll
    for (int j = 0; j < (kWWaveLoads + 7) / 8; ++j) {
        const int wl = j * 8 + wave;
        if (wl < kWWaveLoads) {
            const int U = wl * 64 + lane;
            const int r = U / ROW16, c = U - (U / ROW16) * ROW16;
            const bool ok = c < C / 8 && co0 + r < CO;
            dma16(wrs, ok ? static_cast<uint32_t>((co0 + r) * C + c * 8) * 2u : kOutside,
                  lds_addr(w_lds + wl * 64));
        }
    }

    // This lane's two pixel rows.  Rows past the end are clamped onto the
    // last pixel: their MFMA columns are computed from real memory and never
    // stored, so every load is unconditional and all are in flight at once.
    // With padding, an output pixel whose input pixel lies outside the image
    // reads a valid pixel and zeroes it, so that only the bias remains.
    bool valid[2];
    uint4 bfrag[2][KS];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int64_t m = m0 + p * 16 + col;
        valid[p] = m < M;
        const int64_t mm = valid[p] ? m : M - 1;
        const int64_t img = static_cast<int64_t>(OH) * OW;
        const int64_t n = mm / img;
        const int r = static_cast<int>(mm - n * img);
        const int oh = r / OW, ow = r - (r / OW) * OW;
        const int ih = oh * sh - ph, iw = ow * sw - pw;
        const bool inside = static_cast<unsigned>(ih) < static_cast<unsigned>(H) &&
                            static_cast<unsigned>(iw) < static_cast<unsigned>(W);
        const int64_t src = inside ? (n * H + ih) * W + iw : n * H * W;
        const uint4* xrow = reinterpret_cast<const uint4*>(x + src * C);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 v = xrow[s * 4 + grp];
            bfrag[p][s] = inside ? v : uint4{0u, 0u, 0u, 0u};
        }
    }

    wait_vm<2 * KS>();    // the bias and this wave's weight loads (all but the pixel loads)
    barrier_no_fence();   // every wave's weight loads have landed

    f32x4 acc[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int p = 0; p < 2; ++p) acc[t][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x8 a = as_bf16x8(w_lds[(t * 16 + col) * ROW16 + s * 4 + grp]);
#pragma unroll
            for (int p = 0; p < 2; ++p)
                acc[t][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(bfrag[p][s]),
                                                                   acc[t][p], 0, 0, 0);
        }
    }

    // Lane holds output channels co0 + 16t + 4*grp + {0..3} of pixel m0 + 16p + col.
    uint2 out[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint2 bv = braw[t];
        const float b[4] = {__uint_as_float(bv.x << 16), __uint_as_float(bv.x & 0xffff0000u),
                            __uint_as_float(bv.y << 16), __uint_as_float(bv.y & 0xffff0000u)};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            out[t][p].x = pack_bf16x2(acc[t][p][0] + b[0], acc[t][p][1] + b[1]);
            out[t][p].y = pack_bf16x2(acc[t][p][2] + b[2], acc[t][p][3] + b[3]);
        }
    }
    if (!FULL_LINES) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int co = co0 + t * 16 + grp * 4;
            if (co >= CO) continue;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                if (!valid[p]) continue;
                const int64_t m = m0 + p * 16 + col;
                *reinterpret_cast<uint2*>(y + m * CO + co) = out[t][p];
            }
        }
        return;
    }
    // With C_out a multiple of 8 the wave's 32 pixels x 64 channels go out as
    // whole 16-byte units: staged in LDS as pixel rows of eight units (unit
    // u of pixel q at position u ^ (q & 7), so neither the 8-byte writes nor
    // the 16-byte reads collide in banks), then each store instruction writes
    // eight pixels' 128 contiguous bytes.  Whole lines that nothing reads
    // back go out with the non-temporal hint, so they stream to memory
    // instead of collecting in L2 until the end-of-kernel write-back.
    uint4* const stage = out_lds + wave * (kWaveM * 8);
    uint2* const stage2 = reinterpret_cast<uint2*>(stage);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int q = p * 16 + col;
            const int u = 2 * t + (grp >> 1);
            stage2[(q * 8 + (u ^ (q & 7))) * 2 + (grp & 1)] = out[t][p];
        }
    __builtin_amdgcn_wave_barrier();
    // The resource spans this wave's pixels that exist, so pixels past M drop.
    const int64_t left = M - m0;
    const rsrc_t yr = make_rsrc(y + m0 * CO, left > 0 ? static_cast<uint32_t>(min<int64_t>(left, kWaveM) * CO * 2) : 0u);
#pragma unroll
    for (int r = 0; r < kWaveM / 8; ++r) {
        const int q = r * 8 + (lane >> 3);
        const int u = lane & 7;
        const uint4 v = stage[q * 8 + (u ^ (q & 7))];
        const int co = co0 + u * 8;
        buffer_store16_nt(yr, co < CO ? static_cast<uint32_t>(q * CO + co) * 2u : kOutside, v);
    }
}

}  // namespace

bool can_pointwise(const Geom& g, int dtype)
{
    return dtype == 1 && g.nhwc && g.aligned16 && g.KH == 1 && g.KW == 1 && g.G == 1 &&
           g.C % 32 == 0 && g.C <= kMaxC && g.CO % 4 == 0 &&
           static_cast<int64_t>(g.N) * g.OH * g.OW < (int64_t(1) << 31);
}

hipError_t launch_pointwise(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                            hipStream_t s)
{
    const int64_t M = static_cast<int64_t>(g.N) * g.OH * g.OW;
    const dim3 grid(static_cast<unsigned>((M + kBM - 1) / kBM), (g.CO + kBN - 1) / kBN);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(w);
    const bf16_t* bb = static_cast<const bf16_t*>(bias);
    bf16_t* yb = static_cast<bf16_t*>(y);
    void (*k)(const bf16_t*, const bf16_t*, const bf16_t*, bf16_t*, int64_t, int, int, int, int,
              int, int, int, int, int) = nullptr;
    const bool full = g.CO % 8 == 0;
    switch (g.C / 32) {
#define CASE(ks) case ks: k = full ? pointwise_kernel<ks, true> : pointwise_kernel<ks, false>; break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: return hipErrorInvalidValue;
    }
    return launch(k, grid, dim3(kThreads), 0, s, xb, wb, bb, yb, M, g.CO, g.H, g.W, g.OH, g.OW,
                  g.sh, g.sw, g.ph, g.pw);
}

}  // namespace convmi
