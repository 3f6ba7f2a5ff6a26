// Pointwise (1x1) forward convolution as one GEMM on the MFMA units.
//
// A 1x1 kernel with no padding maps every output pixel to the input pixel
// under it, so the convolution is y[m, co] = bias[co] + sum_c x[m, c] *
// w[co, c] over the M = N*OH*OW pixels, both operands K-major in NHWC/OHWI
// (burn-cubecl 0.22.0-pre.4 src/kernel/conv/im2col.rs, `check_pointwise`,
// `conv_im2col_1x1`, `reshape_weight`).  A stride only selects which input
// pixel row feeds pixel m (`strided_spatial_view` on the same page), which
// the kernel folds into its row addressing instead of a view.
//
// MI355X design: at C=256, C_out=64 the GEMM does 51 FLOP per HBM byte, far
// below the bf16 ridge (~312), so the kernel is an HBM stream.  Each block
// stages its 64 output channels' weights in LDS (padded rows, conflict-free
// reads) and each wave pulls 32 pixel rows straight from HBM into MFMA
// operand registers (16-byte loads), runs v_mfma_f32_16x16x32_bf16 with the
// weights as the A operand (rows = output channels) so every lane ends with
// four consecutive output channels of one pixel, adds the bias in fp32,
// rounds once to bf16 and stores 8 bytes per lane.  Enough blocks are
// resident to keep the whole input in flight.
#include "kernels.hpp"

namespace convmi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBN = 64;          // output channels per block (four 16-row MFMA tiles)
constexpr int kWaveM = 32;       // pixels per wave (two 16-column MFMA tiles)
constexpr int kBM = 4 * kWaveM;  // pixels per block
constexpr int kChunk = 8;        // 32-wide k-steps held in registers at once
constexpr int kMaxC = 448;       // [64][C] weight tile within 64 KB of LDS

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__global__ __launch_bounds__(kThreads) void pointwise_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const bf16_t* __restrict__ bias,
    bf16_t* __restrict__ y, int64_t M, int C, int CO, int H, int W, int OH, int OW, int sh, int sw)
{
    extern __shared__ uint4 w_lds[];  // [64][C/8 + 1] 16-byte units
    const int row16 = C / 8 + 1;
    const int co0 = blockIdx.y * kBN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;  // MFMA column: the pixel within a 16-pixel tile
    const int grp = lane >> 4;  // MFMA k-group: 8 consecutive channels of a 32-step
    const int ksteps = C / 32;
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kBM + wave * kWaveM;
    const uint4 zero = {0u, 0u, 0u, 0u};

    // Input row of each of this lane's two pixels.
    const uint4* xrow[2];
    bool valid[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int64_t m = m0 + p * 16 + col;
        valid[p] = m < M;
        const int64_t mm = valid[p] ? m : 0;
        const int64_t img = static_cast<int64_t>(OH) * OW;
        const int64_t n = mm / img;
        const int r = static_cast<int>(mm - n * img);
        const int oh = r / OW, ow = r - (r / OW) * OW;
        const int64_t src = (n * H + static_cast<int64_t>(oh) * sh) * W + static_cast<int64_t>(ow) * sw;
        xrow[p] = reinterpret_cast<const uint4*>(x + src * C);
    }

    uint4 bfrag[2][kChunk];
    auto load_chunk = [&](int s0) {
#pragma unroll
        for (int s = 0; s < kChunk; ++s)
#pragma unroll
            for (int p = 0; p < 2; ++p)
                bfrag[p][s] = (valid[p] && s0 + s < ksteps) ? xrow[p][(s0 + s) * 4 + grp] : zero;
    };
    load_chunk(0);  // in flight while the weights are staged

    const int per_row = C / 8;
    for (int i = tid; i < kBN * per_row; i += kThreads) {
        const int r = i / per_row;
        const int c = i - r * per_row;
        uint4 v = zero;
        if (co0 + r < CO) v = reinterpret_cast<const uint4*>(w + static_cast<int64_t>(co0 + r) * C)[c];
        w_lds[r * row16 + c] = v;
    }
    __syncthreads();

    f32x4 acc[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int p = 0; p < 2; ++p) acc[t][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < ksteps; s0 += kChunk) {
        if (s0 > 0) load_chunk(s0);
#pragma unroll
        for (int s = 0; s < kChunk; ++s) {
            if (s0 + s < ksteps) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const bf16x8 a = as_bf16x8(w_lds[(t * 16 + col) * row16 + (s0 + s) * 4 + grp]);
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        acc[t][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            a, as_bf16x8(bfrag[p][s]), acc[t][p], 0, 0, 0);
                }
            }
        }
    }

    // Lane holds output channels co0 + 16t + 4*grp + {0..3} of pixel m0 + 16p + col.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int co = co0 + t * 16 + grp * 4;
        if (co >= CO) continue;
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias) {
#pragma unroll
            for (int r = 0; r < 4; ++r) b[r] = bf16_to_f(bias[co + r]);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (!valid[p]) continue;
            const int64_t m = m0 + p * 16 + col;
            uint2 out;
            out.x = pack_bf16x2(acc[t][p][0] + b[0], acc[t][p][1] + b[1]);
            out.y = pack_bf16x2(acc[t][p][2] + b[2], acc[t][p][3] + b[3]);
            *reinterpret_cast<uint2*>(y + m * CO + co) = out;
        }
    }
}

}  // namespace

bool can_pointwise(const Geom& g, int dtype)
{
    return dtype == 1 && g.nhwc && g.aligned16 && g.KH == 1 && g.KW == 1 && g.ph == 0 &&
           g.pw == 0 && g.G == 1 && g.C % 32 == 0 && g.C <= kMaxC && g.CO % 4 == 0 &&
           static_cast<int64_t>(g.N) * g.OH * g.OW < (int64_t(1) << 31);
}

hipError_t launch_pointwise(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                            hipStream_t s)
{
    const int64_t M = static_cast<int64_t>(g.N) * g.OH * g.OW;
    const dim3 grid(static_cast<unsigned>((M + kBM - 1) / kBM), (g.CO + kBN - 1) / kBN);
    const size_t lds = static_cast<size_t>(kBN) * (g.C / 8 + 1) * 16;
    return launch(pointwise_kernel, grid, dim3(kThreads), lds, s, static_cast<const bf16_t*>(x),
                  static_cast<const bf16_t*>(w), static_cast<const bf16_t*>(bias),
                  static_cast<bf16_t*>(y), M, g.C, g.CO, g.H, g.W, g.OH, g.OW, g.sh, g.sw);
}

}  // namespace convmi
