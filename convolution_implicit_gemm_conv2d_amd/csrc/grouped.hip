// Small-group forward convolution (C/G = C_out/G = CG in {4, 8}, 3x3) on
// the 4x4x4 matrix instruction.
//
// Output channel co of group g = co / CG sums over the CG input channels of
// its group and the taps: y[n, oh, ow, co] = bias[co] + sum_{kh, kw, i}
// x[n, oh*sh - ph + kh*dh, ow*sw - pw + kw*dw, g*CG + i] * w[co, kh, kw, i]
// (the per-group loop of teeny-kernels 0.2.0 src/nn/conv/conv2d.rs,
// `conv2d_forward`).  Per group and tap this is a CG x CG matrix against CG
// channels of each pixel: a contraction of length 9 CG that the vector units
// issue at two MACs per lane per instruction, which left the layer bound by
// instruction issue at about twice its HBM time.
//
// v_mfma_f32_4x4x4_16b_bf16 runs 16 independent 4x4x4 products per wave
// (block b on lanes 4b .. 4b+3): lane 4b + i supplies row i of A (4 values
// along k), lane 4b + j column j of B, and lane 4b + j receives column j of
// D, rows 0..3.  With the weights as A (rows = output channels) and pixels
// as B (columns = 4 consecutive output columns), each block is one group
// (CG = 4) or half of one (CG = 8, whose 8 input channels take two
// instructions), nothing is padded, and each lane ends with 4 consecutive
// output channels of one pixel.  Measured on this GPU: 262 TMAC/s for the
// instruction against 69 for v_dot2_f32_bf16.
//
// A wave owns 64 output channels (16 blocks) x 8 output columns (two sets
// of 4, two independent accumulator chains) and walks a segment of R output
// rows; its weights (9 taps x CG/4 operands) stay in registers.  Operands
// read straight from NHWC memory would put neighbouring lanes one pixel
// apart, each load touching many lines; instead each kernel row's input
// columns are loaded whole (16 bytes a lane, consecutive lanes consecutive
// bytes, zero outside the image) one output row ahead, written to the
// wave's own LDS, and the B operands read from there.  The output goes the
// same way in reverse: the 8 x 64 tile is transposed through LDS and leaves
// as 16-byte non-temporal stores of whole lines.  No LDS is shared between
// waves, so no barrier is needed.
//
// LDS layout per pixel: 8 chunks of 16 bytes (64 channels), chunk c stored
// at c ^ 2 (key & 3), key = the pixel's staged column / horizontal stride.
// The four lanes of a block read four pixels whose keys are consecutive, so
// the reads of a 4x4x4 operand (8 or 16 bytes) and the 16-byte row writes
// each use every bank equally.
#include "kernels.hpp"

#include <algorithm>

namespace convmi {
namespace {

typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;
constexpr int KH = 3, KW = 3, TAPS = KH * KW;
constexpr int kCols = 8;             // output columns per wave
constexpr int kWaveTarget = 4096;    // waves in all: about four per SIMD

__device__ __forceinline__ uint32_t swz(uint32_t chunk, uint32_t key) { return chunk ^ ((key & 3u) << 1); }

// Orders this wave's LDS writes before its later reads (and the reverse):
// LDS operations of one wave complete in order, so only the compiler needs
// to be held.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// L = 16-byte loads per lane per kernel row: the wave stages 8 L input
// columns, enough for the 7 sw + 2 dw + 1 it reads.  RING (sh == dh): the
// kernel rows of output row oh are input rows (oh + kh) dh - ph, so
// consecutive output rows share two of them; the three staged rows form a
// ring (input row r in slot r mod 3) and each output row loads one new row.
template <int CG, int L, bool RING>
__global__ __launch_bounds__(kThreads) void grouped_mfma_kernel(const bf16_t* __restrict__ x,
                                                                const bf16_t* __restrict__ w,
                                                                const bf16_t* __restrict__ bias,
                                                                bf16_t* __restrict__ y, Geom g, int col_quads,
                                                                int cblocks, int segs, int R)
{
    constexpr int KQ = CG / 4;  // 4-channel k quarters per tap
    constexpr int kRowBytes = 8 * L * 128;
    constexpr int kInBytes = KH * kRowBytes;
    constexpr int kWaveBytes = kInBytes + kCols * 128;
    __shared__ uint4 lds[kWaves * kWaveBytes / 16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    // Workgroup -> (image, row segment, channel block, four column segments).
    // Consecutive workgroups go to consecutive XCDs; the grid is a multiple
    // of 8 and the remap gives each XCD a contiguous run, so neighbouring
    // segments share an L2.  Padding workgroups get an image past the last.
    const int nb = gridDim.x;
    int b = (static_cast<int>(blockIdx.x) % kXcds) * (nb / kXcds) + static_cast<int>(blockIdx.x) / kXcds;
    const int cq = b % col_quads;
    b /= col_quads;
    const int cb = b % cblocks;
    b /= cblocks;
    const int seg = b % segs;
    const int n = b / segs;
    if (n >= g.N) return;  // grid padding (the whole workgroup; no barrier follows)
    const int ow0 = (cq * kWaves + wave) * kCols;  // this wave's first output column
    if (ow0 >= g.OW) return;                        // no barrier follows: the wave may leave
    const int oh_begin = seg * R, oh_end = min(g.OH, oh_begin + R);
    char* const wl = reinterpret_cast<char*>(lds) + wave * kWaveBytes;

    const int blk = lane >> 2, idx = lane & 3;
    // CG = 4: block blk is group cb*16 + blk.  CG = 8: block blk is half
    // blk % 2 of group cb*8 + blk/2.  base = first output channel of the
    // block.
    const int base = cb * 64 + blk * 4;

    // A operands: lane (blk, idx) holds row idx = output channel base + idx,
    // k quarter q of each tap.
    s4_t wa[TAPS][KQ];
    {
        const uint2* wr = reinterpret_cast<const uint2*>(w + static_cast<int64_t>(base + idx) * TAPS * CG);
#pragma unroll
        for (int t = 0; t < TAPS; ++t)
#pragma unroll
            for (int q = 0; q < KQ; ++q) wa[t][q] = __builtin_bit_cast(s4_t, wr[t * KQ + q]);
    }
    // Accumulators start from the bias of channels base + 0..3 (a null bias
    // is a zero-byte resource, whose loads return zero).
    f4_t b4;
    {
        const rsrc_t br = make_rsrc(bias, bias ? static_cast<uint32_t>(g.C) * 2u : 0u);
        const uint2 v = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(br, static_cast<uint32_t>(base) * 2u, 0, 0));
        b4 = f4_t{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                  __uint_as_float(v.y & 0xffff0000u)};
    }

    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * 2u;
    const uint32_t blk_bytes = static_cast<uint32_t>(cb) * 128u;  // this wave's 64 channels in a pixel
    const uint32_t img_in = static_cast<uint32_t>(g.H) * g.W * pix_bytes;
    const rsrc_t xr = make_rsrc(x + static_cast<int64_t>(n) * g.H * g.W * g.C, img_in);
    const uint32_t img_out = static_cast<uint32_t>(g.OH) * g.OW * pix_bytes;
    const rsrc_t yr = make_rsrc(y + static_cast<int64_t>(n) * g.OH * g.OW * g.C, img_out);
    const uint32_t sw = static_cast<uint32_t>(g.sw);

    // Row loads: lane l fetches chunk l % 8 of staged column p = l / 8 + 8 i,
    // input column ow0 sw - pw + p (kOutside when outside the image).
    // Columns past the last one read are not fetched.
    const int used = (kCols - 1) * g.sw + (KW - 1) * g.dw + 1;
    uint32_t colo[L], wofs[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const uint32_t p = static_cast<uint32_t>(lane >> 3) + 8u * i, c = lane & 7;
        const int iw = ow0 * g.sw - g.pw + static_cast<int>(p);
        colo[i] = static_cast<int>(p) < used && static_cast<unsigned>(iw) < static_cast<unsigned>(g.W)
                      ? static_cast<uint32_t>(iw) * pix_bytes + blk_bytes + c * 16u
                      : kOutside;
        wofs[i] = p * 128u + swz(c, p / sw) * 16u;
    }
    // Operand reads: lane (blk, idx) of column set cs takes staged column
    // p = (4 cs + idx) sw + kw dw, at its channels' chunk (and half, CG = 4).
    uint32_t rofs[2][KW];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs)
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) {
            const uint32_t p = static_cast<uint32_t>(4 * cs + idx) * sw + static_cast<uint32_t>(kw * g.dw);
            rofs[cs][kw] = p * 128u + swz(blk >> 1, p / sw) * 16u + (CG == 4 ? (blk & 1) * 8u : 0u);
        }
    // Output transpose: lane (blk, idx) of column set cs writes column
    // 4 cs + idx, channels base..base+3; lane l then reads chunk l % 8 of
    // column l / 8 and stores it.
    uint32_t owr[2];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
        const uint32_t col = 4 * cs + idx;
        owr[cs] = kInBytes + col * 128u + swz(blk >> 1, col) * 16u + (blk & 1) * 8u;
    }
    const uint32_t ocol = lane >> 3, ochunk = lane & 7;
    const uint32_t ord = kInBytes + ocol * 128u + swz(ochunk, ocol) * 16u;
    const bool ocol_ok = ow0 + static_cast<int>(ocol) < g.OW;
    const uint32_t ost = (static_cast<uint32_t>(ow0) + ocol) * pix_bytes + blk_bytes + ochunk * 16u;

    // Input row ih -> the lane's L chunks (zero outside the image).
    auto load_in = [&](int ih, uint4* dst) __attribute__((always_inline)) {
        const bool row_ok = static_cast<unsigned>(ih) < static_cast<unsigned>(g.H);
        const uint32_t rowo = static_cast<uint32_t>(ih) * g.W * pix_bytes;
#pragma unroll
        for (int i = 0; i < L; ++i) dst[i] = buffer_load16(xr, row_ok && colo[i] != kOutside ? rowo + colo[i] : kOutside);
    };
    auto stage = [&](int slot, const uint4* src) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < L; ++i) *reinterpret_cast<uint4*>(wl + slot * kRowBytes + wofs[i]) = src[i];
    };
    // Output row oh from the staged rows (kernel row kh in slot[kh]): the
    // 4x4x4 products, then the transposed store.
    auto compute_store = [&](int oh, const int* slot) __attribute__((always_inline)) {
        f4_t acc[2] = {b4, b4};
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
            const char* row = wl + slot[kh] * kRowBytes;
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) {
                const int t = kh * KW + kw;
#pragma unroll
                for (int cs = 0; cs < 2; ++cs) {
                    const char* src = row + rofs[cs][kw];
                    if constexpr (KQ == 1) {
                        const s4_t v = *reinterpret_cast<const s4_t*>(src);
                        acc[cs] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(wa[t][0], v, acc[cs], 0, 0, 0);
                    } else {
                        const uint4 v = *reinterpret_cast<const uint4*>(src);
                        acc[cs] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                            wa[t][0], __builtin_bit_cast(s4_t, uint2{v.x, v.y}), acc[cs], 0, 0, 0);
                        acc[cs] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                            wa[t][1], __builtin_bit_cast(s4_t, uint2{v.z, v.w}), acc[cs], 0, 0, 0);
                    }
                }
            }
        }
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
            *reinterpret_cast<uint2*>(wl + owr[cs]) =
                uint2{pack_bf16x2(acc[cs][0], acc[cs][1]), pack_bf16x2(acc[cs][2], acc[cs][3])};
        wave_lds_sync();
        const uint4 o = *reinterpret_cast<const uint4*>(wl + ord);
        buffer_store16_nt(yr, ocol_ok ? static_cast<uint32_t>(oh) * g.OW * pix_bytes + ost : kOutside, o);
        wave_lds_sync();
    };

    if (oh_begin >= oh_end) return;
    if constexpr (RING) {
        // Input row r = oh + kh (in units of dh) sits in slot r % 3.
        const int r0 = oh_begin;
        {
            uint4 t0[L], t1[L];
            load_in(r0 * g.dh - g.ph, t0);
            load_in((r0 + 1) * g.dh - g.ph, t1);
            stage(r0 % 3, t0);
            stage((r0 + 1) % 3, t1);
        }
        uint4 pf[L];
        load_in((r0 + 2) * g.dh - g.ph, pf);
        int s0 = r0 % 3;  // slot of row oh
        for (int oh = oh_begin; oh < oh_end; ++oh) {
            const int s1 = s0 == 2 ? 0 : s0 + 1, s2 = s1 == 2 ? 0 : s1 + 1;
            stage(s2, pf);
            wave_lds_sync();
            if (oh + 1 < oh_end) load_in((oh + 3) * g.dh - g.ph, pf);
            const int slot[KH] = {s0, s1, s2};
            compute_store(oh, slot);
            s0 = s1;
        }
    } else {
        uint4 pf[KH][L];
        auto load_rows = [&](int oh) __attribute__((always_inline)) {
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) load_in(oh * g.sh - g.ph + kh * g.dh, pf[kh]);
        };
        load_rows(oh_begin);
        constexpr int slot[KH] = {0, 1, 2};
        for (int oh = oh_begin; oh < oh_end; ++oh) {
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) stage(kh, pf[kh]);
            wave_lds_sync();
            if (oh + 1 < oh_end) load_rows(oh + 1);
            compute_store(oh, slot);
        }
    }
}

// 16-byte loads per lane per kernel row for this geometry (0: too wide).
int row_loads(const Geom& g)
{
    const int cols = (kCols - 1) * g.sw + (KW - 1) * g.dw + 1;
    return cols <= 16 ? 2 : cols <= 24 ? 3 : 0;
}

}  // namespace

bool can_grouped_mfma(const Geom& g, int dtype)
{
    if (dtype != 1 || !g.nhwc || !g.aligned16) return false;
    if (g.Cg != g.Mg || (g.Cg != 4 && g.Cg != 8) || g.C % 64 != 0) return false;
    if (g.KH != KH || g.KW != KW || row_loads(g) == 0) return false;
    const int64_t img = static_cast<int64_t>(std::max(g.H * g.W, g.OH * g.OW)) * g.C * 2;
    return img < (int64_t(1) << 31);
}

hipError_t launch_grouped_mfma(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                               hipStream_t s)
{
    const int col_segs = (g.OW + kCols - 1) / kCols;
    const int col_quads = (col_segs + kWaves - 1) / kWaves;
    const int cblocks = g.C / 64;
    // Row segments: enough for about kWaveTarget waves, none shorter than
    // four rows (each wave loads its weights once).
    const int64_t base_waves = static_cast<int64_t>(g.N) * col_segs * cblocks;
    int segs = static_cast<int>(std::min<int64_t>((kWaveTarget + base_waves - 1) / base_waves, (g.OH + 3) / 4));
    segs = std::max(1, segs);
    const int R = (g.OH + segs - 1) / segs;
    segs = (g.OH + R - 1) / R;
    const int64_t blocks = (static_cast<int64_t>(g.N) * segs * cblocks * col_quads + kXcds - 1) / kXcds * kXcds;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(w);
    const bf16_t* bb = static_cast<const bf16_t*>(bias);
    bf16_t* yb = static_cast<bf16_t*>(y);
    auto go = [&](auto kernel) {
        return launch(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, xb, wb, bb, yb, g,
                      col_quads, cblocks, segs, R);
    };
    const bool two = row_loads(g) == 2, ring = g.sh == g.dh;
    if (g.Cg == 4) {
        if (two) return ring ? go(grouped_mfma_kernel<4, 2, true>) : go(grouped_mfma_kernel<4, 2, false>);
        return ring ? go(grouped_mfma_kernel<4, 3, true>) : go(grouped_mfma_kernel<4, 3, false>);
    }
    if (two) return ring ? go(grouped_mfma_kernel<8, 2, true>) : go(grouped_mfma_kernel<8, 2, false>);
    return ring ? go(grouped_mfma_kernel<8, 3, true>) : go(grouped_mfma_kernel<8, 3, false>);
}

}  // namespace convmi
