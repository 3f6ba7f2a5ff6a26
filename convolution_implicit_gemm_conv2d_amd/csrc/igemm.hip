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
// is never built: its rows are gathered on the fly from a tile of x held in
// LDS.
//
// MI355X design.  A workgroup owns an output region of R rows x TW columns of
// one image and a 64-wide output-channel tile.  It stages, per chunk of CC
// input channels, (a) the input halo the region reads -- IR x IC pixels, zero
// outside the image, loaded with full-line 16-byte accesses through a buffer
// resource -- and (b) the tile's weight panel [64][taps*CC], both in LDS.
// Every A fragment (weights, 32 channels x 16 k) and B fragment (32 pixels x
// 16 k) of v_mfma_f32_32x32x16_bf16 is then one ds_read_b128 per lane: a lane
// reads 8 channels of one pixel at the halo position of its tap, so each
// input pixel is fetched from HBM once per workgroup and reused by every tap
// from LDS.  Halo pixels keep their 16-byte units XOR-swizzled by pixel index
// so that 16 consecutive pixels hit 16 distinct bank groups; weight rows are
// padded by one unit for the same reason.  The 32x32x16 form keeps the
// matrix pipe near peak with few independent accumulators.  Each wave
// computes up to four 32-pixel tiles x both 32-channel halves of the channel
// tile, so a weight fragment serves up to four MFMAs and a pixel fragment
// two.  Results get the bias in fp32, are rounded once to bf16 and leave as
// runs of four channels (8-byte stores, dropped by the buffer bounds outside
// the output).
#include "kernels.hpp"

namespace convmi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBN = 64;                 // output channels per workgroup
constexpr int kMaxTilesPerWave = 4;     // 32-pixel tiles per wave
constexpr int kMaxPixels = 32 * kWaves * kMaxTilesPerWave;  // per workgroup
constexpr int kLdsBytes = 160 * 1024;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

struct IgemmArgs {
    const bf16_t* x;
    const bf16_t* w;
    const bf16_t* bias;
    bf16_t* y;
    Geom g;
    int R, TW;        // output rows / columns of a workgroup's region
    int IR, IC;       // input halo rows / columns of that region
    int row_tiles, col_tiles, co_tiles;
};

// UP = CC / 8: 16-byte units per staged pixel (2, 4 or 8).  Unit u of halo
// pixel hp lives at position u ^ swz(hp): 16 consecutive pixels then cover
// all 16 bank groups for any fixed u.
template <int UP>
__device__ __forceinline__ int swz(int hp)
{
    return (hp / (16 / UP)) & (UP - 1);
}

// KH_, KW_: compile-time kernel extent (the tap loop is then fully unrolled
// and scheduled), or 0 for a runtime extent.
template <int UP, int KH_, int KW_>
__global__ __launch_bounds__(kThreads) void igemm_kernel(IgemmArgs a)
{
    extern __shared__ uint4 lds[];
    const Geom& g = a.g;
    const int KWr = KW_ ? KW_ : g.KW;
    const int taps = KH_ ? KH_ * KW_ : g.KH * g.KW;
    const int halo_px = a.IR * a.IC;
    const int halo_units = (halo_px * UP + 63) / 64 * 64;  // padded to whole wave loads
    uint4* halo = lds;                       // [IR*IC][UP]
    uint4* wl = lds + halo_units;            // [64][taps*UP + 1]
    const int wrow = taps * UP + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;  // MFMA row (weights) / column (pixels) of this lane
    const int q = lane >> 5;    // MFMA k-group: 8 consecutive channels of a 16-channel step

    // Workgroup -> (image, row tile, column tile) x (group, channel tile).
    int b = blockIdx.x;
    const int ctile = b % a.col_tiles;
    b /= a.col_tiles;
    const int rtile = b % a.row_tiles;
    const int n = b / a.row_tiles;
    const int grp_id = blockIdx.y / a.co_tiles;
    const int co_in_grp = (blockIdx.y - grp_id * a.co_tiles) * kBN;
    const int co0 = grp_id * g.Mg + co_in_grp;
    const int co_last = grp_id * g.Mg + g.Mg - 1;
    const int oh0 = rtile * a.R, ow0 = ctile * a.TW;
    const int ih0 = oh0 * g.sh - g.ph, iw0 = ow0 * g.sw - g.pw;
    const int rows_here = min(a.R, g.OH - oh0), cols_here = min(a.TW, g.OW - ow0);
    const int npx = a.R * a.TW;  // region pixels (some may fall outside the output)

    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * 2u;
    const rsrc_t xr = make_rsrc(a.x + static_cast<int64_t>(n) * g.H * g.W * g.C,
                                static_cast<uint32_t>(g.H * g.W) * pix_bytes);
    const rsrc_t wr = make_rsrc(a.w, static_cast<uint32_t>(g.CO) * static_cast<uint32_t>(g.KH * g.KW * g.Cg) * 2u);

    // This lane's pixels: tile pt = wave + 4j covers region pixels
    // 32*pt .. 32*pt + 31; the lane owns pixel 32*pt + col.  hbase is its halo
    // index for tap (0, 0).
    int hbase[kMaxTilesPerWave];
#pragma unroll
    for (int j = 0; j < kMaxTilesPerWave; ++j) {
        const int p = min((wave + kWaves * j) * 32 + col, npx - 1);
        const int r = p / a.TW, c = p - (p / a.TW) * a.TW;
        hbase[j] = r * g.sh * a.IC + c * g.sw;
    }
    // Every wave runs all kMaxTilesPerWave tiles: a tile past the region
    // computes on a clamped pixel and is never stored, which keeps the inner
    // loop free of branches (the workgroup's time is its busiest wave's).

    f32x16 acc[2][kMaxTilesPerWave];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int j = 0; j < kMaxTilesPerWave; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ct][j][v] = 0.f;

    const int chunks = g.Cg / (UP * 8);
    for (int chunk = 0; chunk < chunks; ++chunk) {
        if (chunk > 0) __syncthreads();  // every wave is done reading the previous chunk
        const uint32_t ch_off = static_cast<uint32_t>(grp_id * g.Cg + chunk * UP * 8) * 2u;
        // Halo: LDS unit L = hp*UP + pos holds unit pos ^ swz(hp) of halo
        // pixel hp = x[n, ih0 + hp / IC, iw0 + hp % IC].  Loaded straight into
        // LDS, 64 consecutive units per wave instruction; out-of-image pixels
        // and the padding past the halo read as zero.
        for (int k = wave; k * 64 < halo_units; k += kWaves) {
            const int L = k * 64 + lane;
            const int hp = L / UP, pos = L - (L / UP) * UP;
            const int u = pos ^ swz<UP>(hp);
            const int hr = hp / a.IC, hc = hp - (hp / a.IC) * a.IC;
            const int ih = ih0 + hr, iw = iw0 + hc;
            const bool in = hp < halo_px && static_cast<unsigned>(ih) < static_cast<unsigned>(g.H) &&
                            static_cast<unsigned>(iw) < static_cast<unsigned>(g.W);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void*)(halo + k * 64), 16,
                in ? (static_cast<uint32_t>(ih) * g.W + iw) * pix_bytes + ch_off + u * 16u : kOutside, 0, 0, 0);
        }
        // Weight panel: LDS unit L = r*wrow + c holds, for c < taps*UP, unit
        // c % UP of tap c / UP of output channel co0 + r (this chunk's
        // channels); the pad unit of each row and channels past the group
        // read as zero.
        // Every workgroup reads the same panel; starting each one at a
        // different wave load spreads the simultaneous requests over the L2
        // channels instead of queueing them all on the same lines.
        const int wunits = (kBN * wrow + 63) / 64 * 64;
        const int wloads = wunits / 64;
        const int rot = static_cast<int>((blockIdx.x * 37u + blockIdx.y * 11u) % static_cast<unsigned>(wloads));
        for (int kk = wave; kk < wloads; kk += kWaves) {
            const int k = kk + rot < wloads ? kk + rot : kk + rot - wloads;
            const int L = k * 64 + lane;
            const int r = L / wrow, c = L - (L / wrow) * wrow;
            const int t = c / UP, u = c - (c / UP) * UP;
            const bool in = r < kBN && c < taps * UP && co0 + r <= co_last;
            const uint32_t off = ((static_cast<uint32_t>(co0 + r) * taps + t) * (g.Cg / 8) + chunk * UP + u) * 16u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (__attribute__((address_space(3))) void*)(wl + k * 64), 16,
                in ? off : kOutside, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS loads have landed
        __syncthreads();                // and every other wave's

        // k-step ks = (tap t, 16-channel step s).  Fragments of step ks+1 are
        // read from LDS while the MFMAs of step ks run.
        constexpr int SPT = UP / 2;  // k-steps per tap
        struct Frags {
            bf16x8 wa[2];
            bf16x8 px[kMaxTilesPerWave];
        };
        auto read_frags = [&](int ks, Frags& f) {
            const int t = ks / SPT, st = ks - (ks / SPT) * SPT;
            const int kh = t / KWr, kw = t - (t / KWr) * KWr;
            const int hoff = kh * g.dh * a.IC + kw * g.dw;
            const int u = st * 2 + q;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) f.wa[ct] = as_bf16x8(wl[(ct * 32 + col) * wrow + t * UP + u]);
#pragma unroll
            for (int j = 0; j < kMaxTilesPerWave; ++j) {
                const int hp = hbase[j] + hoff;
                f.px[j] = as_bf16x8(halo[hp * UP + (u ^ swz<UP>(hp))]);
            }
        };
        auto mfmas = [&](const Frags& f) {
#pragma unroll
            for (int j = 0; j < kMaxTilesPerWave; ++j)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    acc[ct][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.wa[ct], f.px[j], acc[ct][j], 0, 0, 0);
        };
        const int ksteps = taps * SPT;
        Frags fa, fb;
        read_frags(0, fa);
        if constexpr (KH_ > 0) {
            constexpr int KS = KH_ * KW_ * SPT;
#pragma unroll
            for (int ks = 0; ks < KS; ks += 2) {
                if (ks + 1 < KS) read_frags(ks + 1, fb);
                mfmas(fa);
                if (ks + 1 < KS) {
                    if (ks + 2 < KS) read_frags(ks + 2, fa);
                    mfmas(fb);
                }
            }
        } else {
            for (int ks = 0; ks < ksteps; ks += 2) {
                read_frags(min(ks + 1, ksteps - 1), fb);
                mfmas(fa);
                if (ks + 1 < ksteps) {
                    read_frags(min(ks + 2, ksteps - 1), fa);
                    mfmas(fb);
                }
            }
        }
    }

    // Epilogue.  Lane holds, for its pixel of tile j, channels
    // co0 + 32ct + 8i + 4q + {0..3} in acc[ct][j][4i .. 4i+3].  Bias is added
    // in fp32 and each value rounded once; the bf16 tile is staged in LDS as
    // [pixel][64 channels] rows (pitch 144 bytes) and written out as whole
    // 128-byte pixel rows, eight pixels per wave store.
    __syncthreads();  // every wave is done reading the halo and weights
    constexpr int kPitch = 9;  // 16-byte units per staged pixel row (8 + 1 pad)
    uint4* ostage = lds + wave * (32 * kMaxTilesPerWave) * kPitch;
    const rsrc_t br = make_rsrc(a.bias, a.bias ? static_cast<uint32_t>(g.CO) * 2u : 0u);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int co = co0 + ct * 32 + i * 8 + q * 4;
            const uint2 bv = __builtin_bit_cast(
                uint2, __builtin_amdgcn_raw_buffer_load_b64(br, static_cast<uint32_t>(co) * 2u, 0, 0));
            const float b0 = __uint_as_float(bv.x << 16), b1 = __uint_as_float(bv.x & 0xffff0000u);
            const float b2 = __uint_as_float(bv.y << 16), b3 = __uint_as_float(bv.y & 0xffff0000u);
#pragma unroll
            for (int j = 0; j < kMaxTilesPerWave; ++j) {
                const uint2 out = {pack_bf16x2(acc[ct][j][4 * i + 0] + b0, acc[ct][j][4 * i + 1] + b1),
                                   pack_bf16x2(acc[ct][j][4 * i + 2] + b2, acc[ct][j][4 * i + 3] + b3)};
                uint2* row = reinterpret_cast<uint2*>(ostage + (j * 32 + col) * kPitch);
                row[(ct * 4 + i) * 2 + q] = out;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    const uint32_t img_out = static_cast<uint32_t>(g.OH * g.OW) * static_cast<uint32_t>(g.CO) * 2u;
    const rsrc_t yr = make_rsrc(a.y + static_cast<int64_t>(n) * g.OH * g.OW * g.CO, img_out);
    const int u = lane & 7;                 // 16-byte unit (8 channels) of the pixel row
    const int crel = co_in_grp + u * 8;     // first channel of the unit within the group
    const bool full = crel + 8 <= g.Mg;
    const bool half = crel + 4 <= g.Mg;     // channel tiles end on a multiple of 4
#pragma unroll
    for (int k = 0; k < (32 * kMaxTilesPerWave) / 8; ++k) {
        const int lp = k * 8 + (lane >> 3);  // pixel within this wave's tiles
        const int j = lp >> 5;
        const int p = (wave + kWaves * j) * 32 + (lp & 31);
        const int r = p / a.TW, c = p - (p / a.TW) * a.TW;
        const bool ok = p < npx && r < rows_here && c < cols_here;
        const uint4 v = ostage[lp * kPitch + u];
        const uint32_t off = (static_cast<uint32_t>((oh0 + r) * g.OW + ow0 + c) * static_cast<uint32_t>(g.CO) +
                              static_cast<uint32_t>(co0 + u * 8)) * 2u;
        if (full) {
            buffer_store16(yr, ok ? off : kOutside, v);
        } else {
            const uint2 lo = {v.x, v.y};
            __builtin_amdgcn_raw_buffer_store_b64(
                __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(yr, 0, 0, 0)), lo), yr,
                (ok && half) ? off : kOutside, 0, 0);
        }
    }
}

// Host-side plan: region shape and channel chunk for a geometry.
struct Plan {
    int UP, R, TW, IR, IC, row_tiles, col_tiles, co_tiles;
    size_t lds;
    bool ok;
};

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

Plan make_plan(const Geom& g, int cus)
{
    Plan p{};
    p.ok = false;
    if (g.Cg % 64 == 0) p.UP = 8;
    else if (g.Cg % 32 == 0) p.UP = 4;
    else if (g.Cg % 16 == 0) p.UP = 2;
    else return p;
    const int taps = g.KH * g.KW;
    p.TW = g.OW < 64 ? g.OW : 64;
    p.col_tiles = (g.OW + p.TW - 1) / p.TW;
    p.co_tiles = (g.Mg + kBN - 1) / kBN;
    const size_t wbytes = static_cast<size_t>((kBN * (taps * p.UP + 1) + 63) / 64 * 64) * 16;
    // Among region heights that fit LDS and the per-wave tile budget, take
    // the one with the least per-CU work (rounds of workgroups x tiles per
    // wave); ties go to the taller region, which re-reads less halo.
    long best = -1;
    for (int R = 1; R <= g.OH && R * p.TW <= kMaxPixels; ++R) {
        const int IR = (R - 1) * g.sh + (g.KH - 1) * g.dh + 1;
        const int IC = (p.TW - 1) * g.sw + (g.KW - 1) * g.dw + 1;
        size_t lds = static_cast<size_t>((IR * IC * p.UP + 63) / 64 * 64) * 16 + wbytes;
        const size_t stage = static_cast<size_t>(kWaves) * 32 * kMaxTilesPerWave * 9 * 16;  // epilogue rows
        if (lds < stage) lds = stage;
        if (lds > static_cast<size_t>(kLdsBytes)) break;
        const long blocks = static_cast<long>(g.N) * ((g.OH + R - 1) / R) * p.col_tiles * g.G * p.co_tiles;
        const long rounds = (blocks + cus - 1) / cus;
        const long tiles = ((R * p.TW + 31) / 32 + kWaves - 1) / kWaves;
        const long cost = rounds * tiles;
        if (best < 0 || cost <= best) {
            best = cost;
            p.R = R;
            p.IR = IR;
            p.IC = IC;
            p.lds = lds;
            p.row_tiles = (g.OH + R - 1) / R;
        }
    }
    p.ok = best >= 0;
    return p;
}

template <int UP, int KH_, int KW_>
hipError_t launch_up(const IgemmArgs& a, const Plan& p, hipStream_t s)
{
    auto kernel = igemm_kernel<UP, KH_, KW_>;
    static size_t lds_allowed = 64 * 1024;  // the default dynamic LDS limit
    if (p.lds > lds_allowed) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(p.lds));
        if (e != hipSuccess) return e;
        lds_allowed = p.lds;
    }
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.g.N) * p.row_tiles * p.col_tiles),
                    a.g.G * p.co_tiles);
    return launch(kernel, grid, dim3(kThreads), p.lds, s, a);
}

}  // namespace

bool can_igemm(const Geom& g, int dtype)
{
    if (dtype != 1 || !g.nhwc || !g.aligned16) return false;
    if (g.Cg % 16 != 0 || g.Mg % 4 != 0) return false;
    const int64_t x_img = static_cast<int64_t>(g.H) * g.W * g.C * 2;
    const int64_t y_img = static_cast<int64_t>(g.OH) * g.OW * g.CO * 2;
    const int64_t w_bytes = static_cast<int64_t>(g.CO) * g.KH * g.KW * g.Cg * 2;
    if (x_img >= (int64_t(1) << 31) || y_img >= (int64_t(1) << 31) || w_bytes >= (int64_t(1) << 31))
        return false;
    if (static_cast<int64_t>(g.N) * g.OH * g.OW >= (int64_t(1) << 31)) return false;
    return make_plan(g, 256).ok;
}

hipError_t launch_igemm(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                        hipStream_t s)
{
    const Plan p = make_plan(g, num_cus());
    if (!p.ok) return hipErrorInvalidValue;
    IgemmArgs a;
    a.x = static_cast<const bf16_t*>(x);
    a.w = static_cast<const bf16_t*>(w);
    a.bias = static_cast<const bf16_t*>(bias);
    a.y = static_cast<bf16_t*>(y);
    a.g = g;
    a.R = p.R;
    a.TW = p.TW;
    a.IR = p.IR;
    a.IC = p.IC;
    a.row_tiles = p.row_tiles;
    a.col_tiles = p.col_tiles;
    a.co_tiles = p.co_tiles;
    const bool k3 = g.KH == 3 && g.KW == 3;
    switch (p.UP) {
    case 8: return k3 ? launch_up<8, 3, 3>(a, p, s) : launch_up<8, 0, 0>(a, p, s);
    case 4: return k3 ? launch_up<4, 3, 3>(a, p, s) : launch_up<4, 0, 0>(a, p, s);
    default: return k3 ? launch_up<2, 3, 3>(a, p, s) : launch_up<2, 0, 0>(a, p, s);
    }
}

}  // namespace convmi
