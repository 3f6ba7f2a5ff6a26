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
// one image and a 64-wide output-channel tile.  The K loop runs over chunks
// of CC = 8 UP input channels (32 or 16).  For a chunk the workgroup stages
// in LDS (a) the input halo the region reads -- IR x IC pixels x CC
// channels, zero outside the image -- and (b) the tile's weight panel
// [64][taps * CC]; both arrive by 16-byte buffer-to-LDS loads.  Two stages
// alternate, so the next chunk streams in while the current one is
// multiplied.  Every A fragment (weights, 32 channels x 16 k) and B fragment
// (32 pixels x 16 k) of v_mfma_f32_32x32x16_bf16 is one ds_read_b128 per
// lane: a lane reads 8 channels of one pixel at the halo position of its
// tap, so each input pixel is fetched once per workgroup and reused by every
// tap from LDS.  Halo pixels keep their 16-byte units XOR-swizzled by pixel
// index and weight rows are padded by one unit, which makes both fragment
// reads conflict-free.  Eight waves (two per SIMD): wave w computes NT of the
// region's 32-pixel tiles (w, w + 8, ...) for both 32-channel halves of the
// tile -- a k-step's two weight fragments then serve all of the wave's
// tiles -- or, for groups of at most 32 output channels, for the first
// half.  Results get the
// bias in fp32 and are rounded once to bf16; the tile is then restaged in
// LDS so that each pixel's 64 channels leave as whole 128-byte lines
// (measured on a 4096-long sequence, 128 -> 128 channels, 3 taps: 40.2 ->
// 37.5 us against 8-byte stores straight from the accumulators, which remain
// for groups whose channel count is not a multiple of 8).
#include "kernels.hpp"

#include <algorithm>
#include <type_traits>

namespace convmi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;           // eight waves
constexpr int kWaves = kThreads / 64;
constexpr int kBN = 64;                 // output channels per workgroup
constexpr int kMaxNT = 4;               // 32-pixel tiles per wave
constexpr int kMaxPixels = 32 * kWaves * kMaxNT;  // per workgroup
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
    int regions;      // N * row_tiles * col_tiles
    int halo_units;   // 16-byte units of one stage's halo (whole wave loads)
    int w_units;      // ... and of its weight panel
    FastDiv div_ic;   // by IC: halo pixel -> halo row
    FastDiv div_wrow; // by the weight row pitch
};

// UP = CC / 8: 16-byte units per staged pixel (2 or 4).  Unit u of halo
// pixel hp lives at position u ^ swz(hp): 16 consecutive pixels then cover
// all 64 banks for any fixed u.
template <int UP>
__device__ __forceinline__ int swz(int hp)
{
    return (hp / (16 / UP)) & (UP - 1);
}

// KH_, KW_: compile-time kernel extent (the tap loop is then fully unrolled
// and scheduled), or 0 for a runtime extent.  NT: pixel tiles per wave.
// HN: 32-channel halves per wave, 2, or 1 for groups of at most 32 output
// channels.  Against four-wave workgroups on one half per wave: conv1d
// (4096 long, 128 -> 128 channels, 3 taps) 35.1 -> 27.2 us, 3x3 with 8 groups
// of 24 channels at 56x56 x 32 48.5 -> 42.3 us.
template <int UP, int KH_, int KW_, int NT, int HN>
__global__ __launch_bounds__(kThreads) void igemm_kernel(IgemmArgs a)
{
    extern __shared__ uint4 lds[];
    const Geom& g = a.g;
    const int KWr = KW_ ? KW_ : g.KW;
    const int taps = KH_ ? KH_ * KW_ : g.KH * g.KW;
    const int halo_px = a.IR * a.IC;
    const int wrow = taps * UP + 1;
    const int stage_units = a.halo_units + a.w_units;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;  // MFMA row (weights) / column (pixels) of this lane
    const int q = lane >> 5;    // MFMA k-group: 8 consecutive channels of a 16-channel step
    constexpr int ct = 0;         // the wave's first 32-channel half
    const int pw0 = wave;         // its first pixel tile,
    constexpr int pstep = kWaves;  // then every pstep-th one

    // Workgroup -> (image, row tile, column tile) x (group, channel tile).
    // The grid is one-dimensional: eight consecutive regions take
    // consecutive workgroups (one per XCD, workgroup b running on XCD
    // b mod 8), and the (group, channel tile) index advances after each
    // eight, so every channel tile of a region runs on one XCD and close in
    // time: the region's input lines, which every group reads a part of,
    // are fetched into that XCD's L2 once, and the parts of its output lines
    // written by the groups meet there before they are written back.
    const int tiles_y = a.g.G * a.co_tiles;
    const int lin = blockIdx.x;
    const int by = (lin >> 3) % tiles_y;
    int b = ((lin >> 3) / tiles_y) * 8 + (lin & 7);
    if (b >= a.regions) return;  // the grid is padded to whole eights of regions
    const int ctile = b % a.col_tiles;
    b /= a.col_tiles;
    const int rtile = b % a.row_tiles;
    const int n = b / a.row_tiles;
    const int grp_id = by / a.co_tiles;
    const int co_in_grp = (by - grp_id * a.co_tiles) * kBN;
    const int co0 = grp_id * g.Mg + co_in_grp;
    const int oh0 = rtile * a.R, ow0 = ctile * a.TW;
    const int ih0 = oh0 * g.sh - g.ph, iw0 = ow0 * g.sw - g.pw;
    const int rows_here = min(a.R, g.OH - oh0), cols_here = min(a.TW, g.OW - ow0);
    const int npx = a.R * a.TW;  // region pixels (some may fall outside the output)

    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * 2u;
    const uint32x4_t xr = dma_rsrc(a.x + static_cast<int64_t>(n) * g.H * g.W * g.C,
                                   static_cast<uint32_t>(g.H * g.W) * pix_bytes);
    const uint32x4_t wr =
        dma_rsrc(a.w, static_cast<uint32_t>(g.CO) * static_cast<uint32_t>(g.KH * g.KW * g.Cg) * 2u);

    // This lane's pixels: tile pt = pw0 + pstep j covers region pixels
    // 32 pt .. 32 pt + 31; the lane owns pixel 32 pt + col.  hbase is its halo
    // index for tap (0, 0).  A tile past the region computes on a clamped
    // pixel and is never stored, which keeps the inner loop free of branches.
    int hbase[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int p = min((pw0 + pstep * j) * 32 + col, npx - 1);
        const int r = p / a.TW, c = p - (p / a.TW) * a.TW;
        hbase[j] = r * g.sh * a.IC + c * g.sw;
    }

    // Issues the loads of channel chunk `chunk` into the stage at `st`.
    // Halo: LDS unit L = hp*UP + pos holds unit pos ^ swz(hp) of halo pixel
    // hp = x[n, ih0 + hp / IC, iw0 + hp % IC]; out-of-image pixels and the
    // padding past the halo read as zero.  Weight panel: LDS unit
    // L = r*wrow + c holds, for c < taps*UP, unit c % UP of tap c / UP of
    // output channel co0 + r; the pad unit of each row and channels past the
    // group read as zero.  Every workgroup reads the same panel; starting
    // each one at a different wave load spreads the simultaneous requests
    // over the L2 channels.
    // A group whose channel count is a multiple of 8 but not of the chunk
    // width ends in a part chunk: its units past the group's channels load
    // as zero in the halo and in the panel.
    const int cg_units = g.Cg / 8;
    auto issue = [&](int chunk, uint4* st) __attribute__((always_inline)) {
        const uint32_t ch_off = static_cast<uint32_t>(grp_id * g.Cg + chunk * UP * 8) * 2u;
        for (int k = wave; k * 64 < a.halo_units; k += kWaves) {
            const int L = k * 64 + lane;
            const int hp = L / UP, pos = L & (UP - 1);
            const int u = pos ^ swz<UP>(hp);
            const int hr = static_cast<int>(fdiv(static_cast<uint32_t>(hp), a.div_ic));
            const int hc = hp - hr * a.IC;
            const int ih = ih0 + hr, iw = iw0 + hc;
            const bool in = hp < halo_px && static_cast<unsigned>(ih) < static_cast<unsigned>(g.H) &&
                            static_cast<unsigned>(iw) < static_cast<unsigned>(g.W) && chunk * UP + u < cg_units;
            dma16(xr, in ? (static_cast<uint32_t>(ih) * g.W + iw) * pix_bytes + ch_off + u * 16u : kOutside,
                  lds_addr(st + k * 64));
        }
        uint4* wl = st + a.halo_units;
        const int wloads = a.w_units / 64;
        const int rot = static_cast<int>((static_cast<unsigned>(b) * 37u + static_cast<unsigned>(by) * 11u) %
                                         static_cast<unsigned>(wloads));
        for (int kk = wave; kk < wloads; kk += kWaves) {
            const int k = kk + rot < wloads ? kk + rot : kk + rot - wloads;
            const int L = k * 64 + lane;
            const int r = static_cast<int>(fdiv(static_cast<uint32_t>(L), a.div_wrow));
            const int c = L - r * wrow;
            const int t = c / UP, u = c & (UP - 1);
            const bool in = r < kBN && c < taps * UP && co_in_grp + r < g.Mg && chunk * UP + u < cg_units;
            const uint32_t off = ((static_cast<uint32_t>(co0 + r) * taps + t) * (g.Cg / 8) + chunk * UP + u) * 16u;
            dma16(wr, in ? off : kOutside, lds_addr(wl + k * 64));
        }
    };

    f32x16 acc[HN][NT];
#pragma unroll
    for (int h = 0; h < HN; ++h)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[h][j][v] = 0.f;

    // k-step ks = (tap t, 16-channel step s).  Fragments of step ks+1 are
    // read from LDS while the MFMAs of step ks run.
    constexpr int SPT = UP / 2;  // k-steps per tap
    struct Frags {
        bf16x8 wa[HN];
        bf16x8 px[NT];
    };
    const int chunks = (g.Cg + UP * 8 - 1) / (UP * 8);
    issue(0, lds);
    for (int chunk = 0; chunk < chunks; ++chunk) {
        wait_vm<0>();        // this wave's loads of the chunk have landed
        barrier_no_fence();  // and every other wave's; chunk - 1's stage is free
        const uint4* st = lds + (chunk & 1) * stage_units;
        if (chunk + 1 < chunks) issue(chunk + 1, lds + ((chunk + 1) & 1) * stage_units);
        const uint4* halo = st;
        const uint4* wl = st + a.halo_units;
        auto read_frags = [&](int ks, Frags& f) __attribute__((always_inline)) {
            const int t = ks / SPT, s_ = ks - (ks / SPT) * SPT;
            const int kh = t / KWr, kw = t - (t / KWr) * KWr;
            const int hoff = kh * g.dh * a.IC + kw * g.dw;
            const int u = s_ * 2 + q;
#pragma unroll
            for (int h = 0; h < HN; ++h) f.wa[h] = as_bf16x8(wl[((ct + h) * 32 + col) * wrow + t * UP + u]);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int hp = hbase[j] + hoff;
                f.px[j] = as_bf16x8(halo[hp * UP + (u ^ swz<UP>(hp))]);
            }
        };
        auto mfmas = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int h = 0; h < HN; ++h)
                    acc[h][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.wa[h], f.px[j], acc[h][j], 0, 0, 0);
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
            // Runtime taps: a cursor over (tap, 16-channel step) moves one
            // k-step per read (no division in the loop); past the last
            // k-step it stays there (such reads feed no MFMA).
            const int k1 = ksteps > 1 ? 1 : 0;  // the first read is k-step 1 (0 if it is the only one)
            int c_ks = k1, c_s = k1 % SPT, c_t = k1 / SPT, c_kw = c_t, c_hoff = c_t * g.dw;
            if (c_kw == KWr) { c_kw = 0; c_hoff = g.dh * a.IC; }
            auto read_next = [&](Frags& f) __attribute__((always_inline)) {
                const int u = c_s * 2 + q;
#pragma unroll
                for (int h = 0; h < HN; ++h) f.wa[h] = as_bf16x8(wl[((ct + h) * 32 + col) * wrow + c_t * UP + u]);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int hp = hbase[j] + c_hoff;
                    f.px[j] = as_bf16x8(halo[hp * UP + (u ^ swz<UP>(hp))]);
                }
                if (c_ks + 1 < ksteps) {
                    ++c_ks;
                    if (++c_s == SPT) {
                        c_s = 0;
                        ++c_t;
                        c_hoff += g.dw;
                        if (++c_kw == KWr) {
                            c_kw = 0;
                            c_hoff += g.dh * a.IC - KWr * g.dw;
                        }
                    }
                }
            };
            for (int ks = 0; ks < ksteps; ks += 2) {
                read_next(fb);
                mfmas(fa);
                if (ks + 1 < ksteps) {
                    read_next(fa);
                    mfmas(fb);
                }
            }
        }
    }

    // Epilogue.  Lane holds, for its pixel of tile j, channels
    // co0 + 32(ct + h) + 8i + 4q + {0..3} in acc[h][j][4i .. 4i+3].  Bias is added in
    // fp32 and each value rounded once.  When the group's channels come in
    // whole 16-byte units (Mg a multiple of 8), the tile is restaged in LDS
    // as pixel rows of 8 units (unit u of pixel p at u ^ (p & 7)) and each
    // pixel's 64 channels leave as 16-byte stores, eight lanes per 128-byte
    // line (non-temporal when those lines are whole lines of y); otherwise
    // the four channels of a lane are stored as 8 bytes from registers.
    const rsrc_t br = make_rsrc(a.bias, a.bias ? static_cast<uint32_t>(g.CO) * 2u : 0u);
    const uint32_t img_out = static_cast<uint32_t>(g.OH * g.OW) * static_cast<uint32_t>(g.CO) * 2u;
    const rsrc_t yr = make_rsrc(a.y + static_cast<int64_t>(n) * g.OH * g.OW * g.CO, img_out);
    float bv[HN][4][4];
#pragma unroll
    for (int h = 0; h < HN; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int co = co0 + (ct + h) * 32 + i * 8 + q * 4;
            const uint2 v = __builtin_bit_cast(
                uint2, __builtin_amdgcn_raw_buffer_load_b64(br, static_cast<uint32_t>(co) * 2u, 0, 0));
            bv[h][i][0] = __uint_as_float(v.x << 16);
            bv[h][i][1] = __uint_as_float(v.x & 0xffff0000u);
            bv[h][i][2] = __uint_as_float(v.y << 16);
            bv[h][i][3] = __uint_as_float(v.y & 0xffff0000u);
        }
    if ((g.Mg & 7) == 0) {
        __syncthreads();  // every wave is done reading the stages
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int p = (pw0 + pstep * j) * 32 + col;
            if (p < npx) {
#pragma unroll
                for (int h = 0; h < HN; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int u = (ct + h) * 4 + i;
                        uint2* unit = reinterpret_cast<uint2*>(lds + p * 8 + (u ^ (p & 7)));
                        unit[q] = uint2{
                            pack_bf16x2(acc[h][j][4 * i + 0] + bv[h][i][0], acc[h][j][4 * i + 1] + bv[h][i][1]),
                            pack_bf16x2(acc[h][j][4 * i + 2] + bv[h][i][2], acc[h][j][4 * i + 3] + bv[h][i][3])};
                    }
            }
        }
        __syncthreads();
        const bool whole_lines = (g.CO & 63) == 0 && (g.Mg & 63) == 0;
        // Each pixel's units of this tile's channels as 16-byte stores,
        // consecutive lanes along a pixel's units.  A tile with fewer than
        // 64 channels of its group left (UV < 8 units per pixel) stores only
        // those instead of issuing the rest to be dropped.
        auto store_units = [&](auto uv_tag, int UV) __attribute__((always_inline)) {
            constexpr bool kFull = decltype(uv_tag)::value;
            for (int idx = tid; idx < npx * (kFull ? 8 : UV); idx += kThreads) {
                const int p = kFull ? idx >> 3 : idx / UV;
                const int u = kFull ? idx & 7 : idx - p * UV;
                const int r = p / a.TW, c = p - (p / a.TW) * a.TW;
                const bool ok = r < rows_here && c < cols_here && co_in_grp + u * 8 < g.Mg;
                const uint32_t off = ok ? (static_cast<uint32_t>((oh0 + r) * g.OW + ow0 + c) * static_cast<uint32_t>(g.CO) +
                                           static_cast<uint32_t>(co0 + u * 8)) * 2u
                                        : kOutside;
                const uint4 v = lds[p * 8 + (u ^ (p & 7))];
                if (whole_lines)
                    buffer_store16_nt(yr, off, v);
                else
                    buffer_store16(yr, off, v);
            }
        };
        const int UV = min(8, (g.Mg - co_in_grp) / 8);
        if (UV == 8)
            store_units(std::true_type{}, 8);
        else
            store_units(std::false_type{}, UV);
        return;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int p = (pw0 + pstep * j) * 32 + col;
        const int r = p / a.TW, c = p - (p / a.TW) * a.TW;
        const bool pix_ok = p < npx && r < rows_here && c < cols_here;
        const uint32_t pix_off =
            static_cast<uint32_t>((oh0 + r) * g.OW + ow0 + c) * static_cast<uint32_t>(g.CO) * 2u;
#pragma unroll
        for (int h = 0; h < HN; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int crel = co_in_grp + (ct + h) * 32 + i * 8 + q * 4;  // channel within the group
                const bool ok = pix_ok && crel < g.Mg;                        // Mg is a multiple of 4
                const uint2 out = {
                    pack_bf16x2(acc[h][j][4 * i + 0] + bv[h][i][0], acc[h][j][4 * i + 1] + bv[h][i][1]),
                    pack_bf16x2(acc[h][j][4 * i + 2] + bv[h][i][2], acc[h][j][4 * i + 3] + bv[h][i][3])};
                __builtin_amdgcn_raw_buffer_store_b64(
                    __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(yr, 0, 0, 0)), out), yr,
                    ok ? pix_off + static_cast<uint32_t>(co0 - co_in_grp + crel) * 2u : kOutside, 0, 0);
            }
    }
}

// Host-side plan: region shape and channel chunk for a geometry.
struct Plan {
    int UP, NT, HN, R, TW, IR, IC, row_tiles, col_tiles, co_tiles, halo_units, w_units;
    size_t lds;
    bool ok;
};

// Pixel-tile counts per wave with a compiled kernel.
constexpr int kNTs[] = {1, 2, 4};

// Workgroups (two waves per SIMD each) of a pixel-tile count that fit a CU by
// registers (compiler resource reports for gfx950): with both channel
// halves, 3 at one tile, 2 at two (1 with compiled 3x3 taps, 142-153
// registers) and 1 at four; with one half, 3, 2 and 1.
int reg_occupancy(int nt, int hn, bool k3)
{
    if (hn == 1) return nt <= 1 ? 3 : nt <= 2 ? 2 : 1;
    return nt <= 1 ? 3 : nt <= 2 ? (k3 ? 1 : 2) : 1;
}

Plan make_plan(const Geom& g, int cus)
{
    Plan best_plan{};
    best_plan.ok = false;
    long best = -1;
    int best_px = 0;
    // Channel chunks of 32 (UP = 4) or 16 (UP = 2) channels: the smaller
    // chunk halves the stages, so more workgroups share a CU.  Widths that
    // are multiples of 16 take the chunks that divide them; other multiples
    // of 8 (24, 40, 56, ...) end in a part chunk whose missing channels read
    // as zero.
    for (int up : {4, 2}) {
        const bool part = g.Cg % 16 == 8;
        if (part ? g.Cg < 8 * up - 8 : g.Cg % (8 * up) != 0) continue;
        Plan p{};
        p.UP = up;
        const int taps = g.KH * g.KW;
        const int chunks = (g.Cg + p.UP * 8 - 1) / (p.UP * 8);
        const int stages = chunks > 1 ? 2 : 1;
        p.co_tiles = (g.Mg + kBN - 1) / kBN;
        // Groups of at most 32 output channels use half the panel's rows and
        // one channel half per wave (see the kernel).
        const bool narrow = g.Mg <= 32;
        const int HN = narrow ? 1 : 2;
        const bool k3 = g.KH == 3 && g.KW == 3;
        const int w_units = ((narrow ? 32 : kBN) * (taps * p.UP + 1) + 63) / 64 * 64;
        // Among region shapes (TW columns x R rows) that fit LDS and the
        // per-wave tile budget, take the one with the least estimated time
        // per CU: the workgroups a CU runs times the time of one -- the larger
        // of its MFMA cycles (a wave's tiles x k-steps x 32) and its staging
        // cycles (halo and weight-panel bytes at about 50 B/clk into one CU)
        // when two or more workgroups share the CU, their sum when one does
        // -- scaled up where few workgroups are resident to hide each other's
        // prologue and epilogue (x2 for one, x1.4 for two, x1.15 for three).
        // The resident count is the smaller of the LDS and register limits.
        // Ties go to the larger region.  (Measured on one row of 4096,
        // 128 -> 128 channels, 3 taps, as chunk x columns: 16 x 128 and
        // 16 x 256 34.8 us, 32 x 256 37.5, 32 x 128 42.3, 16 x 512 45.8,
        // 16 x 64 49.9, 32 x 64 54.0.)
        for (int tw : {64, 128, 256, 512}) {
            const int TW = g.OW < tw ? g.OW : tw;
            if (tw > 64 && TW <= tw / 2) break;  // a narrower width already covers the row
            const int col_tiles = (g.OW + TW - 1) / TW;
            for (int R = 1; R <= g.OH && R * TW <= kMaxPixels; ++R) {
                const int IR = (R - 1) * g.sh + (g.KH - 1) * g.dh + 1;
                const int IC = (TW - 1) * g.sw + (g.KW - 1) * g.dw + 1;
                const int halo_units = (IR * IC * p.UP + 63) / 64 * 64;
                // The stages, or the output tile restaged as 128-byte pixel rows.
                const size_t lds = std::max(static_cast<size_t>(stages) * (halo_units + w_units) * 16,
                                            static_cast<size_t>(R) * TW * 128);
                if (lds > static_cast<size_t>(kLdsBytes)) break;
                const int need = ((R * TW + 31) / 32 + kWaves - 1) / kWaves;  // tiles per wave
                int nt = 0;
                for (int c : kNTs)
                    if (c >= need && !(HN == 2 && c == 4 && p.UP == 4 && k3)) {  // that one spills
                        nt = c;
                        break;
                    }
                if (nt == 0) break;
                const long occ = std::min(static_cast<long>(kLdsBytes / lds),
                                          static_cast<long>(reg_occupancy(nt, HN, k3)));
                const long blocks = static_cast<long>(g.N) * ((g.OH + R - 1) / R) * col_tiles * g.G * p.co_tiles;
                const long mfma = static_cast<long>(nt) * HN * taps * (p.UP / 2) * chunks * 32;
                const long load = static_cast<long>(halo_units + w_units) * chunks * 16 / 50;
                const long block_time = occ >= 2 ? std::max(mfma, load) : mfma + load;
                const long latency = occ >= 4 ? 100 : occ == 3 ? 115 : occ == 2 ? 140 : 200;  // percent
                const long cost = (blocks + cus - 1) / cus * block_time * latency / 100;
                if (best < 0 || cost < best || (cost == best && R * TW >= best_px)) {
                    best = cost;
                    best_px = R * TW;
                    p.TW = TW;
                    p.col_tiles = col_tiles;
                    p.R = R;
                    p.NT = nt;
                    p.HN = HN;
                    p.IR = IR;
                    p.IC = IC;
                    p.halo_units = halo_units;
                    p.w_units = w_units;
                    p.lds = lds;
                    p.row_tiles = (g.OH + R - 1) / R;
                    p.ok = true;
                    best_plan = p;
                }
            }
        }
    }
    return best_plan;
}

template <int UP, int KH_, int KW_, int NT, int HN>
hipError_t launch_nt(const IgemmArgs& a, const Plan& p, hipStream_t s)
{
    auto kernel = igemm_kernel<UP, KH_, KW_, NT, HN>;
    static size_t lds_allowed = 64 * 1024;  // the default dynamic LDS limit
    if (p.lds > lds_allowed) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(p.lds));
        if (e != hipSuccess) return e;
        lds_allowed = p.lds;
    }
    const int64_t blocks = (static_cast<int64_t>(a.regions) + 7) / 8 * 8 * a.g.G * p.co_tiles;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    return launch(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), p.lds, s, a);
}

template <int UP, int KH_, int KW_>
hipError_t launch_up(const IgemmArgs& a, const Plan& p, hipStream_t s)
{
    if (p.HN == 1) {
        switch (p.NT) {
        case 4: return launch_nt<UP, KH_, KW_, 4, 1>(a, p, s);
        case 2: return launch_nt<UP, KH_, KW_, 2, 1>(a, p, s);
        default: return launch_nt<UP, KH_, KW_, 1, 1>(a, p, s);
        }
    }
    switch (p.NT) {
    case 4:
        // Not planned with 32-channel chunks and compiled 3x3 taps (it spills).
        if constexpr (UP == 4 && KH_ == 3) return hipErrorInvalidValue;
        else return launch_nt<UP, KH_, KW_, 4, 2>(a, p, s);
    case 2: return launch_nt<UP, KH_, KW_, 2, 2>(a, p, s);
    default: return launch_nt<UP, KH_, KW_, 1, 2>(a, p, s);
    }
}

}  // namespace

bool can_igemm(const Geom& g, int dtype)
{
    if (dtype != 1 || !g.nhwc || !g.aligned16) return false;
    if (g.Cg % 8 != 0 || g.Mg % 4 != 0) return false;
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
    const Plan p = make_plan(g, device_cu_count());
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
    {
        const int64_t regions = static_cast<int64_t>(g.N) * p.row_tiles * p.col_tiles;
        if (regions >= (int64_t(1) << 31)) return hipErrorInvalidValue;
        a.regions = static_cast<int>(regions);
    }
    a.halo_units = p.halo_units;
    a.w_units = p.w_units;
    a.div_ic = make_fastdiv(static_cast<uint32_t>(p.IC));
    a.div_wrow = make_fastdiv(static_cast<uint32_t>(g.KH * g.KW * p.UP + 1));
    const bool k3 = g.KH == 3 && g.KW == 3;
    const bool k13 = g.KH == 1 && g.KW == 3;  // a three-tap conv1d
    if (p.UP == 4) return k3 ? launch_up<4, 3, 3>(a, p, s) : k13 ? launch_up<4, 1, 3>(a, p, s) : launch_up<4, 0, 0>(a, p, s);
    return k3 ? launch_up<2, 3, 3>(a, p, s) : k13 ? launch_up<2, 1, 3>(a, p, s) : launch_up<2, 0, 0>(a, p, s);
}

}  // namespace convmi
