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

// Pass 2 (shared with the MFMA path): dw[e] = the sum over pieces s of
// part[s][e], rounded once.  A workgroup takes 64 consecutive elements; its
// four waves sum the pieces s = w, w + 4, ... (in increasing s, sixteen
// loads in flight), and the four sums are added in wave order, so the result
// is the same on every run.
constexpr int kReduceElems = 64;
template <typename T>
__global__ __launch_bounds__(kThreads) void dw_reduce_kernel(const float* __restrict__ part,
                                                             T* __restrict__ dw, int64_t wn,
                                                             int pieces)
{
    __shared__ float sums[kThreads / 64][kReduceElems];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * kReduceElems + lane;
    float acc = 0.f;
    if (e < wn) {
        // Batches of kBatch pieces: every load of a batch is issued before
        // the first addition (addresses clamped to the last piece), so a
        // wave waits for memory once per batch; the additions keep the
        // increasing-s order.
        constexpr int kBatch = 16;
        const float* p = part + e;
        for (int s = wave; s < pieces; s += 4 * kBatch) {
            float a[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) a[i] = p[static_cast<int64_t>(min(s + 4 * i, pieces - 1)) * wn];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                if (s + 4 * i < pieces) acc += a[i];
        }
    }
    sums[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && e < wn) {
        const float total = ((sums[0][lane] + sums[1][lane]) + sums[2][lane]) + sums[3][lane];
        store_f(dw + e, total);
    }
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
    const dim3 grid(static_cast<unsigned>((wn + kReduceElems - 1) / kReduceElems));
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


// ---------------------------------------------------------------------------
// MFMA path (NHWC, bf16): pass 1 as an implicit GEMM per piece of pixels.
//
// Per group, dw[co, k] = sum_m dy[m, co] * A[m, k] with k = (kh, kw, c) in
// the weight's OHWI order and A[m, k] = x at pixel m shifted by tap (kh, kw),
// channel c (the im2col columns of the burn-cubecl page, never built).  The
// reduction runs over pixels m, which are the outer dimension of both NHWC
// operands, so both MFMA fragments (8 consecutive m per lane) are read from
// LDS rows [m][channels] with the gfx950 transpose read (ds_read_b64_tr_b16:
// within each 16-lane group, lane j's element k comes from element j mod 4
// of the 8-byte chunk that lane 4k + j/4 addressed).
//
// A workgroup owns a 64 (co) x 128 (k) tile of one group and one piece of
// the pixels.  Its four waves are independent: wave w takes the 16-pixel
// steps w, w + 4, ... of the piece, stages each step's 16 dy rows (64 co)
// and 16 A rows (128 k) in a private three-stage LDS ring by buffer-to-LDS
// loads, and runs 2 x 4 tiles of v_mfma_f32_32x32x16_bf16 per step.  No
// workgroup barrier sits in the loop.  At the end the four accumulators are
// added through LDS and the tile's fp32 partial is written to the workspace
// slice of its piece, laid out like dw itself, so that the reduction pass is
// the one the generic path uses.
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kCoTile = 64;
constexpr int kKTile = 128;
constexpr int kStepPx = 16;                       // pixels per wave step (one MFMA k-step)
constexpr int kDyUnits = kStepPx * kCoTile / 8;   // 128 16-byte units: 2 wave loads
constexpr int kXUnits = kStepPx * kKTile / 8;     // 256 units: 4 wave loads
constexpr int kStageUnits = kDyUnits + kXUnits;   // 6 KiB
constexpr int kStages = 3;
constexpr int kWaveUnits = kStages * kStageUnits;  // 18 KiB per wave
constexpr int kLoadsPerStep = (kDyUnits + kXUnits) / 64;  // 6

struct DwArgs {
    const bf16_t* x;
    const bf16_t* dy;
    float* part;
    Geom g;
    int Ktot;          // KH * KW * Cg: k extent of one group
    int k_tiles, co_tiles, tiles;  // tiles = k_tiles * co_tiles * G
    int pieces;
    int per;           // pixels per piece, a multiple of 4 * kStepPx
    int M;             // N * OH * OW
    FastDiv div_ow, div_oh, div_cg, div_kw;
    int d_ow, d_oh, d_n;  // one wave's advance per step (4 * kStepPx pixels) as (n, oh, ow) digits
};

// dy rows (8 units, 128 bytes): unit u of row r at position u ^ swz_dy(r);
// A rows (16 units, 256 bytes): unit u of row r at u ^ swz_a(r).  A transposed
// read touches 4 consecutive rows x 4 units per half wave; these maps send
// them to distinct banks.
__device__ __forceinline__ int swz_dy(int r) { return ((r >> 1) & 1) << 2; }
__device__ __forceinline__ int swz_a(int r) { return ((r & 3) << 2) ^ (r & 2); }

__global__ __launch_bounds__(256, 2) void dw_igemm_kernel(DwArgs a)
{
    __shared__ uint4 lds[4 * kWaveUnits];  // 72 KiB: each wave's ring; at the end, the tile exchange
    const Geom& g = a.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint4* const ring = lds + wave * kWaveUnits;

    // Workgroup -> (piece, tile), piece-major.  Workgroup b runs on XCD
    // b mod 8, so the tiles of a piece sit on different XCDs and each of
    // their L2s fetches the piece's pixels: on the 3x3, 64 -> 64 layer at
    // 56x56 x 32 that is 4.9x the algorithmic reads past L2, against 1.1x
    // when a piece's tiles share one XCD -- yet the shared placement measured
    // slower (33.8 against 31.5 us for both passes): five tiles reading the
    // same lines at once through one L2 cost more than the extra fetches,
    // which the cache in front of HBM serves.
    const int b = blockIdx.x;
    const int tile = b % a.tiles;
    const int piece = b / a.tiles;
    const int kt = tile % a.k_tiles;
    const int rest = tile / a.k_tiles;
    const int ct = rest % a.co_tiles;
    const int grp = rest / a.co_tiles;
    const int k0 = kt * kKTile;
    const int co_rel0 = ct * kCoTile;                 // within the group
    const int co0 = grp * g.Mg + co_rel0;
    const int m_begin = piece * a.per;
    const int m_end = min(a.M, m_begin + a.per);
    const int steps = a.per / (4 * kStepPx);          // steps of each wave

    const uint32_t x_bytes = static_cast<uint32_t>(g.N) * static_cast<uint32_t>(g.H * g.W) *
                             static_cast<uint32_t>(g.C) * 2u;
    const uint32_t dy_bytes = static_cast<uint32_t>(a.M) * static_cast<uint32_t>(g.CO) * 2u;
    const uint32x4_t xr = dma_rsrc(a.x, x_bytes);
    const uint32x4_t dyr = dma_rsrc(a.dy, dy_bytes);

    // Staging roles.  dy load j (0, 1) of a lane fills stage position
    // 64 j + lane: row rd[j] = 8 j + lane / 8, holding co unit
    // (lane % 8) ^ swz_dy(row).  A load j (0..3) fills A position 64 j + lane:
    // row ra[j] = 4 j + lane / 16, holding k unit (lane % 16) ^ swz_a(row),
    // i.e. tap (kh, kw) and channels c .. c + 7 of that tap.
    int rd[2], ra[4];
    uint32_t dy_co[2];  // byte offset of the lane's co unit, or kOutside
    uint32_t a_ch[4];   // byte offset of the lane's channels within a pixel, or kOutside
    int a_dh[4], a_dw[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        rd[j] = 8 * j + lane / 8;
        const int u = (lane % 8) ^ swz_dy(rd[j]);
        dy_co[j] = co_rel0 + 8 * u < g.Mg ? static_cast<uint32_t>(co0 + 8 * u) * 2u : kOutside;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ra[j] = 4 * j + lane / 16;
        const int u = (lane % 16) ^ swz_a(ra[j]);
        const int k = k0 + 8 * u;
        const int tap = static_cast<int>(fdiv(static_cast<uint32_t>(k), a.div_cg));
        const int c = k - tap * g.Cg;
        const int kh = static_cast<int>(fdiv(static_cast<uint32_t>(tap), a.div_kw));
        const int kw = tap - kh * g.KW;
        a_ch[j] = k < a.Ktot ? static_cast<uint32_t>(grp * g.Cg + c) * 2u : kOutside;
        a_dh[j] = kh * g.dh - g.ph;
        a_dw[j] = kw * g.dw - g.pw;
    }
    // Pixel bookkeeping, advanced by one wave step (4 kStepPx pixels) per
    // issue: a dy row's offset just grows by that many pixels; an A row keeps
    // its pixel as (n, oh, ow) digits and adds the step's digits with carries,
    // so the loop does no division.
    constexpr int kAdvance = 4 * kStepPx;
    int dm[2];
    uint32_t dy_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        dm[j] = m_begin + wave * kStepPx + rd[j];
        dy_off[j] = static_cast<uint32_t>(dm[j]) * static_cast<uint32_t>(g.CO) * 2u + dy_co[j];
    }
    int am[4], an[4], aoh[4], aow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        am[j] = m_begin + wave * kStepPx + ra[j];
        const uint32_t mm = static_cast<uint32_t>(min(am[j], a.M - 1));
        const uint32_t nohr = fdiv(mm, a.div_ow);
        aow[j] = static_cast<int>(mm - nohr * g.OW);
        an[j] = static_cast<int>(fdiv(nohr, a.div_oh));
        aoh[j] = static_cast<int>(nohr) - an[j] * g.OH;
    }
    const uint32_t dy_step = static_cast<uint32_t>(kAdvance) * static_cast<uint32_t>(g.CO) * 2u;
    const uint32_t row_bytes = static_cast<uint32_t>(g.W) * static_cast<uint32_t>(g.C) * 2u;
    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * 2u;
    // Issues the loads of this wave's next step into ring stage `st`; `live`
    // is false for the steps past the wave's last (they load zeros, which
    // keeps the count of loads in flight fixed).  Pixels past the piece load
    // zeros too.
    auto issue = [&](bool live, int st) __attribute__((always_inline)) {
        uint4* const base = ring + st * kStageUnits;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const bool in = live && dm[j] < m_end && dy_co[j] != kOutside;
            dma16(dyr, in ? dy_off[j] : kOutside, lds_addr(base + 64 * j));
            dm[j] += kAdvance;
            dy_off[j] += dy_step;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ih = aoh[j] * g.sh + a_dh[j];
            const int iw = aow[j] * g.sw + a_dw[j];
            const bool in = live && am[j] < m_end && a_ch[j] != kOutside &&
                            static_cast<unsigned>(ih) < static_cast<unsigned>(g.H) &&
                            static_cast<unsigned>(iw) < static_cast<unsigned>(g.W);
            const uint32_t off = static_cast<uint32_t>(an[j] * g.H + ih) * row_bytes +
                                 static_cast<uint32_t>(iw) * pix_bytes + a_ch[j];
            dma16(xr, in ? off : kOutside, lds_addr(base + kDyUnits + 64 * j));
            am[j] += kAdvance;
            aow[j] += a.d_ow;
            const int c1 = aow[j] >= g.OW;
            aow[j] -= c1 ? g.OW : 0;
            aoh[j] += a.d_oh + c1;
            const int c2 = aoh[j] >= g.OH;
            aoh[j] -= c2 ? g.OH : 0;
            an[j] += a.d_n + c2;
        }
    };

    // Transposed-read byte offsets within a stage.  Lane (group g4, index
    // s16) reads rows 8 (g4 / 2) + 4 h + s16 / 4 (h = 0, 1: the lane's eight
    // pixels) at columns 16 (g4 % 2) + 4 (s16 % 4) of a 32-column tile.
    const int g4 = lane >> 4, s16 = lane & 15;
    int tr_dy[2][2], tr_a[4][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 8 * (g4 >> 1) + 4 * h + (s16 >> 2);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int col = 32 * i + 16 * (g4 & 1) + 4 * (s16 & 3);  // co within the tile
            tr_dy[i][h] = row * 128 + (((col >> 3) ^ swz_dy(row)) << 4) + (col & 7) * 2;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = 32 * i + 16 * (g4 & 1) + 4 * (s16 & 3);  // k within the tile
            tr_a[i][h] = kDyUnits * 16 + row * 256 + (((col >> 3) ^ swz_a(row)) << 4) + (col & 7) * 2;
        }
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    issue(0 < steps, 0);
    issue(1 < steps, 1);
    issue(2 < steps, 2);
    int st = 0;
    for (int t = 0; t < steps; ++t) {
        wait_vm<2 * kLoadsPerStep>();  // step t has landed (steps t+1, t+2 may be in flight)
        asm volatile("" ::: "memory");
        const __attribute__((address_space(3))) char* sb =
            (const __attribute__((address_space(3))) char*)(ring + st * kStageUnits);
        bf16x8 fa[2], fb[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sb + tr_dy[i][0]));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sb + tr_dy[i][1]));
            fa[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sb + tr_a[i][0]));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sb + tr_a[i][1]));
            fb[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        // The first four MFMAs, then the refill of this stage (once this
        // wave's reads of it have returned) with its address arithmetic, then
        // the other four: the vector ALU work of the refill runs while the
        // matrix core works through the first four.
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0], fb[j], acc[0][j], 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        issue(t + 3 < steps, st);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1], fb[j], acc[1][j], 0, 0, 0);
        st = st == kStages - 1 ? 0 : st + 1;
    }
    wait_vm<0>();
    __syncthreads();  // every wave is done with its ring

    // Sum the four waves' accumulators: waves 2, 3 hand theirs to waves 0, 1,
    // then wave 1 to wave 0.  Layout in LDS is register-major (register i of
    // lane l at float 64 i + l), the same in every wave.
    float* const xf = reinterpret_cast<float*>(lds);
    constexpr int kAccFloats = 2 * 4 * 16 * 64;  // 32 KiB per wave
    auto put = [&](float* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) dst[((i * 4 + j) * 16 + v) * 64 + lane] = acc[i][j][v];
    };
    auto add = [&](const float* src) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] += src[((i * 4 + j) * 16 + v) * 64 + lane];
    };
    if (wave >= 2) put(xf + (wave - 2) * kAccFloats);
    __syncthreads();
    if (wave < 2) add(xf + wave * kAccFloats);
    __syncthreads();
    if (wave == 1) put(xf);
    __syncthreads();
    // Wave 0 finishes the sum and lays the tile out as [co][k] fp32 rows.
    if (wave == 0) {
        add(xf);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): its reads returned before its writes below
        const int col = lane & 31, q = lane >> 5;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int co = 32 * i + 8 * (v / 4) + 4 * q + (v % 4);
                    const int k = 32 * j + col;
                    xf[co * kKTile + k] = acc[i][j][v];
                }
    }
    __syncthreads();
    // Every thread writes 16-byte pieces of the tile's rows into the piece's
    // slice of the workspace (laid out like dw: [co][Ktot]).
    float* const slice = a.part + static_cast<int64_t>(piece) * g.CO * a.Ktot;
#pragma unroll
    for (int r = 0; r < kCoTile * kKTile / 4 / 256; ++r) {
        const int idx = r * 256 + tid;
        const int co = idx / (kKTile / 4), k4 = idx % (kKTile / 4);
        const int k = k0 + 4 * k4;
        if (co_rel0 + co < g.Mg && k < a.Ktot) {
            const float4 v = reinterpret_cast<const float4*>(xf)[co * (kKTile / 4) + k4];
            *reinterpret_cast<float4*>(slice + static_cast<int64_t>(co0 + co) * a.Ktot + k) = v;
        }
    }
}

}  // namespace

bool can_dw_igemm(const Geom& g, int dtype)
{
    if (dtype != 1 || !g.nhwc || !g.aligned16) return false;
    if (g.Cg % 8 != 0 || g.Mg % 8 != 0 || g.C % 8 != 0 || g.CO % 8 != 0) return false;
    const int64_t lim = int64_t(1) << 31;
    const int64_t x_bytes = static_cast<int64_t>(g.N) * g.H * g.W * g.C * 2;
    const int64_t dy_bytes = static_cast<int64_t>(g.N) * g.OH * g.OW * g.CO * 2;
    return x_bytes < lim && dy_bytes < lim;
}

// Pieces of the MFMA path: about two workgroups per CU over all tiles, each
// piece a whole number of four-wave steps.
DwPlan plan_dw_igemm(const Geom& g, int cus)
{
    DwPlan p{};
    const int64_t Ktot = static_cast<int64_t>(g.KH) * g.KW * g.Cg;
    const int64_t tiles = (Ktot + kKTile - 1) / kKTile * ((g.Mg + kCoTile - 1) / kCoTile) * g.G;
    const int64_t M = static_cast<int64_t>(g.N) * g.OH * g.OW;
    const int64_t quantum = 4 * kStepPx;
    int64_t S = std::max<int64_t>(1, (cus + tiles - 1) / tiles);
    S = std::min<int64_t>(S, std::max<int64_t>(1, (M + quantum - 1) / quantum));
    p.per = ((M + S - 1) / S + quantum - 1) / quantum * quantum;
    p.pieces = static_cast<int>((M + p.per - 1) / p.per);
    p.workspace = static_cast<size_t>(p.pieces) * static_cast<size_t>(g.CO) * static_cast<size_t>(Ktot) * sizeof(float);
    return p;
}

hipError_t launch_dw_igemm(const void* x, const void* dy, void* dw, void* workspace, const Geom& g,
                           int cus, hipStream_t s)
{
    const DwPlan p = plan_dw_igemm(g, cus);
    DwArgs a{};
    a.x = static_cast<const bf16_t*>(x);
    a.dy = static_cast<const bf16_t*>(dy);
    a.part = static_cast<float*>(workspace);
    a.g = g;
    a.Ktot = g.KH * g.KW * g.Cg;
    a.k_tiles = (a.Ktot + kKTile - 1) / kKTile;
    a.co_tiles = (g.Mg + kCoTile - 1) / kCoTile;
    a.tiles = a.k_tiles * a.co_tiles * g.G;
    a.pieces = p.pieces;
    a.per = static_cast<int>(p.per);
    a.M = g.N * g.OH * g.OW;
    a.div_ow = make_fastdiv(static_cast<uint32_t>(g.OW));
    a.div_oh = make_fastdiv(static_cast<uint32_t>(g.OH));
    a.div_cg = make_fastdiv(static_cast<uint32_t>(g.Cg));
    a.div_kw = make_fastdiv(static_cast<uint32_t>(g.KW));
    const int adv = 4 * kStepPx;
    a.d_ow = adv % g.OW;
    a.d_oh = (adv / g.OW) % g.OH;
    a.d_n = adv / (g.OW * g.OH);
    const int64_t blocks = static_cast<int64_t>(a.tiles) * p.pieces;
    const int64_t wn = static_cast<int64_t>(g.CO) * a.Ktot;
    const ArmedEvents armed = armed_events();
    armed_events() = ArmedEvents{armed.start, nullptr};
    hipError_t e = launch(dw_igemm_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    armed_events() = ArmedEvents{nullptr, armed.stop};
    if (e != hipSuccess) {
        armed_events() = ArmedEvents{nullptr, nullptr};
        return e;
    }
    return launch_dw_reduce(a.part, dw, wn, p.pieces, 1, s);
}

}  // namespace convmi
