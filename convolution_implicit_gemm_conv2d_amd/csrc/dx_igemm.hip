// Input gradient (dx) of a convolution as a gather: one implicit GEMM per
// stride phase on the MFMA units.
//
// dx[n, ih, iw, ci] = sum over co of ci's group and taps (kh, kw) with
// th = ih + ph - kh*dh >= 0, th % sh == 0, th/sh < OH (and likewise for w) of
// dy[n, th/sh, tw/sw, co] * w[co, kh, kw, ci - g*Cg].  This is the adjoint of
// the forward (oarust 0.8.6 src/rs/ml/matrix/conv.rs, `conv_2d_backward`,
// which dispatches the input adjoint over input elements, and the
// statement in `conv_transpose_1d_backward` that a convolution's input
// adjoint is itself a convolution).  teeny-kernels 0.2.0
// src/nn/conv/conv2d.rs `conv2d_backward_dx` computes the same sum by
// scattering with atomics into a zeroed dx; here every dx element is written
// exactly once.
//
// Stride phases.  Split dx pixels by (ih mod sh, iw mod sw) = (rh, rw).  For a
// phase, the taps that reach it are fixed: kh with (rh + ph - kh*dh) a
// multiple of sh, and then th/sh = a + dlt_h for dx row ih = a*sh + rh with
// dlt_h = (rh + ph - kh*dh) / sh.  So per phase the gradient is a dense GEMM
//   dx_phase[m, ci] = sum_k A[m, k] * B[k, ci],  m = (n, a, b),
//   k = (tap of the phase, co),  A = dy gathered at (a + dlt_h, b + dlt_w),
//   B[(tap, co), ci] = w[co, kh, kw, ci],
// with no wasted multiplications (a zero-inserted dy would multiply by
// zeros sh*sw times over).  Phases no tap reaches are written as zeros.
//
// MI355X design.  A workgroup computes 128 phase pixels x 128 input channels
// with four waves in a 2 x 2 arrangement, each 64 x 64 = 2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16.  The K loop runs over (tap, 64-channel chunk of
// co) and is double buffered in LDS: while one chunk is multiplied, the next
// chunk's dy rows arrive by buffer-to-LDS loads (zero outside dy) and its
// weight block is loaded into registers.  The weight is stored co-major
// ([co][kh][kw][ci]) but the MFMA needs 8 consecutive co per lane, so each of
// 128 threads loads an 8 co x 8 ci block and transposes it in registers
// before writing it to LDS as [ci][co].  LDS rows keep their 16-byte units
// XOR-swizzled so fragment reads are bank-conflict free.  Workgroups of the
// phases with the most taps are dispatched first.  The dx tile is restaged
// through LDS and written as whole 256-byte pixel rows.
#include "kernels.hpp"

#include <algorithm>
#include <vector>

namespace convmi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBM = 128;        // phase pixels per workgroup
constexpr int kBN = 128;        // input channels per workgroup
constexpr int kBK = 64;         // output channels per K chunk
constexpr int kUnits = kBK / 8; // 16-byte units per staged row
constexpr int kMaxPhases = 64;
constexpr int kMaxTaps = 128;

struct Phase {
    int rh, rw;        // dx row / column residue of the phase
    int A, B;          // phase grid extent: rows a, columns b
    int tap_begin, ntaps;
    int block_begin;   // first workgroup of the phase
    int m_tiles;       // workgroups along the pixels, per image batch
};

struct DxArgs {
    const bf16_t* dy;
    const bf16_t* w;
    bf16_t* dx;
    Geom g;
    int nphases;
    int n_tiles;       // channel tiles per group: ceil(Cg / 128)
    int co_chunks;     // ceil(Mg / 64)
    Phase ph[kMaxPhases];
    int tap[kMaxTaps];  // packed (kh, kw, dlt_h + 128, dlt_w + 128), one byte each
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Unit u of staged row r lives at position u ^ swz(r): 16 consecutive rows
// cover all 16 bank groups for any fixed u.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(kThreads) void dx_igemm_kernel(DxArgs a)
{
    // Two pipeline stages, each a weight block [kBN ci][8 units] and a dy
    // block [kBM px][8 units].  They are separate objects so that the
    // compiler sees that a buffer-to-LDS load into one stage cannot alias a
    // read of the other (it would otherwise wait for the load first).
    __shared__ uint4 w_s0[kBN * kUnits], d_s0[kBM * kUnits];
    __shared__ uint4 w_s1[kBN * kUnits], d_s1[kBM * kUnits];
    const Geom& g = a.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int q = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;  // this wave's 64-pixel / 64-channel quarter

    // Workgroup -> phase, pixel tile, channel tile, group.
    int pidx = 0;
    while (pidx + 1 < a.nphases && static_cast<int>(blockIdx.x) >= a.ph[pidx + 1].block_begin) ++pidx;
    const Phase P = a.ph[pidx];
    int rest = blockIdx.x - P.block_begin;
    const int mt = rest % P.m_tiles;
    rest /= P.m_tiles;
    const int nt = rest % a.n_tiles;
    const int grp = rest / a.n_tiles;
    const int64_t Mp = static_cast<int64_t>(g.N) * P.A * P.B;  // pixels of the phase
    const int64_t m0 = static_cast<int64_t>(mt) * kBM;
    const int ci_rel0 = nt * kBN;                // first channel of the tile within the group
    const int ci0 = grp * g.Cg + ci_rel0;
    const int co_begin = grp * g.Mg;

    const uint32_t dy_bytes = static_cast<uint32_t>(g.N) * static_cast<uint32_t>(g.OH * g.OW) *
                              static_cast<uint32_t>(g.CO) * 2u;
    const rsrc_t dyr = make_rsrc(a.dy, dy_bytes);
    const uint32_t w_bytes = static_cast<uint32_t>(g.CO) * static_cast<uint32_t>(g.KH * g.KW * g.Cg) * 2u;
    const rsrc_t wr = make_rsrc(a.w, w_bytes);

    // Staging roles.  dy: 128 rows x 8 units = 16 wave loads, four per wave;
    // the slots a lane fills are fixed, so their pixels are decoded once.
    int dy_n[4], dy_a[4], dy_b[4], dy_pos_u[4];
    bool dy_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int L = (wave * 4 + i) * 64 + lane;  // slot = row * 8 + position
        const int r = L >> 3, pos = L & 7;
        dy_pos_u[i] = pos ^ swz(r);
        const int64_t m = m0 + r;
        dy_ok[i] = m < Mp;
        const int64_t mm = dy_ok[i] ? m : 0;
        const int64_t per = static_cast<int64_t>(P.A) * P.B;
        dy_n[i] = static_cast<int>(mm / per);
        const int rr = static_cast<int>(mm - dy_n[i] * per);
        dy_a[i] = rr / P.B;
        dy_b[i] = rr - dy_a[i] * P.B;
    }
    // Weights: threads 0..127 each own an 8 co x 8 ci block of the chunk.
    const bool w_role = tid < 128;
    const int cb = (tid >> 4) & 7;  // co group of 8 within the chunk
    const int ib = tid & 15;        // ci group of 8 within the tile

    const int nchunks = P.ntaps * a.co_chunks;
    auto chunk_tap = [&](int c, int& kh, int& kw, int& dh_, int& dw_, int& co_c) {
        const int t = c / a.co_chunks;
        co_c = (c - t * a.co_chunks) * kBK;
        const int packed = a.tap[P.tap_begin + t];
        kh = packed & 0xff;
        kw = (packed >> 8) & 0xff;
        dh_ = ((packed >> 16) & 0xff) - 128;
        dw_ = ((packed >> 24) & 0xff) - 128;
    };
    // Issues chunk c: dy rows by buffer-to-LDS loads into stage s, the
    // weight block into registers.
    auto issue = [&](int c, uint4* st, uint4 (&wv)[8]) {
        int kh, kw, dh_, dw_, co_c;
        chunk_tap(c, kh, kw, dh_, dw_, co_c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int oh = dy_a[i] + dh_, ow = dy_b[i] + dw_;
            const int co = co_begin + co_c + dy_pos_u[i] * 8;
            const bool in = dy_ok[i] && static_cast<unsigned>(oh) < static_cast<unsigned>(g.OH) &&
                            static_cast<unsigned>(ow) < static_cast<unsigned>(g.OW) &&
                            co_c + dy_pos_u[i] * 8 < g.Mg;
            const uint32_t off =
                ((static_cast<uint32_t>(dy_n[i] * g.OH + oh) * g.OW + ow) * g.CO + co) * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                dyr, (__attribute__((address_space(3))) void*)(st + (wave * 4 + i) * 64), 16,
                in ? off : kOutside, 0, 0, 0);
        }
        if (w_role) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int co_rel = co_c + cb * 8 + r;
                const int ci_rel = ci_rel0 + ib * 8;
                const bool in = co_rel < g.Mg && ci_rel < g.Cg;
                const uint32_t off =
                    ((static_cast<uint32_t>(co_begin + co_rel) * g.KH + kh) * g.KW + kw) * g.Cg * 2u +
                    static_cast<uint32_t>(ci_rel) * 2u;
                wv[r] = buffer_load16(wr, in ? off : kOutside);
            }
        }
    };
    // Writes the transposed weight block: LDS row ci = 8*ib + e holds the 8
    // values w[co = 8*cb + 0..7][ci] as unit cb.
    auto store_w = [&](uint4* st, const uint4 (&wv)[8]) {
        if (!w_role) return;
        uint32_t d[8][4];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            d[r][0] = wv[r].x; d[r][1] = wv[r].y; d[r][2] = wv[r].z; d[r][3] = wv[r].w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int dw = e >> 1;
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = d[2 * k][dw], hi = d[2 * k + 1][dw];
                o[k] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            const int row = ib * 8 + e;
            st[row * kUnits + (cb ^ swz(row))] = uint4{o[0], o[1], o[2], o[3]};
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    auto compute = [&](const uint4* wt, const uint4* dt) {
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int u = ks * 2 + q;
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wn * 64 + i * 32 + col;  // input channel within the tile
                fa[i] = as_bf16x8(wt[row * kUnits + (u ^ swz(row))]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = wm * 64 + j * 32 + col;  // phase pixel within the tile
                fb[j] = as_bf16x8(dt[row * kUnits + (u ^ swz(row))]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };
    // One K chunk: the next chunk's dy rows go to the other stage by
    // buffer-to-LDS loads and its weight block to registers while this
    // chunk is multiplied; then the weight block is transposed into the
    // other stage and the workgroup synchronises.
    uint4 wv[8];
    auto step = [&](int c, const uint4* wcur, const uint4* dcur, uint4* wnext, uint4* dnext) {
        const bool more = c + 1 < nchunks;
        if (more) issue(c + 1, dnext, wv);
        compute(wcur, dcur);
        if (more) {
            __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next chunk have landed
            store_w(wnext, wv);
        }
        __syncthreads();
    };
    if (nchunks > 0) {
        issue(0, d_s0, wv);
        __builtin_amdgcn_s_waitcnt(0);
        store_w(w_s0, wv);
        __syncthreads();
    }
    for (int c = 0; c < nchunks; c += 2) {
        step(c, w_s0, d_s0, w_s1, d_s1);
        if (c + 1 < nchunks) step(c + 1, w_s1, d_s1, w_s0, d_s0);
    }

    // Epilogue.  Lane holds channels wn*64 + 32i + 8v + 4q + {0..3} of phase
    // pixel wm*64 + 32j + col in acc[i][j][4v .. 4v+3].  Stage the bf16 tile
    // as pixel rows of 16 units (pixels 0..63 in one stage array, 64..127 in
    // another; unit u of pixel p at position u ^ (p & 15)), then write each
    // pixel's channels as 16-byte units.
    uint4* my_half = wm ? d_s0 : w_s0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int p = j * 32 + col;  // pixel within this wave's half
                const int ch = wn * 64 + i * 32 + v * 8 + q * 4;
                const int u = ch >> 3;
                uint2* unit = reinterpret_cast<uint2*>(my_half + p * 16 + (u ^ (p & 15)));
                unit[(ch >> 2) & 1] = uint2{pack_bf16x2(acc[i][j][4 * v + 0], acc[i][j][4 * v + 1]),
                                            pack_bf16x2(acc[i][j][4 * v + 2], acc[i][j][4 * v + 3])};
            }
    __syncthreads();
    const uint32_t dx_bytes = static_cast<uint32_t>(g.N) * static_cast<uint32_t>(g.H * g.W) *
                              static_cast<uint32_t>(g.C) * 2u;
    const rsrc_t dxr = make_rsrc(a.dx, dx_bytes);
#pragma unroll
    for (int k = 0; k < (kBM * kBN / 8) / kThreads; ++k) {
        const int idx = k * kThreads + tid;
        const int px = idx / (kBN / 8), u = idx - (idx / (kBN / 8)) * (kBN / 8);
        const int64_t m = m0 + px;
        const int ci_rel = ci_rel0 + u * 8;
        uint32_t off = kOutside;
        if (m < Mp && ci_rel < g.Cg) {
            const int64_t per = static_cast<int64_t>(P.A) * P.B;
            const int n = static_cast<int>(m / per);
            const int rr = static_cast<int>(m - n * per);
            const int ar = rr / P.B, br = rr - (rr / P.B) * P.B;
            const int ih = ar * g.sh + P.rh, iw = br * g.sw + P.rw;
            off = ((static_cast<uint32_t>(n * g.H + ih) * g.W + iw) * g.C + ci0 + u * 8) * 2u;
        }
        const int p = px & 63;
        const uint4* half = (px >> 6) ? d_s0 : w_s0;
        buffer_store16(dxr, off, half[p * 16 + (u ^ (p & 15))]);
    }
}


// Host plan: the phases, their taps and the workgroup layout.
bool make_args(const Geom& g, DxArgs& a, int& blocks)
{
    std::vector<Phase> phases;
    std::vector<int> taps;
    for (int rh = 0; rh < g.sh; ++rh)
        for (int rw = 0; rw < g.sw; ++rw) {
            Phase p{};
            p.rh = rh;
            p.rw = rw;
            p.A = rh < g.H ? (g.H - rh + g.sh - 1) / g.sh : 0;
            p.B = rw < g.W ? (g.W - rw + g.sw - 1) / g.sw : 0;
            if (p.A == 0 || p.B == 0) continue;
            p.tap_begin = static_cast<int>(taps.size());
            for (int kh = 0; kh < g.KH; ++kh) {
                const int th = rh + g.ph - kh * g.dh;
                if (((th % g.sh) + g.sh) % g.sh != 0) continue;
                for (int kw = 0; kw < g.KW; ++kw) {
                    const int tw = rw + g.pw - kw * g.dw;
                    if (((tw % g.sw) + g.sw) % g.sw != 0) continue;
                    const int dh_ = (th - ((th % g.sh) + g.sh) % g.sh) / g.sh;  // exact division
                    const int dw_ = (tw - ((tw % g.sw) + g.sw) % g.sw) / g.sw;
                    if (dh_ < -128 || dh_ > 127 || dw_ < -128 || dw_ > 127 || kh > 255 || kw > 255) return false;
                    taps.push_back(kh | (kw << 8) | ((dh_ + 128) << 16) | ((dw_ + 128) << 24));
                }
            }
            p.ntaps = static_cast<int>(taps.size()) - p.tap_begin;
            phases.push_back(p);
        }
    if (phases.size() > static_cast<size_t>(kMaxPhases) || taps.size() > static_cast<size_t>(kMaxTaps))
        return false;
    // Longest phases first, so that the short ones fill in behind them.
    std::stable_sort(phases.begin(), phases.end(),
                     [](const Phase& x, const Phase& y) { return x.ntaps > y.ntaps; });
    a.g = g;
    a.n_tiles = (g.Cg + kBN - 1) / kBN;
    a.co_chunks = (g.Mg + kBK - 1) / kBK;
    a.nphases = static_cast<int>(phases.size());
    int64_t b = 0;
    for (size_t i = 0; i < phases.size(); ++i) {
        Phase& p = phases[i];
        const int64_t Mp = static_cast<int64_t>(g.N) * p.A * p.B;
        p.m_tiles = static_cast<int>((Mp + kBM - 1) / kBM);
        p.block_begin = static_cast<int>(b);
        b += static_cast<int64_t>(p.m_tiles) * a.n_tiles * g.G;
        a.ph[i] = p;
    }
    for (size_t i = 0; i < taps.size(); ++i) a.tap[i] = taps[i];
    if (b <= 0 || b >= (int64_t(1) << 31)) return false;
    blocks = static_cast<int>(b);
    return true;
}

}  // namespace

bool can_dx_igemm(const Geom& g, int dtype)
{
    if (dtype != 1 || !g.nhwc || !g.aligned16) return false;
    if (g.Cg % 8 != 0 || g.Mg % 8 != 0 || g.C % 8 != 0 || g.CO % 8 != 0) return false;
    const int64_t dy_bytes = static_cast<int64_t>(g.N) * g.OH * g.OW * g.CO * 2;
    const int64_t dx_bytes = static_cast<int64_t>(g.N) * g.H * g.W * g.C * 2;
    const int64_t w_bytes = static_cast<int64_t>(g.CO) * g.KH * g.KW * g.Cg * 2;
    const int64_t lim = int64_t(1) << 31;
    if (dy_bytes >= lim || dx_bytes >= lim || w_bytes >= lim) return false;
    if (static_cast<int64_t>(g.sh) * g.sw > kMaxPhases || g.KH * g.KW > kMaxTaps) return false;
    DxArgs a;
    int blocks = 0;
    return make_args(g, a, blocks);
}

hipError_t launch_dx_igemm(const void* dy, const void* w, void* dx, const Geom& g, hipStream_t s)
{
    DxArgs a;
    int blocks = 0;
    if (!make_args(g, a, blocks)) return hipErrorInvalidValue;
    a.dy = static_cast<const bf16_t*>(dy);
    a.w = static_cast<const bf16_t*>(w);
    a.dx = static_cast<bf16_t*>(dx);
    return launch(dx_igemm_kernel, dim3(blocks), dim3(kThreads), 0, s, a);
}

}  // namespace convmi
