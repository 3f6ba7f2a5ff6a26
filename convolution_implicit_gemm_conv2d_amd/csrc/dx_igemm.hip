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
// exactly once.  The same sum is the transposed convolution of the oarust
// page (`conv_transpose_2d`); its per-channel bias is added in the epilogue.
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
// MI355X design.  A workgroup computes 256 phase pixels x 128 input channels
// with four waves in a 2 x 2 arrangement, each 128 pixels x 64 channels =
// 4 x 2 tiles of v_mfma_f32_32x32x16_bf16.  The K loop runs over (tap,
// 32-channel chunk of co) through an LDS ring of 72 KiB (so two workgroups
// share a CU and hide each other's waits) filled only by buffer-to-LDS loads
// (zero outside dy and outside the weight): three stages for full-height
// tiles, four for half-height ones, so two or three chunks are in flight
// while one is multiplied; the loads of a chunk are issued
// between the MFMAs of the one before, and there is one workgroup barrier
// per chunk.  The weight block is staged as it is stored, [co][ci] rows, and
// the MFMA's weight operand (8 consecutive co of one ci per lane) is read
// with the gfx950 LDS transpose read (ds_read_b64_tr_b16): within each
// 16-lane group, lane j's element k comes from element j mod 4 of the
// 8-byte chunk that lane 4k + j/4 addressed.  LDS rows keep their 16-byte
// units XOR-swizzled so both the pixel reads and the transposed weight reads
// are bank-conflict free.  The dispatch order pairs the tiles of the phases
// with the most taps with those with the fewest on one CU.  The dx tile is
// restaged through LDS and written as whole pixel rows.
#include "kernels.hpp"

#include <algorithm>
#include <type_traits>
#include <vector>

namespace convmi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBMmax = 256;     // phase pixels per workgroup: 256, or 128 for phases with many taps
constexpr int kBN = 128;        // input channels per workgroup
constexpr int kBK = 32;         // output channels per K chunk
constexpr int kDUnits = kBK / 8;   // 16-byte units per staged dy row (one pixel)
constexpr int kWUnits = kBN / 8;   // 16-byte units per staged weight row (one co)
constexpr int kWLoads = kBK * kWUnits / kThreads;   // buffer-to-LDS weight loads per thread per chunk: 2
constexpr int kRingUnits = 3 * (kBK * kWUnits + kBMmax * kDUnits);  // three stages of the largest tile: 72 KiB
constexpr int kMaxPhases = 16;   // stride phases (sh * sw)
constexpr int kMaxSegs = 2 * kMaxPhases;
constexpr int kMaxTaps = 128;

struct Phase {
    int rh, rw;        // dx row / column residue of the phase
    int A, B;          // phase grid extent: rows a, columns b
    int tap_begin, ntaps;
    int bm;            // pixels per tile: 256, or 128 (more, shorter tiles) when the phase has many taps
    int m_tiles;       // pixel tiles, over the whole batch
    FastDiv div_ab;    // by A * B: phase pixel -> image
    FastDiv div_b;     // by B: pixel within the image -> phase row
};

// A run of consecutive workgroups that take consecutive tiles of one phase
// (tile = pixel tile, channel tile, group, pixel tile fastest).
struct Seg {
    int phase;
    int tile0;         // first tile of the run
    int block_begin;   // first workgroup of the run (a multiple of 8)
    int count;         // tiles in the run; workgroups after them up to the next run are idle
};

struct DxArgs {
    const bf16_t* dy;
    const bf16_t* w;
    const bf16_t* bias;  // per input channel, or null (zero)
    bf16_t* dx;
    Geom g;
    int nsegs;
    int n_tiles;       // channel tiles per group: ceil(Cg / kBN)
    int co_chunks;     // ceil(Mg / kBK)
    Phase ph[kMaxPhases];
    Seg seg[kMaxSegs];
    int tap[kMaxTaps];  // packed (kh, kw, dlt_h + 128, dlt_w + 128), one byte each
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// dy rows (4 units, 64 bytes): unit u of row r sits at position u ^ swz_d(r),
// so any 16 consecutive rows read at one unit cover all 64 banks.
__device__ __forceinline__ int swz_d(int r) { return (r >> 2) & 3; }
// Weight rows (16 units, 256 bytes): unit u of row r sits at u ^ swz_w(r).
// A transposed read touches 4 consecutive rows x 4 units per half wave and
// 4 rows x 2 units per quarter wave; this map sends both to distinct banks.
__device__ __forceinline__ int swz_w(int r) { return ((r & 3) << 2) ^ (r & 2); }


// One output tile: BM phase pixels x kBN input channels of phase P; `rest`
// is the tile's index within the phase (pixel tile fastest).  Four waves in
// a 2 x 2 arrangement, each BM/2 pixels x 64 channels = (BM/64) x 2 tiles of
// v_mfma_f32_32x32x16_bf16.
template <int BM, int NS>
__device__ __forceinline__ void dx_tile(const DxArgs& a, uint4* ring, const Phase& P, int rest)
{
    constexpr int kDyLoads = BM * kDUnits / kThreads;  // buffer-to-LDS dy loads per thread per chunk
    constexpr int kStage = kBK * kWUnits + BM * kDUnits;  // 16-byte units per pipeline stage
    constexpr int JT = BM / 64;                          // 32-pixel tiles per wave
    static_assert(NS >= 3 && NS * kStage <= kRingUnits, "the stages fit in the ring");
    const Geom& g = a.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int q = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;  // this wave's pixel half / 64-channel half

    int mt = rest % P.m_tiles;
    rest /= P.m_tiles;
    if (BM == 128) {
        // Half-height tiles 2r, 2r + 1 of 256-pixel region r sit at positions
        // 16k + x and 16k + 8 + x (r = 8k + x), so that both run on the XCD
        // that runs region r of every other phase (workgroup mod 8).
        const int full = P.m_tiles / 16 * 16;
        if (mt < full) mt = (mt / 16) * 16 + 2 * (mt % 8) + ((mt / 8) & 1);
    }
    const int nt = rest % a.n_tiles;
    const int grp = rest / a.n_tiles;
    const uint32_t per = static_cast<uint32_t>(P.A) * P.B;
    const uint32_t Mp = static_cast<uint32_t>(g.N) * per;  // pixels of the phase (< 2^30)
    const uint32_t m0 = static_cast<uint32_t>(mt) * BM;
    const int ci_rel0 = nt * kBN;                // first channel of the tile within the group
    const int ci0 = grp * g.Cg + ci_rel0;
    const int co_begin = grp * g.Mg;

    const uint32_t dy_bytes = static_cast<uint32_t>(g.N) * static_cast<uint32_t>(g.OH * g.OW) *
                              static_cast<uint32_t>(g.CO) * 2u;
    const uint32x4_t dyr = dma_rsrc(a.dy, dy_bytes);
    const int taps_all = g.KH * g.KW;
    const uint32_t w_bytes = static_cast<uint32_t>(g.CO) * static_cast<uint32_t>(taps_all * g.Cg) * 2u;
    const uint32x4_t wr = dma_rsrc(a.w, w_bytes);

    // Staging roles.  dy load i of a thread fills position (i*256 + tid) of
    // the stage: pixel row r = that / 8, position that % 8, holding unit
    // u = position ^ swz_d(r).  Its pixel is decoded once: dy_base is the
    // byte offset of dy[n, a, b, co_begin + 8u] (the tap's shift and the
    // chunk's channels are added per chunk) and (dy_a, dy_b) the phase row
    // and column, which decide whether a tap's dy pixel exists.
    uint32_t dy_base[kDyLoads];
    int dy_a[kDyLoads], dy_b[kDyLoads], dy_c[kDyLoads];
#pragma unroll
    for (int i = 0; i < kDyLoads; ++i) {
        const int L = i * kThreads + tid;
        const int r = L / kDUnits;
        const int u = (L % kDUnits) ^ swz_d(r);
        const uint32_t m = m0 + r;
        const uint32_t n = fdiv(m, P.div_ab);
        const uint32_t rr = m - n * per;
        const uint32_t ar = fdiv(rr, P.div_b);
        const bool ok = m < Mp;
        dy_a[i] = ok ? static_cast<int>(ar) : -(1 << 29);  // no tap brings it in range
        dy_b[i] = static_cast<int>(rr - ar * P.B);
        dy_c[i] = u * 8;
        dy_base[i] = (((n * g.OH + ar) * g.OW + dy_b[i]) * g.CO + co_begin + u * 8) * 2u;
    }
    // Weight load i fills position (i*256 + tid): co row w_row, unit u;
    // w_base is the byte offset of w[co_begin + w_row, tap 0, ci_rel0 + 8u].
    uint32_t w_base[kWLoads];
    int w_row[kWLoads];
    bool w_ci_ok[kWLoads];
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) {
        const int L = i * kThreads + tid;
        w_row[i] = L / kWUnits;
        const int u = (L % kWUnits) ^ swz_w(w_row[i]);
        w_ci_ok[i] = ci_rel0 + u * 8 < g.Cg;
        w_base[i] = (static_cast<uint32_t>(co_begin + w_row[i]) * taps_all * g.Cg + ci_rel0 + u * 8) * 2u;
    }

    // The tile's bias (the transposed convolution's; none for dx): this
    // lane's channels wn*64 + 32i + 8v + 4q + {0..3}, loaded before the
    // pipeline's loads so that its latency hides behind the K loop.  A null
    // bias is a resource of zero bytes, and channels past C read zero;
    // channels of the next group are read but belong to outputs that are
    // not stored.
    const rsrc_t br = make_rsrc(a.bias, a.bias ? static_cast<uint32_t>(g.C) * 2u : 0u);
    uint2 braw[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            braw[i][v] = __builtin_bit_cast(
                uint2, __builtin_amdgcn_raw_buffer_load_b64(
                           br, static_cast<uint32_t>(ci0 + wn * 64 + i * 32 + v * 8 + q * 4) * 2u, 0, 0));

    const int nchunks = P.ntaps * a.co_chunks;
    // Per-chunk uniform values.  A chunk past the last (c >= nchunks) is
    // issued too, as loads that only write zeros, so that every step has the
    // same number of loads in flight and one fixed wait count covers them.
    struct Chunk {
        int dh, dw;        // tap shift in dy rows / columns
        int co_c;          // first output channel of the chunk within the group
        uint32_t dy_delta; // bytes: tap shift + chunk channels
        uint32_t w_delta;  // bytes: chunk channels + tap
    };
    // A cursor over the chunks: chunk c as its (tap t, co chunk cc), advanced
    // one chunk at a time, so that the loop does no division, and the tap's
    // packed entry, read when the cursor reaches the tap (at the end of a
    // step) rather than after the next step's barrier, where the wait for
    // the read would hold up that step's first fragment reads.  Past the last
    // tap the entry is zero (such chunks load nothing).
    struct Cursor {
        int c, t, cc, packed;
    };
    auto tap_entry = [&](int t) __attribute__((always_inline)) {
        return t < P.ntaps ? a.tap[P.tap_begin + t] : 0;
    };
    auto advance = [&](Cursor& u) __attribute__((always_inline)) {
        ++u.c;
        if (++u.cc == a.co_chunks) {
            u.cc = 0;
            ++u.t;
            u.packed = tap_entry(u.t);
        }
    };
    auto chunk = [&](const Cursor& u) __attribute__((always_inline)) {
        Chunk k;
        const bool live = u.c < nchunks;
        k.co_c = live ? u.cc * kBK : g.Mg;  // g.Mg: outside every chunk
        const int packed = u.packed;
        const int kh = packed & 0xff;
        const int kw = (packed >> 8) & 0xff;
        k.dh = live ? ((packed >> 16) & 0xff) - 128 : (1 << 30);
        k.dw = ((packed >> 24) & 0xff) - 128;
        // Modulo 2^32: a negative shift wraps, and the sum with a slot's base
        // is exact whenever the load is in range.
        k.dy_delta = ((static_cast<uint32_t>(k.dh) * static_cast<uint32_t>(g.OW) + static_cast<uint32_t>(k.dw)) *
                          static_cast<uint32_t>(g.CO) +
                      static_cast<uint32_t>(k.co_c)) *
                     2u;
        k.w_delta = (static_cast<uint32_t>(k.co_c) * taps_all + kh * g.KW + kw) * g.Cg * 2u;
        return k;
    };
    // One 16-byte buffer-to-LDS load of each kind; a wave load fills 1 KiB of
    // LDS, lane-consecutive.
    auto issue_w = [&](const Chunk& k, uint4* wst, int i) __attribute__((always_inline)) {
        const bool in = w_ci_ok[i] && w_row[i] < g.Mg - k.co_c;
        dma16(wr, in ? w_base[i] + k.w_delta : kOutside, lds_addr(wst + i * kThreads + wave * 64));
    };
    auto issue_dy = [&](const Chunk& k, uint4* dst, int i) __attribute__((always_inline)) {
        const bool in = static_cast<unsigned>(dy_a[i] + k.dh) < static_cast<unsigned>(g.OH) &&
                        static_cast<unsigned>(dy_b[i] + k.dw) < static_cast<unsigned>(g.OW) &&
                        dy_c[i] < g.Mg - k.co_c;
        dma16(dyr, in ? dy_base[i] + k.dy_delta : kOutside, lds_addr(dst + i * kThreads + wave * 64));
    };
    constexpr int kLoadsPerChunk = kWLoads + kDyLoads;
    constexpr int KSC = kBK / 16;  // k steps per chunk
    static_assert(kWLoads % KSC == 0 && kDyLoads % KSC == 0, "loads are spread evenly over the k steps");

    f32x16 acc[2][JT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Transposed-read addresses (bytes within a weight stage) for weight
    // fragment i, k step ks, half h: lane (group g4, index s) points at co
    // row 16ks + 8(g4/2) + 4h + s/4, channels 4(s%4) .. +3 of the 16-channel
    // run 32i + 16(g4%2) of this wave's 64 channels.
    const int g4 = lane >> 4, s16 = lane & 15;
    int tr_off[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 8 * (g4 >> 1) + 4 * h + (s16 >> 2);
            const int ch = wn * 64 + i * 32 + 16 * (g4 & 1) + 4 * (s16 & 3);
            tr_off[i][h] = row * (kWUnits * 16) + (((ch >> 3) ^ swz_w(row)) << 4) + (ch & 7) * 2;
        }
    // Fragments of one k step: two weight fragments (channels) and JT dy
    // fragments (pixels).  compute() reads step ks + 1 while step ks
    // multiplies, so the LDS latency hides behind the MFMAs.
    struct Frags {
        bf16x8 a[2], b[JT];
    };
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    auto read_frags = [&](Frags& f, const uint4* wt, const uint4* dt, int ks) __attribute__((always_inline)) {
        const __attribute__((address_space(3))) char* wb = (const __attribute__((address_space(3))) char*)wt;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            // Rows 16ks.. of the stage: the swizzle of row 16ks + r equals that of r.
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(wb + tr_off[i][0] + ks * 16 * kWUnits * 16));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(wb + tr_off[i][1] + ks * 16 * kWUnits * 16));
            f.a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        const int u = ks * 2 + q;
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int row = wm * (BM / 2) + j * 32 + col;  // phase pixel within the tile
            f.b[j] = as_bf16x8(dt[row * kDUnits + (u ^ swz_d(row))]);
        }
    };
    // Multiplies the chunk in (wt, dt) and, between its MFMAs, issues the
    // loads of chunk k into (wst, dst), an equal share per k step, so the
    // load traffic is spread over the chunk.
    auto compute = [&](const uint4* wt, const uint4* dt, const Chunk& k, uint4* wst, uint4* dst)
                       __attribute__((always_inline)) {
        Frags f[2];
        read_frags(f[0], wt, dt, 0);
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            if (ks + 1 < KSC) read_frags(f[(ks + 1) & 1], wt, dt, ks + 1);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int j = 0; j < JT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks & 1].a[i], f[ks & 1].b[j],
                                                                        acc[i][j], 0, 0, 0);
                if (i == 0) {
#pragma unroll
                    for (int d = 0; d < kWLoads / KSC; ++d) issue_w(k, wst, ks * (kWLoads / KSC) + d);
                } else {
#pragma unroll
                    for (int d = 0; d < kDyLoads / KSC; ++d) issue_dy(k, dst, ks * (kDyLoads / KSC) + d);
                }
            }
        }
    };
    // Chunk c: wait for this thread's loads of chunk c (those of chunks
    // c + 1 .. c + NS - 2 may still be in flight), synchronise (every wave's
    // loads of chunk c have landed and every wave is done with chunk c - 1,
    // whose stage is refilled next), issue chunk c + NS - 1, multiply chunk c.
    Cursor pre{0, 0, 0, tap_entry(0)};  // the next chunk to issue
    auto step = [&](const uint4* cur, uint4* next) __attribute__((always_inline)) {
        wait_vm<(NS - 2) * kLoadsPerChunk>();
        barrier_no_fence();
        compute(cur, cur + kBK * kWUnits, chunk(pre), next, next + kBK * kWUnits);
        advance(pre);
    };
    auto issue = [&](uint4* st) __attribute__((always_inline)) {
        const Chunk k = chunk(pre);
        advance(pre);
#pragma unroll
        for (int i = 0; i < kWLoads; ++i) issue_w(k, st, i);
#pragma unroll
        for (int i = 0; i < kDyLoads; ++i) issue_dy(k, st + kBK * kWUnits, i);
    };
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) issue(ring + i * kStage);
    for (int c = 0; c < nchunks; c += NS) {
#pragma unroll
        for (int i = 0; i < NS; ++i)
            if (c + i < nchunks) step(ring + i * kStage, ring + ((i + NS - 1) % NS) * kStage);
    }
    wait_vm<0>();     // the zero-filling loads past the last chunk have landed
    __syncthreads();  // and every wave is done reading the stages

    // Epilogue.  Lane holds channels wn*64 + 32i + 8v + 4q + {0..3} of phase
    // pixel wm*BM/2 + 32j + col in acc[i][j][4v .. 4v+3].  Stage the bf16 tile
    // as pixel rows of 16 units in the ring (unit u of pixel p at position
    // u ^ (p & 15)), then write each pixel's channels as 16-byte units.  The
    // stores cover whole cache lines and dx is not read back, so they carry
    // the non-temporal hint.
    static_assert(BM * kBN / 8 <= NS * kStage, "the output tile fits in the ring");
    // The bias is added in fp32 before the single rounding; without one
    // (dx) a separate path rounds the sums as they are.
    float bsum[2][4][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint2 bv = braw[i][v];
            bsum[i][v][0] = __uint_as_float(bv.x << 16);
            bsum[i][v][1] = __uint_as_float(bv.x & 0xffff0000u);
            bsum[i][v][2] = __uint_as_float(bv.y << 16);
            bsum[i][v][3] = __uint_as_float(bv.y & 0xffff0000u);
        }
    uint4* my_half = ring + wm * (BM / 2) * 16;
    auto stage_out = [&](auto with_bias) __attribute__((always_inline)) {
        constexpr bool kBias = decltype(with_bias)::value;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < JT; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int p = j * 32 + col;  // pixel within this wave's half
                    const int ch = wn * 64 + i * 32 + v * 8 + q * 4;
                    const int u = ch >> 3;
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = kBias ? acc[i][j][4 * v + e] + bsum[i][v][e] : acc[i][j][4 * v + e];
                    uint2* unit = reinterpret_cast<uint2*>(my_half + p * 16 + (u ^ (p & 15)));
                    unit[(ch >> 2) & 1] = uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                }
    };
    if (a.bias)
        stage_out(std::true_type{});
    else
        stage_out(std::false_type{});
    __syncthreads();
    const uint32_t dx_bytes = static_cast<uint32_t>(g.N) * static_cast<uint32_t>(g.H * g.W) *
                              static_cast<uint32_t>(g.C) * 2u;
    const rsrc_t dxr = make_rsrc(a.dx, dx_bytes);
#pragma unroll
    for (int k = 0; k < (BM * kBN / 8) / kThreads; ++k) {
        const int idx = k * kThreads + tid;
        const int px = idx / (kBN / 8), u = idx % (kBN / 8);
        const uint32_t m = m0 + px;
        const uint32_t n = fdiv(m, P.div_ab);
        const uint32_t rr = m - n * per;
        const uint32_t ar = fdiv(rr, P.div_b), br = rr - ar * P.B;
        const uint32_t ih = ar * g.sh + P.rh, iw = br * g.sw + P.rw;
        const bool in = m < Mp && ci_rel0 + u * 8 < g.Cg;
        const uint32_t off = in ? ((static_cast<uint32_t>(n * g.H + ih) * g.W + iw) * g.C + ci0 + u * 8) * 2u
                                : kOutside;
        buffer_store16_nt(dxr, off, ring[px * 16 + (u ^ (px & 15))]);
    }
}

__global__ __launch_bounds__(kThreads, 2) void dx_igemm_kernel(DxArgs a)
{
    // Three or four pipeline stages, each a weight block [kBK co][kWUnits]
    // followed by a dy block [BM px][kDUnits]; 72 KiB in all, so two workgroups share a
    // CU and each one's waits, prologue and epilogue hide behind the other's
    // MFMAs.  The loads into it are untracked by the compiler (dma16), so one
    // array serves all stages and, at the end, the output staging.
    __shared__ uint4 ring[kRingUnits];
    // Workgroup -> phase and tile.
    int sidx = 0;
    while (sidx + 1 < a.nsegs && static_cast<int>(blockIdx.x) >= a.seg[sidx + 1].block_begin) ++sidx;
    const Seg S = a.seg[sidx];
    if (static_cast<int>(blockIdx.x) >= S.block_begin + S.count) return;  // alignment padding
    const Phase P = a.ph[S.phase];
    const int rest = S.tile0 + (static_cast<int>(blockIdx.x) - S.block_begin);
    // Half-height tiles take four stages (64 KiB: three chunks in flight),
    // full-height ones three (72 KiB).
    if (P.bm == 128)
        dx_tile<128, 4>(a, ring, P, rest);
    else
        dx_tile<256, 3>(a, ring, P, rest);
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
    a.g = g;
    a.n_tiles = (g.Cg + kBN - 1) / kBN;
    a.co_chunks = (g.Mg + kBK - 1) / kBK;
    // Phases with more than twice the fewest taps get half-height tiles, so
    // that no workgroup carries much more work than the others.
    // (Phases no tap reaches take the full height; when no phase has a tap
    // the rule does not apply at all.)
    int64_t min_taps = 0;
    for (const Phase& p : phases)
        if (p.ntaps > 0) min_taps = min_taps == 0 ? p.ntaps : std::min<int64_t>(min_taps, p.ntaps);
    std::vector<int64_t> tiles(phases.size());
    int64_t total = 0;
    for (size_t i = 0; i < phases.size(); ++i) {
        Phase& p = phases[i];
        const int64_t Mp = static_cast<int64_t>(g.N) * p.A * p.B;
        p.bm = min_taps > 0 && p.ntaps > 2 * min_taps ? 128 : 256;
        p.m_tiles = static_cast<int>((Mp + p.bm - 1) / p.bm);
        p.div_ab = make_fastdiv(static_cast<uint32_t>(p.A) * p.B);
        p.div_b = make_fastdiv(static_cast<uint32_t>(p.B));
        a.ph[i] = p;
        tiles[i] = static_cast<int64_t>(p.m_tiles) * a.n_tiles * g.G;
        total += tiles[i];
    }
    if (total <= 0 || total >= (int64_t(1) << 31)) return false;
    // Dispatch order.  The first `first_round` workgroups go one per CU; a
    // CU's second workgroup is the one `first_round` places later.  So the
    // first round takes the tiles with the most work (taps x pixels),
    // longest first, and the rest follows shortest first: long tiles share a
    // CU with short ones.  Workgroup b runs on XCD b mod 8; every run starts
    // at a multiple of 8 workgroups and of 8 tiles, so region r (phase pixels
    // 256r ..) of every phase lands on XCD r mod 8, and that XCD's L2 serves
    // the dy rows all phases of the region read.
    std::vector<int> desc(phases.size());
    for (size_t i = 0; i < desc.size(); ++i) desc[i] = static_cast<int>(i);
    std::stable_sort(desc.begin(), desc.end(), [&](int x, int y) {
        return phases[x].ntaps * phases[x].bm > phases[y].ntaps * phases[y].bm;
    });
    const int64_t first_round = std::min<int64_t>(total, device_cu_count());
    std::vector<int64_t> taken(phases.size(), 0);
    a.nsegs = 0;
    int64_t b = 0;
    auto add_seg = [&](int ph, int64_t count) {
        if (count <= 0) return;
        b = (b + 7) / 8 * 8;
        a.seg[a.nsegs++] = Seg{ph, static_cast<int>(taken[ph]), static_cast<int>(b), static_cast<int>(count)};
        taken[ph] += count;
        b += count;
    };
    for (int ph : desc) {
        int64_t room = first_round - (b + 7) / 8 * 8;
        if (room < tiles[ph]) room = room / 8 * 8;  // a split leaves the rest starting at a multiple of 8
        add_seg(ph, std::min(tiles[ph], room));
    }
    for (auto it = desc.rbegin(); it != desc.rend(); ++it) add_seg(*it, tiles[*it] - taken[*it]);
    for (size_t i = 0; i < taps.size(); ++i) a.tap[i] = taps[i];
    if (b >= (int64_t(1) << 31)) return false;
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

hipError_t launch_dx_igemm(const void* dy, const void* w, const void* bias, void* dx, const Geom& g,
                           hipStream_t s)
{
    DxArgs a;
    int blocks = 0;
    if (!make_args(g, a, blocks)) return hipErrorInvalidValue;
    a.dy = static_cast<const bf16_t*>(dy);
    a.w = static_cast<const bf16_t*>(w);
    a.bias = static_cast<const bf16_t*>(bias);
    a.dx = static_cast<bf16_t*>(dx);
    return launch(dx_igemm_kernel, dim3(blocks), dim3(kThreads), 0, s, a);
}

}  // namespace convmi
