// Input gradient (dx) of a stride-2 convolution with all four stride phases
// of a band of dx rows computed by one workgroup.
//
// The sum is the one of dx_igemm.hip: dx[n, ih, iw, ci] = sum over co and the
// taps (kh, kw) that reach (ih, iw) of dy[n, oh, ow, co] * w[co, kh, kw, ci],
// ih = oh*2 - ph + kh (the adjoint of the forward: oarust 0.8.6
// src/rs/ml/matrix/conv.rs, `conv_2d_backward`, which dispatches the input
// adjoint over input elements; teeny-kernels 0.2.0 src/nn/conv/conv2d.rs
// `conv2d_backward_dx` computes the same sum by scattering).  With stride 2
// and dilation 1, dx row ih = 2a + rh is reached by the kernel rows kh with
// kh + ph = rh (mod 2), each from dy row a + e(kh) + ph/2, where
// e(kh) = (rh + (ph mod 2) - kh) / 2; columns likewise.  So dx splits into four
// phases (rh, rw), each a dense GEMM over (tap, co), and the phases of one
// phase-grid pixel (a, b) together read dy only at the few shifts
// (e(kh), e(kw)): a 3x3 kernel with odd padding reads four (0 or 1 down,
// 0 or 1 right) for its nine taps.
//
// MI355X design.  One workgroup of eight waves per CU owns a band of R
// phase-grid rows of one image (R * ceil(W/2) <= 256 pixels) and 64 input
// channels, for all four phases: 4 x 2 accumulator tiles of
// v_mfma_f32_32x32x16_bf16 per wave (128 registers).  The K loop runs over
// 16-channel chunks of co through an LDS ring of NS stages; a stage holds the
// chunk's weights for every tap ([tap][co][64 ci] rows, read with the gfx950
// transposed LDS read) and the dy block the band's taps reach (R + 1 rows of
// ceil(W/2) + 1 pixels for 3x3), both filled by 16-byte buffer-to-LDS loads
// (zero outside dy).  Each dy fragment (32 pixels at one shift) is read once
// per chunk and serves every tap with that shift, each into its own phase's
// accumulator, so a chunk costs 17 fragment reads for 18 MFMAs per wave and
// moves 26 KB from L2 per 1.2 M MACs of the workgroup (the per-phase tiles of
// dx_igemm move 16 KB per 0.5 M).  Wave w takes pixel tiles (w mod 4) and
// (w mod 4) + 4 and the 32-channel half w / 4; the two waves of a SIMD share
// their pixel tiles.  The bands of one image and both channel halves of a
// band run on one XCD, so dy comes from HBM once.  The tile is restaged
// through LDS and written as whole 128-byte lines, in dx row order.
#include "kernels.hpp"

#include <algorithm>
#include <type_traits>

namespace convmi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef const __attribute__((address_space(3))) char* lds_cptr;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kKC = 16;                 // output channels (co) per chunk: one MFMA k step
constexpr int kCT = 64;                 // input channels per workgroup
constexpr int kMaxPx = 256;             // band pixels: at most 8 tiles of 32
constexpr int kLdsBytes = 160 * 1024;
constexpr int kXcds = 8;

// One axis of the kernel: residue (phase) of kernel index k for pad parity
// P1, its dy shift e(k), and the shift's index from the smallest.
template <int K, int P1>
struct Axis {
    static constexpr int res(int k) { return (k + P1) & 1; }
    static constexpr int e(int k) { return (res(k) + P1 - k) / 2; }  // exact: the numerator is even
    static constexpr int emin()
    {
        int m = e(0);
        for (int k = 1; k < K; ++k) m = e(k) < m ? e(k) : m;
        return m;
    }
    static constexpr int emax()
    {
        int m = e(0);
        for (int k = 1; k < K; ++k) m = e(k) > m ? e(k) : m;
        return m;
    }
    static constexpr int S = emax() - emin() + 1;  // distinct shifts
    static constexpr int sh(int k) { return e(k) - emin(); }
};

// The taps of a kernel grouped by dy shift: shift index gi = sh * S_w + sw,
// its taps (kh * KW + kw) in order, and the order in which a chunk visits
// the shifts (fewest taps first, so that the last, largest group's MFMAs
// are queued when a wave reaches the next chunk's barrier).
template <int KH_, int KW_, int P1H, int P1W>
struct TapTable {
    using AH = Axis<KH_, P1H>;
    using AW = Axis<KW_, P1W>;
    static constexpr int kShifts = AH::S * AW::S;
    static constexpr int gi_of(int t) { return AH::sh(t / KW_) * AW::S + AW::sh(t % KW_); }
    static constexpr int phase(int t) { return AH::res(t / KW_) * 2 + AW::res(t % KW_); }
    static constexpr int ntaps(int gi)
    {
        int n = 0;
        for (int t = 0; t < KH_ * KW_; ++t) n += gi_of(t) == gi;
        return n;
    }
    static constexpr int tap(int gi, int k)
    {
        for (int t = 0; t < KH_ * KW_; ++t)
            if (gi_of(t) == gi && k-- == 0) return t;
        return -1;
    }
    static constexpr int max_taps()
    {
        int m = 0;
        for (int gi = 0; gi < kShifts; ++gi) m = ntaps(gi) > m ? ntaps(gi) : m;
        return m;
    }
    static constexpr int order(int i)  // i-th shift visited: by tap count, then index
    {
        for (int n = 0; n <= KH_ * KW_; ++n)
            for (int gi = 0; gi < kShifts; ++gi)
                if (ntaps(gi) == n && i-- == 0) return gi;
        return -1;
    }
};

struct BandArgs {
    const bf16_t* dy;
    const bf16_t* w;
    const bf16_t* bias;   // per input channel, or null
    bf16_t* dx;
    Geom g;
    int R;                // phase-grid rows per band
    int Bw;               // phase-grid columns: ceil(W / 2)
    int nb;               // bands per image
    int ctiles;           // 64-channel tiles over all groups
    int total;            // N * nb * ctiles
    int RB, CB;           // dy block: rows, columns
    int wu, dyu;          // units of a stage: weights, then dy
    int row0_off;         // dy row of block row 0, minus the band's first phase row
    int col0;             // dy column of block column 0
    FastDiv div_cb;       // by CB
    FastDiv div_w;        // by W
};

// Weight rows are 8 units (64 channels); unit u of row r (co within the
// chunk) sits at u ^ swz_w(r), so that a transposed read (4 rows x 32 bytes
// per 16 lanes, two 16-lane groups per cycle) covers all 64 banks.
__device__ __forceinline__ int swz_w(int r) { return ((r >> 1) & 1) << 2; }
// dy pixels are 2 units (16 channels); unit u of block pixel i sits at
// u ^ swz_d(i), so 16 consecutive pixels read at one unit cover all banks.
__device__ __forceinline__ int swz_d(int i) { return (i >> 3) & 1; }

template <int KH_, int KW_, int P1H, int P1W, int LW, int NS>
__global__ __launch_bounds__(kThreads) void dx_band_kernel(BandArgs a)
{
    extern __shared__ uint4 ring[];
    using AH = Axis<KH_, P1H>;
    using AW = Axis<KW_, P1W>;
    constexpr int kTaps = KH_ * KW_;
    constexpr int kShifts = AH::S * AW::S;
    constexpr int kStageUnits = LW * kThreads;
    constexpr int kStageBytes = kStageUnits * 16;
    constexpr int JT = 2;  // pixel tiles per wave
    const Geom& g = a.g;

    // Workgroup -> (image, band, channel tile).  Workgroup b runs on XCD
    // b mod 8; consecutive logical indices go to one XCD, so the channel
    // tiles and bands of an image share that XCD's L2.
    const int per_xcd = static_cast<int>(gridDim.x) / kXcds;
    const int logical = (static_cast<int>(blockIdx.x) % kXcds) * per_xcd + static_cast<int>(blockIdx.x) / kXcds;
    if (logical >= a.total) return;
    const int ct_all = logical % a.ctiles;
    const int nb_idx = logical / a.ctiles;
    const int band = nb_idx % a.nb;
    const int n = nb_idx / a.nb;
    const int ct_per_grp = g.Cg / kCT;
    const int grp = ct_all / ct_per_grp;
    const int ci_rel0 = (ct_all - grp * ct_per_grp) * kCT;
    const int ci0 = grp * g.Cg + ci_rel0;
    const int co_g0 = grp * g.Mg;
    const int a0 = band * a.R;
    const int Ah = (g.H + 1) / 2;
    const int rows = min(a.R, Ah - a0);  // phase-grid rows of this band
    const int npx = rows * a.Bw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int q = lane >> 5;
    const int ps = wave & 3;       // pixel tiles ps, ps + 4
    const int ct = wave >> 2;      // 32-channel half

    const uint32_t dy_bytes = static_cast<uint32_t>(g.N) * static_cast<uint32_t>(g.OH * g.OW) *
                              static_cast<uint32_t>(g.CO) * 2u;
    const uint32x4_t dyr = dma_rsrc(a.dy, dy_bytes);
    const uint32_t w_bytes = static_cast<uint32_t>(g.CO) * static_cast<uint32_t>(kTaps * g.Cg) * 2u;
    const uint32x4_t wr = dma_rsrc(a.w, w_bytes);

    // Loads: thread tid's load j fills stage unit U = j*512 + tid.  Units
    // below wu are weights (row U/8 = tap*16 + co, position U%8), then dy
    // (block pixel (U - wu)/2, position (U - wu)%2), then zero padding.  wu
    // is a multiple of 64, so each wave load is of one kind.  off is the
    // byte offset for the current chunk, del its advance per chunk.
    uint32_t off[LW], del[LW];
#pragma unroll
    for (int j = 0; j < LW; ++j) {
        const int U = j * kThreads + tid;
        off[j] = kOutside;
        del[j] = 0;
        if (U < a.wu) {
            const int r = U >> 3;
            const int t = r / kKC, cor = r % kKC;
            const int u = (U & 7) ^ swz_w(cor);
            off[j] = ((static_cast<uint32_t>(co_g0 + cor) * kTaps + t) * g.Cg + ci_rel0 + u * 8) * 2u;
            del[j] = static_cast<uint32_t>(kKC) * kTaps * g.Cg * 2u;
        } else if (U < a.wu + a.dyu) {
            const int V = U - a.wu;
            const int i = V >> 1;
            const int u = (V & 1) ^ swz_d(i);
            const int br = static_cast<int>(fdiv(static_cast<uint32_t>(i), a.div_cb));
            const int bc = i - br * a.CB;
            const int oh = a0 + a.row0_off + br, ow = a.col0 + bc;
            if (static_cast<unsigned>(oh) < static_cast<unsigned>(g.OH) &&
                static_cast<unsigned>(ow) < static_cast<unsigned>(g.OW)) {
                off[j] = (((static_cast<uint32_t>(n) * g.OH + oh) * g.OW + ow) * g.CO + co_g0 + u * 8) * 2u;
                del[j] = static_cast<uint32_t>(kKC) * 2u;
            }
        }
    }
    // Wave loads that hold only padding are not issued: wave w issues the
    // loads j with 8j + w below the chunk's wave-load count, my_loads of them
    // per chunk (between 1 and LW; small bands fill only part of a stage).
    const int wl_chunk = (a.wu + a.dyu + 63) / 64;
    const int my_loads = (wl_chunk - wave + kWaves - 1) / kWaves;
    // Waits until this wave's loads of the chunk NS - 2 chunks back have
    // landed: at most (NS - 2) chunks of my_loads loads still in flight.
    auto wait_chunk = [&]() __attribute__((always_inline)) {
        switch (my_loads) {
        case 1: wait_vm<(NS - 2) * 1>(); break;
        case 2: wait_vm<(NS - 2) * 2>(); break;
        case 3: wait_vm<(NS - 2) * 3>(); break;
        case 4: wait_vm<(NS - 2) * 4>(); break;
        case 5: wait_vm<(NS - 2) * 5>(); break;
        case 6: wait_vm<(NS - 2) * 6>(); break;
        default: wait_vm<0>(); break;
        }
    };
    static_assert(LW <= 6, "wait_chunk covers at most six loads per chunk");
    const uint32_t ring_lds = lds_addr(ring);
    auto issue_one = [&](int stage, bool live, int j) __attribute__((always_inline)) {
        if (j >= my_loads) return;
        const uint32_t sb = ring_lds + static_cast<uint32_t>(stage) * kStageBytes;
        const int wl = j * kThreads + wave * 64;  // first unit of this wave load (uniform)
        dma16(wl < a.wu ? wr : dyr, live ? off[j] : kOutside, sb + static_cast<uint32_t>(wl) * 16u);
        off[j] += del[j];
    };
    auto issue = [&](int stage, bool live) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LW; ++j) issue_one(stage, live, j);
    };

    // Fragment addresses (bytes within a stage).  Weight fragment of tap t:
    // rows 16t + 8(g4/2) + 4h + s/4, channels 32ct + 16(g4%2) + 4(s%4) .. +3
    // (lane = 16 g4 + s), read transposed: lane gets co 8(lane/32) .. +7 of
    // channel 32ct + lane%32.  dy fragment of tile j at shift (sh, sw): block
    // pixel (pa + sh) * CB + pb + sw of the lane's pixel p = (ps + 4j)*32 + col
    // = pa * Bw + pb, unit q.
    const int g4 = lane >> 4, s16 = lane & 15;
    int tr_off[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 8 * (g4 >> 1) + 4 * h + (s16 >> 2);
        const int ch = ct * 32 + 16 * (g4 & 1) + 4 * (s16 & 3);
        tr_off[h] = row * 128 + (((ch >> 3) ^ swz_w(row)) << 4) + (ch & 7) * 2;
    }
    int baddr[JT][kShifts];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
        int p = (ps + 4 * j) * 32 + col;
        p = p < npx ? p : 0;  // padding pixels read pixel 0; their results are not stored
        const int pa = p / a.Bw, pb = p - (p / a.Bw) * a.Bw;
#pragma unroll
        for (int sh = 0; sh < AH::S; ++sh)
#pragma unroll
            for (int sw = 0; sw < AW::S; ++sw) {
                const int i = (pa + sh) * a.CB + pb + sw;
                baddr[j][sh * AW::S + sw] = a.wu * 16 + i * 32 + ((q ^ swz_d(i)) << 4);
            }
    }

    f32x16 acc[4][JT];
#pragma unroll
    for (int P = 0; P < 4; ++P)
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[P][j][v] = 0.f;

    // Multiplies the chunk in `stage` and, after each shift's MFMAs, issues
    // a share of the loads of the chunk that refills `next`: a wave that
    // stalls issuing a load then still has MFMAs in flight.
    // A shift group's fragments: the dy fragments of the wave's tiles at that
    // shift and the weight fragments of the shift's taps.  Group i + 1 is
    // read while group i multiplies.
    using TT = TapTable<KH_, KW_, P1H, P1W>;
    struct GroupFrags {
        bf16x8 b[JT];
        bf16x8 w[TT::max_taps()];
    };
    auto read_group = [&](lds_cptr sb, int gi, GroupFrags& f) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < JT; ++j) f.b[j] = *reinterpret_cast<const lds_bf16x8*>(sb + baddr[j][gi]);
#pragma unroll
        for (int k = 0; k < TT::max_taps(); ++k) {
            if (k >= TT::ntaps(gi)) break;
            const int t = TT::tap(gi, k);
            const bf16x4 lo =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sb + t * (kKC * 128) + tr_off[0]));
            const bf16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sb + t * (kKC * 128) + tr_off[1]));
            f.w[k] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    auto mfma_group = [&](int gi, const GroupFrags& f) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < TT::max_taps(); ++k) {
            if (k >= TT::ntaps(gi)) break;
            const int P = TT::phase(TT::tap(gi, k));
#pragma unroll
            for (int j = 0; j < JT; ++j)
                acc[P][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[k], f.b[j], acc[P][j], 0, 0, 0);
        }
    };
    auto compute = [&](int stage, int next, bool live) __attribute__((always_inline)) {
        const lds_cptr sb = (lds_cptr)(ring + stage * kStageUnits);
        GroupFrags f[2];
        read_group(sb, TT::order(0), f[0]);
#pragma unroll
        for (int i = 0; i < kShifts; ++i) {
            if (i + 1 < kShifts) read_group(sb, TT::order(i + 1), f[(i + 1) & 1]);
            mfma_group(TT::order(i), f[i & 1]);
#pragma unroll
            for (int j = i * LW / kShifts; j < (i + 1) * LW / kShifts; ++j) issue_one(next, live, j);
        }
    };

    // Chunk c: wait for this thread's loads of chunk c (those of the next
    // NS - 2 chunks may still be in flight), synchronise (every wave's loads
    // of chunk c have landed; every wave is done with chunk c - 1, whose
    // stage is refilled now), issue chunk c + NS - 1, multiply chunk c.
    // Chunks past the last are issued as zero loads so that the wait count
    // is fixed.
    // The tile's bias (the transposed convolution's; none for dx): this
    // lane's channels 32ct + 8v + 4q + {0..3}, loaded now so that its latency
    // is hidden by the K loop.  A null bias is a resource of zero bytes.
    const rsrc_t brs = make_rsrc(a.bias, a.bias ? static_cast<uint32_t>(g.C) * 2u : 0u);
    uint2 braw[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        braw[v] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                brs, static_cast<uint32_t>(ci0 + ct * 32 + v * 8 + q * 4) * 2u, 0, 0));

    const int nch = g.Mg / kKC;
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, s < nch);
    for (int c = 0; c < nch; c += NS) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (c + i < nch) {
                wait_chunk();
                barrier_no_fence();
                compute(i, (i + NS - 1) % NS, c + i + NS - 1 < nch);
            }
        }
    }
    wait_vm<0>();     // the zero loads past the last chunk have landed
    __syncthreads();  // and every wave is done reading the stages

    // Epilogue.  Lane holds channels 32ct + 8v + 4q + {0..3} of band pixel
    // p = (ps + 4j)*32 + col of phase P in acc[P][j][4v .. 4v+3].  The bf16
    // tile is staged as [phase][pixel][8 units], unit u of pixel p at
    // u ^ ((p >> 1) & 7) and the phase areas an odd number of pixels apart,
    // so that 16 consecutive pixels written at one unit, and the 8 units of
    // two neighbouring dx pixels read, each cover all 64 banks.  A lane pair
    // (l, l + 32) holds the two 4-channel halves of units v and v + 1; one
    // exchange across the halves of the wave (v_permlane32_swap) gives the
    // lower lane unit v and the upper lane unit v + 1 whole, written as one
    // 16-byte store each.  Then dx is written in its own order: each dx
    // pixel's 64 channels are one 128-byte line, non-temporal (nothing reads
    // dx back).
    float bsum[4][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint2 bv = braw[v];
        bsum[v][0] = __uint_as_float(bv.x << 16);
        bsum[v][1] = __uint_as_float(bv.x & 0xffff0000u);
        bsum[v][2] = __uint_as_float(bv.y << 16);
        bsum[v][3] = __uint_as_float(bv.y & 0xffff0000u);
    }
    const int ppx = (a.R * a.Bw) | 1;  // pixels per phase area of the staging
    // Without a bias (dx) the fp32 sums are rounded as they are: a separate
    // path, so that the common case spends no additions on zeros.
    auto stage_out = [&](auto with_bias) __attribute__((always_inline)) {
        constexpr bool kBias = decltype(with_bias)::value;
        auto val = [&](int P, int j, int v, int i) __attribute__((always_inline)) {
            return kBias ? acc[P][j][4 * v + i] + bsum[v][i] : acc[P][j][4 * v + i];
        };
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                const int p = (ps + 4 * j) * 32 + col;
#pragma unroll
                for (int v = 0; v < 4; v += 2) {
                    const uint32_t x0 = pack_bf16x2(val(P, j, v, 0), val(P, j, v, 1));
                    const uint32_t x1 = pack_bf16x2(val(P, j, v, 2), val(P, j, v, 3));
                    const uint32_t y0 = pack_bf16x2(val(P, j, v + 1, 0), val(P, j, v + 1, 1));
                    const uint32_t y1 = pack_bf16x2(val(P, j, v + 1, 2), val(P, j, v + 1, 3));
                    const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
                    const int u = ct * 4 + v + q;
                    if (p < npx) ring[(P * ppx + p) * 8 + (u ^ ((p >> 1) & 7))] = uint4{s0[0], s1[0], s0[1], s1[1]};
                }
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
    const int units = rows * 2 * g.W * 8;
    for (int idx = tid; idx < units; idx += kThreads) {
        const int u = idx & 7;
        const int pix = idx >> 3;
        const int r2 = static_cast<int>(fdiv(static_cast<uint32_t>(pix), a.div_w));
        const int iw = pix - r2 * g.W;
        const int ar = r2 >> 1, rh = r2 & 1;
        const int ih = 2 * (a0 + ar) + rh;
        const int p = ar * a.Bw + (iw >> 1);
        const int P = rh * 2 + (iw & 1);
        const uint32_t o = ih < g.H ? ((static_cast<uint32_t>(n * g.H + ih) * g.W + iw) * g.C + ci0 + u * 8) * 2u
                                    : kOutside;
        buffer_store16_nt(dxr, o, ring[(P * ppx + p) * 8 + (u ^ ((p >> 1) & 7))]);
    }
}

struct Plan {
    int KH, P1, LW, NS;
    int R, Bw, nb, ctiles, RB, CB, wu, dyu, row0_off, col0, blocks;
    size_t lds;
    bool ok;
};

// Shifts of one axis (host mirror of Axis).
void axis_range(int K, int p1, int& emin, int& emax)
{
    emin = 1 << 20;
    emax = -(1 << 20);
    for (int k = 0; k < K; ++k) {
        const int r = (k + p1) & 1;
        const int e = (r + p1 - k) / 2;
        emin = std::min(emin, e);
        emax = std::max(emax, e);
    }
}

constexpr int stages_for(int lw) { return kLdsBytes / (lw * kThreads * 16) > 5 ? 5 : kLdsBytes / (lw * kThreads * 16); }

Plan make_plan(const Geom& g, int cus)
{
    Plan p{};
    p.ok = false;
    if (g.sh != 2 || g.sw != 2 || g.dh != 1 || g.dw != 1) return p;
    if (g.KH != g.KW || (g.KH != 3 && g.KH != 4)) return p;
    if ((g.ph & 1) != (g.pw & 1)) return p;
    if (g.Cg % kCT != 0 || g.Mg % kKC != 0) return p;
    p.KH = g.KH;
    p.P1 = g.ph & 1;
    const int Ah = (g.H + 1) / 2;
    p.Bw = (g.W + 1) / 2;
    if (p.Bw > kMaxPx) return p;
    const int rmax = kMaxPx / p.Bw;
    p.ctiles = g.G * (g.Cg / kCT);
    int nb = (Ah + rmax - 1) / rmax;
    // More, shorter bands while the grid leaves CUs idle.
    while (static_cast<int64_t>(g.N) * nb * p.ctiles < cus && nb < Ah) ++nb;
    p.R = (Ah + nb - 1) / nb;
    p.nb = (Ah + p.R - 1) / p.R;
    int ehmin, ehmax, ewmin, ewmax;
    axis_range(g.KH, g.ph & 1, ehmin, ehmax);
    axis_range(g.KW, g.pw & 1, ewmin, ewmax);
    p.RB = p.R + ehmax - ehmin;
    p.CB = p.Bw + ewmax - ewmin;
    p.row0_off = ehmin + (g.ph >> 1);
    p.col0 = ewmin + (g.pw >> 1);
    p.wu = g.KH * g.KW * kKC * 8;
    p.dyu = p.RB * p.CB * 2;
    const int need = (p.wu + p.dyu + kThreads - 1) / kThreads;
    // Instantiated load counts: 4 or 5 per thread for 3x3, 6 for 4x4.
    if (g.KH == 3) p.LW = need <= 4 ? 4 : need <= 5 ? 5 : 0;
    else p.LW = need <= 6 ? 6 : 0;
    if (p.LW == 0) return p;
    p.NS = stages_for(p.LW);
    if (p.NS < 3) return p;
    p.lds = static_cast<size_t>(p.NS) * p.LW * kThreads * 16;
    if (static_cast<size_t>(4) * ((p.R * p.Bw) | 1) * 128 > p.lds) return p;  // the output staging
    const int64_t total = static_cast<int64_t>(g.N) * p.nb * p.ctiles;
    if (total >= (int64_t(1) << 30)) return p;
    p.blocks = static_cast<int>((total + kXcds - 1) / kXcds * kXcds);
    p.ok = true;
    return p;
}

template <int K, int P1, int LW>
hipError_t launch_k(const BandArgs& a, const Plan& p, hipStream_t s)
{
    constexpr int NS = stages_for(LW);
    auto kernel = dx_band_kernel<K, K, P1, P1, LW, NS>;
    static size_t lds_allowed = 64 * 1024;  // the default dynamic LDS limit
    if (p.lds > lds_allowed) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(p.lds));
        if (e != hipSuccess) return e;
        lds_allowed = p.lds;
    }
    return launch(kernel, dim3(p.blocks), dim3(kThreads), p.lds, s, a);
}

}  // namespace

bool can_dx_band(const Geom& g, int dtype)
{
    if (dtype != 1 || !g.nhwc || !g.aligned16) return false;
    const int64_t dy_bytes = static_cast<int64_t>(g.N) * g.OH * g.OW * g.CO * 2;
    const int64_t dx_bytes = static_cast<int64_t>(g.N) * g.H * g.W * g.C * 2;
    const int64_t w_bytes = static_cast<int64_t>(g.CO) * g.KH * g.KW * g.Cg * 2;
    const int64_t lim = int64_t(1) << 31;
    if (dy_bytes >= lim || dx_bytes >= lim || w_bytes >= lim) return false;
    return make_plan(g, 256).ok;
}

hipError_t launch_dx_band(const void* dy, const void* w, const void* bias, void* dx, const Geom& g,
                          hipStream_t s)
{
    const Plan p = make_plan(g, device_cu_count());
    if (!p.ok) return hipErrorInvalidValue;
    BandArgs a;
    a.dy = static_cast<const bf16_t*>(dy);
    a.w = static_cast<const bf16_t*>(w);
    a.bias = static_cast<const bf16_t*>(bias);
    a.dx = static_cast<bf16_t*>(dx);
    a.g = g;
    a.R = p.R;
    a.Bw = p.Bw;
    a.nb = p.nb;
    a.ctiles = p.ctiles;
    a.total = static_cast<int>(static_cast<int64_t>(g.N) * p.nb * p.ctiles);
    a.RB = p.RB;
    a.CB = p.CB;
    a.wu = p.wu;
    a.dyu = p.dyu;
    a.row0_off = p.row0_off;
    a.col0 = p.col0;
    a.div_cb = make_fastdiv(static_cast<uint32_t>(p.CB));
    a.div_w = make_fastdiv(static_cast<uint32_t>(g.W));
    switch (p.KH * 100 + p.P1 * 10 + p.LW) {
    case 314: return launch_k<3, 1, 4>(a, p, s);
    case 315: return launch_k<3, 1, 5>(a, p, s);
    case 304: return launch_k<3, 0, 4>(a, p, s);
    case 305: return launch_k<3, 0, 5>(a, p, s);
    case 416: return launch_k<4, 1, 6>(a, p, s);
    case 406: return launch_k<4, 0, 6>(a, p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace convmi
