// Dense forward convolution as an implicit GEMM, streamed over output-row
// bands by persistent workgroups.
//
// The product computed is the one of igemm.hip (per group,
// y[m, co] = bias[co] + sum_k A[m, k] B[co, k], k = (kh, kw, c), A the im2col
// rows of x, B the OHWI weight), following the im2col column definition of
// burn-cubecl 0.22.0-pre.4 src/kernel/conv/im2col.rs (`im2col`).  This
// variant serves groups whose whole 64-channel weight panel
// [64][KH KW Cg] fits in LDS next to a ring of input rows (Cg <= 64 for 3x3).
//
// MI355X design.  The dense layers of the workloads here move more bytes
// than their MFMA time (a 3x3, 64 -> 64 layer reads and writes 128 bytes per
// output pixel for 73.7 kFLOP), so the kernel is shaped to keep HBM busy
// from start to end rather than to load, multiply and store in lockstep.
// One workgroup of eight waves per CU holds its weight panel in LDS for the
// whole launch and walks a band of consecutive output rows (of one 64-channel
// tile) in groups of up to Gmax rows.  When the whole band fits the LDS as
// one group it is one group: two waves per SIMD then hide each other's
// fragment reads (a 64 x 64 wave tile fed from LDS runs at most ~57 % of the
// MFMA rate with one wave per SIMD, ~73 % with two), which outweighs the
// overlap of loads and stores across groups (3x3, 64 -> 64 at 56x56 x 32,
// seven rows per band: 16.7 -> 15.1 us against four waves in groups of four
// and three rows).  Input rows live in a ring of LDS row slots; while a
// group is multiplied, the rows the next group adds stream into free slots
// (16-byte buffer-to-LDS loads, zero outside the image), and the group's
// results leave as 8-byte stores straight from the accumulators, overlapping
// the next group's MFMAs.  The last group's stores overlap nothing, so its
// tile is restaged in the idle ring and leaves as whole 128-byte lines
// (3x3, 64 -> 64 channels at 56x56 x 32: 18.0 -> 17.15 us).  Loads of a group are issued before the stores of
// the previous one, so one fixed vmcnt wait (the number of stores a wave
// issues per group) means "this group's rows have landed".  Every fragment
// of v_mfma_f32_32x32x16_bf16 is one ds_read_b128 per lane: the weight
// operand from the panel (rows padded by one unit), the pixel operand from
// the ring at the pixel's tap position (units XOR-swizzled by pixel index).
// Wave w computes all 64 channels of the group's 32-pixel tiles w, w + 8, ...
#include "kernels.hpp"

namespace convmi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBN = 64;       // output channels per workgroup
constexpr int kLdsBytes = 160 * 1024;
constexpr int kMaxGroupRows = 8;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

struct BandArgs {
    const bf16_t* x;
    const bf16_t* w;
    const bf16_t* bias;
    bf16_t* y;
    Geom g;
    int TW, IC, col_tiles;
    int Gmax;          // output rows per group
    int ring;          // input row slots
    int row_units;     // 16-byte units per slot (IC * Cg / 8, padded to whole wave loads)
    int w_units;       // units of the weight panel (padded to whole wave loads)
    int total_rows;    // N * col_tiles * OH: band rows, image-major
    int bands;         // workgroups along the rows
    int co_tiles;
    int stage_last;    // the last group's tile fits the ring as 128-byte pixel rows
    FastDiv div_oh;    // by OH
    FastDiv div_ct;    // by col_tiles
    FastDiv div_tw;    // by TW
    FastDiv div_wrow;  // by the weight row pitch
};

// Ring slot layout.  UPX = Cg / 8 units per pixel; pixels come in packs of
// PG = 16 / UPX (256 bytes) followed by one pad unit, so pixel hc's unit u
// sits at unit (hc / PG) * 17 + (hc % PG) * UPX + u.  Any 16 consecutive
// pixels read at one unit then hit 16 distinct bank groups, and a lane's
// address for the next 16 channels is the same plus a constant, which the
// reads take as an immediate offset.
template <int UPX>
__device__ __forceinline__ int pix_unit(int hc)
{
    constexpr int PG = 16 / UPX;
    return (hc / PG) * 17 + (hc % PG) * UPX;
}

// Position of output row r of the band space.
struct RowPos {
    int n, ct, oh;
};

constexpr int kMaxRowLoads = 4;  // wave loads per ring row per wave (row_units <= 1024)

template <int UPX, int KH_, int KW_, int NT>
__global__ __launch_bounds__(kThreads) void igemm_band_kernel(BandArgs a)
{
    extern __shared__ uint4 lds[];
    const Geom& g = a.g;
    constexpr int taps = KH_ * KW_;
    constexpr int wrow = taps * UPX + 1;
    constexpr int SPT = UPX / 2;  // 16-channel k-steps per tap
    constexpr int PG = 16 / UPX;
    uint4* const wl = lds;
    uint4* const bias_l = lds + a.w_units;       // 64 units: the tile's bias, bf16
    uint4* const ring = lds + a.w_units + 64;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int q = lane >> 5;

    const int grp_id = blockIdx.y / a.co_tiles;
    const int co_in_grp = (blockIdx.y - grp_id * a.co_tiles) * kBN;
    const int co0 = grp_id * g.Mg + co_in_grp;
    // Band of this workgroup: with a multiple of 8 bands, XCD x (workgroup b
    // runs on XCD b mod 8) takes the x-th eighth of the bands, consecutive
    // rows, so that the input rows two neighbouring bands share are fetched
    // into one L2.
    const int band = a.bands % 8 == 0
                         ? static_cast<int>(blockIdx.x & 7) * (a.bands / 8) + static_cast<int>(blockIdx.x >> 3)
                         : static_cast<int>(blockIdx.x);
    const int64_t r_begin = static_cast<int64_t>(a.total_rows) * band / a.bands;
    const int64_t r_end = static_cast<int64_t>(a.total_rows) * (band + 1) / a.bands;

    const uint32_t x_bytes = static_cast<uint32_t>(g.N) * static_cast<uint32_t>(g.H * g.W) *
                             static_cast<uint32_t>(g.C) * 2u;
    const uint32x4_t xr = dma_rsrc(a.x, x_bytes);
    const uint32x4_t wr =
        dma_rsrc(a.w, static_cast<uint32_t>(g.CO) * static_cast<uint32_t>(taps * g.Cg) * 2u);
    const uint32_t y_bytes = static_cast<uint32_t>(g.N) * static_cast<uint32_t>(g.OH * g.OW) *
                             static_cast<uint32_t>(g.CO) * 2u;
    const rsrc_t yr = make_rsrc(a.y, y_bytes);

    // The tile's bias (zero past the group and without bias) is staged in
    // LDS with the weights, two channels per lane of wave 0.
    if (wave == 0) {
        const uint32x4_t br = dma_rsrc(a.bias, a.bias ? static_cast<uint32_t>(g.CO) * 2u : 0u);
        const int crel = co_in_grp + 2 * lane;
        dma4(br, (lane < kBN / 2 && crel < g.Mg) ? static_cast<uint32_t>(co0 + 2 * lane) * 2u : kOutside,
             lds_addr(bias_l));
    }

    // Input rows.  A ring row of column tile ct is row_units units; wave w
    // fills its wave loads w, w + 8, ... (row_units is a multiple of 512, so
    // each wave has the same per_row of them).  What a lane loads in wave
    // load m depends only on ct: the byte offset of its 16 bytes within an
    // image row (colo) and whether they are inside the image (colok); the
    // row adds a uniform offset.
    const int per_row = a.row_units / (64 * kWaves);
    uint32_t colo[kMaxRowLoads];
    bool colok[kMaxRowLoads];
    int col_ct = -1;
    auto set_columns = [&](int ct) __attribute__((always_inline)) {
        col_ct = ct;
#pragma unroll
        for (int m = 0; m < kMaxRowLoads; ++m) {
            const int L = (wave + kWaves * m) * 64 + lane;
            const int grp17 = L / 17, rr17 = L - grp17 * 17;
            const int hc = grp17 * PG + rr17 / UPX, u = rr17 % UPX;
            const int iw = ct * a.TW * g.sw - g.pw + hc;
            colok[m] = m < per_row && rr17 < 16 && hc < a.IC && static_cast<unsigned>(iw) < static_cast<unsigned>(g.W);
            colo[m] = (static_cast<uint32_t>(iw) * g.C + grp_id * g.Cg + u * 8) * 2u;
        }
    };
    // Issues this wave's loads of input row ih of image n into ring slot.
    auto load_row = [&](int n, int ih, int slot) __attribute__((always_inline)) {
        const bool row_ok = static_cast<unsigned>(ih) < static_cast<unsigned>(g.H);
        const uint32_t rowo = static_cast<uint32_t>(n * g.H + ih) * static_cast<uint32_t>(g.W * g.C) * 2u;
        uint4* dst = ring + slot * a.row_units + wave * 64;
#pragma unroll
        for (int m = 0; m < kMaxRowLoads; ++m)
            if (m < per_row) dma16(xr, (row_ok && colok[m]) ? rowo + colo[m] : kOutside, lds_addr(dst + m * kWaves * 64));
    };
    auto decode = [&](int64_t r) __attribute__((always_inline)) {
        RowPos p;
        const uint32_t nct = fdiv(static_cast<uint32_t>(r), a.div_oh);
        p.oh = static_cast<int>(static_cast<uint32_t>(r) - nct * g.OH);
        p.n = static_cast<int>(fdiv(nct, a.div_ct));
        p.ct = static_cast<int>(nct) - p.n * a.col_tiles;
        return p;
    };
    // Input rows a group of `rows` output rows reads.
    const int span_extra = (KH_ - 1) * g.dh + 1;
    auto in_rows = [&](int rows) __attribute__((always_inline)) { return (rows - 1) * g.sh + span_extra; };

    // A group's results wait in registers, rounded to bf16 with the bias,
    // and are stored while the next group is multiplied: store s of a wave
    // writes run (h, i) = ((s / 4) % 2, s % 4) of tile j = s / 8, channels
    // co0 + 32h + 8i + 4q + {0..3} of the lane's pixel (lanes q = 0, 1 of a
    // pixel write 16 contiguous bytes).
    constexpr int kStores = NT * 8;  // stores per wave per group
    uint32_t ch_bytes[2][4];
    bool ch_ok[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int crel = co_in_grp + h * 32 + i * 8 + q * 4;
            ch_ok[h][i] = crel < g.Mg;  // Mg is a multiple of 4
            ch_bytes[h][i] = static_cast<uint32_t>(co0 - co_in_grp + crel) * 2u;
        }
    uint2 outv[NT][2][4];
    uint32_t out_off[NT];  // byte offset of the pixel's channel 0, or kOutside
    auto store_one = [&](int s_) __attribute__((always_inline)) {
        const int j = s_ / 8, h = (s_ / 4) % 2, i = s_ % 4;
        const bool ok = out_off[j] != kOutside && ch_ok[h][i];
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(yr, 0, 0, 0)), outv[j][h][i]), yr,
            ok ? out_off[j] + ch_bytes[h][i] : kOutside, 0, 0);
    };

    f32x16 acc[2][NT];
    float bv[2][4][4];
    constexpr int KS = taps * SPT;  // k-steps per group

    // Ring bookkeeping (uniform).  The current group's nr input rows occupy
    // slots slot_base .. slot_base + nr - 1 (mod ring).  The next group keeps
    // the rows it shares with the current one in their slots and takes
    // `fresh` new rows in the slots that follow; they are loaded while the
    // current group is multiplied (one row per k-step) when they do not
    // touch its slots, else right after it (deferred).
    int64_t r = r_begin;
    RowPos cur = decode(r);
    int rows = static_cast<int>(min(static_cast<int64_t>(min(a.Gmax, g.OH - cur.oh)), r_end - r));
    int nr = in_rows(rows);
    int slot_base = 0;
    if (r < r_end) {
        set_columns(cur.ct);
        for (int i = 0; i < nr; ++i) load_row(cur.n, cur.oh * g.sh - g.ph + i, i);
    }
    // The weight panel is issued after the first group's rows: those come
    // from HBM and take longer, so their latency overlaps the panel's transfer.
    // Weight panel: LDS unit L = r*wrow + c holds, for c < taps*UPX, unit
    // c % UPX of tap c / UPX of output channel co0 + r; the pad unit of each
    // row and channels past the group are zero.  Workgroups start at
    // different wave loads so that their requests spread over the L2.
    {
        const int wloads = a.w_units / 64;
        const int rot = static_cast<int>((blockIdx.x * 37u + blockIdx.y * 11u) % static_cast<unsigned>(wloads));
        for (int kk = wave; kk < wloads; kk += kWaves) {
            const int k = kk + rot < wloads ? kk + rot : kk + rot - wloads;
            const int L = k * 64 + lane;
            const int r = static_cast<int>(fdiv(static_cast<uint32_t>(L), a.div_wrow));
            const int c = L - r * wrow;
            const int t = c / UPX, u = c - (c / UPX) * UPX;
            const bool in = r < kBN && c < taps * UPX && co_in_grp + r < g.Mg;
            const uint32_t off = ((static_cast<uint32_t>(co0 + r) * taps + t) * static_cast<uint32_t>(g.Cg) +
                                  static_cast<uint32_t>(u * 8)) * 2u;
            dma16(wr, in ? off : kOutside, lds_addr(wl + k * 64));
        }
    }

    bool have_prev = false;    // outv holds a group not yet stored
    RowPos last{};             // position and pixels of the group in outv
    int last_npx = 0;
    bool stores_sent = false;  // the previous iteration issued kStores stores after its loads
    int pend_first = 0, pend_count = 0, pend_slot = 0;  // deferred rows of the current group

    while (r < r_end) {
        if (pend_count > 0) {
            if (col_ct != cur.ct) set_columns(cur.ct);
            for (int i = 0; i < pend_count; ++i) {
                int sl = pend_slot + i;
                sl = sl >= a.ring ? sl - a.ring : sl;
                load_row(cur.n, pend_first + i, sl);
            }
        }
        if (stores_sent && pend_count == 0)
            wait_vm<kStores>();  // this group's rows (issued before those stores) have landed
        else
            wait_vm<0>();
        barrier_no_fence();  // every wave's rows for this group have landed; old slots are free
        if (!have_prev) {
            // Bias of this lane's channels co0 + 32h + 8i + 4q + {0..3}.
            const uint2* bl = reinterpret_cast<const uint2*>(bias_l);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint2 v = bl[h * 8 + i * 2 + q];
                    bv[h][i][0] = __uint_as_float(v.x << 16);
                    bv[h][i][1] = __uint_as_float(v.x & 0xffff0000u);
                    bv[h][i][2] = __uint_as_float(v.y << 16);
                    bv[h][i][3] = __uint_as_float(v.y & 0xffff0000u);
                }
        }

        const int64_t r2 = r + rows;
        RowPos nx{};
        int rows2 = 0, nr2 = 0, slot_base2 = 0;
        int fresh_first = 0, fresh = 0, fresh_slot = 0;
        bool deferred = false;
        if (r2 < r_end) {
            nx = decode(r2);
            rows2 = static_cast<int>(min(static_cast<int64_t>(min(a.Gmax, g.OH - nx.oh)), r_end - r2));
            nr2 = in_rows(rows2);
            const bool contiguous = nx.n == cur.n && nx.ct == cur.ct;
            const int keep = contiguous ? max(nr - rows * g.sh, 0) : 0;
            slot_base2 = (keep > 0 ? slot_base + rows * g.sh : slot_base + nr) % a.ring;
            fresh = nr2 - keep;
            fresh_first = nx.oh * g.sh - g.ph + keep;
            fresh_slot = (slot_base2 + keep) % a.ring;
            // Prefetched rows go out in the first KS/4 k-steps, all before
            // any store, so that the top-of-group wait can count stores.
            deferred = nr + fresh > a.ring || fresh > KS / 4 || nx.ct != col_ct;
        }
        const int now_rows = deferred ? 0 : fresh;

        // This lane's pixels: tile t = wave + 4j covers group pixels
        // 32t .. 32t + 31 (clamped to the group).  rb[j][kh] is the unit of
        // the pixel's tap-(kh, 0) input in the ring, plus q (the lane's half
        // of each 16-channel step); tap (kh, kw) adds cw[j][kw].
        const int npx = rows * a.TW;
        int rb[NT][KH_], cw[NT][KW_];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int p = min((wave + kWaves * j) * 32 + col, npx - 1);
            const int orow = static_cast<int>(fdiv(static_cast<uint32_t>(p), a.div_tw));
            const int ocol = p - orow * a.TW;
            const int base0 = pix_unit<UPX>(ocol * g.sw);
#pragma unroll
            for (int kw = 0; kw < KW_; ++kw) cw[j][kw] = pix_unit<UPX>(ocol * g.sw + kw * g.dw) - base0;
#pragma unroll
            for (int kh = 0; kh < KH_; ++kh) {
                int sl = slot_base + orow * g.sh + kh * g.dh;
                sl %= a.ring;
                rb[j][kh] = sl * a.row_units + base0 + q;
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[h][j][v] = 0.f;

        struct Frags {
            bf16x8 wa[2];
            bf16x8 px[NT];
        };
        const uint4* wlane = wl + col * wrow + q;  // + h*32*wrow + t*UPX + 2s: immediates
        auto read_frags = [&](int ks, Frags& f) __attribute__((always_inline)) {
            const int t = ks / SPT, s_ = ks - (ks / SPT) * SPT;
            const int kh = t / KW_, kw = t - (t / KW_) * KW_;
#pragma unroll
            for (int h = 0; h < 2; ++h) f.wa[h] = as_bf16x8(wlane[h * 32 * wrow + t * UPX + 2 * s_]);
#pragma unroll
            for (int j = 0; j < NT; ++j) f.px[j] = as_bf16x8(ring[rb[j][kh] + cw[j][kw] + 2 * s_]);
        };
        // Memory work spread over the k-steps, so that a wave blocked on
        // issuing it still has MFMAs in flight: one of the next group's rows
        // per k-step, then the previous group's stores.
        auto side_work = [&](int ks) __attribute__((always_inline)) {
            if (ks < KS / 4 && ks < now_rows) {
                int sl = fresh_slot + ks;
                sl = sl >= a.ring ? sl - a.ring : sl;
                load_row(nx.n, fresh_first + ks, sl);
            }
            if (have_prev) {
                constexpr int first_store = KS / 4;
#pragma unroll
                for (int s_ = 0; s_ < kStores; ++s_)
                    if (ks == first_store + s_ * (KS - first_store) / kStores) store_one(s_);
            }
        };
        auto mfmas = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[h][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.wa[h], f.px[j], acc[h][j], 0, 0, 0);
        };
        // Fragments are read two k-steps ahead of their MFMAs.
        Frags fr[3];
        read_frags(0, fr[0]);
        if (KS > 1) read_frags(1, fr[1]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) read_frags(ks + 2, fr[(ks + 2) % 3]);
            side_work(ks);
            mfmas(fr[ks % 3]);
        }
        stores_sent = have_prev;

        // This group's results, to be stored during the next one.
        last = cur;
        last_npx = npx;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int p = (wave + kWaves * j) * 32 + col;
            const int orow = static_cast<int>(fdiv(static_cast<uint32_t>(p), a.div_tw));
            const int ocol = p - orow * a.TW;
            const int ow = cur.ct * a.TW + ocol;
            out_off[j] = (p < npx && ow < g.OW)
                             ? static_cast<uint32_t>((cur.n * g.OH + cur.oh + orow) * g.OW + ow) *
                                   static_cast<uint32_t>(g.CO) * 2u
                             : kOutside;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    outv[j][h][i] = uint2{
                        pack_bf16x2(acc[h][j][4 * i + 0] + bv[h][i][0], acc[h][j][4 * i + 1] + bv[h][i][1]),
                        pack_bf16x2(acc[h][j][4 * i + 2] + bv[h][i][2], acc[h][j][4 * i + 3] + bv[h][i][3])};
        }
        have_prev = true;

        if (deferred) barrier_no_fence();  // every wave is done with the ring: the deferred rows may land

        r = r2;
        cur = nx;
        rows = rows2;
        nr = nr2;
        slot_base = slot_base2;
        pend_count = deferred ? fresh : 0;
        pend_first = fresh_first;
        pend_slot = fresh_slot;
    }
    if (!have_prev) return;
    if (!a.stage_last) {
#pragma unroll
        for (int s_ = 0; s_ < kStores; ++s_) store_one(s_);
        return;
    }
    // The last group's stores overlap no MFMAs, so they go out as whole
    // lines: the tile is restaged in the (now idle) ring as pixel rows of 8
    // units (64 channels, unit u of pixel p at u ^ (p & 7)) and each pixel's
    // channels leave as 16-byte stores, eight lanes per 128-byte line
    // (non-temporal when those are whole lines of y).
    barrier_no_fence();  // every wave is done reading the ring
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int p = (wave + kWaves * j) * 32 + col;
        if (p < last_npx) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int u = h * 4 + i;
                    reinterpret_cast<uint2*>(ring + p * 8 + (u ^ (p & 7)))[q] = outv[j][h][i];
                }
        }
    }
    __syncthreads();
    const bool whole_lines = (g.CO & 63) == 0 && (g.Mg & 63) == 0;
    for (int idx = tid; idx < last_npx * 8; idx += kThreads) {
        const int p = idx >> 3, u = idx & 7;
        const int orow = static_cast<int>(fdiv(static_cast<uint32_t>(p), a.div_tw));
        const int ow = last.ct * a.TW + p - orow * a.TW;
        const bool ok = ow < g.OW && co_in_grp + u * 8 < g.Mg;
        const uint32_t off =
            ok ? (static_cast<uint32_t>((last.n * g.OH + last.oh + orow) * g.OW + ow) * static_cast<uint32_t>(g.CO) +
                  static_cast<uint32_t>(co0 + u * 8)) * 2u
               : kOutside;
        const uint4 v = ring[p * 8 + (u ^ (p & 7))];
        if (whole_lines)
            buffer_store16_nt(yr, off, v);
        else
            buffer_store16(yr, off, v);
    }
}

struct BandPlan {
    int UPX, NT, TW, IC, col_tiles, co_tiles, Gmax, ring, row_units, w_units, bands, stage_last;
    size_t lds;
    bool one_group;  // every band is one group
    bool ok;
};

BandPlan make_band_plan(const Geom& g, int cus)
{
    BandPlan p{};
    p.ok = false;
    if (g.KH != 3 || g.KW != 3) return p;
    if (g.Cg != 16 && g.Cg != 32 && g.Cg != 64) return p;
    p.UPX = g.Cg / 8;
    p.TW = g.OW < 64 ? g.OW : 64;
    p.col_tiles = (g.OW + p.TW - 1) / p.TW;
    p.co_tiles = (g.Mg + kBN - 1) / kBN;
    p.IC = (p.TW - 1) * g.sw + (g.KW - 1) * g.dw + 1;
    const int PG = 16 / p.UPX;  // pixels per 17-unit pack
    p.row_units = ((p.IC + PG - 1) / PG * 17 + 64 * kWaves - 1) / (64 * kWaves) * (64 * kWaves);
    if (p.row_units > 64 * kWaves * kMaxRowLoads) return p;
    p.w_units = (kBN * (g.KH * g.KW * p.UPX + 1) + 63) / 64 * 64;
    const int bias_units = 64;
    // Bands: one workgroup per CU and 64-channel tile.
    const int64_t total_rows = static_cast<int64_t>(g.N) * p.col_tiles * g.OH;
    const int64_t per_y = static_cast<int64_t>(g.G) * p.co_tiles;
    int64_t bands = cus / per_y;
    if (bands < 1) bands = 1;
    if (bands > total_rows) bands = total_rows;
    p.bands = static_cast<int>(bands);
    const int rpb = static_cast<int>((total_rows + bands - 1) / bands);  // rows of the longest band
    // One group per band when the whole band's input rows fit beside the
    // panel; otherwise the tallest group (at most 8 rows, at most 16 pixel
    // tiles: two per wave) whose ring -- the group's input rows plus the
    // next group's new ones -- fits.
    {
        const int G = rpb;
        const int in_rows = (G - 1) * g.sh + (g.KH - 1) * g.dh + 1;
        const size_t lds = static_cast<size_t>(p.w_units + bias_units + in_rows * p.row_units) * 16;
        if (G <= kMaxGroupRows && (G * p.TW + 31) / 32 <= 2 * kWaves && lds <= static_cast<size_t>(kLdsBytes)) {
            p.Gmax = G;
            p.ring = in_rows;
            p.lds = lds;
            p.NT = (G * p.TW + 31) / 32 > kWaves ? 2 : 1;
            p.one_group = true;
            p.ok = true;
        }
    }
    for (int G = kMaxGroupRows; G >= 1 && !p.ok; --G) {
        if ((G * p.TW + 31) / 32 > 2 * kWaves) continue;
        const int in_rows = (G - 1) * g.sh + (g.KH - 1) * g.dh + 1;
        const int ring = in_rows + G * g.sh;
        const size_t lds = static_cast<size_t>(p.w_units + bias_units + ring * p.row_units) * 16;
        if (lds > static_cast<size_t>(kLdsBytes)) continue;
        p.Gmax = G;
        p.ring = ring;
        p.lds = lds;
        p.NT = (G * p.TW + 31) / 32 > kWaves ? 2 : 1;
        p.ok = true;
        break;
    }
    if (!p.ok) return p;
    // The last group's tile (Gmax x TW pixels x 128 bytes) restaged in the
    // ring, for groups of whole 8-channel units.
    p.stage_last = g.Mg % 8 == 0 &&
                   static_cast<int64_t>(p.ring) * p.row_units * 16 >= static_cast<int64_t>(p.Gmax) * p.TW * 128;
    return p;
}

template <int UPX, int NT>
hipError_t launch_band(const BandArgs& a, const BandPlan& p, hipStream_t s)
{
    auto kernel = igemm_band_kernel<UPX, 3, 3, NT>;
    static size_t lds_allowed = 64 * 1024;  // the default dynamic LDS limit
    if (p.lds > lds_allowed) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(p.lds));
        if (e != hipSuccess) return e;
        lds_allowed = p.lds;
    }
    return launch(kernel, dim3(p.bands, a.g.G * p.co_tiles), dim3(kThreads), p.lds, s, a);
}

}  // namespace

bool can_igemm_band(const Geom& g, int dtype)
{
    if (dtype != 1 || !g.nhwc || !g.aligned16) return false;
    if (g.Mg % 4 != 0) return false;
    const int64_t x_bytes = static_cast<int64_t>(g.N) * g.H * g.W * g.C * 2;
    const int64_t y_bytes = static_cast<int64_t>(g.N) * g.OH * g.OW * g.CO * 2;
    const int64_t w_bytes = static_cast<int64_t>(g.CO) * g.KH * g.KW * g.Cg * 2;
    const int64_t lim = int64_t(1) << 31;
    if (x_bytes >= lim || y_bytes >= lim || w_bytes >= lim) return false;
    return make_band_plan(g, 256).ok;
}

// Whether the band kernel beats the generic implicit GEMM: when each band
// is one group of 64-channel groups (on a device of 256 CUs).  Measured
// against eight-wave igemm, 3x3 x 32 images (event-timed, both paths
// forced): 64 -> 64 channels at 56x56 26.8 against 28.2 us, at 28x28 20.6
// against 21.3, stride 2 at 56x56 21.6 against 22.6, 64 -> 128 channels x 16
// images 24.8 against 26.5; but 32 -> 32 channels 21.6 against 19.8,
// 16 -> 16 19.3 against 17.6, and 112x112 (28 rows per band, several
// groups) 126.7 against 66.1.
bool igemm_band_preferred(const Geom& g)
{
    const BandPlan p = make_band_plan(g, 256);
    return p.ok && p.one_group && g.Cg == 64;
}

hipError_t launch_igemm_band(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                             hipStream_t s)
{
    const BandPlan p = make_band_plan(g, device_cu_count());
    if (!p.ok) return hipErrorInvalidValue;
    BandArgs a;
    a.x = static_cast<const bf16_t*>(x);
    a.w = static_cast<const bf16_t*>(w);
    a.bias = static_cast<const bf16_t*>(bias);
    a.y = static_cast<bf16_t*>(y);
    a.g = g;
    a.TW = p.TW;
    a.IC = p.IC;
    a.col_tiles = p.col_tiles;
    a.Gmax = p.Gmax;
    a.ring = p.ring;
    a.row_units = p.row_units;
    a.w_units = p.w_units;
    a.total_rows = static_cast<int>(static_cast<int64_t>(g.N) * p.col_tiles * g.OH);
    a.bands = p.bands;
    a.co_tiles = p.co_tiles;
    a.stage_last = p.stage_last;
    a.div_oh = make_fastdiv(static_cast<uint32_t>(g.OH));
    a.div_ct = make_fastdiv(static_cast<uint32_t>(p.col_tiles));
    a.div_tw = make_fastdiv(static_cast<uint32_t>(p.TW));
    a.div_wrow = make_fastdiv(static_cast<uint32_t>(g.KH * g.KW * p.UPX + 1));
    switch (p.UPX * 10 + p.NT) {
    case 82: return launch_band<8, 2>(a, p, s);
    case 81: return launch_band<8, 1>(a, p, s);
    case 42: return launch_band<4, 2>(a, p, s);
    case 41: return launch_band<4, 1>(a, p, s);
    case 22: return launch_band<2, 2>(a, p, s);
    default: return launch_band<2, 1>(a, p, s);
    }
}

}  // namespace convmi
