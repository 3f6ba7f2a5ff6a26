// Depthwise and small-group forward convolution: a direct, HBM-bound kernel.
//
// With C/G = 1 each output is a per-channel 2-D cross-correlation,
// y[n, oh, ow, c] = bias[c] + sum_{kh, kw} x[n, oh*sh - ph + kh*dh,
// ow*sw - pw + kw*dw, c] * w[c, kh, kw], so there is no cross-channel
// contraction for a matrix unit to exploit (the grouped case of teeny-kernels
// 0.2.0 src/nn/conv/conv2d.rs, `conv2d_forward`, with G = C).  With a small
// group, C/G = C_out/G = CG in {2, 4, 8}, output channel co sums over the CG
// input channels of its own group as well, y[.., co] = bias[co] +
// sum_{kh, kw, i} x[.., (co / CG) * CG + i] * w[co, kh, kw, i] (the same
// page's per-group loop over (C_in/G) * KH * KW): a contraction of length
// 9 CG for a 3x3 kernel, which leaves the layer HBM-bound (at CG = 8 and
// bf16, 18 FLOP per byte moved).  Here it runs on the vector units, whose
// dot-product issue rate bounds it from CG = 4 on; bf16 3x3 groups of 4 and
// 8 over a multiple of 64 channels go to the matrix-core kernel of
// grouped.hip instead.
//
// MI355X design.  In NHWC the channels of one pixel are contiguous, so a lane
// owns 16 bytes of channels (8 bf16 or 4 fp32) and a wavefront covers
// 64 x 16 = 1 KB of contiguous memory per load.
//
// A lane's 16 bytes of channels then hold whole groups (CG divides the vector
// width), whose inputs are exactly the lane's own input channels: the
// arithmetic below changes, the data movement does not.
//
// Unit stride with a compile-time kernel and dilation takes the streaming
// kernel: a lane walks down one output column over a segment of rows.  Each
// input row it needs is loaded once per kernel column, several rows ahead of
// use, into a per-wave LDS ring (buffer-to-LDS loads), and feeds every output
// row that reads it; finished output rows are stored as the walk passes them.
// Accumulators are indexed by compile-time slots (the loop is unrolled by
// their ring length), padding rows and columns load as zero through
// buffer-resource bounds, so the loop has no data-dependent branches.  The
// arithmetic is what bounds the walk next to HBM, so bf16 taps are paired
// into dot products and never widened.  Workgroups are numbered so that every
// XCD receives a contiguous run of whole images: the halo rows and columns
// that neighbouring workgroups share are then served by the same L2.
//
// Other shapes take a generic strip kernel that loads per tap.  Accumulation
// is fp32 and includes the bias, and each output is rounded once.
#include "kernels.hpp"

#include <algorithm>
#include <type_traits>

namespace convmi {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin over 8 XCDs

template <typename T>
struct Vec;
template <>
struct Vec<bf16_t> {
    static constexpr int N = 8;
    __device__ static void unpack(const uint4& v, float* f)
    {
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    __device__ static uint4 pack(const float* f)
    {
        return uint4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7])};
    }
};
template <>
struct Vec<float> {
    static constexpr int N = 4;
    __device__ static void unpack(const uint4& v, float* f)
    {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    __device__ static uint4 pack(const float* f)
    {
        return uint4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                     __float_as_uint(f[3])};
    }
};

// Work decomposition shared by both kernels.  Workgroup b covers kThreads
// consecutive (column, channel-vector) slots of one (image, row segment);
// segments are `seg_rows` output rows tall.  The launch order is remapped so
// that XCD k (which receives workgroups k, k+8, ...) gets a contiguous block
// of logical workgroups when the count divides evenly.
struct Slot {
    int cg, ow, n, oh_begin, oh_end;
    bool live;
};
__device__ __forceinline__ Slot slot_of(const Geom& g, int cgroups, int col_blocks, int segs,
                                        int seg_rows, int lanes = kThreads)
{
    // Workgroup b runs on XCD b mod 8; the grid is a multiple of 8 and the
    // remap gives each XCD a contiguous run of workgroups, so neighbouring
    // segments share an L2.  Padding workgroups get an image past the last.
    const int nb = gridDim.x;
    const int b = (static_cast<int>(blockIdx.x) % kXcds) * (nb / kXcds) + static_cast<int>(blockIdx.x) / kXcds;
    const int colb = b % col_blocks;
    const int rest = b / col_blocks;
    const int seg = rest % segs;
    Slot s;
    s.n = rest / segs;
    const int f = colb * lanes + threadIdx.x;
    s.live = static_cast<int>(threadIdx.x) < lanes && f < g.OW * cgroups;
    s.cg = f % cgroups;
    s.ow = f / cgroups;
    s.oh_begin = seg * seg_rows;
    s.oh_end = min(g.OH, s.oh_begin + seg_rows);
    return s;
}

// The lane's OV bias values (a whole vector, or half of a bf16 one) as one
// load; a null bias is a resource of zero bytes, whose loads return zero.
template <typename T, int OV>
__device__ __forceinline__ void load_bias(const T* bias, int C, int c0, float (&b)[OV])
{
    const rsrc_t br = make_rsrc(bias, bias ? static_cast<uint32_t>(C) * sizeof(T) : 0u);
    if constexpr (OV == Vec<T>::N) {
        Vec<T>::unpack(buffer_load16(br, static_cast<uint32_t>(c0) * sizeof(T)), b);
    } else {
        static_assert(sizeof(T) == 2 && OV == 4, "half vectors exist for bf16 only");
        const uint2 v = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(br, static_cast<uint32_t>(c0) * 2u, 0, 0));
        b[0] = __uint_as_float(v.x << 16);
        b[1] = __uint_as_float(v.x & 0xffff0000u);
        b[2] = __uint_as_float(v.y << 16);
        b[3] = __uint_as_float(v.y & 0xffff0000u);
    }
}

// Lanes per input vector in the streaming walk.  A bf16 lane that owned all
// eight outputs of an eight-channel group would hold 288 weight registers
// for a 3x3 kernel, more than a lane has; two lanes then share the input
// vector and each computes four of its outputs.
template <typename T, int CG>
constexpr int lanes_per_vector()
{
    return sizeof(T) == 2 && CG == 8 ? 2 : 1;
}

// Tap arithmetic of the streaming walk.  A lane receives the V channels of
// one input pixel as one 16-byte vector per kernel column; `row` turns the KW
// vectors of an input row into operands and `dot` adds the KW taps of kernel
// row kh for channel e to an accumulator.  With C/G = 1 a lane's channels keep
// their taps back to back in w[c][kh][kw], so its weights are TAPS 16-byte
// vectors starting at channel c0.
template <typename T, int KH, int KW, int CG = 1, int MG = 1>
struct TapMath;

// Depthwise with a channel multiplier MG (C/G = 1, C_out/G = MG): a lane's
// V outputs co0 .. co0 + V - 1 read the V / MG input channels from co0 / MG,
// which sit at sub-vector k = (co0 / MG) % V / (V / MG) of an aligned input
// vector.  `select` moves those channels to the front of the vector (one or
// two v_cndmask per dword), so that output e reads channel e / MG at a
// compile-time position.  With MG = 1 it is the identity.
template <int MG, int V>
__device__ __forceinline__ uint4 select_sub(uint4 u, int k)
{
    // The components pass through an empty asm so that the selects below
    // act on register values: selects between two loads of one local array
    // would otherwise be folded into one load at a lane-dependent address,
    // which moves the array to scratch memory, and the kernel's walk would
    // then wait on those scratch loads (vmcnt) at every row.
    if constexpr (MG != 1) asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
    if constexpr (MG == 1) {
        return u;
    } else if constexpr (V / MG == 4) {  // bf16 x2: two dwords
        return uint4{k ? u.z : u.x, k ? u.w : u.y, 0u, 0u};
    } else if constexpr (V / MG == 2 && V == 8) {  // bf16 x4: one dword
        const uint32_t lo = k & 1 ? u.y : u.x, hi = k & 1 ? u.w : u.z;
        return uint4{k & 2 ? hi : lo, 0u, 0u, 0u};
    } else if constexpr (V / MG == 1 && V == 8) {  // bf16 x8: half a dword
        const uint32_t lo = k & 2 ? u.y : u.x, hi = k & 2 ? u.w : u.z;
        const uint32_t d = k & 4 ? hi : lo;
        return uint4{k & 1 ? d >> 16 : d, 0u, 0u, 0u};
    } else if constexpr (V / MG == 2) {  // fp32 x2: two floats
        return uint4{k ? u.z : u.x, k ? u.w : u.y, 0u, 0u};
    } else {  // fp32 x4: one float
        static_assert(V == 4 && MG == 4, "multiplier not supported");
        const uint32_t lo = k & 1 ? u.y : u.x, hi = k & 1 ? u.w : u.z;
        return uint4{k & 2 ? hi : lo, 0u, 0u, 0u};
    }
}

// fp32: one FMA per tap and channel.
template <int KH, int KW, int MG>
struct TapMath<float, KH, KW, 1, MG> {
    static constexpr int OV = 4;  // outputs per lane
    static constexpr int TAPS = KH * KW;
    float wt[KH][KW][4];
    struct Row {
        float x[KW][4];
    };
    __device__ void load(const float* w, int c0)
    {
        const uint4* wv = reinterpret_cast<const uint4*>(w + static_cast<int64_t>(c0) * TAPS);
        float flat[TAPS * 4];
#pragma unroll
        for (int i = 0; i < TAPS; ++i) Vec<float>::unpack(wv[i], flat + i * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int t = 0; t < TAPS; ++t) wt[t / KW][t % KW][e] = flat[e * TAPS + t];
    }
    __device__ static Row row(const uint4 (&u)[KW], int k)
    {
        Row r;
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) Vec<float>::unpack(select_sub<MG, 4>(u[kw], k), r.x[kw]);
        return r;
    }
    __device__ float dot(const Row& r, int kh, int e, float c) const
    {
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) c = fmaf(r.x[kw][e / MG], wt[kh][kw][e], c);
        return c;
    }
};

// bf16: neighbouring kernel columns are paired and each pair costs one
// v_dot2_f32_bf16 (two exact bf16 products added to an fp32 accumulator), so
// the inputs are never widened to fp32.  A byte permute regroups the two
// columns' vectors into per-channel pairs; with KW odd the last column is
// taken against a weight pair holding zero in the other channel's half.
template <int KH, int KW, int MG>
struct TapMath<bf16_t, KH, KW, 1, MG> {
    static constexpr int OV = 8;
    static constexpr int TAPS = KH * KW;
    static constexpr int NP = KW / 2;
    static constexpr bool ODD = KW % 2 != 0;
    uint32_t wp[KH][NP > 0 ? NP : 1][8];  // channel e: {w[e][kh][2p], w[e][kh][2p+1]}
    uint32_t ws[KH][8];                   // output e: w[e][kh][KW-1] in the half of its input channel
    struct Row {
        uint32_t lo[NP > 0 ? NP : 1][4], hi[NP > 0 ? NP : 1][4];  // channel 2d / 2d+1 pairs
        uint32_t last[4];
    };
    __device__ void load(const bf16_t* w, int c0)
    {
        const uint4* wv = reinterpret_cast<const uint4*>(w + static_cast<int64_t>(c0) * TAPS);
        uint32_t words[TAPS * 4];
#pragma unroll
        for (int i = 0; i < TAPS; ++i) {
            const uint4 v = wv[i];
            words[4 * i] = v.x; words[4 * i + 1] = v.y; words[4 * i + 2] = v.z; words[4 * i + 3] = v.w;
        }
        // bf16 number k of the lane's run (channel k / TAPS, tap k % TAPS)
        auto h = [&](int k) __attribute__((always_inline)) {
            return (words[k >> 1] >> (16 * (k & 1))) & 0xffffu;
        };
#pragma unroll
        for (int kh = 0; kh < KH; ++kh)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    wp[kh][p][e] = h(e * TAPS + kh * KW + 2 * p) | (h(e * TAPS + kh * KW + 2 * p + 1) << 16);
                ws[kh][e] = h(e * TAPS + kh * KW + KW - 1) << (16 * ((e / MG) & 1));
            }
    }
    __device__ static Row row(const uint4 (&u0)[KW], int k)
    {
        uint4 u[KW];
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) u[kw] = select_sub<MG, 8>(u0[kw], k);
        Row r;
        constexpr int ND = (8 / MG + 1) / 2;  // dwords holding the lane's input channels
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            if (d >= ND) continue;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const uint32_t a = (&u[2 * p].x)[d], b = (&u[2 * p + 1].x)[d];
                r.lo[p][d] = __builtin_amdgcn_perm(b, a, 0x05040100u);  // {a.lo, b.lo}
                r.hi[p][d] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // {a.hi, b.hi}
            }
            r.last[d] = (&u[KW - 1].x)[d];
        }
        return r;
    }
    __device__ float dot(const Row& r, int kh, int e, float c) const
    {
        const int ch = e / MG;  // the output's input channel within the lane's channels
        const int d = ch >> 1;
#pragma unroll
        for (int p = 0; p < NP; ++p)
            c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, (ch & 1) ? r.hi[p][d] : r.lo[p][d]),
                                                __builtin_bit_cast(bf16x2_t, wp[kh][p][e]), c, false);
        if (ODD)
            c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, r.last[d]),
                                                __builtin_bit_cast(bf16x2_t, ws[kh][e]), c, false);
        return c;
    }
};

// Groups of CG > 1 channels (C_out = C).  Output channel co keeps its
// TAPS x CG weights back to back in w[co][kh][kw][i], so the weights of a
// lane's OV outputs are one run of OV * TAPS * CG values from its first
// output channel.  Output e of a lane that owns the whole vector belongs to
// group e / CG, whose inputs are channels (e / CG) * CG ... + CG - 1 of each
// input vector.
//
// fp32: one FMA per tap and input channel.
template <typename T, int KH, int KW, int CG>
struct TapMathGroup;
template <int KH, int KW, int CG>
struct TapMathGroup<float, KH, KW, CG> {
    static_assert(CG == 2 || CG == 4, "fp32 groups must divide the 4-channel vector");
    static constexpr int OV = 4;
    static constexpr int TAPS = KH * KW;
    float wt[KH][KW][4][CG];
    struct Row {
        float x[KW][4];
    };
    __device__ void load(const float* w, int c0)
    {
        const uint4* wv = reinterpret_cast<const uint4*>(w + static_cast<int64_t>(c0) * TAPS * CG);
        float flat[4 * TAPS * CG];
#pragma unroll
        for (int i = 0; i < TAPS * CG; ++i) Vec<float>::unpack(wv[i], flat + 4 * i);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int t = 0; t < TAPS; ++t)
#pragma unroll
                for (int i = 0; i < CG; ++i) wt[t / KW][t % KW][e][i] = flat[(e * TAPS + t) * CG + i];
    }
    __device__ static Row row(const uint4 (&u)[KW], int /*k: no multiplier*/)
    {
        Row r;
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) Vec<float>::unpack(u[kw], r.x[kw]);
        return r;
    }
    __device__ float dot(const Row& r, int kh, int e, float c) const
    {
        const int c_in = (e / CG) * CG;
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
#pragma unroll
            for (int i = 0; i < CG; ++i) c = fmaf(r.x[kw][c_in + i], wt[kh][kw][e][i], c);
        return c;
    }
};

// bf16: the group's input channels come as bf16 pairs already (dword d of a
// vector holds channels 2d, 2d + 1), so each pair against the matching
// weight pair is one v_dot2_f32_bf16 with no regrouping.  With CG = 8 the
// lane computes OV = 4 outputs (see lanes_per_vector), all of the one group
// that fills the vector.
template <int KH, int KW, int CG>
struct TapMathGroup<bf16_t, KH, KW, CG> {
    static_assert(CG == 2 || CG == 4 || CG == 8, "bf16 groups must divide the 8-channel vector");
    static constexpr int OV = 8 / lanes_per_vector<bf16_t, CG>();
    static constexpr int TAPS = KH * KW;
    static constexpr int PR = CG / 2;  // input-channel pairs per group
    uint32_t wt[KH][KW][OV][PR];       // {w[e][kh][kw][2p], w[e][kh][kw][2p+1]}
    struct Row {
        uint32_t x[KW][4];
    };
    __device__ void load(const bf16_t* w, int c0)
    {
        const uint4* wv = reinterpret_cast<const uint4*>(w + static_cast<int64_t>(c0) * TAPS * CG);
#pragma unroll
        for (int i = 0; i < OV * TAPS * PR / 4; ++i) {
            const uint4 v = wv[i];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = 4 * i + j;  // dword k of the run: channel k / (TAPS PR), then tap, then pair
                const int e = k / (TAPS * PR), t = (k / PR) % TAPS, p = k % PR;
                wt[t / KW][t % KW][e][p] = d[j];
            }
        }
    }
    __device__ static Row row(const uint4 (&u)[KW], int /*k: no multiplier*/)
    {
        Row r;
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) {
            r.x[kw][0] = u[kw].x; r.x[kw][1] = u[kw].y; r.x[kw][2] = u[kw].z; r.x[kw][3] = u[kw].w;
        }
        return r;
    }
    __device__ float dot(const Row& r, int kh, int e, float c) const
    {
        const int d0 = OV == 8 ? (e / CG) * PR : 0;
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
#pragma unroll
            for (int p = 0; p < PR; ++p)
                c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, r.x[kw][d0 + p]),
                                                    __builtin_bit_cast(bf16x2_t, wt[kh][kw][e][p]), c, false);
        return c;
    }
};

// LDS row slots per wave: three rows in flight ahead of the one in use.
constexpr int kRS = 4;
// Waves the launch aims at.  Fewer, longer walks stream better than many
// short ones: with one wave per CU-SIMD the concurrent 1 KiB streams stay
// few enough that HBM sees long runs, and every extra segment re-reads its
// halo rows.  (Measured on the 56x56x256 dilated 3x3 case: one segment per
// column and a 4-slot ring ran at 4.5 TB/s; two segments, 8-wave
// workgroups or 2-wave workgroups were 15-25% slower.)
// The same target holds for small groups, where the walk is bound by its dot
// products rather than by HBM (measured with 32 groups of 4 channels,
// C = 128 at 56x56: 1024 waves 17.7 us, 2048 19.5, 4096 26.8).
constexpr int kWaveTarget = 1024;

// Unit stride, compile-time kernel and dilation: the streaming walk.
//   L  = (KH-1)*DH + 1 output rows are live at once (accumulator ring);
//   each wave stages its input rows in a private LDS ring of RS row slots
//   (KW x 1 KiB each: the lane's 16 bytes at its KW column taps), filled by
//   buffer-to-LDS loads RS - 1 rows ahead.  The loads are invisible to the
//   compiler, so it never drains them; the wave waits for a row with one
//   fixed vmcnt (the loads and stores issued after it), and since loads and
//   stores retire in issue order, that wait never covers the later stores.
// Row i of the walk feeds output i - kh*DH through kernel row kh; the
// accumulator of an output starts from the bias with its kh = 0 term.
// Offsets that must read zero or be dropped are pushed past the end of their
// buffer resource: an input row outside the image starts at the image's end,
// a column outside it (or a lane past the last column) adds kOutside, and the
// sum of the two stays below 2^32 because images are under 2 GiB.
//
// With a channel multiplier MG (C/G = 1, C_out/G = MG) a lane owns V output
// channels co0 .. co0 + V - 1, stages the aligned input vector that holds
// their V / MG input channels, and picks those out when it builds a row's
// operands; input and output pixels then differ in size.
template <typename T, int KH, int KW, int DH, int DW, int RS, int CG, int MG = 1>
__global__ __launch_bounds__(kThreads) void depthwise_stream_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, Geom g, int cgroups, int col_blocks, int segs, int seg_rows)
{
    constexpr int V = Vec<T>::N;
    static_assert(MG == 1 || CG == 1, "multipliers with one input channel per group");
    using TM = std::conditional_t<CG == 1, TapMath<T, KH, KW, 1, MG>, TapMathGroup<T, KH, KW, CG>>;
    constexpr int OV = TM::OV;                    // outputs per lane
    constexpr int HV = V / OV;                    // lanes per input vector
    constexpr int L = (KH - 1) * DH + 1;
    constexpr int PF = RS - 1;                    // rows in flight ahead of the one in use
    __shared__ uint4 lds[(kThreads / 64) * RS * KW * 64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    uint4* const my = lds + wave * (RS * KW * 64);  // this wave's ring: [slot][kw][lane]
    const Slot s = slot_of(g, cgroups, col_blocks & 0xffff, segs, seg_rows, col_blocks >> 16);
    if (s.n >= g.N) return;  // grid padding (the whole workgroup)
    // Lanes past the last column keep walking (their loads read zero and
    // their stores are dropped) so the wave's loads stay uniform.  The lane
    // reads input channels c0 .. c0 + V - 1 and writes outputs co0 ..
    // co0 + OV - 1.
    // With a multiplier: output vector s.cg, whose input channels are
    // sub-vector k of aligned input vector s.cg / MG.
    const int c0 = s.live ? (MG > 1 ? s.cg / MG * V : s.cg / HV * V) : 0;
    const int co0 = s.live ? (MG > 1 ? s.cg * V : c0 + s.cg % HV * OV) : 0;
    const int k_sub = MG > 1 ? s.cg % MG : 0;

    const int n_u = __builtin_amdgcn_readfirstlane(s.n);  // uniform: resources live in scalar registers
    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * sizeof(T);     // input pixel
    const uint32_t opix_bytes = static_cast<uint32_t>(g.CO) * sizeof(T);   // output pixel
    const uint32_t lane_bytes = static_cast<uint32_t>(c0) * sizeof(T);
    const uint32_t row_bytes = static_cast<uint32_t>(g.W) * pix_bytes;
    const uint32_t img_bytes = row_bytes * static_cast<uint32_t>(g.H);
    const uint32x4_t xr = dma_rsrc(x + static_cast<int64_t>(n_u) * g.H * g.W * g.C, img_bytes);
    uint32_t col_off[KW];
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) {
        const int iw = s.ow - g.pw + kw * DW;
        col_off[kw] = s.live && static_cast<unsigned>(iw) < static_cast<unsigned>(g.W)
                          ? static_cast<uint32_t>(iw) * pix_bytes + lane_bytes
                          : kOutside;
    }
    // Input row i of the walk is image row r_start + i.  Every segment has a
    // row (the segments split OH), which the compiler is told, so that the
    // walk below is not guarded by a branch the weight and bias loads could
    // be moved behind (past the rows' loads).
    const int count = s.oh_end - s.oh_begin;
    __builtin_assume(count > 0);
    const int nrows = count + L - 1;
    const int r_start = s.oh_begin - g.ph;
    auto issue_row = [&](int i, int slot) __attribute__((always_inline)) {
        const int r = r_start + i;
        const uint32_t roff = static_cast<unsigned>(r) < static_cast<unsigned>(g.H) && i < nrows
                                  ? static_cast<uint32_t>(r) * row_bytes
                                  : img_bytes;
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) dma16(xr, roff + col_off[kw], lds_addr(my + (slot * KW + kw) * 64));
    };
    const uint32_t yrow_bytes = static_cast<uint32_t>(g.OW) * opix_bytes;
    const uint32_t yimg_bytes = yrow_bytes * static_cast<uint32_t>(g.OH);
    const rsrc_t yr = make_rsrc(y + static_cast<int64_t>(n_u) * g.OH * g.OW * g.CO, yimg_bytes);
    const uint32_t ycol_off =
        s.live ? static_cast<uint32_t>(s.ow) * opix_bytes + static_cast<uint32_t>(co0) * sizeof(T) : kOutside;

    // Each row's loads are followed by one store (of the row finished then);
    // the first PF rows get a dropped store each, so the count of operations
    // issued after any row's loads is the same from the first row on.
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        issue_row(u, u);
        buffer_store16(yr, kOutside, uint4{0u, 0u, 0u, 0u});
    }
    // The weights and bias load behind the first rows' loads, so the two
    // latencies overlap; once both have landed no load the compiler tracks
    // is outstanding, and the walk's own counted waits are the only ones in
    // its loop.
    TM tm;
    tm.load(w, co0);
    float b[OV];
    load_bias<T, OV>(bias, g.CO, co0, b);
    wait_vm<0>();

    // Slots of outputs before the segment collect partial sums that are never
    // stored; they start at zero only to keep the registers defined.
    float acc[L][OV];
#pragma unroll
    for (int j = 0; j < L; ++j)
#pragma unroll
        for (int e = 0; e < OV; ++e) acc[j][e] = 0.f;

    // The walk runs in whole periods of L rows, so that accumulator slot
    // (i mod L) is compile-time; the ring slot (i mod RS) is counted.  Rows
    // past nrows load as zero and their stores are dropped.
    int slot = 0;  // ring slot of row i
    for (int it = 0; it < nrows; it += L) {
#pragma unroll
        for (int u = 0; u < L; ++u) {
            const int i = it + u;
            const int slot_pf = slot == 0 ? RS - 1 : slot - 1;  // (i + PF) mod RS: the slot row i - 1 used
            issue_row(i + PF, slot_pf);
            // Row i landed once at most the loads of rows i+1 .. i+PF and the
            // stores of the PF previous rows are outstanding.
            wait_vm<PF * KW + PF>();
            asm volatile("" ::: "memory");
            uint4 raw[KW];
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) raw[kw] = my[(slot * KW + kw) * 64 + lane];
            slot = slot == RS - 1 ? 0 : slot + 1;
            const typename TM::Row row = TM::row(raw, k_sub);
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int as = ((u - kh * DH) % L + L) % L;
#pragma unroll
                for (int e = 0; e < OV; ++e) acc[as][e] = tm.dot(row, kh, e, kh == 0 ? b[e] : acc[as][e]);
            }
            // Output j = i - (L-1) has now received every tap.
            const int jd = i - (L - 1);
            const uint32_t yro = jd >= 0 && jd < count ? static_cast<uint32_t>(s.oh_begin + jd) * yrow_bytes
                                                       : yimg_bytes;
            if constexpr (OV == V) {
                buffer_store16_nt(yr, yro + ycol_off, Vec<T>::pack(acc[(u + 1) % L]));
            } else {
                const float* o = acc[(u + 1) % L];
                buffer_store8_nt(yr, yro + ycol_off, uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])});
            }
        }
    }
}

// Any stride, kernel extent and dilation: a strip of kRH rows, per-tap loads.
constexpr int kRH = 8;
template <typename T, int CG>
__global__ __launch_bounds__(kThreads) void depthwise_generic_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, Geom g, int cgroups, int col_blocks, int segs, int seg_rows)
{
    constexpr int V = Vec<T>::N;
    const Slot s = slot_of(g, cgroups, col_blocks, segs, seg_rows);
    if (s.n >= g.N) return;  // grid padding (the whole workgroup)
    if (!s.live) return;
    const int c0 = s.cg * V;
    const int taps = g.KH * g.KW;
    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * sizeof(T);
    const rsrc_t xr = make_rsrc(x + static_cast<int64_t>(s.n) * g.H * g.W * g.C,
                                static_cast<uint32_t>(g.H) * g.W * pix_bytes);
    const uint32_t lane_off = static_cast<uint32_t>(c0) * sizeof(T);
    float b[V];
    load_bias<T>(bias, g.C, c0, b);
    for (int oh0 = s.oh_begin; oh0 < s.oh_end; oh0 += kRH) {
        float acc[kRH][V];
#pragma unroll
        for (int j = 0; j < kRH; ++j)
#pragma unroll
            for (int e = 0; e < V; ++e) acc[j][e] = 0.f;
        for (int kh = 0; kh < g.KH; ++kh) {
            for (int kw = 0; kw < g.KW; ++kw) {
                const int iw = s.ow * g.sw - g.pw + kw * g.dw;
                const bool col_in = static_cast<unsigned>(iw) < static_cast<unsigned>(g.W);
                float wv[V][CG];
#pragma unroll
                for (int e = 0; e < V; ++e)
#pragma unroll
                    for (int i = 0; i < CG; ++i)
                        wv[e][i] = load_f(w + (static_cast<int64_t>(c0 + e) * taps + kh * g.KW + kw) * CG + i);
#pragma unroll
                for (int j = 0; j < kRH; ++j) {
                    const int ih = (oh0 + j) * g.sh - g.ph + kh * g.dh;
                    const bool in = col_in && static_cast<unsigned>(ih) < static_cast<unsigned>(g.H);
                    const uint32_t off =
                        in ? (static_cast<uint32_t>(ih) * g.W + iw) * pix_bytes + lane_off : kOutside;
                    float xv[V];
                    Vec<T>::unpack(buffer_load16(xr, off), xv);
#pragma unroll
                    for (int e = 0; e < V; ++e)
#pragma unroll
                        for (int i = 0; i < CG; ++i)
                            acc[j][e] = fmaf(xv[(e / CG) * CG + i], wv[e][i], acc[j][e]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kRH; ++j) {
            const int oh = oh0 + j;
            if (oh >= s.oh_end) break;
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = acc[j][e] + b[e];
            T* yp = y + ((static_cast<int64_t>(s.n) * g.OH + oh) * g.OW + s.ow) * g.C + c0;
            *reinterpret_cast<uint4*>(yp) = Vec<T>::pack(o);
        }
    }
}

// Channel multipliers: C_out/G = MG output channels per group, a
// power-of-two multiple of C/G = CG input channels (MG / CG = 2, 4 or 8; with
// CG = 1 a depthwise convolution with that multiplier).  Output channel co
// reads input channels (co / MG) * CG .. + CG - 1 (teeny-kernels
// src/nn/conv/conv2d.rs, `conv2d_forward`: group g = c_out / (C_OUT / G)).  A
// lane owns V consecutive output channels co0 .. co0 + V - 1; the input
// channels they read form one aligned window of WD = max(V / MG, 1) * CG
// channels starting at (co0 / MG) * CG, loaded once per tap as one 2- to
// 16-byte buffer load, and output e takes its input i from window position
// (e / MG) * CG + i when MG <= V (else i): every index is compile-time.
template <typename T, int WD>
__device__ __forceinline__ void load_window(rsrc_t r, uint32_t off, float (&f)[WD])
{
    constexpr int bytes = WD * static_cast<int>(sizeof(T));
    if constexpr (bytes == 16) {
        Vec<T>::unpack(buffer_load16(r, off), f);
    } else if constexpr (bytes == 8) {
        const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
        if constexpr (sizeof(T) == 2) {
            f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
            f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
        } else {
            f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        }
    } else if constexpr (bytes == 4) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        if constexpr (sizeof(T) == 2) {
            f[0] = __uint_as_float(v << 16); f[1] = __uint_as_float(v & 0xffff0000u);
        } else {
            f[0] = __uint_as_float(v);
        }
    } else {
        static_assert(bytes == 2, "window of one bf16 channel");
        const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
        f[0] = __uint_as_float(static_cast<uint32_t>(v) << 16);
    }
}

template <typename T, int CG, int MG>
__global__ __launch_bounds__(kThreads) void depthwise_mult_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, Geom g, int cgroups, int col_blocks, int segs, int seg_rows)
{
    constexpr int V = Vec<T>::N;
    constexpr int WD = (MG <= V ? V / MG : 1) * CG;  // input window of the lane
    const Slot s = slot_of(g, cgroups, col_blocks, segs, seg_rows);
    if (s.n >= g.N) return;  // grid padding (the whole workgroup)
    if (!s.live) return;
    const int co0 = s.cg * V;
    const int in0 = co0 / MG * CG;
    const int taps = g.KH * g.KW;
    const uint32_t pix_bytes = static_cast<uint32_t>(g.C) * sizeof(T);
    const rsrc_t xr = make_rsrc(x + static_cast<int64_t>(s.n) * g.H * g.W * g.C,
                                static_cast<uint32_t>(g.H) * g.W * pix_bytes);
    const uint32_t lane_off = static_cast<uint32_t>(in0) * sizeof(T);
    float b[V];
    load_bias<T>(bias, g.CO, co0, b);
    for (int oh0 = s.oh_begin; oh0 < s.oh_end; oh0 += kRH) {
        float acc[kRH][V];
#pragma unroll
        for (int j = 0; j < kRH; ++j)
#pragma unroll
            for (int e = 0; e < V; ++e) acc[j][e] = 0.f;
        for (int kh = 0; kh < g.KH; ++kh) {
            for (int kw = 0; kw < g.KW; ++kw) {
                const int iw = s.ow * g.sw - g.pw + kw * g.dw;
                const bool col_in = static_cast<unsigned>(iw) < static_cast<unsigned>(g.W);
                float wv[V][CG];
#pragma unroll
                for (int e = 0; e < V; ++e)
#pragma unroll
                    for (int i = 0; i < CG; ++i)
                        wv[e][i] = load_f(w + (static_cast<int64_t>(co0 + e) * taps + kh * g.KW + kw) * CG + i);
#pragma unroll
                for (int j = 0; j < kRH; ++j) {
                    const int ih = (oh0 + j) * g.sh - g.ph + kh * g.dh;
                    const bool in = col_in && static_cast<unsigned>(ih) < static_cast<unsigned>(g.H);
                    const uint32_t off =
                        in ? (static_cast<uint32_t>(ih) * g.W + iw) * pix_bytes + lane_off : kOutside;
                    float xv[WD];
                    load_window<T, WD>(xr, off, xv);
#pragma unroll
                    for (int e = 0; e < V; ++e)
#pragma unroll
                        for (int i = 0; i < CG; ++i)
                            acc[j][e] = fmaf(xv[(MG <= V ? e / MG : 0) * CG + i], wv[e][i], acc[j][e]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kRH; ++j) {
            const int oh = oh0 + j;
            if (oh >= s.oh_end) break;
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = acc[j][e] + b[e];
            T* yp = y + ((static_cast<int64_t>(s.n) * g.OH + oh) * g.OW + s.ow) * g.CO + co0;
            *reinterpret_cast<uint4*>(yp) = Vec<T>::pack(o);
        }
    }
}

template <typename T, int CG, int MG>
hipError_t launch_mult(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                       hipStream_t s)
{
    constexpr int V = Vec<T>::N;
    const int cgroups = g.CO / V;  // lane slots per pixel: one per output vector
    const int col_blocks = (g.OW * cgroups + kThreads - 1) / kThreads;
    const int64_t waves_per_seg = static_cast<int64_t>(g.N) * col_blocks * (kThreads / 64);
    int segs = static_cast<int>(kWaveTarget / waves_per_seg);
    segs = max(1, min(segs, g.OH / 8));
    const int seg_rows = (g.OH + segs - 1) / segs;
    segs = (g.OH + seg_rows - 1) / seg_rows;
    const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(g.N) * segs * col_blocks + kXcds - 1) / kXcds * kXcds));
    return launch(depthwise_mult_kernel<T, CG, MG>, grid, dim3(kThreads), 0, s, static_cast<const T*>(x),
                  static_cast<const T*>(w), static_cast<const T*>(bias), static_cast<T*>(y), g, cgroups,
                  col_blocks, segs, seg_rows);
}

// Input gradient of a small-group convolution (C/G = C_out/G = CG, up to one
// vector): dx[n, ih, iw, ci] = sum over the taps (kh, kw) whose output
// position oh = (ih + ph - kh*dh) / sh (integral, in range; likewise ow)
// exists and over the CG output channels co of ci's group of
// dy[n, oh, ow, co] * w[co, kh, kw, ci mod CG] -- the gather form of the
// adjoint, each dx element written once (teeny-kernels
// src/nn/conv/conv2d.rs `conv2d_backward_dx` scatters the same sum with
// atomics).  With C_out/G = C/G the output channels of a lane's groups have
// the same indices as its input channels, so the dy vector at the lane's
// channels holds them all.  A lane owns V consecutive channels of one dx
// pixel and a strip of kRH rows; a per-channel bias (the transposed
// convolution's) is added before the single rounding.
template <typename T, int CG>
__global__ __launch_bounds__(kThreads) void depthwise_dx_kernel(
    const T* __restrict__ dy, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ dx, Geom g, Geom grid_g, int cgroups, int col_blocks, int segs, int seg_rows)
{
    constexpr int V = Vec<T>::N;
    // grid_g is g with the output extent replaced by the input's: the slots
    // run over dx pixels.
    const Slot s = slot_of(grid_g, cgroups, col_blocks, segs, seg_rows);
    if (s.n >= g.N) return;  // grid padding (the whole workgroup)
    if (!s.live) return;
    const int c0 = s.cg * V;
    const int taps = g.KH * g.KW;
    const uint32_t pix_bytes = static_cast<uint32_t>(g.CO) * sizeof(T);
    const rsrc_t dyr = make_rsrc(dy + static_cast<int64_t>(s.n) * g.OH * g.OW * g.CO,
                                 static_cast<uint32_t>(g.OH) * g.OW * pix_bytes);
    const uint32_t lane_off = static_cast<uint32_t>(c0) * sizeof(T);
    float b[V];
    load_bias<T>(bias, g.C, c0, b);
    const int iw = s.ow;  // the dx column of this lane
    for (int ih0 = s.oh_begin; ih0 < s.oh_end; ih0 += kRH) {
        float acc[kRH][V];
#pragma unroll
        for (int j = 0; j < kRH; ++j)
#pragma unroll
            for (int e = 0; e < V; ++e) acc[j][e] = 0.f;
        for (int kw = 0; kw < g.KW; ++kw) {
            const int tw = iw + g.pw - kw * g.dw;
            if (tw < 0 || tw % g.sw != 0 || tw / g.sw >= g.OW) continue;  // no output column
            const int ow = tw / g.sw;
            for (int kh = 0; kh < g.KH; ++kh) {
                float wv[V][CG];
#pragma unroll
                for (int e = 0; e < V; ++e)
#pragma unroll
                    for (int i = 0; i < CG; ++i) {
                        const int co = (c0 + e) / CG * CG + i;
                        wv[e][i] = load_f(w + (static_cast<int64_t>(co) * taps + kh * g.KW + kw) * CG + (c0 + e) % CG);
                    }
#pragma unroll
                for (int j = 0; j < kRH; ++j) {
                    const int th = ih0 + j + g.ph - kh * g.dh;
                    const bool in = th >= 0 && th % g.sh == 0 && th / g.sh < g.OH;
                    const uint32_t off =
                        in ? (static_cast<uint32_t>(th / g.sh) * g.OW + ow) * pix_bytes + lane_off : kOutside;
                    float dv[V];
                    Vec<T>::unpack(buffer_load16(dyr, off), dv);
#pragma unroll
                    for (int e = 0; e < V; ++e)
#pragma unroll
                        for (int i = 0; i < CG; ++i)
                            acc[j][e] = fmaf(dv[(e / CG) * CG + i], wv[e][i], acc[j][e]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kRH; ++j) {
            const int ih = ih0 + j;
            if (ih >= s.oh_end) break;
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = acc[j][e] + b[e];
            T* xp = dx + ((static_cast<int64_t>(s.n) * g.H + ih) * g.W + iw) * g.C + c0;
            *reinterpret_cast<uint4*>(xp) = Vec<T>::pack(o);
        }
    }
}

template <typename T, int CG>
hipError_t launch_dx_small_t(const void* dy, const void* w, const void* bias, void* dx, const Geom& g,
                             hipStream_t s)
{
    constexpr int V = Vec<T>::N;
    Geom grid_g = g;  // the slots run over dx pixels
    grid_g.OH = g.H;
    grid_g.OW = g.W;
    const int cgroups = g.C / V;
    const int col_blocks = (g.W * cgroups + kThreads - 1) / kThreads;
    const int64_t waves_per_seg = static_cast<int64_t>(g.N) * col_blocks * (kThreads / 64);
    int segs = static_cast<int>(kWaveTarget / waves_per_seg);
    segs = max(1, min(segs, g.H / 8));
    const int seg_rows = (g.H + segs - 1) / segs;
    segs = (g.H + seg_rows - 1) / seg_rows;
    const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(g.N) * segs * col_blocks + kXcds - 1) / kXcds * kXcds));
    return launch(depthwise_dx_kernel<T, CG>, grid, dim3(kThreads), 0, s, static_cast<const T*>(dy),
                  static_cast<const T*>(w), static_cast<const T*>(bias), static_cast<T*>(dx), g, grid_g,
                  cgroups, col_blocks, segs, seg_rows);
}

// (C/G, C_out/G) pairs of the multiplier kernel.
template <typename T, int CG, int MG = 1>
hipError_t launch_t(const void* x, const void* w, const void* bias, void* y, const Geom& g, hipStream_t s);

template <typename T>
hipError_t launch_mult_cg(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                          hipStream_t s)
{
    switch (g.Cg * 1000 + g.Mg) {
    // One input channel per group: the streaming walk where the geometry
    // allows it (launch_t falls back to launch_mult otherwise).
    case 1002: return launch_t<T, 1, 2>(x, w, bias, y, g, s);
    case 1004: return launch_t<T, 1, 4>(x, w, bias, y, g, s);
    case 1008:
        if constexpr (Vec<T>::N == 8) return launch_t<T, 1, 8>(x, w, bias, y, g, s);
        return launch_mult<T, 1, 8>(x, w, bias, y, g, s);
    case 2004: return launch_mult<T, 2, 4>(x, w, bias, y, g, s);
    case 2008: return launch_mult<T, 2, 8>(x, w, bias, y, g, s);
    case 2016: return launch_mult<T, 2, 16>(x, w, bias, y, g, s);
    case 4008: return launch_mult<T, 4, 8>(x, w, bias, y, g, s);
    case 4016: return launch_mult<T, 4, 16>(x, w, bias, y, g, s);
    case 4032: return launch_mult<T, 4, 32>(x, w, bias, y, g, s);
    default:
        if constexpr (Vec<T>::N == 8) {
            switch (g.Cg * 1000 + g.Mg) {
            case 8016: return launch_mult<T, 8, 16>(x, w, bias, y, g, s);
            case 8032: return launch_mult<T, 8, 32>(x, w, bias, y, g, s);
            case 8064: return launch_mult<T, 8, 64>(x, w, bias, y, g, s);
            default: break;
            }
        }
        return hipErrorInvalidValue;
    }
}

template <typename T, int CG, int MG>
hipError_t launch_t(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                    hipStream_t s)
{
    constexpr int V = Vec<T>::N;
    const bool unit = g.sh == 1 && g.sw == 1;
    const bool k3d1 = unit && g.KH == 3 && g.KW == 3 && g.dh == 1 && g.dw == 1;
    const bool k3d2 = CG == 1 && unit && g.KH == 3 && g.KW == 3 && g.dh == 2 && g.dw == 2;
    const bool k5d1 = CG == 1 && unit && g.KH == 5 && g.KW == 5 && g.dh == 1 && g.dw == 1;
    // With a multiplier the walk stages whole input vectors, which need
    // input pixels of whole 16-byte vectors (C a multiple of V).
    const bool stream = (k3d1 || k3d2 || k5d1) && (MG == 1 || g.C % V == 0);
    if constexpr (MG > 1) {
        if (!stream) return launch_mult<T, CG, MG>(x, w, bias, y, g, s);
    }
    // Lane slots per pixel: one per input vector, or per half vector where
    // the streaming walk splits a vector's outputs over two lanes; with a
    // multiplier, one per output vector.
    const int cgroups = MG > 1 ? g.CO / V : g.C / V * (stream ? lanes_per_vector<T, CG>() : 1);
    int col_blocks = (g.OW * cgroups + kThreads - 1) / kThreads;
    // The walk's workgroups sit one per CU; when the columns of the batch
    // give fewer workgroups than CUs, each takes fewer lanes (whole pixels,
    // at least three waves' worth) so that every CU holds one (56x56 x 256
    // channels x 32 images: 224 lanes x 256 workgroups instead of 256 x 224,
    // 22.9 -> 22.5 us).  The lane count rides in the high half of col_blocks.
    int lanes = kThreads;
    {
        const int cus = device_cu_count();
        if (stream && static_cast<int64_t>(g.N) * col_blocks < cus && kThreads % cgroups == 0) {
            const int want = std::min((g.OW * cgroups + 63) / 64, std::max(col_blocks, cus / std::max(g.N, 1)));
            const int per = ((g.OW * cgroups + want - 1) / want + cgroups - 1) / cgroups * cgroups;
            if (per >= kThreads * 3 / 4 && per <= kThreads) {
                lanes = per;
                col_blocks = (g.OW * cgroups + lanes - 1) / lanes;
            }
        }
    }
    // Row segments: enough for about kWaveTarget waves in all (every one
    // resident at once), but no shorter than eight rows (each segment
    // re-reads its halo).
    const int64_t waves_per_seg = static_cast<int64_t>(g.N) * col_blocks * (kThreads / 64);
    int segs = static_cast<int>(kWaveTarget / waves_per_seg);
    segs = max(1, min(segs, g.OH / 8));
    const int seg_rows = (g.OH + segs - 1) / segs;
    segs = (g.OH + seg_rows - 1) / seg_rows;
    const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(g.N) * segs * col_blocks + kXcds - 1) / kXcds * kXcds));
    const T* xb = static_cast<const T*>(x);
    const T* wb = static_cast<const T*>(w);
    const T* bb = static_cast<const T*>(bias);
    T* yb = static_cast<T*>(y);
    auto go = [&](auto kernel) {
        return launch(kernel, grid, dim3(kThreads), 0, s, xb, wb, bb, yb, g, cgroups, col_blocks,
                      segs, seg_rows);
    };
    auto go_stream = [&](auto kernel) {
        return launch(kernel, grid, dim3(kThreads), 0, s, xb, wb, bb, yb, g, cgroups, col_blocks | (lanes << 16),
                      segs, seg_rows);
    };
    if (k3d1) return go_stream(depthwise_stream_kernel<T, 3, 3, 1, 1, kRS, CG, MG>);
    if constexpr (CG == 1) {
        if (k3d2) return go_stream(depthwise_stream_kernel<T, 3, 3, 2, 2, kRS, 1, MG>);
        if (k5d1) return go_stream(depthwise_stream_kernel<T, 5, 5, 1, 1, kRS, 1, MG>);
    }
    if constexpr (MG > 1) return launch_mult<T, CG, MG>(x, w, bias, y, g, s);
    return go(depthwise_generic_kernel<T, CG>);
}

template <typename T>
hipError_t launch_cg(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                     hipStream_t s)
{
    switch (g.Cg) {
    case 1: return launch_t<T, 1>(x, w, bias, y, g, s);
    case 2: return launch_t<T, 2>(x, w, bias, y, g, s);
    case 4: return launch_t<T, 4>(x, w, bias, y, g, s);
    default:
        if constexpr (Vec<T>::N == 8) return launch_t<T, 8>(x, w, bias, y, g, s);
        return hipErrorInvalidValue;
    }
}

}  // namespace

bool can_depthwise(const Geom& g, int dtype)
{
    const int vec = dtype == 1 ? 8 : 4;
    const int64_t esz = dtype == 1 ? 2 : 4;
    const int64_t img_bytes = static_cast<int64_t>(std::max(g.H * g.W, g.OH * g.OW)) * g.C * esz;
    const int64_t col_blocks = (static_cast<int64_t>(g.OW) * (g.C / vec) * 2 + kThreads - 1) / kThreads;
    const bool cg_ok = g.Cg == 1 || g.Cg == 2 || g.Cg == 4 || (g.Cg == 8 && vec == 8);
    if (!g.nhwc || !g.aligned16 || !cg_ok || img_bytes >= (int64_t(1) << 31)) return false;
    if (g.Mg == g.Cg) return g.C % vec == 0 && col_blocks * g.N * g.OH < (int64_t(1) << 24);
    // Channel multipliers 2, 4 and 8: whole output vectors, and input
    // windows (of WD channels) that stay aligned within a pixel.
    const int m = g.Mg / g.Cg;
    if (g.Mg % g.Cg != 0 || (m != 2 && m != 4 && m != 8) || g.CO % vec != 0) return false;
    const int wd = (g.Mg <= vec ? vec / g.Mg : 1) * g.Cg;
    const int64_t out_blocks = (static_cast<int64_t>(g.OW) * (g.CO / vec) + kThreads - 1) / kThreads;
    const int64_t out_img = static_cast<int64_t>(g.OH) * g.OW * g.CO * esz;
    return g.C % wd == 0 && out_img < (int64_t(1) << 31) && out_blocks * g.N * g.OH < (int64_t(1) << 24);
}

hipError_t launch_depthwise(const void* x, const void* w, const void* bias, void* y,
                            const Geom& g, int dtype, hipStream_t s)
{
    if (g.Mg != g.Cg)
        return dtype == 1 ? launch_mult_cg<bf16_t>(x, w, bias, y, g, s) : launch_mult_cg<float>(x, w, bias, y, g, s);
    if (can_grouped_mfma(g, dtype)) return launch_grouped_mfma(x, w, bias, y, g, s);
    return dtype == 1 ? launch_cg<bf16_t>(x, w, bias, y, g, s) : launch_cg<float>(x, w, bias, y, g, s);
}

bool can_dx_depthwise(const Geom& g, int dtype)
{
    const int vec = dtype == 1 ? 8 : 4;
    const int64_t esz = dtype == 1 ? 2 : 4;
    const bool cg_ok = g.Cg == 1 || g.Cg == 2 || g.Cg == 4 || (g.Cg == 8 && vec == 8);
    const int64_t img = static_cast<int64_t>(std::max(g.H * g.W, g.OH * g.OW)) * g.C * esz;
    const int64_t col_blocks = (static_cast<int64_t>(g.W) * (g.C / vec) + kThreads - 1) / kThreads;
    return g.nhwc && g.aligned16 && cg_ok && g.Mg == g.Cg && g.C % vec == 0 &&
           img < (int64_t(1) << 31) && col_blocks * g.N * g.H < (int64_t(1) << 24);
}

hipError_t launch_dx_depthwise(const void* dy, const void* w, const void* bias, void* dx, const Geom& g,
                               int dtype, hipStream_t s)
{
    if (dtype == 1) {
        switch (g.Cg) {
        case 1: return launch_dx_small_t<bf16_t, 1>(dy, w, bias, dx, g, s);
        case 2: return launch_dx_small_t<bf16_t, 2>(dy, w, bias, dx, g, s);
        case 4: return launch_dx_small_t<bf16_t, 4>(dy, w, bias, dx, g, s);
        case 8: return launch_dx_small_t<bf16_t, 8>(dy, w, bias, dx, g, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (g.Cg) {
    case 1: return launch_dx_small_t<float, 1>(dy, w, bias, dx, g, s);
    case 2: return launch_dx_small_t<float, 2>(dy, w, bias, dx, g, s);
    case 4: return launch_dx_small_t<float, 4>(dy, w, bias, dx, g, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace convmi
