// Shared device helpers and the launch geometry of the convolution library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

namespace convmi {

// Resolved geometry of one forward convolution (see include/convmi.h for the
// definition).  Extents of one image fit in int32 (checked on the host);
// batch offsets are formed in int64.
struct Geom {
    int N, C, H, W;     // input
    int CO, KH, KW;     // output channels, kernel extent
    int sh, sw, ph, pw, dh, dw;
    int G, Cg, Mg;      // groups, input / output channels per group
    int OH, OW;         // output extent
    int nhwc;           // 1: NHWC / OHWI, 0: NCHW / OIHW
    int aligned16;      // every tensor pointer is 16-byte aligned
};

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float load_f(const float* p) { return *p; }
__device__ __forceinline__ float load_f(const bf16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
__device__ __forceinline__ float bf16_to_f(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even (the conversion of the language type,
// which gfx950 performs in hardware).
__device__ __forceinline__ bf16_t f_to_bf16(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(bf16_t, b);
}

// Raw buffer access.  A buffer resource covers `bytes` bytes from `base`; a
// load at a byte offset at or past `bytes` returns zero without touching
// memory, which supplies zero padding without branches (kOutside is such an
// offset).  The resource lives in scalar registers, so it must be uniform
// across the wavefront.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutside = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(rsrc_t r, uint32_t offset)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0));
}

// Buffer-to-LDS staging with explicit ordering.
typedef uint32_t uint32x4_t __attribute__((ext_vector_type(4)));

// VM <= 63.
template <int VM>
__device__ __forceinline__ void wait_vm()
{
    // s_waitcnt vmcnt(VM), leaving the other counters unconstrained.
    __builtin_amdgcn_s_waitcnt((VM & 15) | (0x7 << 4) | (0xf << 8) | ((VM >> 4) << 14));
}

// 16-byte buffer-to-LDS load: lane i of the wave writes the 16 bytes at
// buffer byte `voffset` (zeros at or past the buffer's end) to LDS address
// lds_base + 16 i.  It is issued as inline assembly so that the compiler does
// not track it: the kernel orders these loads itself (explicit vmcnt waits
// and barriers), which lets reads of one pipeline stage proceed while loads
// into another are in flight.  `lds_base` must be uniform across the wave.
__device__ __forceinline__ void dma16(uint32x4_t rsrc, uint32_t voffset, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "s"(lds_base)
                 : "memory");
}

// 4-byte form of dma16: lane i writes the 4 bytes at `voffset` (zero at or
// past the buffer's end) to LDS address lds_base + 4 i.
__device__ __forceinline__ void dma4(uint32x4_t rsrc, uint32_t voffset, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "s"(lds_base)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// Buffer resource words for dma16: base, no stride, `bytes` records, raw
// (untyped) access.  Base and size must be uniform across the wave; the
// words are read from the first lane so that they live in scalar registers
// even where the compiler cannot prove the uniformity.
__device__ __forceinline__ uint32x4_t dma_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return uint32x4_t{static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a))),
                      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu))),
                      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bytes))), 0x00020000u};
}

// Workgroup barrier without a memory fence.  __syncthreads() would also wait
// for every buffer-to-LDS load still in flight (the fence orders them), which
// would drain the pipeline; here the caller has already waited for the loads
// that must have landed, and every LDS read before the barrier has been
// consumed.  The clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void barrier_no_fence()
{
    asm volatile("s_barrier" ::: "memory");
}

// A store at or past the resource's end is dropped by the hardware.
__device__ __forceinline__ void buffer_store16(rsrc_t r, uint32_t offset, uint4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, offset, 0, 0);
}

// The same store with the non-temporal hint (cache-policy bit nt): for
// outputs that nothing in the kernel reads back, so that streaming them out
// does not displace cached inputs.
__device__ __forceinline__ void buffer_store16_nt(rsrc_t r, uint32_t offset, uint4 v)
{
    constexpr int kNonTemporal = 2;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, offset, 0, kNonTemporal);
}

// 8-byte form: a wave of consecutive lanes still covers whole lines.
__device__ __forceinline__ void buffer_store8_nt(rsrc_t r, uint32_t offset, uint2 v)
{
    constexpr int kNonTemporal = 2;
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)), v), r, offset, 0, kNonTemporal);
}

__device__ __forceinline__ void store_f(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_f(bf16_t* p, float v) { *p = f_to_bf16(v); }

// Packs two fp32 values into one dword of two bf16 (lo in bits 0..15),
// rounding to nearest even: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t{lo, hi}), bf16x2_t));
}

// Division by a runtime constant d >= 1 for dividends below 2^31, as a
// multiply-high, an add and a shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994: with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l).  The
// host fills it; kernels use it instead of the much longer software divide.
struct FastDiv {
    uint32_t d, m, l;
};
inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{d, static_cast<uint32_t>(m), l};
}
__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f)
{
#ifdef __HIP_DEVICE_COMPILE__
    const uint32_t hi = __umulhi(n, f.m);
#else
    const uint32_t hi = static_cast<uint32_t>((uint64_t(n) * f.m) >> 32);
#endif
    return (hi + n) >> f.l;
}

// Host: drops a stale error left by an earlier runtime call, so that the
// status read right after a launch belongs to that launch.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Events armed by conv_arm_launch_events for the next launch on this thread.
struct ArmedEvents {
    hipEvent_t start;
    hipEvent_t stop;
};
ArmedEvents& armed_events();

// Host: launches `kernel` on stream `s`.  If events are armed, the launch goes
// through hipExtLaunchKernel so that the runtime stamps the kernel's own start
// and end into them (no extra packets on the stream), and the events are
// disarmed.  Returns the launch status.
template <typename... Params, typename... Args>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                  Args... args)
{
    clear_stale_error();
    ArmedEvents& ev = armed_events();
    if (ev.start || ev.stop) {
        const hipEvent_t a = ev.start, b = ev.stop;
        ev = ArmedEvents{nullptr, nullptr};
        std::tuple<Params...> vals{static_cast<Params>(args)...};
        return std::apply(
            [&](auto&... v) {
                void* ptrs[] = {static_cast<void*>(&v)...};
                return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs,
                                          lds, s, a, b, 0);
            },
            vals);
    }
    hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<Params>(args)...);
    return hipGetLastError();
}

}  // namespace convmi
