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

// A store at or past the resource's end is dropped by the hardware.
__device__ __forceinline__ void buffer_store16(rsrc_t r, uint32_t offset, uint4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, offset, 0, 0);
}

__device__ __forceinline__ void store_f(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_f(bf16_t* p, float v) { *p = f_to_bf16(v); }

// Packs two fp32 values into one dword of two bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f_to_bf16(lo)) | (static_cast<uint32_t>(f_to_bf16(hi)) << 16);
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
