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

__device__ __forceinline__ void store_f(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_f(bf16_t* p, float v) { *p = f_to_bf16(v); }

// Packs two fp32 values into one dword of two bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f_to_bf16(lo)) | (static_cast<uint32_t>(f_to_bf16(hi)) << 16);
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
