// Launchers of the HIP kernels (host side).  Each returns hipSuccess or the
// launch error; arguments were validated by the caller.
#pragma once

#include "common.hpp"

namespace convmi {

// Compute units of the current device (queried once per device).
int device_cu_count();

// Generic direct forward, any geometry, layout and dtype (dtype 0 fp32, 1 bf16).
hipError_t launch_fwd_direct(const void* x, const void* w, const void* bias, void* y,
                             const Geom& g, int dtype, hipStream_t s);
// Generic input gradient as a per-element gather, plus a per-channel bias
// (NULL for none; the transposed convolution has one).
hipError_t launch_dx_gather(const void* dy, const void* w, const void* bias, void* dx,
                            const Geom& g, int dtype, hipStream_t s);

// Fast paths.  Each has a predicate (can_*) that the dispatcher checks first.
bool can_pointwise(const Geom& g, int dtype);
hipError_t launch_pointwise(const void* x, const void* w, const void* bias, void* y,
                            const Geom& g, hipStream_t s);

bool can_igemm(const Geom& g, int dtype);
hipError_t launch_igemm(const void* x, const void* w, const void* bias, void* y,
                        const Geom& g, hipStream_t s);

bool can_igemm_band(const Geom& g, int dtype);
// Output rows per band (0 when the band kernel declines); automatic
// selection prefers the band kernel from 5 rows on.
bool igemm_band_preferred(const Geom& g);
hipError_t launch_igemm_band(const void* x, const void* w, const void* bias, void* y,
                             const Geom& g, hipStream_t s);

bool can_depthwise(const Geom& g, int dtype);
// Small groups (C/G = C_out/G = 4 or 8, 3x3, bf16, C a multiple of 64) on the
// 4x4x4 matrix instruction; the depthwise path takes it where it applies.
bool can_grouped_mfma(const Geom& g, int dtype);
hipError_t launch_grouped_mfma(const void* x, const void* w, const void* bias, void* y, const Geom& g,
                               hipStream_t s);
hipError_t launch_depthwise(const void* x, const void* w, const void* bias, void* y,
                            const Geom& g, int dtype, hipStream_t s);

// Weight gradient, split over the pixels of the batch into `pieces` pieces of
// `per` pixels whose fp32 partials (pieces x weight elements) go to a
// workspace of `workspace` bytes, then reduced in piece order.
struct DwPlan {
    int64_t per;
    int pieces;
    size_t workspace;
};
DwPlan plan_dw_direct(const Geom& g);
bool can_dw_igemm(const Geom& g, int dtype);
DwPlan plan_dw_igemm(const Geom& g, int cus);
hipError_t launch_dw_igemm(const void* x, const void* dy, void* dw, void* workspace, const Geom& g,
                           int cus, hipStream_t s);
hipError_t launch_dw_direct(const void* x, const void* dy, void* dw, void* workspace,
                            const Geom& g, int dtype, hipStream_t s);
hipError_t launch_dw_reduce(const float* part, void* dw, int64_t wn, int pieces, int dtype,
                            hipStream_t s);

// The fixed device scratch of conv_bwd_dw_noalloc: kScratchBytes bytes,
// 256-byte aligned, one array per device; *out receives this device's
// address (looked up once per device).
constexpr size_t kScratchBytes = size_t(16) << 20;
hipError_t scratch_buffer(void** out);

bool can_dx_igemm(const Geom& g, int dtype);
// Input gradient of small groups (C/G = C_out/G = 1, 2, 4, or 8 in bf16),
// NHWC: per-channel gather on the vector units, per-channel bias.
bool can_dx_depthwise(const Geom& g, int dtype);
hipError_t launch_dx_depthwise(const void* dy, const void* w, const void* bias, void* dx, const Geom& g,
                               int dtype, hipStream_t s);
hipError_t launch_dx_igemm(const void* dy, const void* w, const void* bias, void* dx,
                           const Geom& g, hipStream_t s);
// Input gradient of stride-2, dilation-1 3x3 and 4x4 kernels: all four
// stride phases of a band of rows per workgroup.
bool can_dx_band(const Geom& g, int dtype);
hipError_t launch_dx_band(const void* dy, const void* w, const void* bias, void* dx,
                          const Geom& g, hipStream_t s);

}  // namespace convmi
