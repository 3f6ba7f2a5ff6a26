// C ABI of the convolution library: argument validation, geometry, static
// path selection and launch on the caller's stream.  See include/convmi.h.
//
// Validation follows the checks of oarust 0.8.6 src/rs/ml/matrix/conv.rs,
// `Conv2dGeometry::resolve` and `Conv1dGeometry::resolve`: nonzero extents,
// stride, dilation and groups; channels divisible by groups; the dilated
// kernel must fit the padded input; coordinates must fit a signed 32-bit
// index.  Every check runs on the host before anything is launched, so a
// rejected call writes nothing.
#include "convmi.h"
#include "kernels.hpp"

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

using convmi::Geom;

namespace convmi {
ArmedEvents& armed_events()
{
    static thread_local ArmedEvents ev{nullptr, nullptr};
    return ev;
}

int device_cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
}  // namespace convmi

namespace {

thread_local std::string t_last_error;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_last_error = buf;
    return code;
}

int64_t extent(int64_t in, int64_t k, int64_t stride, int64_t pad, int64_t dil)
{
    const int64_t effective = (k - 1) * dil + 1;
    const int64_t padded = in + 2 * pad;
    if (padded < effective) return -1;
    return (padded - effective) / stride + 1;
}

// Validates the forward geometry and fills `g`.  `op` names the entry point
// in messages.
int resolve(Geom& g, const char* op, int N, int C, int H, int W, int CO, int KH, int KW,
            int sh, int sw, int ph, int pw, int dh, int dw, int G, int layout, int dtype)
{
    if (layout != CONV_NCHW && layout != CONV_NHWC)
        return fail(CONV_ERR_INVALID_ARG, "%s: layout must be CONV_NCHW or CONV_NHWC, got %d", op, layout);
    if (dtype != CONV_F32 && dtype != CONV_BF16)
        return fail(CONV_ERR_INVALID_ARG, "%s: dtype must be CONV_F32 or CONV_BF16, got %d", op, dtype);
    if (N < 1 || C < 1 || H < 1 || W < 1 || CO < 1 || KH < 1 || KW < 1)
        return fail(CONV_ERR_INVALID_ARG,
                    "%s: N, C, H, W, C_out, KH and KW must be >= 1 (got %d %d %d %d %d %d %d)", op,
                    N, C, H, W, CO, KH, KW);
    if (sh < 1 || sw < 1 || dh < 1 || dw < 1 || G < 1)
        return fail(CONV_ERR_INVALID_ARG, "%s: stride, dilation and groups must be >= 1", op);
    if (ph < 0 || pw < 0)
        return fail(CONV_ERR_INVALID_ARG, "%s: padding must be >= 0", op);
    if (C % G != 0 || CO % G != 0)
        return fail(CONV_ERR_INVALID_ARG,
                    "%s: channels must be divisible by groups (C=%d, C_out=%d, groups=%d)", op, C,
                    CO, G);
    const int64_t OH = extent(H, KH, sh, ph, dh);
    const int64_t OW = extent(W, KW, sw, pw, dw);
    if (OH < 1 || OW < 1)
        return fail(CONV_ERR_INVALID_ARG, "%s: dilated kernel does not fit the padded input", op);
    const int64_t lim = INT32_MAX;
    const int64_t in_img = static_cast<int64_t>(H) * W * C;
    const int64_t out_img = OH * OW * CO;
    const int64_t w_count = static_cast<int64_t>(CO) * (C / G) * KH * KW;
    if (in_img > lim || out_img > lim || w_count > lim)
        return fail(CONV_ERR_OVERFLOW,
                    "%s: one image of x or y, or the weight, exceeds INT32_MAX elements", op);
    const int64_t last_h = (OH - 1) * sh + static_cast<int64_t>(KH - 1) * dh;
    const int64_t last_w = (OW - 1) * sw + static_cast<int64_t>(KW - 1) * dw;
    if (last_h > lim || last_w > lim || static_cast<int64_t>(H) + 2 * ph > lim ||
        static_cast<int64_t>(W) + 2 * pw > lim)
        return fail(CONV_ERR_OVERFLOW, "%s: a padded coordinate exceeds INT32_MAX", op);
    g.N = N; g.C = C; g.H = H; g.W = W; g.CO = CO; g.KH = KH; g.KW = KW;
    g.sh = sh; g.sw = sw; g.ph = ph; g.pw = pw; g.dh = dh; g.dw = dw;
    g.G = G; g.Cg = C / G; g.Mg = CO / G;
    g.OH = static_cast<int>(OH); g.OW = static_cast<int>(OW);
    g.nhwc = layout == CONV_NHWC;
    g.aligned16 = 1;
    return CONV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int select_fwd(const Geom& g, int dtype)
{
    if (convmi::can_pointwise(g, dtype)) return CONV_PATH_POINTWISE;
    if (convmi::can_depthwise(g, dtype)) return CONV_PATH_DEPTHWISE;
    if (convmi::can_igemm_band(g, dtype) && convmi::igemm_band_preferred(g)) return CONV_PATH_IGEMM_BAND;
    if (convmi::can_igemm(g, dtype)) return CONV_PATH_IGEMM;
    return CONV_PATH_DIRECT;
}

int select_dx(const Geom& g, int dtype)
{
    if (convmi::can_dx_igemm(g, dtype)) return CONV_PATH_DX_IGEMM;
    if (convmi::can_dx_depthwise(g, dtype)) return CONV_PATH_DX_DEPTHWISE;
    return CONV_PATH_DX_GATHER;
}

int select_dw(const Geom& g, int dtype)
{
    if (convmi::can_dw_igemm(g, dtype)) return CONV_PATH_DW_IGEMM;
    return CONV_PATH_DW_DIRECT;
}

// Workspace bytes of a weight-gradient path for a geometry (0 if the path
// does not serve it or is not a weight-gradient path).
size_t dw_workspace(const Geom& g, int dtype, int path)
{
    switch (path) {
    case CONV_PATH_DW_DIRECT: return convmi::plan_dw_direct(g).workspace;
    case CONV_PATH_DW_IGEMM:
        return convmi::can_dw_igemm(g, dtype) ? convmi::plan_dw_igemm(g, convmi::device_cu_count()).workspace : 0;
    default: return 0;
    }
}

int launched(hipError_t e, const char* op, int path)
{
    if (e != hipSuccess)
        return fail(CONV_ERR_HIP, "%s: launch of path '%s' failed: %s", op, conv_path_name(path),
                    hipGetErrorString(e));
    return CONV_OK;
}

// Launches a forward path on a validated geometry (conv_fwd, conv1d_fwd).
int run_fwd(const char* op, const void* x, const void* w, const void* bias, void* y, Geom g,
            int dtype, int path, void* stream)
{
    g.aligned16 = aligned16(x) && aligned16(w) && aligned16(bias) && aligned16(y);
    if (path == CONV_PATH_AUTO) path = select_fwd(g, dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (path) {
    case CONV_PATH_DIRECT:
        return launched(convmi::launch_fwd_direct(x, w, bias, y, g, dtype, s), op, path);
    case CONV_PATH_POINTWISE:
        if (!convmi::can_pointwise(g, dtype)) break;
        return launched(convmi::launch_pointwise(x, w, bias, y, g, s), op, path);
    case CONV_PATH_DEPTHWISE:
        if (!convmi::can_depthwise(g, dtype)) break;
        return launched(convmi::launch_depthwise(x, w, bias, y, g, dtype, s), op, path);
    case CONV_PATH_IGEMM:
        if (!convmi::can_igemm(g, dtype)) break;
        return launched(convmi::launch_igemm(x, w, bias, y, g, s), op, path);
    case CONV_PATH_IGEMM_BAND:
        if (!convmi::can_igemm_band(g, dtype)) break;
        return launched(convmi::launch_igemm_band(x, w, bias, y, g, s), op, path);
    default:
        return fail(CONV_ERR_INVALID_ARG, "%s: %d is not a forward path", op, path);
    }
    return fail(CONV_ERR_UNSUPPORTED, "%s: path '%s' does not support this geometry/layout/dtype",
                op, conv_path_name(path));
}

// Launches an input-gradient path on a validated forward geometry, adding a
// per-channel bias of dx when one is given (conv_bwd_dx: none;
// conv_transpose2d: its bias).
int run_dx(const char* op, const void* dy, const void* w, const void* bias, void* dx, Geom g,
           int dtype, int path, void* stream)
{
    g.aligned16 = aligned16(dy) && aligned16(w) && aligned16(bias) && aligned16(dx);
    if (path == CONV_PATH_AUTO) path = select_dx(g, dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (path) {
    case CONV_PATH_DX_GATHER:
        return launched(convmi::launch_dx_gather(dy, w, bias, dx, g, dtype, s), op, path);
    case CONV_PATH_DX_IGEMM:
        if (!convmi::can_dx_igemm(g, dtype)) break;
        return launched(convmi::launch_dx_igemm(dy, w, bias, dx, g, s), op, path);
    case CONV_PATH_DX_DEPTHWISE:
        if (!convmi::can_dx_depthwise(g, dtype)) break;
        return launched(convmi::launch_dx_depthwise(dy, w, bias, dx, g, dtype, s), op, path);
    case CONV_PATH_DX_BAND:
        if (!convmi::can_dx_band(g, dtype)) break;
        return launched(convmi::launch_dx_band(dy, w, bias, dx, g, s), op, path);
    default:
        return fail(CONV_ERR_INVALID_ARG, "%s: %d is not an input-gradient path", op, path);
    }
    return fail(CONV_ERR_UNSUPPORTED, "%s: path '%s' does not support this geometry/layout/dtype",
                op, conv_path_name(path));
}

// Launches a weight-gradient path on a validated forward geometry with the
// given fp32 workspace.
int run_dw(const char* op, const void* x, const void* dy, void* dw, void* workspace,
           size_t workspace_bytes, Geom g, int dtype, int path, void* stream)
{
    g.aligned16 = aligned16(x) && aligned16(dy) && aligned16(dw);
    if (path == CONV_PATH_AUTO) path = select_dw(g, dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (path) {
    case CONV_PATH_DW_DIRECT: {
        const size_t need = dw_workspace(g, dtype, path);
        if (workspace_bytes < need || (need > 0 && (!workspace || !aligned16(workspace))))
            return fail(CONV_ERR_INVALID_ARG,
                        "%s: path '%s' needs a 16-byte aligned workspace of %zu bytes (got %zu)",
                        op, conv_path_name(path), need, workspace_bytes);
        return launched(convmi::launch_dw_direct(x, dy, dw, workspace, g, dtype, s), op, path);
    }
    case CONV_PATH_DW_IGEMM: {
        if (!convmi::can_dw_igemm(g, dtype)) break;
        const size_t need = dw_workspace(g, dtype, path);
        if (workspace_bytes < need || !workspace || !aligned16(workspace))
            return fail(CONV_ERR_INVALID_ARG,
                        "%s: path '%s' needs a 16-byte aligned workspace of %zu bytes (got %zu)",
                        op, conv_path_name(path), need, workspace_bytes);
        return launched(convmi::launch_dw_igemm(x, dy, dw, workspace, g, convmi::device_cu_count(), s),
                        op, path);
    }
    default:
        return fail(CONV_ERR_INVALID_ARG, "%s: %d is not a weight-gradient path", op, path);
    }
    return fail(CONV_ERR_UNSUPPORTED, "%s: path '%s' does not support this geometry/layout/dtype",
                op, conv_path_name(path));
}

// Output extent of a transposed convolution along one axis,
// (in - 1)*stride - 2*pad + dil*(k - 1) + 1 + out_pad, or -1 when an argument
// is out of its domain or the padding leaves nothing.
int64_t transpose_extent(int64_t in, int64_t k, int64_t stride, int64_t pad, int64_t dil,
                         int64_t out_pad)
{
    if (in < 1 || k < 1 || stride < 1 || dil < 1 || pad < 0 || out_pad < 0 || out_pad >= stride)
        return -1;
    const int64_t e = (in - 1) * stride - 2 * pad + dil * (k - 1) + 1 + out_pad;
    return e >= 1 ? e : -1;
}

}  // namespace

extern "C" {

const char* conv_path_name(int path)
{
    switch (path) {
    case CONV_PATH_AUTO: return "auto";
    case CONV_PATH_DIRECT: return "direct";
    case CONV_PATH_IGEMM: return "igemm";
    case CONV_PATH_POINTWISE: return "pointwise";
    case CONV_PATH_DEPTHWISE: return "depthwise";
    case CONV_PATH_DX_GATHER: return "dx_gather";
    case CONV_PATH_DX_IGEMM: return "dx_igemm";
    case CONV_PATH_IGEMM_BAND: return "igemm_band";
    case CONV_PATH_DW_DIRECT: return "dw_direct";
    case CONV_PATH_DW_IGEMM: return "dw_igemm";
    case CONV_PATH_DX_DEPTHWISE: return "dx_depthwise";
    case CONV_PATH_DX_BAND: return "dx_band";
    default: return "unknown";
    }
}

const char* conv_last_error(void) { return t_last_error.c_str(); }

int conv_arm_launch_events(void* start, void* stop)
{
    convmi::armed_events() = convmi::ArmedEvents{static_cast<hipEvent_t>(start),
                                                  static_cast<hipEvent_t>(stop)};
    return CONV_OK;
}

int conv_out_size(int in, int k, int stride, int pad, int dil, int* out)
{
    if (!out) return fail(CONV_ERR_INVALID_ARG, "conv_out_size: out is NULL");
    if (in < 1 || k < 1 || stride < 1 || dil < 1 || pad < 0)
        return fail(CONV_ERR_INVALID_ARG,
                    "conv_out_size: in, k, stride and dil must be >= 1 and pad >= 0");
    const int64_t e = extent(in, k, stride, pad, dil);
    if (e < 1)
        return fail(CONV_ERR_INVALID_ARG, "conv_out_size: dilated kernel does not fit the padded input");
    if (e > INT32_MAX) return fail(CONV_ERR_OVERFLOW, "conv_out_size: extent exceeds INT32_MAX");
    *out = static_cast<int>(e);
    return CONV_OK;
}

int conv_select_path(int backward, int N, int C, int H, int W, int C_out, int KH, int KW,
                     int stride_h, int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                     int groups, int layout, int dtype, int* path_out)
{
    if (!path_out) return fail(CONV_ERR_INVALID_ARG, "conv_select_path: path_out is NULL");
    Geom g;
    int rc = resolve(g, "conv_select_path", N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h,
                     pad_w, dil_h, dil_w, groups, layout, dtype);
    if (rc) return rc;
    *path_out = backward == 2 ? select_dw(g, dtype) : backward ? select_dx(g, dtype) : select_fwd(g, dtype);
    return CONV_OK;
}

int conv_fwd_ex(const void* x, const void* w, const void* bias, void* y, int N, int C, int H,
                int W, int C_out, int KH, int KW, int stride_h, int stride_w, int pad_h,
                int pad_w, int dil_h, int dil_w, int groups, int layout, int dtype, int path,
                void* stream)
{
    static const char* op = "conv_fwd";
    if (!x || !w || !y) return fail(CONV_ERR_INVALID_ARG, "%s: x, w and y must not be NULL", op);
    Geom g;
    int rc = resolve(g, op, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w, dil_h,
                     dil_w, groups, layout, dtype);
    if (rc) return rc;
    return run_fwd(op, x, w, bias, y, g, dtype, path, stream);
}

int conv_fwd(const void* x, const void* w, const void* bias, void* y, int N, int C, int H, int W,
             int C_out, int KH, int KW, int stride_h, int stride_w, int pad_h, int pad_w,
             int dil_h, int dil_w, int groups, int layout, int dtype, void* stream)
{
    return conv_fwd_ex(x, w, bias, y, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
                       dil_h, dil_w, groups, layout, dtype, CONV_PATH_AUTO, stream);
}

int conv_bwd_dx_ex(const void* dy, const void* w, void* dx, int N, int C, int H, int W, int C_out,
                   int KH, int KW, int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                   int dil_w, int groups, int layout, int dtype, int path, void* stream)
{
    static const char* op = "conv_bwd_dx";
    if (!dy || !w || !dx) return fail(CONV_ERR_INVALID_ARG, "%s: dy, w and dx must not be NULL", op);
    Geom g;
    int rc = resolve(g, op, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w, dil_h,
                     dil_w, groups, layout, dtype);
    if (rc) return rc;
    return run_dx(op, dy, w, nullptr, dx, g, dtype, path, stream);
}

int conv_bwd_dx(const void* dy, const void* w, void* dx, int N, int C, int H, int W, int C_out,
                int KH, int KW, int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                int dil_w, int groups, int layout, int dtype, void* stream)
{
    return conv_bwd_dx_ex(dy, w, dx, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
                          dil_h, dil_w, groups, layout, dtype, CONV_PATH_AUTO, stream);
}

int conv1d_fwd_ex(const void* x, const void* w, const void* bias, void* y, int N, int C, int L,
                  int C_out, int K, int stride, int pad, int dil, int groups, int layout,
                  int dtype, int path, void* stream)
{
    static const char* op = "conv1d_fwd";
    if (!x || !w || !y) return fail(CONV_ERR_INVALID_ARG, "%s: x, w and y must not be NULL", op);
    // A sequence is an image of one row: H = 1, KH = 1, no vertical stride,
    // padding or dilation; NCL / NLC are NCHW / NHWC with that row.
    Geom g;
    int rc = resolve(g, op, N, C, 1, L, C_out, 1, K, 1, stride, 0, pad, 1, dil, groups, layout,
                     dtype);
    if (rc) return rc;
    return run_fwd(op, x, w, bias, y, g, dtype, path, stream);
}

int conv1d_fwd(const void* x, const void* w, const void* bias, void* y, int N, int C, int L,
               int C_out, int K, int stride, int pad, int dil, int groups, int layout, int dtype,
               void* stream)
{
    return conv1d_fwd_ex(x, w, bias, y, N, C, L, C_out, K, stride, pad, dil, groups, layout, dtype,
                         CONV_PATH_AUTO, stream);
}

int conv_transpose_out_size(int in, int k, int stride, int pad, int dil, int out_pad, int* out)
{
    if (!out) return fail(CONV_ERR_INVALID_ARG, "conv_transpose_out_size: out is NULL");
    const int64_t e = transpose_extent(in, k, stride, pad, dil, out_pad);
    if (e == -1)
        return fail(CONV_ERR_INVALID_ARG,
                    "conv_transpose_out_size: in, k, stride and dil must be >= 1, pad >= 0 and "
                    "0 <= out_pad < stride, and the padding must leave a nonempty output");
    if (e > INT32_MAX) return fail(CONV_ERR_OVERFLOW, "conv_transpose_out_size: extent exceeds INT32_MAX");
    *out = static_cast<int>(e);
    return CONV_OK;
}

int conv_transpose2d_ex(const void* x, const void* w, const void* bias, void* y, int N, int C_in,
                        int H, int W, int C_out, int KH, int KW, int stride_h, int stride_w,
                        int pad_h, int pad_w, int out_pad_h, int out_pad_w, int dil_h, int dil_w,
                        int groups, int layout, int dtype, int path, void* stream)
{
    static const char* op = "conv_transpose2d";
    if (!x || !w || !y) return fail(CONV_ERR_INVALID_ARG, "%s: x, w and y must not be NULL", op);
    if (N < 1 || C_in < 1 || H < 1 || W < 1 || C_out < 1 || KH < 1 || KW < 1)
        return fail(CONV_ERR_INVALID_ARG,
                    "%s: N, C_in, H, W, C_out, KH and KW must be >= 1 (got %d %d %d %d %d %d %d)",
                    op, N, C_in, H, W, C_out, KH, KW);
    const int64_t OH = transpose_extent(H, KH, stride_h, pad_h, dil_h, out_pad_h);
    const int64_t OW = transpose_extent(W, KW, stride_w, pad_w, dil_w, out_pad_w);
    if (OH == -1 || OW == -1)
        return fail(CONV_ERR_INVALID_ARG,
                    "%s: stride and dilation must be >= 1, padding >= 0, 0 <= output padding < "
                    "stride, and the padding must leave a nonempty output", op);
    if (OH > INT32_MAX || OW > INT32_MAX)
        return fail(CONV_ERR_OVERFLOW, "%s: an output extent exceeds INT32_MAX", op);
    // The forward convolution whose input gradient this is: input y
    // [N, C_out, OH, OW], output x [N, C_in, H, W], weight w read as that
    // forward's weight (C_out of the forward = C_in here).  With
    // 0 <= output padding < stride the forward's output extent is exactly
    // H x W.
    Geom g;
    int rc = resolve(g, op, N, C_out, static_cast<int>(OH), static_cast<int>(OW), C_in, KH, KW,
                     stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups, layout, dtype);
    if (rc) return rc;
    if (g.OH != H || g.OW != W)
        return fail(CONV_ERR_INVALID_ARG, "%s: inconsistent geometry", op);
    return run_dx(op, x, w, bias, y, g, dtype, path, stream);
}

int conv_transpose2d(const void* x, const void* w, const void* bias, void* y, int N, int C_in,
                     int H, int W, int C_out, int KH, int KW, int stride_h, int stride_w,
                     int pad_h, int pad_w, int out_pad_h, int out_pad_w, int dil_h, int dil_w,
                     int groups, int layout, int dtype, void* stream)
{
    return conv_transpose2d_ex(x, w, bias, y, N, C_in, H, W, C_out, KH, KW, stride_h, stride_w,
                               pad_h, pad_w, out_pad_h, out_pad_w, dil_h, dil_w, groups, layout,
                               dtype, CONV_PATH_AUTO, stream);
}

int conv_bwd_dw_workspace_size(int N, int C, int H, int W, int C_out, int KH, int KW, int stride_h,
                               int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                               int groups, int layout, int dtype, int path, size_t* bytes)
{
    static const char* op = "conv_bwd_dw_workspace_size";
    if (!bytes) return fail(CONV_ERR_INVALID_ARG, "%s: bytes is NULL", op);
    Geom g;
    int rc = resolve(g, op, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w, dil_h,
                     dil_w, groups, layout, dtype);
    if (rc) return rc;
    if (path == CONV_PATH_AUTO) path = select_dw(g, dtype);
    if (path != CONV_PATH_DW_DIRECT && path != CONV_PATH_DW_IGEMM)
        return fail(CONV_ERR_INVALID_ARG, "%s: %d is not a weight-gradient path", op, path);
    *bytes = dw_workspace(g, dtype, path);
    return CONV_OK;
}

int conv_bwd_dw_ex(const void* x, const void* dy, void* dw, void* workspace,
                   size_t workspace_bytes, int N, int C, int H, int W, int C_out, int KH, int KW,
                   int stride_h, int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                   int groups, int layout, int dtype, int path, void* stream)
{
    static const char* op = "conv_bwd_dw";
    if (!x || !dy || !dw) return fail(CONV_ERR_INVALID_ARG, "%s: x, dy and dw must not be NULL", op);
    Geom g;
    int rc = resolve(g, op, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w, dil_h,
                     dil_w, groups, layout, dtype);
    if (rc) return rc;
    return run_dw(op, x, dy, dw, workspace, workspace_bytes, g, dtype, path, stream);
}
int conv_bwd_dw_noalloc(const void* x, const void* dy, void* dw, int N, int C, int H, int W,
                        int C_out, int KH, int KW, int stride_h, int stride_w, int pad_h,
                        int pad_w, int dil_h, int dil_w, int groups, int layout, int dtype,
                        void* stream)
{
    static const char* op = "conv_bwd_dw_noalloc";
    if (!x || !dy || !dw) return fail(CONV_ERR_INVALID_ARG, "%s: x, dy and dw must not be NULL", op);
    Geom g;
    int rc = resolve(g, op, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w, dil_h,
                     dil_w, groups, layout, dtype);
    if (rc) return rc;
    g.aligned16 = aligned16(x) && aligned16(dy) && aligned16(dw);
    const int path = select_dw(g, dtype);
    const size_t need = dw_workspace(g, dtype, path);
    if (need > convmi::kScratchBytes)
        return fail(CONV_ERR_UNSUPPORTED,
                    "%s: this weight gradient needs %zu bytes of scratch, more than the %zu this "
                    "entry point holds; call conv_bwd_dw with a workspace instead",
                    op, need, convmi::kScratchBytes);
    void* scratch = nullptr;
    const hipError_t e = convmi::scratch_buffer(&scratch);
    if (e != hipSuccess)
        return fail(CONV_ERR_HIP, "%s: device scratch lookup failed: %s", op, hipGetErrorString(e));
    return run_dw(op, x, dy, dw, scratch, convmi::kScratchBytes, g, dtype, path, stream);
}
int conv_bwd_dw(const void* x, const void* dy, void* dw, void* workspace, size_t workspace_bytes,
                int N, int C, int H, int W, int C_out, int KH, int KW, int stride_h, int stride_w,
                int pad_h, int pad_w, int dil_h, int dil_w, int groups, int layout, int dtype,
                void* stream)
{
    return conv_bwd_dw_ex(x, dy, dw, workspace, workspace_bytes, N, C, H, W, C_out, KH, KW,
                          stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups, layout, dtype,
                          CONV_PATH_AUTO, stream);
}

}  // extern "C"
