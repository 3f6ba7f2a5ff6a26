/*
 * convmi -- 2-D convolution forward and input gradient on AMD Instinct
 * MI355X (gfx950), hand-written HIP kernels behind a plain C ABI.
 *
 * The operation is the cross-correlation used by deep-learning frameworks:
 *
 *   y[n, co, oh, ow] = bias[co] + sum_{c < C/G} sum_{kh < KH} sum_{kw < KW}
 *        x[n, g*C/G + c, oh*sh - ph + kh*dh, ow*sw - pw + kw*dw]
 *        * w[co, c, kh, kw],                         g = co / (C_out/G),
 *
 * with x read as zero outside [0,H) x [0,W).  Sources: teeny-kernels 0.2.0,
 * src/nn/conv/conv2d.rs, the `conv2d_forward` doc comment and body (tap
 * indexing oh*stride + kh - pad, grouping, zero padding through the load
 * mask) and `conv2d_bias_forward` (fused per-channel bias); burn-cubecl
 * 0.22.0-pre.4, src/kernel/conv/im2col.rs, `im2col` (dilation enters as
 * k*dilation); oarust 0.8.6, src/rs/ml/matrix/conv.rs,
 * `Conv1dGeometry::resolve` (extent with dilation) and
 * `Conv2dGeometry::resolve` (argument checks).
 *
 * Layouts (one flag governs every tensor of a call):
 *   CONV_NCHW: x [N, C, H, W], w [C_out, C/G, KH, KW], y [N, C_out, OH, OW]
 *   CONV_NHWC: x [N, H, W, C], w [C_out, KH, KW, C/G], y [N, OH, OW, C_out]
 *   bias: [C_out].  All tensors dense (no strides), same dtype.
 *
 * Arithmetic: products are formed from the stored values and accumulated in
 * fp32; the bias is added in fp32; the result is rounded once to the stored
 * dtype (round to nearest even for bf16).
 *
 * Ownership: every pointer is a device pointer owned by the caller, who
 * allocates every output.  The library keeps no reference past the call and
 * allocates no device memory.  Outputs are fully overwritten; they need no
 * zeroing beforehand.
 *
 * Execution: every call validates all arguments on the host first; on error
 * nothing is launched and nothing is written.  Work is then enqueued on
 * `stream` (a hipStream_t; NULL = the null stream of the current device) and
 * the call returns without waiting.  Launch failures are reported as
 * CONV_ERR_HIP.  The message for the last failure on the calling thread is
 * available from conv_last_error().  Results are deterministic: no kernel
 * uses atomics, each output element is written by exactly one lane.
 */
#ifndef CONVMI_H
#define CONVMI_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum conv_status {
    CONV_OK = 0,
    CONV_ERR_INVALID_ARG = 1, /* a shape, pointer or enum is invalid       */
    CONV_ERR_UNSUPPORTED = 2, /* a forced path declines this geometry      */
    CONV_ERR_OVERFLOW = 3,    /* a per-image extent exceeds INT32_MAX      */
    CONV_ERR_HIP = 4          /* the HIP runtime reported an error         */
} conv_status_t;

typedef enum conv_layout {
    CONV_NCHW = 0,
    CONV_NHWC = 1,
    CONV_NCL = 0, /* conv1d: channels before length (the NCHW of one row) */
    CONV_NLC = 1  /* conv1d: channels innermost (the NHWC of one row)    */
} conv_layout_t;

typedef enum conv_dtype { CONV_F32 = 0, CONV_BF16 = 1 } conv_dtype_t;

/* Kernel paths.  CONV_PATH_AUTO picks the fastest path whose preconditions
 * hold; any other value forces that path and fails with
 * CONV_ERR_UNSUPPORTED when its preconditions do not hold. */
typedef enum conv_path {
    CONV_PATH_AUTO = 0,
    CONV_PATH_DIRECT = 1,    /* forward, any geometry/layout/dtype          */
    CONV_PATH_IGEMM = 2,     /* forward, NHWC bf16, C/G a multiple of 8:
                                implicit GEMM on MFMA                      */
    CONV_PATH_POINTWISE = 3, /* forward, NHWC bf16 1x1 (any stride and
                                padding), one GEMM                         */
    CONV_PATH_DEPTHWISE = 4, /* forward, NHWC, groups of 1, 2, 4 (or 8 in
                                bf16) channels with C_out/G = C/G, or
                                C_out/G = 2, 4 or 8 times C/G (channel
                                multipliers); bf16 3x3 groups of 4 or 8
                                over a multiple of 64 channels use the
                                4x4x4 matrix instruction                   */
    CONV_PATH_DX_GATHER = 5, /* input grad, any geometry/layout/dtype       */
    CONV_PATH_DX_IGEMM = 6,  /* input grad, NHWC bf16, per-phase MFMA GEMM  */
    CONV_PATH_IGEMM_BAND = 7, /* forward, NHWC bf16 3x3 with Cg in {16, 32,
                                 64}: implicit GEMM streamed over row bands */
    CONV_PATH_DW_DIRECT = 8,  /* weight grad, any geometry/layout/dtype     */
    CONV_PATH_DW_IGEMM = 9,   /* weight grad, NHWC bf16: implicit GEMM on
                                 MFMA per piece of pixels                  */
    CONV_PATH_DX_DEPTHWISE = 10, /* input grad, NHWC, groups with C/G = C_out/G
                                   of 1, 2, 4 (or 8 in bf16): per-channel
                                   gather on the vector units             */
    CONV_PATH_DX_BAND = 11 /* input grad, NHWC bf16, stride 2, dilation 1,
                              3x3 or 4x4 with equal pad parities, C/G a
                              multiple of 64, C_out/G of 16: all four
                              stride phases of a band of rows per
                              workgroup on MFMA                          */
} conv_path_t;

/*
 * Output extent along one spatial axis:
 *   out = floor((in + 2*pad - dil*(k-1) - 1) / stride) + 1.
 * Source: oarust 0.8.6, src/rs/ml/matrix/conv.rs, `Conv1dGeometry::resolve`
 * (effective kernel (k-1)*d + 1; error when the padded input is shorter).
 * Returns CONV_ERR_INVALID_ARG when in, k, stride or dil < 1, pad < 0, the
 * dilated kernel does not fit the padded input, or `out` is NULL.
 */
int conv_out_size(int in, int k, int stride, int pad, int dil, int *out);

/*
 * Forward convolution y = conv(x, w) + bias (see the definition above).
 *   x, w, y : device pointers, layout and dtype per `layout`, `dtype`.
 *   bias    : device pointer to C_out values, or NULL for no bias.
 *   N, C, H, W       : input batch, channels, height, width (>= 1).
 *   C_out, KH, KW    : output channels and kernel extent (>= 1).
 *   stride_*, dil_* : >= 1;  pad_* : >= 0 (the same pad on both sides).
 *   groups : >= 1, dividing both C and C_out.
 *   layout : conv_layout_t;  dtype : conv_dtype_t;  stream : hipStream_t.
 * Errors: CONV_ERR_INVALID_ARG (null x/w/y, a value out of range, groups not
 * dividing the channels, kernel larger than the padded input, bad enum),
 * CONV_ERR_OVERFLOW (x, y or w of one image beyond INT32_MAX elements, or
 * a padded coordinate beyond INT32_MAX), CONV_ERR_HIP (launch failed).
 */
int conv_fwd(const void *x, const void *w, const void *bias, void *y, int N,
             int C, int H, int W, int C_out, int KH, int KW, int stride_h,
             int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
             int groups, int layout, int dtype, void *stream);

/* conv_fwd with an explicit path (conv_path_t). */
int conv_fwd_ex(const void *x, const void *w, const void *bias, void *y,
                int N, int C, int H, int W, int C_out, int KH, int KW,
                int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                int dil_w, int groups, int layout, int dtype, int path,
                void *stream);

/*
 * Input gradient of the bias-free forward convolution:
 *   dx[n, ci, ih, iw] = sum over co in ci's group and taps (kh, kw) with
 *     t_h = ih + ph - kh*dh >= 0, t_h % sh == 0, t_h / sh < OH (and the same
 *     for w) of dy[n, co, t_h/sh, t_w/sw] * w[co, ci - g*C/G, kh, kw].
 * It is the adjoint of the forward: <conv(x), dy> = <x, dx(dy)>.  Sources:
 * teeny-kernels 0.2.0, src/nn/conv/conv2d.rs, `conv2d_backward_dx` (the same
 * sum, there scattered with atomics); oarust 0.8.6, src/rs/ml/matrix/conv.rs,
 * `conv_2d_backward` (input adjoint dispatched over input elements, i.e. a
 * gather, with the output-gradient shape check).  Computed here as a gather:
 * every dx element is written exactly once, elements no tap reaches get 0.
 *   dy : device pointer, shape [N, C_out, OH, OW] (NCHW) or
 *        [N, OH, OW, C_out] (NHWC), OH/OW from conv_out_size.
 *   w  : the forward weight, layout as in conv_fwd.
 *   dx : device pointer, the forward input's shape; fully overwritten.
 *   The geometry arguments describe the FORWARD convolution, exactly as
 *   passed to conv_fwd; dx is sized from H and W, never from a transposed-
 *   convolution extent formula.
 * Errors as conv_fwd.
 */
int conv_bwd_dx(const void *dy, const void *w, void *dx, int N, int C, int H,
                int W, int C_out, int KH, int KW, int stride_h, int stride_w,
                int pad_h, int pad_w, int dil_h, int dil_w, int groups,
                int layout, int dtype, void *stream);

/* conv_bwd_dx with an explicit path (conv_path_t). */
int conv_bwd_dx_ex(const void *dy, const void *w, void *dx, int N, int C,
                   int H, int W, int C_out, int KH, int KW, int stride_h,
                   int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                   int groups, int layout, int dtype, int path, void *stream);

/*
 * One-dimensional forward convolution
 *   y[n, co, t] = bias[co] + sum_{c < C/G} sum_{k < K}
 *                 x[n, g*C/G + c, t*stride - pad + k*dil] * w[co, c, k],
 * x zero outside [0, L), g = co / (C_out/G), output length
 * OL = floor((L + 2*pad - dil*(K-1) - 1) / stride) + 1.  Source: oarust
 * 0.8.6, src/rs/ml/matrix/conv.rs, `conv_1d` and `Conv1dGeometry::resolve`
 * (NCL input, OIK weight, per-channel bias, stride, padding, dilation inside
 * the kernel window); groups as in conv_fwd.  It is the one-row case of
 * conv_fwd (H = 1, KH = 1) and runs on the same kernels.
 *   layout CONV_NCL: x [N, C, L], w [C_out, C/G, K], y [N, C_out, OL];
 *   layout CONV_NLC: x [N, L, C], w [C_out, K, C/G], y [N, OL, C_out].
 *   bias: C_out values or NULL.  Ownership, execution and errors as conv_fwd.
 */
int conv1d_fwd(const void *x, const void *w, const void *bias, void *y, int N,
               int C, int L, int C_out, int K, int stride, int pad, int dil,
               int groups, int layout, int dtype, void *stream);

/* conv1d_fwd with an explicit forward path (conv_path_t). */
int conv1d_fwd_ex(const void *x, const void *w, const void *bias, void *y,
                  int N, int C, int L, int C_out, int K, int stride, int pad,
                  int dil, int groups, int layout, int dtype, int path,
                  void *stream);

/*
 * Output extent of a transposed convolution along one axis:
 *   out = (in - 1)*stride - 2*pad + dil*(k - 1) + 1 + out_pad.
 * Source: oarust 0.8.6, src/rs/ml/matrix/conv.rs,
 * `ConvTranspose2dGeometry::resolve` ((in - 1)*stride + k - 2*pad, an error
 * when the padding removes the whole output), with dilation and an output
 * padding 0 <= out_pad < stride added per axis.  Returns
 * CONV_ERR_INVALID_ARG when an argument is out of that domain, the output is
 * empty or `out` is NULL.
 */
int conv_transpose_out_size(int in, int k, int stride, int pad, int dil,
                            int out_pad, int *out);

/*
 * Transposed 2-D convolution: every input element spreads over a window of
 * the output,
 *   y[n, co, ih*sh - ph + kh*dh, iw*sw - pw + kw*dw]
 *       += x[n, ci, ih, iw] * w[ci, co - g*C_out/G, kh, kw]
 * (ci and co in the same group g; positions outside the output dropped),
 * then y += bias[co].  Source: oarust 0.8.6, src/rs/ml/matrix/conv.rs,
 * `conv_transpose_2d` and `ConvTranspose2dGeometry::resolve` (weight
 * [C_in, C_out, K, K], output extent from conv_transpose_out_size, bias per
 * output channel); per-axis kernels, dilation, groups and output padding
 * generalise the page's square, undilated, ungrouped case.  It is the input
 * gradient (conv_bwd_dx) of the forward convolution whose input is y and
 * whose output is x, plus the bias, and runs on the same gather kernels:
 * every y element is written exactly once.
 *   layout CONV_NCHW: x [N, C_in, H, W], w [C_in, C_out/G, KH, KW],
 *                     y [N, C_out, OH, OW];
 *   layout CONV_NHWC: x [N, H, W, C_in], w [C_in, KH, KW, C_out/G],
 *                     y [N, OH, OW, C_out];
 *   OH, OW from conv_transpose_out_size.  bias: C_out values or NULL.
 * Ownership and execution as conv_fwd.  Errors: CONV_ERR_INVALID_ARG (null
 * x/w/y, a value out of range, groups not dividing both channel counts,
 * output padding not below the stride, an empty output, bad enum),
 * CONV_ERR_OVERFLOW (an extent or one image beyond INT32_MAX elements),
 * CONV_ERR_HIP (launch failed).
 */
int conv_transpose2d(const void *x, const void *w, const void *bias, void *y,
                     int N, int C_in, int H, int W, int C_out, int KH, int KW,
                     int stride_h, int stride_w, int pad_h, int pad_w,
                     int out_pad_h, int out_pad_w, int dil_h, int dil_w,
                     int groups, int layout, int dtype, void *stream);

/* conv_transpose2d with an explicit input-gradient path (conv_path_t:
 * CONV_PATH_DX_GATHER, CONV_PATH_DX_IGEMM or CONV_PATH_DX_DEPTHWISE). */
int conv_transpose2d_ex(const void *x, const void *w, const void *bias,
                        void *y, int N, int C_in, int H, int W, int C_out,
                        int KH, int KW, int stride_h, int stride_w, int pad_h,
                        int pad_w, int out_pad_h, int out_pad_w, int dil_h,
                        int dil_w, int groups, int layout, int dtype, int path,
                        void *stream);

/*
 * Weight gradient of the forward convolution:
 *   dw[co, c, kh, kw] = sum over n, oh, ow of dy[n, co, oh, ow]
 *        * x[n, g*C/G + c, oh*sh - ph + kh*dh, ow*sw - pw + kw*dw],
 * x read as zero outside the image, g = co / (C_out/G).  Sources:
 * burn-cubecl 0.22.0-pre.4, src/kernel/conv/im2col.rs, `wgrad_im2col_1x1`
 * and `wgrad_im2col` (the sum over the pixels of the batch of grad_out times
 * the input or its im2col columns), with the contraction cut into pieces
 * whose partial products are summed afterwards (`wgrad_im2col_1x1_split`,
 * `split_count`); teeny-kernels 0.2.0, src/nn/conv/conv2d.rs,
 * `conv2d_backward_dw` (the same sum, there with atomics into a zeroed dw).
 * Computed here in two kernels on `stream`: fp32 partial sums over S pieces
 * of the pixels into `workspace`, then their sum in piece order, rounded
 * once to dtype.  No atomics: the result is deterministic.
 *   x  : the forward input, layout as in conv_fwd.
 *   dy : the gradient of the forward output, [N, C_out, OH, OW] (NCHW) or
 *        [N, OH, OW, C_out] (NHWC), OH/OW from conv_out_size.
 *   dw : the weight's shape and layout (OIHW or OHWI); fully overwritten.
 *   workspace : device memory owned by the caller, 16-byte aligned, of at
 *        least the size conv_bwd_dw_workspace_size reports for the same
 *        geometry and path; its contents on entry are ignored and on return
 *        unspecified.  It may be NULL when that size is 0.
 *   The geometry arguments describe the FORWARD convolution, as for
 *   conv_fwd.  With conv_arm_launch_events, the start event stamps the first
 *   kernel and the stop event the second.
 * Errors as conv_fwd, and CONV_ERR_INVALID_ARG when the workspace is missing,
 * misaligned or too small.
 */
int conv_bwd_dw(const void *x, const void *dy, void *dw, void *workspace,
                size_t workspace_bytes, int N, int C, int H, int W, int C_out,
                int KH, int KW, int stride_h, int stride_w, int pad_h,
                int pad_w, int dil_h, int dil_w, int groups, int layout,
                int dtype, void *stream);

/* conv_bwd_dw with an explicit weight-gradient path (conv_path_t). */
int conv_bwd_dw_ex(const void *x, const void *dy, void *dw, void *workspace,
                   size_t workspace_bytes, int N, int C, int H, int W,
                   int C_out, int KH, int KW, int stride_h, int stride_w,
                   int pad_h, int pad_w, int dil_h, int dil_w, int groups,
                   int layout, int dtype, int path, void *stream);

/*
 * Workspace bytes conv_bwd_dw needs for this forward geometry, dtype and
 * path (CONV_PATH_AUTO: the path conv_bwd_dw would take), written to *bytes.
 * Host only.  Errors as conv_fwd, and CONV_ERR_INVALID_ARG for a path that
 * is not a weight-gradient path or a NULL `bytes`.
 */
int conv_bwd_dw_workspace_size(int N, int C, int H, int W, int C_out, int KH,
                               int KW, int stride_h, int stride_w, int pad_h,
                               int pad_w, int dil_h, int dil_w, int groups,
                               int layout, int dtype, int path, size_t *bytes);

/*
 * conv_bwd_dw without a workspace argument and without allocating: for
 * callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The fp32
 * partials that conv_bwd_dw keeps in the caller's workspace live instead in
 * a fixed device array of the library, 16 MiB per device, held by every
 * device the library runs on until the process ends.  The call allocates
 * nothing (no hipMalloc or allocating library routine); it takes the path
 * CONV_PATH_AUTO takes and computes exactly what conv_bwd_dw computes.
 * Arguments, layouts, ownership and errors as conv_bwd_dw (minus the
 * workspace), and CONV_ERR_UNSUPPORTED when the geometry needs more scratch
 * than 16 MiB (conv_bwd_dw_workspace_size reports the need) -- nothing is
 * launched then.  All calls on one device share the array: calls that
 * overlap on one device (other streams, other threads) race and must be
 * serialised by the caller.  The array's contents between calls are
 * unspecified; no call relies on them.
 */
int conv_bwd_dw_noalloc(const void *x, const void *dy, void *dw, int N, int C,
                        int H, int W, int C_out, int KH, int KW, int stride_h,
                        int stride_w, int pad_h, int pad_w, int dil_h,
                        int dil_w, int groups, int layout, int dtype,
                        void *stream);

/*
 * The path CONV_PATH_AUTO would take for this geometry, written to
 * *path_out.  Host only; launches nothing.  `backward` = 0 selects among the
 * forward paths, 1 among the input-gradient paths, 2 among the
 * weight-gradient paths.  Errors as conv_fwd.
 * (conv1d_fwd takes the forward path of H = 1, KH = 1; conv_transpose2d the
 * input-gradient path of its forward geometry.)
 */
int conv_select_path(int backward, int N, int C, int H, int W, int C_out,
                     int KH, int KW, int stride_h, int stride_w, int pad_h,
                     int pad_w, int dil_h, int dil_w, int groups, int layout,
                     int dtype, int *path_out);

/* Name of a conv_path_t value ("direct", "igemm", ...), or "unknown". */
const char *conv_path_name(int path);

/*
 * Measurement hook.  The next kernel launched by a conv_* call on the
 * calling thread stamps its own execution start into `start` and its end
 * into `stop` (hipEvent_t handles created by the caller with timing enabled;
 * either may be NULL), through hipExtLaunchKernel, which adds no packets to
 * the stream.  Every forward and input-gradient path launches exactly one
 * kernel per call, so hipEventElapsedTime(start, stop) is that kernel's
 * duration; a weight gradient stamps the start of its first kernel and the
 * end of its second.  The events
 * are disarmed by that launch; a call that fails validation leaves them
 * armed.  Always returns CONV_OK.
 */
int conv_arm_launch_events(void *start, void *stop);

/* Message describing the last failure on the calling thread ("" if none). */
const char *conv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVMI_H */
