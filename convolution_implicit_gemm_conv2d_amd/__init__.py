"""Python binding of the convmi C ABI (include/convmi.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libconvmi.so``.  PyTorch provides device memory and the current
stream.  The low-level functions carry the C names and arguments;
``conv2d``, ``conv2d_input_grad``, ``conv2d_weight_grad``, ``conv1d`` and
``conv2d_transposed`` derive the sizes from tensor shapes and allocate the
output (and the weight gradient's workspace, when none is given).
"""
from __future__ import annotations

import ctypes

from . import _lib

CONV_OK = 0
CONV_ERR_INVALID_ARG = 1
CONV_ERR_UNSUPPORTED = 2
CONV_ERR_OVERFLOW = 3
CONV_ERR_HIP = 4

CONV_NCHW = 0
CONV_NHWC = 1
CONV_NCL = 0
CONV_NLC = 1
CONV_F32 = 0
CONV_BF16 = 1

PATHS = {
    "auto": 0,
    "direct": 1,
    "igemm": 2,
    "pointwise": 3,
    "depthwise": 4,
    "dx_gather": 5,
    "dx_igemm": 6,
    "igemm_band": 7,
    "dw_direct": 8,
    "dw_igemm": 9,
    "dx_depthwise": 10,
    "dx_band": 11,
}

__all__ = [
    "ConvError", "conv_out_size", "conv_fwd", "conv_fwd_ex", "conv_bwd_dx", "conv_bwd_dx_ex",
    "conv_select_path", "conv_path_name", "conv_last_error", "conv_arm_launch_events", "conv2d",
    "conv2d_input_grad", "conv1d_fwd", "conv1d_fwd_ex", "conv_transpose_out_size",
    "conv_transpose2d", "conv_transpose2d_ex", "conv1d", "conv2d_transposed", "conv_bwd_dw",
    "conv_bwd_dw_ex", "conv_bwd_dw_workspace_size", "conv2d_weight_grad",
    "library_path", "PATHS",
]


class ConvError(RuntimeError):
    """A nonzero conv_status_t, with the library's message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"convmi status {status}: {message}")
        self.status = status
        self.message = message


def library_path() -> str:
    return _lib.LIB_PATH


def _check(rc: int) -> None:
    if rc != CONV_OK:
        raise ConvError(rc, conv_last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors passed to convmi must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError("tensors passed to convmi must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def conv_path_name(path: int) -> str:
    return _lib.load().conv_path_name(int(path)).decode()


def conv_last_error() -> str:
    return _lib.load().conv_last_error().decode()


def conv_arm_launch_events(start, stop) -> None:
    """Arms raw hipEvent_t handles (ints) for the next launch on this thread."""
    _check(_lib.load().conv_arm_launch_events(start, stop))


def conv_out_size(n: int, k: int, stride: int, pad: int, dil: int) -> int:
    out = ctypes.c_int(0)
    _check(_lib.load().conv_out_size(n, k, stride, pad, dil, ctypes.byref(out)))
    return out.value


def conv_fwd(x, w, bias, y, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
             dil_h, dil_w, groups, layout, dtype, stream=None) -> None:
    _check(_lib.load().conv_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, C, H, W, C_out, KH, KW,
                                stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups, layout,
                                dtype, _stream(stream)))


def conv_fwd_ex(x, w, bias, y, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
                dil_h, dil_w, groups, layout, dtype, path, stream=None) -> None:
    _check(_lib.load().conv_fwd_ex(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, C, H, W, C_out, KH,
                                   KW, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups,
                                   layout, dtype, path, _stream(stream)))


def conv_bwd_dx(dy, w, dx, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w, dil_h,
                dil_w, groups, layout, dtype, stream=None) -> None:
    _check(_lib.load().conv_bwd_dx(_ptr(dy), _ptr(w), _ptr(dx), N, C, H, W, C_out, KH, KW,
                                   stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups, layout,
                                   dtype, _stream(stream)))


def conv_bwd_dx_ex(dy, w, dx, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w, dil_h,
                   dil_w, groups, layout, dtype, path, stream=None) -> None:
    _check(_lib.load().conv_bwd_dx_ex(_ptr(dy), _ptr(w), _ptr(dx), N, C, H, W, C_out, KH, KW,
                                      stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups,
                                      layout, dtype, path, _stream(stream)))


def conv_select_path(backward, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
                     dil_h, dil_w, groups, layout, dtype) -> int:
    out = ctypes.c_int(0)
    _check(_lib.load().conv_select_path(int(backward), N, C, H, W, C_out, KH, KW, stride_h,
                                        stride_w, pad_h, pad_w, dil_h, dil_w, groups, layout,
                                        dtype, ctypes.byref(out)))
    return out.value


def conv1d_fwd(x, w, bias, y, N, C, L, C_out, K, stride, pad, dil, groups, layout, dtype,
               stream=None) -> None:
    _check(_lib.load().conv1d_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, C, L, C_out, K,
                                  stride, pad, dil, groups, layout, dtype, _stream(stream)))


def conv1d_fwd_ex(x, w, bias, y, N, C, L, C_out, K, stride, pad, dil, groups, layout, dtype, path,
                  stream=None) -> None:
    _check(_lib.load().conv1d_fwd_ex(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, C, L, C_out, K,
                                     stride, pad, dil, groups, layout, dtype, path,
                                     _stream(stream)))


def conv_transpose_out_size(n: int, k: int, stride: int, pad: int, dil: int = 1,
                            out_pad: int = 0) -> int:
    out = ctypes.c_int(0)
    _check(_lib.load().conv_transpose_out_size(n, k, stride, pad, dil, out_pad, ctypes.byref(out)))
    return out.value


def conv_transpose2d(x, w, bias, y, N, C_in, H, W, C_out, KH, KW, stride_h, stride_w, pad_h,
                     pad_w, out_pad_h, out_pad_w, dil_h, dil_w, groups, layout, dtype,
                     stream=None) -> None:
    _check(_lib.load().conv_transpose2d(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, C_in, H, W,
                                        C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
                                        out_pad_h, out_pad_w, dil_h, dil_w, groups, layout, dtype,
                                        _stream(stream)))


def conv_transpose2d_ex(x, w, bias, y, N, C_in, H, W, C_out, KH, KW, stride_h, stride_w, pad_h,
                        pad_w, out_pad_h, out_pad_w, dil_h, dil_w, groups, layout, dtype, path,
                        stream=None) -> None:
    _check(_lib.load().conv_transpose2d_ex(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, C_in, H, W,
                                           C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
                                           out_pad_h, out_pad_w, dil_h, dil_w, groups, layout,
                                           dtype, path, _stream(stream)))


def conv_bwd_dw(x, dy, dw, workspace, workspace_bytes, N, C, H, W, C_out, KH, KW, stride_h,
                stride_w, pad_h, pad_w, dil_h, dil_w, groups, layout, dtype, stream=None) -> None:
    _check(_lib.load().conv_bwd_dw(_ptr(x), _ptr(dy), _ptr(dw), _ptr(workspace), workspace_bytes,
                                   N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
                                   dil_h, dil_w, groups, layout, dtype, _stream(stream)))


def conv_bwd_dw_ex(x, dy, dw, workspace, workspace_bytes, N, C, H, W, C_out, KH, KW, stride_h,
                   stride_w, pad_h, pad_w, dil_h, dil_w, groups, layout, dtype, path,
                   stream=None) -> None:
    _check(_lib.load().conv_bwd_dw_ex(_ptr(x), _ptr(dy), _ptr(dw), _ptr(workspace),
                                      workspace_bytes, N, C, H, W, C_out, KH, KW, stride_h,
                                      stride_w, pad_h, pad_w, dil_h, dil_w, groups, layout, dtype,
                                      path, _stream(stream)))


def conv_bwd_dw_noalloc(x, dy, dw, N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
                        dil_h, dil_w, groups, layout, dtype, stream=None) -> None:
    _check(_lib.load().conv_bwd_dw_noalloc(_ptr(x), _ptr(dy), _ptr(dw), N, C, H, W, C_out, KH, KW,
                                           stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups,
                                           layout, dtype, _stream(stream)))


def conv_bwd_dw_workspace_size(N, C, H, W, C_out, KH, KW, stride_h, stride_w, pad_h, pad_w,
                               dil_h, dil_w, groups, layout, dtype, path=0) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.load().conv_bwd_dw_workspace_size(N, C, H, W, C_out, KH, KW, stride_h, stride_w,
                                                  pad_h, pad_w, dil_h, dil_w, groups, layout,
                                                  dtype, path, ctypes.byref(out)))
    return out.value


# ----------------------------------------------------------- tensor level --

def _pair(v):
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _dtype_code(t):
    import torch

    if t.dtype == torch.float32:
        return CONV_F32
    if t.dtype == torch.bfloat16:
        return CONV_BF16
    raise ValueError(f"unsupported dtype {t.dtype}; convmi takes float32 or bfloat16")


def _layout_code(layout: str) -> int:
    try:
        return {"NCHW": CONV_NCHW, "NHWC": CONV_NHWC}[layout]
    except KeyError:
        raise ValueError(f"layout must be 'NCHW' or 'NHWC', got {layout!r}") from None


def _dims(x_shape, w, layout):
    if len(x_shape) != 4 or w.dim() != 4:
        raise ValueError("input and weight must both have rank four")
    if layout == "NHWC":
        N, H, W, C = x_shape
        C_out, KH, KW, Cg = w.shape
    else:
        N, C, H, W = x_shape
        C_out, Cg, KH, KW = w.shape
    return int(N), int(C), int(H), int(W), int(C_out), int(KH), int(KW), int(Cg)


def conv2d(x, w, bias=None, stride=1, padding=0, dilation=1, groups=1, layout="NHWC",
           path="auto", out=None, stream=None):
    """Forward convolution of torch tensors on the GPU; returns ``y``."""
    import torch

    lay = _layout_code(layout)
    dt = _dtype_code(x)
    for t in (w, bias, out):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("x, w, bias and out must share one dtype")
    N, C, H, W, C_out, KH, KW, Cg = _dims(tuple(x.shape), w, layout)
    if groups < 1 or C % groups or Cg != C // groups:
        raise ValueError(f"weight expects {Cg} input channels per group; x has {C} channels "
                         f"in {groups} groups")
    if bias is not None and tuple(bias.shape) != (C_out,):
        raise ValueError(f"bias must have shape [{C_out}]")
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    OH = conv_out_size(H, KH, sh, ph, dh)
    OW = conv_out_size(W, KW, sw, pw, dw)
    shape = (N, OH, OW, C_out) if lay == CONV_NHWC else (N, C_out, OH, OW)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    conv_fwd_ex(x, w, bias, out, N, C, H, W, C_out, KH, KW, sh, sw, ph, pw, dh, dw, groups, lay,
                dt, PATHS[path], stream)
    return out


def conv2d_input_grad(dy, w, input_shape, stride=1, padding=0, dilation=1, groups=1,
                      layout="NHWC", path="auto", out=None, stream=None):
    """Input gradient of the forward convolution; returns ``dx`` of ``input_shape``."""
    import torch

    lay = _layout_code(layout)
    dt = _dtype_code(dy)
    if w.dtype != dy.dtype or (out is not None and out.dtype != dy.dtype):
        raise ValueError("dy, w and out must share one dtype")
    input_shape = tuple(int(v) for v in input_shape)
    N, C, H, W, C_out, KH, KW, Cg = _dims(input_shape, w, layout)
    if groups < 1 or C % groups or Cg != C // groups:
        raise ValueError(f"weight expects {Cg} input channels per group; input has {C} "
                         f"channels in {groups} groups")
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    OH = conv_out_size(H, KH, sh, ph, dh)
    OW = conv_out_size(W, KW, sw, pw, dw)
    dy_shape = (N, OH, OW, C_out) if lay == CONV_NHWC else (N, C_out, OH, OW)
    if tuple(dy.shape) != dy_shape:
        raise ValueError(f"output gradient must have shape {dy_shape}; found {tuple(dy.shape)}")
    if out is None:
        out = torch.empty(input_shape, dtype=dy.dtype, device=dy.device)
    elif tuple(out.shape) != input_shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {input_shape}")
    conv_bwd_dx_ex(dy, w, out, N, C, H, W, C_out, KH, KW, sh, sw, ph, pw, dh, dw, groups, lay, dt,
                   PATHS[path], stream)
    return out


def conv1d(x, w, bias=None, stride=1, padding=0, dilation=1, groups=1, layout="NLC", path="auto",
           out=None, stream=None):
    """1-D forward convolution of torch tensors on the GPU; returns ``y``.
    ``layout`` "NCL": x [N, C, L], w [C_out, C/G, K]; "NLC": x [N, L, C],
    w [C_out, K, C/G]."""
    import torch

    try:
        lay = {"NCL": CONV_NCL, "NLC": CONV_NLC}[layout]
    except KeyError:
        raise ValueError(f"layout must be 'NCL' or 'NLC', got {layout!r}") from None
    dt = _dtype_code(x)
    for t in (w, bias, out):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("x, w, bias and out must share one dtype")
    if x.dim() != 3 or w.dim() != 3:
        raise ValueError("input and weight must both have rank three")
    if lay == CONV_NLC:
        N, L, C = (int(v) for v in x.shape)
        C_out, K, Cg = (int(v) for v in w.shape)
    else:
        N, C, L = (int(v) for v in x.shape)
        C_out, Cg, K = (int(v) for v in w.shape)
    if groups < 1 or C % groups or Cg != C // groups:
        raise ValueError(f"weight expects {Cg} input channels per group; x has {C} channels "
                         f"in {groups} groups")
    if bias is not None and tuple(bias.shape) != (C_out,):
        raise ValueError(f"bias must have shape [{C_out}]")
    OL = conv_out_size(L, K, int(stride), int(padding), int(dilation))
    shape = (N, OL, C_out) if lay == CONV_NLC else (N, C_out, OL)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    conv1d_fwd_ex(x, w, bias, out, N, C, L, C_out, K, int(stride), int(padding), int(dilation),
                  int(groups), lay, dt, PATHS[path], stream)
    return out


def conv2d_transposed(x, w, bias=None, stride=1, padding=0, output_padding=0, dilation=1,
                      groups=1, layout="NHWC", path="auto", out=None, stream=None):
    """Transposed 2-D convolution of torch tensors on the GPU; returns ``y``.
    NCHW: x [N, C_in, H, W], w [C_in, C_out/G, KH, KW]; NHWC: x [N, H, W, C_in],
    w [C_in, KH, KW, C_out/G]."""
    import torch

    lay = _layout_code(layout)
    dt = _dtype_code(x)
    for t in (w, bias, out):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("x, w, bias and out must share one dtype")
    if x.dim() != 4 or w.dim() != 4:
        raise ValueError("input and weight must both have rank four")
    if lay == CONV_NHWC:
        N, H, W, C_in = (int(v) for v in x.shape)
        C_in_w, KH, KW, Mg = (int(v) for v in w.shape)
    else:
        N, C_in, H, W = (int(v) for v in x.shape)
        C_in_w, Mg, KH, KW = (int(v) for v in w.shape)
    if C_in_w != C_in:
        raise ValueError(f"weight has {C_in_w} input channels; x has {C_in}")
    if groups < 1 or C_in % groups:
        raise ValueError(f"{groups} groups do not divide {C_in} input channels")
    C_out = Mg * int(groups)
    if bias is not None and tuple(bias.shape) != (C_out,):
        raise ValueError(f"bias must have shape [{C_out}]")
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    oph, opw = _pair(output_padding)
    dh, dw = _pair(dilation)
    OH = conv_transpose_out_size(H, KH, sh, ph, dh, oph)
    OW = conv_transpose_out_size(W, KW, sw, pw, dw, opw)
    shape = (N, OH, OW, C_out) if lay == CONV_NHWC else (N, C_out, OH, OW)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    conv_transpose2d_ex(x, w, bias, out, N, C_in, H, W, C_out, KH, KW, sh, sw, ph, pw, oph, opw,
                        dh, dw, int(groups), lay, dt, PATHS[path], stream)
    return out


def conv2d_weight_grad(x, dy, w_shape, stride=1, padding=0, dilation=1, groups=1, layout="NHWC",
                       path="auto", out=None, workspace=None, stream=None):
    """Weight gradient of the forward convolution; returns ``dw`` of ``w_shape``.
    ``workspace`` (a byte tensor on the device) is allocated when not given."""
    import torch

    lay = _layout_code(layout)
    dt = _dtype_code(x)
    if dy.dtype != x.dtype or (out is not None and out.dtype != x.dtype):
        raise ValueError("x, dy and out must share one dtype")
    w_shape = tuple(int(v) for v in w_shape)
    if len(w_shape) != 4 or x.dim() != 4:
        raise ValueError("input and weight must both have rank four")
    if lay == CONV_NHWC:
        N, H, W, C = (int(v) for v in x.shape)
        C_out, KH, KW, Cg = w_shape
    else:
        N, C, H, W = (int(v) for v in x.shape)
        C_out, Cg, KH, KW = w_shape
    if groups < 1 or C % groups or Cg != C // groups:
        raise ValueError(f"weight expects {Cg} input channels per group; x has {C} channels "
                         f"in {groups} groups")
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw_ = _pair(dilation)
    OH = conv_out_size(H, KH, sh, ph, dh)
    OW = conv_out_size(W, KW, sw, pw, dw_)
    dy_shape = (N, OH, OW, C_out) if lay == CONV_NHWC else (N, C_out, OH, OW)
    if tuple(dy.shape) != dy_shape:
        raise ValueError(f"output gradient must have shape {dy_shape}; found {tuple(dy.shape)}")
    if out is None:
        out = torch.empty(w_shape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != w_shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {w_shape}")
    code = PATHS[path]
    need = conv_bwd_dw_workspace_size(N, C, H, W, C_out, KH, KW, sh, sw, ph, pw, dh, dw_, groups,
                                      lay, dt, code)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    conv_bwd_dw_ex(x, dy, out, workspace, workspace.numel() * workspace.element_size(), N, C, H, W,
                   C_out, KH, KW, sh, sw, ph, pw, dh, dw_, groups, lay, dt, code, stream)
    return out
