"""fp64 CPU reference for 2-D convolution and its input gradient.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark import this package.  The product library never
imports, links or calls it, and the two share no code.

The arithmetic lives in ``conv_oracle.c`` (plain C, fp64, OpenMP); this module
only marshals numpy arrays into it.  Sources, per function:

* ``out_size`` -- oarust 0.8.6 ``src/rs/ml/matrix/conv.rs``,
  ``Conv1dGeometry::resolve``: effective kernel ``(k-1)*d+1``, extent
  ``(in + 2p - effective) / s + 1``, error when the kernel does not fit.
* ``conv2d_forward`` / ``conv2d_forward_at`` -- teeny-kernels 0.2.0
  ``src/nn/conv/conv2d.rs``, ``conv2d_forward`` (tap indexing, grouping,
  zero padding) and ``conv2d_bias_forward`` (bias); dilation as in
  burn-cubecl 0.22.0-pre.4 ``src/kernel/conv/im2col.rs``, ``im2col``.
* ``conv2d_input_grad`` -- the adjoint of the bias-free forward, as the
  scatter that transposes the forward loop (teeny-kernels,
  ``conv2d_backward_dx``, without atomics).
* ``conv2d_input_grad_at`` -- the same adjoint evaluated per input element
  as a gather (oarust, ``conv_2d_backward``, input adjoint dispatched over
  input elements).
* ``conv2d_weight_grad`` -- burn-cubecl, ``wgrad_im2col_1x1`` and
  ``wgrad_im2col`` (the sum over pixels of grad_out times the input, or its
  im2col columns), teeny-kernels ``conv2d_backward_dw`` (the same sum per
  weight element), as the defining sum per weight element.
* ``conv1d_forward`` -- oarust, ``conv_1d`` and ``Conv1dGeometry::resolve``
  (NCL input, OIK weight, bias, stride, padding, dilation), as the defining
  sum; groups as in the 2-D forward.
* ``conv_transpose_size`` / ``conv_transpose2d`` -- oarust,
  ``conv_transpose_2d`` and ``ConvTranspose2dGeometry::resolve`` (weight
  [C_in, C_out, K, K], extent (H-1)*s + K - 2p, bias), as the scatter of
  every input element over its output window; per-axis dilation, groups and
  output padding generalise the page's case.

Every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, hand-worked examples, brute-force im2col + GEMM, identities and the
torch CPU fp64 library convolution.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
# Built with AddressSanitizer and UndefinedBehaviorSanitizer (clang, whose
# runtime the process must preload); loaded instead of the plain build when
# CONVMI_SANITIZED=1.
_SO_SAN = os.path.join(_HERE, "liboracle_san.so")
_CLANG = "/opt/rocm/llvm/bin/clang"
_lib = None

_L = ctypes.c_long
_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)
_GEOM = [_L] * 14 + [ctypes.c_int]


def build(sanitize: bool = False) -> str:
    """Compile ``conv_oracle.c`` into ``liboracle.so`` with gcc, or with
    ``sanitize`` into ``liboracle_san.so`` with clang under AddressSanitizer
    and UndefinedBehaviorSanitizer (any report aborts)."""
    if sanitize:
        out = _SO_SAN
        cmd = [_CLANG, "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-shared-libasan"]
    else:
        out = _SO
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall"]
    tmp = out + ".tmp"
    subprocess.run(cmd + ["-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    sanitized = os.environ.get("CONVMI_SANITIZED") == "1"
    so = _SO_SAN if sanitized else _SO
    if not os.path.exists(so):
        build(sanitize=sanitized)
    lib = ctypes.CDLL(so)
    lib.oracle_out_size.restype = _L
    lib.oracle_out_size.argtypes = [_L] * 5
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_conv2d_forward.restype = ctypes.c_int
    lib.oracle_conv2d_forward.argtypes = [_D, _D, _D, _D, _D] + _GEOM
    lib.oracle_conv2d_forward_at.restype = ctypes.c_int
    lib.oracle_conv2d_forward_at.argtypes = [_D, _D, _D, _I64, _L, _D, _D] + _GEOM
    lib.oracle_conv2d_input_grad.restype = ctypes.c_int
    lib.oracle_conv2d_input_grad.argtypes = [_D, _D, _D, _D] + _GEOM
    lib.oracle_conv2d_input_grad_at.restype = ctypes.c_int
    lib.oracle_conv2d_input_grad_at.argtypes = [_D, _D, _I64, _L, _D, _D] + _GEOM
    lib.oracle_conv2d_weight_grad.restype = ctypes.c_int
    lib.oracle_conv2d_weight_grad.argtypes = [_D, _D, _D, _D] + _GEOM
    lib.oracle_conv1d_forward.restype = ctypes.c_int
    lib.oracle_conv1d_forward.argtypes = [_D, _D, _D, _D, _D] + [_L] * 9 + [ctypes.c_int]
    lib.oracle_conv_transpose_size.restype = _L
    lib.oracle_conv_transpose_size.argtypes = [_L] * 6
    lib.oracle_conv_transpose2d.restype = ctypes.c_int
    lib.oracle_conv_transpose2d.argtypes = [_D, _D, _D, _D, _D] + [_L] * 16 + [ctypes.c_int]
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_threads())


def out_size(n: int, k: int, stride: int, pad: int, dil: int):
    """Output extent along one axis, or ``None`` if the kernel does not fit."""
    r = int(_load().oracle_out_size(n, k, stride, pad, dil))
    return None if r < 0 else r


def _pair(v):
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor: exact upcast to fp64
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_D)


def _geometry(x_shape, w_shape, stride, padding, dilation, groups, layout):
    nhwc = {"NCHW": 0, "NHWC": 1}[layout]
    if nhwc:
        N, H, W, C = x_shape
        CO, KH, KW, _ = w_shape
    else:
        N, C, H, W = x_shape
        CO, _, KH, KW = w_shape
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    geom = (N, C, H, W, CO, KH, KW, sh, sw, ph, pw, dh, dw, int(groups), nhwc)
    OH = out_size(H, KH, sh, ph, dh)
    OW = out_size(W, KW, sw, pw, dw)
    if OH is None or OW is None:
        raise ValueError("kernel does not fit the padded input")
    y_shape = (N, OH, OW, CO) if nhwc else (N, CO, OH, OW)
    return geom, y_shape


def conv2d_forward(x, w, bias=None, stride=1, padding=0, dilation=1, groups=1, layout="NCHW"):
    """Full forward convolution in fp64.  Returns ``(y, norm)``."""
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    geom, y_shape = _geometry(x.shape, w.shape, stride, padding, dilation, groups, layout)
    y = np.empty(y_shape, np.float64)
    norm = np.empty(y_shape, np.float64)
    rc = _load().oracle_conv2d_forward(_ptr(x), _ptr(w), _ptr(b), _ptr(y), _ptr(norm), *geom)
    if rc != 0:
        raise ValueError(f"oracle rejected the geometry (rc={rc})")
    return y, norm


def conv2d_forward_at(x, w, bias, idx, stride=1, padding=0, dilation=1, groups=1, layout="NCHW"):
    """Forward outputs at flat offsets ``idx`` of ``y``.  Returns ``(vals, norm)``."""
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    geom, _ = _geometry(x.shape, w.shape, stride, padding, dilation, groups, layout)
    out = np.empty(idx.shape, np.float64)
    norm = np.empty(idx.shape, np.float64)
    rc = _load().oracle_conv2d_forward_at(
        _ptr(x), _ptr(w), _ptr(b), idx.ctypes.data_as(_I64), idx.size, _ptr(out), _ptr(norm), *geom
    )
    if rc != 0:
        raise ValueError(f"oracle rejected the request (rc={rc})")
    return out, norm


def conv2d_input_grad(dy, w, input_shape, stride=1, padding=0, dilation=1, groups=1, layout="NCHW"):
    """Input gradient (scatter form) in fp64.  Returns ``(dx, norm)``."""
    dy, w = _f64(dy), _f64(w)
    geom, y_shape = _geometry(tuple(input_shape), w.shape, stride, padding, dilation, groups, layout)
    if tuple(dy.shape) != tuple(y_shape):
        raise ValueError(f"dy has shape {dy.shape}, expected {y_shape}")
    dx = np.empty(tuple(input_shape), np.float64)
    norm = np.empty(tuple(input_shape), np.float64)
    rc = _load().oracle_conv2d_input_grad(_ptr(dy), _ptr(w), _ptr(dx), _ptr(norm), *geom)
    if rc != 0:
        raise ValueError(f"oracle rejected the geometry (rc={rc})")
    return dx, norm


def conv2d_input_grad_at(dy, w, input_shape, idx, stride=1, padding=0, dilation=1, groups=1,
                         layout="NCHW"):
    """Input gradient (gather form) at flat offsets ``idx`` of ``dx``."""
    dy, w = _f64(dy), _f64(w)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    geom, y_shape = _geometry(tuple(input_shape), w.shape, stride, padding, dilation, groups, layout)
    if tuple(dy.shape) != tuple(y_shape):
        raise ValueError(f"dy has shape {dy.shape}, expected {y_shape}")
    out = np.empty(idx.shape, np.float64)
    norm = np.empty(idx.shape, np.float64)
    rc = _load().oracle_conv2d_input_grad_at(
        _ptr(dy), _ptr(w), idx.ctypes.data_as(_I64), idx.size, _ptr(out), _ptr(norm), *geom
    )
    if rc != 0:
        raise ValueError(f"oracle rejected the request (rc={rc})")
    return out, norm


def conv2d_weight_grad(x, dy, w_shape, stride=1, padding=0, dilation=1, groups=1, layout="NCHW"):
    """Weight gradient in fp64, laid out like the forward's weight of shape
    ``w_shape``.  Returns ``(dw, norm)``."""
    x, dy = _f64(x), _f64(dy)
    geom, y_shape = _geometry(x.shape, tuple(w_shape), stride, padding, dilation, groups, layout)
    if tuple(dy.shape) != tuple(y_shape):
        raise ValueError(f"dy has shape {dy.shape}, expected {y_shape}")
    dw = np.empty(tuple(w_shape), np.float64)
    norm = np.empty(tuple(w_shape), np.float64)
    rc = _load().oracle_conv2d_weight_grad(_ptr(x), _ptr(dy), _ptr(dw), _ptr(norm), *geom)
    if rc != 0:
        raise ValueError(f"oracle rejected the geometry (rc={rc})")
    return dw, norm


def conv1d_forward(x, w, bias=None, stride=1, padding=0, dilation=1, groups=1, layout="NCL"):
    """1-D forward convolution in fp64.  ``layout`` is "NCL" (x [N, C, L],
    w [C_out, C/G, K]) or "NLC" (x [N, L, C], w [C_out, K, C/G]).  Returns
    ``(y, norm)``."""
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    nlc = {"NCL": 0, "NLC": 1}[layout]
    if nlc:
        N, L, C = x.shape
        CO, K, _ = w.shape
    else:
        N, C, L = x.shape
        CO, _, K = w.shape
    OL = out_size(L, K, stride, padding, dilation)
    if OL is None:
        raise ValueError("kernel does not fit the padded input")
    y_shape = (N, OL, CO) if nlc else (N, CO, OL)
    y = np.empty(y_shape, np.float64)
    norm = np.empty(y_shape, np.float64)
    rc = _load().oracle_conv1d_forward(_ptr(x), _ptr(w), _ptr(b), _ptr(y), _ptr(norm), N, C, L, CO,
                                       K, int(stride), int(padding), int(dilation), int(groups), nlc)
    if rc != 0:
        raise ValueError(f"oracle rejected the geometry (rc={rc})")
    return y, norm


def conv_transpose_size(n: int, k: int, stride: int, pad: int, dil: int = 1, out_pad: int = 0):
    """Output extent of a transposed convolution along one axis, or ``None``."""
    r = int(_load().oracle_conv_transpose_size(n, k, stride, pad, dil, out_pad))
    return None if r < 0 else r


def conv_transpose2d(x, w, bias=None, stride=1, padding=0, output_padding=0, dilation=1, groups=1,
                     layout="NCHW"):
    """Transposed 2-D convolution (scatter form) in fp64.  NCHW: x [N, C_in, H, W],
    w [C_in, C_out/G, KH, KW]; NHWC: x [N, H, W, C_in], w [C_in, KH, KW, C_out/G].
    Returns ``(y, norm)``."""
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    nhwc = {"NCHW": 0, "NHWC": 1}[layout]
    if nhwc:
        N, H, W, CI = x.shape
        _, KH, KW, Mg = w.shape
    else:
        N, CI, H, W = x.shape
        _, Mg, KH, KW = w.shape
    CO = Mg * int(groups)
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    oph, opw = _pair(output_padding)
    dh, dw = _pair(dilation)
    OH = conv_transpose_size(H, KH, sh, ph, dh, oph)
    OW = conv_transpose_size(W, KW, sw, pw, dw, opw)
    if OH is None or OW is None:
        raise ValueError("invalid transposed-convolution geometry")
    y_shape = (N, OH, OW, CO) if nhwc else (N, CO, OH, OW)
    y = np.empty(y_shape, np.float64)
    norm = np.empty(y_shape, np.float64)
    rc = _load().oracle_conv_transpose2d(_ptr(x), _ptr(w), _ptr(b), _ptr(y), _ptr(norm), N, CI, H, W,
                                         CO, KH, KW, sh, sw, ph, pw, oph, opw, dh, dw, int(groups),
                                         nhwc)
    if rc != 0:
        raise ValueError(f"oracle rejected the geometry (rc={rc})")
    return y, norm


def max_normalised_error(got, ref, norm) -> float:
    """``max |got - ref| / norm``; where ``norm == 0`` any difference is infinite."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    norm = np.asarray(norm, np.float64)
    diff = np.abs(got - ref)
    if diff.size == 0:
        return 0.0
    zero = norm == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    return float(np.max(diff[~zero] / norm[~zero], initial=0.0))
