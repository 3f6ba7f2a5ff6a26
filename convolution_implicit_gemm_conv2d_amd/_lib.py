"""Loads ``libconvmi.so`` and declares the C signatures of include/convmi.h."""
from __future__ import annotations

import ctypes
import os

# CONVMI_SANITIZED=1 loads the build whose host code runs under ASan and
# UBSan (the process must preload the sanitizer runtime); the kernels are the
# same.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libconvmi_san.so" if os.environ.get("CONVMI_SANITIZED") == "1"
                        else "libconvmi.so")

_I = ctypes.c_int
_P = ctypes.c_void_p

# Name -> (restype, argtypes), mirroring include/convmi.h.
_GEOM = [_I] * 16  # N C H W C_out KH KW sh sw ph pw dh dw groups layout dtype
SIGNATURES = {
    "conv_out_size": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(_I)]),
    "conv_fwd": (_I, [_P, _P, _P, _P] + _GEOM + [_P]),
    "conv_fwd_ex": (_I, [_P, _P, _P, _P] + _GEOM + [_I, _P]),
    "conv_bwd_dx": (_I, [_P, _P, _P] + _GEOM + [_P]),
    "conv_bwd_dx_ex": (_I, [_P, _P, _P] + _GEOM + [_I, _P]),
    "conv_select_path": (_I, [_I] + _GEOM + [ctypes.POINTER(_I)]),
    # N C L C_out K stride pad dil groups layout dtype
    "conv1d_fwd": (_I, [_P, _P, _P, _P] + [_I] * 11 + [_P]),
    "conv1d_fwd_ex": (_I, [_P, _P, _P, _P] + [_I] * 12 + [_P]),
    "conv_transpose_out_size": (_I, [_I] * 6 + [ctypes.POINTER(_I)]),
    # N C_in H W C_out KH KW sh sw ph pw oph opw dh dw groups layout dtype
    "conv_transpose2d": (_I, [_P, _P, _P, _P] + [_I] * 18 + [_P]),
    "conv_transpose2d_ex": (_I, [_P, _P, _P, _P] + [_I] * 19 + [_P]),
    "conv_bwd_dw": (_I, [_P, _P, _P, _P, ctypes.c_size_t] + _GEOM + [_P]),
    "conv_bwd_dw_ex": (_I, [_P, _P, _P, _P, ctypes.c_size_t] + _GEOM + [_I, _P]),
    "conv_bwd_dw_workspace_size": (_I, _GEOM + [_I, ctypes.POINTER(ctypes.c_size_t)]),
    "conv_bwd_dw_noalloc": (_I, [_P, _P, _P] + _GEOM + [_P]),
    "conv_path_name": (ctypes.c_char_p, [_I]),
    "conv_last_error": (ctypes.c_char_p, []),
    "conv_arm_launch_events": (_I, [_P, _P]),
}

_lib = None


def load():
    """Returns the loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: the HIP library has not been built "
            "(run convolution_implicit_gemm_conv2d_amd.build.build())"
        )
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
