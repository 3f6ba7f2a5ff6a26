"""Host-side checks of the C ABI: the library loads, exports every function
include/convmi.h declares, and rejects every invalid argument on the host
before anything is launched.  No call here reaches a GPU: each one fails
validation first (or is a pure host query)."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import convolution_implicit_gemm_conv2d_amd as cm
import oracle
from convolution_implicit_gemm_conv2d_amd import _lib, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convmi.h")

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(conv\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for name in names:
        assert hasattr(lib, name), name


def test_library_does_not_link_the_oracle():
    data = open(_lib.LIB_PATH, "rb").read()
    assert b"oracle_" not in data


def test_out_size_matches_oracle():
    for n, k, s, p, d in itertools.product(range(1, 9), range(1, 5), range(1, 4), range(0, 3), range(1, 3)):
        ref = oracle.out_size(n, k, s, p, d)
        if ref is None:
            with pytest.raises(cm.ConvError) as e:
                cm.conv_out_size(n, k, s, p, d)
            assert e.value.status == cm.CONV_ERR_INVALID_ARG
        else:
            assert cm.conv_out_size(n, k, s, p, d) == ref


def test_out_size_rejects_null_and_bad_values():
    lib = _lib.load()
    assert lib.conv_out_size(5, 3, 1, 1, 1, None) == cm.CONV_ERR_INVALID_ARG
    for args in [(0, 3, 1, 1, 1), (5, 0, 1, 1, 1), (5, 3, 0, 1, 1), (5, 3, 1, -1, 1), (5, 3, 1, 1, 0)]:
        with pytest.raises(cm.ConvError):
            cm.conv_out_size(*args)


GOOD = dict(N=2, C=4, H=8, W=8, C_out=6, KH=3, KW=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=2,
            layout=1, dtype=1)


def call_fwd(x=FAKE, w=FAKE, b=None, y=FAKE, path=0, **kw):
    a = dict(GOOD, **kw)
    return _lib.load().conv_fwd_ex(x, w, b, y, a["N"], a["C"], a["H"], a["W"], a["C_out"], a["KH"],
                                   a["KW"], a["sh"], a["sw"], a["ph"], a["pw"], a["dh"], a["dw"],
                                   a["G"], a["layout"], a["dtype"], path, None)


def call_dx(dy=FAKE, w=FAKE, dx=FAKE, path=0, **kw):
    a = dict(GOOD, **kw)
    return _lib.load().conv_bwd_dx_ex(dy, w, dx, a["N"], a["C"], a["H"], a["W"], a["C_out"],
                                      a["KH"], a["KW"], a["sh"], a["sw"], a["ph"], a["pw"],
                                      a["dh"], a["dw"], a["G"], a["layout"], a["dtype"], path, None)


INVALID = [
    dict(layout=2), dict(layout=-1), dict(dtype=2), dict(N=0), dict(C=0), dict(H=0), dict(W=0),
    dict(C_out=0), dict(KH=0), dict(KW=0), dict(sh=0), dict(sw=0), dict(dh=0), dict(dw=0),
    dict(G=0), dict(ph=-1), dict(pw=-1), dict(G=3), dict(C=5), dict(C_out=5),
    dict(KH=11), dict(KW=11), dict(KH=4, dh=4), dict(H=1, KH=3, ph=0),
]


@pytest.mark.parametrize("bad", INVALID)
@pytest.mark.parametrize("fn", [call_fwd, call_dx])
def test_invalid_arguments_are_rejected_on_host(fn, bad):
    assert fn(**bad) == cm.CONV_ERR_INVALID_ARG
    assert cm.conv_last_error() != ""


def test_null_pointers_are_rejected():
    assert call_fwd(x=None) == cm.CONV_ERR_INVALID_ARG
    assert call_fwd(w=None) == cm.CONV_ERR_INVALID_ARG
    assert call_fwd(y=None) == cm.CONV_ERR_INVALID_ARG
    assert "NULL" in cm.conv_last_error()
    assert call_dx(dy=None) == cm.CONV_ERR_INVALID_ARG
    assert call_dx(dx=None) == cm.CONV_ERR_INVALID_ARG


@pytest.mark.parametrize("big", [
    dict(N=1, C=1 << 16, H=1 << 8, W=1 << 8, C_out=2, G=1),         # x image 2^32 elements
    dict(N=1, C=2, H=1 << 16, W=1 << 16, C_out=2, G=1, KH=1, KW=1, ph=0, pw=0),
    dict(C=1 << 16, C_out=1 << 16, G=1, H=4, W=4, KH=1, KW=1, ph=0, pw=0),  # weight 2^32
])
@pytest.mark.parametrize("fn", [call_fwd, call_dx])
def test_int32_extent_overflow_is_reported(fn, big):
    assert fn(**big) == cm.CONV_ERR_OVERFLOW


def test_unknown_and_mismatched_paths():
    assert call_fwd(path=99) == cm.CONV_ERR_INVALID_ARG
    assert call_fwd(path=cm.PATHS["dx_gather"]) == cm.CONV_ERR_INVALID_ARG
    assert call_dx(path=cm.PATHS["direct"]) == cm.CONV_ERR_INVALID_ARG


def test_forced_fast_paths_decline_foreign_geometry():
    # fp32 NCHW grouped 3x3: no specialised forward path takes it.
    for p in ("igemm", "igemm_band", "pointwise", "depthwise"):
        assert call_fwd(path=cm.PATHS[p], layout=0, dtype=0) == cm.CONV_ERR_UNSUPPORTED
    assert call_dx(path=cm.PATHS["dx_igemm"], layout=0, dtype=0) == cm.CONV_ERR_UNSUPPORTED
    assert call_dx(path=cm.PATHS["dx_band"], layout=0, dtype=0) == cm.CONV_ERR_UNSUPPORTED


def test_dx_band_is_forced_only():
    # The automatic input-gradient path never picks the all-phase band kernel.
    sel = lambda *a: cm.conv_path_name(cm.conv_select_path(1, *a, cm.CONV_NHWC, cm.CONV_BF16))
    for geo in [(32, 128, 56, 56, 256, 3, 3, 2, 2, 1, 1, 1, 1, 1),
                (32, 128, 56, 56, 256, 4, 4, 2, 2, 1, 1, 1, 1, 1),
                (32, 64, 56, 56, 128, 3, 3, 2, 2, 1, 1, 1, 1, 1)]:
        assert sel(*geo) == "dx_igemm", geo


def test_path_names():
    for name, v in cm.PATHS.items():
        assert cm.conv_path_name(v) == name
    assert cm.conv_path_name(1234) == "unknown"


def workload_path(name):
    s = inputs.WORKLOADS[name]
    return cm.conv_select_path(s["kind"] == "dx", s["N"], s["C"], s["H"], s["W"], s["C_out"],
                               s["KH"], s["KW"], s["stride"], s["stride"], s["pad"], s["pad"],
                               s["dil"], s["dil"], s["groups"],
                               cm.CONV_NHWC if s["layout"] == "NHWC" else cm.CONV_NCHW,
                               cm.CONV_BF16 if s["dtype"] == "bf16" else cm.CONV_F32)


EXPECTED_PATH = {
    "tiny_3x3_fp32_nchw": "direct",
    "pointwise_1x1_c256_k64_56x56_n32_bf16_nhwc": "pointwise",
    "dense_3x3_c64_k64_56x56_n32_bf16_nhwc": "igemm_band",
    "depthwise_3x3_d2_c256_56x56_n32_bf16_nhwc": "depthwise",
    "dx_3x3_s2_c128_k256_56x56_n32_bf16_nhwc": "dx_igemm",
}


@pytest.mark.parametrize("name", sorted(EXPECTED_PATH))
def test_workloads_select_their_specialised_path(name):
    assert cm.conv_path_name(workload_path(name)) == EXPECTED_PATH[name]


@pytest.mark.parametrize("name,path", [
    ("grouped_3x3_g32_c128_56x56_n32_bf16_nhwc", "depthwise"),
    ("grouped_3x3_g32_c256_28x28_n32_bf16_nhwc", "depthwise"),
    ("grouped_3x3_g8_c192_56x56_n32_bf16_nhwc", "igemm"),
    ("depthwise_mult2_3x3_c64_k128_56x56_n32_bf16_nhwc", "depthwise"),
])
def test_grouped_workloads_take_the_small_group_kernel(name, path):
    s = inputs.NEXT_WORKLOADS[name]
    got = cm.conv_select_path(0, s["N"], s["C"], s["H"], s["W"], s["C_out"], s["KH"], s["KW"],
                              s["stride"], s["stride"], s["pad"], s["pad"], s["dil"], s["dil"],
                              s["groups"], cm.CONV_NHWC, cm.CONV_BF16)
    assert cm.conv_path_name(got) == path


def test_small_groups_outside_the_vector_are_declined():
    # C/G = 8 in fp32 (a 4-channel vector), C_out/G below C/G and
    # multipliers other than 2, 4 and 8 are not taken by the small-group
    # kernels; multipliers 2, 4 and 8 of C/G = 1, 2, 4 are.
    def sel(C, CO, G, dtype):
        return cm.conv_path_name(cm.conv_select_path(0, 2, C, 8, 8, CO, 3, 3, 1, 1, 1, 1, 1, 1, G,
                                                     cm.CONV_NHWC, dtype))
    assert sel(64, 64, 8, cm.CONV_F32) != "depthwise"
    assert sel(64, 32, 16, cm.CONV_BF16) != "depthwise"     # C/G 4, C_out/G 2
    assert sel(64, 64 * 16, 64, cm.CONV_BF16) != "depthwise"  # multiplier 16
    assert sel(64, 192, 64, cm.CONV_BF16) != "depthwise"    # multiplier 3
    assert sel(64, 64, 16, cm.CONV_F32) == "depthwise"
    assert sel(64, 64, 8, cm.CONV_BF16) == "depthwise"
    assert sel(64, 128, 16, cm.CONV_BF16) == "depthwise"    # C/G 4, multiplier 2
    assert sel(3, 24, 3, cm.CONV_BF16) == "depthwise"       # RGB input, multiplier 8
    assert sel(12, 48, 12, cm.CONV_F32) == "depthwise"      # fp32, multiplier 4


def test_group_widths_below_32_take_a_specialised_kernel():
    # NHWC bf16 group widths below 32 of 1, 2, 4 and multiples of 8: those on the implicit
    # GEMM, 1, 2, 4, 8 (and their multipliers) on the small-group kernels;
    # the input gradient of groups with C_out/G = C/G <= 8 on the
    # small-group gather, multiples of 8 on the per-phase implicit GEMM.
    def sel(bwd, C, CO, G):
        return cm.conv_path_name(cm.conv_select_path(bwd, 2, C, 14, 14, CO, 3, 3, 1, 1, 1, 1, 1, 1, G,
                                                     cm.CONV_NHWC, cm.CONV_BF16))
    for cg in (1, 2, 4, 8, 16, 24):
        G = 96 // cg
        assert sel(0, 96, 96, G) in ("depthwise", "igemm", "igemm_band"), cg
        assert sel(1, 96, 96, G) in ("dx_depthwise", "dx_igemm"), cg
    assert sel(1, 96, 96, 96) == "dx_depthwise"
    assert sel(1, 96, 96, 24) == "dx_depthwise"



def test_binding_checks_shapes_before_touching_memory():
    import torch

    w = torch.zeros(8, 3, 3, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="output gradient must have shape"):
        cm.conv2d_input_grad(torch.zeros(1, 5, 5, 8, dtype=torch.bfloat16), w, (1, 8, 8, 4),
                             padding=1)
    with pytest.raises(ValueError, match="input channels per group"):
        cm.conv2d(torch.zeros(1, 8, 8, 6, dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="unsupported dtype"):
        cm.conv2d(torch.zeros(1, 8, 8, 4, dtype=torch.float16), w.half())


# ------------------------------------------------- conv1d / conv_transpose2d --

def test_transpose_out_size_matches_oracle():
    for n, k, s, p, d, op in itertools.product(range(1, 6), range(1, 5), range(1, 4), range(0, 3),
                                               range(1, 3), range(0, 3)):
        ref = oracle.conv_transpose_size(n, k, s, p, d, op)
        if ref is None:
            with pytest.raises(cm.ConvError) as e:
                cm.conv_transpose_out_size(n, k, s, p, d, op)
            assert e.value.status == cm.CONV_ERR_INVALID_ARG
        else:
            assert cm.conv_transpose_out_size(n, k, s, p, d, op) == ref


def conv1d_call(**kw):
    a = dict(x=FAKE, w=FAKE, bias=None, y=FAKE, N=2, C=8, L=16, C_out=8, K=3, stride=1, pad=1,
             dil=1, groups=1, layout=cm.CONV_NLC, dtype=cm.CONV_BF16)
    a.update(kw)
    return _lib.load().conv1d_fwd(a["x"], a["w"], a["bias"], a["y"], a["N"], a["C"], a["L"],
                                  a["C_out"], a["K"], a["stride"], a["pad"], a["dil"], a["groups"],
                                  a["layout"], a["dtype"], None)


@pytest.mark.parametrize("bad", [
    dict(x=None), dict(w=None), dict(y=None), dict(N=0), dict(L=0), dict(K=0), dict(stride=0),
    dict(dil=0), dict(pad=-1), dict(groups=3), dict(K=40), dict(layout=2), dict(dtype=5),
])
def test_conv1d_rejects_invalid_arguments(bad):
    assert conv1d_call(**bad) == cm.CONV_ERR_INVALID_ARG
    assert "conv1d_fwd" in cm.conv_last_error()


def transpose_call(**kw):
    a = dict(x=FAKE, w=FAKE, bias=None, y=FAKE, N=2, C_in=8, H=5, W=5, C_out=8, KH=3, KW=3, sh=2,
             sw=2, ph=1, pw=1, oph=1, opw=1, dh=1, dw=1, groups=1, layout=cm.CONV_NHWC,
             dtype=cm.CONV_BF16)
    a.update(kw)
    return _lib.load().conv_transpose2d(
        a["x"], a["w"], a["bias"], a["y"], a["N"], a["C_in"], a["H"], a["W"], a["C_out"], a["KH"],
        a["KW"], a["sh"], a["sw"], a["ph"], a["pw"], a["oph"], a["opw"], a["dh"], a["dw"],
        a["groups"], a["layout"], a["dtype"], None)


@pytest.mark.parametrize("bad", [
    dict(x=None), dict(w=None), dict(y=None), dict(N=0), dict(C_in=0), dict(KH=0), dict(sh=0),
    dict(dw=0), dict(ph=-1), dict(oph=2), dict(opw=-1), dict(groups=3), dict(H=1, KH=1, ph=1, oph=0),
    dict(layout=7), dict(dtype=2),
])
def test_conv_transpose2d_rejects_invalid_arguments(bad):
    assert transpose_call(**bad) == cm.CONV_ERR_INVALID_ARG
    assert "conv_transpose2d" in cm.conv_last_error()


# ---------------------------------------------------------- weight gradient --

def dw_call(ws_bytes, ws=FAKE, path=0, **kw):
    a = dict(N=2, C=8, H=6, W=6, C_out=8, KH=3, KW=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1,
             groups=1, layout=cm.CONV_NHWC, dtype=cm.CONV_BF16)
    a.update(kw)
    geom = [a[k] for k in ("N", "C", "H", "W", "C_out", "KH", "KW", "sh", "sw", "ph", "pw", "dh",
                           "dw", "groups", "layout", "dtype")]
    return _lib.load().conv_bwd_dw_ex(FAKE, FAKE, FAKE, ws, ws_bytes, *geom, path, None)


def test_dw_workspace_size_is_reported_and_enforced():
    need = cm.conv_bwd_dw_workspace_size(2, 8, 6, 6, 8, 3, 3, 1, 1, 1, 1, 1, 1, 1, cm.CONV_NHWC,
                                         cm.CONV_BF16, 0)
    assert need >= 4 * 8 * 8 * 9  # at least one fp32 partial per weight element
    assert dw_call(need - 1) == cm.CONV_ERR_INVALID_ARG
    assert "workspace" in cm.conv_last_error()
    assert dw_call(need, ws=None) == cm.CONV_ERR_INVALID_ARG
    assert dw_call(need, ws=FAKE + 4) == cm.CONV_ERR_INVALID_ARG  # misaligned
    assert dw_call(need, path=cm.PATHS["igemm"]) == cm.CONV_ERR_INVALID_ARG
    assert dw_call(need, groups=3) == cm.CONV_ERR_INVALID_ARG
    with pytest.raises(cm.ConvError):
        cm.conv_bwd_dw_workspace_size(2, 8, 6, 6, 8, 3, 3, 1, 1, 1, 1, 1, 1, 1, cm.CONV_NHWC,
                                      cm.CONV_BF16, cm.PATHS["dx_igemm"])


def test_random_sweep_reaches_every_specialised_path():
    # The seeded sweep of test_gpu_random goes through automatic selection;
    # it must reach each kernel family (and the generic fallbacks).  The band
    # kernel is chosen only for long bands (at least 5 output rows per CU),
    # which these small shapes never give; its own tests force it.
    import random_cases
    seen = set()
    for c in random_cases.cases():
        seen.add(cm.conv_path_name(cm.conv_select_path(
            c["kind"] == "dx", c["N"], c["C"], c["H"], c["W"], c["CO"], c["KH"], c["KW"], *c["stride"],
            *c["pad"], *c["dil"], c["groups"], 1 if c["layout"] == "NHWC" else 0,
            1 if c["dtype"] == "bf16" else 0)))
    assert {"direct", "pointwise", "igemm", "depthwise", "dx_igemm", "dx_gather"} <= seen, seen


@pytest.mark.parametrize("H,s,C,path", [
    (56, 1, 64, "igemm_band"),   # 7 output rows per band: one group each
    (28, 1, 64, "igemm_band"),   # 3.5 rows per band
    (56, 2, 64, "igemm_band"),   # stride 2: 28 output rows per image
    (112, 1, 64, "igemm"),       # 28 rows per band: several groups per band
    (56, 1, 32, "igemm"),        # 32-channel groups
])
def test_band_kernel_only_for_one_group_bands_of_64_channels(H, s, C, path):
    got = cm.conv_path_name(cm.conv_select_path(0, 32, C, H, H, C, 3, 3, s, s, 1, 1, 1, 1, 1,
                                                cm.CONV_NHWC, cm.CONV_BF16))
    assert got == path


def test_dx_plan_with_no_tap_in_any_phase():
    # H = W = 1, a 1x1 kernel, stride 2, padding 1: the one stride phase that
    # holds a pixel is reached by no tap, so dx is all zeros.  The planner's
    # tile-height rule compares tap counts against the fewest taps of any
    # phase; with no tap anywhere it must not apply (it once doubled an
    # "infinity" sentinel in int, which is undefined behaviour).
    p = cm.conv_select_path(1, 2, 8, 1, 1, 8, 1, 1, 2, 2, 1, 1, 1, 1, 1, cm.CONV_NHWC, cm.CONV_BF16)
    assert cm.conv_path_name(p) == "dx_igemm"


def test_noalloc_weight_gradient_rejects_geometries_beyond_its_scratch():
    # 2048 -> 2048 channels, 3x3: the fp32 partials alone exceed the 16 MiB
    # array, so the call fails on the host before touching the device.
    geom = (1, 2048, 8, 8, 2048, 3, 3, 1, 1, 1, 1, 1, 1, 1, cm.CONV_NHWC, cm.CONV_BF16)
    need = cm.conv_bwd_dw_workspace_size(*geom, cm.PATHS["auto"])
    assert need > 16 << 20
    with pytest.raises(cm.ConvError) as e:
        cm.conv_bwd_dw_noalloc(0x1000, 0x2000, 0x3000, *geom, stream=0)
    assert e.value.status == cm.CONV_ERR_UNSUPPORTED
    assert "scratch" in e.value.message
    with pytest.raises(cm.ConvError) as e:
        cm.conv_bwd_dw_noalloc(None, 0x2000, 0x3000, *geom, stream=0)
    assert e.value.status == cm.CONV_ERR_INVALID_ARG
