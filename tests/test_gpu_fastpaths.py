"""GPU parity of the specialised kernels against the fp64 oracle.

Every case forces its path through conv_fwd_ex / conv_bwd_dx_ex, so a path
that declined the geometry fails the test (CONV_ERR_UNSUPPORTED) instead of
silently falling back.  Shapes cover several tiles plus ragged tails in
pixels and channels, strides, dilations, bias and no bias.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_conv2d_amd as cm
import oracle
from helpers import (TOL, dx_error, f64, fwd_error, gpu_dx, gpu_fwd, out_shape, random_case,
                     random_dy)

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def fwd_case(path, N, C, H, W, CO, KH, KW, s, p, d, G, dtype=BF16, bias=True, seed=0):
    print(f"{path}: N={N} C={C} H={H} W={W} CO={CO} K={KH}x{KW} s={s} p={p} d={d} G={G} "
          f"{dtype} bias={bias}", flush=True)
    x, w, b = random_case(seed, N, C, H, W, CO, KH, KW, G, "NHWC", dtype, bias=bias)
    geo = dict(stride=s, padding=p, dilation=d, groups=G, layout="NHWC")
    y = gpu_fwd(x, w, b, geo, path=path)
    err = fwd_error(x, w, b, y, geo)
    assert err <= TOL[dtype], err
    return x, w, b, y, geo


# ------------------------------------------------------------- pointwise --

@pytest.mark.parametrize("N,C,H,W,CO,s", [
    (2, 256, 7, 9, 64, 1),     # 126 pixels: one partial block
    (3, 32, 11, 13, 4, 1),     # smallest channel counts
    (1, 96, 17, 15, 100, 1),   # two channel tiles, ragged
    (4, 256, 6, 5, 128, 1),    # largest C the path takes
    (2, 64, 15, 14, 36, 2),    # strided 1x1
    (1, 128, 9, 10, 68, 3),
    # Unit stride, C_out a multiple of 8: whole-line stores.
    (1, 96, 13, 11, 24, 1),    # odd C/32: pixel rows at an LDS pitch of 13 units
    (2, 160, 9, 7, 72, 1),     # second channel block holds 8 channels
    (1, 224, 5, 13, 8, 1),     # C_out of one store unit
    (3, 64, 1, 1, 64, 1),      # three pixels: one partial tile, every other wave idle
    (10, 32, 128, 128, 16, 1), # 10240 tiles: each wave's ring wraps twice
])
@pytest.mark.parametrize("bias", [True, False])
def test_pointwise(N, C, H, W, CO, s, bias):
    fwd_case("pointwise", N, C, H, W, CO, 1, 1, s, 0, 1, 1, bias=bias)


@pytest.mark.parametrize("N,C,H,W,CO,s,p", [
    (2, 64, 7, 9, 36, 1, (1, 1)),      # a one-pixel frame of bias-only outputs
    (1, 128, 10, 11, 68, 2, (2, 0)),   # padding on one axis, strided
    (3, 32, 5, 6, 4, (1, 3), (3, 2)),  # padding wider than a stride step
    (2, 256, 6, 5, 64, 3, (1, 1)),
])
@pytest.mark.parametrize("bias", [True, False])
def test_pointwise_padded(N, C, H, W, CO, s, p, bias):
    fwd_case("pointwise", N, C, H, W, CO, 1, 1, s, p, 1, 1, bias=bias)


def test_pointwise_padded_border_is_bias():
    # Padded positions see only zeros, so their outputs are the bias rounded
    # to bf16, exactly.
    x, w, b = random_case(2, 2, 64, 5, 6, 32, 1, 1, 1, "NHWC", BF16, bias=True)
    geo = dict(stride=1, padding=2, dilation=1, groups=1, layout="NHWC")
    y = gpu_fwd(x, w, b, geo, path="pointwise").float().cpu()
    ref = b.float().cpu()
    for oh, ow in [(0, 0), (1, 4), (8, 9), (4, 0), (0, 6)]:
        assert torch.equal(y[:, oh, ow, :], ref.expand(2, 32)), (oh, ow)


def test_pointwise_impulse_bit_exact():
    x, w, _ = random_case(1, 2, 64, 5, 6, 32, 1, 1, 1, "NHWC", BF16, bias=False)
    x = torch.zeros_like(x)
    x[1, 3, 2, 17] = 1
    geo = dict(stride=1, padding=0, dilation=1, groups=1, layout="NHWC")
    y = gpu_fwd(x, w, None, geo, path="pointwise")
    ref, _ = oracle.conv2d_forward(x, w, None, **geo)
    np.testing.assert_array_equal(f64(y), ref)


# ------------------------------------------------------------- depthwise --

@pytest.mark.parametrize("dtype", [BF16, torch.float32])
@pytest.mark.parametrize("N,C,H,W,K,s,p,d", [
    (2, 256, 13, 11, 3, 1, 2, 2),   # rows kernel, dilation 2, ragged rows
    (1, 64, 17, 9, 3, 1, 1, 1),     # rows kernel, dilation 1
    (1, 32, 12, 12, 5, 1, 2, 1),    # rows kernel 5x5
    (2, 40, 10, 13, 3, 2, 1, 1),    # generic: stride 2
    (1, 24, 11, 9, 2, 1, 1, 3),     # generic: even kernel, dilation 3
    (1, 16, 3, 4, 3, 1, 0, 1),      # one output row
])
def test_depthwise(dtype, N, C, H, W, K, s, p, d):
    fwd_case("depthwise", N, C, H, W, C, K, K, s, p, d, C, dtype=dtype, bias=True)


def test_depthwise_no_bias_and_impulse():
    x, w, _ = random_case(2, 1, 32, 9, 9, 32, 3, 3, 32, "NHWC", BF16, bias=False)
    x = torch.zeros_like(x)
    x[0, 4, 5, 9] = 1
    geo = dict(stride=1, padding=2, dilation=2, groups=32, layout="NHWC")
    y = gpu_fwd(x, w, None, geo, path="depthwise")
    ref, _ = oracle.conv2d_forward(x, w, None, **geo)
    np.testing.assert_array_equal(f64(y), ref)


# ------------------------------------- small groups: C/G = C_out/G = 2, 4, 8 --

@pytest.mark.parametrize("dtype,CG", [(BF16, 2), (BF16, 4), (BF16, 8),
                                      (torch.float32, 2), (torch.float32, 4)])
@pytest.mark.parametrize("N,C,H,W,K,s,p,d", [
    (2, 64, 13, 11, 3, 1, 1, 1),    # streaming walk, ragged rows and columns
    (2, 128, 9, 56, 3, 1, 1, 1),    # several workgroups across a row
    (1, 32, 9, 17, 3, 1, 0, 1),     # no padding
    (2, 48, 10, 13, 3, 2, 1, 1),    # generic: stride 2
    (1, 32, 11, 9, 3, 1, 2, 2),     # generic: dilation 2
    (1, 16, 8, 8, 5, 1, 2, 1),      # generic: 5x5
])
def test_small_groups(dtype, CG, N, C, H, W, K, s, p, d):
    fwd_case("depthwise", N, C, H, W, C, K, K, s, p, d, C // CG, dtype=dtype, bias=True)


@pytest.mark.parametrize("CG", [2, 4, 8])
def test_small_groups_no_bias_and_impulse(CG):
    # An impulse at input channel c reaches exactly the outputs of c's group,
    # each through its own weight for c: exact in bf16.
    C = 32
    x, w, _ = random_case(3, 1, C, 9, 9, C, 3, 3, C // CG, "NHWC", BF16, bias=False)
    x = torch.zeros_like(x)
    x[0, 4, 5, 13] = 1
    geo = dict(stride=1, padding=1, dilation=1, groups=C // CG, layout="NHWC")
    y = gpu_fwd(x, w, None, geo, path="depthwise")
    ref, _ = oracle.conv2d_forward(x, w, None, **geo)
    np.testing.assert_array_equal(f64(y), ref)
    fwd_case("depthwise", 2, 64, 7, 10, 64, 3, 3, 1, 1, 1, 64 // CG, bias=False)


# Small groups of 4 and 8 channels with C a multiple of 64 (bf16, 3x3) run on
# the 4x4x4 matrix instruction; these cases cover its geometry handling.
@pytest.mark.parametrize("CG", [4, 8])
@pytest.mark.parametrize("N,C,H,W,s,p,d", [
    (1, 64, 10, 9, 2, 1, 1),        # stride 2
    (2, 192, 7, 10, 1, 2, 2),       # dilation 2, three 64-channel blocks
    (1, 128, 6, 5, 1, 0, 1),        # no padding: 3 output columns (one ragged segment)
    (3, 64, 17, 21, (2, 1), (1, 0), (1, 2)),  # per-axis stride, pad, dilation
    (2, 64, 23, 19, 2, 2, 2),       # stride = dilation: staged rows reused
    (1, 64, 37, 12, 1, 1, 1),       # ten row segments, the last one row long
    (1, 512, 9, 13, 1, 1, 1),       # eight 64-channel blocks
    (2, 64, 20, 40, 3, 2, 2),       # 7*3 + 2*2 + 1 = 26 staged columns: the vector kernel
])
@pytest.mark.parametrize("bias", [True, False])
def test_small_groups_matrix_core(CG, N, C, H, W, s, p, d, bias):
    fwd_case("depthwise", N, C, H, W, C, 3, 3, s, p, d, C // CG, bias=bias)


@pytest.mark.parametrize("CG", [4, 8])
def test_small_groups_matrix_core_impulse(CG):
    C = 64
    x, w, _ = random_case(4, 1, C, 9, 10, C, 3, 3, C // CG, "NHWC", BF16, bias=False)
    x = torch.zeros_like(x)
    x[0, 4, 6, 37] = 1
    geo = dict(stride=1, padding=1, dilation=1, groups=C // CG, layout="NHWC")
    y = gpu_fwd(x, w, None, geo, path="depthwise")
    ref, _ = oracle.conv2d_forward(x, w, None, **geo)
    np.testing.assert_array_equal(f64(y), ref)


# ----------------------------------------------------------------- igemm --

@pytest.mark.parametrize("N,C,H,W,CO,K,s,p,d,G", [
    (2, 64, 14, 14, 64, (3, 3), 1, 1, 1, 1),      # the dense 3x3 shape, small batch
    (3, 32, 9, 11, 20, (3, 3), 1, 1, 1, 1),       # partial channel tile, ragged pixels
    (1, 96, 10, 9, 72, (3, 3), 2, 1, 1, 1),       # three k-steps per tap, stride 2
    (2, 128, 7, 8, 128, (3, 3), 1, 2, 2, 1),      # four k-steps per tap, dilation 2
    (1, 64, 12, 10, 36, (1, 3), (2, 1), (0, 1), (1, 2), 1),
    (2, 128, 8, 8, 64, (3, 3), 1, 1, 1, 2),       # two groups of 64 -> 32
    (1, 32, 6, 6, 8, (5, 5), 1, 2, 1, 1),         # 25 taps (odd tap count)
    (2, 512, 5, 6, 68, (1, 1), 1, 0, 1, 1),       # 1x1 with C beyond the pointwise path
    (1, 32, 4, 4, 4, (4, 4), 1, 0, 1, 1),         # single output pixel
    (1, 16, 9, 7, 12, (3, 3), 1, 1, 1, 1),        # one 16-channel step per tap
    (2, 48, 8, 8, 32, (3, 3), 1, 1, 1, 1),        # three steps per tap
    (1, 96, 7, 9, 24, (2, 2), 1, 0, 1, 3),        # three groups of 32 -> 8
    (1, 64, 9, 100, 136, (3, 3), 1, 1, 1, 1),     # two column tiles, three channel tiles
    (2, 64, 20, 56, 64, (3, 3), 1, 1, 1, 1),      # 8-row regions: seven pixel tiles per wave
    (1, 32, 1, 70, 40, (1, 3), 1, (0, 1), (1, 3), 1),   # compiled 1x3 taps, 32-channel chunks, 40 outputs
    (2, 96, 6, 7, 96, (1, 3), 1, (0, 1), 1, 1),   # compiled 1x3, second channel tile of 32 (four units stored)
    (3, 64, 5, 5, 48, (3, 3), 1, 1, 1, 4),        # four groups of 16 -> 12: regions not a multiple of 8
])
@pytest.mark.parametrize("bias", [True, False])
def test_igemm(N, C, H, W, CO, K, s, p, d, G, bias):
    fwd_case("igemm", N, C, H, W, CO, K[0], K[1], s, p, d, G, bias=bias)


def test_igemm_impulse_bit_exact():
    x, w, _ = random_case(4, 2, 64, 9, 8, 64, 3, 3, 1, "NHWC", BF16, bias=False)
    x = torch.zeros_like(x)
    x[1, 4, 5, 37] = 1
    geo = dict(stride=1, padding=1, dilation=1, groups=1, layout="NHWC")
    y = gpu_fwd(x, w, None, geo, path="igemm")
    ref, _ = oracle.conv2d_forward(x, w, None, **geo)
    np.testing.assert_array_equal(f64(y), ref)


# ------------------------------------------------------------ igemm_band --

@pytest.mark.parametrize("N,C,H,W,CO,s,p,d,G", [
    (2, 64, 14, 14, 64, 1, 1, 1, 1),      # the dense 3x3 shape, small batch
    (3, 64, 17, 56, 64, 1, 1, 1, 1),      # 56-wide rows: seven pixel tiles per group
    (1, 32, 9, 11, 20, 1, 1, 1, 1),       # partial channel tile, ragged pixels
    (2, 16, 10, 9, 12, 1, 1, 1, 1),       # one 16-channel step per tap
    (1, 64, 12, 100, 136, 1, 1, 1, 1),    # two column tiles, three channel tiles
    (2, 32, 15, 13, 40, 2, 1, 1, 1),      # stride 2
    (1, 64, 11, 12, 64, 1, 2, 2, 1),      # dilation 2
    (2, 128, 8, 8, 64, 1, 1, 1, 2),       # two groups of 64 -> 32
    (1, 48, 9, 9, 24, 1, 0, 1, 3),        # three groups of 16 -> 8, no padding
    (5, 32, 3, 4, 8, 1, 1, 1, 1),         # tiny images: bands cross images
    (1, 64, 3, 5, 64, 1, 0, 1, 1),        # a single output row of three pixels
    (1, 64, 24, 20, 64, 1, 1, 1, 1),      # 24 one-row bands: each XCD takes three consecutive bands
    (2, 64, 20, 9, 64, 1, 1, 1, 1),       # 40 bands over two images, five per XCD
])
@pytest.mark.parametrize("bias", [True, False])
def test_igemm_band(N, C, H, W, CO, s, p, d, G, bias):
    fwd_case("igemm_band", N, C, H, W, CO, 3, 3, s, p, d, G, bias=bias)


def test_igemm_band_impulse_bit_exact():
    x, w, _ = random_case(4, 2, 64, 9, 8, 64, 3, 3, 1, "NHWC", BF16, bias=False)
    x = torch.zeros_like(x)
    x[1, 4, 5, 37] = 1
    x[0, 0, 0, 3] = 1
    geo = dict(stride=1, padding=1, dilation=1, groups=1, layout="NHWC")
    y = gpu_fwd(x, w, None, geo, path="igemm_band")
    ref, _ = oracle.conv2d_forward(x, w, None, **geo)
    np.testing.assert_array_equal(f64(y), ref)


# -------------------------------------------------------------- dx_igemm --

def dx_case(N, C, H, W, CO, K, s, p, d, G, seed=0):
    print(f"dx_igemm: N={N} C={C} H={H} W={W} CO={CO} K={K} s={s} p={p} d={d} G={G}", flush=True)
    x, w, _ = random_case(seed, N, C, H, W, CO, K[0], K[1], G, "NHWC", BF16, bias=False)
    geo = dict(stride=s, padding=p, dilation=d, groups=G, layout="NHWC")
    dy = random_dy(seed + 1, out_shape(x.shape, w.shape, geo), BF16)
    dx = gpu_dx(dy, w, tuple(x.shape), geo, path="dx_igemm")
    err = dx_error(dy, w, tuple(x.shape), dx, geo)
    assert err <= TOL[BF16], err
    return dy, w, dx, geo


@pytest.mark.parametrize("N,C,H,W,CO,K,s,p,d,G", [
    (2, 128, 14, 14, 256, (3, 3), 2, 1, 1, 1),      # the stride-2 shape, small batch
    (1, 64, 9, 11, 64, (3, 3), 1, 1, 1, 1),         # unit stride: one phase, 9 taps
    (2, 32, 6, 6, 16, (3, 3), 2, 0, 1, 1),          # unread last row and column -> 0
    (1, 136, 10, 9, 72, (3, 3), 2, 1, 1, 1),        # ragged channel tiles (136 ci, 72 co)
    (1, 48, 13, 12, 40, (5, 3), (3, 2), (2, 1), (1, 2), 1),  # 6 phases, uneven taps
    (2, 64, 8, 8, 64, (3, 3), 2, 1, 1, 2),          # two groups
    (1, 256, 7, 7, 128, (1, 1), 1, 0, 1, 1),        # 1x1: dx = dy . W
    (1, 16, 5, 6, 8, (2, 2), 2, 0, 1, 1),           # every phase has exactly one tap
    (1, 24, 7, 5, 16, (3, 3), 3, 0, 1, 1),          # phases no tap reaches (written as 0)
    (3, 64, 40, 40, 96, (3, 3), 2, 1, 1, 1),        # several pixel tiles per phase, ragged tail
    (1, 64, 9, 300, 32, (3, 3), 2, 1, 1, 1),        # long phase rows (150 columns)
    (2, 32, 12, 10, 24, (3, 3), 1, 4, 4, 1),        # stride 1, dilation 4: taps 4 rows apart
])
def test_dx_igemm(N, C, H, W, CO, K, s, p, d, G):
    dx_case(N, C, H, W, CO, K, s, p, d, G)


def test_dx_igemm_unreached_elements_are_zero():
    dy, w, dx, geo = dx_case(1, 24, 7, 5, 16, (3, 3), 3, 0, 1, 1, seed=3)
    ref, norm = oracle.conv2d_input_grad(dy, w, tuple(dx.shape), **geo)
    unreached = norm == 0
    assert unreached.any()
    assert np.all(f64(dx)[unreached] == 0)


def test_dx_igemm_impulse_bit_exact():
    x, w, _ = random_case(6, 1, 64, 10, 10, 64, 3, 3, 1, "NHWC", BF16, bias=False)
    geo = dict(stride=2, padding=1, dilation=1, groups=1, layout="NHWC")
    dy = torch.zeros(out_shape(x.shape, w.shape, geo), dtype=BF16)
    dy[0, 2, 3, 17] = 1
    dx = gpu_dx(dy, w, tuple(x.shape), geo, path="dx_igemm")
    ref, _ = oracle.conv2d_input_grad(dy, w, tuple(x.shape), **geo)
    np.testing.assert_array_equal(f64(dx), ref)


# --------------------------------------------------------------- dx_band --

def dx_band_case(N, C, H, W, CO, K, p, G=1, seed=0):
    print(f"dx_band: N={N} C={C} H={H} W={W} CO={CO} K={K} p={p} G={G}", flush=True)
    x, w, _ = random_case(seed, N, C, H, W, CO, K, K, G, "NHWC", BF16, bias=False)
    geo = dict(stride=2, padding=p, dilation=1, groups=G, layout="NHWC")
    dy = random_dy(seed + 1, out_shape(x.shape, w.shape, geo), BF16)
    dx = gpu_dx(dy, w, tuple(x.shape), geo, path="dx_band")
    err = dx_error(dy, w, tuple(x.shape), dx, geo)
    assert err <= TOL[BF16], err
    return dy, w, dx, geo


# Bands are as tall as fill the CUs: one row at small batches, several rows
# (pixel tiles across rows, a shorter last band, a part-filled last tile)
# once N * bands * channel tiles reaches the CU count.
@pytest.mark.parametrize("N,C,H,W,CO,K,p,G", [
    (2, 128, 14, 14, 256, 3, 1, 1),     # the stride-2 shape, small batch
    (1, 64, 9, 11, 16, 3, 1, 1),        # odd extents: phase 1 has a row and column fewer
    (2, 64, 12, 10, 32, 3, 0, 1),       # even padding: shifts up and left
    (1, 64, 10, 8, 16, 3, 2, 1),        # padding 2
    (2, 128, 8, 8, 64, 3, 1, 2),        # two groups of 64
    (32, 64, 30, 30, 32, 3, 1, 1),      # two-row bands, the last one row
    (64, 64, 22, 30, 16, 3, 1, 1),      # three-row bands of 15 columns: two tiles, the last part-filled
    (32, 128, 40, 40, 32, 3, 1, 1),     # five-row bands of 20 columns: four tiles
    (1, 64, 8, 8, 16, 4, 1, 1),         # 4x4: nine shifts, four taps per phase
    (32, 64, 28, 28, 32, 4, 1, 1),      # 4x4, two-row bands
    (2, 64, 9, 12, 16, 4, 0, 1),        # 4x4, even padding
    (1, 128, 12, 12, 64, 3, 1, 1),      # one-row bands of 6 pixels: a stage mostly empty, waves
                                        # issuing two or three loads per chunk
])
def test_dx_band(N, C, H, W, CO, K, p, G):
    dx_band_case(N, C, H, W, CO, K, p, G)


def test_dx_band_declines_other_geometries():
    # Stride 1, dilation 2 and channel widths off the 64 / 16 grid are not its.
    dev = torch.device("cuda:0")
    for (C, CO, H, s, p, d) in [(64, 16, 4, 1, 1, 1), (64, 16, 8, 2, 2, 2), (32, 16, 8, 2, 1, 1),
                                (64, 24, 8, 2, 1, 1)]:
        dy = torch.zeros((1, 4, 4, CO), dtype=BF16, device=dev)
        w = torch.zeros((CO, 3, 3, C), dtype=BF16, device=dev)
        with pytest.raises(cm.ConvError):
            cm.conv2d_input_grad(dy, w, (1, H, H, C), stride=s, padding=p, dilation=d, layout="NHWC",
                                 path="dx_band")


def test_dx_band_impulse_bit_exact():
    x, w, _ = random_case(6, 1, 64, 10, 10, 64, 3, 3, 1, "NHWC", BF16, bias=False)
    geo = dict(stride=2, padding=1, dilation=1, groups=1, layout="NHWC")
    dy = torch.zeros(out_shape(x.shape, w.shape, geo), dtype=BF16)
    dy[0, 2, 3, 17] = 1
    dx = gpu_dx(dy, w, tuple(x.shape), geo, path="dx_band")
    ref, _ = oracle.conv2d_input_grad(dy, w, tuple(x.shape), **geo)
    np.testing.assert_array_equal(f64(dx), ref)


# ------------------------------------- group widths of 24, 40, 56 (igemm) --

@pytest.mark.parametrize("N,C,H,W,CO,K,s,p,d,G", [
    (2, 96, 14, 13, 96, (3, 3), 1, 1, 1, 4),      # C/G = 24: 16 + an 8-channel part chunk
    (1, 80, 11, 12, 40, (3, 3), 2, 1, 1, 2),      # C/G = 40, C_out/G = 20, stride 2
    (2, 112, 9, 10, 112, (3, 3), 1, 2, 2, 2),     # C/G = 56, dilation 2
    (1, 24, 17, 16, 36, (5, 5), 1, 2, 1, 1),      # dense C = 24, 5x5, ragged channel tile
    (2, 192, 12, 11, 192, (3, 3), 1, 1, 1, 8),    # C/G = 24 over 8 groups
    (1, 72, 7, 30, 72, (1, 3), (1, 2), (0, 1), 1, 3),
])
@pytest.mark.parametrize("bias", [True, False])
def test_igemm_group_widths_multiple_of_8(N, C, H, W, CO, K, s, p, d, G, bias):
    fwd_case("igemm", N, C, H, W, CO, K[0], K[1], s, p, d, G, bias=bias)


# ------------------------------------ channel multipliers (depthwise path) --

@pytest.mark.parametrize("N,C,H,W,CO,K,s,p,d,G,dtype", [
    (2, 64, 12, 13, 128, (3, 3), 1, 1, 1, 64, BF16),    # depthwise, multiplier 2
    (1, 32, 10, 9, 128, (3, 3), 2, 1, 1, 32, BF16),     # multiplier 4, stride 2
    (2, 3, 15, 14, 24, (3, 3), 1, 1, 1, 3, BF16),       # RGB input, multiplier 8
    (1, 16, 9, 11, 64, (5, 5), 1, 4, 2, 8, BF16),       # C/G 2 -> 8, dilation 2
    (2, 64, 8, 8, 256, (3, 3), 1, 1, 1, 8, BF16),       # C/G 8 -> 32
    (1, 64, 7, 9, 128, (3, 3), 1, 1, 1, 16, BF16),      # C/G 4 -> 8
    (2, 12, 10, 10, 48, (3, 3), 1, 1, 1, 12, torch.float32),  # fp32, multiplier 4
    (1, 16, 9, 8, 64, (3, 1), (2, 1), (1, 0), 1, 4, torch.float32),  # fp32 C/G 4 -> 16
])
@pytest.mark.parametrize("bias", [True, False])
def test_depthwise_channel_multipliers(N, C, H, W, CO, K, s, p, d, G, dtype, bias):
    fwd_case("depthwise", N, C, H, W, CO, K[0], K[1], s, p, d, G, dtype=dtype, bias=bias)


# ------------------------------------------- dx of small groups (gather) --

def dx_small_case(N, C, H, W, K, s, p, d, G, dtype, seed=0):
    print(f"dx_depthwise: N={N} C={C} H={H} W={W} K={K} s={s} p={p} d={d} G={G} {dtype}", flush=True)
    x, w, _ = random_case(seed, N, C, H, W, C, K[0], K[1], G, "NHWC", dtype, bias=False)
    geo = dict(stride=s, padding=p, dilation=d, groups=G, layout="NHWC")
    dy = random_dy(seed + 1, out_shape(x.shape, w.shape, geo), dtype)
    dx = gpu_dx(dy, w, tuple(x.shape), geo, path="dx_depthwise")
    err = dx_error(dy, w, tuple(x.shape), dx, geo)
    assert err <= TOL[dtype], err
    return dy, w, dx, geo


@pytest.mark.parametrize("N,C,H,W,K,s,p,d,G,dtype", [
    (2, 64, 13, 12, (3, 3), 1, 1, 1, 64, BF16),       # depthwise, unit stride
    (1, 128, 16, 15, (3, 3), 2, 1, 1, 128, BF16),     # stride 2: taps of every phase
    (2, 64, 11, 10, (3, 3), 1, 2, 2, 16, BF16),       # groups of 4, dilation 2
    (1, 32, 9, 14, (5, 5), 3, 2, 1, 16, BF16),        # groups of 2, stride 3
    (2, 64, 8, 9, (3, 3), 2, 0, 1, 8, BF16),          # groups of 8, unread last rows -> 0
    (1, 16, 10, 7, (2, 3), (2, 1), (0, 1), (1, 2), 16, BF16),
    (2, 32, 9, 9, (3, 3), 1, 1, 1, 32, torch.float32),
    (1, 16, 12, 11, (3, 3), 2, 1, 1, 4, torch.float32),  # fp32 groups of 4
])
def test_dx_depthwise(N, C, H, W, K, s, p, d, G, dtype):
    dx_small_case(N, C, H, W, K, s, p, d, G, dtype)


def test_dx_depthwise_impulse_bit_exact():
    x, w, _ = random_case(9, 1, 32, 9, 9, 32, 3, 3, 8, "NHWC", BF16, bias=False)
    geo = dict(stride=2, padding=1, dilation=1, groups=8, layout="NHWC")
    dy = torch.zeros(out_shape(x.shape, w.shape, geo), dtype=BF16)
    dy[0, 2, 3, 13] = 1
    dx = gpu_dx(dy, w, tuple(x.shape), geo, path="dx_depthwise")
    ref, _ = oracle.conv2d_input_grad(dy, w, tuple(x.shape), **geo)
    np.testing.assert_array_equal(f64(dx), ref)


def test_depthwise_multiplier_impulse_bit_exact():
    x, w, _ = random_case(10, 1, 16, 7, 8, 64, 3, 3, 16, "NHWC", BF16, bias=False)
    x = torch.zeros_like(x)
    x[0, 3, 4, 5] = 1
    geo = dict(stride=1, padding=1, dilation=1, groups=16, layout="NHWC")
    y = gpu_fwd(x, w, None, geo, path="depthwise")
    ref, _ = oracle.conv2d_forward(x, w, None, **geo)
    np.testing.assert_array_equal(f64(y), ref)
