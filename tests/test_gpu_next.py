"""GPU parity of conv1d and the transposed 2-D convolution against the fp64
oracle, through the C ABI.

conv1d runs on the forward kernels (a sequence is an image of one row) and
the transposed convolution on the input-gradient kernels plus a fused bias;
every case forces its path, so a path that declined would fail the test.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_conv2d_amd as cm
import oracle
from convolution_implicit_gemm_conv2d_amd import inputs
from helpers import TOL, f64, record

pytestmark = pytest.mark.gpu
BF16, F32 = torch.bfloat16, torch.float32
DEV = torch.device("cuda:0")


def rnd(seed, shape, dtype):
    gen = torch.Generator().manual_seed(seed)
    return inputs.draw(tuple(shape), ("uniform", -1.0, 1.0), gen, dtype)


# ------------------------------------------------------------------ conv1d --

# (N, C, L, C_out, K, stride, pad, dil, groups, layout, dtype, path)
CONV1D = [
    (2, 5, 33, 7, 3, 2, 1, 2, 1, "NCL", F32, "direct"),
    (2, 6, 29, 4, 4, 1, 3, 1, 2, "NCL", BF16, "direct"),
    (1, 3, 40, 5, 5, 3, 2, 2, 1, "NLC", F32, "direct"),
    (2, 64, 100, 40, 3, 1, 2, 2, 1, "NLC", BF16, "igemm"),
    (3, 32, 70, 36, 5, 2, 2, 1, 1, "NLC", BF16, "igemm"),
    (2, 128, 45, 64, 3, 1, 1, 1, 2, "NLC", BF16, "igemm"),
    (3, 64, 77, 32, 1, 1, 0, 1, 1, "NLC", BF16, "pointwise"),
    (2, 96, 50, 100, 1, 2, 0, 1, 1, "NLC", BF16, "pointwise"),
    (2, 64, 41, 40, 1, 2, 3, 1, 1, "NLC", BF16, "pointwise"),
    (2, 64, 90, 64, 3, 1, 2, 2, 64, "NLC", BF16, "depthwise"),
    (1, 32, 61, 32, 5, 2, 2, 1, 32, "NLC", F32, "depthwise"),
]


@pytest.mark.parametrize("case", CONV1D)
@pytest.mark.parametrize("bias", [True, False])
def test_conv1d(case, bias):
    N, C, L, CO, K, s, p, d, G, layout, dtype, path = case
    print(f"conv1d {path}: N={N} C={C} L={L} CO={CO} K={K} s={s} p={p} d={d} G={G} {layout} "
          f"{dtype} bias={bias}", flush=True)
    x = rnd(1, (N, C, L) if layout == "NCL" else (N, L, C), dtype)
    w = rnd(2, (CO, C // G, K) if layout == "NCL" else (CO, K, C // G), dtype)
    b = rnd(3, (CO,), dtype) if bias else None
    y = cm.conv1d(x.to(DEV), w.to(DEV), None if b is None else b.to(DEV), s, p, d, G, layout,
                  path=path)
    torch.cuda.synchronize()
    ref, norm = oracle.conv1d_forward(x, w, b, s, p, d, G, layout)
    assert tuple(y.shape) == ref.shape
    err = oracle.max_normalised_error(f64(y.cpu()), ref, norm)
    assert err <= TOL[dtype], err


def test_conv1d_auto_path_matches_oracle():
    x = rnd(4, (4, 64, 256), BF16)   # NLC: N, L, C
    w = rnd(5, (128, 3, 256), BF16)
    b = rnd(6, (128,), BF16)
    y = cm.conv1d(x.to(DEV), w.to(DEV), b.to(DEV), 1, 4, 4, 1, "NLC")
    torch.cuda.synchronize()
    ref, norm = oracle.conv1d_forward(x, w, b, 1, 4, 4, 1, "NLC")
    assert oracle.max_normalised_error(f64(y.cpu()), ref, norm) <= TOL[BF16]


# -------------------------------------------------------- transposed conv2d --

# (N, C_in, H, W, C_out, KH, KW, stride, pad, out_pad, dil, groups, layout, dtype, path)
TRANSPOSED = [
    (2, 6, 5, 4, 4, 3, 3, 2, 1, 1, 1, 2, "NCHW", F32, "dx_gather"),
    (1, 4, 3, 6, 6, 2, 3, (3, 1), (0, 1), (2, 0), (1, 2), 1, "NCHW", F32, "dx_gather"),
    (1, 6, 4, 4, 5, 3, 3, 2, 0, 1, 1, 1, "NHWC", BF16, "dx_gather"),
    (2, 128, 7, 9, 64, 4, 4, 2, 1, 0, 1, 1, "NHWC", BF16, "dx_igemm"),
    (1, 64, 6, 6, 32, 3, 3, 2, 1, 1, 1, 1, "NHWC", BF16, "dx_igemm"),
    (2, 64, 5, 5, 64, 3, 3, 1, 1, 0, 1, 2, "NHWC", BF16, "dx_igemm"),
    (1, 256, 9, 8, 136, 3, 3, 2, 1, 1, 1, 1, "NHWC", BF16, "dx_igemm"),
    (3, 64, 14, 14, 96, 4, 4, 2, 1, 0, 1, 1, "NHWC", BF16, "dx_igemm"),
    (2, 128, 7, 9, 64, 4, 4, 2, 1, 0, 1, 1, "NHWC", BF16, "dx_band"),
    (1, 64, 6, 6, 128, 3, 3, 2, 1, 1, 1, 1, "NHWC", BF16, "dx_band"),
    (2, 256, 14, 14, 128, 4, 4, 2, 1, 0, 1, 1, "NHWC", BF16, "dx_band"),
    (2, 64, 7, 9, 64, 3, 3, 2, 1, 1, 1, 64, "NHWC", BF16, "dx_depthwise"),   # depthwise, upsampling
    (1, 32, 6, 5, 32, 4, 4, 2, 1, 0, 1, 8, "NHWC", BF16, "dx_depthwise"),    # groups of 4
]


def run_transposed(case, bias, seed=7):
    N, CI, H, W, CO, KH, KW, s, p, op, d, G, layout, dtype, path = case
    print(f"conv_transpose2d {path}: N={N} C_in={CI} H={H} W={W} C_out={CO} K={KH}x{KW} s={s} "
          f"p={p} op={op} d={d} G={G} {layout} {dtype} bias={bias}", flush=True)
    xs = (N, CI, H, W) if layout == "NCHW" else (N, H, W, CI)
    ws = (CI, CO // G, KH, KW) if layout == "NCHW" else (CI, KH, KW, CO // G)
    x, w = rnd(seed, xs, dtype), rnd(seed + 1, ws, dtype)
    b = rnd(seed + 2, (CO,), dtype) if bias else None
    y = cm.conv2d_transposed(x.to(DEV), w.to(DEV), None if b is None else b.to(DEV), s, p, op, d,
                             G, layout, path=path)
    torch.cuda.synchronize()
    ref, norm = oracle.conv_transpose2d(x, w, b, s, p, op, d, G, layout)
    assert tuple(y.shape) == ref.shape
    return x, w, b, y.cpu(), ref, norm


@pytest.mark.parametrize("case", TRANSPOSED)
@pytest.mark.parametrize("bias", [True, False])
def test_conv_transpose2d(case, bias):
    dtype = case[13]
    _, _, _, y, ref, norm = run_transposed(case, bias)
    err = oracle.max_normalised_error(f64(y), ref, norm)
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("path", ["dx_igemm", "dx_band", "dx_gather"])
def test_conv_transpose2d_impulse_bit_exact(path):
    # A one-hot input spreads one weight per output: single products, exact.
    N, CI, H, W, CO, K = 1, 64, 5, 6, 64, 3
    x = torch.zeros((N, H, W, CI), dtype=BF16)
    x[0, 2, 3, 17] = 1
    w = rnd(9, (CI, K, K, CO), BF16)
    y = cm.conv2d_transposed(x.to(DEV), w.to(DEV), None, 2, 1, 1, 1, 1, "NHWC", path=path)
    torch.cuda.synchronize()
    ref, _ = oracle.conv_transpose2d(x, w, None, 2, 1, 1, 1, 1, "NHWC")
    np.testing.assert_array_equal(f64(y.cpu()), ref)


def test_conv_transpose2d_equals_input_grad_plus_bias():
    # The two entry points run the same kernel: conv_transpose2d(x) - bias is
    # bitwise conv_bwd_dx with dy = x on the forward geometry, when the bias
    # is zero.
    case = TRANSPOSED[3]
    N, CI, H, W, CO, KH, KW, s, p, op, d, G = case[:12]
    x = rnd(11, (N, H, W, CI), BF16).to(DEV)
    w = rnd(12, (CI, KH, KW, CO // G), BF16).to(DEV)
    y = cm.conv2d_transposed(x, w, torch.zeros(CO, dtype=BF16, device=DEV), s, p, op, d, G, "NHWC")
    OH = cm.conv_transpose_out_size(H, KH, s, p, d, op)
    OW = cm.conv_transpose_out_size(W, KW, s, p, d, op)
    dx = cm.conv2d_input_grad(x, w, (N, OH, OW, CO), stride=s, padding=p, dilation=d, groups=G,
                              layout="NHWC")
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), dx.cpu())


# --------------------------------------------------------- weight gradient --

# (N, C, H, W, C_out, KH, KW, stride, pad, dil, groups, layout, dtype, path)
DW = [
    (2, 3, 9, 8, 5, 3, 3, 1, 1, 1, 1, "NCHW", F32, "dw_direct"),
    (1, 4, 10, 9, 6, 3, 2, (2, 1), (1, 0), (1, 2), 2, "NCHW", F32, "dw_direct"),
    (2, 6, 7, 7, 6, 3, 3, 2, 2, 2, 3, "NHWC", F32, "dw_direct"),
    (2, 16, 12, 11, 8, 3, 3, 1, 1, 1, 1, "NHWC", BF16, "dw_direct"),
    (3, 8, 6, 6, 8, 1, 1, 1, 0, 1, 1, "NHWC", BF16, "dw_direct"),
    (1, 8, 9, 9, 8, 3, 3, 1, 2, 2, 8, "NHWC", BF16, "dw_direct"),
    (2, 64, 14, 14, 64, 3, 3, 1, 1, 1, 1, "NHWC", BF16, "dw_igemm"),
    (2, 128, 9, 11, 72, 3, 3, 2, 1, 1, 1, "NHWC", BF16, "dw_igemm"),   # 9 k tiles, ragged co tile
    (1, 32, 12, 12, 16, 3, 3, 1, 2, 2, 1, "NHWC", BF16, "dw_igemm"),   # dilation
    (2, 64, 8, 8, 64, 3, 3, 1, 1, 1, 2, "NHWC", BF16, "dw_igemm"),     # two groups
    (3, 16, 7, 9, 24, 5, 5, 1, 2, 1, 1, "NHWC", BF16, "dw_igemm"),     # Ktot = 400: ragged k tile
    (2, 256, 7, 7, 128, 1, 1, 1, 0, 1, 1, "NHWC", BF16, "dw_igemm"),   # 1x1
    (2, 8, 5, 6, 8, 3, 3, 1, 1, 1, 1, "NHWC", BF16, "dw_igemm"),       # Ktot = 72 < one k tile
    (1, 24, 13, 10, 40, 3, 2, (3, 1), (1, 0), (2, 3), 1, "NHWC", BF16, "dw_igemm"),
]


def run_dw(case, seed=21):
    N, C, H, W, CO, KH, KW, s, p, d, G, layout, dtype, path = case
    print(f"conv_bwd_dw {path}: N={N} C={C} H={H} W={W} C_out={CO} K={KH}x{KW} s={s} p={p} d={d} "
          f"G={G} {layout} {dtype}", flush=True)
    sp = s if isinstance(s, tuple) else (s, s)
    pp = p if isinstance(p, tuple) else (p, p)
    dp = d if isinstance(d, tuple) else (d, d)
    OH = oracle.out_size(H, KH, sp[0], pp[0], dp[0])
    OW = oracle.out_size(W, KW, sp[1], pp[1], dp[1])
    xs = (N, C, H, W) if layout == "NCHW" else (N, H, W, C)
    ys = (N, CO, OH, OW) if layout == "NCHW" else (N, OH, OW, CO)
    ws = (CO, C // G, KH, KW) if layout == "NCHW" else (CO, KH, KW, C // G)
    x, dy = rnd(seed, xs, dtype), rnd(seed + 1, ys, dtype)
    dw = cm.conv2d_weight_grad(x.to(DEV), dy.to(DEV), ws, s, p, d, G, layout, path=path)
    torch.cuda.synchronize()
    ref, norm = oracle.conv2d_weight_grad(x, dy, ws, s, p, d, G, layout)
    assert tuple(dw.shape) == ref.shape
    return dw.cpu(), ref, norm


@pytest.mark.parametrize("case", DW)
def test_conv_bwd_dw(case):
    dw, ref, norm = run_dw(case)
    err = oracle.max_normalised_error(f64(dw), ref, norm)
    assert err <= TOL[case[12]], err


def test_conv_bwd_dw_is_deterministic_and_ignores_workspace_contents():
    case = DW[3]
    N, C, H, W, CO, KH, KW, s, p, d, G, layout, dtype, path = case
    x = rnd(31, (N, H, W, C), dtype).to(DEV)
    dy = rnd(32, (N, H, W, CO), dtype).to(DEV)
    ws_bytes = cm.conv_bwd_dw_workspace_size(N, C, H, W, CO, KH, KW, s, s, p, p, d, d, G,
                                             cm.CONV_NHWC, cm.CONV_BF16, cm.PATHS[path])
    work = torch.full((ws_bytes,), 0x7f, dtype=torch.uint8, device=DEV)  # garbage partials
    a = cm.conv2d_weight_grad(x, dy, (CO, KH, KW, C), s, p, d, G, "NHWC", path=path, workspace=work)
    b = cm.conv2d_weight_grad(x, dy, (CO, KH, KW, C), s, p, d, G, "NHWC", path=path)
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), b.cpu())


def test_conv_bwd_dw_igemm_dense_layer_full_size():
    # The weight gradient of the dense 3x3 layer of the benchmark (N=32,
    # 56x56, 64 -> 64) at full size, in the launch configuration bench.py
    # times, against the oracle on every element.
    case = (32, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1, "NHWC", BF16, "dw_igemm")
    dw, ref, norm = run_dw(case, seed=41)
    err = oracle.max_normalised_error(f64(dw), ref, norm)
    record("dw_3x3_c64_k64_56x56_n32_bf16_nhwc", err, TOL[BF16], compared="every output")
    assert err <= TOL[BF16], err


# ------------------------------------------ next rows at the measured sizes --

def test_conv1d_full_size_every_image():
    # The conv1d workload bench.py measures, at full size and in its launch
    # configuration, against the oracle on every image.
    from convolution_implicit_gemm_conv2d_amd import inputs as inp

    name = "conv1d_k3_d4_c128_k128_l4096_n32_bf16_nlc"
    s = inp.NEXT_WORKLOADS[name]
    d = inp.make(name)
    y = cm.conv1d(d["x"].to(DEV), d["w"].to(DEV), d["bias"].to(DEV), s["stride"], s["pad"], s["dil"],
                  s["groups"], s["layout"])
    torch.cuda.synchronize()
    ref, norm = oracle.conv1d_forward(d["x"], d["w"], d["bias"], s["stride"], s["pad"], s["dil"],
                                      s["groups"], s["layout"])
    err = oracle.max_normalised_error(f64(y.cpu()), ref, norm)
    record(name, err, TOL[BF16], compared="every output")
    assert err <= TOL[BF16], err


def test_conv_transpose2d_full_size_every_image():
    from convolution_implicit_gemm_conv2d_amd import inputs as inp

    name = "convT_4x4_s2_c256_k128_28to56_n32_bf16_nhwc"
    s = inp.NEXT_WORKLOADS[name]
    d = inp.make(name)
    y = cm.conv2d_transposed(d["x"].to(DEV), d["w"].to(DEV), d["bias"].to(DEV), s["stride"], s["pad"],
                             s["out_pad"], s["dil"], s["groups"], s["layout"])
    torch.cuda.synchronize()
    ref, norm = oracle.conv_transpose2d(d["x"], d["w"], d["bias"], s["stride"], s["pad"],
                                        s["out_pad"], s["dil"], s["groups"], s["layout"])
    err = oracle.max_normalised_error(f64(y.cpu()), ref, norm)
    record(name, err, TOL[BF16], compared="every output")
    assert err <= TOL[BF16], err


@pytest.mark.parametrize("name,path", [("grouped_3x3_g32_c128_56x56_n32_bf16_nhwc", "depthwise"),
                                       ("grouped_3x3_g32_c256_28x28_n32_bf16_nhwc", "depthwise"),
                                       ("grouped_3x3_g8_c192_56x56_n32_bf16_nhwc", "igemm"),
                                       ("depthwise_mult2_3x3_c64_k128_56x56_n32_bf16_nhwc", "depthwise")])
def test_grouped_full_size_every_image(name, path):
    # The grouped workloads bench.py measures, through the path it times,
    # against the oracle on every image.
    from convolution_implicit_gemm_conv2d_amd import inputs as inp

    s = inp.NEXT_WORKLOADS[name]
    d = inp.make(name)
    print(f"{name}", flush=True)
    b = None if d["bias"] is None else d["bias"].to(DEV)
    y = cm.conv2d(d["x"].to(DEV), d["w"].to(DEV), b, s["stride"], s["pad"], s["dil"], s["groups"],
                  s["layout"], path=path)
    torch.cuda.synchronize()
    ref, norm = oracle.conv2d_forward(d["x"], d["w"], d["bias"], stride=s["stride"],
                                      padding=s["pad"], dilation=s["dil"], groups=s["groups"],
                                      layout=s["layout"])
    err = oracle.max_normalised_error(f64(y.cpu()), ref, norm)
    record(name, err, TOL[BF16], path=path, compared="every output")
    assert err <= TOL[BF16], err
