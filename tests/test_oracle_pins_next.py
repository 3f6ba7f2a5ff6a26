"""Pins of the oracle's conv1d, transposed-conv2d and weight-gradient
functions (CPU only).

Each test fixes a function of ``oracle/`` to something independent of it:
torch's CPU fp64 library convolutions and weight gradient, the
unfold-then-GEMM formulation the oarust page gives for ``conv_1d``, the
extent formula of the page's ``ConvTranspose2dGeometry::resolve``, the
burn-cubecl page's weight gradient as one matmul (1x1) and over im2col
columns, the adjoint identities against the already pinned 2-D forward,
impulses and the bias.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

# (N, C, L, C_out, K, stride, pad, dil, groups)
SWEEP_1D = [
    (2, 3, 11, 4, 3, 1, 1, 1, 1),
    (1, 4, 17, 6, 3, 2, 2, 3, 2),
    (2, 6, 9, 6, 2, 3, 0, 1, 3),
    (1, 8, 20, 8, 5, 1, 4, 2, 8),
    (3, 2, 7, 5, 1, 2, 0, 1, 1),
    (1, 4, 6, 4, 6, 1, 0, 1, 1),
]


def rand_1d(rng, N, C, L, CO, K, G, layout, bias=True):
    Cg = C // G
    x = rng.standard_normal((N, C, L))
    w = rng.standard_normal((CO, Cg, K))
    b = rng.standard_normal(CO) if bias else None
    if layout == "NLC":
        return np.transpose(x, (0, 2, 1)).copy(), np.transpose(w, (0, 2, 1)).copy(), b, x, w
    return x, w, b, x, w


@pytest.mark.parametrize("case", SWEEP_1D)
@pytest.mark.parametrize("layout", ["NCL", "NLC"])
def test_conv1d_matches_torch_cpu_fp64(case, layout):
    N, C, L, CO, K, s, p, d, G = case
    rng = np.random.default_rng(11)
    x, w, b, x_ncl, w_oik = rand_1d(rng, N, C, L, CO, K, G, layout)
    y, norm = oracle.conv1d_forward(x, w, b, s, p, d, G, layout)
    ref = F.conv1d(torch.from_numpy(x_ncl), torch.from_numpy(w_oik), torch.from_numpy(b), s, p, d, G)
    ref = ref.numpy()
    if layout == "NLC":
        ref = np.transpose(ref, (0, 2, 1))
    assert y.shape == ref.shape
    assert oracle.max_normalised_error(y, ref, norm) < 1e-13


@pytest.mark.parametrize("case", SWEEP_1D)
def test_conv1d_equals_unfold_then_gemm(case):
    # The oarust page lowers conv_1d to an unfold -- rows (n, t), columns
    # (c, k) holding x[n, c, t*s - p + k*d] or zero -- followed by a GEMM with
    # the weight viewed as [C_out, C*K] and a bias add.  Per group here.
    N, C, L, CO, K, s, p, d, G = case
    rng = np.random.default_rng(12)
    x, w, b, _, _ = rand_1d(rng, N, C, L, CO, K, G, "NCL")
    OL = (L + 2 * p - (K - 1) * d - 1) // s + 1
    Cg, Mg = C // G, CO // G
    y_ref = np.zeros((N, CO, OL))
    for g in range(G):
        cols = np.zeros((N * OL, Cg * K))
        for n, t, c, k in itertools.product(range(N), range(OL), range(Cg), range(K)):
            l = t * s - p + k * d
            if 0 <= l < L:
                cols[n * OL + t, c * K + k] = x[n, g * Cg + c, l]
        wm = w[g * Mg:(g + 1) * Mg].reshape(Mg, Cg * K)
        out = cols @ wm.T + b[g * Mg:(g + 1) * Mg]
        y_ref[:, g * Mg:(g + 1) * Mg, :] = out.reshape(N, OL, Mg).transpose(0, 2, 1)
    y, norm = oracle.conv1d_forward(x, w, b, s, p, d, G, "NCL")
    assert oracle.max_normalised_error(y, y_ref, norm) < 1e-13


@pytest.mark.parametrize("layout", ["NCL", "NLC"])
def test_conv1d_impulse_reproduces_flipped_weights(layout):
    N, C, L, CO, K, s, p, d, G = 2, 4, 13, 6, 3, 1, 2, 2, 2
    rng = np.random.default_rng(13)
    _, w, _, _, w_oik = rand_1d(rng, N, C, L, CO, K, G, layout, bias=False)
    n0, c0, l0 = 1, 3, 6
    x_ncl = np.zeros((N, C, L))
    x_ncl[n0, c0, l0] = 1.0
    x = x_ncl if layout == "NCL" else np.transpose(x_ncl, (0, 2, 1)).copy()
    y, _ = oracle.conv1d_forward(x, w, None, s, p, d, G, layout)
    y_ncl = y if layout == "NCL" else np.transpose(y, (0, 2, 1))
    Cg, Mg = C // G, CO // G
    g0 = c0 // Cg
    expect = np.zeros_like(y_ncl)
    for m, k in itertools.product(range(Mg), range(K)):
        t = l0 + p - k * d
        if t % s == 0 and 0 <= t // s < expect.shape[2]:
            expect[n0, g0 * Mg + m, t // s] = w_oik[g0 * Mg + m, c0 - g0 * Cg, k]
    np.testing.assert_array_equal(y_ncl, expect)


def test_conv1d_is_the_one_row_case_of_conv2d():
    N, C, L, CO, K, s, p, d, G = 2, 6, 15, 4, 3, 2, 1, 2, 2
    rng = np.random.default_rng(14)
    x, w, b, _, _ = rand_1d(rng, N, C, L, CO, K, G, "NCL")
    y1, n1 = oracle.conv1d_forward(x, w, b, s, p, d, G, "NCL")
    y2, n2 = oracle.conv2d_forward(x[:, :, None, :], w[:, :, None, :], b, stride=(1, s),
                                   padding=(0, p), dilation=(1, d), groups=G, layout="NCHW")
    np.testing.assert_array_equal(y1, y2[:, :, 0, :])
    np.testing.assert_array_equal(n1, n2[:, :, 0, :])


# ------------------------------------------------------- transposed conv2d --

# (N, C_in, H, W, C_out, KH, KW, stride, pad, out_pad, dil, groups)
SWEEP_T = [
    (2, 3, 4, 5, 4, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1), 1),
    (1, 4, 5, 3, 6, 4, 4, (2, 2), (1, 1), (0, 0), (1, 1), 2),
    (2, 6, 3, 4, 3, 3, 2, (3, 1), (0, 1), (2, 0), (1, 2), 3),
    (1, 2, 6, 6, 2, 2, 3, (1, 2), (0, 1), (0, 1), (2, 1), 1),
    (1, 4, 2, 3, 8, 5, 5, (2, 3), (2, 1), (1, 2), (1, 1), 4),
    (3, 2, 3, 3, 5, 1, 1, (2, 2), (0, 0), (1, 0), (1, 1), 1),
]


def rand_t(rng, N, CI, H, W, CO, KH, KW, G, layout, bias=True):
    x = rng.standard_normal((N, CI, H, W))
    w = rng.standard_normal((CI, CO // G, KH, KW))
    b = rng.standard_normal(CO) if bias else None
    if layout == "NHWC":
        return (np.transpose(x, (0, 2, 3, 1)).copy(), np.transpose(w, (0, 2, 3, 1)).copy(), b, x, w)
    return x, w, b, x, w


def to_nchw_y(y, layout):
    return y if layout == "NCHW" else np.transpose(y, (0, 3, 1, 2))


@pytest.mark.parametrize("case", SWEEP_T)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_conv_transpose2d_matches_torch_cpu_fp64(case, layout):
    N, CI, H, W, CO, KH, KW, s, p, op, d, G = case
    rng = np.random.default_rng(21)
    x, w, b, x_nchw, w_iokk = rand_t(rng, N, CI, H, W, CO, KH, KW, G, layout)
    y, norm = oracle.conv_transpose2d(x, w, b, s, p, op, d, G, layout)
    ref = F.conv_transpose2d(torch.from_numpy(x_nchw), torch.from_numpy(w_iokk), torch.from_numpy(b),
                             stride=s, padding=p, output_padding=op, groups=G, dilation=d).numpy()
    y_nchw = to_nchw_y(y, layout)
    assert y_nchw.shape == ref.shape
    assert oracle.max_normalised_error(to_nchw_y(y, layout), ref, to_nchw_y(norm, layout)) < 1e-13


def test_conv_transpose_size_is_the_pages_extent():
    # The page's square, undilated case: (H - 1)*s + K - 2p, an error when the
    # padding removes the whole output.
    for H, K, s, p in itertools.product(range(1, 7), range(1, 6), range(1, 4), range(0, 4)):
        want = (H - 1) * s + K - 2 * p
        got = oracle.conv_transpose_size(H, K, s, p)
        assert got == (want if want > 0 else None), (H, K, s, p)
    assert oracle.conv_transpose_size(4, 3, 2, 1, 1, 2) is None  # output padding must be < stride


@pytest.mark.parametrize("case", SWEEP_T)
def test_conv_transpose2d_is_the_adjoint_of_the_forward(case):
    # <convT(x), z> = <x, conv(z)> with the same weight read as the forward's
    # OIHW weight [C_out_fwd = C_in, C_in_fwd / G = C_out / G, KH, KW].
    N, CI, H, W, CO, KH, KW, s, p, op, d, G = case
    rng = np.random.default_rng(22)
    x, w, _, _, _ = rand_t(rng, N, CI, H, W, CO, KH, KW, G, "NCHW", bias=False)
    y, _ = oracle.conv_transpose2d(x, w, None, s, p, op, d, G, "NCHW")
    z = rng.standard_normal(y.shape)
    fz, _ = oracle.conv2d_forward(z, w, None, stride=s, padding=p, dilation=d, groups=G, layout="NCHW")
    assert fz.shape == x.shape
    lhs, rhs = float(np.sum(y * z)), float(np.sum(x * fz))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, np.sum(np.abs(y * z)))


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_conv_transpose2d_impulse_spreads_the_weights(layout):
    N, CI, H, W, CO, KH, KW, s, p, op, d, G = 2, 4, 4, 5, 6, 3, 2, (2, 3), (1, 0), (1, 2), (1, 2), 2
    rng = np.random.default_rng(23)
    _, w, _, _, w_iokk = rand_t(rng, N, CI, H, W, CO, KH, KW, G, layout, bias=False)
    n0, c0, h0, w0 = 1, 2, 3, 1
    x_nchw = np.zeros((N, CI, H, W))
    x_nchw[n0, c0, h0, w0] = 1.0
    x = x_nchw if layout == "NCHW" else np.transpose(x_nchw, (0, 2, 3, 1)).copy()
    y, _ = oracle.conv_transpose2d(x, w, None, s, p, op, d, G, layout)
    y_nchw = to_nchw_y(y, layout)
    Cg, Mg = CI // G, CO // G
    g0 = c0 // Cg
    expect = np.zeros_like(y_nchw)
    for m, kh, kw in itertools.product(range(Mg), range(KH), range(KW)):
        oh, ow = h0 * s[0] - p[0] + kh * d[0], w0 * s[1] - p[1] + kw * d[1]
        if 0 <= oh < expect.shape[2] and 0 <= ow < expect.shape[3]:
            expect[n0, g0 * Mg + m, oh, ow] = w_iokk[c0, m, kh, kw]
    np.testing.assert_array_equal(y_nchw, expect)


def test_conv_transpose2d_bias_is_added_once_per_channel():
    N, CI, H, W, CO, KH, KW, s, p, op, d, G = SWEEP_T[0]
    rng = np.random.default_rng(24)
    x, w, b, _, _ = rand_t(rng, N, CI, H, W, CO, KH, KW, G, "NCHW")
    y1, _ = oracle.conv_transpose2d(x, w, b, s, p, op, d, G, "NCHW")
    y0, _ = oracle.conv_transpose2d(x, w, None, s, p, op, d, G, "NCHW")
    np.testing.assert_allclose(y1 - y0, np.broadcast_to(b[None, :, None, None], y0.shape), rtol=0,
                               atol=1e-12)


# ---------------------------------------------------------- weight gradient --

# (N, C, H, W, CO, KH, KW, stride, pad, dil, groups)
SWEEP_DW = [
    (2, 3, 7, 6, 4, 3, 3, (1, 1), (1, 1), (1, 1), 1),
    (1, 4, 9, 8, 6, 3, 2, (2, 1), (1, 0), (1, 2), 2),
    (2, 4, 8, 9, 4, 3, 3, (2, 2), (2, 1), (2, 1), 4),
    (1, 6, 10, 7, 3, 2, 3, (3, 2), (0, 2), (2, 2), 3),
    (2, 5, 6, 6, 3, 1, 1, (1, 1), (0, 0), (1, 1), 1),
    (1, 3, 4, 11, 5, 4, 5, (1, 3), (2, 1), (1, 1), 1),
]


def rand_dw(rng, N, C, H, W, CO, KH, KW, s, p, d, G, layout):
    OH = (H + 2 * p[0] - d[0] * (KH - 1) - 1) // s[0] + 1
    OW = (W + 2 * p[1] - d[1] * (KW - 1) - 1) // s[1] + 1
    x = rng.standard_normal((N, C, H, W))
    dy = rng.standard_normal((N, CO, OH, OW))
    w_shape = (CO, C // G, KH, KW)
    if layout == "NHWC":
        return (np.transpose(x, (0, 2, 3, 1)).copy(), np.transpose(dy, (0, 2, 3, 1)).copy(),
                (CO, KH, KW, C // G), x, dy)
    return x, dy, w_shape, x, dy


def w_to_oihw(w, layout):
    return w if layout == "NCHW" else np.transpose(w, (0, 3, 1, 2))


@pytest.mark.parametrize("case", SWEEP_DW)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_weight_grad_matches_torch_cpu_fp64(case, layout):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(31)
    x, dy, w_shape, x_nchw, dy_nchw = rand_dw(rng, N, C, H, W, CO, KH, KW, s, p, d, G, layout)
    dw, norm = oracle.conv2d_weight_grad(x, dy, w_shape, s, p, d, G, layout)
    ref = torch.nn.grad.conv2d_weight(torch.from_numpy(x_nchw), (CO, C // G, KH, KW),
                                      torch.from_numpy(dy_nchw), stride=s, padding=p, dilation=d,
                                      groups=G).numpy()
    assert oracle.max_normalised_error(w_to_oihw(dw, layout), ref, w_to_oihw(norm, layout)) < 1e-13


@pytest.mark.parametrize("case", SWEEP_DW)
def test_weight_grad_is_the_weight_adjoint_of_the_forward(case):
    # conv(x, w) is linear in w: <conv(x, w), dy> = <w, dw(x, dy)>.
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(32)
    x, dy, w_shape, _, _ = rand_dw(rng, N, C, H, W, CO, KH, KW, s, p, d, G, "NCHW")
    w = rng.standard_normal(w_shape)
    y, _ = oracle.conv2d_forward(x, w, None, stride=s, padding=p, dilation=d, groups=G, layout="NCHW")
    dw, _ = oracle.conv2d_weight_grad(x, dy, w_shape, s, p, d, G, "NCHW")
    lhs, rhs = float(np.sum(y * dy)), float(np.sum(w * dw))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, float(np.sum(np.abs(y * dy))))


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_pointwise_weight_grad_is_dy_transpose_times_x(layout):
    # The page's 1x1 weight gradient: grad_w[c_out, c_in] = sum over pixels of
    # grad_out[pixel, c_out] * input[pixel, c_in], one matmul.
    N, C, H, W, CO = 2, 5, 4, 6, 3
    rng = np.random.default_rng(33)
    x, dy, w_shape, x_nchw, dy_nchw = rand_dw(rng, N, C, H, W, CO, 1, 1, (1, 1), (0, 0), (1, 1), 1,
                                              layout)
    dw, _ = oracle.conv2d_weight_grad(x, dy, w_shape, 1, 0, 1, 1, layout)
    xm = np.transpose(x_nchw, (0, 2, 3, 1)).reshape(-1, C)
    dym = np.transpose(dy_nchw, (0, 2, 3, 1)).reshape(-1, CO)
    np.testing.assert_allclose(w_to_oihw(dw, layout)[:, :, 0, 0], dym.T @ xm, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("case", SWEEP_DW)
def test_weight_grad_equals_columns_gemm(case):
    # The page's dense weight gradient: [c_out, m] @ [m, (kernel..., c_in)]
    # over the im2col columns of the input, per group.
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(34)
    x, dy, w_shape, _, _ = rand_dw(rng, N, C, H, W, CO, KH, KW, s, p, d, G, "NHWC")
    OH, OW = dy.shape[1], dy.shape[2]
    Cg, Mg = C // G, CO // G
    ref = np.zeros((CO, KH, KW, Cg))
    for g in range(G):
        cols = np.zeros((N * OH * OW, KH * KW * Cg))
        for n, oh, ow, kh, kw in itertools.product(range(N), range(OH), range(OW), range(KH), range(KW)):
            ih, iw = oh * s[0] - p[0] + kh * d[0], ow * s[1] - p[1] + kw * d[1]
            if 0 <= ih < H and 0 <= iw < W:
                cols[(n * OH + oh) * OW + ow, (kh * KW + kw) * Cg:(kh * KW + kw + 1) * Cg] = \
                    x[n, ih, iw, g * Cg:(g + 1) * Cg]
        dym = dy[..., g * Mg:(g + 1) * Mg].reshape(-1, Mg)
        ref[g * Mg:(g + 1) * Mg] = (dym.T @ cols).reshape(Mg, KH, KW, Cg)
    dw, norm = oracle.conv2d_weight_grad(x, dy, w_shape, s, p, d, G, "NHWC")
    assert oracle.max_normalised_error(dw, ref, norm) < 1e-13


def test_weight_grad_of_two_impulses_is_one_tap():
    N, C, H, W, CO, KH, KW, s, p, d, G = 2, 4, 7, 8, 6, 3, 3, (2, 1), (1, 2), (1, 2), 2
    x = np.zeros((N, C, H, W))
    n0, c0, h0, w0 = 1, 3, 4, 5
    x[n0, c0, h0, w0] = 1.0
    OH = (H + 2 * p[0] - d[0] * (KH - 1) - 1) // s[0] + 1
    OW = (W + 2 * p[1] - d[1] * (KW - 1) - 1) // s[1] + 1
    dy = np.zeros((N, CO, OH, OW))
    co0, oh0, ow0 = 4, 2, 3  # co0 in group 1, as c0
    dy[n0, co0, oh0, ow0] = 1.0
    dw, _ = oracle.conv2d_weight_grad(x, dy, (CO, C // G, KH, KW), s, p, d, G, "NCHW")
    expect = np.zeros_like(dw)
    kh, kw = (h0 - oh0 * s[0] + p[0]) / d[0], (w0 - ow0 * s[1] + p[1]) / d[1]
    assert kh == int(kh) and kw == int(kw)
    expect[co0, c0 - (co0 // (CO // G)) * (C // G), int(kh), int(kw)] = 1.0
    np.testing.assert_array_equal(dw, expect)
