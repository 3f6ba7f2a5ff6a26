"""Pins of the fp64 CPU oracle against facts that do not come from the oracle.

Each test fixes one part of ``oracle/`` to something independent of it: a
brute-force count, hand-worked examples, an im2col + GEMM formulation written
from the burn-cubecl ``im2col`` page, algebraic identities, scipy's 2-D
correlation and torch's CPU fp64 convolution.  CPU only.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy import signal

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def rel_err(a, b, norm):
    return oracle.max_normalised_error(a, b, norm)


def rand_case(rng, N, C, H, W, CO, KH, KW, G, layout, bias=True):
    Cg = C // G
    if layout == "NCHW":
        x = rng.standard_normal((N, C, H, W))
        w = rng.standard_normal((CO, Cg, KH, KW))
    else:
        x = rng.standard_normal((N, H, W, C))
        w = rng.standard_normal((CO, KH, KW, Cg))
    b = rng.standard_normal(CO) if bias else None
    return x, w, b


def to_nchw(x, w, layout):
    if layout == "NCHW":
        return x, w
    return np.transpose(x, (0, 3, 1, 2)), np.transpose(w, (0, 3, 1, 2))


def from_nchw(y, layout):
    return y if layout == "NCHW" else np.transpose(y, (0, 2, 3, 1))


# Geometries swept by several pins: (N, C, H, W, CO, KH, KW, s, p, d, G)
SWEEP = [
    (2, 3, 7, 6, 4, 3, 3, (1, 1), (1, 1), (1, 1), 1),
    (1, 4, 9, 8, 6, 3, 2, (2, 1), (1, 0), (1, 2), 2),
    (2, 4, 8, 9, 4, 3, 3, (2, 2), (2, 1), (2, 1), 4),
    (1, 6, 10, 7, 3, 2, 3, (3, 2), (0, 2), (2, 2), 3),
    (1, 2, 5, 5, 4, 1, 1, (1, 1), (0, 0), (1, 1), 1),
    (1, 2, 6, 6, 2, 1, 1, (2, 3), (1, 0), (1, 1), 2),
    (2, 8, 6, 5, 8, 3, 3, (1, 2), (2, 2), (2, 1), 8),
    (1, 3, 4, 11, 5, 4, 5, (1, 3), (2, 1), (1, 1), 1),
    (2, 16, 7, 8, 16, 3, 3, (1, 1), (1, 1), (1, 1), 4),   # groups of 4 channels, C_out = C
    (1, 16, 6, 7, 16, 3, 3, (1, 1), (1, 1), (1, 1), 2),   # groups of 8 channels
]


# ---------------------------------------------------------------- out size --

def brute_out_size(n, k, s, p, d):
    """Count window starts o >= 0 whose dilated window ends inside the padded
    extent [0, n + 2p); None if there are none."""
    count = 0
    o = 0
    while o * s + (k - 1) * d <= n + 2 * p - 1:
        count += 1
        o += 1
    return count or None


def test_out_size_matches_enumeration():
    for n, k, s, p, d in itertools.product(range(1, 10), range(1, 6), range(1, 5), range(0, 4), range(1, 4)):
        assert oracle.out_size(n, k, s, p, d) == brute_out_size(n, k, s, p, d), (n, k, s, p, d)


def test_out_size_rejects_bad_arguments():
    assert oracle.out_size(0, 3, 1, 0, 1) is None
    assert oracle.out_size(5, 0, 1, 0, 1) is None
    assert oracle.out_size(5, 3, 0, 0, 1) is None
    assert oracle.out_size(5, 3, 1, -1, 1) is None
    assert oracle.out_size(5, 3, 1, 0, 0) is None
    # Effective kernel (3-1)*3+1 = 7 does not fit 5 + 2*0.
    assert oracle.out_size(5, 3, 1, 0, 3) is None
    assert oracle.out_size(5, 3, 1, 1, 3) == 1


# ------------------------------------------------------------ hand-worked --

def test_hand_worked_forward():
    cases = json.load(open(GOLDEN))["forward"]
    for c in cases:
        x = np.array(c["x"], np.float64)
        w = np.array(c["w"], np.float64)
        b = None if c["bias"] is None else np.array(c["bias"], np.float64)
        y, _ = oracle.conv2d_forward(x, w, b, c["stride"], c["padding"], c["dilation"], c["groups"])
        np.testing.assert_array_equal(y, np.array(c["y"], np.float64), err_msg=c["name"])
        # The same case in NHWC must give the transposed answer.
        yt, _ = oracle.conv2d_forward(np.transpose(x, (0, 2, 3, 1)), np.transpose(w, (0, 2, 3, 1)), b,
                                      c["stride"], c["padding"], c["dilation"], c["groups"], layout="NHWC")
        np.testing.assert_array_equal(yt, np.transpose(np.array(c["y"], np.float64), (0, 2, 3, 1)))


def test_hand_worked_input_grad():
    cases = json.load(open(GOLDEN))["input_grad"]
    for c in cases:
        dy = np.array(c["dy"], np.float64)
        w = np.array(c["w"], np.float64)
        dx, _ = oracle.conv2d_input_grad(dy, w, c["input_shape"], c["stride"], c["padding"],
                                         c["dilation"], c["groups"])
        np.testing.assert_array_equal(dx, np.array(c["dx"], np.float64), err_msg=c["name"])
        idx = np.arange(dx.size)
        g, _ = oracle.conv2d_input_grad_at(dy, w, c["input_shape"], idx, c["stride"], c["padding"],
                                           c["dilation"], c["groups"])
        np.testing.assert_array_equal(g.reshape(dx.shape), dx, err_msg=c["name"])


# ------------------------------------------------- im2col + GEMM (brute) --

def im2col_gemm(x, w, b, stride, padding, dilation, G):
    """Forward by materialised columns and a plain matmul, NHWC.

    Columns follow burn-cubecl 0.22.0-pre.4 src/kernel/conv/im2col.rs,
    ``im2col``: columns[(n, oh, ow), (kh, kw, c)] = x[n, oh*s + kh*d - p,
    ow*s + kw*d - p, c], zero where that is outside the image, filled one
    tap-block at a time over the outputs [first, last) whose read lands
    inside (first = ceil(-base/s) for a negative base, last = min(O,
    (extent - 1 - base)/s + 1)).
    """
    N, H, W, C = x.shape
    CO, KH, KW, Cg = w.shape
    Mg = CO // G
    (sh, sw), (ph, pw), (dh, dw) = stride, padding, dilation
    OH = brute_out_size(H, KH, sh, ph, dh)
    OW = brute_out_size(W, KW, sw, pw, dw)
    y = np.zeros((N, OH, OW, CO))
    for g in range(G):
        xg = x[..., g * Cg:(g + 1) * Cg]
        cols = np.zeros((N, OH, OW, KH * KW * Cg))
        for tap in range(KH * KW):
            kh, kw = divmod(tap, KW)
            spans = []
            for k, d, p, s, ext, O in ((kh, dh, ph, sh, H, OH), (kw, dw, pw, sw, W, OW)):
                base = k * d - p
                first = 0 if base >= 0 else (-base + s - 1) // s
                reach = ext - 1 - base
                last = 0 if reach < 0 else min(O, reach // s + 1)
                spans.append((first, last, first * s + base, s))
            (fh, lh, sh0, s_h), (fw, lw, sw0, s_w) = spans
            if lh <= fh or lw <= fw:
                continue
            src = xg[:, sh0:sh0 + (lh - fh - 1) * s_h + 1:s_h, sw0:sw0 + (lw - fw - 1) * s_w + 1:s_w, :]
            cols[:, fh:lh, fw:lw, tap * Cg:(tap + 1) * Cg] = src
        wg = w[g * Mg:(g + 1) * Mg].reshape(Mg, KH * KW * Cg)  # [Mg, (kh, kw, c)]
        y[..., g * Mg:(g + 1) * Mg] = (cols.reshape(-1, KH * KW * Cg) @ wg.T).reshape(N, OH, OW, Mg)
    if b is not None:
        y += b
    return y


@pytest.mark.parametrize("case", SWEEP)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_forward_equals_im2col_gemm(case, layout):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(hash((case, layout)) % 2**32)
    x, w, b = rand_case(rng, N, C, H, W, CO, KH, KW, G, layout)
    y, norm = oracle.conv2d_forward(x, w, b, s, p, d, G, layout)
    xn, wn = to_nchw(x, w, layout)
    ref = im2col_gemm(np.transpose(xn, (0, 2, 3, 1)), np.transpose(wn, (0, 2, 3, 1)), b, s, p, d, G)
    ref = np.transpose(ref, (0, 3, 1, 2))
    assert rel_err(y, from_nchw(ref, layout), norm) < 1e-13


# ------------------------------------------------------- torch library --

@pytest.mark.parametrize("case", SWEEP)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_forward_matches_torch_cpu_fp64(case, layout):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(7 + hash((case, layout)) % 2**31)
    x, w, b = rand_case(rng, N, C, H, W, CO, KH, KW, G, layout)
    y, norm = oracle.conv2d_forward(x, w, b, s, p, d, G, layout)
    xn, wn = to_nchw(x, w, layout)
    ref = F.conv2d(torch.from_numpy(xn), torch.from_numpy(wn), torch.from_numpy(b),
                   stride=s, padding=p, dilation=d, groups=G).numpy()
    assert rel_err(y, from_nchw(ref, layout), norm) < 1e-13


@pytest.mark.parametrize("case", SWEEP)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_input_grad_matches_torch_cpu_fp64(case, layout):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(11 + hash((case, layout)) % 2**31)
    x, w, _ = rand_case(rng, N, C, H, W, CO, KH, KW, G, layout, bias=False)
    OH = brute_out_size(H, KH, s[0], p[0], d[0])
    OW = brute_out_size(W, KW, s[1], p[1], d[1])
    dy = rng.standard_normal((N, CO, OH, OW))
    _, wn = to_nchw(x, w, layout)
    ref = torch.nn.grad.conv2d_input((N, C, H, W), torch.from_numpy(wn), torch.from_numpy(dy),
                                     stride=s, padding=p, dilation=d, groups=G).numpy()
    dyl = from_nchw(dy, layout)
    dx, norm = oracle.conv2d_input_grad(dyl, w, x.shape, s, p, d, G, layout)
    assert rel_err(dx, from_nchw(ref, layout), norm) < 1e-13


# ------------------------------------------------------------- identities --

@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_impulse_reproduces_flipped_weights(layout):
    N, C, H, W, CO, KH, KW, G = 2, 4, 9, 8, 6, 3, 2, 2
    s, p, d = (2, 1), (1, 1), (1, 2)
    rng = np.random.default_rng(3)
    _, w, _ = rand_case(rng, N, C, H, W, CO, KH, KW, G, layout, bias=False)
    n0, c0, h0, w0 = 1, 3, 4, 3
    xn = np.zeros((N, C, H, W))
    xn[n0, c0, h0, w0] = 1.0
    x = from_nchw(xn, layout)
    y, _ = oracle.conv2d_forward(x, w, None, s, p, d, G, layout)
    OH, OW = brute_out_size(H, KH, s[0], p[0], d[0]), brute_out_size(W, KW, s[1], p[1], d[1])
    _, wn = to_nchw(x, w, layout)
    Cg, Mg = C // G, CO // G
    g = c0 // Cg
    expect = np.zeros((N, CO, OH, OW))
    # Enumerate taps and place each weight on the output that read the impulse.
    for co in range(g * Mg, (g + 1) * Mg):
        for kh in range(KH):
            th = h0 + p[0] - kh * d[0]
            if th < 0 or th % s[0] or th // s[0] >= OH:
                continue
            for kw in range(KW):
                tw = w0 + p[1] - kw * d[1]
                if tw < 0 or tw % s[1] or tw // s[1] >= OW:
                    continue
                expect[n0, co, th // s[0], tw // s[1]] = wn[co, c0 - g * Cg, kh, kw]
    np.testing.assert_array_equal(y, from_nchw(expect, layout))
    assert np.count_nonzero(expect) > 0


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_pointwise_is_matmul(layout):
    rng = np.random.default_rng(5)
    N, C, H, W, CO = 2, 5, 4, 3, 7
    x, w, _ = rand_case(rng, N, C, H, W, CO, 1, 1, 1, layout, bias=False)
    y, norm = oracle.conv2d_forward(x, w, None, 1, 0, 1, 1, layout)
    xn, wn = to_nchw(x, w, layout)
    W2 = wn[:, :, 0, 0]  # [CO, C]
    ref = np.zeros((N, CO, H, W))
    for n in range(N):
        ref[n] = (W2 @ xn[n].reshape(C, H * W)).reshape(CO, H, W)
    assert rel_err(y, from_nchw(ref, layout), norm) < 1e-14


def test_bias_is_added_once_per_channel():
    rng = np.random.default_rng(9)
    x, w, b = rand_case(rng, 2, 4, 6, 6, 6, 3, 3, 2, "NCHW")
    y1, _ = oracle.conv2d_forward(x, w, b, 1, 1, 1, 2)
    y0, _ = oracle.conv2d_forward(x, w, None, 1, 1, 1, 2)
    # Far from cancellation, y1 - y0 recovers b to fp64 rounding of y1.
    np.testing.assert_allclose(y1 - y0, np.broadcast_to(b[None, :, None, None], y1.shape),
                               rtol=0, atol=1e-13 * (1 + np.abs(y1).max()))
    # And with x = 0 the output is exactly b.
    yz, nz = oracle.conv2d_forward(np.zeros_like(x), w, b, 1, 1, 1, 2)
    np.testing.assert_array_equal(yz, np.broadcast_to(b[None, :, None, None], yz.shape))
    np.testing.assert_array_equal(nz, np.broadcast_to(np.abs(b)[None, :, None, None], nz.shape))


def test_groups_split_into_independent_convolutions():
    rng = np.random.default_rng(13)
    N, C, H, W, CO, G = 2, 6, 7, 5, 9, 3
    x, w, b = rand_case(rng, N, C, H, W, CO, 3, 2, G, "NCHW")
    y, norm = oracle.conv2d_forward(x, w, b, (2, 1), (1, 0), (1, 2), G)
    Cg, Mg = C // G, CO // G
    parts = []
    for g in range(G):
        yg, _ = oracle.conv2d_forward(x[:, g * Cg:(g + 1) * Cg], w[g * Mg:(g + 1) * Mg], b[g * Mg:(g + 1) * Mg],
                                      (2, 1), (1, 0), (1, 2), 1)
        parts.append(yg)
    np.testing.assert_array_equal(y, np.concatenate(parts, axis=1))


@pytest.mark.parametrize("dil", [1, 2])
def test_depthwise_is_per_channel_correlate2d(dil):
    rng = np.random.default_rng(17 + dil)
    N, C, H, W, K, P = 2, 5, 9, 8, 3, 2
    x = rng.standard_normal((N, H, W, C))
    w = rng.standard_normal((C, K, K, 1))
    y, norm = oracle.conv2d_forward(x, w, None, 1, P, dil, C, "NHWC")
    for n in range(N):
        for c in range(C):
            ker = np.zeros(((K - 1) * dil + 1,) * 2)
            ker[::dil, ::dil] = w[c, :, :, 0]
            img = np.pad(x[n, :, :, c], P)
            ref = signal.correlate2d(img, ker, mode="valid")
            assert rel_err(y[n, :, :, c], ref, norm[n, :, :, c]) < 1e-14


def test_linearity():
    rng = np.random.default_rng(19)
    x1, w, _ = rand_case(rng, 2, 4, 7, 7, 4, 3, 3, 2, "NHWC", bias=False)
    x2 = rng.standard_normal(x1.shape)
    a, b = 0.75, -2.5
    y, _ = oracle.conv2d_forward(a * x1 + b * x2, w, None, 2, 1, 1, 2, "NHWC")
    y1, n1 = oracle.conv2d_forward(x1, w, None, 2, 1, 1, 2, "NHWC")
    y2, n2 = oracle.conv2d_forward(x2, w, None, 2, 1, 1, 2, "NHWC")
    assert rel_err(y, a * y1 + b * y2, abs(a) * n1 + abs(b) * n2) < 1e-14


@pytest.mark.parametrize("case", SWEEP)
def test_adjoint_identity(case):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(23)
    x, w, _ = rand_case(rng, N, C, H, W, CO, KH, KW, G, "NHWC", bias=False)
    y, _ = oracle.conv2d_forward(x, w, None, s, p, d, G, "NHWC")
    dy = rng.standard_normal(y.shape)
    dx, _ = oracle.conv2d_input_grad(dy, w, x.shape, s, p, d, G, "NHWC")
    lhs, rhs = float(np.sum(y * dy)), float(np.sum(x * dx))
    scale = float(np.sum(np.abs(y * dy))) + float(np.sum(np.abs(x * dx)))
    assert abs(lhs - rhs) <= 1e-12 * scale


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_pointwise_input_grad_is_dy_times_w(layout):
    rng = np.random.default_rng(29)
    N, C, H, W, CO = 2, 5, 3, 4, 6
    x, w, _ = rand_case(rng, N, C, H, W, CO, 1, 1, 1, layout, bias=False)
    dyn = rng.standard_normal((N, CO, H, W))
    dx, norm = oracle.conv2d_input_grad(from_nchw(dyn, layout), w, x.shape, 1, 0, 1, 1, layout)
    _, wn = to_nchw(x, w, layout)
    W2 = wn[:, :, 0, 0]  # [CO, C]
    ref = np.einsum("nohw,oc->nchw", dyn, W2)
    assert rel_err(dx, from_nchw(ref, layout), norm) < 1e-14


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_input_grad_impulse(layout):
    N, C, H, W, CO, KH, KW, G = 1, 4, 9, 10, 6, 3, 3, 2
    s, p, d = (2, 2), (1, 2), (2, 1)
    rng = np.random.default_rng(31)
    x, w, _ = rand_case(rng, N, C, H, W, CO, KH, KW, G, layout, bias=False)
    OH, OW = brute_out_size(H, KH, s[0], p[0], d[0]), brute_out_size(W, KW, s[1], p[1], d[1])
    n0, co0, oh0, ow0 = 0, 4, 2, 3
    dyn = np.zeros((N, CO, OH, OW))
    dyn[n0, co0, oh0, ow0] = 1.0
    dx, _ = oracle.conv2d_input_grad(from_nchw(dyn, layout), w, x.shape, s, p, d, G, layout)
    _, wn = to_nchw(x, w, layout)
    Cg, Mg = C // G, CO // G
    g = co0 // Mg
    expect = np.zeros((N, C, H, W))
    for c in range(Cg):
        for kh in range(KH):
            ih = oh0 * s[0] - p[0] + kh * d[0]
            for kw in range(KW):
                iw = ow0 * s[1] - p[1] + kw * d[1]
                if 0 <= ih < H and 0 <= iw < W:
                    expect[n0, g * Cg + c, ih, iw] = wn[co0, c, kh, kw]
    np.testing.assert_array_equal(dx, from_nchw(expect, layout))


def test_input_grad_coverage_edges():
    rng = np.random.default_rng(37)
    # H = 56, K = 3, S = 2, P = 1: OH = 28, and the last input row 55 is read
    # by output row 27 through kh = 2 (27*2 - 1 + 2 = 55), so its gradient
    # is nonzero; an extent computed as (OH-1)*S + K - 2P = 55 would miss it.
    N, C, H, W, CO = 1, 2, 56, 8, 3
    w = rng.standard_normal((CO, 3, 3, C))
    dy = rng.standard_normal((N, 28, 4, CO))
    dx, _ = oracle.conv2d_input_grad(dy, w, (N, H, W, C), 2, 1, 1, 1, "NHWC")
    assert np.all(dx[:, 55] != 0)
    # H = 6, K = 3, S = 2, P = 0: OH = 2, windows cover rows 0..4, so row 5
    # is never read and its gradient is exactly zero.
    w = rng.standard_normal((CO, 3, 3, C))
    dy = rng.standard_normal((N, 2, 2, CO))
    dx, norm = oracle.conv2d_input_grad(dy, w, (N, 6, 6, C), 2, 0, 1, 1, "NHWC")
    assert np.all(dx[:, 5] == 0) and np.all(dx[:, :, 5] == 0) and np.all(norm[:, 5] == 0)
    assert np.all(dx[:, 4, :5] != 0)


@pytest.mark.parametrize("case", SWEEP[:4])
def test_sampled_functions_agree_with_full(case):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(41)
    x, w, b = rand_case(rng, N, C, H, W, CO, KH, KW, G, "NHWC")
    y, norm = oracle.conv2d_forward(x, w, b, s, p, d, G, "NHWC")
    idx = rng.choice(y.size, size=min(50, y.size), replace=False)
    v, nv = oracle.conv2d_forward_at(x, w, b, idx, s, p, d, G, "NHWC")
    np.testing.assert_array_equal(v, y.reshape(-1)[idx])
    np.testing.assert_array_equal(nv, norm.reshape(-1)[idx])
    dy = rng.standard_normal(y.shape)
    dx, dnorm = oracle.conv2d_input_grad(dy, w, x.shape, s, p, d, G, "NHWC")
    idx = np.arange(dx.size)
    g, gn = oracle.conv2d_input_grad_at(dy, w, x.shape, idx, s, p, d, G, "NHWC")
    assert rel_err(g, dx.reshape(-1), dnorm.reshape(-1)) < 1e-13
    np.testing.assert_allclose(gn, dnorm.reshape(-1), rtol=1e-13, atol=0)


def test_oracle_rejects_invalid_geometry():
    x = np.zeros((1, 4, 5, 5))
    with pytest.raises(ValueError):
        oracle.conv2d_forward(x, np.zeros((3, 4, 3, 3)), None, 1, 0, 1, 2)  # 3 % 2 != 0
    with pytest.raises(ValueError):
        oracle.conv2d_forward(x, np.zeros((4, 4, 7, 7)), None, 1, 0, 1, 1)  # kernel too big
    with pytest.raises(ValueError):
        oracle.conv2d_forward_at(x, np.zeros((4, 4, 3, 3)), None, [10**6], 1, 0, 1, 1)
