"""Pins of the oracle's normalisers and of its error metric (CPU only).

Every parity bound in the GPU tests is a ratio ``|gpu - ref| / norm``, with
``norm`` the oracle's second output: ``|b| + sum |x*w|`` over the taps that
land inside the image for the forward (``sum |dy*w|`` for the input gradient,
``sum |dy*x|`` for the weight gradient), as the tolerance is stated per output
in the method's accuracy requirement.  Since ``|x*w| = |x|*|w|``, each
normaliser is the same convolution taken over absolute values; torch's CPU
fp64 library convolutions of ``|x|`` and ``|w|`` fix it independently of the
oracle.  A second identity ties each normaliser to the oracle's own (already
pinned) value path: ``norm(x, w, b) == value(|x|, |w|, |b|)``.

``max_normalised_error`` is fixed on hand-built arrays whose answer is known.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from test_oracle_pins import SWEEP, from_nchw, rand_case, to_nchw
from test_oracle_pins_next import SWEEP_1D, SWEEP_DW, SWEEP_T, rand_1d, rand_dw, rand_t, to_nchw_y, \
    w_to_oihw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
RTOL = 1e-13


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a))


# ------------------------------------------------------------ forward norm --

@pytest.mark.parametrize("case", SWEEP)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("bias", [True, False])
def test_forward_norm_is_conv_of_absolute_values(case, layout, bias):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(101)
    x, w, b = rand_case(rng, N, C, H, W, CO, KH, KW, G, layout, bias=bias)
    _, norm = oracle.conv2d_forward(x, w, b, s, p, d, G, layout)
    xn, wn = to_nchw(x, w, layout)
    ref = F.conv2d(t(np.abs(xn)), t(np.abs(wn)), None if b is None else t(np.abs(b)), s, p, d, G)
    ref = from_nchw(ref.numpy(), layout)
    assert norm.shape == ref.shape
    np.testing.assert_allclose(norm, ref, rtol=RTOL, atol=0)


@pytest.mark.parametrize("case", SWEEP)
def test_forward_norm_is_the_value_of_absolute_inputs(case):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(102)
    x, w, b = rand_case(rng, N, C, H, W, CO, KH, KW, G, "NHWC")
    _, norm = oracle.conv2d_forward(x, w, b, s, p, d, G, "NHWC")
    y_abs, _ = oracle.conv2d_forward(np.abs(x), np.abs(w), np.abs(b), s, p, d, G, "NHWC")
    np.testing.assert_array_equal(norm, y_abs)


@pytest.mark.parametrize("case", SWEEP[:4])
def test_sampled_forward_norm_is_conv_of_absolute_values(case):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(103)
    x, w, b = rand_case(rng, N, C, H, W, CO, KH, KW, G, "NCHW")
    ref = F.conv2d(t(np.abs(x)), t(np.abs(w)), t(np.abs(b)), s, p, d, G).numpy().reshape(-1)
    idx = rng.choice(ref.size, size=min(40, ref.size), replace=False)
    _, nv = oracle.conv2d_forward_at(x, w, b, idx, s, p, d, G, "NCHW")
    np.testing.assert_allclose(nv, ref[idx], rtol=RTOL, atol=0)


def test_hand_worked_forward_norms():
    # The hand-worked examples with every input replaced by its absolute
    # value: their normaliser is the forward of |x|, |w|, |b|.
    for c in json.load(open(GOLDEN))["forward"]:
        x = np.array(c["x"], np.float64)
        w = np.array(c["w"], np.float64)
        b = None if c["bias"] is None else np.array(c["bias"], np.float64)
        _, norm = oracle.conv2d_forward(x, w, b, c["stride"], c["padding"], c["dilation"], c["groups"])
        ref = F.conv2d(t(np.abs(x)), t(np.abs(w)), None if b is None else t(np.abs(b)), c["stride"],
                       c["padding"], c["dilation"], c["groups"]).numpy()
        np.testing.assert_allclose(norm, ref, rtol=RTOL, atol=0, err_msg=c["name"])


# ----------------------------------------------------- input-gradient norm --

@pytest.mark.parametrize("case", SWEEP)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_input_grad_norm_is_conv_input_of_absolute_values(case, layout):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(104)
    x, w, _ = rand_case(rng, N, C, H, W, CO, KH, KW, G, layout, bias=False)
    y, _ = oracle.conv2d_forward(x, w, None, s, p, d, G, layout)
    dy = rng.standard_normal(y.shape)
    _, norm = oracle.conv2d_input_grad(dy, w, x.shape, s, p, d, G, layout)
    xn, wn = to_nchw(x, w, layout)
    dyn = dy if layout == "NCHW" else np.transpose(dy, (0, 3, 1, 2))
    ref = torch.nn.grad.conv2d_input(xn.shape, t(np.abs(wn)), t(np.abs(dyn)), s, p, d, G).numpy()
    ref = from_nchw(ref, layout)
    assert norm.shape == ref.shape
    np.testing.assert_allclose(norm, ref, rtol=RTOL, atol=0)
    # Per element, the gather form's normaliser agrees.
    idx = np.arange(norm.size)
    _, gn = oracle.conv2d_input_grad_at(dy, w, x.shape, idx, s, p, d, G, layout)
    np.testing.assert_allclose(gn, ref.reshape(-1), rtol=RTOL, atol=0)


@pytest.mark.parametrize("case", SWEEP)
def test_input_grad_norm_is_the_value_of_absolute_inputs(case):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(105)
    x, w, _ = rand_case(rng, N, C, H, W, CO, KH, KW, G, "NHWC", bias=False)
    y, _ = oracle.conv2d_forward(x, w, None, s, p, d, G, "NHWC")
    dy = rng.standard_normal(y.shape)
    _, norm = oracle.conv2d_input_grad(dy, w, x.shape, s, p, d, G, "NHWC")
    v_abs, _ = oracle.conv2d_input_grad(np.abs(dy), np.abs(w), x.shape, s, p, d, G, "NHWC")
    np.testing.assert_allclose(norm, v_abs, rtol=RTOL, atol=0)


# ---------------------------------------------------- weight-gradient norm --

@pytest.mark.parametrize("case", SWEEP_DW)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_weight_grad_norm_is_conv_weight_of_absolute_values(case, layout):
    N, C, H, W, CO, KH, KW, s, p, d, G = case
    rng = np.random.default_rng(106)
    x, dy, w_shape, x_nchw, dy_nchw = rand_dw(rng, N, C, H, W, CO, KH, KW, s, p, d, G, layout)
    _, norm = oracle.conv2d_weight_grad(x, dy, w_shape, s, p, d, G, layout)
    ref = torch.nn.grad.conv2d_weight(t(np.abs(x_nchw)), (CO, C // G, KH, KW), t(np.abs(dy_nchw)),
                                      s, p, d, G).numpy()
    np.testing.assert_allclose(w_to_oihw(norm, layout), ref, rtol=RTOL, atol=0)


# ------------------------------------------------------------- conv1d norm --

@pytest.mark.parametrize("case", SWEEP_1D)
@pytest.mark.parametrize("layout", ["NCL", "NLC"])
def test_conv1d_norm_is_conv_of_absolute_values(case, layout):
    N, C, L, CO, K, s, p, d, G = case
    rng = np.random.default_rng(107)
    x, w, b, x_ncl, w_oik = rand_1d(rng, N, C, L, CO, K, G, layout)
    _, norm = oracle.conv1d_forward(x, w, b, s, p, d, G, layout)
    ref = F.conv1d(t(np.abs(x_ncl)), t(np.abs(w_oik)), t(np.abs(b)), s, p, d, G).numpy()
    if layout == "NLC":
        ref = np.transpose(ref, (0, 2, 1))
    np.testing.assert_allclose(norm, ref, rtol=RTOL, atol=0)


# ---------------------------------------------------- transposed-conv norm --

@pytest.mark.parametrize("case", SWEEP_T)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_conv_transpose2d_norm_is_conv_transpose_of_absolute_values(case, layout):
    N, CI, H, W, CO, KH, KW, s, p, op, d, G = case
    rng = np.random.default_rng(108)
    x, w, b, x_nchw, w_iokk = rand_t(rng, N, CI, H, W, CO, KH, KW, G, layout)
    _, norm = oracle.conv_transpose2d(x, w, b, s, p, op, d, G, layout)
    ref = F.conv_transpose2d(t(np.abs(x_nchw)), t(np.abs(w_iokk)), t(np.abs(b)), stride=s, padding=p,
                             output_padding=op, groups=G, dilation=d).numpy()
    np.testing.assert_allclose(to_nchw_y(norm, layout), ref, rtol=RTOL, atol=0)


# ------------------------------------------------------ max_normalised_error --

def test_error_of_equal_arrays_is_zero():
    rng = np.random.default_rng(109)
    ref = rng.standard_normal((3, 5))
    norm = np.abs(rng.standard_normal((3, 5))) + 0.1
    norm[1, 2] = 0.0  # a zero normaliser with an equal value is fine
    assert oracle.max_normalised_error(ref.copy(), ref, norm) == 0.0


def test_error_is_the_largest_ratio_not_the_largest_difference():
    ref = np.zeros(6)
    got = np.zeros(6)
    norm = np.ones(6)
    got[1], norm[1] = 1.0, 100.0     # difference 1.0, ratio 0.01
    got[4], norm[4] = -0.1, 0.125    # difference 0.1 (below the reference), ratio 0.8
    got[5], norm[5] = 0.25, 1.0      # ratio 0.25
    assert oracle.max_normalised_error(got, ref, norm) == 0.8


def test_error_of_one_planted_difference():
    rng = np.random.default_rng(110)
    ref = rng.standard_normal((4, 4, 3))
    norm = np.full(ref.shape, 2.0)
    got = ref.copy()
    got[2, 1, 0] += 0.5
    assert oracle.max_normalised_error(got, ref, norm) == pytest.approx(0.25, rel=1e-15)
    # The same difference measured against the reference in the other direction.
    assert oracle.max_normalised_error(ref, got, norm) == pytest.approx(0.25, rel=1e-15)


def test_error_at_a_zero_normaliser_is_infinite():
    ref = np.array([1.0, 0.0, 2.0])
    got = np.array([1.0, 1e-300, 2.0])
    norm = np.array([1.0, 0.0, 1.0])
    assert oracle.max_normalised_error(got, ref, norm) == float("inf")


def test_error_of_empty_arrays_is_zero():
    e = np.zeros((0, 3))
    assert oracle.max_normalised_error(e, e, e) == 0.0


def test_error_takes_any_float_dtype():
    ref = np.array([1.0, 2.0, 3.0])
    got = torch.tensor([1.0, 2.5, 3.0], dtype=torch.float32).numpy()
    norm = np.array([1.0, 2.0, 1.0])
    assert oracle.max_normalised_error(got, ref, norm) == 0.25
