"""Tensors past 2 GiB, through the C ABI, against the fp64 oracle.

A 3x3, 16 -> 16 channel layer over 5 images of 4096 x 4096 (NHWC bf16): x,
y, dy and dx each hold 2.68 GB, past the 2^31 bytes where the band and
input-gradient implicit GEMMs decline.  The forward runs the automatic path
(the implicit GEMM with int64 image offsets) and the generic direct kernel,
the input gradient the automatic path (the generic gather).  Images are
independent, so the oracle recomputes sampled outputs of the first, second
and last images from those images alone: the last image's outputs sit past
2^31 bytes from the base.  Inputs are drawn on the device from a seeded
generator (uniform [-1, 1]); the oracle reads the same bytes copied back.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_conv2d_amd as cm
import oracle
from helpers import TOL, record

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF16 = torch.bfloat16
N, H, W, C, CO, K = 5, 4096, 4096, 16, 16, 3
GEO = dict(stride=1, padding=1, dilation=1, groups=1, layout="NHWC")
SAMPLES = 3000


def device_uniform(seed, shape):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    return torch.empty(shape, device=DEV).uniform_(-1, 1, generator=gen).to(BF16)


@pytest.fixture(scope="module")
def tensors():
    x = device_uniform(1, (N, H, W, C))
    w = device_uniform(2, (CO, K, K, C))
    b = device_uniform(3, (CO,))
    assert x.numel() * 2 > (1 << 31)
    yield x, w, b
    del x
    torch.cuda.empty_cache()


def sampled_error(got_img, ref_vals, norm, idx):
    g = got_img.reshape(-1)[torch.from_numpy(idx)].double().numpy()
    return oracle.max_normalised_error(g, ref_vals, norm)


@pytest.mark.parametrize("path", ["auto", "direct"])
def test_forward_past_2gib(tensors, path):
    x, w, b = tensors
    chosen = cm.conv_path_name(cm.conv_select_path(0, N, C, H, W, CO, K, K, 1, 1, 1, 1, 1, 1, 1,
                                                   cm.CONV_NHWC, cm.CONV_BF16))
    print(f"forward N={N} {H}x{W} C={C}->{CO} 3x3 path {path} (auto takes {chosen})", flush=True)
    assert chosen not in ("igemm_band",)
    y = cm.conv2d(x, w, b, path=path, **GEO)
    torch.cuda.synchronize()
    assert y.numel() * 2 > (1 << 31)
    wc, bc = w.cpu(), b.cpu()
    rng = np.random.default_rng(5)
    worst = 0.0
    for n in (0, 1, N - 1):
        idx = rng.choice(H * W * CO, size=SAMPLES, replace=False).astype(np.int64)
        idx[:4] = [0, CO - 1, H * W * CO - CO, H * W * CO - 1]  # corners of the image
        vals, norm = oracle.conv2d_forward_at(x[n:n + 1].cpu(), wc, bc, idx, **GEO)
        err = sampled_error(y[n].cpu(), vals, norm, idx)
        worst = max(worst, err)
    record(f"forward_3x3_c16_k16_4096x4096_n5_bf16_nhwc[{path}]", worst, TOL[BF16],
           path=chosen if path == "auto" else path, compared=f"{SAMPLES} outputs of images 0, 1, {N - 1}")
    assert worst <= TOL[BF16], worst


def test_input_grad_past_2gib(tensors):
    _, w, _ = tensors
    dy = device_uniform(4, (N, H, W, CO))
    chosen = cm.conv_path_name(cm.conv_select_path(1, N, C, H, W, CO, K, K, 1, 1, 1, 1, 1, 1, 1,
                                                   cm.CONV_NHWC, cm.CONV_BF16))
    print(f"input gradient N={N} {H}x{W} C={C}<-{CO} 3x3 path {chosen}", flush=True)
    assert chosen == "dx_gather"
    dx = cm.conv2d_input_grad(dy, w, (N, H, W, C), **GEO)
    torch.cuda.synchronize()
    wc = w.cpu()
    rng = np.random.default_rng(6)
    worst = 0.0
    for n in (0, 1, N - 1):
        idx = rng.choice(H * W * C, size=SAMPLES, replace=False).astype(np.int64)
        idx[:4] = [0, C - 1, H * W * C - C, H * W * C - 1]
        vals, norm = oracle.conv2d_input_grad_at(dy[n:n + 1].cpu(), wc, (1, H, W, C), idx, **GEO)
        err = sampled_error(dx[n].cpu(), vals, norm, idx)
        worst = max(worst, err)
    record("dx_3x3_c16_k16_4096x4096_n5_bf16_nhwc[auto]", worst, TOL[BF16], path=chosen,
           compared=f"{SAMPLES} outputs of images 0, 1, {N - 1}")
    assert worst <= TOL[BF16], worst
    del dy, dx
