"""The weight gradient's entry point that allocates nothing
(conv_bwd_dw_noalloc) against the one that takes a workspace (conv_bwd_dw),
through the C ABI.

Two calls in a row on each path the automatic selection takes (the matrix-
core implicit GEMM for NHWC bf16, the generic kernel for NCHW fp32), the
second with a smaller input, so the second runs on the scratch the first
left behind.  Each result must equal conv_bwd_dw's bit for bit (the same
kernels and plan) and match the fp64 oracle within the dtype's normalised
tolerance.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_conv2d_amd as cm
import oracle
from helpers import TOL, f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# (N, C, H, W, C_out, K, stride, pad, dil, groups): larger first, then smaller.
CALLS = {
    ("NHWC", torch.bfloat16): [(4, 64, 28, 28, 96, 3, 2, 1, 1, 1), (2, 32, 9, 11, 24, 3, 1, 2, 2, 1)],
    ("NCHW", torch.float32): [(3, 12, 17, 15, 10, 3, 1, 1, 1, 2), (1, 4, 7, 6, 6, 2, 2, 0, 1, 1)],
}


def draw(seed, shape, dtype):
    gen = torch.Generator().manual_seed(seed)
    return torch.empty(shape).uniform_(-1, 1, generator=gen).to(dtype)


@pytest.mark.parametrize("layout,dtype", list(CALLS))
def test_noalloc_equals_workspace_entry_point_twice(layout, dtype):
    lay = cm.CONV_NHWC if layout == "NHWC" else cm.CONV_NCHW
    dt = cm.CONV_BF16 if dtype == torch.bfloat16 else cm.CONV_F32
    for k, (N, C, H, W, CO, K, s, p, d, G) in enumerate(CALLS[(layout, dtype)]):
        path = cm.conv_path_name(cm.conv_select_path(2, N, C, H, W, CO, K, K, s, s, p, p, d, d, G, lay, dt))
        print(f"call {k}: {layout} {dtype} N={N} C={C} H={H} W={W} C_out={CO} K={K} s={s} p={p} "
              f"d={d} G={G} path {path}", flush=True)
        OH = oracle.out_size(H, K, s, p, d)
        OW = oracle.out_size(W, K, s, p, d)
        xs = (N, H, W, C) if layout == "NHWC" else (N, C, H, W)
        ys = (N, OH, OW, CO) if layout == "NHWC" else (N, CO, OH, OW)
        ws = (CO, K, K, C // G) if layout == "NHWC" else (CO, C // G, K, K)
        x, dy = draw(100 + k, xs, dtype), draw(200 + k, ys, dtype)
        xd, dyd = x.to(DEV), dy.to(DEV)
        geom = (N, C, H, W, CO, K, K, s, s, p, p, d, d, G, lay, dt)
        got = torch.full(ws, float("nan"), dtype=dtype, device=DEV)
        cm.conv_bwd_dw_noalloc(xd, dyd, got, *geom)
        need = cm.conv_bwd_dw_workspace_size(*geom, cm.PATHS["auto"])
        work = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        want = torch.full(ws, float("nan"), dtype=dtype, device=DEV)
        cm.conv_bwd_dw(xd, dyd, want, work, work.numel(), *geom)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), want.cpu())
        ref, norm = oracle.conv2d_weight_grad(x, dy, ws, s, p, d, G, layout)
        err = oracle.max_normalised_error(f64(got.cpu()), ref, norm)
        print(f"  normalised error {err:.3e}", flush=True)
        assert err <= TOL[dtype], err
