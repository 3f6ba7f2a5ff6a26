"""A seeded random sweep through automatic path selection.

Each geometry from random_cases runs with path "auto" -- whatever kernel the
library picks for it -- and is compared with the fp64 oracle element by
element, at the tolerance of its dtype.  The geometry is printed before the
GPU call so that a failure names its case.
"""
import pytest
import torch

import convolution_implicit_gemm_conv2d_amd as cm
import random_cases
from helpers import TOL, dx_error, fwd_error, gpu_dx, gpu_fwd, out_shape, random_case, random_dy

pytestmark = pytest.mark.gpu
CASES = random_cases.cases()
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.mark.parametrize("i", range(len(CASES)), ids=[random_cases.label(c) for c in CASES])
def test_auto_path_matches_oracle(i):
    c = CASES[i]
    dtype = DT[c["dtype"]]
    geo = dict(stride=c["stride"], padding=c["pad"], dilation=c["dil"], groups=c["groups"],
               layout=c["layout"])
    path = cm.conv_path_name(cm.conv_select_path(
        c["kind"] == "dx", c["N"], c["C"], c["H"], c["W"], c["CO"], c["KH"], c["KW"], *c["stride"],
        *c["pad"], *c["dil"], c["groups"], 1 if c["layout"] == "NHWC" else 0, 1 if c["dtype"] == "bf16" else 0))
    print(f"case {i}: {random_cases.label(c)} -> {path}", flush=True)
    x, w, b = random_case(1000 + i, c["N"], c["C"], c["H"], c["W"], c["CO"], c["KH"], c["KW"],
                          c["groups"], c["layout"], dtype, bias=c["kind"] == "fwd")
    if c["kind"] == "fwd":
        y = gpu_fwd(x, w, b, geo)
        err = fwd_error(x, w, b, y, geo)
    else:
        dy = random_dy(2000 + i, out_shape(x.shape, w.shape, geo), dtype)
        dx = gpu_dx(dy, w, tuple(x.shape), geo)
        err = dx_error(dy, w, tuple(x.shape), dx, geo)
    assert err <= TOL[dtype], (path, err)
