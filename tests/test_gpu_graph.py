"""The hot path under HIP graph capture.

The library allocates nothing and issues no memset, so a caller can capture
its launches in a graph and replay them.  The five hot-path kernels (and the
small-group matrix-core kernel and the weight gradient's two) are captured on one torch CUDA graph at small sizes;
each replay follows eager work and cleared outputs, and must reproduce the
eager results bit for bit (every kernel is deterministic).
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_conv2d_amd as cm
import oracle
from helpers import TOL, f64, random_case, random_dy

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
DEV = torch.device("cuda:0")


def cases():
    """(name, call(out), out) for a forward of each path, dx and dw."""
    out = []
    geo = dict(stride=1, padding=1, dilation=1, groups=1, layout="NCHW")
    x, w, b = random_case(0, 2, 3, 16, 16, 8, 3, 3, 1, "NCHW", torch.float32)
    x, w, b = x.to(DEV), w.to(DEV), b.to(DEV)
    y = torch.empty(2, 8, 16, 16, device=DEV)
    out.append(("direct", lambda o, x=x, w=w, b=b: cm.conv2d(x, w, b, out=o, path="direct", **geo), y))

    nhwc = dict(stride=1, dilation=1, layout="NHWC")
    x, w, _ = random_case(1, 2, 256, 14, 14, 64, 1, 1, 1, "NHWC", BF16, bias=False)
    x, w = x.to(DEV), w.to(DEV)
    out.append(("pointwise", lambda o, x=x, w=w: cm.conv2d(x, w, None, padding=0, groups=1, out=o,
                                                           path="pointwise", **nhwc),
                torch.empty(2, 14, 14, 64, device=DEV, dtype=BF16)))

    x, w, b = random_case(2, 2, 64, 14, 14, 64, 3, 3, 1, "NHWC", BF16)
    x, w, b = x.to(DEV), w.to(DEV), b.to(DEV)
    out.append(("igemm_band", lambda o, x=x, w=w, b=b: cm.conv2d(x, w, b, padding=1, groups=1, out=o,
                                                                 path="igemm_band", **nhwc),
                torch.empty(2, 14, 14, 64, device=DEV, dtype=BF16)))

    x, w, _ = random_case(3, 2, 256, 14, 14, 256, 3, 3, 256, "NHWC", BF16, bias=False)
    x, w = x.to(DEV), w.to(DEV)
    out.append(("depthwise", lambda o, x=x, w=w: cm.conv2d(x, w, None, padding=2, groups=256, out=o,
                                                           path="depthwise", stride=1, dilation=2,
                                                           layout="NHWC"),
                torch.empty(2, 14, 14, 256, device=DEV, dtype=BF16)))

    x, w, b = random_case(10, 2, 64, 14, 14, 64, 3, 3, 16, "NHWC", BF16)  # groups of 4: matrix core
    x, w, b = x.to(DEV), w.to(DEV), b.to(DEV)
    out.append(("small groups", lambda o, x=x, w=w, b=b: cm.conv2d(x, w, b, padding=1, groups=16, out=o,
                                                                   path="depthwise", stride=1, dilation=1,
                                                                   layout="NHWC"),
                torch.empty(2, 14, 14, 64, device=DEV, dtype=BF16)))

    _, w, _ = random_case(4, 2, 128, 14, 14, 256, 3, 3, 1, "NHWC", BF16, bias=False)
    dy = random_dy(5, (2, 7, 7, 256), BF16).to(DEV)
    w = w.to(DEV)
    out.append(("dx_igemm", lambda o, dy=dy, w=w: cm.conv2d_input_grad(
        dy, w, (2, 14, 14, 128), stride=2, padding=1, out=o, path="dx_igemm"),
        torch.empty(2, 14, 14, 128, device=DEV, dtype=BF16)))

    x, _, _ = random_case(6, 2, 64, 14, 14, 64, 3, 3, 1, "NHWC", BF16, bias=False)
    dyw = random_dy(7, (2, 14, 14, 64), BF16).to(DEV)
    x = x.to(DEV)
    ws_bytes = cm.conv_bwd_dw_workspace_size(2, 64, 14, 14, 64, 3, 3, 1, 1, 1, 1, 1, 1, 1,
                                             cm.CONV_NHWC, cm.CONV_BF16, cm.PATHS["dw_igemm"])
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    out.append(("dw_igemm", lambda o, x=x, dyw=dyw, ws=ws: cm.conv2d_weight_grad(
        x, dyw, (64, 3, 3, 64), padding=1, path="dw_igemm", out=o, workspace=ws),
        torch.empty(64, 3, 3, 64, device=DEV, dtype=BF16)))
    return out


def test_hot_path_graph_replays_match_eager():
    cs = cases()
    eager = []
    for name, call, o in cs:
        call(o)
        eager.append(o.clone())
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _, call, o in cs:
            call(o)
    torch.cuda.synchronize()

    for rep in range(3):
        # Eager work between replays: the same calls into scratch outputs,
        # then the captured outputs are cleared so a replay must rewrite them.
        for _, call, o in cs:
            call(torch.empty_like(o))
        for _, _, o in cs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (name, _, o), e in zip(cs, eager):
            print(f"replay {rep} {name}", flush=True)
            assert torch.equal(o, e), (rep, name)


def test_graph_replay_matches_oracle():
    # The captured dx (the dominant kernel) is also right, not just repeatable.
    _, w, _ = random_case(8, 1, 64, 10, 10, 128, 3, 3, 1, "NHWC", BF16, bias=False)
    dy = random_dy(9, (1, 5, 5, 128), BF16)
    geo = dict(stride=2, padding=1, dilation=1, groups=1, layout="NHWC")
    dyd, wd = dy.to(DEV), w.to(DEV)
    dx = torch.empty(1, 10, 10, 64, device=DEV, dtype=BF16)
    cm.conv2d_input_grad(dyd, wd, (1, 10, 10, 64), out=dx, path="dx_igemm", **geo)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cm.conv2d_input_grad(dyd, wd, (1, 10, 10, 64), out=dx, path="dx_igemm", **geo)
    dx.zero_()
    graph.replay()
    torch.cuda.synchronize()
    ref, norm = oracle.conv2d_input_grad(dy, w, (1, 10, 10, 64), **geo)
    err = oracle.max_normalised_error(f64(dx.cpu()), ref, norm)
    assert err <= TOL[BF16], err
    assert np.isfinite(f64(dx.cpu())).all()
