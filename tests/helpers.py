"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and compare with the fp64 oracle on the same bytes."""
import json
import os

import numpy as np
import torch

import convolution_implicit_gemm_conv2d_amd as cm
import oracle
from convolution_implicit_gemm_conv2d_amd import inputs

# Normalised tolerances: max |gpu - ref| / (|b| + sum |x*w|) per output.
TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


def geo_of(spec):
    return dict(stride=spec["stride"], padding=spec["pad"], dilation=spec["dil"],
                groups=spec["groups"], layout=spec["layout"])


def f64(t):
    return t.detach().cpu().double().numpy()


def gpu_fwd(x, w, b, geo, path="auto"):
    dev = torch.device("cuda:0")
    y = cm.conv2d(x.to(dev), w.to(dev), None if b is None else b.to(dev), path=path, **geo)
    torch.cuda.synchronize()
    return y.cpu()


def gpu_dx(dy, w, x_shape, geo, path="auto"):
    dev = torch.device("cuda:0")
    dx = cm.conv2d_input_grad(dy.to(dev), w.to(dev), x_shape, path=path, **geo)
    torch.cuda.synchronize()
    return dx.cpu()


def fwd_error(x, w, b, y, geo):
    ref, norm = oracle.conv2d_forward(x, w, b, **geo)
    assert tuple(y.shape) == ref.shape
    return oracle.max_normalised_error(f64(y), ref, norm)


def dx_error(dy, w, x_shape, dx, geo):
    ref, norm = oracle.conv2d_input_grad(dy, w, x_shape, **geo)
    assert tuple(dx.shape) == ref.shape
    return oracle.max_normalised_error(f64(dx), ref, norm)


def random_case(seed, N, C, H, W, CO, KH, KW, G, layout, dtype, bias=True):
    """Seeded x, w, bias for a small test geometry (uniform [-1, 1])."""
    spec = dict(kind="fwd", N=N, C=C, H=H, W=W, C_out=CO, KH=KH, KW=KW, groups=G, layout=layout,
                dtype="fp32" if dtype == torch.float32 else "bf16", x=("uniform", -1.0, 1.0),
                w=("uniform", -1.0, 1.0), bias=("uniform", -1.0, 1.0) if bias else None)
    d = inputs.make(spec, seed=seed)
    return d["x"], d["w"], d["bias"]


def random_dy(seed, shape, dtype):
    gen = torch.Generator().manual_seed(seed)
    return inputs.draw(shape, ("uniform", -1.0, 1.0), gen, dtype)


def out_shape(x_shape, w_shape, geo):
    s = geo["stride"] if isinstance(geo["stride"], tuple) else (geo["stride"],) * 2
    p = geo["padding"] if isinstance(geo["padding"], tuple) else (geo["padding"],) * 2
    d = geo["dilation"] if isinstance(geo["dilation"], tuple) else (geo["dilation"],) * 2
    if geo["layout"] == "NHWC":
        N, H, W, _ = x_shape
        CO, KH, KW, _ = w_shape
    else:
        N, _, H, W = x_shape
        CO, _, KH, KW = w_shape
    OH = oracle.out_size(H, KH, s[0], p[0], d[0])
    OW = oracle.out_size(W, KW, s[1], p[1], d[1])
    return (N, OH, OW, CO) if geo["layout"] == "NHWC" else (N, CO, OH, OW)


def record(name, err, tol, **extra):
    """Prints a measured normalised error and, when CONVMI_PARITY_LOG names a
    file, appends it there as one JSON line (the full-size workloads' errors
    are kept from the GPU runs)."""
    print(f"  {name}: normalised error {err:.3e} (tolerance {tol})", flush=True)
    path = os.environ.get("CONVMI_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": name, "error": float(err), "tolerance": float(tol), **extra}) + "\n")
