"""Seeded synthetic inputs for the convolution workloads.

Holds no convolution arithmetic: only tensor shapes, value distributions and
a seeded draw.  The same bytes feed the HIP path and the CPU oracle.

Recipe: a torch CPU ``Generator`` seeded with ``seed`` (0 by default) draws,
in this order, the input (``x``, or ``dy`` for an input-gradient workload),
the weight and then the bias, each in fp32 in its stored layout's shape, then
rounds to the workload's dtype (round to nearest even for bf16).
``("normal", mean, var)`` takes a variance; ``("uniform", lo, hi)`` a range.
"""
from __future__ import annotations

import math

import torch

# Every workload: the geometry of the forward convolution, the layout and
# dtype, the distributions, and (for input gradients) the shape of dy.
WORKLOADS = {
    "tiny_3x3_fp32_nchw": dict(
        kind="fwd", N=2, C=3, H=16, W=16, C_out=8, KH=3, KW=3, stride=1, pad=1, dil=1, groups=1,
        layout="NCHW", dtype="fp32", x=("uniform", -1.0, 1.0), w=("uniform", -1.0, 1.0),
        bias=("uniform", -0.1, 0.1)),
    "pointwise_1x1_c256_k64_56x56_n32_bf16_nhwc": dict(
        kind="fwd", N=32, C=256, H=56, W=56, C_out=64, KH=1, KW=1, stride=1, pad=0, dil=1,
        groups=1, layout="NHWC", dtype="bf16", x=("normal", 0.0, 1.0),
        w=("normal", 0.0, 1.0 / 256), bias=None),
    "dense_3x3_c64_k64_56x56_n32_bf16_nhwc": dict(
        kind="fwd", N=32, C=64, H=56, W=56, C_out=64, KH=3, KW=3, stride=1, pad=1, dil=1,
        groups=1, layout="NHWC", dtype="bf16", x=("normal", 0.0, 1.0),
        w=("normal", 0.0, 2.0 / (9 * 64)), bias=("normal", 0.0, 0.01)),
    "depthwise_3x3_d2_c256_56x56_n32_bf16_nhwc": dict(
        kind="fwd", N=32, C=256, H=56, W=56, C_out=256, KH=3, KW=3, stride=1, pad=2, dil=2,
        groups=256, layout="NHWC", dtype="bf16", x=("normal", 0.0, 1.0),
        w=("normal", 0.0, 1.0 / 9), bias=None),
    "dx_3x3_s2_c128_k256_56x56_n32_bf16_nhwc": dict(
        kind="dx", N=32, C=128, H=56, W=56, C_out=256, KH=3, KW=3, stride=2, pad=1, dil=1,
        groups=1, layout="NHWC", dtype="bf16", dy_shape=(32, 28, 28, 256),
        dy=("normal", 0.0, 1.0), w=("normal", 0.0, 2.0 / (9 * 128)), bias=None),
}

# Workloads of the rows after the hot path: a dilated 1-D convolution over
# long sequences (a temporal-convolution layer), the weight gradient of the
# dense 3x3 layer above, a stride-2 transposed convolution that doubles a
# 28x28 map (a decoder up-sampling layer), and two grouped 3x3 layers with
# 32 groups of 4 and of 8 channels (the group widths of aggregated-residual
# networks' first two stages).  They are measured beside the hot path, not
# inside its step.
NEXT_WORKLOADS = {
    "conv1d_k3_d4_c128_k128_l4096_n32_bf16_nlc": dict(
        kind="conv1d", N=32, C=128, L=4096, C_out=128, K=3, stride=1, pad=4, dil=4, groups=1,
        layout="NLC", dtype="bf16", x=("normal", 0.0, 1.0), w=("normal", 0.0, 2.0 / (3 * 128)),
        bias=("normal", 0.0, 0.01)),
    "dw_3x3_c64_k64_56x56_n32_bf16_nhwc": dict(
        kind="dw", N=32, C=64, H=56, W=56, C_out=64, KH=3, KW=3, stride=1, pad=1, dil=1,
        groups=1, layout="NHWC", dtype="bf16", dy_shape=(32, 56, 56, 64), x=("normal", 0.0, 1.0),
        dy=("normal", 0.0, 1.0), w=None, bias=None),
    "convT_4x4_s2_c256_k128_28to56_n32_bf16_nhwc": dict(
        kind="convT", N=32, C=256, H=28, W=28, C_out=128, KH=4, KW=4, stride=2, pad=1,
        out_pad=0, dil=1, groups=1, layout="NHWC", dtype="bf16", x=("normal", 0.0, 1.0),
        w=("normal", 0.0, 2.0 / (16 * 256)), bias=("normal", 0.0, 0.01)),
    "grouped_3x3_g32_c128_56x56_n32_bf16_nhwc": dict(
        kind="fwd", N=32, C=128, H=56, W=56, C_out=128, KH=3, KW=3, stride=1, pad=1, dil=1,
        groups=32, layout="NHWC", dtype="bf16", x=("normal", 0.0, 1.0),
        w=("normal", 0.0, 2.0 / (9 * 4)), bias=("normal", 0.0, 0.01)),
    "grouped_3x3_g32_c256_28x28_n32_bf16_nhwc": dict(
        kind="fwd", N=32, C=256, H=28, W=28, C_out=256, KH=3, KW=3, stride=1, pad=1, dil=1,
        groups=32, layout="NHWC", dtype="bf16", x=("normal", 0.0, 1.0),
        w=("normal", 0.0, 2.0 / (9 * 8)), bias=("normal", 0.0, 0.01)),
    # Groups of 24 channels (a multiple of 8, not of 16): 8 groups over 192.
    "grouped_3x3_g8_c192_56x56_n32_bf16_nhwc": dict(
        kind="fwd", N=32, C=192, H=56, W=56, C_out=192, KH=3, KW=3, stride=1, pad=1, dil=1,
        groups=8, layout="NHWC", dtype="bf16", x=("normal", 0.0, 1.0),
        w=("normal", 0.0, 2.0 / (9 * 24)), bias=("normal", 0.0, 0.01)),
    # A depthwise 3x3 with channel multiplier 2 (64 -> 128 channels).
    "depthwise_mult2_3x3_c64_k128_56x56_n32_bf16_nhwc": dict(
        kind="fwd", N=32, C=64, H=56, W=56, C_out=128, KH=3, KW=3, stride=1, pad=1, dil=1,
        groups=64, layout="NHWC", dtype="bf16", x=("normal", 0.0, 1.0),
        w=("normal", 0.0, 1.0 / 9), bias=None),
}

TORCH_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


def draw(shape, dist, gen: torch.Generator, dtype=torch.float32) -> torch.Tensor:
    """One seeded fp32 draw of ``shape`` from ``dist``, rounded to ``dtype``."""
    kind, a, b = dist
    t = torch.empty(tuple(shape), dtype=torch.float32)
    if kind == "uniform":
        t.uniform_(a, b, generator=gen)
    elif kind == "normal":
        t.normal_(a, math.sqrt(b), generator=gen)
    else:
        raise ValueError(f"unknown distribution {kind!r}")
    return t.to(dtype)


def shapes(spec: dict) -> dict:
    """Stored shapes of the tensors of a workload, from its stated sizes."""
    if spec["kind"] == "conv1d":
        N, C, L, CO, K, G = (spec[k] for k in ("N", "C", "L", "C_out", "K", "groups"))
        nlc = spec["layout"] == "NLC"
        return {"x": (N, L, C) if nlc else (N, C, L),
                "w": (CO, K, C // G) if nlc else (CO, C // G, K), "bias": (CO,)}
    if spec["kind"] == "convT":
        # C is the transposed convolution's input channel count; the weight
        # is [C_in, KH, KW, C_out/G] (NHWC) or [C_in, C_out/G, KH, KW].
        N, C, H, W, CO = spec["N"], spec["C"], spec["H"], spec["W"], spec["C_out"]
        KH, KW, G = spec["KH"], spec["KW"], spec["groups"]
        nhwc = spec["layout"] == "NHWC"
        return {"x": (N, H, W, C) if nhwc else (N, C, H, W),
                "w": (C, KH, KW, CO // G) if nhwc else (C, CO // G, KH, KW), "bias": (CO,)}
    N, C, H, W, CO = spec["N"], spec["C"], spec["H"], spec["W"], spec["C_out"]
    KH, KW, G = spec["KH"], spec["KW"], spec["groups"]
    nhwc = spec["layout"] == "NHWC"
    out = {
        "x": (N, H, W, C) if nhwc else (N, C, H, W),
        "w": (CO, KH, KW, C // G) if nhwc else (CO, C // G, KH, KW),
        "bias": (CO,),
    }
    if spec["kind"] in ("dx", "dw"):
        out["dy"] = tuple(spec["dy_shape"])
    return out


def make(spec_or_name, seed: int = 0, batch: int | None = None) -> dict:
    """CPU tensors of one workload: ``x`` (or ``dy``), ``w`` and ``bias``.

    ``batch`` keeps only the first images of the input (the rest of the draw
    is made and discarded, so the kept values equal the full workload's).
    """
    if isinstance(spec_or_name, str):
        spec = WORKLOADS.get(spec_or_name) or NEXT_WORKLOADS[spec_or_name]
    else:
        spec = spec_or_name
    dt = TORCH_DTYPES[spec["dtype"]]
    shp = shapes(spec)
    gen = torch.Generator().manual_seed(seed)
    out = {}
    if spec["kind"] == "dw":
        # the forward input, then the output gradient (no weight is drawn)
        for name in ("x", "dy"):
            t = draw(shp[name], spec[name], gen, dt)
            out[name] = t[:batch].contiguous() if batch else t
        out["w"] = None
        out["bias"] = None
        return out
    lead = "dy" if spec["kind"] == "dx" else "x"
    t = draw(shp[lead], spec[lead], gen, dt)
    out[lead] = t[:batch].contiguous() if batch else t
    out["w"] = draw(shp["w"], spec["w"], gen, dt)
    out["bias"] = draw(shp["bias"], spec["bias"], gen, dt) if spec.get("bias") else None
    return out
