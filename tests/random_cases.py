"""Seeded random convolution geometries for the automatic-path sweep.

Only shapes and options are drawn here (no convolution arithmetic).  The
mix leans towards what the specialised kernels take -- NHWC bf16, group
widths of 1, 4, 8, 16 and 32 channels, 1x1 and 3x3 kernels -- and keeps
the rest (rectangular and even kernels, strides up to 3, dilations up to 3,
asymmetric padding, NCHW and fp32, extents down to one pixel) so that every
kernel's declines and ragged edges are exercised too.  Sizes are capped so
that the fp64 oracle finishes each case in well under a second.
"""
import numpy as np

KERNELS = [(1, 1), (1, 1), (3, 3), (3, 3), (3, 3), (5, 5), (1, 3), (3, 1), (2, 2), (4, 4)]
MAX_MACS = 60_000_000


def out_size(n, k, s, p, d):
    return (n + 2 * p - d * (k - 1) - 1) // s + 1


def cases(n=64, seed=20261202):
    """n dicts: kind ("fwd" or "dx"), N, C, H, W, CO, KH, KW, stride, pad,
    dil (pairs), groups, layout, dtype ("bf16" or "fp32")."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        kind = "dx" if rng.random() < 0.35 else "fwd"
        C = int(rng.choice([8, 16, 32, 48, 64, 96, 128, 192, 256]))
        width = rng.choice(["dense", "dense", "depthwise", "4", "8", "16", "32"])
        if width == "dense":
            G = 2 if (C % 2 == 0 and rng.random() < 0.2) else 1
            CO = int(rng.choice([8, 16, 32, 48, 64, 128])) * G
        elif width == "depthwise":
            G, CO = C, C
        else:
            cg = int(width)
            if C % cg:
                continue
            G, CO = C // cg, C
        KH, KW = KERNELS[int(rng.integers(len(KERNELS)))]
        sh, sw = (int(rng.choice([1, 1, 1, 2, 3])) for _ in range(2))
        if rng.random() < 0.6:
            sw = sh
        dh, dw = (int(rng.choice([1, 1, 1, 2, 3])) for _ in range(2))
        if rng.random() < 0.6:
            dw = dh
        ph = int(rng.integers(0, (KH - 1) * dh + 1))
        pw = int(rng.integers(0, (KW - 1) * dw + 1))
        N = int(rng.integers(1, 4))
        H = int(rng.integers(1, 25))
        W = int(rng.integers(1, 25))
        OH, OW = out_size(H, KH, sh, ph, dh), out_size(W, KW, sw, pw, dw)
        if OH < 1 or OW < 1:
            continue
        if N * OH * OW * CO * (C // G) * KH * KW > MAX_MACS:
            continue
        layout = "NHWC" if rng.random() < 0.85 else "NCHW"
        dtype = "bf16" if rng.random() < 0.8 else "fp32"
        out.append(dict(kind=kind, N=N, C=C, H=H, W=W, CO=CO, KH=KH, KW=KW, stride=(sh, sw),
                        pad=(ph, pw), dil=(dh, dw), groups=G, layout=layout, dtype=dtype))
    return out


def label(c):
    return (f"{c['kind']} N{c['N']} C{c['C']} {c['H']}x{c['W']} CO{c['CO']} k{c['KH']}x{c['KW']} "
            f"s{c['stride']} p{c['pad']} d{c['dil']} g{c['groups']} {c['layout']} {c['dtype']}")
