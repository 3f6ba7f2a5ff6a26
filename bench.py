"""Throughput of the convolution hot path on one MI355X.

One step runs every workload of the path once -- the tiny fp32 NCHW 3x3
(generic direct kernel), the 1x1 bf16 pointwise GEMM, the dense 3x3 bf16
implicit GEMM, the dilated depthwise 3x3 and the stride-2 3x3 input gradient
-- each at its full size, through the C ABI, on device-resident synthetic
inputs.  Inputs and outputs rotate over several buffer sets so that no call
finds its operands in the 256 MB Infinity Cache.

Prints ONE JSON line: whole-step TFLOP/s (``value``), per-workload kernel
times with their fraction of the MFMA or HBM roofline, the roofline of the
dominant kernel (time measured here with HIP events on the launch stream,
over the timed steps themselves), and the fp64 CPU oracle timed on this host
as a baseline.  ``next_rows`` adds, outside the step, the rows after the hot
path (a dilated conv1d, the dense layer's weight gradient and a stride-2
transposed conv2d) with their kernel times, roofline fractions and the
oracle timed on one image.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (vector / MFMA)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "conv TFLOP/s & % MFMA peak (dense); GB/s & % HBM peak (depthwise)"

# The roofline that bounds a workload follows from its arithmetic intensity
# (algorithmic FLOP / algorithmic bytes) against the ridge of the peak it
# computes at: below the ridge the HBM bandwidth bounds it, above it the
# matrix (or fp32) peak.  The attainable rate is min(peak, AI x HBM).
# Set from --path: a forced kernel path for the workloads of this run.
FORCED_PATH = None


def ridge(peak_tflops: float) -> float:
    return peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9)


# Kernel source each workload's path runs, for the staleness check of the
# committed counter summary.
KERNEL_SOURCE = {
    "direct": "direct.hip", "dx_gather": "direct.hip", "pointwise": "pointwise.hip",
    "igemm": "igemm.hip", "igemm_band": "igemm_band.hip", "depthwise": "depthwise.hip",
    "dx_igemm": "dx_igemm.hip", "dx_band": "dx_band.hip", "dx_depthwise": "depthwise.hip",
    "dw_igemm": "dw.hip", "dw_direct": "dw.hip",
}


def source_digest(path_name: str) -> str | None:
    if path_name not in KERNEL_SOURCE:
        return None
    f = os.path.join(ROOT, "convolution_implicit_gemm_conv2d_amd", "csrc", KERNEL_SOURCE[path_name])
    if not os.path.exists(f):
        return None
    return hashlib.sha256(open(f, "rb").read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=4, help="buffer sets cycled through")
    ap.add_argument("--only", default=None, help="run a single workload (for profiling)")
    ap.add_argument("--path", default=None,
                    help="with --only: force this kernel path (a name of the C ABI's path list) "
                         "instead of the automatic one, to profile an alternative kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the bench, time a plain device copy of this many MiB "
                         "(counter calibration)")
    ap.add_argument("--platform-floor", action="store_true",
                    help="instead of the bench, time an empty kernel and a plain 51.4 MB "
                         "device copy (the fixed cost of a launch and the practical HBM rate)")
    return ap.parse_args()


class Workload:
    """Device buffers and the C-ABI call of one workload."""

    def __init__(self, name, rotate, dev):
        import torch

        import convolution_implicit_gemm_conv2d_amd as cm
        from convolution_implicit_gemm_conv2d_amd import inputs

        self.cm = cm
        self.name = name
        s = self.spec = inputs.WORKLOADS[name]
        self.lay = cm.CONV_NHWC if s["layout"] == "NHWC" else cm.CONV_NCHW
        self.dt = cm.CONV_BF16 if s["dtype"] == "bf16" else cm.CONV_F32
        self.esize = 2 if s["dtype"] == "bf16" else 4
        self.geom = (s["N"], s["C"], s["H"], s["W"], s["C_out"], s["KH"], s["KW"], s["stride"],
                     s["stride"], s["pad"], s["pad"], s["dil"], s["dil"], s["groups"], self.lay,
                     self.dt)
        self.bwd = s["kind"] == "dx"
        self.path = cm.conv_select_path(self.bwd, *self.geom)
        if FORCED_PATH:
            self.path = cm.PATHS[FORCED_PATH]
        self.path_name = cm.conv_path_name(self.path)
        OH = cm.conv_out_size(s["H"], s["KH"], s["stride"], s["pad"], s["dil"])
        OW = cm.conv_out_size(s["W"], s["KW"], s["stride"], s["pad"], s["dil"])
        d = inputs.make(name)
        self.host = d
        x_elems = s["N"] * s["C"] * s["H"] * s["W"]
        y_elems = s["N"] * s["C_out"] * OH * OW
        w_elems = d["w"].numel()
        b_elems = 0 if d["bias"] is None else d["bias"].numel()
        self.flops = 2 * s["N"] * OH * OW * s["C_out"] * (s["C"] // s["groups"]) * s["KH"] * s["KW"]
        self.bytes = (x_elems + y_elems + w_elems + b_elems) * self.esize
        src = d["dy"] if self.bwd else d["x"]
        out_shape = ((s["N"], s["H"], s["W"], s["C"]) if s["layout"] == "NHWC"
                     else (s["N"], s["C"], s["H"], s["W"])) if self.bwd else None
        self.sets = []
        for _ in range(rotate):
            a = src.to(dev)
            w = d["w"].to(dev)
            b = None if d["bias"] is None else d["bias"].to(dev)
            if self.bwd:
                o = torch.empty(out_shape, dtype=src.dtype, device=dev)
            else:
                oshape = (s["N"], OH, OW, s["C_out"]) if s["layout"] == "NHWC" else (s["N"], s["C_out"], OH, OW)
                o = torch.empty(oshape, dtype=src.dtype, device=dev)
            self.sets.append((a.data_ptr(), w.data_ptr(), None if b is None else b.data_ptr(),
                              o.data_ptr(), (a, w, b, o)))

    def launch(self, k, stream):
        a, w, b, o, _ = self.sets[k % len(self.sets)]
        if self.bwd:
            self.cm.conv_bwd_dx_ex(a, w, o, *self.geom, self.path, stream)
        else:
            self.cm.conv_fwd_ex(a, w, b, o, *self.geom, self.path, stream)

    def peak_tflops(self):
        return PEAK_FP32_TFLOPS if self.dt == self.cm.CONV_F32 else PEAK_BF16_TFLOPS

    def roofline(self):
        """(bound, algorithmic work per launch, peak, unit) of the roofline
        that bounds this workload."""
        ai = self.flops / self.bytes
        if ai < ridge(self.peak_tflops()):
            return "hbm", self.bytes / 1e9, PEAK_HBM_GBS, "GB/s"
        return "mfma", self.flops / 1e12, self.peak_tflops(), "TFLOP/s"

    def attainable_tflops(self):
        return min(self.peak_tflops(), self.flops / self.bytes * PEAK_HBM_GBS / 1e3)


class NextWorkload:
    """A workload of the rows after the hot path (conv1d, weight gradient,
    transposed conv2d, grouped forward): measured beside the step, not
    inside it."""

    def __init__(self, name, rotate, dev):
        import torch

        import convolution_implicit_gemm_conv2d_amd as cm
        from convolution_implicit_gemm_conv2d_amd import inputs

        self.cm = cm
        self.name = name
        s = self.spec = inputs.NEXT_WORKLOADS[name]
        self.dt = cm.CONV_BF16 if s["dtype"] == "bf16" else cm.CONV_F32
        self.esize = 2 if s["dtype"] == "bf16" else 4
        d = self.host = inputs.make(name)
        N, C, CO, G = s["N"], s["C"], s["C_out"], s["groups"]
        self.workspace = None
        if s["kind"] == "dw":
            self.lay = cm.CONV_NHWC if s["layout"] == "NHWC" else cm.CONV_NCHW
            KH, KW = s["KH"], s["KW"]
            OH = cm.conv_out_size(s["H"], KH, s["stride"], s["pad"], s["dil"])
            OW = cm.conv_out_size(s["W"], KW, s["stride"], s["pad"], s["dil"])
            out_shape = (CO, KH, KW, C // G) if s["layout"] == "NHWC" else (CO, C // G, KH, KW)
            self.flops = 2 * N * OH * OW * CO * (C // G) * KH * KW
            self.geom = (N, C, s["H"], s["W"], CO, KH, KW, s["stride"], s["stride"], s["pad"],
                         s["pad"], s["dil"], s["dil"], G, self.lay, self.dt)
            self.path = cm.conv_select_path(2, *self.geom)
            self.ws_bytes = cm.conv_bwd_dw_workspace_size(*self.geom, self.path)
        elif s["kind"] == "fwd":
            self.lay = cm.CONV_NHWC if s["layout"] == "NHWC" else cm.CONV_NCHW
            KH, KW = s["KH"], s["KW"]
            OH = cm.conv_out_size(s["H"], KH, s["stride"], s["pad"], s["dil"])
            OW = cm.conv_out_size(s["W"], KW, s["stride"], s["pad"], s["dil"])
            out_shape = (N, OH, OW, CO) if s["layout"] == "NHWC" else (N, CO, OH, OW)
            self.flops = 2 * N * OH * OW * CO * (C // G) * KH * KW
            self.geom = (N, C, s["H"], s["W"], CO, KH, KW, s["stride"], s["stride"], s["pad"],
                         s["pad"], s["dil"], s["dil"], G, self.lay, self.dt)
            self.path = cm.conv_select_path(0, *self.geom)
        elif s["kind"] == "conv1d":
            self.lay = cm.CONV_NLC if s["layout"] == "NLC" else cm.CONV_NCL
            OL = cm.conv_out_size(s["L"], s["K"], s["stride"], s["pad"], s["dil"])
            out_shape = (N, OL, CO) if s["layout"] == "NLC" else (N, CO, OL)
            self.flops = 2 * N * OL * CO * (C // G) * s["K"]
            self.path = cm.conv_select_path(0, N, C, 1, s["L"], CO, 1, s["K"], 1, s["stride"], 0,
                                            s["pad"], 1, s["dil"], G, self.lay, self.dt)
        else:
            self.lay = cm.CONV_NHWC if s["layout"] == "NHWC" else cm.CONV_NCHW
            OH = cm.conv_transpose_out_size(s["H"], s["KH"], s["stride"], s["pad"], s["dil"], s["out_pad"])
            OW = cm.conv_transpose_out_size(s["W"], s["KW"], s["stride"], s["pad"], s["dil"], s["out_pad"])
            out_shape = (N, OH, OW, CO) if s["layout"] == "NHWC" else (N, CO, OH, OW)
            # every input element meets every tap of its group's output channels
            self.flops = 2 * N * s["H"] * s["W"] * C * (CO // G) * s["KH"] * s["KW"]
            self.path = cm.conv_select_path(1, N, CO, OH, OW, C, s["KH"], s["KW"], s["stride"],
                                            s["stride"], s["pad"], s["pad"], s["dil"], s["dil"], G,
                                            self.lay, self.dt)
        if FORCED_PATH:
            self.path = cm.PATHS[FORCED_PATH]
        self.path_name = cm.conv_path_name(self.path)
        y_elems = 1
        for v in out_shape:
            y_elems *= v
        ins = [t for t in (d["x"], d.get("dy"), d["w"], d["bias"]) if t is not None]
        self.bytes = (sum(t.numel() for t in ins) + y_elems) * self.esize
        self.sets = []
        for _ in range(rotate):
            a = d["x"].to(dev)
            w = (d["dy"] if s["kind"] == "dw" else d["w"]).to(dev)
            b = None if d["bias"] is None else d["bias"].to(dev)
            o = torch.empty(out_shape, dtype=a.dtype, device=dev)
            self.sets.append((a, w, b, o))
        if s["kind"] == "dw":
            self.workspace = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)

    def launch(self, k, stream):
        a, w, b, o = self.sets[k % len(self.sets)]
        s, cm, G = self.spec, self.cm, self.spec["groups"]
        if s["kind"] == "dw":
            cm.conv_bwd_dw_ex(a, w, o, self.workspace, self.workspace.numel(), *self.geom,
                              self.path, stream)
        elif s["kind"] == "fwd":
            cm.conv_fwd_ex(a, w, b, o, *self.geom, self.path, stream)
        elif s["kind"] == "conv1d":
            cm.conv1d_fwd_ex(a, w, b, o, s["N"], s["C"], s["L"], s["C_out"], s["K"], s["stride"],
                             s["pad"], s["dil"], G, self.lay, self.dt, self.path, stream)
        else:
            cm.conv_transpose2d_ex(a, w, b, o, s["N"], s["C"], s["H"], s["W"], s["C_out"], s["KH"],
                                   s["KW"], s["stride"], s["stride"], s["pad"], s["pad"],
                                   s["out_pad"], s["out_pad"], s["dil"], s["dil"], G, self.lay,
                                   self.dt, self.path, stream)

    def oracle_sample(self):
        """The oracle on the first image of the same inputs: (seconds, flop)."""
        import oracle
        from convolution_implicit_gemm_conv2d_amd import inputs

        s = self.spec
        d = inputs.make(self.name, batch=1)
        t0 = time.perf_counter()
        if s["kind"] == "dw":
            w_shape = (s["C_out"], s["KH"], s["KW"], s["C"] // s["groups"])
            oracle.conv2d_weight_grad(d["x"], d["dy"], w_shape, s["stride"], s["pad"], s["dil"],
                                      s["groups"], s["layout"])
        elif s["kind"] == "fwd":
            oracle.conv2d_forward(d["x"], d["w"], d["bias"], stride=s["stride"], padding=s["pad"],
                                  dilation=s["dil"], groups=s["groups"], layout=s["layout"])
        elif s["kind"] == "conv1d":
            oracle.conv1d_forward(d["x"], d["w"], d["bias"], s["stride"], s["pad"], s["dil"],
                                  s["groups"], s["layout"])
        else:
            oracle.conv_transpose2d(d["x"], d["w"], d["bias"], s["stride"], s["pad"], s["out_pad"],
                                    s["dil"], s["groups"], s["layout"])
        return time.perf_counter() - t0, self.flops // s["N"]


def measure_next(names, rotate, dev, stream, sp, steps, with_oracle):
    """Kernel time of each next-row workload from armed launches (warm-up
    first), with its roofline and the oracle timed on one image."""
    import torch

    import convolution_implicit_gemm_conv2d_amd as cm

    rows = []
    for name in names:
        wl = NextWorkload(name, rotate, dev)
        for k in range(3):
            wl.launch(k, sp)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.01 + steps * 2.4e9 * 40e-6))
        for k in range(steps):
            cm.conv_arm_launch_events(evs[k][0].cuda_event, evs[k][1].cuda_event)
            wl.launch(3 + k, sp)
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in evs) / steps * 1e3
        tflops = wl.flops / (us * 1e-6) / 1e12
        gbs = wl.bytes / (us * 1e-6) / 1e9
        ai = wl.flops / wl.bytes
        bound = "hbm" if ai < ridge(PEAK_BF16_TFLOPS) else "mfma"
        frac = gbs / PEAK_HBM_GBS if bound == "hbm" else tflops / PEAK_BF16_TFLOPS
        att = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3)
        row = {"workload": name, "path": wl.path_name, "us_per_call": round(us, 3),
               "tflops": round(tflops, 3), "gbs": round(gbs, 1), "bound": bound,
               "roofline_frac": round(frac, 4), "arith_intensity": round(ai, 1),
               "attainable_tflops": round(att, 1), "pct_attainable": round(100 * tflops / att, 2),
               "flop": wl.flops, "bytes": wl.bytes}
        if with_oracle:
            import oracle

            sec, flop = wl.oracle_sample()
            row["cpu_oracle"] = {"value": flop / sec / 1e12, "unit": "TFLOP/s",
                                 "cores": oracle.threads(), "kind": "oracle",
                                 "seconds": round(sec, 3), "sample": "the first image"}
        rows.append(row)
    return rows


def copy_calibration(mib, dev):
    """A plain device-to-device copy of known size, for scaling HBM counters."""
    import torch

    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 5}))


def platform_floor(dev, reps=200):
    """Event-timed duration of an empty kernel and of a device copy of the
    size of the 1x1 and depthwise workloads' input (51.4 MB), median of
    `reps`: the fixed cost every launch pays and the HBM rate a plain stream
    reaches."""
    import statistics

    import torch

    stream = torch.cuda.current_stream()
    n = 32 * 56 * 56 * 256  # bf16 elements of [32, 56, 56, 256]
    srcs = [torch.ones(n, dtype=torch.bfloat16, device=dev) for _ in range(4)]
    dsts = [torch.empty_like(a) for a in srcs]
    out = {}
    for what in ("empty_kernel", "copy"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for k in range(reps + 10):
            e = evs[k - 10] if k >= 10 else None
            if e:
                e[0].record(stream)
            if what == "empty_kernel":
                torch.cuda._sleep(0)
            else:
                dsts[k % 4].copy_(srcs[k % 4])
            if e:
                e[1].record(stream)
        torch.cuda.synchronize()
        us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)
        out[what + "_us"] = round(us, 3)
    out["copy_bytes"] = 2 * n * 2
    out["copy_GBps_algorithmic"] = round(2 * n * 2 / (out["copy_us"] * 1e-6) / 1e9, 1)
    print(json.dumps(out), flush=True)


def cpu_baseline(works):
    """The fp64 oracle timed over the same step (every image of every workload)."""
    import oracle

    flops = 0
    t0 = time.perf_counter()
    for wl in works:
        s, d = wl.spec, wl.host
        geo = dict(stride=s["stride"], padding=s["pad"], dilation=s["dil"], groups=s["groups"],
                   layout=s["layout"])
        if wl.bwd:
            shp = (s["N"], s["H"], s["W"], s["C"]) if s["layout"] == "NHWC" else (s["N"], s["C"], s["H"], s["W"])
            oracle.conv2d_input_grad(d["dy"], d["w"], shp, **geo)
        else:
            oracle.conv2d_forward(d["x"], d["w"], d["bias"], **geo)
        flops += wl.flops
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": "one full step: every image of every workload, fp64 direct loops "
                      "(scatter form for the input gradient), OpenMP over images/channels"}


def load_traffic(dominant):
    """HBM bytes per launch from the committed counter summary, if it still
    describes the current kernel source."""
    f = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(f):
        return None
    rec = json.load(open(f)).get(dominant.name)
    if not rec or rec.get("source_sha256_16") != source_digest(dominant.path_name):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this "
              "build (the path shards over images with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from convolution_implicit_gemm_conv2d_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.path:
        if not args.only:
            print("--path needs --only", file=sys.stderr)
            sys.exit(2)
        global FORCED_PATH
        FORCED_PATH = args.path
    if args.copy_mib:
        copy_calibration(args.copy_mib, dev)
        return
    if args.platform_floor:
        platform_floor(dev)
        return
    if args.only in inputs.NEXT_WORKLOADS:
        # One next-row workload alone (for profiling): its warm-up and armed
        # launches, reported like next_rows.
        stream = torch.cuda.current_stream()
        rows = measure_next([args.only], args.rotate, dev, stream, stream.cuda_stream, args.steps,
                            False)
        print(json.dumps({"next_rows": rows}), flush=True)
        return
    names = [args.only] if args.only else list(inputs.WORKLOADS)
    works = [Workload(n, args.rotate, dev) for n in names]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    for k in range(args.warmup):
        for wl in works:
            wl.launch(k, sp)
    torch.cuda.synchronize()

    K = args.steps
    import convolution_implicit_gemm_conv2d_amd as cm

    # Kernel durations come from (start, stop) event pairs that a launch
    # stamps with its own kernel start and end (conv_arm_launch_events,
    # through hipExtLaunchKernel).  Arming adds a few microseconds of
    # dispatch work to the launch it is attached to, so arming every launch
    # of the timed steps would time the event machinery along with the path.
    # Hence two passes of K steps each:
    #   1. every launch armed, untimed as a whole: per-workload durations,
    #      which name the dominant (longest) kernel;
    #   2. the timed steps, with only the dominant kernel's launches armed:
    #      the step time and, live over that same region, the dominant
    #      kernel's duration for the roofline.
    def make_events(n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:  # creates the underlying HIP events
            a.record(stream)
            b.record(stream)
        return evs

    def spin_ahead(launches):
        # Queue a spin ahead of the launches so the host can enqueue all of
        # them before the GPU reaches them: the region then measures the
        # GPU, not the Python launch overhead.
        torch.cuda._sleep(int(2.4e9 * 0.02 + launches * 2.4e9 * 40e-6))

    ev = [make_events(K) for _ in works]
    torch.cuda.synchronize()
    spin_ahead(K * len(works))
    for k in range(K):
        for i, wl in enumerate(works):
            cm.conv_arm_launch_events(ev[i][k][0].cuda_event, ev[i][k][1].cuda_event)
            wl.launch(args.warmup + k, sp)
    torch.cuda.synchronize()
    us_all = [sum(a.elapsed_time(b) for a, b in ev[i]) / K * 1e3 for i in range(len(works))]
    dom_i = max(range(len(works)), key=lambda i: us_all[i])

    dev_ev = make_events(K)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    spin_ahead(K * len(works))
    t_start.record(stream)
    for k in range(K):
        for i, wl in enumerate(works):
            if i == dom_i:
                cm.conv_arm_launch_events(dev_ev[k][0].cuda_event, dev_ev[k][1].cuda_event)
            wl.launch(args.warmup + K + k, sp)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / K
    us_all[dom_i] = sum(a.elapsed_time(b) for a, b in dev_ev) / K * 1e3

    per = []
    for i, wl in enumerate(works):
        us = us_all[i]
        bound, work, peak, unit = wl.roofline()
        tflops = wl.flops / (us * 1e-6) / 1e12
        gbs = wl.bytes / (us * 1e-6) / 1e9
        att = wl.attainable_tflops()
        per.append({
            "workload": wl.name, "path": wl.path_name, "us_per_call": round(us, 3),
            "timed_in": "timed steps" if i == dom_i else "armed pass",
            "tflops": round(tflops, 3), "gbs": round(gbs, 1),
            "pct_mfma_peak": round(100 * tflops / wl.peak_tflops(), 2),
            "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2), "bound": bound,
            "arith_intensity": round(wl.flops / wl.bytes, 1),
            "attainable_tflops": round(att, 1), "pct_attainable": round(100 * tflops / att, 2),
            "flop": wl.flops, "bytes": wl.bytes,
        })
    total_flops = sum(wl.flops for wl in works)
    value = total_flops / (ms_step * 1e-3) / 1e12

    dom = works[dom_i]
    bound, work, peak, unit = dom.roofline()
    achieved = work / (per[dom_i]["us_per_call"] * 1e-6)
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": load_traffic(dom),
            "kernel": f"{dom.path_name} ({dom.name})",
            "algorithmic_per_launch": dom.bytes if bound == "hbm" else dom.flops}

    cpu = None if args.no_cpu_baseline else cpu_baseline(works)
    next_rows = [] if args.only else measure_next(list(inputs.NEXT_WORKLOADS), args.rotate, dev,
                                                  stream, sp, K, not args.no_cpu_baseline)
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "conv2d hot path, one step = " + " + ".join(names),
                   "global_batch": 32, "rotating_buffer_sets": args.rotate},
        "roofline": roof, "cpu_baseline": cpu, "per_workload": per, "next_rows": next_rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
