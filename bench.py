#!/usr/bin/env python3
"""Throughput of the fp32 tiled GEMM (addmm and implicit-im2col conv2d) on
one MI355X, in fp32 TFLOP/s and as a fraction of the fp32 matrix peak.

One step = one pass over the largest workload shapes, each launched once
through the C ABI on torch's current stream, inputs already resident in HBM:

  conv3x3_56_s1   [4,256,56,56] * [256,256,3,3], s1 p1       (M=256 N=12544 K=2304)
  conv3x3_56_d2   same, dilation 2, pad 2                      (M=256 N=12544 K=2304)
  conv3x3_57_s2   [4,256,57,57], stride 2, pad 1               (M=256 N=3364  K=2304)
  up_proj         addmm 4096x1024 @ 1024x4096, self [N]
  down_proj       addmm 4096x4096 @ 4096x1024, self [N]
  ragged_577      addmm 577x1024 @ 1024x4096, self [M,N]

flops = 2*M*N*K per launch (the conv's bias adds are not counted).  Prints
ONE JSON line.  ``--gpus`` above 1 is refused: the measurement is of one GPU.

After the settle and warm-up steps, K steps run with a HIP event pair around
every launch (the per-case times, ``ms_per_step_with_case_events``), then the
K timed steps run back to back with an event pair only around the dominant
kernel's launches (its duration for ``roofline``): ``value`` and
``ms_per_step`` come from that second pass.
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

PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak (datasheet)
HBM_GBS = 8000.0     # MI355X HBM3E bandwidth (datasheet)
METRIC = "fp32 TFLOP/s (addmm, im2col conv2d) and % of MI355X fp32 MFMA peak"
STEP_CASES = ["conv3x3_56_s1", "conv3x3_56_d2", "conv3x3_57_s2",
              "up_proj_4096x1024x4096", "down_proj_4096x4096x1024",
              "ragged_577x1024x4096_full_self"]
# Every kernel and host source of the library plus the compiler flags: the
# committed counter runs (which cover the step's cases and every other case
# bench.py times) are only valid for exactly these.
CSRC = os.path.join(ROOT, "bias_addmm_im2col_amd", "csrc")
KERNEL_SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp", ".cpp", ".h")))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps, so the timed steps "
                         "run at the GPU's steady clock")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--profile-cases", default=None, metavar="NAMES",
                    help="instead of the metric, launch each named case (comma list; 'step' is the "
                         "step's cases, 'all' every case) once when it is set up, then --steps "
                         "times back to back, case after case: a fixed dispatch sequence for the "
                         "rocprofv3 counter runs that bench_counters.py reads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="instead of the GEMM workload, run plain device-to-device copies of a "
                         "known size (reference for scaling the FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def calibrate_copy():
    """Ten copies of a 256 MiB fp32 buffer (read 256 MiB + write 256 MiB each)."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                      "copies": 10}), flush=True)


def all_case_names(I):
    return (STEP_CASES + OTHER_CONFIG_CASES + list(I.LINEAR_CASES) + list(I.GROUPED_CASES)
            + list(I.NHWC_CASES) + list(I.CONVT_CASES) + list(I.SDPA_CASES))


def profile_case_names(spec, I):
    names = []
    for n in spec.split(","):
        names += STEP_CASES if n == "step" else all_case_names(I) if n == "all" else [n]
    return names


def profile_cases(torch, baim, I, names, steps):
    """Dispatch order: every case's set-up launch, in the order given, then
    `steps` launches of the first case, `steps` of the second, and so on.
    A one-element torch fill (a kernel of torch's own, named after its fill
    functor) follows the set-up launches and each case's run, so that a
    counter trace splits into the cases' dispatches without knowing how many
    kernels one call launches.  Prints the sequence as one JSON line."""
    cases = [Case(n, torch, baim, I) for n in names]
    marker = torch.empty(1, device="cuda")
    torch.cuda.synchronize()
    marker.fill_(1.0)
    for cs in cases:
        for _ in range(steps):
            cs.launch()
        marker.fill_(1.0)
    torch.cuda.synchronize()
    print(json.dumps({"profile_cases": names, "kernels": [cs.kernel for cs in cases],
                      "algorithmic_bytes": [cs.bytes for cs in cases],
                      "flops": [cs.flops for cs in cases], "launches": steps,
                      "marker": "FillFunctor", "step_cases": STEP_CASES,
                      "kernel_source_sha": kernel_source_hash()}), flush=True)


def kernel_source_hash() -> str:
    from bias_addmm_im2col_amd import build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES + ["../../include/baim.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    h.update(" ".join(build.HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def load_counters(kernel: str):
    """(HBM bytes per launch, MFMA-busy fraction) from the committed
    rocprofv3 counter runs, only while the kernel sources are the ones the
    counters were taken on; (None, None) otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, None
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None, None
    entry = t.get("kernels", {}).get(kernel)
    if entry is None:
        return None, None
    return entry.get("bytes_per_launch"), entry.get("mfma_busy")


def raw_call(torch, fname, *args):
    """A zero-argument launcher calling the C ABI entry point `fname` with
    pointers and sizes resolved once (tensors become their device
    addresses), on torch's current stream.  It keeps the Python binding's
    per-call checks (several microseconds) out of the timed loops, so short
    kernels are timed by the GPU, not by the launch rate.  Raises if the
    call does not return BAIM_OK."""
    import ctypes
    from bias_addmm_im2col_amd import _capi
    fn = getattr(_capi.lib(), fname)
    conv = [a.data_ptr() if hasattr(a, "data_ptr") else a for a in args]
    conv.append(torch.cuda.current_stream().cuda_stream)
    st = fn(*conv)
    if st != 0:
        raise RuntimeError(f"{fname}: status {st}: {_capi.last_error()}")
    return lambda: fn(*conv)


class Case:
    def __init__(self, name, torch, baim, I):
        self.name = name
        c = (I.CASES.get(name) or I.LINEAR_CASES.get(name) or I.GROUPED_CASES.get(name)
             or I.NHWC_CASES.get(name) or I.CONVT_CASES.get(name) or I.SDPA_CASES[name])
        self.c = c
        self.op = c.kind
        self.flops = c.flops
        if c.kind == "convt":
            x, w, bias = I.convt_inputs(c)
            self.host = (x, w, bias)
            self.x, self.w, self.bias = x.cuda(), w.cuda(), bias.cuda()
            OH, OW = c.out_hw()
            self.out = torch.empty((c.B, c.OC, OH, OW), dtype=torch.float32, device="cuda")
            # the one-GEMM path takes kernel == stride, no padding, no output
            # padding, 128 | H*W and 4 | (OC/groups)*KH*KW (aligned tensors);
            # the rest run one GEMM per output phase
            fused = ((c.KH, c.KW) == tuple(c.stride) and tuple(c.padding) == (0, 0)
                     and tuple(c.output_padding) == (0, 0) and (c.H * c.W) % 128 == 0
                     and (c.OC * c.KH * c.KW) % 4 == 0)
            self.kernel = "baim::convt_fused_kernel" if fused else "baim::conv_transpose_kernel"
            self.run = lambda: baim.conv_transpose2d_f32(self.out, self.x, self.w, self.bias,
                                                         c.stride, c.padding, c.output_padding,
                                                         1, c.dilation)
            self.run()
            self.launch = raw_call(torch, "conv_transpose2d_f32", self.out, self.x, self.w,
                                   self.bias, c.B, c.IC, c.H, c.W, c.OC, c.KH, c.KW, *c.stride,
                                   *c.padding, *c.dilation, *c.output_padding, 1)
            self.bytes = 4 * (x.numel() + w.numel() + bias.numel() + self.out.numel())
            return
        if c.kind == "sdpa":
            q, k, v, m = I.sdpa_inputs(c)
            self.host = (q, k, v, m)
            self.q, self.k, self.v = q.cuda(), k.cuda(), v.cuda()
            self.m = None if m is None else m.cuda()
            self.out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
            dp = -(-c.D // 32) * 32
            self.kernel = f"baim::sdpa_kernel<D {dp}{', mask' if m is not None else ''}>"
            self.run = lambda: baim.sdpa_f32(self.out, self.q, self.k, self.v, self.m, c.scale)
            self.run()
            import ctypes
            self._scale = None if c.scale is None else ctypes.byref(ctypes.c_float(c.scale))
            self.launch = raw_call(torch, "sdpa_f32", self.out, self.q, self.k, self.v, self.m,
                                   c.B * c.H, c.Sq, c.Skv, c.D, self._scale)
            self.bytes = 4 * sum(t.numel() for t in (q, k, v, self.out) + ((m,) if m is not None else ()))
            return
        M, N, K = (c.M, c.N, c.K) if c.kind != "conv" else c.gemm_mnk
        if c.kind == "conv" and c.channels_last:  # out[B*OH*OW, OC]: the linear-shaped GEMM
            M, N = N, M
        p = baim.gemm_plan(M, N, K)
        kname = "conv2d_gemm_kernel" if c.kind == "conv" and not c.channels_last else "addmm_kernel"
        if p["bm"] == 256:  # the 256x256 tile: addmm's own kernel; the others run 128x128
            if c.kind == "addmm":
                kname = "addmm_big_kernel"
            else:
                p = dict(p, bm=128, bn=128, bk=32, waves=8, kgroups=1)
        geom = ""
        if c.kind == "conv" and not c.channels_last:
            p = baim.conv2d_plan((c.B, c.IC, c.H, c.W), (c.OC, c.IC // c.groups, c.KH, c.KW),
                                 c.stride, c.padding, c.dilation, c.groups)
            if p["kernel"] in (1, 3):  # the LDS-window and stem kernels
                kname = "conv_window_kernel" if p["kernel"] == 1 else "conv_stem_kernel"
                geom = (f"{c.KH}x{c.KW} s{c.stride[0]} d{c.dilation[0]}, ")
        nhwc_stem = False
        if c.kind == "conv" and c.channels_last:
            nhwc_stem = baim.conv2d_nhwc_plan((c.B, c.H, c.W, c.IC), (c.OC, c.KH, c.KW, c.IC),
                                              c.stride, c.padding, c.dilation)["kernel"] == 3
            if nhwc_stem:  # the stem kernel's channels-last instance
                kname = "conv_stem_kernel"
                geom = (f"{c.KH}x{c.KW} s{c.stride[0]} d{c.dilation[0]}, ")
                p = dict(p, bm=128, bn=144, bk=c.IC * c.KH * c.KW, waves=16, kgroups=1, splits=1,
                         stream_blocks=0)
        self.plan = p
        # one kernel instance per (op, geometry, block tile, waves, wave groups, K split)
        self.kernel = (f"baim::{kname}"
                       f"<{geom}Tile {p['bm']}x{p['bn']}x{p['bk']}, {p['waves']} waves, "
                       f"{p['kgroups']} k-groups>" + (f" split {p['splits']}" if p['splits'] > 1 else "")
                       + (f" stream {p['stream_blocks']}" if p['stream_blocks'] > 0 else ""))
        if c.kind == "addmm":
            a, b, s = I.addmm_inputs(c)
            self.host = (a, b, s)
            self.a, self.b, self.s = a.cuda(), b.cuda(), s.cuda()
            self.out = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
            self.K = c.K
            self.run = lambda: baim.addmm_f32(self.out, self.s, self.a, self.b, c.beta, c.alpha)
            self.run()
            self.launch = raw_call(torch, "addmm_f32", self.out, self.s, int(c.self_2d), self.a,
                                   self.b, c.M, c.N, c.K, float(c.beta), float(c.alpha))
            self.bytes = 4 * (a.numel() + b.numel() + s.numel() + self.out.numel())
        elif c.kind == "linear":
            x, w, b = I.linear_inputs(c)
            self.host = (x, w, b)
            self.x, self.w = x.cuda(), w.cuda()
            self.bias = None if b is None else b.cuda()
            self.out = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
            self.K = c.K
            self.run = lambda: baim.linear_f32(self.out, self.x, self.w, self.bias)
            self.run()
            self.launch = raw_call(torch, "linear_f32", self.out, self.x, self.w, self.bias, c.M,
                                   c.N, c.K)
            self.bytes = 4 * (x.numel() + w.numel() + (0 if b is None else b.numel())
                              + self.out.numel())
        else:
            x, w, bias = I.conv_inputs(c)
            self.host = (x, w, bias)
            self.x, self.w, self.bias = x.cuda(), w.cuda(), bias.cuda()
            OH, OW = c.out_hw()
            self.out = torch.empty((c.B, c.OC, OH, OW), dtype=torch.float32, device="cuda")
            self.K = c.IC * c.KH * c.KW
            self.run = lambda: baim.conv2d_gemm_f32(self.out, self.x, self.w, self.bias,
                                                    c.stride, c.padding, c.dilation, c.groups)
            geo = (c.B, c.IC, c.H, c.W, c.OC, c.KH, c.KW, *c.stride, *c.padding, *c.dilation)
            if c.channels_last:
                self.out = torch.empty((c.B, OH, OW, c.OC), dtype=torch.float32, device="cuda")
                self.kernel += " (NHWC)" if nhwc_stem else " (im2col NHWC)"
                self.run = lambda: baim.conv2d_nhwc_f32(self.out, self.x, self.w, self.bias,
                                                        c.stride, c.padding, c.dilation)
                self.run()
                self.launch = raw_call(torch, "conv2d_nhwc_f32", self.out, self.x, self.w,
                                       self.bias, *geo)
            else:
                self.run()
                self.launch = raw_call(torch, "conv2d_gemm_f32", self.out, self.x, self.w,
                                       self.bias, *geo, c.groups)
            self.bytes = 4 * (x.numel() + w.numel() + bias.numel() + self.out.numel())
            if c.groups > 1 and not (c.OC // c.groups >= 32 and c.IC // c.groups * c.KH * c.KW >= 32):
                # the direct path; one input channel per output channel with a
                # "same" odd kernel at stride 1 on rows of 4k <= 256 floats
                # takes the register-blocked kernel
                dw = (c.IC == c.groups and c.KH == c.KW and c.KH in (3, 5, 7)
                      and c.padding == ((c.KH - 1) // 2,) * 2 and c.stride == (1, 1)
                      and c.dilation == (1, 1) and c.W % 4 == 0 and c.W <= 256)
                self.kernel = "baim::conv_dw_rows_kernel" if dw else "baim::conv_direct_tiled_kernel"


# The other addmm and conv configurations of the same metric (the small
# 64x96x80 addmm, the FFN linear with self [N] and with a full self, the
# 7x7 stride-4 stem): reported beside the step, not part of `value`.
OTHER_CONFIG_CASES = ["addmm_small_64x96x80", "ffn_2048x768x3072_bias",
                      "ffn_2048x768x3072_full_self", "stem_conv7x7_s4_768"]


def time_widened(torch, baim, I, names=None, warmup_s=0.05, iters=50):
    """Ops beyond the step's workload (linear with weight [N,K], grouped and
    depthwise conv, channels-last conv, transposed conv, attention), or the
    cases `names`, timed the same way but reported separately: they are not
    part of `value`.  Each case first runs for `warmup_s` seconds (clocks
    settle over ~20 ms after a switch to new buffers)."""
    rows = []
    if names is None:
        names = (list(I.LINEAR_CASES) + list(I.GROUPED_CASES) + list(I.NHWC_CASES)
                 + list(I.CONVT_CASES) + list(I.SDPA_CASES))
    for name in names:
        cs = Case(name, torch, baim, I)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warmup_s:
            for _ in range(10):
                cs.launch()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            cs.launch()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        tf = cs.flops / us / 1e6
        row = {"case": name, "op": cs.op, "kernel": cs.kernel, "us": round(us, 2),
               "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_TFLOPS, 4)}
        if cs.kernel in ("baim::conv_direct_tiled_kernel", "baim::conv_dw_rows_kernel"):
            # memory-bound: achieved bandwidth on the algorithmic bytes
            gbs = cs.bytes / us / 1e3
            row.update({"bound": "hbm", "gbytes_per_s": round(gbs, 1),
                        "frac_of_hbm": round(gbs / HBM_GBS, 4)})
        rows.append(row)
    return rows


def cpu_baseline(cases, budget_s):
    """The fp64 oracle on the host cores, on a bounded sample of each case's
    outputs (full K-term dot products at random output coordinates)."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    rng = np.random.default_rng(0)
    per_case = budget_s / len(cases)
    flops = 0
    secs = 0.0
    samples = []
    for cs in cases:
        c = cs.c
        n = 256
        while True:
            if c.kind == "addmm":
                rows, cols = rng.integers(0, c.M, n), rng.integers(0, c.N, n)
                a, b, s = cs.host
                t0 = time.perf_counter()
                oracle.addmm_at(a, b, s, c.self_2d, c.beta, c.alpha, rows, cols)
                dt = time.perf_counter() - t0
            else:
                OH, OW = c.out_hw()
                idx = rng.integers(0, c.B * c.OC * OH * OW, n)
                x, w, bias = cs.host
                t0 = time.perf_counter()
                oracle.conv2d_at(x, w, bias, c.stride, c.padding, c.dilation, idx)
                dt = time.perf_counter() - t0
            if dt >= per_case / 4 or n >= (1 << 22):
                break
            n *= 4
        flops += 2 * cs.K * n
        secs += dt
        samples.append(f"{cs.name}:{n}")
    return {
        "value": round(flops / secs / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": ("fp64 oracle (plain loops, OpenMP) at random output coordinates, each a "
                   "full K-term dot product plus epilogue; outputs per case: " +
                   ", ".join(samples) + f"; {secs:.1f} s of wall time"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: bench.py measures one MI355X. "
              "The path needs no collective: addmm shards by rows of mat1 and conv by batch or "
              "output channels, each GPU running this same kernel on its share.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no ROCm GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import bias_addmm_im2col_amd as baim
    from bias_addmm_im2col_amd import _capi
    from bias_addmm_im2col_amd import inputs as I
    _capi.lib()  # fail loudly if libbaim.so is missing
    if args.profile_cases:
        profile_cases(torch, baim, I, profile_case_names(args.profile_cases, I), args.steps)
        return

    cases = [Case(n, torch, baim, I) for n in STEP_CASES]
    torch.cuda.synchronize()

    def step(events=None):
        for i, cs in enumerate(cases):
            if events is not None:
                events[i][0].record()
            cs.launch()
            if events is not None:
                events[i][1].record()

    # The clock ramps for tens of milliseconds after the GPU turns busy: run
    # untimed steps for --settle-s seconds, then the warmup steps.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # First a pass of K steps with a HIP event pair around every launch: the
    # per-case times, and which kernel dominates the step.  The event records
    # serialise the stream, so that pass is reported beside the value, not
    # as it.
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in cases] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    launch_ms = [sorted(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps))
                 for i in range(len(cases))]
    per_case_ms = [sum(t) / len(t) for t in launch_ms]
    flops_step = sum(cs.flops for cs in cases)

    case_rows = []
    k_time = {}
    k_flops = {}
    k_launch = {}
    for cs, ms, ts in zip(cases, per_case_ms, launch_ms):
        tf = cs.flops / (ms * 1e-3) / 1e12
        # "us" is the mean over the per-case pass; median and minimum beside it
        case_rows.append({"case": cs.name, "op": cs.op, "kernel": cs.kernel, "us": round(ms * 1e3, 2),
                          "us_median": round(ts[len(ts) // 2] * 1e3, 2), "us_min": round(ts[0] * 1e3, 2),
                          "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_TFLOPS, 4)})
        k_time[cs.kernel] = k_time.get(cs.kernel, 0.0) + ms
        k_flops[cs.kernel] = k_flops.get(cs.kernel, 0) + cs.flops
        k_launch[cs.kernel] = k_launch.get(cs.kernel, 0) + 1
    dom = max(k_time, key=k_time.get)
    n_launch = k_launch[dom]

    # The timed K steps: the cases back to back, with one event pair around
    # each launch of the dominant kernel (its duration for the roofline).
    dom_cases = [i for i, cs in enumerate(cases) if cs.kernel == dom]
    dev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in dom_cases] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, cs in enumerate(cases):
            if i in dom_cases:
                e = dev[s][dom_cases.index(i)]
                e[0].record()
                cs.launch()
                e[1].record()
            else:
                cs.launch()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = flops_step * args.steps / wall / 1e12
    dom_ms = sum(e[0].elapsed_time(e[1]) for row in dev for e in row) / args.steps
    achieved = k_flops[dom] / (dom_ms * 1e-3) / 1e12
    traffic, mfma_busy = load_counters(dom)
    counters_from = None
    if traffic is not None or mfma_busy is not None:
        counters_from = {"file": os.path.relpath(TRAFFIC_FILE, ROOT),
                         "kernel_source_sha": kernel_source_hash(),
                         "what": "traffic, mfma_busy and hbm_gbytes_per_s come from committed "
                                 "rocprofv3 counter runs on these exact kernel sources, not "
                                 "from this run"}

    widened = time_widened(torch, baim, I)
    other_configs = time_widened(torch, baim, I, OTHER_CONFIG_CASES)

    cpu = cpu_baseline(cases, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle_s,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "ms_per_step_with_case_events": round(wall_ev / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded torch.Generator draws with the workload distributions)",
        "config": {
            "workload": "largest shapes: 3x3 mid-stage conv2d (s1, d2, s2 on 57x57) and "
                        "up-proj / down-proj / ragged-577 addmm, one launch each per step",
            "cases": STEP_CASES,
            "flops_per_step": flops_step,
        },
        "frac_of_peak": round(value / PEAK_TFLOPS, 4),
        "cases": case_rows,
        "roofline": {
            "bound": "mfma",
            "kernel": dom,
            "achieved": round(achieved, 3),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": traffic,
            "launches_per_step": n_launch,
            "flops_per_launch_avg": k_flops[dom] // n_launch,
            "avg_launch_us": round(dom_ms / n_launch * 1e3, 2),
            # from the same committed counter runs as `traffic` (null likewise).
            # MFMA-busy cycles over elapsed cycles is the fraction of the
            # clock-adjusted peak 256*256*f_clk at whatever clock the chip
            # held; the clock it implies is achieved / (256*256*busy).
            "mfma_busy": mfma_busy,
            "frac_of_clock_adjusted_peak": mfma_busy,
            "implied_clock_ghz": (None if not mfma_busy
                                  else round(achieved * 1e12 / (256 * 256 * mfma_busy) / 1e9, 3)),
            "hbm_gbytes_per_s": (None if traffic is None
                                 else round(traffic / (dom_ms / n_launch * 1e-3) / 1e9, 1)),
            "counters_from": counters_from,
        },
        "cpu_baseline": cpu,
        "other_configs": other_configs,
        "widened": widened,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
