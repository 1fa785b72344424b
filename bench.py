"""Throughput of the packed 4-direction MDLSTM layer, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload line] [--no-cpu-baseline]

A step is one pass of the whole device path over one batch whose inputs are
already in HBM: scatter the examples onto the packed canvas, forward wavefront
(with the input projection), direction sum + un-packing, reverse wavefront,
weight and input gradients. The metric counts real cell-direction updates only:
4 * sum(h*w) / step time (forward + backward). Prints one JSON line. The
headline batch is the line-like one (32 images of 32 x 256..1024, H = 32), the
largest of the workloads; the word-like batch (packed, as a minimal-padding
stack, and on exact-height rows) and the three-level stack are reported beside
it.

Timing: after the warmup, a breakdown pass of K steps times every kernel
group with HIP events that each dispatch records itself (the library's timing
hook) and names the dominant group; then the K timed steps carry events on
that group's dispatches only, since each timed dispatch costs the stream a few
microseconds.

Also reported: the per-kernel-group times of the breakdown pass; the roofline
of the dominant kernel (its launch time from the timed region) against the
algorithmic flops and minimum bytes of each kernel; the host packer's time;
the word-like images packed, as a minimal-padding stack and on exact-height
rows; the stack; and the CPU oracle (float32, one process per host core) on
the headline batch.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X = {
    "hbm_GBps": 8000.0,          # HBM3E peak
    "fp32_vector_TFLOPs": 157.3,  # 256 CU x 2.4 GHz x 256 fp32 flop/clk/CU
    "fp32_mfma_TFLOPs": 157.3,
    "bf16_mfma_TFLOPs": 2500.0,
    "f16_mfma_TFLOPs": 2500.0,
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="line", choices=["line", "word", "tiny"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-padded", action="store_true")
    ap.add_argument("--no-literal", action="store_true", help="skip the exact-height / skewed-canvas comparison")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the word-like companion runs (packed, as a padded stack, on exact-height rows)")
    ap.add_argument("--no-stack", action="store_true", help="skip the three-level stack companion run")
    ap.add_argument("--no-leaky", action="store_true", help="skip the Leaky LP cell runs (word and line batches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum wall time of the CPU oracle baseline")
    ap.add_argument("--no-overlap", action="store_true",
                    help="weight gradients after the reverse wavefront only (one kernel at a time, for counter runs)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB on the device (counter calibration under rocprofv3 --pmc)")
    return ap.parse_args()


def link_count(rects):
    """Predecessor links of all four directions: an h x w region has h(w-1) left and (h-1)w upper links."""
    return sum(4 * (int(h) * (int(w) - 1) + (int(h) - 1) * int(w)) for (_, _, h, w) in rects)


def kernel_model(info, rects, C, H, x_bytes, nchunks=None, fwd_zero=False, leaky=False):
    """Design bytes and algorithmic flops of one launch of each kernel group (one layer, one step).

    T = computed cells per direction, N = real pixels; every tensor of this
    design (gate stash, gate gradients) is counted once at its storage size, so
    re-reads show up as counter traffic above these bytes. The recurrent flops
    count 10 H^2 per predecessor link (a 5H x H matrix-vector product), both in
    the forward and in the backward pass. fwd_zero: the forward wavefront also
    zeroes h outside the computed regions (no zero-fill launch).
    """
    T = info["computed_cells"]
    N = info["real_pixels"]
    P = info["canvas_h"] * info["canvas_w"]
    G = 5 * H
    R = C + 1 + 2 * H
    # per predecessor link: 10 H^2 for the hidden state into five gates; the Leaky LP cell adds 6 H^2 for the
    # memory state into three (its Vl, Vu products)
    rec = (16 if leaky else 10) * H * H * link_count(rects)
    f = 4  # bytes per float
    extra = {}
    # gate stash floats per cell and direction: (i, f_l, f_u, o) and (g, tanh c, c_l, c_u) per hidden unit; the
    # Leaky LP cell keeps six values per unit
    sw = 6 * H if leaky else 8 * H
    if leaky:
        # dVl, dVu: [s_l | s_u]^T da3 over the computed cells of each direction; s_l, s_u and da3 in, partials out
        extra["wgrad_mem"] = (4 * T * (2 * H + 3 * H) * f, 4 * T * 2 * (2 * H) * (3 * H))
    return {**extra,
        # x (canvas pixels) in for each direction; gate stash and h out; the input projection x Wx + b is
        # computed in the same kernel
        "fwd_wavefront": (4 * T * (C * x_bytes + (sw + H) * f) + (4 * (P - T) * H * f if fwd_zero else 0),
                          rec + 4 * T * 2 * C * G),
        # four h planes in, y out
        "dirsum": (N * 5 * H * f, 3 * N * H),
        # gate stash and dy in (dy once per direction), dA (5H gate pre-activation gradients) out
        "bwd_wavefront": (4 * T * (sw + G) * f + 4 * N * H * f, rec),
        # dA and h in (each h once), x in (once per direction), dx out; the design's own intermediates: each
        # direction's dx share written and read back (4 T C floats), the task partial sums written and read by
        # the reduction (4 groups x R x G floats), the weight gradients out; r^T dA and dA Wx^T on the matrix cores
        "wgrad": (4 * T * (G + H) * f + 4 * T * C * x_bytes + N * C * f + 2 * 4 * T * C * f
                  + 2 * 4 * info.get("wg_groups", 0) * R * G * f + 4 * R * G * f,
                  4 * T * 2 * R * G + 4 * T * 2 * G * C),
        # flat x in, canvas x out
        "scatter": (N * C * x_bytes + P * C * x_bytes, 0),
        # h planes outside the examples zeroed
        "zero_fill": (4 * (P - T) * H * f, 0),
        # shapes without the fused forward: x in, Z = x Wx + b for four directions out
        "projection": (T * C * x_bytes + 4 * T * G * f, 4 * T * 2 * C * G),
    }


def min_bytes(N, C, H, x_bytes):
    """The minimum HBM bytes of one forward + backward step over N real pixels (all four directions), split by
    kernel group: x read by the forward and by the weight gradients, one (h, c) pair per cell-direction written
    by the forward and read back by the reverse wavefront, dy read, y and dx written. Their sum is
    N (2 C x_bytes + 4 C + 72 H); gate stashes, gate gradients and re-reads are the design's, not counted."""
    f = 4
    return {"fwd_wavefront": N * (C * x_bytes + 4 * 2 * H * f), "dirsum": N * H * f,
            "bwd_wavefront": N * (H * f + 4 * 2 * H * f), "wgrad": N * (C * x_bytes + C * f),
            "scatter": 0, "zero_fill": 0, "projection": 0}


# f16 matrix-core products issued per fp32 product of the recurrence: h and da as f16 pairs, the forward's weights
# as three pieces (hidden sizes up to 32), the backward's as a pair
F16_PIECES = {"fwd_wavefront": lambda H: 4 if H <= 32 else 3, "bwd_wavefront": lambda H: 3}


def roofline(kernel, avg_ms, model, bmin, H=None):
    """Fractions of the fp32 peak (algorithmic flops) and of HBM (minimum bytes of the step that belong to this
    kernel); the bound is the larger fraction. The design's own bytes and their HBM fraction are kept beside."""
    nbytes, flops = model[kernel]
    mb = bmin.get(kernel, 0)
    t = avg_ms * 1e-3
    tfs = flops / t / 1e12
    fm = tfs / MI355X["fp32_mfma_TFLOPs"]
    fh = mb / t / 1e9 / MI355X["hbm_GBps"]
    if fm >= fh:
        r = {"bound": "mfma", "achieved": round(tfs, 4), "peak": MI355X["fp32_mfma_TFLOPs"], "unit": "TFLOP/s",
             "frac": round(fm, 6)}
    else:
        r = {"bound": "hbm", "achieved": round(mb / t / 1e9, 2), "peak": MI355X["hbm_GBps"], "unit": "GB/s",
             "frac": round(fh, 6)}
    r.update({"kernel": kernel, "avg_launch_ms": round(avg_ms, 5), "algorithmic_flops": int(flops),
              "fp32_frac": round(fm, 6), "min_bytes": int(mb), "min_bytes_hbm_frac": round(fh, 6),
              "design_bytes": int(nbytes), "design_bytes_hbm_frac": round(nbytes / t / 1e9 / MI355X["hbm_GBps"], 6)})
    if H is not None and kernel in F16_PIECES:
        k = F16_PIECES[kernel](H)
        r["f16_products_per_fp32_product"] = k
        r["f16_issue_frac"] = round(flops * k / t / 1e12 / MI355X["f16_mfma_TFLOPs"], 6)
    return r


# Every source file a kernel group is compiled from; a counter summary holds for the digest of all of them.
_COMMON = ("devmath.h", "kernels.h")
KERNEL_SOURCES = {
    "projection": ("k_proj.hip",), "fwd_wavefront": ("k_fwd16.hip", "k_fwd16.h", "k_fwd16_h32.hip", "k_small.hip", "k_chain.hip")
    + _COMMON,
    "bwd_wavefront": ("k_bwd16.hip", "k_small.hip", "k_chain.hip") + _COMMON,
    "wgrad": ("k_wgrad2.hip", "k_wgrad.hip") + _COMMON, "wgrad_mem": ("k_leaky.hip",) + _COMMON,
    "dirsum": ("k_layout.hip",), "scatter": ("k_layout.hip",), "zero_fill": ("k_layout.hip",),
    "conv_fwd": ("k_conv.hip",), "conv_bwd_data": ("k_conv.hip",), "conv_wgrad": ("k_conv.hip",),
}


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "directional_mdlstm_handwriting_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy
    kernel of known size), or None when there is none or the kernel's source has changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(kernel) or "traffic_bytes_per_launch" not in kv:
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def copy_calibration(mib):
    """A plain device-to-device copy of a known size, for scaling the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy calibration: 3 copies of {mib} MiB", file=sys.stderr, flush=True)


class Runner:
    def __init__(self, wl, mode, device, stream):
        import torch
        from directional_mdlstm_handwriting_amd.layer import (DeviceLayout, DeviceParams, LayerGrads, PackedLayer,
                                                              flat_input)
        from workloads import cotangent
        t0 = time.perf_counter()
        self.dl = DeviceLayout(wl.heights, wl.widths, wl.canvas_w_min[0], wl.sep, mode, device, stream)
        self.pack_s = time.perf_counter() - t0
        self.layer = PackedLayer(self.dl, wl.C, wl.H, wl.x_dtype)
        self.P = DeviceParams.from_host(wl.layers[0], device)
        self.g = LayerGrads.like(self.P)
        self.x = flat_input(wl.xs, wl.x_dtype, device)
        dys = cotangent(wl.seed, wl.heights, wl.widths, wl.H)
        self.dy = torch.as_tensor(np.concatenate([d.reshape(-1) for d in dys]), device=device)
        self.dx = torch.empty(int(sum(x.size for x in wl.xs)), device=device)
        self.stream = stream

    def step(self):
        L, s = self.layer, self.stream
        L.scatter(self.x, s)
        L.forward_dirsum(self.P, s)  # the forward wavefront and the direction sum (beside it where it can)
        L.backward(self.P, self.g, dy_flat=self.dy, dx_flat=self.dx, stream=s)

    def run(self, steps, only):
        """ms per step over `steps` steps, and {kernel group: ms per launch} of the timed groups: every group
        if `only` is None, else that one (each timed dispatch costs the stream a few microseconds)."""
        import torch
        import directional_mdlstm_handwriting_amd as M
        torch.cuda.synchronize()
        M.mdl_timing_report()      # drop anything recorded so far
        M.mdl_timing_only(only)
        M.mdl_timing(True)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(self.stream)
        for _ in range(steps):
            self.step()
        stop.record(self.stream)
        torch.cuda.synchronize()
        M.mdl_timing(False)
        M.mdl_timing_only(None)
        per_kernel = M.mdl_timing_report()
        return start.elapsed_time(stop) / steps, {k: v[0] / v[1] for k, v in per_kernel.items()}

    def time(self, steps, warmup):
        """Untimed warmup; a breakdown pass with every kernel group timed and the weight gradients' overlap
        with the reverse wavefront switched off, so that each group's time is its own (it names the dominant
        group); a second breakdown pass with the overlap on (the launch beside the wavefront, mostly waiting,
        and the rest after it); then the timed region, overlap on, where only the dominant group carries events.
        Returns (ms per step of the timed region, dominant group, its ms per launch there, breakdown without
        the overlap, breakdown with it)."""
        import directional_mdlstm_handwriting_amd as M
        for _ in range(warmup):
            self.step()
        M.mdl_set_wgrad_overlap(0)
        try:
            _, kern = self.run(steps, None)
        finally:
            M.mdl_set_wgrad_overlap(OVERLAP)
        _, kern_ov = self.run(steps, None)
        dom = max(kern, key=kern.get)
        ms, kd = self.run(steps, dom)
        return ms, dom, kd[dom], kern, kern_ov


class SkewRunner:
    """The same layer step with the pages' schedule (mdl_forward_skewed / mdl_backward_skewed: one launch per
    column of the input-skewed canvas), timed with events around the steps only."""

    def __init__(self, wl, mode, device, stream):
        import torch
        import directional_mdlstm_handwriting_amd as M
        from directional_mdlstm_handwriting_amd.layer import (DeviceLayout, DeviceParams, LayerGrads, PackedLayer,
                                                              flat_input)
        from workloads import cotangent
        self.M = M
        self.dl = DeviceLayout(wl.heights, wl.widths, wl.canvas_w_min[0], wl.sep, mode, device, stream)
        self.layer = PackedLayer(self.dl, wl.C, wl.H, wl.x_dtype)
        self.nb = M.mdl_skewed_workspace_size(self.dl.layout, wl.C, wl.H)
        self.ws = torch.empty(self.nb, dtype=torch.uint8, device=device)
        self.P = DeviceParams.from_host(wl.layers[0], device)
        self.g = LayerGrads.like(self.P)
        self.x = flat_input(wl.xs, wl.x_dtype, device)
        dys = cotangent(wl.seed, wl.heights, wl.widths, wl.H)
        self.dy = torch.as_tensor(np.concatenate([d.reshape(-1) for d in dys]), device=device)
        self.dx = torch.empty(int(sum(x.size for x in wl.xs)), device=device)
        self.stream = stream
        self.C, self.H = wl.C, wl.H

    def step(self):
        L, s, P, M = self.layer, self.stream, self.P, self.M
        L.scatter(self.x, s)
        M.mdl_forward_skewed(L.dl.layout, L.dl.desc, L.x_canvas, L.x_dtype, self.C, self.H, P.Wx, P.Ul, P.Uu, P.b,
                             L.h_dirs, self.ws, self.nb, s)
        L.dirsum(s)
        M.mdl_backward_skewed(L.dl.layout, L.dl.desc, L.x_canvas, L.x_dtype, self.C, self.H, P.Wx, P.Ul, P.Uu,
                              L.h_dirs, self.dy, None, self.dx, None, self.g.dWx, self.g.dUl, self.g.dUu, self.g.db,
                              self.ws, self.nb, s)

    def time(self, steps, warmup):
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(self.stream)
        for _ in range(steps):
            self.step()
        stop.record(self.stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps


class StackRunner:
    """The three-level stack (MDLSTM -> 2x4 block conv -> MDLSTM -> block conv -> MDLSTM, each level re-packed)
    and the model head (height collapse, shared fully-connected layer to 80 classes, CTC loss on synthetic
    labels): forward, loss and backward over one batch, timed like Runner."""

    def __init__(self, wl, device, stream):
        import torch
        import directional_mdlstm_handwriting_amd as M
        from directional_mdlstm_handwriting_amd.layer import (CTCHead, DeviceParams, LayerGrads, PackedStack,
                                                              flat_input)
        from workloads import ctc_labels, head_params
        Hs = [P.H for P in wl.layers]
        couts = [c.b.shape[0] for c in wl.convs]
        self.st = PackedStack(wl.heights, wl.widths, wl.C, Hs, couts, wl.canvas_w_min, sep=wl.sep, device=device)
        self.params = [DeviceParams.from_host(P, device) for P in wl.layers]
        self.convs = [(torch.as_tensor(c.W, device=device), torch.as_tensor(c.b, device=device)) for c in wl.convs]
        self.lg = [LayerGrads.like(p) for p in self.params]
        self.cg = [(torch.empty_like(W), torch.empty_like(b)) for W, b in self.convs]
        self.x = flat_input(wl.xs, "f32", device)
        last = self.st.levels[-1]
        _, real = M.mdl_layout_rects(last.dl.layout)
        frames = real[:, 3]
        Wfc, bfc = head_params(wl.seed, last.H)
        self.head = CTCHead(last.dl, last.H, Wfc.shape[1], ctc_labels(wl.seed, frames))
        self.Wfc, self.bfc = torch.as_tensor(Wfc, device=device), torch.as_tensor(bfc, device=device)
        self.dWfc, self.dbfc = torch.empty_like(self.Wfc), torch.empty_like(self.bfc)
        self.frames = int(frames.sum())
        self.dx = torch.empty(int(sum(x.size for x in wl.xs)), device=device)
        self.stream = stream

    def step(self):
        y = self.st.forward(self.x, self.params, self.convs, self.stream)
        self.head.run(y, self.Wfc, self.bfc, self.dWfc, self.dbfc, stream=self.stream)
        self.st.backward(self.params, self.convs, self.head.dy, self.lg, self.cg, dx_flat=self.dx,
                         stream=self.stream)

    def time(self, steps, warmup):
        """ms per step with no events inside the timed region, and the breakdown pass's ms per step of each
        kernel group (summed over the levels)."""
        import torch
        import directional_mdlstm_handwriting_amd as M
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        M.mdl_timing_report()
        M.mdl_timing_only(None)
        M.mdl_timing(True)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        M.mdl_timing(False)
        per_kernel = {k: v[0] / steps for k, v in M.mdl_timing_report().items()}
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(self.stream)
        for _ in range(steps):
            self.step()
        stop.record(self.stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps, per_kernel


_CPU_WL = {}


def _cpu_init(name, seed):
    """Worker start-up: one BLAS thread, the workload drawn once."""
    from workloads import make_workload
    _CPU_WL["wl"] = make_workload(name, seed)


def _cpu_part(idx):
    """The oracle, float32, on the examples `idx` of the worker's workload (packed on their own canvas: examples
    are independent on the canvas, so this is the batch's work split by example): pack + forward + backward."""
    import numpy as np
    from oracle import mdlstm as omd, pack as opack
    from workloads import cotangent
    wl = _CPU_WL["wl"]
    h, w = wl.heights[idx], wl.widths[idx]
    xs = [wl.xs[i] for i in idx]
    dys = cotangent(wl.seed, h, w, wl.H)
    num = omd.Num(np.float32)
    lay = opack.pack_alg1(h, w, wl.canvas_w_min[0], wl.sep)
    ys, cache = omd.layer_forward(lay, xs, wl.layers[0], num=num)
    omd.layer_backward(lay, wl.layers[0], cache, dys=dys, num=num)
    return len(idx)


def cpu_baseline(wl, min_seconds):
    """The oracle (its per-diagonal form, float32 arrays) on the whole batch, split over one worker process per
    host core: examples dealt by the greedy largest-cost-into-least-loaded rule (cost h w (h + w)), each worker
    single-threaded. Passes of pack + forward + backward are repeated until min_seconds of wall time have
    passed; the rate is real cell-direction updates per second."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))
    cores = max(1, min(cores, wl.n))
    cost = [int(h) * int(w) * (int(h) + int(w)) for h, w in zip(wl.heights, wl.widths)]
    bins = [[] for _ in range(cores)]
    load = [0] * cores
    for e in sorted(range(wl.n), key=lambda e: -cost[e]):
        k = int(np.argmin(load))
        bins[k].append(e)
        load[k] += cost[e]
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(cores, initializer=_cpu_init, initargs=(wl.name, wl.seed)) as pool:
            pool.map(_cpu_part, [[bins[k][0]] for k in range(cores)])  # start-up and imports, untimed
            passes = 0
            t0 = time.perf_counter()
            while True:
                pool.map(_cpu_part, bins, chunksize=1)
                passes += 1
                t = time.perf_counter() - t0
                if t >= min_seconds:
                    break
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    N = int(np.sum(wl.heights.astype(np.int64) * wl.widths))
    return {"value": 4 * N * passes / t, "unit": "cell-direction updates/s", "cores": cores, "kind": "oracle",
            "sample": f"all {wl.n} {wl.name} images (seed {wl.seed}, {N} pixels), {passes} passes of pack + "
                      f"forward + backward of the oracle's per-diagonal form in float32, split by example over "
                      f"{cores} single-threaded worker processes, {t:.1f} s"}


def step_roofline(model, bmin, ms):
    """Whole-step fractions: all algorithmic flops against the fp32 peak, all minimum bytes against HBM."""
    flops = sum(f for _, f in model.values())
    mb = sum(bmin.values())
    t = ms * 1e-3
    return {"algorithmic_flops": int(flops), "fp32_frac": round(flops / t / 1e12 / MI355X["fp32_mfma_TFLOPs"], 6),
            "min_bytes": int(mb), "min_bytes_hbm_frac": round(mb / t / 1e9 / MI355X["hbm_GBps"], 6)}


def layer_report(runner, wl, ms, kern):
    """Per-kernel rooflines of one layer's step, and the model the fractions come from."""
    import directional_mdlstm_handwriting_amd as M
    info = runner.dl.info
    rects, _ = M.mdl_layout_rects(runner.dl.layout)
    xb = 2 if wl.x_dtype == "bf16" else 4
    model = kernel_model(info, rects, wl.C, wl.H, xb, fwd_zero="zero_fill" not in kern,
                         leaky=hasattr(wl.layers[0], "Vl"))
    bmin = min_bytes(info["real_pixels"], wl.C, wl.H, xb)
    per = {k: roofline(k, v, model, bmin, wl.H) for k, v in kern.items() if k in model}
    return model, bmin, per


# the weight gradients' overlap with the reverse wavefront in the warmup, the second breakdown pass and the
# timed region (mdl_set_wgrad_overlap mode: 1 on, 0 off)
OVERLAP = 1


def main():
    global OVERLAP
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the examples of a batch would be split across GPUs, one process each)", file=sys.stderr)
        sys.exit(2)
    from workloads import make_workload
    wl = make_workload(args.workload, args.seed)
    N = int(np.sum(wl.heights.astype(np.int64) * wl.widths))

    # the CPU oracle first, before this process touches the GPU (its workers are fresh processes)
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_seconds)

    import torch
    import directional_mdlstm_handwriting_amd as M
    device = "cuda:0"
    torch.cuda.set_device(0)
    OVERLAP = 0 if args.no_overlap else 1
    M.mdl_set_wgrad_overlap(OVERLAP)
    stream = torch.cuda.current_stream()

    print(f"bench: {wl.name} packed", file=sys.stderr, flush=True)
    torch.cuda.reset_peak_memory_stats()
    packed = Runner(wl, "packed", device, stream)
    ms, dom, dom_ms, kern, kern_ov = packed.time(args.steps, args.warmup)
    info = packed.dl.info
    value = 4 * N / (ms * 1e-3)

    # host packer alone (median of repeats)
    reps = []
    for _ in range(20):
        t0 = time.perf_counter()
        M.mdl_pack(wl.heights, wl.widths, wl.canvas_w_min[0], wl.sep)
        reps.append(time.perf_counter() - t0)
    pack_us = float(np.median(reps) * 1e6)

    # roofline of the dominant kernel group, from HIP events its dispatches recorded in the timed region
    model, bmin, per_kernel = layer_report(packed, wl, ms, kern)
    roof = roofline(dom, dom_ms, model, bmin, wl.H)
    roof["traffic"] = measured_traffic(dom, wl.name)
    roof["dependent_steps"] = info["max_depth"]
    roof["us_per_dependent_step"] = round(dom_ms * 1e3 / info["max_depth"], 4)
    H, C = wl.H, wl.C
    bf16 = wl.x_dtype == "bf16"
    out = {
        "metric": "MDLSTM cell-direction updates/sec (fwd+bwd) on packed canvas; % of roofline",
        "value": value,
        "unit": "cell-direction updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 input, " if bf16 else "") + "f32 (recurrent products on f16 matrix cores, operands "
                 "split into f16 pieces, fp32 accumulation)",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.n} images, C={C}, H={H}, seed {wl.seed}, canvas "
                               f"{info['canvas_h']}x{info['canvas_w']}",
                   "real_pixels": N, "computed_cells": info["computed_cells"],
                   "max_depth": info["max_depth"], "parallelism": "single GPU"},
        "roofline": roof,
        "step_roofline": step_roofline(model, bmin, ms),
        "kernels_ms": {k: round(v, 5) for k, v in kern.items()},
        "kernels_ms_source": "breakdown pass before the timed region, events on every dispatch, the weight "
                             "gradients run after the reverse wavefront",
        "kernels_ms_overlap": {k: round(v, 5) for k, v in kern_ov.items()},
        "kernels_ms_overlap_source": ("second breakdown pass, the weight gradients' overlap on as in the timed "
                                      "region: wgrad_overlap spans the launch beside the reverse wavefront "
                                      "(mostly waiting for its units to finish), wgrad the tasks left after it; "
                                      "dirsum_overlap and dirsum likewise for the direction sum beside the "
                                      "forward wavefront"
                                      if OVERLAP else "the weight gradients' overlap is off in this run"),
        "kernels_roofline": {k: {kk: r[kk] for kk in ("bound", "frac", "fp32_frac", "min_bytes_hbm_frac",
                                                       "design_bytes_hbm_frac")}
                             for k, r in per_kernel.items()},
        "pack_host_us": round(pack_us, 2),
    }
    out["config"]["canvas_waste"] = round(1.0 - N / (info["canvas_h"] * info["canvas_w"]), 4)
    del packed
    torch.cuda.empty_cache()

    # the word-like batch: packed, as a minimal-padding stack, and on exact-height rows (the pages' own layout)
    ww = wl if wl.name == "word" else make_workload("word", args.seed)
    Nw = int(np.sum(ww.heights.astype(np.int64) * ww.widths))
    if wl.name == "tiny":
        ww = None
    if ww is not None and ww is wl:
        # the headline is the word batch itself
        wms, wk, wi = ms, kern, info
        peak_packed = torch.cuda.max_memory_allocated()
    elif ww is not None and not args.no_other:
        print("bench: word packed", file=sys.stderr, flush=True)
        torch.cuda.reset_peak_memory_stats()
        rw = Runner(ww, "packed", device, stream)
        wms, _, _, wk, _ = rw.time(args.steps, 2)
        peak_packed = torch.cuda.max_memory_allocated()
        wi = rw.dl.info
        wmodel, wbmin, wper = layer_report(rw, ww, wms, wk)
        out["word_workload"] = {
            "workload": f"word: {ww.n} images, C={ww.C}, H={ww.H}, seed {ww.seed}, canvas "
                        f"{wi['canvas_h']}x{wi['canvas_w']}",
            "value": 4 * Nw / (wms * 1e-3), "unit": "cell-direction updates/s", "ms_per_step": wms,
            "max_depth": wi["max_depth"], "kernels_ms": {k: round(v, 5) for k, v in wk.items()},
            "kernels_roofline": {k: {kk: r[kk] for kk in ("bound", "frac", "fp32_frac", "min_bytes_hbm_frac")}
                                 for k, r in wper.items()},
            "step_roofline": step_roofline(wmodel, wbmin, wms),
        }
        del rw
        torch.cuda.empty_cache()
    else:
        ww = None
    if ww is not None:
        if not args.no_padded:
            print("bench: word padded", file=sys.stderr, flush=True)
            torch.cuda.reset_peak_memory_stats()
            padded = Runner(ww, "padded", device, stream)
            pms, _, _, pk, _ = padded.time(max(5, args.steps // 2), 2)
            peak_padded = torch.cuda.max_memory_allocated()
            pinfo = padded.dl.info
            out["packed_vs_padded"] = {
                "workload": "the word-like batch above",
                "ms_per_step_packed": wms, "ms_per_step_padded": pms, "speedup": pms / wms,
                "padded_cell_fraction": round(1.0 - Nw / pinfo["computed_cells"], 4),
                # padded zeros relative to the real pixels (the ZPR measure of the speech-batching page)
                "zpr": round((pinfo["computed_cells"] - Nw) / Nw, 4),
                "computed_cells_padded": pinfo["computed_cells"],
                "computed_cell_direction_updates_per_s_padded": 4 * pinfo["computed_cells"] / (pms * 1e-3),
                "peak_device_bytes_packed": int(peak_packed), "peak_device_bytes_padded": int(peak_padded),
                "padded_kernels_ms": {k: round(v, 5) for k, v in pk.items()},
                "pages_context": "6.6x for IAM words: whole-model training epochs, 2x GTX 1080, batch 20 padded vs "
                                 "200 packed (No Padding Please, Table IV)",
            }
            del padded
            torch.cuda.empty_cache()

        # the pages' own layout for the same images: exact-height rows, whole canvas skewed for column-parallel
        # steps; its canvas, skew padding and dependent-step count next to this schedule's, and this schedule
        # timed on the exact-height canvas
        if not args.no_literal:
            print("bench: word on exact-height rows", file=sys.stderr, flush=True)

            def skewed(li):
                Hc, Wc = li["canvas_h"], li["canvas_w"]
                cells = Hc * (Wc + Hc - 1)
                return {"canvas": f"{Hc}x{Wc}", "canvas_waste": round(1.0 - Nw / (Hc * Wc), 4),
                        "skewed_cells": cells, "skewed_padding_fraction": round(1.0 - Nw / cells, 4),
                        "global_depth": Hc + Wc - 1, "cells_per_column": Hc}
            ex = Runner(ww, "exact", device, stream)
            ems, _, _, ek, _ = ex.time(max(5, args.steps // 2), 2)
            ei = ex.dl.info
            del ex
            torch.cuda.empty_cache()
            print("bench: word, the skewed column schedule", file=sys.stderr, flush=True)
            sk = SkewRunner(ww, "exact", device, stream)
            sms = sk.time(3, 1)
            del sk
            torch.cuda.empty_cache()
            out["paper_literal_layout"] = {
                "workload": "the word-like batch above",
                "alg1_rows": skewed(wi), "exact_height_rows": skewed(ei),
                "local_depth": wi["max_depth"], "widest_local_diagonal": wi["max_diag"],
                "ms_per_step_alg1": wms, "ms_per_step_exact_height": ems,
                "ms_per_step_skewed_columns_exact_height": sms,
                "skewed_column_steps_per_pass": ei["canvas_h"] + ei["canvas_w"] - 1,
                "skewed_note": "the pages' schedule on the exact-height canvas: one launch per skewed column, "
                               "every skewed cell computed and masked, fp32 (mdl_forward_skewed / "
                               "mdl_backward_skewed); the local-diagonal schedule on the same canvas is "
                               "ms_per_step_exact_height",
                "exact_height_kernels_ms": {k: round(v, 5) for k, v in ek.items()},
            }

    # the three-level stack of the pages' model (128 word-like images) and its head, timed the same way
    if not args.no_stack and wl.name != "tiny":
        print("bench: stack", file=sys.stderr, flush=True)
        ws_ = make_workload("stack", args.seed)
        sr = StackRunner(ws_, device, stream)
        sms, sk = sr.time(max(5, args.steps // 2), 2)
        lv = []
        for lay, P in zip(sr.st.levels, ws_.layers):
            li = lay.dl.info
            lv.append({"canvas": f"{li['canvas_h']}x{li['canvas_w']}", "real_pixels": li["real_pixels"],
                       "C": P.C, "H": P.H, "max_depth": li["max_depth"]})
        Ns = sum(v["real_pixels"] for v in lv)
        loss = sr.head.loss.float().cpu().numpy()
        out["stack_workload"] = {
            "workload": f"stack: {ws_.n} word-like images, MDLSTM H={[P.H for P in ws_.layers]} with 2x4 block "
                        f"convs to {[c.b.shape[0] for c in ws_.convs]} channels, shared fully-connected head to "
                        f"{sr.head.K} classes and CTC loss on synthetic labels, seed {ws_.seed}",
            "ctc_frames": sr.frames, "ctc_loss_mean": float(loss.mean()),
            "value": 4 * Ns / (sms * 1e-3), "unit": "cell-direction updates/s (all three levels)",
            "ms_per_step": sms, "levels": lv,
            "kernels_ms_per_step": {k: round(v, 5) for k, v in sk.items()},
        }
        del sr

    # the Leaky LP cell (the pages' stable cell) on the same word and line batches, timed the same way
    if not args.no_leaky and wl.name != "tiny":
        out["leaky_cell"] = {}
        for nm in ("line", "word"):
            print(f"bench: {nm} with the Leaky LP cell", file=sys.stderr, flush=True)
            wk_ = make_workload(nm, args.seed, cell="leaky")
            Nk = int(np.sum(wk_.heights.astype(np.int64) * wk_.widths))
            rk = Runner(wk_, "packed", device, stream)
            kms, kdom, kdom_ms, kk, _ = rk.time(max(5, args.steps // 2), 2)
            kmodel, kbmin, kper = layer_report(rk, wk_, kms, kk)
            kroof = roofline(kdom, kdom_ms, kmodel, kbmin, wk_.H)
            kroof["dependent_steps"] = rk.dl.info["max_depth"]
            kroof["us_per_dependent_step"] = round(kdom_ms * 1e3 / rk.dl.info["max_depth"], 4)
            out["leaky_cell"][nm] = {
                "workload": f"{nm}: {wk_.n} images, C={wk_.C}, H={wk_.H}, seed {wk_.seed}, Leaky LP cell",
                "value": 4 * Nk / (kms * 1e-3), "unit": "cell-direction updates/s", "ms_per_step": kms,
                "dtype": ("f32 (recurrent products on 16-bit matrix cores, operands split into pieces: forward f16, "
                          "reverse bf16; fp32 accumulation)" + (", bf16 input" if wk_.x_dtype == "bf16" else "")),
                "roofline": kroof, "step_roofline": step_roofline(kmodel, kbmin, kms),
                "kernels_ms": {k: round(v, 5) for k, v in kk.items()},
                "kernels_roofline": {k: {kk2: r[kk2] for kk2 in ("bound", "frac", "fp32_frac", "min_bytes_hbm_frac")}
                                     for k, r in kper.items()},
            }
            del rk
            torch.cuda.empty_cache()

    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    if args.copy_calib:
        copy_calibration(args.copy_calib)


if __name__ == "__main__":
    main()
