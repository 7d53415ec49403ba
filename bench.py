#!/usr/bin/env python3
"""Benchmark of the NF4 + LoRA linear layer on one MI355X.

Headline (`value`): a step is the forward (Y, U) and the backward (dX, dA,
dB) of all seven linears of a 7B-style decoder block (q/k/v/o 4096x4096,
gate/up 11008x4096, down 4096x11008; NF4 blocks of 64, double quantisation in
groups of 256), T = 8192 tokens, r = 64, alpha = 16.  The weights are
quantised once before timing (a load-time cost); every linear call of every
step dequantises its weight again: at 2048 tokens and more once per call into
a 16-bit workspace copy that the GEMM streams by DMA, below that inside the
GEMM, per 256-token tile (the line also carries the headline workload timed
with the in-GEMM decode, `block_7b_in_lds_decode`).  The same line carries the other
workloads: the 4096x4096 attention projection at 4096 tokens, the 65B-style
block at 2048 tokens (fwd+bwd) and at 16 tokens (forward, skinny path, GB/s),
the bulk quantize / dequantize of an 8192x22016 weight, and the rows built
after those (merge, AdamW, lora_dropout, storage/compute variants).

Prints one JSON line.  Timing uses HIP events on the stream the library
launches on: whole steps for `value`, and per-kernel events (the library's
timing hook) for the roofline of the dominant kernel.  The CPU oracle is
timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E

HEADLINE = "block_7b"            # the training workload with the most flops per step
# the headline workload again with the weight decoded into LDS inside the GEMM
# for every 256-token tile (the path below qlora_pre_dequant_min_tokens())
HEADLINE_LDS = "block_7b_in_lds_decode"
NEVER = 2 ** 63 - 1
SMALL_TRAIN = "attn_4096"        # one 4096 x 4096 linear, 4096 tokens
TRAIN_65B = "block_65b_train"
DECODE_65B = "block_65b_decode"
BULK = "bulk_8192x22016"
MERGE = "merge_8192x22016"
DROPOUT_P = 0.05              # lora_dropout of the adapter configs on the pages


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    # the clock ramps over the first ~10-30 ms of load; a step count alone
    # does not cover that for short steps, so warm-up also lasts at least this
    ap.add_argument("--warmup-seconds", type=float, default=1.0)
    ap.add_argument("--bulk-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1024,
                    help="tokens of the 7B block the CPU oracle is timed on")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle step until this much time has passed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--only", default=None,
                    help="comma-separated subset of: block_7b, block_7b_in_lds_decode, "
                         "attn_4096, block_65b_train, "
                         "block_65b_decode, bulk, adamw, dropout, variants (profiling runs)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t helpers through the HIP runtime torch has loaded."""

    def __init__(self):
        import torch
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.h = ctypes.CDLL(path)
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    # hipEventDisableSystemFence: the event only takes a timestamp.  A default
    # event's system-scope release writes back and invalidates the caches,
    # which left about 5 us of idle GPU around each bracketed kernel; the
    # timestamps are read only after a full synchronize, so nothing here needs
    # the fence.  The start and stop of a whole timed region keep it.
    DISABLE_SYSTEM_FENCE = 0x20000000

    def new(self, fence=False):
        ev = ctypes.c_void_p()
        if fence:
            rc = self.h.hipEventCreate(ctypes.byref(ev))
        else:
            rc = self.h.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        self.pool.append(ev.value)
        return ev.value

    def record(self, ev, stream):
        rc = self.h.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def ms(self, a, b):
        self.h.hipEventSynchronize(ctypes.c_void_p(b))
        out = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(out.value)

    def close(self):
        for ev in self.pool:
            self.h.hipEventDestroy(ctypes.c_void_p(ev))
        self.pool = []


def flops_fwd_bwd(t, n, k, r):
    """Algorithmic FLOPs of forward + backward (dX, dA, dB; no dW)."""
    return 4 * t * n * k + 6 * t * r * (n + k)


def packed_bytes(n_elems):
    n_b = n_elems // 64
    n_g = (n_b + 255) // 256
    return n_elems // 2 + n_b + 4 * n_g + 4


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_nf4_quantized_06_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip().lstrip("-* ")
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def to_dev_bf16(bits, dev, dtype="bf16"):
    """16-bit bit patterns to a device tensor of that type (bf16 or fp16)."""
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)
    return t.view(torch.float16 if dtype == "fp16" else torch.bfloat16)


class LinearSet:
    """Device-resident inputs, packed weights and outputs of a workload."""

    def __init__(self, wl, dev, tokens=None, backward=True, dropout=None, dtype="bf16",
                 double_quant=True, weights=None):
        import torch

        import bit_nf4_quantized_06_amd as q
        import workloads as WL
        self.wl = wl
        self.dropout = dropout          # lora_dropout probability, or None
        self.T = wl.tokens if tokens is None else tokens
        self.r, self.alpha = wl.rank, wl.alpha
        self.backward = backward and wl.backward
        self.items = []
        for li, lin in enumerate(wl.linears):
            inp = WL.linear_inputs(wl, li, tokens=self.T, dtype=dtype,
                                   with_weight=weights is None)
            if weights is None:
                wq = q.qlora_nf4_quantize(torch.from_numpy(inp["w"]).to(dev),
                                          double_quant=double_quant, compute_dtype=dtype)
            else:
                wq = weights[li]      # the same packed weight (same draws), another token count
            it = {"lin": lin, "wq": wq, "X": to_dev_bf16(inp["x"], dev, dtype),
                  "A": to_dev_bf16(inp["a"], dev, dtype), "B": to_dev_bf16(inp["b"], dev, dtype)}
            n, k, r, t = lin.out_features, lin.in_features, self.r, self.T
            it["Y"] = torch.empty(t, n, dtype=wq.dtype16, device=dev)
            it["U"] = torch.empty(t, r, dtype=wq.dtype16, device=dev)
            wsz = q.qlora_linear_workspace if dropout is None else q.qlora_linear_workspace_dropout
            it["wsf"] = torch.empty(wsz(t, n, k, r, False), dtype=torch.uint8, device=dev)
            if dropout is not None:
                it["keep"] = torch.empty((t + 3) // 4, k // 2, dtype=torch.uint8, device=dev)
                # the dropped input, kept for the backward as autograd keeps a
                # dropout's output
                it["Xd"] = torch.empty(t, k, dtype=wq.dtype16, device=dev)
            if self.backward and "dy" in inp:
                it["dY"] = to_dev_bf16(inp["dy"], dev, dtype)
                it["dX"] = torch.empty(t, k, dtype=wq.dtype16, device=dev)
                it["dA"] = torch.empty(r, k, dtype=torch.float32, device=dev)
                it["dB"] = torch.empty(n, r, dtype=torch.float32, device=dev)
                it["wsb"] = torch.empty(wsz(t, n, k, r, True), dtype=torch.uint8, device=dev)
            self.items.append(it)
            del inp
        torch.cuda.synchronize()

    def step(self, hook=None):
        """One step: the forward of every linear, then (training workloads)
        the backward of every linear.  hook(li, "fwd" | "bwd"), if given, runs
        before each call (the kernel-timing pass sets its events there)."""
        import bit_nf4_quantized_06_amd as q
        for li, it in enumerate(self.items):
            if hook:
                hook(li, "fwd")
            if self.dropout is not None:
                q.qlora_linear_fwd_dropout(it["wq"], it["X"], it["A"], it["B"], self.alpha,
                                           self.dropout, 1234, li, Y=it["Y"], U_save=it["U"],
                                           keep_save=it["keep"], workspace=it["wsf"],
                                           X_dropped_save=it["Xd"])
            else:
                q.qlora_linear_fwd(it["wq"], it["X"], it["A"], it["B"], self.alpha, Y=it["Y"],
                                   U_save=it["U"], workspace=it["wsf"])
        if not self.backward:
            return
        for li in reversed(range(len(self.items))):
            it = self.items[li]
            if "dY" not in it:
                continue
            if hook:
                hook(li, "bwd")
            if self.dropout is not None:
                q.qlora_linear_bwd_dropout(it["wq"], it["X"], it["dY"], it["A"], it["B"],
                                           self.alpha, self.dropout, 1234, li,
                                           keep_saved=it["keep"], U_saved=it["U"],
                                           dX=it["dX"], dA=it["dA"], dB=it["dB"],
                                           workspace=it["wsb"], X_dropped_saved=it["Xd"])
            else:
                q.qlora_linear_bwd(it["wq"], it["X"], it["dY"], it["A"], it["B"], self.alpha,
                                   U_saved=it["U"], dX=it["dX"], dA=it["dA"], dB=it["dB"],
                                   workspace=it["wsb"])

    def flops(self):
        tot = 0
        for it in self.items:
            n, k = it["lin"].out_features, it["lin"].in_features
            if self.backward:
                tot += flops_fwd_bwd(self.T, n, k, self.r)
            else:
                tot += 2 * self.T * n * k + 2 * self.T * self.r * (n + k)
        return tot

    def gemm_flops(self):
        """Algorithmic flops of the fused forward GEMMs and of the dX GEMMs
        (the LoRA seed included) over one step."""
        fwd = dx = 0
        for it in self.items:
            n, k, t, r = it["lin"].out_features, it["lin"].in_features, self.T, self.r
            fwd += 2 * t * n * (k + r)
            if self.backward:
                dx += 2 * t * k * (n + r)
        return fwd, dx

    def hbm_bytes_fwd(self):
        """Algorithmic bytes of a forward-only step: packed weights, A, B, X
        and Y once each."""
        return sum(packed_bytes(it["lin"].out_features * it["lin"].in_features)
                   + 2 * (it["A"].numel() + it["B"].numel() + it["X"].numel() + it["Y"].numel())
                   for it in self.items)


def warm_up(ls, steps, seconds):
    """At least `steps` steps and at least `seconds` of steady work: the clock
    of the part ramps over the first ~10-30 ms of load and settles
    (power-limited) after that, so a step count alone is not enough for a
    short step.  Returns (steps run, seconds)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    for _ in range(steps):
        ls.step()
        n += 1
    torch.cuda.synchronize()
    chunk = max(1, steps)
    while time.perf_counter() - t0 < seconds:
        for _ in range(chunk):
            ls.step()
        n += chunk
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def time_steps(ls, ev, steps, warmup, warmup_s, kernel_timing=True):
    """Whole-step time (ms) over `steps` timed steps with no event between
    their kernels, then (kernel_timing) the same number of steps again with
    a pair of HIP events around every fused GEMM (or skinny forward) on the
    library's stream; returns per-kernel totals and launch counts."""
    import torch

    from bit_nf4_quantized_06_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    wsteps, wsec = warm_up(ls, warmup, warmup_s)
    start, stop = ev.new(fence=True), ev.new(fence=True)
    t_wall = time.perf_counter()
    ev.record(start, stream)
    for _ in range(steps):
        ls.step()
    ev.record(stop, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total = ev.ms(start, stop)
    res = {"ms_per_step": total / steps, "wall_s": wall, "warmup_steps_run": wsteps,
           "warmup_s": wsec}
    if not kernel_timing:
        return res
    pairs = {"fwd": [], "dx": []}

    def hook(li, phase):
        if phase == "fwd":
            p = (ev.new(), ev.new())
            lib.qlora_set_timing_events(0, p[0], p[1])
            lib.qlora_set_timing_events(1, None, None)
            pairs["fwd"].append(p)
        else:
            p = (ev.new(), ev.new())
            lib.qlora_set_timing_events(0, None, None)
            lib.qlora_set_timing_events(1, p[0], p[1])
            pairs["dx"].append(p)

    start2, stop2 = ev.new(fence=True), ev.new(fence=True)
    ev.record(start2, stream)
    for _ in range(steps):
        ls.step(hook)
    ev.record(stop2, stream)
    torch.cuda.synchronize()
    lib.qlora_set_timing_events(0, None, None)
    lib.qlora_set_timing_events(1, None, None)
    res["ms_per_step_with_kernel_events"] = ev.ms(start2, stop2) / steps
    for k, v in pairs.items():
        if v:
            res[k] = {"total_ms": sum(ev.ms(a, b) for a, b in v) / steps,
                      "launches": len(v) // steps}
    return res


def time_graph(ls, ev, steps):
    """The same step captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed `steps` times: the per-call host work (argument checks, kernel
    launches) leaves the timed region, as in a serving loop.  Returns ms per
    step, or None if capture fails."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            ls.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ls.step()
        torch.cuda.synchronize()
    except Exception as e:  # pragma: no cover - reported, not fatal
        print(f"[bench] graph capture failed: {e}", file=sys.stderr, flush=True)
        return None
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(max(3, steps // 4)):
        g.replay()
    torch.cuda.synchronize()
    start, stop = ev.new(fence=True), ev.new(fence=True)
    ev.record(start, stream)
    for _ in range(steps):
        g.replay()
    ev.record(stop, stream)
    torch.cuda.synchronize()
    ms = ev.ms(start, stop) / steps
    del g
    return ms


def training_config(name, ev, dev, steps, warmup, warmup_s, keep_weights=False,
                    traffic_name=None):
    """fwd+bwd TFLOP/s of a training workload and the roofline of its
    dominant fused GEMM (achieved = its algorithmic flops over its event-timed
    duration, summed over the step's launches of it)."""
    import torch

    import workloads as WL
    wl = WL.WORKLOADS[name]
    ls = LinearSet(wl, dev)
    tm = time_steps(ls, ev, steps, warmup, warmup_s)
    fl = ls.flops()
    fwd_fl, dx_fl = ls.gemm_flops()
    kern = {"qlora_gemm_fwd": (tm["fwd"], fwd_fl), "qlora_gemm_dx": (tm["dx"], dx_fl)}
    dom = max(kern, key=lambda k: kern[k][0]["total_ms"])
    kt, kfl = kern[dom]
    achieved = kfl / (kt["total_ms"] / 1e3) / 1e12
    digest = source_digest("gemm.hip", "device_common.h")
    shapes = sorted({(it["lin"].out_features, it["lin"].in_features) for it in ls.items})
    from bit_nf4_quantized_06_amd import qlora_pre_dequant_min_tokens
    path = ("weight dequantised once per call into a 16-bit workspace copy, both GEMM "
            "operands by DMA" if ls.T >= qlora_pre_dequant_min_tokens() else
            "weight tiles decoded into LDS inside the GEMM, once per 256-token tile")
    out = {
        "gemm_weight_path": path,
        "ms_per_step": round(tm["ms_per_step"], 4),
        "TFLOPs": round(fl / (tm["ms_per_step"] / 1e3) / 1e12, 2),
        "mfma_frac": round(fl / (tm["ms_per_step"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": fl,
        "tokens": ls.T, "rank": ls.r, "alpha": ls.alpha, "linears": len(ls.items),
        "shapes": [f"{n}x{k}" for n, k in shapes],
        "warmup_steps_run": tm["warmup_steps_run"], "warmup_s": round(tm["warmup_s"], 3),
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic(dom, traffic_name or name, digest),
                     "flops_per_launch": kfl // max(1, kt["launches"]),
                     "avg_launch_ms": round(kt["total_ms"] / max(1, kt["launches"]), 4),
                     "launches_per_step": kt["launches"], "source_digest": digest},
        "kernels_ms_per_step": {k: round(v[0]["total_ms"], 4) for k, v in kern.items()},
        "ms_per_step_with_kernel_events": round(tm["ms_per_step_with_kernel_events"], 4),
    }
    gms = time_graph(ls, ev, steps)
    if gms is not None:
        out["graph_replay"] = {"ms_per_step": round(gms, 4),
                               "TFLOPs": round(fl / (gms / 1e3) / 1e12, 2)}
    weights = [it["wq"] for it in ls.items] if keep_weights else None
    del ls
    torch.cuda.empty_cache()
    return (out, weights) if keep_weights else out


def decode_config(name, ev, dev, steps, warmup, warmup_s, weights=None):
    """Forward-only skinny workload: GB/s of the algorithmic bytes (packed
    weights, A, B, X, Y) against 8 TB/s, and the skinny forward's own rate."""
    import torch

    import workloads as WL
    wl = WL.WORKLOADS[name]
    ls = LinearSet(wl, dev, backward=False, weights=weights)
    tm = time_steps(ls, ev, steps, warmup, warmup_s)
    by = ls.hbm_bytes_fwd()
    fl = ls.flops()
    kt = tm["fwd"]
    gbps = by / (tm["ms_per_step"] / 1e3) / 1e9
    kgbps = by / (kt["total_ms"] / 1e3) / 1e9
    digest = source_digest("gemv.hip", "device_common.h")
    out = {
        "ms_per_step": round(tm["ms_per_step"], 4),
        "GBps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "TFLOPs": round(fl / (tm["ms_per_step"] / 1e3) / 1e12, 3),
        "bytes_per_step": by, "tokens": ls.T, "linears": len(ls.items),
        "warmup_steps_run": tm["warmup_steps_run"], "warmup_s": round(tm["warmup_s"], 3),
        "roofline": {"kernel": "qlora_gemv", "bound": "hbm", "achieved": round(kgbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(kgbps / PEAK_HBM_GBPS, 4),
                     "traffic": profiled_traffic("qlora_gemv", name, digest),
                     "bytes_per_launch": by // max(1, kt["launches"]),
                     "avg_launch_ms": round(kt["total_ms"] / max(1, kt["launches"]), 4),
                     "launches_per_step": kt["launches"], "source_digest": digest},
        "ms_per_step_with_kernel_events": round(tm["ms_per_step_with_kernel_events"], 4),
    }
    gms = time_graph(ls, ev, steps)
    if gms is not None:
        gg = by / (gms / 1e3) / 1e9
        out["graph_replay"] = {"ms_per_step": round(gms, 4), "GBps": round(gg, 1),
                               "hbm_frac": round(gg / PEAK_HBM_GBPS, 4)}
    del ls
    torch.cuda.empty_cache()
    return out


def time_bulk(ev, dev, reps):
    import numpy as np
    import torch

    import bit_nf4_quantized_06_amd as q
    import workloads as WL
    from bit_nf4_quantized_06_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    wl = WL.WORKLOADS[BULK]
    lin = wl.linears[0]
    mwl = WL.WORKLOADS[MERGE]          # the same weight with a rank-64 adapter
    minp = WL.linear_inputs(mwl, 0)
    w = torch.from_numpy(minp["w"]).to(dev)
    A = torch.from_numpy(minp["a"].view(np.int16)).to(dev).view(torch.bfloat16)
    B = torch.from_numpy(minp["b"].view(np.int16)).to(dev).view(torch.bfloat16)
    n = lin.out_features * lin.in_features
    out = q.NF4Weight.empty(lin.out_features, lin.in_features, dev)
    ws = torch.empty(lib.qlora_nf4_quantize_workspace(lin.out_features, lin.in_features),
                     dtype=torch.uint8, device=dev)
    wbf = torch.empty(lin.out_features, lin.in_features, dtype=torch.bfloat16, device=dev)
    wmg = torch.empty_like(wbf)
    for _ in range(2):
        q.qlora_nf4_quantize(w, out=out, workspace=ws)
        q.qlora_nf4_dequantize(out, out=wbf)
        q.qlora_nf4_merge(out, A, B, mwl.alpha, out=wmg)
    torch.cuda.synchronize()
    qp, dp, mp = [], [], []
    for _ in range(reps):
        a = (ev.new(), ev.new())
        b = (ev.new(), ev.new())
        c = (ev.new(), ev.new())
        lib.qlora_set_timing_events(2, a[0], a[1])
        lib.qlora_set_timing_events(3, b[0], b[1])
        lib.qlora_set_timing_events(4, c[0], c[1])
        q.qlora_nf4_quantize(w, out=out, workspace=ws)
        q.qlora_nf4_dequantize(out, out=wbf)
        q.qlora_nf4_merge(out, A, B, mwl.alpha, out=wmg)
        qp.append(a)
        dp.append(b)
        mp.append(c)
    torch.cuda.synchronize()
    for g in (2, 3, 4):
        lib.qlora_set_timing_events(g, None, None)
    q_ms = sum(ev.ms(a, b) for a, b in qp) / reps
    d_ms = sum(ev.ms(a, b) for a, b in dp) / reps
    m_ms = sum(ev.ms(a, b) for a, b in mp) / reps
    qbytes = 4 * n + packed_bytes(n)
    dbytes = packed_bytes(n) + 2 * n
    r = mwl.rank
    mbytes = packed_bytes(n) + 2 * r * (lin.out_features + lin.in_features) + 2 * n
    return {
        "workload": "bulk_8192x22016: quantize (NF4/64 + DQ/256) and dequantize-to-bf16 of an "
                    "8192x22016 float32 weight with 0.1% outliers x20",
        "quantize_ms": round(q_ms, 4), "quantize_bytes": qbytes,
        "quantize_GBps": round(qbytes / q_ms / 1e6, 1),
        "quantize_hbm_frac": round(qbytes / q_ms / 1e6 / PEAK_HBM_GBPS, 4),
        "dequant_ms": round(d_ms, 4), "dequant_bytes": dbytes,
        "dequant_GBps": round(dbytes / d_ms / 1e6, 1),
        "dequant_hbm_frac": round(dbytes / d_ms / 1e6 / PEAK_HBM_GBPS, 4),
        "merge_workload": "merge_8192x22016: bf16(dequant(W) + (16/64) B A) of the same weight "
                          "with a rank-64 adapter",
        "merge_ms": round(m_ms, 4), "merge_bytes": mbytes,
        "merge_GBps": round(mbytes / m_ms / 1e6, 1),
        "merge_hbm_frac": round(mbytes / m_ms / 1e6 / PEAK_HBM_GBPS, 4),
    }


def time_adamw(ev, dev, reps):
    """One AdamW step over the adapters of the 7B block (A and B of its seven
    linears, r = 64, float32 parameters and moments, bf16 copy written)."""
    import torch

    import bit_nf4_quantized_06_amd as q
    import workloads as WL
    from bit_nf4_quantized_06_amd import _lib
    lib = _lib.load()
    wl = WL.WORKLOADS["block_7b"]
    n = sum(wl.rank * (lin.in_features + lin.out_features) for lin in wl.linears)
    gen = torch.Generator(device=dev).manual_seed(0)
    p = torch.randn(n, device=dev, generator=gen) * 0.05
    g = torch.randn(n, device=dev, generator=gen) * 1e-3
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    pb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    for step in range(1, 3):
        q.qlora_adamw_step(p, m, v, g, step, 2e-4, weight_decay=0.01, param_bf16=pb)
    torch.cuda.synchronize()
    pairs = []
    for i in range(reps):
        a, b = ev.new(), ev.new()
        lib.qlora_set_timing_events(5, a, b)
        q.qlora_adamw_step(p, m, v, g, 3 + i, 2e-4, weight_decay=0.01, param_bf16=pb)
        pairs.append((a, b))
    torch.cuda.synchronize()
    lib.qlora_set_timing_events(5, None, None)
    ms = sum(ev.ms(a, b) for a, b in pairs) / reps
    nbytes = 30 * n
    return {
        "workload": f"adamw_7b_adapters: one AdamW step on the A and B of the 7B block's seven "
                    f"linears (r = 64, {n} float32 parameters and moments, bf16 copy)",
        "params": n, "ms": round(ms, 4), "bytes": nbytes,
        "GBps": round(nbytes / ms / 1e6, 1),
        "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBPS, 4),
    }


def time_dropout(ev, dev, steps, warmup, warmup_s, reps, p):
    """The headline workload with lora_dropout p (mask drawn in the forward,
    kept for the backward), and the mask kernel alone on its X (draws the
    mask, writes the dropped input)."""
    import torch

    import bit_nf4_quantized_06_amd as q
    import workloads as WL
    from bit_nf4_quantized_06_amd import _lib
    lib = _lib.load()
    wl = WL.WORKLOADS[SMALL_TRAIN]
    ls = LinearSet(wl, dev, dropout=p)
    tm = time_steps(ls, ev, steps, warmup, warmup_s, kernel_timing=False)
    fl = ls.flops()
    it = ls.items[0]
    T, K = ls.T, it["lin"].in_features
    keep = torch.empty((T + 3) // 4, K // 2, dtype=torch.uint8, device=dev)
    xd = torch.empty_like(it["X"])
    for i in range(3):
        q.qlora_dropout_mask(T, K, p, 1234, i, X=it["X"], X_dropped=xd, keep=keep)
    torch.cuda.synchronize()
    pairs = []
    for i in range(reps):
        a, b = ev.new(), ev.new()
        lib.qlora_set_timing_events(6, a, b)
        q.qlora_dropout_mask(T, K, p, 1234, 3 + i, X=it["X"], X_dropped=xd, keep=keep)
        pairs.append((a, b))
    torch.cuda.synchronize()
    lib.qlora_set_timing_events(6, None, None)
    mask_ms = sum(ev.ms(a, b) for a, b in pairs) / reps
    nbytes = 4 * T * K + ((T + 3) // 4) * (K // 2)
    del ls
    return {
        "workload": f"{SMALL_TRAIN} with lora_dropout {p:g} on the adapter input (Philox-4x32-10 "
                    "keep mask drawn in the forward; the mask and the dropped input kept for "
                    "the backward)",
        "p": p, "ms_per_step": round(tm["ms_per_step"], 4),
        "TFLOPs": round(fl / (tm["ms_per_step"] / 1e3) / 1e12, 2),
        "mask_ms": round(mask_ms, 4), "mask_bytes": nbytes,
        "mask_GBps": round(nbytes / mask_ms / 1e6, 1),
        "mask_hbm_frac": round(nbytes / mask_ms / 1e6 / PEAK_HBM_GBPS, 4),
    }


def time_variants(ev, dev, steps, warmup, warmup_s, reps):
    """The storage and compute variants: the headline step with fp16 compute
    and with float32 block constants (no double quantisation), and quantize /
    dequantize of the bulk weight in the other formats."""
    import torch

    import bit_nf4_quantized_06_amd as q
    import workloads as WL
    from bit_nf4_quantized_06_amd import _lib
    lib = _lib.load()
    res = {}
    wl = WL.WORKLOADS[SMALL_TRAIN]
    for name, dt, dq in (("fp16", "fp16", True), ("bf16_no_double_quant", "bf16", False)):
        ls = LinearSet(wl, dev, dtype=dt, double_quant=dq)
        tm = time_steps(ls, ev, steps, warmup, warmup_s, kernel_timing=False)
        fl = ls.flops()
        res[f"{SMALL_TRAIN}_{name}"] = {"ms_per_step": round(tm["ms_per_step"], 4),
                                      "TFLOPs": round(fl / (tm["ms_per_step"] / 1e3) / 1e12, 2)}
        del ls
        torch.cuda.empty_cache()
    lin = WL.WORKLOADS[BULK].linears[0]
    rows, cols = lin.out_features, lin.in_features
    w = torch.from_numpy(WL.linear_inputs(WL.WORKLOADS[BULK], 0)["w"]).to(dev)
    n = rows * cols
    ws = torch.empty(lib.qlora_nf4_quantize_workspace(rows, cols), dtype=torch.uint8, device=dev)
    for name, qt, dq, dt in (("nf4_no_double_quant", "nf4", False, "bf16"),
                             ("int4", "int4", True, "bf16"), ("nf4_fp16", "nf4", True, "fp16")):
        wq = q.NF4Weight.empty(rows, cols, dev, qt, dq, dt)
        deq = torch.empty(rows, cols, dtype=wq.dtype16, device=dev)
        for _ in range(2):
            q.qlora_nf4_quantize(w, out=wq, workspace=ws)
            q.qlora_nf4_dequantize(wq, out=deq)
        torch.cuda.synchronize()
        qp, dp = [], []
        for _ in range(reps):
            a, b = (ev.new(), ev.new()), (ev.new(), ev.new())
            lib.qlora_set_timing_events(2, a[0], a[1])
            lib.qlora_set_timing_events(3, b[0], b[1])
            q.qlora_nf4_quantize(w, out=wq, workspace=ws)
            q.qlora_nf4_dequantize(wq, out=deq)
            qp.append(a)
            dp.append(b)
        torch.cuda.synchronize()
        for g in (2, 3):
            lib.qlora_set_timing_events(g, None, None)
        q_ms = sum(ev.ms(x, y) for x, y in qp) / reps
        d_ms = sum(ev.ms(x, y) for x, y in dp) / reps
        packed = packed_bytes(n) if dq else n // 2 + 4 * (n // 64)
        qb, db = 4 * n + packed, packed + 2 * n
        res[f"bulk_{name}"] = {
            "quantize_ms": round(q_ms, 4), "quantize_GBps": round(qb / q_ms / 1e6, 1),
            "quantize_hbm_frac": round(qb / q_ms / 1e6 / PEAK_HBM_GBPS, 4),
            "dequant_ms": round(d_ms, 4), "dequant_GBps": round(db / d_ms / 1e6, 1),
            "dequant_hbm_frac": round(db / d_ms / 1e6 / PEAK_HBM_GBPS, 4)}
        del wq, deq
    del w
    torch.cuda.empty_cache()
    return res


def copy_calibration():
    """A plain device-to-device copy of a known size: its FETCH_SIZE and
    WRITE_SIZE counters give the scale between counter units and bytes."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def cpu_baseline(tokens, min_seconds):
    """The oracle on a bounded sample of the headline workload, timed on the
    host cores: every linear of the 7B block, its packed weight dequantised
    by the oracle (as every step does) and the float64 forward + backward
    (NumPy / BLAS) on the first `tokens` of its 8192 tokens."""
    import numpy as np

    import workloads as WL
    from oracle import qlora_nf4_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = None
    wl = WL.WORKLOADS[HEADLINE]
    lin_data = []
    for li in range(len(wl.linears)):
        inp = WL.linear_inputs(wl, li, tokens=tokens)
        st = O.quantize(inp["w"])
        del inp["w"]
        vals = {k: WL.bf16_bits_value(inp[k]).astype(np.float64) for k in ("x", "a", "b", "dy")}
        lin_data.append((st, vals))
    reps = 0
    t0 = time.perf_counter()
    while True:
        for st, v in lin_data:
            w_hat = O.dequantize(st)
            O.linear_forward(v["x"], w_hat, v["a"], v["b"], wl.alpha, wl.rank)
            O.linear_backward(v["x"], v["dy"], w_hat, v["a"], v["b"], wl.alpha, wl.rank)
            del w_hat
        reps += 1
        if time.perf_counter() - t0 >= min_seconds or reps >= 20:
            break
    dt = (time.perf_counter() - t0) / reps
    fl = sum(flops_fwd_bwd(tokens, lin.out_features, lin.in_features, wl.rank)
             for lin in wl.linears)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads or cores,
            "kind": "oracle",
            "sample": f"{HEADLINE}: all {len(wl.linears)} linears, oracle dequantise of each "
                      f"full packed weight + float64 forward + backward (NumPy/BLAS) on "
                      f"{tokens} of the {wl.tokens} tokens; {dt:.2f} s per step, mean of {reps}; "
                      f"{cores} host cores visible, {threads} BLAS threads",
            "seconds_per_step": round(dt, 3)}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this library and its benchmark run "
              "on one GPU (the token-sharded multi-GPU layout is described in DESIGN.md, not "
              "built)", file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads as WL
    if args.copy_calibration:
        copy_calibration()
        return
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    ev = HipEvents()
    only = set(args.only.split(",")) if args.only else None

    def want(k):
        return only is None or k in only

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    head = None
    configs = {}
    if want(HEADLINE):
        log(f"timing {HEADLINE} fwd+bwd (headline)")
        head = training_config(HEADLINE, ev, dev, args.steps, args.warmup, args.warmup_seconds)
    if want(HEADLINE_LDS):
        import bit_nf4_quantized_06_amd as q
        log(f"timing {HEADLINE} fwd+bwd with the in-LDS weight decode")
        prev = q.qlora_set_pre_dequant_min_tokens(NEVER)
        try:
            r = training_config(HEADLINE, ev, dev, args.steps, args.warmup, args.warmup_seconds,
                                traffic_name=HEADLINE_LDS)
        finally:
            q.qlora_set_pre_dequant_min_tokens(prev)
        configs[HEADLINE_LDS] = {k: r[k] for k in ("gemm_weight_path", "ms_per_step", "TFLOPs",
                                                   "mfma_frac", "roofline",
                                                   "kernels_ms_per_step")}
    if want(SMALL_TRAIN):
        log(f"timing {SMALL_TRAIN} fwd+bwd")
        configs[SMALL_TRAIN] = training_config(SMALL_TRAIN, ev, dev, args.steps, args.warmup,
                                               args.warmup_seconds)
    w65 = None
    if want(TRAIN_65B):
        log(f"timing {TRAIN_65B} fwd+bwd")
        configs[TRAIN_65B], w65 = training_config(TRAIN_65B, ev, dev, args.steps, args.warmup,
                                                  args.warmup_seconds, keep_weights=True)
        if not want(DECODE_65B):
            w65 = None
    if want(DECODE_65B):
        # the decode block is the same 65B-style block (same weight draws) at 16 tokens
        log(f"timing {DECODE_65B} forward (skinny path)")
        configs[DECODE_65B] = decode_config(DECODE_65B, ev, dev, args.steps, args.warmup,
                                            args.warmup_seconds, weights=w65)
    del w65
    torch.cuda.empty_cache()
    if want("bulk"):
        log("timing bulk quantize/dequantize/merge")
        configs[BULK] = time_bulk(ev, dev, args.bulk_reps)
    nxt = {}
    if want("adamw"):
        log("timing the adapter AdamW step")
        nxt["adamw"] = time_adamw(ev, dev, args.bulk_reps)
        torch.cuda.empty_cache()
    if want("dropout"):
        log("timing fwd+bwd with lora_dropout")
        nxt["dropout"] = time_dropout(ev, dev, args.steps, args.warmup, args.warmup_seconds,
                                      args.bulk_reps, DROPOUT_P)
        torch.cuda.empty_cache()
    if want("variants"):
        log("timing the storage and compute variants")
        nxt["variants"] = time_variants(ev, dev, args.steps, args.warmup, args.warmup_seconds,
                                        args.bulk_reps)
    ev.close()

    cpu = None
    if not args.no_cpu_baseline and head is not None:
        log("timing CPU oracle")
        cpu = cpu_baseline(args.cpu_tokens, args.cpu_seconds)

    wl = WL.WORKLOADS[HEADLINE]
    line = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s (NF4 dequant-fused); NF4 dequant GB/s",
        "value": head["TFLOPs"] if head else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": head["warmup_steps_run"] if head else None,
        "warmup_s": head["warmup_s"] if head else None,
        "ms_per_step": head["ms_per_step"] if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded W ~ N(0, 0.02^2) (0.1% of entries x20 where the workload asks), "
                "bf16 X, dY ~ N(0,1), A ~ N(0, 1/r), B ~ N(0, 0.01^2); no dataset",
        "config": {"workload": f"{HEADLINE}: one 7B-style decoder block, all 7 QLoRA linears "
                               "(q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008), NF4/64 "
                               f"+ double quant/256, T={wl.tokens} tokens (16x512), r={wl.rank}, "
                               f"alpha={wl.alpha:g}; step = forward (Y, U) of every linear + "
                               "backward (dX, dA, dB) of every linear, no dW",
                   "tokens": wl.tokens, "rank": wl.rank, "alpha": wl.alpha,
                   "flops_per_step": head["flops_per_step"] if head else None},
        "roofline": head["roofline"] if head else None,
        "kernels_ms_per_step": head["kernels_ms_per_step"] if head else None,
        "ms_per_step_with_kernel_events": head["ms_per_step_with_kernel_events"] if head else None,
        "configs": configs,
        "next": nxt,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
