#!/usr/bin/env python3
"""Benchmark of the NF4 + LoRA linear layer on one MI355X.

A step is one forward (Y, U) plus one backward (dX, dA, dB) of the
attention-projection workload: W 4096x4096 (NF4 blocks of 64, double
quantisation in groups of 256, 0.1% outliers x20), T = 4096 tokens, r = 16,
alpha = 32.  The weight is quantised once before timing (a load-time cost);
every step dequantises it on the fly inside the fused GEMMs.  The bulk path
(quantise and dequantise an 8192 x 22016 weight) is timed in the same run.

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

HEADLINE = "attn_4096"
BULK = "bulk_8192x22016"
MERGE = "merge_8192x22016"
DROPOUT_P = 0.05              # lora_dropout of the adapter configs on the pages


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clock settles over the first ~10 ms of steady work: with 5 warm-up
    # steps the first timed pass ran about 8% slower than the next ones
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--bulk-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens of the headline workload the CPU oracle is timed on")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle step until this much time has passed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--extended", action="store_true",
                    help="also time the 7B-block, 65B-block and decode workloads")
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
                 double_quant=True):
        import torch

        import bit_nf4_quantized_06_amd as q
        import workloads as WL
        self.wl = wl
        self.dropout = dropout          # lora_dropout probability, or None
        self.T = wl.tokens if tokens is None else tokens
        self.r, self.alpha = wl.rank, wl.alpha
        self.items = []
        for li, lin in enumerate(wl.linears):
            inp = WL.linear_inputs(wl, li, tokens=self.T, dtype=dtype)
            wq = q.qlora_nf4_quantize(torch.from_numpy(inp["w"]).to(dev),
                                      double_quant=double_quant, compute_dtype=dtype)
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
            if backward and "dy" in inp:
                it["dY"] = to_dev_bf16(inp["dy"], dev, dtype)
                it["dX"] = torch.empty(t, k, dtype=wq.dtype16, device=dev)
                it["dA"] = torch.empty(r, k, dtype=torch.float32, device=dev)
                it["dB"] = torch.empty(n, r, dtype=torch.float32, device=dev)
                it["wsb"] = torch.empty(wsz(t, n, k, r, True), dtype=torch.uint8, device=dev)
            self.items.append(it)
            del inp
        torch.cuda.synchronize()

    def step(self, backward=True):
        import bit_nf4_quantized_06_amd as q
        if self.dropout is not None:
            for li, it in enumerate(self.items):
                q.qlora_linear_fwd_dropout(it["wq"], it["X"], it["A"], it["B"], self.alpha,
                                           self.dropout, 1234, li, Y=it["Y"], U_save=it["U"],
                                           keep_save=it["keep"], workspace=it["wsf"],
                                           X_dropped_save=it["Xd"])
                if backward and "dY" in it:
                    q.qlora_linear_bwd_dropout(it["wq"], it["X"], it["dY"], it["A"], it["B"],
                                               self.alpha, self.dropout, 1234, li,
                                               keep_saved=it["keep"], U_saved=it["U"],
                                               dX=it["dX"], dA=it["dA"], dB=it["dB"],
                                               workspace=it["wsb"], X_dropped_saved=it["Xd"])
            return
        for it in self.items:
            q.qlora_linear_fwd(it["wq"], it["X"], it["A"], it["B"], self.alpha, Y=it["Y"],
                               U_save=it["U"], workspace=it["wsf"])
            if backward and "dY" in it:
                q.qlora_linear_bwd(it["wq"], it["X"], it["dY"], it["A"], it["B"], self.alpha,
                                   U_saved=it["U"], dX=it["dX"], dA=it["dA"], dB=it["dB"],
                                   workspace=it["wsb"])

    def flops(self, backward=True):
        tot = 0
        for it in self.items:
            n, k = it["lin"].out_features, it["lin"].in_features
            if backward:
                tot += flops_fwd_bwd(self.T, n, k, self.r)
            else:
                tot += 2 * self.T * n * k + 2 * self.T * self.r * (n + k)
        return tot


def time_steps(ls, ev, steps, warmup, backward=True, kernel_timing=True):
    """Whole-step and per-GEMM times (ms) over `steps` timed steps."""
    import torch

    from bit_nf4_quantized_06_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        ls.step(backward)
    torch.cuda.synchronize()
    per_step = []
    fwd_pairs, dx_pairs = [], []
    start, stop = ev.new(fence=True), ev.new(fence=True)
    t_wall = time.perf_counter()
    ev.record(start, stream)
    for _ in range(steps):
        if kernel_timing:
            fp = (ev.new(), ev.new())
            dp = (ev.new(), ev.new())
            lib.qlora_set_timing_events(0, fp[0], fp[1])
            lib.qlora_set_timing_events(1, dp[0], dp[1])
            fwd_pairs.append(fp)
            dx_pairs.append(dp)
        ls.step(backward)
    ev.record(stop, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    lib.qlora_set_timing_events(0, None, None)
    lib.qlora_set_timing_events(1, None, None)
    total = ev.ms(start, stop)
    res = {"ms_per_step": total / steps, "wall_s": wall}
    if kernel_timing and len(ls.items) == 1:
        res["fwd_gemm_ms"] = sum(ev.ms(a, b) for a, b in fwd_pairs) / steps
        if backward:
            res["dx_gemm_ms"] = sum(ev.ms(a, b) for a, b in dx_pairs) / steps
    return res


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


def time_dropout(ev, dev, steps, warmup, reps, p):
    """The headline workload with lora_dropout p (mask drawn in the forward,
    kept for the backward), and the mask kernel alone on its X (draws the
    mask, writes the dropped input)."""
    import torch

    import bit_nf4_quantized_06_amd as q
    import workloads as WL
    from bit_nf4_quantized_06_amd import _lib
    lib = _lib.load()
    wl = WL.WORKLOADS[HEADLINE]
    ls = LinearSet(wl, dev, dropout=p)
    tm = time_steps(ls, ev, steps, warmup, kernel_timing=False)
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
        "workload": f"{HEADLINE} with lora_dropout {p:g} on the adapter input (Philox-4x32-10 "
                    "keep mask drawn in the forward; the mask and the dropped input kept for "
                    "the backward)",
        "p": p, "ms_per_step": round(tm["ms_per_step"], 4),
        "TFLOPs": round(fl / (tm["ms_per_step"] / 1e3) / 1e12, 2),
        "mask_ms": round(mask_ms, 4), "mask_bytes": nbytes,
        "mask_GBps": round(nbytes / mask_ms / 1e6, 1),
        "mask_hbm_frac": round(nbytes / mask_ms / 1e6 / PEAK_HBM_GBPS, 4),
    }


def time_variants(ev, dev, steps, warmup, reps):
    """The storage and compute variants: the headline step with fp16 compute
    and with float32 block constants (no double quantisation), and quantize /
    dequantize of the bulk weight in the other formats."""
    import torch

    import bit_nf4_quantized_06_amd as q
    import workloads as WL
    from bit_nf4_quantized_06_amd import _lib
    lib = _lib.load()
    res = {}
    wl = WL.WORKLOADS[HEADLINE]
    for name, dt, dq in (("fp16", "fp16", True), ("bf16_no_double_quant", "bf16", False)):
        ls = LinearSet(wl, dev, dtype=dt, double_quant=dq)
        tm = time_steps(ls, ev, steps, warmup, kernel_timing=False)
        fl = ls.flops()
        res[f"{HEADLINE}_{name}"] = {"ms_per_step": round(tm["ms_per_step"], 4),
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
    """The oracle (dequantise the packed weight + float64 forward + backward)
    on `tokens` tokens of the headline workload, timed on the host cores."""
    import numpy as np

    import workloads as WL
    from oracle import qlora_nf4_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = None
    wl = WL.WORKLOADS[HEADLINE]
    lin = wl.linears[0]
    inp = WL.linear_inputs(wl, 0, tokens=tokens)
    st = O.quantize(inp["w"])
    x = WL.bf16_bits_value(inp["x"]).astype(np.float64)
    a = WL.bf16_bits_value(inp["a"]).astype(np.float64)
    b = WL.bf16_bits_value(inp["b"]).astype(np.float64)
    dy = WL.bf16_bits_value(inp["dy"]).astype(np.float64)
    reps = 0
    t0 = time.perf_counter()
    while True:
        w_hat = O.dequantize(st)
        O.linear_forward(x, w_hat, a, b, wl.alpha, wl.rank)
        O.linear_backward(x, dy, w_hat, a, b, wl.alpha, wl.rank)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds or reps >= 50:
            break
    dt = (time.perf_counter() - t0) / reps
    fl = flops_fwd_bwd(tokens, lin.out_features, lin.in_features, wl.rank)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads or cores,
            "kind": "oracle",
            "sample": f"{HEADLINE} at T={tokens} of {wl.tokens} tokens: oracle dequantise of the "
                      f"full {lin.out_features}x{lin.in_features} weight + float64 forward + "
                      f"backward (NumPy/BLAS), {dt:.2f} s per step, mean of {reps}; "
                      f"{cores} host cores visible",
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

    wl = WL.WORKLOADS[HEADLINE]
    lin = wl.linears[0]
    print(f"[bench] preparing {HEADLINE}", file=sys.stderr, flush=True)
    ls = LinearSet(wl, dev)
    print("[bench] timing fwd+bwd", file=sys.stderr, flush=True)
    # the timed steps: the hot path alone, no events between its kernels
    tm = time_steps(ls, ev, args.steps, args.warmup, kernel_timing=False)
    # kernel durations: the same number of steps again, with a pair of HIP
    # events around each GEMM on the library's stream (each event record
    # costs several microseconds of idle GPU, so these steps are slower)
    tk = time_steps(ls, ev, args.steps, 0)
    fl = ls.flops()
    value = fl / (tm["ms_per_step"] / 1e3) / 1e12
    T, N, K, r = wl.tokens, lin.out_features, lin.in_features, wl.rank
    kern = {
        "qlora_gemm_fwd": (tk["fwd_gemm_ms"], 2 * T * N * (K + r)),
        "qlora_gemm_dx": (tk["dx_gemm_ms"], 2 * T * K * (N + r)),
    }
    dom = max(kern, key=lambda k: kern[k][0])
    dom_ms, dom_flops = kern[dom]
    achieved = dom_flops / (dom_ms / 1e3) / 1e12
    digest = source_digest("gemm.hip", "device_common.h")
    traffic = profiled_traffic(dom, HEADLINE, digest)
    del ls
    torch.cuda.empty_cache()

    print("[bench] timing bulk quantize/dequantize", file=sys.stderr, flush=True)
    bulk = time_bulk(ev, dev, args.bulk_reps)
    print("[bench] timing the adapter AdamW step", file=sys.stderr, flush=True)
    adamw = time_adamw(ev, dev, args.bulk_reps)
    torch.cuda.empty_cache()
    print("[bench] timing fwd+bwd with lora_dropout", file=sys.stderr, flush=True)
    dropout = time_dropout(ev, dev, max(5, args.steps // 2), args.warmup, args.bulk_reps,
                           DROPOUT_P)
    torch.cuda.empty_cache()
    print("[bench] timing the storage and compute variants", file=sys.stderr, flush=True)
    variants = time_variants(ev, dev, max(5, args.steps // 2), args.warmup, args.bulk_reps)

    extended = None
    if args.extended:
        extended = {}
        for name, bwd in (("block_7b", True), ("block_65b_train", True),
                          ("block_65b_decode", False)):
            print(f"[bench] timing {name}", file=sys.stderr, flush=True)
            w2 = WL.WORKLOADS[name]
            ls2 = LinearSet(w2, dev, backward=bwd)
            t2 = time_steps(ls2, ev, max(3, args.steps // 10), 2, backward=bwd,
                            kernel_timing=False)
            f2 = ls2.flops(bwd)
            extended[name] = {"ms_per_step": round(t2["ms_per_step"], 4),
                              "TFLOPs": round(f2 / (t2["ms_per_step"] / 1e3) / 1e12, 2),
                              "fwd_bwd" if bwd else "fwd_only": True}
            if not bwd:
                by = sum(packed_bytes(it["lin"].out_features * it["lin"].in_features)
                         + 2 * (it["A"].numel() + it["B"].numel() + it["X"].numel()
                                + it["Y"].numel()) for it in ls2.items)
                extended[name]["GBps"] = round(by / (t2["ms_per_step"] / 1e3) / 1e9, 1)
                extended[name]["hbm_frac"] = round(extended[name]["GBps"] / PEAK_HBM_GBPS, 4)
            del ls2
            torch.cuda.empty_cache()
    ev.close()

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.cpu_tokens, args.cpu_seconds)

    line = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s (NF4 dequant-fused); NF4 dequant GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tm["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded W ~ N(0, 0.02^2) with 0.1% of entries x20, bf16 X, dY ~ N(0,1),"
                " A ~ N(0, 1/r), B ~ N(0, 0.01^2)",
        "config": {"workload": f"{HEADLINE}: one QLoRA linear, W {N}x{K} NF4/64 + double quant/256, "
                               f"T={T} tokens (8x512), r={r}, alpha={wl.alpha:g}; step = forward "
                               "(Y, U) + backward (dX, dA, dB), no dW",
                   "tokens": T, "out_features": N, "in_features": K, "rank": r,
                   "alpha": wl.alpha, "flops_per_step": fl},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": dom_flops, "avg_launch_ms": round(dom_ms, 4),
                     "source_digest": digest},
        "kernels_ms": {k: round(v[0], 4) for k, v in kern.items()},
        "kernel_timing": {"steps": args.steps,
                          "ms_per_step_with_kernel_events": round(tk["ms_per_step"], 4),
                          "how": "a second pass of the same steps with HIP events around "
                                 "each GEMM on the library's stream"},
        "bulk": bulk,
        "adamw": adamw,
        "dropout": dropout,
        "variants": variants,
        "cpu_baseline": cpu,
    }
    if extended is not None:
        line["extended"] = extended
    print(json.dumps(line))


if __name__ == "__main__":
    main()
