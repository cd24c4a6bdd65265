#!/usr/bin/env python3
"""Throughput of the shifted-window attention block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one pass of the whole forward over one batch: for the default
workload (SwinV2-G-like stage 1: one 1536 x 1536 image at patch 4, i.e. 384 x
384 tokens, C = 512, 16 heads, window 24, shift 12, scaled cosine attention,
bf16) that is one SW-MSA block forward.
Inputs are seeded synthetic tensors already resident in HBM; x is rotated over
enough copies to exceed the 256 MB last-level cache.

Prints ONE JSON line on stdout (logs go to stderr) with:
  value        tokens/s over the timed steps (block-tokens: every token of every
               block forward counts once),
  roofline     the dominant kernel's achieved algorithmic bytes or flops per
               launch divided by its average launch duration, measured with HIP
               events recorded by the library around each of its kernels on the
               stream they run on,
  cpu_baseline the float64 CPU oracle timed on a bounded sample of the same
               workload on this host,
  workloads    the same measurement for the other workload shapes,
  full_block   informational: the whole block forward (LayerNorms, attention,
               MLP, residual adds) of each workload's last block,
  backward     informational: the attention sub-layer backward of each
               workload's last block (float32 compute),
  fp8_qkv      informational: the FP8 (E4M3) linear layer on each 16-bit
               workload's QKV shape (quantisation and product timed apart),
               and the 2:4-sparse linear layer on the same shape.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import glob
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shifted-window attention tokens/s + TFLOP/s as % of MFMA peak, 1 MI355X"
MAIN = "swinv2_g_stage1_384_w24_bf16"
PEAK_TFLOPS = {"fp16": 2500.0, "bf16": 2500.0, "fp32": 157.3}   # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0                                             # HBM3E, MI355X
PEAK_FP8_TFLOPS = 5000.0                                          # dense fp8 MFMA, MI355X
ELEM = {"fp32": 4, "fp16": 2, "bf16": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_per_token(C, N):
    """Algorithmic flops per token: QKV 6C^2, QK^T 2NC, AV 2NC, projection 2C^2."""
    return 8 * C * C + 4 * N * C


def stage_work(case):
    """Algorithmic (flops, bytes) per launch of each kernel: the data its
    interface must move once (activations in and out, the weights and the bias
    table), not what it re-reads."""
    T, C, N, heads = case.tokens, case.C, case.M * case.M, case.heads
    e = ELEM[case.dtype]
    eqk = 2 if (case.mode == "v2" and case.dtype != "fp32") else e
    tab = (2 * case.M - 1) ** 2 * heads * 4
    return {
        "fused_window_kernel": ((8 * C * C + 4 * N * C) * T, T * 2 * C * e + 4 * C * C * e + tab),
        "fused_w16_kernel": ((8 * C * C + 4 * N * C) * T, T * 2 * C * e + 4 * C * C * e + tab),
        "fused_w8_kernel": ((8 * C * C + 4 * N * C) * T, T * 2 * C * e + 4 * C * C * e + tab),
        # QKV projection + attention: x in, O out, the QKV weights and the table
        "fused_qkv_attn_kernel": ((6 * C * C + 4 * N * C) * T, T * 2 * C * e + 3 * C * C * e + tab),
        # the exact passes over flagged items (none on the workloads): flags only
        "fused_qkv_attn_redo_kernel": (0, 1),
        "fused_w16_redo_kernel": (0, 1),
        "qkv_gemm_kernel": (6 * C * C * T, T * (C * e + 2 * C * eqk + C * e) + 3 * C * C * e),
        "qkv_tiled_kernel": (6 * C * C * T, T * (C * e + 2 * C * eqk + C * e) + 3 * C * C * e),
        "proj_tiled_kernel": (2 * C * C * T, T * 2 * C * e + C * C * e),
        "window_attn_kernel": (4 * N * C * T, T * (2 * C * eqk + C * e + C * e) + tab),
        "tiled_attn_kernel": (4 * N * C * T, T * (2 * C * eqk + C * e + C * e) + tab),
        "w8_attn_kernel": (4 * N * C * T, T * (2 * C * eqk + C * e + C * e) + tab),
        "proj_gemm_kernel": (2 * C * C * T, T * 2 * C * e + C * C * e),
    }


class HipEvents:
    """Raw hipEvent_t handles for the library's per-kernel event records."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


class Runner:
    """Device-resident inputs of one workload and one forward step."""

    def __init__(self, name, min_rotate_bytes=512 << 20, max_copies=16):
        import torch
        import shifted_window_attention_roll_amd as swin
        import workloads
        self.swin, self.torch = swin, torch
        self.name = name
        self.case = case = workloads.make_workload(name)
        dev = "cuda"
        xb = case.x.numel() * case.x.element_size()
        self.copies = max(1, min(max_copies, math.ceil(min_rotate_bytes / max(xb, 1))))
        x0 = case.x.to(dev)
        self.xs = [x0] + [x0.clone() for _ in range(self.copies - 1)]
        self.blocks = []
        for blk in case.blocks:
            if case.mode == "v1":
                table = blk.table.to(dev)
            else:
                table = swin.cpb_table(blk.cpb_w1.to(dev), blk.cpb_b1.to(dev), blk.cpb_w2.to(dev),
                                       blk.cpb_b2.to(dev), case.M)
            self.blocks.append(dict(
                s=blk.s, w_qkv=blk.w_qkv.to(dev), b_qkv=blk.b_qkv.to(dev),
                w_proj=blk.w_proj.to(dev), b_proj=blk.b_proj.to(dev), table=table,
                tau=None if blk.tau is None else blk.tau.to(dev),
                out=torch.empty_like(x0)))
        desc = swin.make_desc(case.B, case.H, case.W, case.C, case.heads, case.M,
                              case.blocks[0].s, case.mode, case.torch_dtype)
        self.ws = torch.empty(swin.workspace_size(desc), dtype=torch.uint8, device=dev)
        self.kernels = swin.kernel_names(desc)
        self.tokens_per_step = case.tokens * len(case.blocks)
        self.flops_per_step = flops_per_token(case.C, case.M * case.M) * self.tokens_per_step

    def step(self, i, events=None):
        x = self.xs[i % self.copies]
        for bi, b in enumerate(self.blocks):
            ev = None if events is None else events[bi]
            x = self.swin.wmsa_fwd(x, b["w_qkv"], b["b_qkv"], b["w_proj"], b["b_proj"], b["table"],
                                   self.case.M, b["s"], self.case.heads, self.case.mode,
                                   tau=b["tau"], out=b["out"], workspace=self.ws, events=ev)
        return x

    def time_steps(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            self.step(i)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    def time_kernels(self, steps, hip):
        """Average duration (ms) per launch of each kernel, from the library's event
        records around its launches on the stream."""
        torch = self.torch
        nk = len(self.kernels)
        nb = len(self.blocks)
        evs = hip.create(steps * nb * (nk + 1))
        per = [evs[j * (nk + 1):(j + 1) * (nk + 1)] for j in range(steps * nb)]
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(i, events=per[i * nb:(i + 1) * nb])
        torch.cuda.synchronize()
        tot = {k: 0.0 for k in self.kernels}
        for ev in per:
            for ki, k in enumerate(self.kernels):
                tot[k] += hip.elapsed_ms(ev[ki], ev[ki + 1])
        hip.destroy(evs)
        return {k: v / (steps * nb) for k, v in tot.items()}


# Source file of each kernel; its digest also covers the headers that file
# includes (directly or not) and the host-side launch code, so traffic counters
# taken on a kernel stay valid while only other kernels change.
KERNEL_SOURCE = {
    "fused_window_kernel": "fused_window.hip", "fused_w8_kernel": "fused_w8.hip",
    "fused_w16_kernel": "fused_w16.hip", "fused_w16_redo_kernel": "fused_w16.hip",
    "tiled_attn_kernel": "tiled_attn.hip",
    "fused_qkv_attn_kernel": "fused_qkv_attn.hip", "fused_qkv_attn_redo_kernel": "fused_qkv_attn.hip",
    "window_attn_kernel": "window_attn.hip", "w8_attn_kernel": "w8_attn.hip",
    "qkv_tiled_kernel": "gemm_tiled.hip",
    "proj_tiled_kernel": "gemm_tiled.hip", "qkv_gemm_kernel": "gemm.hip",
    "proj_gemm_kernel": "gemm.hip",
}
_INCLUDE = re.compile(r'^\s*#\s*include\s+"([^"]+)"', re.M)


def _source_closure(csrc, names):
    """The named files plus every local header they include, transitively."""
    seen, todo = set(), list(names)
    while todo:
        n = todo.pop()
        p = os.path.join(csrc, n)
        if n in seen or not os.path.exists(p):
            continue
        seen.add(n)
        with open(p) as f:
            todo.extend(_INCLUDE.findall(f.read()))
    return sorted(os.path.join(csrc, n) for n in seen)


def source_digest(kernel=None):
    csrc = os.path.join(ROOT, "shifted_window_attention_roll_amd", "csrc")
    if kernel in KERNEL_SOURCE:
        paths = _source_closure(csrc, [KERNEL_SOURCE[kernel], "api.hip"])
    else:
        paths = sorted(glob.glob(os.path.join(csrc, "*")))
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get("entries", {}).get(f"{workload}:{kernel}")
    if not ent or ent.get("source_digest") != source_digest(kernel):
        return None
    return ent.get("bytes_per_launch")


def roofline(runner, kern_ms):
    case = runner.case
    work = stage_work(case)
    dom = max(kern_ms, key=lambda k: kern_ms[k])
    flops, nbytes = work[dom]
    peak_f = PEAK_TFLOPS[case.dtype]
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    sec = kern_ms[dom] * 1e-3
    if flops / nbytes >= ridge:
        ach = flops / sec / 1e12
        r = {"bound": "mfma", "achieved": ach, "peak": peak_f, "unit": "TFLOP/s"}
    else:
        ach = nbytes / sec / 1e9
        r = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = measured_traffic(dom, runner.name)
    r["kernel"] = dom
    r["kernel_ms"] = kern_ms[dom]
    r["algorithmic_flops"] = flops
    r["algorithmic_bytes"] = nbytes
    return r


def _sample_windows(B, H, W, M, n):
    """n windows spread evenly over the batch (every stride-th window, so the
    masked last row / column of the grid is represented)."""
    total = B * (H // M) * (W // M)
    n = max(1, min(n, total))
    return sorted({int(round(i * (total - 1) / max(n - 1, 1))) for i in range(n)})


def cpu_baseline(name, budget_s=15.0):
    """The float64 oracle as it stands, on a bounded sample of the workload: whole
    images when the batch has several, else a subset of the image's windows."""
    import workloads
    from oracle import swin_oracle as so
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: BLAS thread count unknown
        blas = None
    case = workloads.make_workload(name)
    N = case.M * case.M
    tables = []
    for blk in case.blocks:
        tables.append(workloads.f64(blk.table) if case.mode == "v1" else
                      so.cpb_table(workloads.f64(blk.cpb_w1), workloads.f64(blk.cpb_b1),
                                   workloads.f64(blk.cpb_w2), workloads.f64(blk.cpb_b2), case.M))

    def fwd(blk, table, x, windows=None):
        return so.wmsa_forward(x, workloads.f64(blk.w_qkv), workloads.f64(blk.b_qkv),
                               workloads.f64(blk.w_proj), workloads.f64(blk.b_proj), table,
                               case.M, blk.s, case.heads, case.mode,
                               tau=None if blk.tau is None else workloads.f64(blk.tau),
                               windows=windows)

    if case.B > 1:
        def run(n):
            x = workloads.f64(case.x[:n])
            t0 = time.perf_counter()
            for blk, table in zip(case.blocks, tables):
                x = fwd(blk, table, x)
            return time.perf_counter() - t0, n * case.H * case.W * len(case.blocks)
        unit, limit = "image", case.B
    else:
        x64 = workloads.f64(case.x)
        nwin = (case.H // case.M) * (case.W // case.M)

        def run(n):
            wins = _sample_windows(1, case.H, case.W, case.M, n)
            t0 = time.perf_counter()
            for blk, table in zip(case.blocks, tables):
                fwd(blk, table, x64, windows=wins)
            return time.perf_counter() - t0, len(wins) * N * len(case.blocks)
        unit, limit = "window", nwin

    t1, _ = run(1)
    n = int(max(1, min(limit, budget_s / max(t1, 1e-3) / 2)))
    t, tokens, passes = 0.0, 0, 0
    while passes == 0 or (t < 0.66 * budget_s and passes < 100):
        dt, tok = run(n)
        t += dt
        tokens += tok
        passes += 1
    return {"value": tokens / t, "unit": "tokens/s", "cores": blas or affinity, "kind": "oracle",
            "affinity_cores": affinity, "blas_threads": blas,
            "sample": f"{passes} pass(es) over {n} of {limit} {unit}s of {name}, all "
                      f"{len(case.blocks)} block(s), {tokens} block-tokens in {t:.2f} s "
                      f"(float64 numpy; {affinity} cores in the affinity set, BLAS threads "
                      f"{blas})"}


def measure(name, steps, warmup, hip):
    r = Runner(name)
    ms = r.time_steps(steps, warmup)
    kern = r.time_kernels(min(steps, 20), hip)
    tok_s = r.tokens_per_step / (ms * 1e-3)
    tflops = r.flops_per_step / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[r.case.dtype]
    out = {"tokens_per_s": tok_s, "ms_per_step": ms, "tflops": tflops,
           "mfma_peak_tflops": peak, "frac_of_mfma_peak": tflops / peak,
           "kernel_ms": kern, "roofline": roofline(r, kern),
           "tokens_per_step": r.tokens_per_step, "buffer_copies": r.copies}
    del r
    return out


def block_time(name, steps, warmup):
    """Full block forward (LayerNorms, attention, MLP with hidden 4C, the
    residual adds) on the workload's last block, timed like a step: average ms
    per block forward and the rates that gives.  Informational: the headline
    value is the attention step above."""
    import torch
    import shifted_window_attention_roll_amd as swin
    import workloads
    case = workloads.make_workload(name)
    blk, dev = case.blocks[-1], "cuda"
    if case.mode == "v1":
        table = blk.table.to(dev)
    else:
        table = swin.cpb_table(blk.cpb_w1.to(dev), blk.cpb_b1.to(dev), blk.cpb_w2.to(dev),
                               blk.cpb_b2.to(dev), case.M)
    p = {"w_qkv": blk.w_qkv.to(dev), "b_qkv": blk.b_qkv.to(dev), "w_proj": blk.w_proj.to(dev),
         "b_proj": blk.b_proj.to(dev), "table": table}
    if blk.tau is not None:
        p["tau"] = blk.tau.to(dev)
    p.update({k: v.to(dev) for k, v in
              workloads.make_block_params(case.C, case.dtype, 77, fc_std=0.02).items()})
    x = case.x.to(dev)
    out = torch.empty_like(x)
    d = swin.make_block_desc(case.B, case.H, case.W, case.C, case.heads, case.M, blk.s,
                             case.mode, x.dtype)
    ws = torch.empty(swin.block_workspace_size(d), dtype=torch.uint8, device=dev)

    def run():
        swin.block_fwd(x, p, case.M, blk.s, case.heads, case.mode, out=out, workspace=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    T, C = case.tokens, case.C
    flops = T * (flops_per_token(C, case.M * case.M) + 16 * C * C)
    del x, out, ws, p
    return {"block_ms": ms, "block_tokens_per_s": T / (ms * 1e-3),
            "block_tflops": flops / (ms * 1e-3) / 1e12, "hidden": 4 * C}


def backward_flops_per_token(C, N):
    """Algorithmic flops per token of the sub-layer backward: the QKV recompute
    6C^2, dO 2C^2, dWp 2C^2, dWqkv 6C^2, dx 6C^2; attention recompute (S, O) 4NC
    and gradients (dP, dV, dQ, dK) 8NC."""
    return 22 * C * C + 12 * N * C


def backward_time(name, steps, warmup):
    """Sub-layer backward (swin_wmsa_bwd) on the workload's last block, timed
    like a step.  Informational; its rate is set against the float32
    matrix-core peak, that of the attention backward's products (the GEMMs run
    on the 16-bit matrix cores)."""
    import torch
    import shifted_window_attention_roll_amd as swin
    import workloads
    case = workloads.make_workload(name)
    blk, dev = case.blocks[-1], "cuda"
    if case.mode == "v1":
        table = blk.table.to(dev)
    else:
        table = swin.cpb_table(blk.cpb_w1.to(dev), blk.cpb_b1.to(dev), blk.cpb_w2.to(dev),
                               blk.cpb_b2.to(dev), case.M)
    x = case.x.to(dev)
    dy = workloads.make_upstream_grad(case.x.shape, case.dtype, 3).to(dev)
    args = (x, blk.w_qkv.to(dev), blk.b_qkv.to(dev), blk.w_proj.to(dev), table, dy, case.M,
            blk.s, case.heads, case.mode)
    tau = None if blk.tau is None else blk.tau.to(dev)
    d = swin.make_desc(case.B, case.H, case.W, case.C, case.heads, case.M, blk.s, case.mode,
                       x.dtype)
    ws = torch.empty(swin.bwd_workspace_size(d), dtype=torch.uint8, device=dev)
    grads = swin.wmsa_bwd(*args, tau=tau, workspace=ws)
    for _ in range(warmup):
        swin.wmsa_bwd(*args, tau=tau, grads=grads, workspace=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        swin.wmsa_bwd(*args, tau=tau, grads=grads, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    T = case.tokens
    tf = T * backward_flops_per_token(case.C, case.M * case.M) / (ms * 1e-3) / 1e12
    del x, dy, ws, grads
    return {"bwd_ms": ms, "bwd_tokens_per_s": T / (ms * 1e-3), "bwd_tflops": tf,
            "bwd_frac_of_fp32_mfma_peak": tf / PEAK_TFLOPS["fp32"],
            "compute": "fp32 attention products; GEMMs on 16-bit matrix cores (exact, or "
                       "operands as two bf16 terms), fp32 accumulation"}


def fp8_time(name, steps, warmup):
    """FP8 (E4M3) linear layer on the workload's QKV shape (tokens x 3C x C):
    per-token quantisation of x and the scaled product, timed separately.
    Informational; the product's roofline is the dense fp8 peak."""
    import torch
    import shifted_window_attention_roll_amd as swin
    import workloads
    case = workloads.make_workload(name)
    if case.dtype == "fp32":
        return None
    blk = case.blocks[-1]
    T, C = case.tokens, case.C
    x = case.x.reshape(T, C).cuda()
    qw, sw = swin.fp8_quantize(blk.w_qkv.cuda())
    qa, sa = swin.fp8_quantize(x)
    b = blk.b_qkv.cuda()
    y = swin.fp8_linear(qa, sa, qw, sw, b, out_dtype=x.dtype)
    for _ in range(warmup):
        swin.fp8_quantize(x)
        swin.fp8_linear(qa, sa, qw, sw, b, out=y)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(steps):
        swin.fp8_quantize(x)
    ev[1].record()
    for _ in range(steps):
        swin.fp8_linear(qa, sa, qw, sw, b, out=y)
    ev[2].record()
    torch.cuda.synchronize()
    tq = ev[0].elapsed_time(ev[1]) / steps
    tl = ev[1].elapsed_time(ev[2]) / steps
    tf = 2.0 * T * 3 * C * C / (tl * 1e-3) / 1e12
    out = {"shape": [T, 3 * C, C], "quantize_ms": tq, "linear_ms": tl, "linear_tflops": tf,
           "frac_of_fp8_mfma_peak": tf / PEAK_FP8_TFLOPS}
    if C % 64 == 0:
        # The same shape with 2:4-pruned weights on the sparse matrix cores
        # (flops counted as the dense product's; peak: dense 16-bit x 2).
        vals, codes = swin.sparse24_compress(blk.w_qkv.cuda())
        for _ in range(warmup):
            swin.sparse24_linear(x, vals, codes, b, out=y)
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            swin.sparse24_linear(x, vals, codes, b, out=y)
        ev[1].record()
        torch.cuda.synchronize()
        ts = ev[0].elapsed_time(ev[1]) / steps
        out["sparse24_linear_ms"] = ts
        out["sparse24_dense_equiv_tflops"] = 2.0 * T * 3 * C * C / (ts * 1e-3) / 1e12
    del x, y, qa, sa
    return out


CALIB_BYTES = 256 << 20   # size of the plain device copy that calibrates the HBM counters
CALIB_REPS = 4


def traffic_run(name, steps):
    """Workload steps followed by CALIB_REPS plain device-to-device copies of
    CALIB_BYTES, for two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE)."""
    import torch
    import shifted_window_attention_roll_amd as swin
    swin.load_library()
    r = Runner(name)
    for i in range(steps):
        r.step(i)
    torch.cuda.synchronize()
    src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(CALIB_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"traffic run done: {name}, {steps} steps, {CALIB_REPS} x {CALIB_BYTES} B copies")


def _counter_rows(d):
    import csv
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _per_kernel_kib(rows, counter, kernels):
    """Average counter value (KiB per dispatch) of each named kernel, and the
    per-copy value of the calibration copies (the copy dispatches issued after
    the last workload kernel)."""
    per = {}
    sums = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        did, k, v = int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])
        sums.setdefault((did, k), 0.0)
        sums[(did, k)] += v          # a counter may come as several per-XCD rows
    last = max([d for (d, k) in sums if any(n in k for n in kernels)] or [0])
    calib = [v for (d, k), v in sums.items() if d > last and "copyBuffer" in k]
    for n in kernels:
        vals = [v for (d, k), v in sums.items() if n in k]
        if vals:
            per[n] = (sum(vals) / len(vals), len(vals))
    return per, (sum(calib) / CALIB_REPS if calib else None), len(calib)


def traffic_summarize(name, fetch_dir, write_dir, command):
    """Scale the FETCH_SIZE / WRITE_SIZE counters by what they read for a plain
    copy of known size and store bytes per launch of each kernel."""
    import shifted_window_attention_roll_amd as swin
    import workloads
    case = workloads.make_workload(name, B=1)
    desc = swin.make_desc(case.B, case.H, case.W, case.C, case.heads, case.M,
                          case.blocks[0].s, case.mode, case.torch_dtype)
    kernels = swin.kernel_names(desc)
    fk, fcal, nfc = _per_kernel_kib(_counter_rows(fetch_dir), "FETCH_SIZE", kernels)
    wk, wcal, nwc = _per_kernel_kib(_counter_rows(write_dir), "WRITE_SIZE", kernels)
    if not fcal or not wcal:
        raise SystemExit("calibration copies not found in the counter output")
    fscale = CALIB_BYTES / (fcal * 1024.0)
    wscale = CALIB_BYTES / (wcal * 1024.0)
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    rec = {"entries": {}}
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
    full = workloads.make_workload(name)
    lines = [f"# HBM traffic per launch, {name}", "",
             f"Command: `{command}`", "",
             f"Calibration: {CALIB_REPS} device copies of {CALIB_BYTES} B; FETCH_SIZE reads "
             f"{fcal:.1f} KiB per copy (scale {fscale:.4f}), WRITE_SIZE {wcal:.1f} KiB "
             f"(scale {wscale:.4f}).", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes/launch | "
             "algorithmic bytes/launch | ratio |", "|---|---|---|---|---|---|---|"]
    work = stage_work(full)
    for k in kernels:
        if k not in fk or k not in wk:
            continue
        b = fk[k][0] * 1024.0 * fscale + wk[k][0] * 1024.0 * wscale
        alg = work[k][1]
        rec["entries"][f"{name}:{k}"] = {
            "fetch_kib": fk[k][0], "write_kib": wk[k][0], "fetch_scale": fscale,
            "write_scale": wscale, "bytes_per_launch": b, "algorithmic_bytes": alg,
            "source_digest": source_digest(k), "command": command}
        lines.append(f"| {k} | {fk[k][1]} | {fk[k][0]:.1f} | {wk[k][0]:.1f} | {b:.4g} | "
                     f"{alg:.4g} | {b / alg:.3f} |")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print("\n".join(lines))


def _stats_rows(d):
    import csv
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    return rows


def _launch_durations(d):
    """Per-launch durations (us) by kernel name, in dispatch order, from the
    kernel_trace.csv files under d."""
    import csv
    import collections
    out = collections.defaultdict(list)
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        with open(f) as fh:
            rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
        for r in rows:
            out[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def trace_summarize(name, trace_dir, command):
    """rocprofv3 --kernel-trace --stats output -> profiles/kernel_trace_<workload>.md:
    per kernel of the forward, calls, average / min / max duration and the
    algorithmic rate that average gives."""
    import workloads
    import shifted_window_attention_roll_amd as swin
    case = workloads.make_workload(name)
    desc = swin.make_desc(case.B, case.H, case.W, case.C, case.heads, case.M,
                          case.blocks[0].s, case.mode, case.torch_dtype)
    kernels = swin.kernel_names(desc)
    work = stage_work(case)
    peak_f = PEAK_TFLOPS[case.dtype]
    lines = [f"# Kernel trace, {name}", "", f"Command: `{command}`", "",
             "Durations from rocprofv3 `--kernel-trace --stats` (every launch of the run, "
             "warm-up included); `avg after 5` and `median` from the per-launch trace of the "
             "same run, without each kernel's first 5 launches (the bench's warm-up), for "
             "comparison with the bench's event-timed launches.  Rate = the kernel's "
             "algorithmic flops (bytes) per launch / its average duration.", "",
             "| kernel | calls | avg us | min us | max us | avg after 5 us | median us | "
             "algorithmic GFLOP | TFLOP/s | frac of MFMA peak | algorithmic MB | GB/s |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    launches = _launch_durations(trace_dir)
    total = 0.0
    for r in _stats_rows(trace_dir):
        k = next((n for n in kernels if n in r["Name"]), None)
        if k is None:
            continue
        avg, mn, mx = float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3
        fl, by = work[k]
        total += avg
        ds = launches.get(r["Name"], [])[5:]
        tail = f"{sum(ds) / len(ds):.1f} | {sorted(ds)[len(ds) // 2]:.1f}" if ds else "- | -"
        lines.append(f"| {k} | {r['Calls']} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {tail} | {fl / 1e9:.2f} | "
                     f"{fl / (avg * 1e-6) / 1e12:.0f} | {fl / (avg * 1e-6) / 1e12 / peak_f:.3f} | "
                     f"{by / 1e6:.1f} | {by / (avg * 1e-6) / 1e9:.0f} |")
    T = case.tokens * len(case.blocks)
    fl_step = flops_per_token(case.C, case.M * case.M) * T
    lines += ["", f"Sum of the average durations per step ({len(case.blocks)} block(s)): "
              f"{total * len(case.blocks):.1f} us -> {fl_step / (total * len(case.blocks) * 1e-6) / 1e12:.0f} "
              f"TFLOP/s, {fl_step / (total * len(case.blocks) * 1e-6) / 1e12 / peak_f:.3f} of the "
              f"{peak_f:.0f} TFLOP/s dense {case.dtype} peak."]
    out = os.path.join(ROOT, "profiles", f"kernel_trace_{name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS",
            "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE")


def counters_summarize(name, pmc_dir, command):
    """One rocprofv3 --pmc pass over COUNTERS -> profiles/counters_<workload>.md:
    per kernel, matrix-core busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over the
    SIMDs x GPU cycles; GRBM_GUI_ACTIVE is reported once per XCD), instruction
    mix per matrix-core instruction, and the share of wave time spent waiting."""
    import collections
    import workloads
    import shifted_window_attention_roll_amd as swin
    case = workloads.make_workload(name)
    desc = swin.make_desc(case.B, case.H, case.W, case.C, case.heads, case.M,
                          case.blocks[0].s, case.mode, case.torch_dtype)
    kernels = swin.kernel_names(desc)
    rows = _counter_rows(pmc_dir)
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in rows:
        k = next((n for n in kernels if n in r["Kernel_Name"]), None)
        if k is None:
            continue
        acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    simds = 4 * 256
    lines = [f"# Counters, {name}", "", f"Command: `{command}`", "",
             "Per launch (averaged over the launches of the run).  GPU cycles = "
             "GRBM_GUI_ACTIVE / 8 (one count per XCD).  Matrix-core busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GPU cycles).", "",
             "| kernel | launches | GPU cycles | MFMA instr | matrix-core busy | VALU / MFMA | "
             "LDS / MFMA | wait share of wave cycles |", "|---|---|---|---|---|---|---|---|"]
    for k in kernels:
        if k not in acc:
            continue
        n = len(disp[k])
        a = {c: v / n for c, v in acc[k].items()}
        cyc = a.get("GRBM_GUI_ACTIVE", 0.0) / 8
        mf = a.get("SQ_INSTS_MFMA", 0.0)
        busy = a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (simds * cyc) if cyc else float("nan")
        lines.append(f"| {k} | {n} | {cyc:.0f} | {mf:.0f} | {busy:.3f} | "
                     f"{a.get('SQ_INSTS_VALU', 0.0) / max(mf, 1):.2f} | "
                     f"{a.get('SQ_INSTS_LDS', 0.0) / max(mf, 1):.2f} | "
                     f"{a.get('SQ_WAIT_INST_ANY', 0.0) / max(a.get('SQ_WAVE_CYCLES', 1.0), 1):.3f} |")
    out = os.path.join(ROOT, "profiles", f"counters_{name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=MAIN)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-others", action="store_true", help="skip the other workload shapes")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the informational full-block and backward timings")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the sub-layer backward of --workload, print its JSON")
    ap.add_argument("--traffic-run", action="store_true",
                    help="run --steps steps and the counter calibration copies, print no JSON")
    ap.add_argument("--traffic-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc outputs into profiles/hbm_traffic.json")
    ap.add_argument("--trace-summarize", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace --stats output into "
                         "profiles/kernel_trace_<workload>.md")
    ap.add_argument("--counters-summarize", metavar="PMC_DIR",
                    help="turn a rocprofv3 --pmc output (COUNTERS) into profiles/counters_<workload>.md")
    ap.add_argument("--traffic-command", default="", help="command recorded with the summary")
    args = ap.parse_args()
    if args.traffic_summarize:
        traffic_summarize(args.workload, *args.traffic_summarize, args.traffic_command)
        return
    if args.trace_summarize:
        trace_summarize(args.workload, args.trace_summarize, args.traffic_command)
        return
    if args.counters_summarize:
        counters_summarize(args.workload, args.counters_summarize, args.traffic_command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every window is independent). "
              "Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import shifted_window_attention_roll_amd as swin
    import workloads
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    swin.load_library()
    if args.traffic_run:
        traffic_run(args.workload, args.steps)
        return
    if args.backward_only:
        print(json.dumps({"workload": args.workload,
                          "backward": backward_time(args.workload, args.steps, args.warmup)}),
              flush=True)
        return
    hip = HipEvents()

    log(f"timing {args.workload}: warmup {args.warmup}, steps {args.steps}")
    main_res = measure(args.workload, args.steps, args.warmup, hip)
    log(json.dumps({"workload": args.workload, **{k: main_res[k] for k in
                                                  ("tokens_per_s", "ms_per_step", "tflops",
                                                   "kernel_ms")}}))
    blocks = {}
    backs, fp8s = {}, {}
    if not args.no_block:
        blocks[args.workload] = block_time(args.workload, min(args.steps, 20), 3)
        log(json.dumps({"workload": args.workload, **blocks[args.workload]}))
        backs[args.workload] = backward_time(args.workload, min(args.steps, 10), 2)
        log(json.dumps({"workload": args.workload, "backward": backs[args.workload]}))
        fp8s[args.workload] = fp8_time(args.workload, min(args.steps, 10), 2)
        log(json.dumps({"workload": args.workload, "fp8_qkv": fp8s[args.workload]}))
    others = {}
    if not args.no_others:
        for name in workloads.WORKLOADS:
            if name == args.workload:
                continue
            log(f"timing {name}")
            res = measure(name, min(args.steps, 20), 3, hip)
            others[name] = {k: res[k] for k in ("tokens_per_s", "ms_per_step", "tflops",
                                                "frac_of_mfma_peak", "kernel_ms", "roofline")}
            log(json.dumps({"workload": name, **others[name]}))
            if not args.no_block:
                blocks[name] = block_time(name, min(args.steps, 20), 3)
                log(json.dumps({"workload": name, **blocks[name]}))
                backs[name] = backward_time(name, min(args.steps, 10), 2)
                log(json.dumps({"workload": name, "backward": backs[name]}))
                fp8s[name] = fp8_time(name, min(args.steps, 10), 2)
                log(json.dumps({"workload": name, "fp8_qkv": fp8s[name]}))
    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline(args.workload)
        log(json.dumps(cpu))

    case = workloads.make_workload(args.workload, B=1)
    w = workloads.WORKLOADS[args.workload]
    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "B": w["B"], "H": w["H"], "W": w["W"],
                   "C": w["C"], "heads": w["heads"], "window": w["M"],
                   "shifts": list(w["shifts"]), "mode": w["mode"],
                   "tokens_per_step": main_res["tokens_per_step"], "parallelism": "none"},
        "tflops": main_res["tflops"],
        "frac_of_mfma_peak": main_res["frac_of_mfma_peak"],
        "kernel_ms": main_res["kernel_ms"],
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "workloads": others,
        "full_block": blocks,
        "backward": backs,
        "fp8_qkv": fp8s,
        "source_digest": source_digest(),
    }
    del case
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
