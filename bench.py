#!/usr/bin/env python3
"""Throughput of the fine-grained-scaled FP8 GEMM library on one MI355X.

One step = one call of the library's hot path on one batch of seeded synthetic input that
is already resident in device memory.  The headline workload is the largest one, the
contiguous M-grouped MoE GEMM (8 experts sharing N=4096, K=7168, 32768 routed token rows
padded per expert to multiples of 128, bf16 D); the other workloads (the dense prefill GEMM
M=4096 N=7168 K=2048 with an FP32 C, small and skinny dense, masked MoE replayed from a
captured graph, the UE8M0 forms, the K-grouped MoE weight gradient, the dense NN/TN/TT layouts
and the fused SwiGLU FP8 cast) are timed too and reported under "workloads", each with its own
roofline block.  Inputs rotate over several device-resident copies whose
total exceeds the 256 MB Infinity Cache, so every launch reads its operands from HBM.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOPS (and % of FP8 MFMA / HBM roofline) at 1 GPU"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
ROTATE_BYTES = 1.2e9          # total bytes of rotated input copies per workload
GRAPH_STEPS = 8               # steps captured back to back in one graph


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# the library files each workload's kernels (and their host-side dispatch) are built from
_COMMON_SOURCES = ("dg_api.cpp", "dg_device.h", "dg_internal.h", "dg_tiles.h")
_GEMM = ("dg_gemm.hip",)
WORKLOAD_SOURCES = {
    "dense_small": ("dg_stream.hip",),
    "dense_skinny": ("dg_stream.hip",),
    "dense_skinny_ue8m0": ("dg_stream.hip",),
    "dense_prefill": _GEMM,
    "dense_prefill_ue8m0": _GEMM,
    "dense_prefill_nn": _GEMM + ("dg_layout.hip",),
    "dense_prefill_tn": _GEMM + ("dg_layout.hip",),
    "dense_prefill_tt": _GEMM + ("dg_layout.hip",),
    "moe_contiguous": _GEMM,
    "moe_contiguous_ue8m0": _GEMM,
    "moe_contiguous_swiglu": _GEMM,
    "moe_masked": _GEMM,
    "moe_masked_ue8m0": _GEMM,
    "moe_block": _GEMM,
    "moe_block_unfused": _GEMM + ("dg_quant.hip",),
    "moe_wgrad": ("dg_layout.hip",),
    "moe_swiglu_quant": ("dg_quant.hip",),
}


def kernel_source_hash(workload: str) -> str:
    """Hash of the code of the library files that the workload's kernels are built from, with
    comments and whitespace removed, so that a counter record stays valid across edits that
    cannot change those kernels."""
    h = hashlib.sha256()
    for f in WORKLOAD_SOURCES[workload] + _COMMON_SOURCES:
        with open(os.path.join(ROOT, "moe_grouped_gemm_fp8_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"//[^\n]*|/\*.*?\*/", " ", src, flags=re.S)
        h.update("".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return rec.get("hbm_bytes_per_launch")


class Case:
    """One workload: device copies of its inputs and a launch(i) that runs step i."""

    def __init__(self, name):
        self.name = name
        self.sets = []
        self.config = {}

    def launch(self, i):
        raise NotImplementedError

    def flops(self, i):
        raise NotImplementedError

    def bytes(self, i):
        raise NotImplementedError


def _dev(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _copies(torch, tensors, set_bytes):
    n = int(min(64, max(3, math.ceil(ROTATE_BYTES / max(set_bytes, 1)))))
    out = [tensors]
    for _ in range(n - 1):
        out.append({k: (None if v is None else v.clone()) for k, v in tensors.items()})
    return out


def _capture(torch, sets, call, per_graph=1):
    """Captured graphs over the input copies, as (singles, multi): singles[i] replays the
    library call once on copy i; multi[g] replays it on copies per_graph*g ..
    per_graph*(g+1)-1 in turn, so that back-to-back steps run without a host-side launch
    between them.  An uncaptured call on each copy comes first, on a side stream, so lazily
    allocated state exists before capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in sets:
            call(s)
    torch.cuda.current_stream().wait_stream(side)

    def cap(chunk):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):        # the stream whose workspaces exist
            for s in chunk:
                call(s)
        return gr

    # graphs of earlier workloads are destroyed here, not by the cyclic garbage collector in the
    # middle of a capture (destroying a graph while a stream captures is not permitted)
    gc.collect()
    torch.cuda.synchronize()
    gc.disable()
    try:
        singles = [cap([s]) for s in sets]
        multi = [cap(sets[g0:g0 + per_graph])
                 for g0 in range(0, len(sets) - per_graph + 1, per_graph)]
    finally:
        gc.enable()
    torch.cuda.synchronize()
    return singles, multi


def _steps_per_graph(nsets):
    """Steps per multi-step graph: the largest count up to GRAPH_STEPS that divides the
    number of input copies, so step i always runs on copy i % nsets."""
    return max(d for d in range(1, min(nsets, GRAPH_STEPS) + 1) if nsets % d == 0)


def _graph_launcher(c, singles, multi, per_graph):
    """launch(i, n) runs steps i .. i+n-1: one single-step replay, or (n == per_graph) one
    replay of a multi-step graph."""
    c.cycle = per_graph if multi else 1

    def launch(i, n=1):
        if n == 1:
            singles[i % len(singles)].replay()
        else:
            assert n == c.cycle
            multi[(i // n) % len(multi)].replay()
    c.launch = launch


def _scale_words(k, ue8m0):
    """4-byte scale words per row (or B block) along K: one per K block, or (UE8M0) one per
    four K blocks."""
    kb = k // 128
    return (kb + 3) // 4 if ue8m0 else kb


def make_dense_case(torch, dg, W, name, ue8m0=False, layout="nt"):
    p = W.make_config(name, seed=0, ue8m0=ue8m0)
    if layout != "nt":
        p = W.stored_layout(p, layout)
    c = Case(name + ("_ue8m0" if ue8m0 else "") + ("" if layout == "nt" else "_" + layout))
    t = dict(a=_dev(torch, p.a), sfa=_dev(torch, p.sfa), b=_dev(torch, p.b), sfb=_dev(torch, p.sfb),
             c=None if p.c is None else _dev(torch, p.c),
             d=torch.empty(p.m, p.n, dtype=torch.bfloat16, device="cuda"))
    kb, nb = _scale_words(p.k, ue8m0), (p.n + 127) // 128
    nbytes = (p.m * p.k + p.n * p.k + 4 * p.m * kb + 4 * nb * kb + 2 * p.m * p.n
              + (4 * p.m * p.n if p.c is not None else 0))
    fn = dg.fp8_gemm_nt_ue8m0 if ue8m0 else getattr(dg, "fp8_gemm_" + layout)
    c.sets = _copies(torch, t, nbytes)
    per_graph = _steps_per_graph(len(c.sets))

    def call(s):
        fn(s["a"], s["sfa"], s["b"], s["sfb"], s["d"], s["c"])

    _graph_launcher(c, *_capture(torch, c.sets, call, per_graph), per_graph)
    c.config = dict(workload=c.name, m=p.m, n=p.n, k=p.k, c="fp32" if p.c is not None else None,
                    scales="ue8m0" if ue8m0 else "fp32", layout=layout,
                    d="bf16", launched_as=f"captured graph replay, {c.cycle} steps per graph",
                    rotating_copies=len(c.sets))
    c.flops = lambda i: 2.0 * p.m * p.n * p.k
    c.bytes = lambda i: float(nbytes)
    c.problem = p
    return c


def make_contiguous_case(torch, dg, W, ue8m0=False):
    p = W.make_config("moe_contiguous", seed=0, ue8m0=ue8m0)
    c = Case("moe_contiguous" + ("_ue8m0" if ue8m0 else ""))
    t = dict(a=_dev(torch, p.a), sfa=_dev(torch, p.sfa), b=_dev(torch, p.b), sfb=_dev(torch, p.sfb),
             idx=_dev(torch, p.m_indices),
             d=torch.empty(p.m_total, p.n, dtype=torch.bfloat16, device="cuda"))
    kb, nb = _scale_words(p.k, ue8m0), (p.n + 127) // 128
    valid = int(p.counts.sum())
    used = int((p.counts > 0).sum())
    nbytes = (valid * p.k + used * p.n * p.k + 4 * valid * kb + 4 * used * nb * kb
              + 2 * valid * p.n + 4 * p.m_total)
    c.sets = _copies(torch, t, nbytes)
    per_graph = _steps_per_graph(len(c.sets))

    fn = dg.m_grouped_fp8_gemm_nt_contiguous_ue8m0 if ue8m0 else dg.m_grouped_fp8_gemm_nt_contiguous

    def call(s):
        fn(s["a"], s["sfa"], s["b"], s["sfb"], s["d"], s["idx"])

    _graph_launcher(c, *_capture(torch, c.sets, call, per_graph), per_graph)
    c.config = dict(workload=c.name, groups=p.num_groups, valid_rows=valid,
                    scales="ue8m0" if ue8m0 else "fp32",
                    padded_rows=p.m_total, n=p.n, k=p.k,
                    launched_as=f"captured graph replay, {c.cycle} steps per graph",
                    rotating_copies=len(c.sets))
    c.flops = lambda i: 2.0 * valid * p.n * p.k
    c.bytes = lambda i: float(nbytes)
    c.problem = p
    return c


def make_block_case(torch, dg, W, variant):
    """The experts of an MoE block on the contiguous workload's routing: linear 1 (N = 2I =
    4096 gate and up columns, K = 7168), SwiGLU and the 1x128 FP8 cast, linear 2 (N = 7168,
    K = I = 2048).  variant: "fused" (linear 1 with the activation step in its epilogue, then
    linear 2), "unfused" (linear 1 to bf16, the activation step kernel, linear 2), or
    "linear1_fused" (the fused first GEMM alone)."""
    blk = W.make_config("moe_block", seed=0)
    p = blk.up
    name = {"fused": "moe_block", "unfused": "moe_block_unfused",
            "linear1_fused": "moe_contiguous_swiglu"}[variant]
    c = Case(name)
    i, n2, k = p.n // 2, blk.n2, p.k
    ld = W.sf_aligned(p.m_total)
    t = dict(a=_dev(torch, p.a), sfa=_dev(torch, p.sfa), b=_dev(torch, p.b), sfb=_dev(torch, p.sfb),
             idx=_dev(torch, p.m_indices), b2=_dev(torch, blk.b2), sfb2=_dev(torch, blk.sfb2),
             q=torch.empty(p.m_total, i, dtype=torch.uint8, device="cuda"),
             sfq=torch.zeros(i // 128, ld, dtype=torch.float32, device="cuda"),
             d1=(torch.empty(p.m_total, p.n, dtype=torch.bfloat16, device="cuda")
                 if variant == "unfused" else None),
             d2=(torch.empty(p.m_total, n2, dtype=torch.bfloat16, device="cuda")
                 if variant != "linear1_fused" else None))
    valid = int(p.counts.sum())
    used = int((p.counts > 0).sum())
    kb, nb = k // 128, p.n // 128
    # algorithmic bytes: linear 1's A and B, the codes and scales (written by the activation,
    # read by linear 2), linear 2's B and D; the unfused chain also writes and reads the bf16
    # linear-1 result
    l1 = valid * k + used * p.n * k + 4 * valid * kb + 4 * used * nb * kb + 4 * p.m_total
    act = valid * i + 4 * valid * (i // 128)
    l2 = used * n2 * i + 4 * used * ((n2 + 127) // 128) * (i // 128) + 2 * valid * n2
    if variant == "linear1_fused":
        nbytes, flops = l1 + act, 2.0 * valid * p.n * k
    else:
        nbytes = l1 + 2 * act + l2 + (2 * 2 * valid * p.n if variant == "unfused" else 0)
        flops = 2.0 * valid * (p.n * k + n2 * i)
    c.sets = _copies(torch, t, nbytes)
    per_graph = _steps_per_graph(len(c.sets))

    def call(s):
        if variant == "unfused":
            dg.m_grouped_fp8_gemm_nt_contiguous(s["a"], s["sfa"], s["b"], s["sfb"], s["d1"],
                                                s["idx"])
            dg.swiglu_fp8_quant(s["d1"], s["q"], s["sfq"])
        else:
            dg.m_grouped_fp8_gemm_nt_contiguous_swiglu(s["a"], s["sfa"], s["b"], s["sfb"],
                                                       s["q"], s["sfq"], s["idx"])
        if variant != "linear1_fused":
            dg.m_grouped_fp8_gemm_nt_contiguous(s["q"], s["sfq"], s["b2"], s["sfb2"], s["d2"],
                                                s["idx"])

    _graph_launcher(c, *_capture(torch, c.sets, call, per_graph), per_graph)
    c.config = dict(workload=name, groups=p.num_groups, valid_rows=valid, padded_rows=p.m_total,
                    hidden=k, intermediate=i, out=n2 if variant != "linear1_fused" else None,
                    launched_as=f"captured graph replay, {c.cycle} steps per graph",
                    rotating_copies=len(c.sets))
    c.flops = lambda i_: flops
    c.bytes = lambda i_: float(nbytes)
    return c


def make_masked_case(torch, dg, W, ue8m0=False):
    p = W.make_config("moe_masked", seed=0, ue8m0=ue8m0)
    c = Case("moe_masked" + ("_ue8m0" if ue8m0 else ""))
    g, m_max, n, k = p.num_groups, p.m_max, p.n, p.k
    t = dict(a=_dev(torch, p.a), sfa=_dev(torch, p.sfa), b=_dev(torch, p.b), sfb=_dev(torch, p.sfb),
             d=torch.empty(g, m_max, n, dtype=torch.bfloat16, device="cuda"))
    kb, nb = _scale_words(k, ue8m0), (n + 127) // 128
    set_bytes = g * m_max * k + g * n * k + 2 * g * m_max * n
    c.sets = _copies(torch, t, set_bytes)
    # one masked_m draw per input copy, resident on the device before timing: every step of a
    # replayed graph reads its own draw, so nothing is updated inside the timed region
    table = [W.masked_counts(g, m_max, seed=0, replay=r) for r in range(len(c.sets))]
    for s_, mm in zip(c.sets, table):
        s_["mm"] = _dev(torch, mm)
    per_graph = _steps_per_graph(len(c.sets))
    fn = dg.m_grouped_fp8_gemm_nt_masked_ue8m0 if ue8m0 else dg.m_grouped_fp8_gemm_nt_masked
    _graph_launcher(c, *_capture(torch, c.sets, lambda s_: fn(
        s_["a"], s_["sfa"], s_["b"], s_["sfb"], s_["d"], s_["mm"]), per_graph), per_graph)
    c.config = dict(workload=c.name, groups=g, m_max=m_max, n=n, k=k,
                    scales="ue8m0" if ue8m0 else "fp32",
                    masked_m=f"U{{0..256}} per group, a new draw per step ({len(table)} draws)",
                    launched_as=f"captured graph replay, {c.cycle} steps per graph",
                    rotating_copies=len(c.sets))

    def flops(i):
        return 2.0 * float(table[i % len(table)].sum()) * n * k

    def nbytes(i):
        mm = table[i % len(table)]
        rows = float(mm.sum())
        used = float((mm > 0).sum())
        return (rows * k + used * n * k + 4 * rows * kb + 4 * used * nb * kb + 2 * rows * n + 4 * g)

    c.flops = flops
    c.bytes = nbytes
    return c


def make_kgrouped_case(torch, dg, W):
    p = W.make_config("moe_wgrad", seed=0)
    c = Case("moe_wgrad")
    g, m, n = p.num_groups, p.m, p.n
    t = dict(a=_dev(torch, p.a), sfa=_dev(torch, p.sfa), b=_dev(torch, p.b), sfb=_dev(torch, p.sfb),
             d=torch.empty(g, m, n, dtype=torch.float32, device="cuda"))
    kbt = p.k_total // 128
    tokens = int(p.counts.sum())
    nbytes = p.k_total * (m + n) + 4 * kbt * (m + n) + 4 * g * m * n
    c.sets = _copies(torch, t, nbytes)
    per_graph = _steps_per_graph(len(c.sets))
    ks = [int(x) for x in p.ks]

    def call(s):
        dg.k_grouped_fp8_gemm_tn_contiguous(s["a"], s["sfa"], s["b"], s["sfb"], s["d"], ks)

    _graph_launcher(c, *_capture(torch, c.sets, call, per_graph), per_graph)
    c.config = dict(workload="moe_wgrad", groups=g, m=m, n=n, tokens=tokens,
                    padded_k=p.k_total, d="fp32",
                    launched_as=f"captured graph replay, {c.cycle} steps per graph",
                    rotating_copies=len(c.sets))
    c.flops = lambda i: 2.0 * tokens * m * n
    c.bytes = lambda i: float(nbytes)
    return c


def make_quant_case(torch, dg, W):
    x = W.make_config("moe_swiglu_quant", seed=0)
    m, i = x.shape[0], x.shape[1] // 2
    c = Case("moe_swiglu_quant")
    ld = (m + 3) // 4 * 4
    t = dict(x=_dev(torch, x.view(np.int16)),
             q=torch.empty(m, i, dtype=torch.uint8, device="cuda"),
             sf=torch.empty(i // 128, ld, dtype=torch.float32, device="cuda"))
    nbytes = 4 * m * i + m * i + 4 * m * (i // 128)
    c.sets = _copies(torch, t, nbytes)
    per_graph = _steps_per_graph(len(c.sets))

    def call(s):
        dg.swiglu_fp8_quant(s["x"], s["q"], s["sf"])

    _graph_launcher(c, *_capture(torch, c.sets, call, per_graph), per_graph)
    c.config = dict(workload="moe_swiglu_quant", m=m, i=i, x="bf16 [M, 2I]", q="e4m3 [M, I]",
                    launched_as=f"captured graph replay, {c.cycle} steps per graph",
                    rotating_copies=len(c.sets))
    c.flops = lambda i_: 0.0
    c.bytes = lambda i_: float(nbytes)
    return c


MIN_WARMUP_S = 0.5   # the warm-up also runs until this much time has passed (--min-warmup-s)


def time_case(torch, case, steps, warmup):
    """Warm up, then time exactly `steps` steps as one region bracketed by HIP events on the
    launch stream (the step time and, for cases without a per-step device update, the kernel's
    average launch duration); then a second pass with an event pair around every replay gives
    the spread (and the average for cases whose update copy must stay outside the pair).
    Cases captured `cycle` steps to a graph run whole graphs while at least `cycle` steps
    remain and single-step graphs for the rest, so the count stays exact."""
    cyc = getattr(case, "cycle", 1)
    prep = getattr(case, "prepare", None)

    def chunks(start, count):
        i = 0
        while i < count:
            n = cyc if (cyc > 1 and count - i >= cyc) else 1
            yield start + i, n
            i += n

    # warm-up: the requested steps, then more until half a second has passed, so that clocks
    # and caches are in their steady state when the timed region starts
    t_w = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t_w < MIN_WARMUP_S:
        for i, n in chunks(done, max(cyc, 16)):
            if prep:
                prep(i)
            case.launch(i, n)
        done += max(cyc, 16)
        torch.cuda.synchronize()
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_all0.record()
    for i, n in chunks(warmup, steps):
        if prep:
            prep(i)
        case.launch(i, n)
    t_all1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total = t_all0.elapsed_time(t_all1) * 1e-3
    plan = list(chunks(warmup, steps))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in plan]
    for (i, n), (e0, e1) in zip(plan, ev):
        if prep:
            prep(i)
        e0.record()
        case.launch(i, n)
        e1.record()
    torch.cuda.synchronize()
    per = np.concatenate([np.full(n, e0.elapsed_time(e1) * 1e-3 / n)
                          for (i, n), (e0, e1) in zip(plan, ev)])   # seconds per step
    flops = np.array([case.flops(warmup + i) for i in range(steps)])
    nbytes = np.array([case.bytes(warmup + i) for i in range(steps)])
    avg = per.mean() if prep else total / steps
    return dict(total_s=total, wall_s=wall, per_launch_s=per, avg_s=avg,
                timing="per-launch event pairs" if prep else "timed region / steps",
                steps=steps, flops=flops, bytes=nbytes)


# workloads bound by HBM (their roofline is bytes); the others by the FP8 MFMA rate
HBM_BOUND = ("dense_skinny", "moe_masked", "dense_skinny_ue8m0", "moe_masked_ue8m0",
             "moe_swiglu_quant", "dense_small")


def summarize(name, res):
    per = res["per_launch_s"]
    avg = float(res["avg_s"])
    tflops = float(res["flops"].mean() / avg / 1e12)
    gbs = float(res["bytes"].mean() / avg / 1e9)
    if name in HBM_BOUND:
        roof = dict(bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=gbs / PEAK_HBM_GBS)
    else:
        roof = dict(bound="mfma", achieved=tflops, peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                    frac=tflops / PEAK_FP8_TFLOPS)
    roof["traffic"] = measured_traffic(name)
    roof["algorithmic_bytes"] = float(res["bytes"].mean())
    return dict(avg_kernel_us=avg * 1e6, timing=res["timing"],
                per_launch_event_us=float(per.mean() * 1e6),
                p50_us=float(np.percentile(per, 50) * 1e6),
                p10_us=float(np.percentile(per, 10) * 1e6),
                p90_us=float(np.percentile(per, 90) * 1e6), tflops=tflops, hbm_gbs=gbs,
                frac_fp8_peak=tflops / PEAK_FP8_TFLOPS, frac_hbm_peak=gbs / PEAK_HBM_GBS,
                roofline=roof)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rows(W, p, rows):
    """One oracle call on the first `rows` rows of the workload's A (all of N and K); returns
    the valid-row FLOPs it computed."""
    import oracle
    sfa, sfb = p.sfa, p.sfb
    if sfa.dtype == np.int32:                         # packed UE8M0: the oracle decodes them
        sfa = oracle.ue8m0_decode(sfa, 0, p.k // 128)
        sfb = oracle.ue8m0_decode(sfb, sfb.ndim - 1, p.k // 128)
    sub_sfa = W.mn_major(sfa[:, :rows].T)
    if hasattr(p, "m_indices"):                       # contiguous MoE
        idx = p.m_indices[:rows]
        oracle.m_grouped_contiguous(p.a[:rows], sub_sfa, p.b, sfb, idx)
        return 2.0 * float((idx >= 0).sum()) * p.n * p.k
    oracle.fp8_gemm_nt(p.a[:rows], sub_sfa, p.b, sfb, None if p.c is None else p.c[:rows])
    return 2.0 * rows * p.n * p.k


# the oracle on the two small dense workloads (whole problems), on one thread, in a child process
# (so the parent's thread pool is left as it is)
_ONE_THREAD = r"""
import json, sys, time
sys.path.insert(0, sys.argv[1])
import oracle, workloads as W
oracle.set_num_threads(1)
out = {}
for name in ("dense_small", "dense_skinny"):
    p = W.make_config(name, seed=0)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.fp8_gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 2.0:
            break
    out[name] = dict(tflops=2.0 * p.m * p.n * p.k * reps / dt / 1e12, reps=reps,
                     seconds=round(dt, 2), threads=oracle.num_threads())
print(json.dumps(out))
"""


def cpu_baseline(W, case, target_s):
    """The CPU oracle on a bounded sample of the workload: the first rows of A (all of N and K),
    grown until one call takes a good part of `target_s`, then repeated to about `target_s`;
    plus the two small dense workloads in full on one thread."""
    import subprocess

    import oracle
    p = case.problem
    m_rows = p.m_total if hasattr(p, "m_total") else p.m
    log("timing the CPU oracle on a row sample of the workload")
    rows = 2
    while True:
        t0 = time.perf_counter()
        _oracle_rows(W, p, rows)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or rows >= m_rows:
            break
        rows = int(min(m_rows, max(rows * 2, rows * target_s / 4 / max(dt, 1e-3))))
    flops = 0.0
    t_all = time.perf_counter()
    reps = 0
    while time.perf_counter() - t_all < target_s:
        flops += _oracle_rows(W, p, rows)
        reps += 1
    total = time.perf_counter() - t_all
    out = dict(value=flops / total / 1e12, unit="TFLOPS", cores=oracle.num_threads(),
               kind="oracle", cpu_model=_cpu_model(),
               sample=f"{reps} x the first {rows} of {m_rows} rows of the {case.name} workload "
                      f"(all N={p.n}, K={p.k}), {total:.1f} s of float64 work")
    log("timing the CPU oracle on one thread (dense_small, dense_skinny)")
    r = subprocess.run([sys.executable, "-c", _ONE_THREAD, ROOT], capture_output=True,
                       text=True, timeout=120)
    if r.returncode == 0 and r.stdout.strip():
        out["one_thread"] = json.loads(r.stdout.strip().splitlines()[-1])
    else:
        out["one_thread"] = dict(error=(r.stderr or "")[-300:])
    return out


def calibration_copy(torch):
    """A plain device-to-device copy of 1 GiB from a source written long before (evicted from
    the caches by 2 GiB of other writes): the HBM-traffic counters of this copy, divided by
    its known 1 GiB read and 1 GiB write, give their scale factors."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    flush = torch.empty(2 * n, dtype=torch.uint8, device="cuda")
    flush.fill_(2)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log("calibration copy of 1 GiB done")
    del src, flush, dst
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="moe_contiguous",
                    choices=["dense_small", "dense_prefill", "dense_skinny", "moe_contiguous",
                             "moe_masked", "dense_prefill_ue8m0", "dense_skinny_ue8m0",
                             "moe_contiguous_ue8m0", "moe_masked_ue8m0", "moe_wgrad",
                             "dense_prefill_nn", "dense_prefill_tn", "dense_prefill_tt",
                             "moe_swiglu_quant", "moe_contiguous_swiglu", "moe_block",
                             "moe_block_unfused"])
    ap.add_argument("--only", action="store_true", help="time the headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--min-warmup-s", type=float, default=MIN_WARMUP_S,
                    help="warm-up time floor (0 under a profiler: warm-up steps only)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a 1 GiB device copy (reference for HBM-traffic counters)")
    args = ap.parse_args()
    globals()["MIN_WARMUP_S"] = args.min_warmup_s

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this library"
              " has no multi-GPU path: each GPU would run its own shard independently)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_grouped_gemm_fp8_amd as dg
    import workloads as W

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    log(f"device {torch.cuda.get_device_name(0)}, {dg.get_num_cus()} CUs")
    if args.calibrate_copy:
        calibration_copy(torch)

    makers = {
        "dense_small": lambda: make_dense_case(torch, dg, W, "dense_small"),
        "dense_prefill": lambda: make_dense_case(torch, dg, W, "dense_prefill"),
        "dense_skinny": lambda: make_dense_case(torch, dg, W, "dense_skinny"),
        "moe_contiguous": lambda: make_contiguous_case(torch, dg, W),
        "moe_masked": lambda: make_masked_case(torch, dg, W),
        "dense_prefill_ue8m0": lambda: make_dense_case(torch, dg, W, "dense_prefill", True),
        "dense_skinny_ue8m0": lambda: make_dense_case(torch, dg, W, "dense_skinny", True),
        "moe_contiguous_ue8m0": lambda: make_contiguous_case(torch, dg, W, True),
        "moe_masked_ue8m0": lambda: make_masked_case(torch, dg, W, True),
        "moe_wgrad": lambda: make_kgrouped_case(torch, dg, W),
        "dense_prefill_nn": lambda: make_dense_case(torch, dg, W, "dense_prefill", layout="nn"),
        "dense_prefill_tn": lambda: make_dense_case(torch, dg, W, "dense_prefill", layout="tn"),
        "dense_prefill_tt": lambda: make_dense_case(torch, dg, W, "dense_prefill", layout="tt"),
        "moe_swiglu_quant": lambda: make_quant_case(torch, dg, W),
        "moe_contiguous_swiglu": lambda: make_block_case(torch, dg, W, "linear1_fused"),
        "moe_block": lambda: make_block_case(torch, dg, W, "fused"),
        "moe_block_unfused": lambda: make_block_case(torch, dg, W, "unfused"),
    }
    order = [args.workload] + ([] if args.only else [w for w in makers if w != args.workload])
    results = {}
    head = None
    for name in order:
        log(f"preparing {name}")
        case = makers[name]()
        # the short workloads take many steps (their spread matters); the long ones fewer
        steps = args.steps if name == args.workload else (
            200 if name in ("dense_small", "dense_skinny", "moe_masked", "dense_skinny_ue8m0",
                            "moe_masked_ue8m0", "moe_swiglu_quant")
            else max(20, args.steps // 2))
        log(f"timing {name}: {args.warmup} warm-up + {steps} steps")
        res = time_case(torch, case, steps, args.warmup)
        summ = summarize(name, res)
        summ["config"] = case.config
        results[name] = summ
        log(f"{name}: {summ['avg_kernel_us']:.1f} us/launch, {summ['tflops']:.1f} TFLOPS, "
            f"{summ['hbm_gbs']:.0f} GB/s")
        if name == args.workload:
            head = (case, res, summ, steps)
        else:
            del case
            gc.collect()
            torch.cuda.empty_cache()

    case, res, summ, _ = head
    steps = res["steps"]
    total_flops = float(res["flops"].sum())
    value = total_flops / res["total_s"] / 1e12
    dom = case.name
    roofline = dict(summ["roofline"], kernel_avg_us=summ["avg_kernel_us"],
                    hbm_gbs_algorithmic=summ["hbm_gbs"],
                    hbm_frac_algorithmic=summ["hbm_gbs"] / PEAK_HBM_GBS)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": res["total_s"] / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic (seeded N(0,1) cast to e4m3 with 1x128 / 128x128 FP32 scales)",
        "config": case.config,
        "roofline": roofline,
        "workloads": results,
    }
    if not args.no_cpu and hasattr(case, "problem"):
        out["cpu_baseline"] = cpu_baseline(W, case, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
