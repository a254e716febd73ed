#!/usr/bin/env python3
"""Benchmark of the long-context causal attention hot path on one MI355X.

Headline step (``value``): one training pass of causal attention at the
largest single-GPU workload, ``train_64k`` (B = 1, 8 heads, N = 65536,
D = 128, seeded bf16 N(0,1) inputs already resident in HBM):

  attn_fwd (O, LSE)  ->  attn_bwd (dQ, dK, dV from the forward's O and LSE)

``value`` = algorithmic flops of the step (forward 2 B H D N (N+1), backward
2.5x that; masked pairs are not counted) / step time.  ``roofline`` is the
dominant kernel of that step (most GPU time), timed with HIP events around
each of its launches over the timed steps.

Legs timed apart from the step, each with the roofline of its kernels
(``rooflines``): the glossary example's 4K shape (forward, plain and
split-KV), one Ulysses shard of a 32K-token layer (relayout GB/s, forward,
the four ring partials + merge, backward, inverse relayout), the ring workload
at its configured shape (8 heads, four 8192-key fp32 partials + the 609 MB
merge), the 512K-token forward of one Ulysses share, and the backward of the
64K shape again from the other legs' viewpoint.  ``cpu_baseline`` times the
fp64 oracle on the host cores on bounded samples of every workload.

``--only WORKLOAD`` runs one workload alone (for a profiler: its kernels and
nothing else).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBPS = 8000.0
WORKLOAD_NAMES = ("train_64k", "listing_4k", "ulysses_shard_32k", "ring_blocks_32k", "ulysses_512k")


def fwd_flops(B, Hq, N, D):
    """Causal forward: 4*D flops per visible (query, key) pair, N(N+1)/2 pairs."""
    return 2.0 * B * Hq * D * N * (N + 1)


def pair_flops_block(Hq, D, N, a, b):
    """Forward flops of queries 0..N-1 against keys [a, b) (causal, global
    positions): key j is seen by the N - j queries at or after it."""
    pairs = (b - a) * N - (b * (b - 1) // 2 - a * (a - 1) // 2)
    return 4.0 * Hq * D * pairs


# (the dK/dV kernel's dense D = 128 instances are compiled from attn_bwd.hip
# in the units attn_bwd_ds.hip and attn_bwd_dkdv_recompute.hip, with their
# flags)
KERNEL_SOURCES = {"bwd_dkdv_kernel": ("attn_bwd.hip", "attn_bwd_ds.hip", "attn_bwd_dkdv_recompute.hip"),
                  "bwd_dq_kernel": "attn_bwd.hip", "bwd_dq_ds_kernel": "attn_bwd.hip",
                  "bwd_delta_kernel": "attn_bwd.hip", "bwd_dkdv_reduce_kernel": "attn_bwd.hip",
                  "attn_fwd_kernel": "attn_fwd.hip", "attn_fwd_kernel_fp32out": "attn_fwd.hip",
                  "transpose_rows_kernel": "relayout.hip", "merge_kernel": "merge.hip"}


def kernel_source_digest(name):
    """sha256 of the sources a kernel is compiled from and of that file's
    own compiler flags (to tell whether committed counter figures still
    describe it)."""
    from long_context_attention_fwd_amd.build import PER_FILE
    f = KERNEL_SOURCES.get(name)
    if f is None:
        return None
    files = f if isinstance(f, tuple) else (f,)
    csrc = os.path.join(ROOT, "long_context_attention_fwd_amd", "csrc")
    h = hashlib.sha256()
    for fn in (*files, "device_common.hpp"):
        with open(os.path.join(csrc, fn), "rb") as fh:
            h.update(fh.read())
    for fn in files:
        flags = PER_FILE.get(fn)
        if flags:
            h.update(" ".join(flags).encode())
    return h.hexdigest()


def measured_traffic(name, workload):
    """HBM bytes per launch of kernel ``name`` on ``workload`` from the
    committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled by
    a copy of known size), or None when there is none or the kernel's
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_digest(name):
        return None
    try:
        return {"read_bytes": float(fields["read_bytes_per_launch"]),
                "write_bytes": float(fields["write_bytes_per_launch"]),
                "source": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError):
        return None


def bwd_workspace(lc, torch, dev, B, Hq, Hkv, N, D):
    """attn_bwd's workspace as the binding allocates it by default: room for
    the stored dS (dq as its product) when the shape has that path and it
    fits lc.STORED_DS_AUTO_BYTES, else the minimal one (dq recomputed).
    Returns (workspace, stored)."""
    need = lc.attn_bwd_ds_workspace_size(B, Hq, Hkv, N, D, True)
    stored = 0 < need <= lc.STORED_DS_AUTO_BYTES
    if not stored:
        need = lc.attn_bwd_workspace_size(B, Hq, Hkv, N, D)
    return torch.empty(max(16, need), dtype=torch.uint8, device=dev), stored


def ds_pass_bytes(B, Hq, Hkv, N, D):
    """Algorithmic HBM bytes of the product pass dq = scale dS K (causal,
    Nq = Nk = N): every stored 64 x 64 dS block a query tile's rows see, read
    once (bf16), K read once per key/value head, dq written (bf16)."""
    nqt = (N + 63) // 64
    blocks = sum(min(nqt, 2 * (qt // 2) + 2) for qt in range(nqt))
    return B * Hq * blocks * 64 * 64 * 2 + 2 * B * Hkv * N * D + 2 * B * Hq * N * D


def tflops(f, ms):
    return f / (ms * 1e-3) / 1e12


def gbps(b, ms):
    return b / (ms * 1e-3) / 1e9


def roofline_entry(kernel, traced, work_per_launch, unit, workload):
    """Roofline of one kernel from its traced launches: algorithmic work per
    launch / average launch duration, against the MI355X peak of its bound."""
    tot_ms, calls = traced[kernel]
    avg_ms = tot_ms / calls
    mfma = unit == "TFLOP/s"
    achieved = tflops(work_per_launch, avg_ms) if mfma else gbps(work_per_launch, avg_ms)
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBPS
    ent = {"bound": "mfma" if mfma else "hbm", "kernel": kernel, "achieved": round(achieved, 2), "peak": peak,
           "unit": "TFLOP/s" if mfma else "GB/s", "frac": round(achieved / peak, 4), "traffic": None,
           "avg_launch_us": round(1e3 * avg_ms, 2), "launches": calls, "algorithmic_per_launch": work_per_launch}
    t = measured_traffic(kernel, workload)
    if t is not None:
        ent["traffic"] = t["read_bytes"] + t["write_bytes"]
        ent["traffic_detail"] = t
    return ent


def traced_calls(lc, torch, fn, iters, warmup):
    """fn() warmup times, then iters times with every library kernel
    bracketed by HIP events; returns (ms per call from events around all
    iters, {kernel: (total_ms, launches)})."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    lc.trace_collect()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lc.trace_enable(True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    lc.trace_enable(False)
    return e0.elapsed_time(e1) / iters, lc.trace_collect()


def time_calls(torch, fn, iters=10, warmup=3, rounds=3):
    """ms of fn() on the current stream (events): the median over rounds of
    the average over iters calls, so that a one-off stall of the machine does not
    set the figure."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    avgs = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        avgs.append(e0.elapsed_time(e1) / iters)
    return sorted(avgs)[len(avgs) // 2]


_HOST_INPUTS = {}


def host_inputs(name):
    """Seeded bf16 bit patterns of a workload (the same arrays the oracle
    baseline decodes), drawn once per run."""
    from long_context_attention_fwd_amd.inputs import WORKLOADS, make_workload_inputs, normal_bf16
    if name not in _HOST_INPUTS:
        w = WORKLOADS[name]
        d = make_workload_inputs(w)
        if name == "ulysses_shard_32k":  # the shard step's backward needs dO, drawn token-major like q
            import numpy as np
            d["do"] = normal_bf16(np.random.default_rng(w.seed + 17), (w.P, w.N // w.P, w.Hq, w.D))
        _HOST_INPUTS[name] = d
    return _HOST_INPUTS[name]


def to_dev(torch, bits, dev):
    import numpy as np
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--only", choices=list(WORKLOAD_NAMES) + ["ulysses_shard_32k_extras"],
                   help="run one workload alone (for a profiler); ulysses_shard_32k_extras: the shard leg with "
                        "its extra variants")
    p.add_argument("--calibration-copy", action="store_true",
                   help="with --only: first one elementwise kernel of known traffic (1 GiB fp32 read, 1 GiB "
                        "written), the reference for scaling the profiler's byte counters")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the shard leg's extra variants (token-major, streamed ring, ring sharding)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# headline: the 64K training step
# ---------------------------------------------------------------------------
def train_64k(lc, torch, dev, steps, warmup):
    from long_context_attention_fwd_amd.inputs import WORKLOADS
    w = WORKLOADS["train_64k"]
    d = host_inputs(w.name)
    q, k, v, do = (to_dev(torch, d[n], dev) for n in ("q", "k", "v", "do"))
    B, Hq, N, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws, stored = bwd_workspace(lc, torch, dev, B, Hq, w.Hkv, N, D)
    stream = torch.cuda.current_stream(dev)
    f_fwd = fwd_flops(B, Hq, N, D)
    f_bwd = 2.5 * f_fwd

    def step(record):
        marks = []

        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                marks.append(e)
        mark()
        lc.attn_fwd(q, k, v, causal=True, scale=w.scale, o=o, lse=lse)
        mark()
        lc.attn_bwd(q, k, v, o, do, lse, causal=True, scale=w.scale, workspace=ws, dq=dq, dk=dk, dv=dv)
        mark()
        return marks

    torch.cuda.synchronize()
    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    lc.trace_collect()  # drop the warmup's records
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    all_marks = []
    torch.cuda.synchronize()
    lc.trace_enable(True)
    t0.record(stream)
    for _ in range(steps):
        all_marks.append(step(True))
    t1.record(stream)
    torch.cuda.synchronize()
    lc.trace_enable(False)
    tr = lc.trace_collect()
    ms_step = t0.elapsed_time(t1) / steps
    ph = [sum(m[i].elapsed_time(m[i + 1]) for m in all_marks) / steps for i in range(2)]
    work = {"attn_fwd_kernel": ("TFLOP/s", f_fwd), "bwd_dkdv_kernel": ("TFLOP/s", 0.8 * f_bwd),
            "bwd_dq_kernel": ("TFLOP/s", 0.2 * f_bwd), "bwd_dq_ds_kernel": ("GB/s", ds_pass_bytes(B, Hq, w.Hkv, N, D)),
            "bwd_delta_kernel": ("GB/s", 2 * 2 * B * Hq * N * D + 4 * B * Hq * N)}
    gpu_kernels = {}
    for name, (tot, calls) in tr.items():
        ent = {"calls_per_step": calls / steps, "avg_us": round(1e3 * tot / calls, 2),
               "share_of_step": round(tot / (ms_step * steps), 4)}
        if name in work:
            unit, wk = work[name]
            rate = tflops(wk, tot / calls) if unit == "TFLOP/s" else gbps(wk, tot / calls)
            ent[unit] = round(rate, 2)
            ent["frac_peak"] = round(rate / (PEAK_BF16_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBPS), 4)
        gpu_kernels[name] = ent
    dom = max(tr, key=lambda n: tr[n][0])
    rl = {n: roofline_entry(n, tr, work[n][1], work[n][0], w.name) for n in work if n in tr}
    res = {
        "value": round(tflops(f_fwd + f_bwd, ms_step), 3), "ms_per_step": round(ms_step, 4),
        "config": {"workload": w.name, "B": B, "Hq": Hq, "Hkv": w.Hkv, "N": N, "D": D, "causal": True,
                   "seed": w.seed, "step": "attn_fwd -> attn_bwd (dQ, dK, dV from the forward's O and LSE)",
                   "dq_path": "product of the stored dS" if stored else "recomputing dQ pass",
                   "bwd_workspace_bytes": ws.numel(), "algorithmic_flops_per_step": f_fwd + f_bwd},
        "phases": {"fwd": {"ms": round(ph[0], 4), "TFLOP/s": round(tflops(f_fwd, ph[0]), 2),
                           "frac_peak": round(tflops(f_fwd, ph[0]) / PEAK_BF16_TFLOPS, 4)},
                   "bwd": {"ms": round(ph[1], 4), "TFLOP/s": round(tflops(f_bwd, ph[1]), 2),
                           "frac_peak": round(tflops(f_bwd, ph[1]) / PEAK_BF16_TFLOPS, 4)}},
        "gpu_kernels": gpu_kernels,
        "roofline": rl[dom],
        "rooflines": {f"{w.name}.{n}": r for n, r in rl.items()},
    }
    return res


# ---------------------------------------------------------------------------
# legs
# ---------------------------------------------------------------------------
def leg_listing_4k(lc, torch, dev, iters=50, warmup=10):
    """The glossary example's shape ([1, 4, 4096, 64], causal): its whole
    training step (split-KV forward, the gradient of its loss mean(O^2), i.e.
    dO = 2 O / numel, and the backward), eager and replayed as one HIP graph;
    then attn_fwd, and attn_fwd_splitkv with the library's choice of key
    ranges (one workgroup per 256 query rows gives only 64 workgroups here, so
    the longest row sets attn_fwd's time); then attn_bwd alone, whose passes
    run over query and key ranges at this size, the dQ pass beside the dK/dV
    pass."""
    from long_context_attention_fwd_amd.inputs import WORKLOADS
    w = WORKLOADS["listing_4k"]
    d = host_inputs(w.name)
    q, k, v = (to_dev(torch, d[n], dev) for n in "qkv")
    B, Hq, N, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    ws = torch.empty(lc.attn_fwd_splitkv_workspace_size(B, Hq, w.Hkv, N, N, D, True, 0), dtype=torch.uint8,
                     device=dev)
    f = fwd_flops(B, Hq, N, D)
    f_bwd = 2.5 * f
    res = {"workload": w.name, "shape": [B, Hq, N, D], "causal": True, "algorithmic_flops": f}
    rls = {}
    do = torch.empty_like(q)
    wsb = torch.empty(max(16, lc.attn_bwd_workspace_size(B, Hq, w.Hkv, N, D)), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    # the example's whole training step at this size is launch-bound (two
    # forward launches, the loss gradient, five backward launches and the side
    # stream's fork and join): eager, and captured once into a HIP graph
    def train_step():
        lc.attn_fwd_splitkv(q, k, v, scale=w.scale, workspace=ws, o=o, lse=lse)
        torch.mul(o, 2.0 / o.numel(), out=do)
        lc.attn_bwd(q, k, v, o, do, lse, scale=w.scale, workspace=wsb, dq=dq, dk=dk, dv=dv)
    step = {"call": "attn_fwd_splitkv, dO of mean(O^2), attn_bwd"}
    ms = time_calls(torch, train_step, iters, warmup)
    step["eager"] = {"us": round(1e3 * ms, 2), "TFLOP/s": round(tflops(f + f_bwd, ms), 2)}
    try:  # a secondary figure: a failed capture is reported, not fatal to the run
        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            train_step()  # the capture stream's side stream exists before the capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            train_step()
        ms = time_calls(torch, graph.replay, iters, warmup)
        step["graph"] = {"us": round(1e3 * ms, 2), "TFLOP/s": round(tflops(f + f_bwd, ms), 2)}
    except RuntimeError as e:
        step["graph"] = {"error": str(e)[:200]}
        torch.cuda.synchronize()
    res["train_step"] = step

    # the kernels, one call at a time (after the step, so that the launches a
    # profiler sees last are the ones timed here)
    for name, fn in (("attn_fwd", lambda: lc.attn_fwd(q, k, v, scale=w.scale, o=o, lse=lse)),
                     ("attn_fwd_splitkv", lambda: lc.attn_fwd_splitkv(q, k, v, scale=w.scale, workspace=ws, o=o,
                                                                      lse=lse))):
        ms, tr = traced_calls(lc, torch, fn, iters, warmup)
        ms_plain = time_calls(torch, fn, iters, warmup)  # without the per-launch events
        res[name] = {"us": round(1e3 * ms_plain, 2), "TFLOP/s": round(tflops(f, ms_plain), 2),
                     "frac_peak": round(tflops(f, ms_plain) / PEAK_BF16_TFLOPS, 4),
                     "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in tr.items()}}
        kern = "attn_fwd_kernel" if name == "attn_fwd" else "attn_fwd_kernel_fp32out"
        rls[f"{w.name}.{name}"] = roofline_entry(kern, tr, f, "TFLOP/s", w.name)
    lc.attn_fwd(q, k, v, scale=w.scale, o=o, lse=lse)
    torch.mul(o, 2.0 / o.numel(), out=do)

    def bwd():
        lc.attn_bwd(q, k, v, o, do, lse, scale=w.scale, workspace=wsb, dq=dq, dk=dk, dv=dv)
    ms, tr = traced_calls(lc, torch, bwd, iters, warmup)
    ms_plain = time_calls(torch, bwd, iters, warmup)
    res["attn_bwd"] = {"us": round(1e3 * ms_plain, 2), "TFLOP/s": round(tflops(f_bwd, ms_plain), 2),
                       "frac_peak": round(tflops(f_bwd, ms_plain) / PEAK_BF16_TFLOPS, 4),
                       "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in tr.items()},
                       "loss": "mean(O^2): dO = 2 O / numel"}
    rls[f"{w.name}.bwd_dkdv_kernel"] = roofline_entry("bwd_dkdv_kernel", tr, 0.8 * f_bwd, "TFLOP/s", w.name)
    rls[f"{w.name}.bwd_dq_kernel"] = roofline_entry("bwd_dq_kernel", tr, 0.2 * f_bwd, "TFLOP/s", w.name)

    return res, rls


def leg_ulysses_512k(lc, torch, dev, iters=3, warmup=1):
    """The 512K-token forward of one Ulysses share: 4 query heads on 1
    key/value head, seeded inputs 0.5 N(0,1)."""
    from long_context_attention_fwd_amd.inputs import WORKLOADS
    w = WORKLOADS["ulysses_512k"]
    d = host_inputs(w.name)
    q, k, v = (to_dev(torch, d[n], dev) for n in "qkv")
    B, Hq, N, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    f = fwd_flops(B, Hq, N, D)
    ms, tr = traced_calls(lc, torch, lambda: lc.attn_fwd(q, k, v, scale=w.scale, o=o, lse=lse), iters, warmup)
    res = {"workload": w.name, "shape": [B, Hq, N, D], "kv_heads": w.Hkv, "ms": round(ms, 3),
           "TFLOP/s": round(tflops(f, ms), 2), "frac_peak": round(tflops(f, ms) / PEAK_BF16_TFLOPS, 4),
           "algorithmic_flops": f}
    return res, {f"{w.name}.attn_fwd": roofline_entry("attn_fwd_kernel", tr, f, "TFLOP/s", w.name)}


def leg_ring_blocks_32k(lc, torch, dev, iters=10, warmup=2):
    """The ring workload at its configured shape: B = 1, 8 heads (8 KV heads),
    N = 32768, four contiguous 8192-key blocks: the four partial forwards
    (fp32 O and LSE per block, one grouped launch: they are independent) and
    attn_partial_merge of the four fp32 partials (609 MB of HBM traffic), and
    the full attn_fwd for comparison."""
    from long_context_attention_fwd_amd.inputs import WORKLOADS
    w = WORKLOADS["ring_blocks_32k"]
    d = host_inputs(w.name)
    q, k, v = (to_dev(torch, d[n], dev) for n in "qkv")
    B, H, N, D = q.shape
    nb = w.kv_blocks
    blk = N // nb
    kb = [k[:, :, a:a + blk].contiguous() for a in range(0, N, blk)]
    vb = [v[:, :, a:a + blk].contiguous() for a in range(0, N, blk)]
    o_parts = torch.empty((nb, B, H, N, D), dtype=torch.float32, device=dev)
    lse_parts = torch.empty((nb, B, H, N), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    f_parts = sum(pair_flops_block(H, D, N, a, a + blk) for a in range(0, N, blk))
    merge_bytes = o_parts.numel() * 4 + lse_parts.numel() * 4 + o.numel() * 2 + lse.numel() * 4

    def partials():
        lc.attn_fwd_accumulate_group([dict(q=q, k=kb[i], v=vb[i], o_acc=o_parts[i], lse_acc=lse_parts[i], first=True,
                                           k_pos0=i * blk) for i in range(nb)], causal=True, scale=w.scale)
    ms_p, tr_p = traced_calls(lc, torch, partials, iters, warmup)
    ms_m, tr_m = traced_calls(lc, torch, lambda: lc.attn_partial_merge(o_parts, lse_parts, o=o, lse=lse), iters,
                              warmup)
    ms_f, tr_f = traced_calls(lc, torch, lambda: lc.attn_fwd(q, k, v, scale=w.scale, o=o, lse=lse), iters, warmup)
    res = {"workload": w.name, "shape": [B, H, N, D], "kv_blocks": nb,
           "partials_x4": {"ms": round(ms_p, 4), "TFLOP/s": round(tflops(f_parts, ms_p), 2),
                           "frac_peak": round(tflops(f_parts, ms_p) / PEAK_BF16_TFLOPS, 4)},
           "merge": {"ms": round(ms_m, 4), "bytes": merge_bytes, "GB/s": round(gbps(merge_bytes, ms_m), 1),
                     "frac_peak": round(gbps(merge_bytes, ms_m) / PEAK_HBM_GBPS, 4)},
           "partials_plus_merge_ms": round(ms_p + ms_m, 4),
           "full_attn_fwd": {"ms": round(ms_f, 4), "TFLOP/s": round(tflops(f_parts, ms_f), 2),
                             "frac_peak": round(tflops(f_parts, ms_f) / PEAK_BF16_TFLOPS, 4)}}
    rls = {f"{w.name}.partials": roofline_entry("attn_fwd_kernel_fp32out", tr_p, f_parts, "TFLOP/s", w.name),
           f"{w.name}.merge": roofline_entry("merge_kernel", tr_m, merge_bytes, "GB/s", w.name),
           f"{w.name}.attn_fwd": roofline_entry("attn_fwd_kernel", tr_f, f_parts, "TFLOP/s", w.name)}
    return res, rls


def leg_ulysses_shard_32k(lc, torch, dev, steps, warmup, extras):
    """One GPU's Ulysses share of a Llama-3-8B-shaped layer (32 query / 8
    key-value heads, D = 128, N = 32768 split P = 8 ways), the whole path in
    one step:
      1. seq_to_head_relayout_batch of Q, K, V, dO (all P shards, one launch)
      2. attn_fwd on shard 0 (4 query heads, 1 KV head, causal GQA)
      3. the ring form of the same forward: 4 partial calls over 8192-key
         blocks (fp32, one grouped launch) + attn_partial_merge
      4. attn_bwd on shard 0 (from step 2's O and LSE)
      5. head_to_seq_relayout_batch of O, dQ, dK, dV (one launch)"""
    from long_context_attention_fwd_amd.inputs import WORKLOADS
    w = WORKLOADS["ulysses_shard_32k"]
    P, N, D, Hq, Hkv = w.P, w.N, w.D, w.Hq, w.Hkv
    hq, hkv = Hq // P, Hkv // P
    d = host_inputs(w.name)
    xs = {n: to_dev(torch, d[n], dev) for n in ("q", "k", "v", "do")}
    heads = {"q": torch.empty((P, hq, N, D), dtype=torch.bfloat16, device=dev),
             "do": torch.empty((P, hq, N, D), dtype=torch.bfloat16, device=dev),
             "k": torch.empty((P, hkv, N, D), dtype=torch.bfloat16, device=dev),
             "v": torch.empty((P, hkv, N, D), dtype=torch.bfloat16, device=dev)}
    # shard 0's results go straight into slot 0 of the head-major buffers; the
    # inverse relayout moves all P shards' bytes, as the exchange would
    o_all = torch.zeros((P, hq, N, D), dtype=torch.bfloat16, device=dev)
    dq_all = torch.zeros_like(o_all)
    dk_all = torch.zeros((P, hkv, N, D), dtype=torch.bfloat16, device=dev)
    dv_all = torch.zeros_like(dk_all)
    o, dq, dk, dv = o_all[0:1], dq_all[0:1], dk_all[0:1], dv_all[0:1]
    lse = torch.empty((1, hq, N), dtype=torch.float32, device=dev)
    o_tok = torch.empty((P, N // P, Hq, D), dtype=torch.bfloat16, device=dev)
    dq_tok = torch.empty_like(o_tok)
    dk_tok = torch.empty((P, N // P, Hkv, D), dtype=torch.bfloat16, device=dev)
    dv_tok = torch.empty_like(dk_tok)
    n_blk = 4
    blk = N // n_blk
    o_parts = torch.empty((n_blk, 1, hq, N, D), dtype=torch.float32, device=dev)
    lse_parts = torch.empty((n_blk, 1, hq, N), dtype=torch.float32, device=dev)
    o_ring = torch.empty((1, hq, N, D), dtype=torch.bfloat16, device=dev)
    lse_ring = torch.empty_like(lse)
    ws, stored = bwd_workspace(lc, torch, dev, 1, hq, hkv, N, D)
    scale = w.scale
    stream = torch.cuda.current_stream(dev)
    ring_blocks = [(a, heads["k"][0:1, :, a:a + blk], heads["v"][0:1, :, a:a + blk]) for a in range(0, N, blk)]
    assert all(kb.is_contiguous() and vb.is_contiguous() for _, kb, vb in ring_blocks)
    names = ["relayout_in", "fwd", "ring_partials", "merge", "bwd", "relayout_out"]

    def step(record):
        marks = []

        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                marks.append(e)
        mark()
        lc.seq_to_head_relayout_batch([xs[n] for n in ("q", "k", "v", "do")], P,
                                      outs=[heads[n] for n in ("q", "k", "v", "do")])
        mark()
        q0, k0, v0, do0 = (heads[n][0:1] for n in ("q", "k", "v", "do"))
        lc.attn_fwd(q0, k0, v0, causal=True, scale=scale, o=o, lse=lse)
        mark()
        lc.attn_fwd_accumulate_group(
            [dict(q=q0, k=kb, v=vb, o_acc=o_parts[i], lse_acc=lse_parts[i], first=True, k_pos0=a)
             for i, (a, kb, vb) in enumerate(ring_blocks)], causal=True, scale=scale)
        mark()
        lc.attn_partial_merge(o_parts, lse_parts, o=o_ring, lse=lse_ring)
        mark()
        lc.attn_bwd(q0, k0, v0, o, do0, lse, causal=True, scale=scale, workspace=ws, dq=dq, dk=dk, dv=dv)
        mark()
        lc.head_to_seq_relayout_batch([o_all, dq_all, dk_all, dv_all], P, outs=[o_tok, dq_tok, dk_tok, dv_tok])
        mark()
        return marks

    torch.cuda.synchronize()
    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    lc.trace_collect()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    all_marks = []
    lc.trace_enable(True)
    t0.record(stream)
    for _ in range(steps):
        all_marks.append(step(True))
    t1.record(stream)
    torch.cuda.synchronize()
    lc.trace_enable(False)
    tr = lc.trace_collect()
    ms_step = t0.elapsed_time(t1) / steps
    per = {n: sum(m[i].elapsed_time(m[i + 1]) for m in all_marks) / steps for i, n in enumerate(names)}
    f_fwd = fwd_flops(1, hq, N, D)
    f_ring = sum(pair_flops_block(hq, D, N, a, a + blk) for a in range(0, N, blk))
    f_bwd = 2.5 * f_fwd
    rel_in = 2 * 2 * sum(xs[n].numel() for n in ("q", "k", "v", "do"))
    rel_out = 2 * 2 * (o_all.numel() + dq_all.numel() + dk_all.numel() + dv_all.numel())
    merge_bytes = o_parts.numel() * 4 + lse_parts.numel() * 4 + o_ring.numel() * 2 + lse_ring.numel() * 4

    def ph(ms, f=None, b=None):
        if f is not None:
            return {"ms": round(ms, 4), "TFLOP/s": round(tflops(f, ms), 2),
                    "frac_peak": round(tflops(f, ms) / PEAK_BF16_TFLOPS, 4)}
        return {"ms": round(ms, 4), "GB/s": round(gbps(b, ms), 1), "frac_peak": round(gbps(b, ms) / PEAK_HBM_GBPS, 4)}
    res = {"workload": w.name, "P": P, "N": N, "shard_heads_q": hq, "shard_heads_kv": hkv, "D": D,
           "step": "relayout q,k,v,dO -> fwd -> 4 partial fwd + merge -> bwd -> relayout o,dq,dk,dv",
           "dq_path": "product of the stored dS" if stored else "recomputing dQ pass",
           "ms_per_step": round(ms_step, 4),
           "attention_TFLOP/s": round(tflops(f_fwd + f_ring + f_bwd, ms_step), 2),
           "phases": {"relayout_seq_to_head_qkvdo": ph(per["relayout_in"], b=rel_in),
                      "fwd": ph(per["fwd"], f=f_fwd), "ring_partials_x4": ph(per["ring_partials"], f=f_ring),
                      "merge": ph(per["merge"], b=merge_bytes), "bwd": ph(per["bwd"], f=f_bwd),
                      "relayout_head_to_seq_o_grads": ph(per["relayout_out"], b=rel_out)}}
    rls = {f"{w.name}.relayout": roofline_entry("transpose_rows_kernel", tr, (rel_in + rel_out) / 2, "GB/s", w.name),
           f"{w.name}.attn_fwd": roofline_entry("attn_fwd_kernel", tr, f_fwd, "TFLOP/s", w.name),
           f"{w.name}.ring_partials": roofline_entry("attn_fwd_kernel_fp32out", tr, f_ring, "TFLOP/s", w.name),
           f"{w.name}.merge": roofline_entry("merge_kernel", tr, merge_bytes, "GB/s", w.name),
           f"{w.name}.bwd_dkdv_kernel": roofline_entry("bwd_dkdv_kernel", tr, 0.8 * f_bwd, "TFLOP/s", w.name)}
    if stored:
        rls[f"{w.name}.bwd_dq_ds_kernel"] = roofline_entry("bwd_dq_ds_kernel", tr, ds_pass_bytes(1, hq, hkv, N, D),
                                                           "GB/s", w.name)
    else:
        rls[f"{w.name}.bwd_dq_kernel"] = roofline_entry("bwd_dq_kernel", tr, 0.2 * f_bwd, "TFLOP/s", w.name)
    if extras:
        res.update(shard_extras(lc, torch, dev, w, xs, heads, o, dq, dk, dv, lse, o_parts, lse_parts, o_ring, ws,
                                f_fwd, f_ring, f_bwd))
    return res, rls


def shard_extras(lc, torch, dev, w, xs, heads, o, dq, dk, dv, lse, o_parts, lse_parts, o_ring, ws, f_fwd, f_ring,
                 f_bwd):
    """Variants of the shard's attention: read token-major without a relayout
    (forward and backward), the ring streamed into one running result, the
    ring's backward, and ring sharding over 4 ranks."""
    P, N, D, Hq, Hkv = w.P, w.N, w.D, w.Hq, w.Hkv
    hq, hkv = Hq // P, Hkv // P
    scale = w.scale
    blk = N // 4
    out = {}

    def r(ms, f):
        return {"ms": round(ms, 4), "TFLOP/s": round(tflops(f, ms), 2),
                "frac_peak": round(tflops(f, ms) / PEAK_BF16_TFLOPS, 4)}
    qv = xs["q"].view(N, Hq, D)[:, :hq].permute(1, 0, 2).unsqueeze(0)
    kv_ = xs["k"].view(N, Hkv, D)[:, :hkv].permute(1, 0, 2).unsqueeze(0)
    vv = xs["v"].view(N, Hkv, D)[:, :hkv].permute(1, 0, 2).unsqueeze(0)
    o_tm = torch.empty((1, hq, N, D), dtype=torch.bfloat16, device=dev)
    ms = time_calls(torch, lambda: lc.attn_fwd_strided(qv, kv_, vv, causal=True, scale=scale, o=o_tm, lse=lse))
    out["token_major_forward"] = {"call": "attn_fwd_strided on shard 0's heads of the token-major input", **r(ms, f_fwd)}

    def tm_heads(x, H, n):
        return x.view(N, H, D)[:, :n].permute(1, 0, 2).unsqueeze(0)
    o_tmb = torch.empty((N, Hq, D), dtype=torch.bfloat16, device=dev)
    g_tm = [torch.empty((N, H, D), dtype=torch.bfloat16, device=dev) for H in (Hq, Hkv, Hkv)]
    ov = tm_heads(o_tmb, Hq, hq)
    lc.attn_fwd_strided(qv, kv_, vv, causal=True, scale=scale, o=ov, lse=lse)
    dov = tm_heads(xs["do"], Hq, hq)
    gq, gk, gv = tm_heads(g_tm[0], Hq, hq), tm_heads(g_tm[1], Hkv, hkv), tm_heads(g_tm[2], Hkv, hkv)
    ms = time_calls(torch, lambda: lc.attn_bwd_strided(qv, kv_, vv, ov, dov, lse, causal=True, scale=scale,
                                                       workspace=ws, dq=gq, dk=gk, dv=gv))
    out["token_major_backward"] = {"call": "attn_bwd_strided on shard 0's heads of token-major Q, K, V, O, dO",
                                   **r(ms, f_bwd)}
    del o_tmb, g_tm
    o_acc = o_parts[0]
    q0, k0, v0, do0 = (heads[n][0:1] for n in ("q", "k", "v", "do"))

    def streamed():
        for i, a in enumerate(range(0, N, blk)):
            lc.attn_fwd_accumulate(q0, k0[:, :, a:a + blk], v0[:, :, a:a + blk], o_acc, lse_parts[0],
                                   first=(i == 0), causal=True, scale=scale, k_pos0=a,
                                   o_final=o_ring if a + blk >= N else None)
    out["ring_streamed"] = {"call": "4 x attn_fwd_accumulate (running fp32 O, LSE; bf16 O from the last)",
                            **r(time_calls(torch, streamed), f_ring)}
    lc.attn_fwd(q0, k0, v0, causal=True, scale=scale, o=o, lse=lse)
    dq_acc = o_parts[1]
    delta = torch.empty_like(lse)
    ws_min = torch.empty(max(16, lc.attn_bwd_block_workspace_size(1, hq, hkv, blk, D)), dtype=torch.uint8,
                         device=dev)
    big = lc.attn_bwd_block_ds_workspace_size(1, hq, hkv, N, blk, D)
    ws_ds = torch.empty(big, dtype=torch.uint8, device=dev) if 0 < big <= lc.STORED_DS_AUTO_BYTES else None

    def ring_backward(ws_blk):
        lc.attn_bwd_delta(o, do0, delta=delta)
        for i, a in enumerate(range(0, N, blk)):
            lc.attn_bwd_block(q0, k0[:, :, a:a + blk], v0[:, :, a:a + blk], do0, lse, delta, causal=True,
                              scale=scale, k_pos0=a, dq_acc=dq_acc, dq_accumulate=i > 0,
                              dq=dq if a + blk >= N else None, dk=dk[:, :, a:a + blk], dv=dv[:, :, a:a + blk],
                              workspace=ws_blk)
    out["ring_backward"] = {"call": "attn_bwd_delta + 4 x attn_bwd_block (fp32 dQ accumulated)",
                            "dq_path": "product of the stored dS" if ws_ds is not None else "recomputing dQ pass",
                            **r(time_calls(torch, lambda: ring_backward(ws_ds if ws_ds is not None else ws_min)),
                                2.5 * f_ring)}
    if ws_ds is not None:
        out["ring_backward_recomputing_dq"] = {"call": "the same with the minimal workspace",
                                               **r(time_calls(torch, lambda: ring_backward(ws_min)), 2.5 * f_ring)}
        del ws_ds
    out["ring_sharding"] = ring_sharding(lc, torch, dev, heads, hq, N, D, scale, f_fwd, o, lse)
    return out


def ring_sharding(lc, torch, dev, heads, hq, N, D, scale, f_fwd, o_full, lse_full, Pr=4):
    """Shard 0's causal attention as a Pr-rank ring over 2*Pr chunks, every
    rank's every step timed on this GPU: the ring waits for the slowest rank
    at each step, so its critical path is the sum over steps of the maximum
    over ranks.  Contiguous sharding against zigzag (rank r holds chunks r
    and 2*Pr-1-r); forward, then backward (from the full forward's O and
    LSE), each one call at a time and with a step's independent calls in one
    launch."""
    from long_context_attention_fwd_amd.ring import SCHEMES, rank_chunks, ring_backward, ring_forward
    C = N // (2 * Pr)
    q0, k0, v0 = (heads[n][0:1] for n in ("q", "k", "v"))
    cq = [q0[:, :, c * C:(c + 1) * C].contiguous() for c in range(2 * Pr)]
    ck = [k0[:, :, c * C:(c + 1) * C].contiguous() for c in range(2 * Pr)]
    cv = [v0[:, :, c * C:(c + 1) * C].contiguous() for c in range(2 * Pr)]
    o_acc = [torch.empty((1, hq, C, D), dtype=torch.float32, device=dev) for _ in range(2)]
    lse = [torch.empty((1, hq, C), dtype=torch.float32, device=dev) for _ in range(2)]
    o_fin = [torch.empty((1, hq, C, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    hkv = ck[0].shape[1]
    n_split = lc.attn_fwd_split_suggest(1, hq, hkv, C, C, True, 2)
    fws = [torch.empty(max(16, lc.attn_fwd_accumulate_workspace_size(1, hq, C, D, n_split)), dtype=torch.uint8,
                       device=dev) for _ in range(4)]
    res = {"ranks": Pr, "chunk_tokens": C,
           "call": "attn_fwd_accumulate per visible (query chunk, key chunk) pair, in sequence; _grouped: a step's "
                   "independent calls in one launch; _grouped_split: that launch with each call's keys in "
                   f"{n_split} ranges (attn_fwd_accumulate_group_split) and a merge per call"}
    for scheme, grouped, split in [(sc, g, sp) for g, sp in ((False, 1), (True, 1), (True, n_split))
                                   for sc in SCHEMES]:
        t = [[0.0] * Pr for _ in range(Pr)]
        for r in range(Pr):
            qs = [cq[c] for c in rank_chunks(r, Pr, scheme)]

            def kv(src, scheme=scheme):
                return tuple((ck[c], cv[c]) for c in rank_chunks(src, Pr, scheme))
            for st in range(Pr):
                t[r][st] = time_calls(torch, lambda: ring_forward(qs, kv, r, Pr, C, o_acc=o_acc, lse_acc=lse,
                                                                  o_final=o_fin, scheme=scheme, scale=scale,
                                                                  steps={st}, grouped=grouped, n_splits=split,
                                                                  workspaces=fws))
        crit = sum(max(t[r][s] for r in range(Pr)) for s in range(Pr))
        res[scheme + ("_grouped" if grouped else "") + ("_split" if split > 1 else "")] = {
            "critical_path_ms": round(crit, 4), "ring_TFLOP/s": round(tflops(f_fwd, crit), 2),
            "per_rank_TFLOP/s": round(tflops(f_fwd, crit) / Pr, 2),
            "per_rank_ms": [round(sum(t[r]), 4) for r in range(Pr)],
            "per_step_max_ms": [round(max(t[r][s] for r in range(Pr)), 4) for s in range(Pr)]}
    # backward: Dv of the full forward, chunked like Q; fp32 dQ per query
    # chunk and dK, dV per key/value chunk (they travel with the chunk)
    do0 = heads["do"][0:1]
    delta = lc.attn_bwd_delta(o_full, do0)
    cdo = [do0[:, :, c * C:(c + 1) * C].contiguous() for c in range(2 * Pr)]
    clse = [lse_full[:, :, c * C:(c + 1) * C].contiguous() for c in range(2 * Pr)]
    cdl = [delta[:, :, c * C:(c + 1) * C].contiguous() for c in range(2 * Pr)]
    dq_acc = [torch.zeros((1, hq, C, D), dtype=torch.float32, device=dev) for _ in range(2 * Pr)]
    dkv_acc = [tuple(torch.zeros((1, ck[0].shape[1], C, D), dtype=torch.float32, device=dev) for _ in range(2))
               for _ in range(2 * Pr)]
    wsz = max(16, lc.attn_bwd_block_workspace_size(1, hq, ck[0].shape[1], C, D))
    wss = [torch.empty(wsz, dtype=torch.uint8, device=dev) for _ in range(4)]
    f_bwd = 2.5 * f_fwd
    res["backward_call"] = ("attn_bwd_block per visible (query chunk, key chunk) pair, or "
                            "attn_bwd_block_group per set of a step's pairs that share no chunk")
    for scheme, grouped in [(sc, g) for g in (False, True) for sc in SCHEMES]:
        t = [[0.0] * Pr for _ in range(Pr)]
        for r in range(Pr):
            mine = rank_chunks(r, Pr, scheme)

            def kv(src, scheme=scheme):
                return tuple((ck[c], cv[c]) for c in rank_chunks(src, Pr, scheme))

            def acc(src, ki, scheme=scheme):
                return dkv_acc[rank_chunks(src, Pr, scheme)[ki]]
            for st in range(Pr):
                t[r][st] = time_calls(torch, lambda: ring_backward(
                    [cq[c] for c in mine], [cdo[c] for c in mine], [clse[c] for c in mine],
                    [cdl[c] for c in mine], kv, r, Pr, C, dq_acc=[dq_acc[c] for c in mine], dkv_acc=acc,
                    scheme=scheme, scale=scale, steps={st}, grouped=grouped, workspaces=wss))
        crit = sum(max(t[r][s] for r in range(Pr)) for s in range(Pr))
        res["backward_" + scheme + ("_grouped" if grouped else "")] = {
            "critical_path_ms": round(crit, 4), "ring_TFLOP/s": round(tflops(f_bwd, crit), 2),
            "per_rank_TFLOP/s": round(tflops(f_bwd, crit) / Pr, 2),
            "per_rank_ms": [round(sum(t[r]), 4) for r in range(Pr)],
            "per_step_max_ms": [round(max(t[r][s] for r in range(Pr)), 4) for s in range(Pr)]}
    return res


# ---------------------------------------------------------------------------
# the oracle on the host cores
# ---------------------------------------------------------------------------
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _blas_config():
    import numpy as np
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')} ({b.get('openblas configuration', '').strip()})"
    except Exception:  # noqa: BLE001 -- reporting only
        return "unknown"


def _run_tasks(tasks, fn, workers):
    """fn over tasks in a thread pool, BLAS held to one thread per task (the
    tasks are independent query rows of the oracle's definition)."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        if workers == 1:
            return [fn(t) for t in tasks]
        with cf.ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, tasks))


def _chunks(rows, n):
    return [rows[i:i + n] for i in range(0, len(rows), n)]


def cpu_baseline():
    """The fp64 oracle as it stands (oracle/attention.py, untuned) on the host
    cores, per workload, on the work the parity tests give it: the 4K shape in
    full (all threads, and one thread), 256 sampled query rows of every head
    for the 32K shard, the 32K ring (partials + merge) and the 512K share, and
    for the 64K training shape the full fp64 forward (LSE and Dv of every row)
    plus the gradients at 128 sampled rows.  Independent query rows run in a
    thread pool with BLAS held to one thread per task.  Rates are algorithmic
    flops (as on the GPU) per second; full-workload times at those rates are
    extrapolations and labelled so."""
    import numpy as np

    import oracle
    from long_context_attention_fwd_amd.inputs import WORKLOADS, sample_rows

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    per = {}

    def f64(bits):
        return oracle.bf16_bits_to_f64(bits)

    def rows_flops(rows, nh, D):  # forward flops of causal rows (all keys up to the row)
        return 4.0 * nh * D * float((np.asarray(rows) + 1).sum())

    def fwd_rows(q, k, v, s, G, k_pos0=0):
        def run(t):
            h, rows = t
            return oracle.attention_forward(q[:, h:h + 1], k[:, h // G:h // G + 1], v[:, h // G:h // G + 1], s, True,
                                            0, k_pos0, rows=rows)
        return run

    # listing_4k: every row and head, all threads and one thread
    w = WORKLOADS["listing_4k"]
    d = host_inputs(w.name)
    q, k, v = (f64(d[n]) for n in "qkv")
    G = w.Hq // w.Hkv
    tasks = [(h, r) for h in range(w.Hq) for r in _chunks(np.arange(w.N)[::-1].copy(), 256)]
    f = fwd_flops(1, w.Hq, w.N, w.D)
    for n_thr in (workers, 1):
        t0 = time.perf_counter()
        _run_tasks(tasks, fwd_rows(q, k, v, w.scale, G), n_thr)
        dt = time.perf_counter() - t0
        per[f"{w.name}" + ("" if n_thr > 1 else "_1thread")] = {
            "work": "fp64 forward, every row and head", "threads": n_thr, "seconds": round(dt, 3),
            "GFLOP/s": round(f / dt / 1e9, 2), "algorithmic_flops": f}

    # ulysses_shard_32k: 256 sampled rows x 4 heads of shard 0 (the oracle's own relayout)
    w = WORKLOADS["ulysses_shard_32k"]
    d = host_inputs(w.name)
    ref = {n: f64(oracle.seq_to_head(d[n], w.P)[0:1]) for n in "qkv"}
    hq = w.Hq // w.P
    rows = sample_rows(w.N, w.seed, w.sampled_rows)
    tasks = [(h, r) for h in range(hq) for r in _chunks(rows[::-1].copy(), 16)]
    t0 = time.perf_counter()
    _run_tasks(tasks, fwd_rows(ref["q"], ref["k"], ref["v"], w.scale, hq), workers)
    dt = time.perf_counter() - t0
    fs = rows_flops(rows, hq, w.D)
    full = fwd_flops(1, hq, w.N, w.D)
    per[w.name] = {"work": f"fp64 forward, {len(rows)} sampled rows x {hq} heads of shard 0", "threads": workers,
                   "seconds": round(dt, 3), "GFLOP/s": round(fs / dt / 1e9, 2), "algorithmic_flops": fs,
                   "extrapolated_full_forward_s": round(full / (fs / dt), 1)}

    # ring_blocks_32k: 256 sampled rows x 8 heads, four 8192-key partials + merge
    w = WORKLOADS["ring_blocks_32k"]
    d = host_inputs(w.name)
    q, k, v = (f64(d[n]) for n in "qkv")
    blk = w.N // w.kv_blocks
    rows = sample_rows(w.N, w.seed, w.sampled_rows, block=blk)

    def ring_rows(t):
        h, rr = t
        parts = [oracle.attention_forward(q[:, h:h + 1], k[:, h:h + 1, a:a + blk], v[:, h:h + 1, a:a + blk], w.scale,
                                          True, 0, a, rows=rr) for a in range(0, w.N, blk)]
        return oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    tasks = [(h, r) for h in range(w.Hq) for r in _chunks(rows[::-1].copy(), 16)]
    t0 = time.perf_counter()
    _run_tasks(tasks, ring_rows, workers)
    dt = time.perf_counter() - t0
    fs = rows_flops(rows, w.Hq, w.D)
    full = fwd_flops(1, w.Hq, w.N, w.D)
    per[w.name] = {"work": f"fp64 partials over 4 key blocks + LSE merge, {len(rows)} sampled rows x {w.Hq} heads",
                   "threads": workers, "seconds": round(dt, 3), "GFLOP/s": round(fs / dt / 1e9, 2),
                   "algorithmic_flops": fs, "extrapolated_full_partials_s": round(full / (fs / dt), 1)}
    del q, k, v

    # ulysses_512k: 256 sampled rows x 4 heads
    w = WORKLOADS["ulysses_512k"]
    d = host_inputs(w.name)
    q, k, v = (f64(d[n]) for n in "qkv")
    rows = sample_rows(w.N, w.seed, w.sampled_rows)
    tasks = [(h, r) for h in range(w.Hq) for r in _chunks(rows[::-1].copy(), 8)]
    t0 = time.perf_counter()
    _run_tasks(tasks, fwd_rows(q, k, v, w.scale, w.Hq // w.Hkv), workers)
    dt = time.perf_counter() - t0
    fs = rows_flops(rows, w.Hq, w.D)
    full = fwd_flops(1, w.Hq, w.N, w.D)
    per[w.name] = {"work": f"fp64 forward, {len(rows)} sampled rows x {w.Hq} heads", "threads": workers,
                   "seconds": round(dt, 3), "GFLOP/s": round(fs / dt / 1e9, 2), "algorithmic_flops": fs,
                   "extrapolated_full_forward_s": round(full / (fs / dt), 1)}
    del q, k, v

    # train_64k: full fp64 forward (LSE, Dv of every row) + gradients at 128 sampled rows
    w = WORKLOADS["train_64k"]
    d = host_inputs(w.name)
    q, k, v, do = (f64(d[n]) for n in ("q", "k", "v", "do"))
    rows = sample_rows(w.N, w.seed, w.sampled_rows)
    L = np.empty((1, w.Hq, w.N))
    Dv = np.empty((1, w.Hq, w.N))

    def fwd_task(t):
        h, rr = t
        O, l = oracle.attention_forward(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], w.scale, True, rows=rr)
        L[0, h, rr] = l[0, 0]
        Dv[0, h, rr] = np.einsum("nd,nd->n", do[0, h, rr], O[0, 0])
    tasks = [(h, np.arange(r0, min(w.N, r0 + 2048))) for r0 in range(w.N - 2048, -1, -2048) for h in range(w.Hq)]
    t0 = time.perf_counter()
    _run_tasks(tasks, fwd_task, workers)

    def grad_task(h):
        return oracle.attention_backward_sampled(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], do[:, h:h + 1],
                                                 w.scale, rows, rows, True, lse=L[:, h:h + 1], dv=Dv[:, h:h + 1])
    _run_tasks(list(range(w.Hq)), grad_task, workers)
    dt = time.perf_counter() - t0
    f_fwd = fwd_flops(1, w.Hq, w.N, w.D)
    # gradients: dQ rows need S, dP, dQ (6 D flops per visible pair), dK/dV
    # rows S, dP, dK, dV (8 D per pair)
    f_grad = w.Hq * w.D * (6.0 * float((rows + 1).sum()) + 8.0 * float((w.N - rows).sum()))
    fs = f_fwd + f_grad
    per[w.name] = {"work": f"fp64 forward of every row x {w.Hq} heads (LSE, Dv) + dQ, dK, dV at {len(rows)} "
                           "sampled rows", "threads": workers, "seconds": round(dt, 3),
                   "GFLOP/s": round(fs / dt / 1e9, 2), "algorithmic_flops": fs,
                   "extrapolated_full_fwd_bwd_s": round(3.5 * f_fwd / (fs / dt), 1)}
    del q, k, v, do
    head = per["train_64k"]
    return {"value": round(head["GFLOP/s"] / 1e3, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"train_64k: {head['work']}; {head['seconds']} s (the headline workload; "
                      f"{head['extrapolated_full_fwd_bwd_s']} s extrapolated for its full forward + backward)",
            "cpu_model": _cpu_model(), "blas": _blas_config(), "per_workload": per,
            "seconds_total": round(sum(p["seconds"] for p in per.values()), 2)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share only: the library runs no collectives, so --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_attention_fwd_amd as lc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    device_info = {"name": props.name, "compute_units": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", None), "hip": torch.version.hip}

    if args.only and args.calibration_copy:
        # a plain streaming kernel of known bytes, not one of the library's:
        # its FETCH_SIZE / WRITE_SIZE calibrate the counters of the same run
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.mul(a, 2.0, out=b)
        torch.cuda.synchronize()
        del a, b
    if args.only and args.only != "train_64k":
        legs = {"listing_4k": lambda: leg_listing_4k(lc, torch, dev),
                "ulysses_shard_32k": lambda: leg_ulysses_shard_32k(lc, torch, dev, args.steps, args.warmup, False),
                "ulysses_shard_32k_extras": lambda: leg_ulysses_shard_32k(lc, torch, dev, args.steps, args.warmup,
                                                                          True),
                "ring_blocks_32k": lambda: leg_ring_blocks_32k(lc, torch, dev, args.steps, args.warmup),
                "ulysses_512k": lambda: leg_ulysses_512k(lc, torch, dev, args.steps, args.warmup)}
        res, rls = legs[args.only]()
        print(json.dumps({"only": args.only, "result": res, "rooflines": rls, "device_info": device_info}),
              flush=True)
        return

    head = train_64k(lc, torch, dev, args.steps, args.warmup)
    out = {
        "metric": "causal attention TFLOP/s fwd/bwd at 1 GPU + % bf16 MFMA peak; relayout GB/s",
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) bf16 (numpy PCG64), no dataset or weights",
        "config": head["config"],
        "phases": head["phases"],
        "gpu_kernels": head["gpu_kernels"],
        "roofline": head["roofline"],
        "rooflines": dict(head["rooflines"]),
        "device_info": device_info,
    }
    if args.only is None:
        legs = {}
        for name, fn in (("listing_4k", lambda: leg_listing_4k(lc, torch, dev)),
                         ("ulysses_shard_32k", lambda: leg_ulysses_shard_32k(lc, torch, dev, 10, 2,
                                                                             not args.no_extras)),
                         ("ring_blocks_32k", lambda: leg_ring_blocks_32k(lc, torch, dev)),
                         ("ulysses_512k", lambda: leg_ulysses_512k(lc, torch, dev))):
            res, rls = fn()
            legs[name] = res
            out["rooflines"].update(rls)
            torch.cuda.synchronize()
        out["legs"] = legs
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
