#!/usr/bin/env python3
"""Benchmark of the long-context causal attention hot path on one MI355X.

One step is one pass over the whole hot path on one GPU's Ulysses share of a
Llama-3-8B-shaped layer (32 query / 8 key-value heads, D = 128, N = 32768
tokens split P = 8 ways), with inputs already resident in HBM:

  1. seq_to_head_relayout_batch of Q, K, V, dO (all P shards, one launch)
     -- the all-to-all's data movement
  2. attn_fwd on shard 0 (4 query heads, 1 KV head, causal GQA, N = 32768)
  3. the ring form of the same forward: 4 partial attention calls over
     8192-key blocks (fp32 partials, one attn_fwd_accumulate_group launch)
     + attn_partial_merge
  4. attn_bwd on shard 0 (from step 2's O and LSE)
  5. head_to_seq_relayout_batch of O, dQ, dK, dV (one launch)

``value`` is the attention work of the step (forward + ring forward +
backward, algorithmic flops: masked pairs not counted) divided by the step
time.  The per-kernel breakdown, the roofline of the dominant kernel and the
oracle's CPU rate on a bounded sample of the same workload are printed in the
same JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBPS = 8000.0


def fwd_flops(B, Hq, N, D):
    """Causal forward: 4*D flops per visible (query, key) pair, N(N+1)/2 pairs."""
    return 2.0 * B * Hq * D * N * (N + 1)


def pair_flops_block(Hq, D, N, a, b):
    """Forward flops of queries 0..N-1 against keys [a, b) (causal, global
    positions): key j is seen by the N - j queries at or after it."""
    pairs = (b - a) * N - (b * (b - 1) // 2 - a * (a - 1) // 2)
    return 4.0 * Hq * D * pairs


def kernel_source_digest(name):
    """sha256 of the sources a kernel is compiled from (to tell whether
    committed counter figures still describe it)."""
    csrc = os.path.join(ROOT, "long_context_attention_fwd_amd", "csrc")
    files = {"bwd_dkdv_kernel": "attn_bwd.hip", "bwd_dq_kernel": "attn_bwd.hip", "attn_fwd_kernel": "attn_fwd.hip",
             "attn_fwd_kernel_fp32out": "attn_fwd.hip",
             "transpose_rows_kernel": "relayout.hip", "merge_kernel": "merge.hip"}.get(name)
    if files is None:
        return None
    h = hashlib.sha256()
    for f in (files, "device_common.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a copy of known size), or None when
    there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
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


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    p.add_argument("--profile-steps", action="store_true", help="short run for rocprofv3 (no CPU leg)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share only: this build runs no collectives, so --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_context_attention_fwd_amd as lc
    from long_context_attention_fwd_amd.inputs import WORKLOADS, make_workload_inputs, normal_bf16

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = WORKLOADS["ulysses_shard_32k"]
    P, N, D, Hq, Hkv = w.P, w.N, w.D, w.Hq, w.Hkv
    hq, hkv = Hq // P, Hkv // P  # one shard's heads: 4 and 1

    # ---- inputs, resident in HBM before timing ------------------------------
    d = make_workload_inputs(w)
    rng = np.random.default_rng(w.seed + 17)
    d["do"] = normal_bf16(rng, (P, N // P, Hq, D))

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    xs = {k: dev_bf16(v) for k, v in d.items()}
    del d
    heads = {"q": torch.empty((P, hq, N, D), dtype=torch.bfloat16, device=dev),
             "do": torch.empty((P, hq, N, D), dtype=torch.bfloat16, device=dev),
             "k": torch.empty((P, hkv, N, D), dtype=torch.bfloat16, device=dev),
             "v": torch.empty((P, hkv, N, D), dtype=torch.bfloat16, device=dev)}
    # token-major outputs of the inverse relayout.  Shard 0's results are
    # written straight into slot 0 of the head-major buffers; the inverse
    # relayout moves all P shards' bytes, as the exchange would.
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
    ws = torch.empty(lc.attn_bwd_workspace_size(1, hq, hkv, N, D), dtype=torch.uint8, device=dev)
    scale = w.scale
    stream = torch.cuda.current_stream(dev)
    # the key/value blocks of the ring (views of shard 0's head-major K, V:
    # contiguous, as a ring step receives them, since a shard has one KV head)
    ring_blocks = [(a, heads["k"][0:1, :, a:a + blk], heads["v"][0:1, :, a:a + blk]) for a in range(0, N, blk)]
    assert all(kb.is_contiguous() and vb.is_contiguous() for _, kb, vb in ring_blocks)

    names = ["relayout_in", "fwd", "ring_partials", "merge", "bwd", "relayout_out"]
    ev = {n: [] for n in names}

    def step(record):
        marks = []

        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                marks.append(e)

        mark()
        # one launch for the four tensors of the exchange
        lc.seq_to_head_relayout_batch([xs[n] for n in ("q", "k", "v", "do")], P,
                                      outs=[heads[n] for n in ("q", "k", "v", "do")])
        mark()
        q0, k0, v0, do0 = (heads[n][0:1] for n in ("q", "k", "v", "do"))
        lc.attn_fwd(q0, k0, v0, causal=True, scale=scale, o=o, lse=lse)
        mark()
        # The ring's partials, one per KV block [a, a + blk), fp32 O and LSE
        # each.  All blocks are resident on this GPU and the partials are
        # independent, so the four calls go out as one grouped launch (a late
        # block has work only for the last queries and alone would leave most
        # CUs idle); the merge follows.
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

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    all_marks = []
    torch.cuda.synchronize()
    lc.trace_collect()          # drop records of the warmup
    lc.trace_enable(True)       # every library kernel bracketed by HIP events
    t_start.record(stream)
    for _ in range(args.steps):
        all_marks.append(step(True))
    t_end.record(stream)
    torch.cuda.synchronize()
    lc.trace_enable(False)
    traced = lc.trace_collect()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    per = {n: 0.0 for n in names}
    for marks in all_marks:
        for i, n in enumerate(names):
            per[n] += marks[i].elapsed_time(marks[i + 1])
    per = {n: v / args.steps for n, v in per.items()}

    B = 1
    f_fwd = fwd_flops(B, hq, N, D)
    f_ring = sum(pair_flops_block(hq, D, N, a, a + blk) for a in range(0, N, blk))
    f_bwd = 2.5 * f_fwd
    attn_flops = f_fwd + f_ring + f_bwd
    relayout_in_bytes = 2 * 2 * (xs["q"].numel() + xs["k"].numel() + xs["v"].numel() + xs["do"].numel())
    relayout_out_bytes = 2 * 2 * (o_all.numel() + dq_all.numel() + dk_all.numel() + dv_all.numel())
    merge_bytes = o_parts.numel() * 4 + lse_parts.numel() * 4 + o_ring.numel() * 2 + lse_ring.numel() * 4

    def tflops(f, ms):
        return f / (ms * 1e-3) / 1e12

    def gbps(b, ms):
        return b / (ms * 1e-3) / 1e9

    kernels = {
        "fwd": {"ms": per["fwd"], "TFLOP/s": tflops(f_fwd, per["fwd"]),
                "frac_peak": tflops(f_fwd, per["fwd"]) / PEAK_BF16_TFLOPS},
        "ring_partials_x4": {"ms": per["ring_partials"], "TFLOP/s": tflops(f_ring, per["ring_partials"]),
                             "frac_peak": tflops(f_ring, per["ring_partials"]) / PEAK_BF16_TFLOPS},
        "merge": {"ms": per["merge"], "GB/s": gbps(merge_bytes, per["merge"]),
                  "frac_peak": gbps(merge_bytes, per["merge"]) / PEAK_HBM_GBPS},
        "bwd": {"ms": per["bwd"], "TFLOP/s": tflops(f_bwd, per["bwd"]),
                "frac_peak": tflops(f_bwd, per["bwd"]) / PEAK_BF16_TFLOPS},
        "relayout_seq_to_head_qkvdo": {"ms": per["relayout_in"], "GB/s": gbps(relayout_in_bytes, per["relayout_in"]),
                                       "frac_peak": gbps(relayout_in_bytes, per["relayout_in"]) / PEAK_HBM_GBPS},
        "relayout_head_to_seq_o_grads": {"ms": per["relayout_out"],
                                         "GB/s": gbps(relayout_out_bytes, per["relayout_out"]),
                                         "frac_peak": gbps(relayout_out_bytes, per["relayout_out"]) / PEAK_HBM_GBPS},
    }
    # Per GPU kernel, from the library's HIP events over the timed region:
    # algorithmic work of all its launches / its total time.  The backward's
    # five counted contractions are S, dP, dV, dK (dK/dV kernel) and dQ (dQ
    # kernel); the dQ kernel's recomputed S and dP are not counted.
    # kernels whose launches share the GPU with one another (none since the
    # ring partials became one grouped launch)
    OVERLAPPED = set()
    alg = {
        "attn_fwd_kernel": ("TFLOP/s", args.steps * f_fwd),
        # the ring partials: one grouped launch of four fp32-output calls
        "attn_fwd_kernel_fp32out": ("TFLOP/s", args.steps * f_ring),
        "bwd_dkdv_kernel": ("TFLOP/s", args.steps * 0.8 * f_bwd),
        "bwd_dq_kernel": ("TFLOP/s", args.steps * 0.2 * f_bwd),
        "transpose_rows_kernel": ("GB/s", args.steps * (relayout_in_bytes + relayout_out_bytes)),
        "merge_kernel": ("GB/s", args.steps * merge_bytes),
        "bwd_delta_kernel": ("GB/s", args.steps * 2 * 2 * o_ring.numel() + args.steps * 4 * lse.numel()),
        "bwd_dkdv_reduce_kernel": ("GB/s", args.steps * (2 * 4 * hq + 2 * 2 * hkv) * N * D),
    }
    gpu_kernels = {}
    for name, (tot_ms, calls) in traced.items():
        unit, work = alg.get(name, (None, None))
        ent = {"calls_per_step": calls / args.steps, "avg_us": round(1e3 * tot_ms / calls, 2),
               "share_of_step": round(tot_ms / total_ms, 4)}
        if unit == "TFLOP/s":
            ent["TFLOP/s"] = round(tflops(work, tot_ms), 2)
            ent["frac_peak"] = round(tflops(work, tot_ms) / PEAK_BF16_TFLOPS, 4)
        elif unit == "GB/s":
            ent["GB/s"] = round(gbps(work, tot_ms), 1)
            ent["frac_peak"] = round(gbps(work, tot_ms) / PEAK_HBM_GBPS, 4)
        if name in OVERLAPPED:
            ent["overlapped"] = True  # launches share the GPU: avg_us is not one launch's own time
        gpu_kernels[name] = ent
    # The dominant kernel is the one with the most time among kernels that run
    # alone, so that its launch duration is its own.
    dom = max((n for n in traced if n not in OVERLAPPED), key=lambda n: traced[n][0])
    tot_ms, calls = traced[dom]
    unit, work = alg[dom]
    mfma = unit == "TFLOP/s"
    achieved = tflops(work, tot_ms) if mfma else gbps(work, tot_ms)
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBPS
    roofline = {"bound": "mfma" if mfma else "hbm", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": None, "avg_launch_us": round(1e3 * tot_ms / calls, 2),
                "algorithmic_per_launch": work / calls}
    t = measured_traffic(dom)
    if t is not None:
        roofline["traffic"] = t["read_bytes"] + t["write_bytes"]
        roofline["traffic_detail"] = t

    out = {
        "metric": "causal attention TFLOP/s fwd/bwd at 1 GPU + % bf16 MFMA peak; relayout GB/s",
        "value": round(tflops(attn_flops, ms_step), 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) bf16 (numpy PCG64), no dataset or weights",
        "config": {"workload": w.name, "P": P, "N": N, "Hq_total": Hq, "Hkv_total": Hkv, "D": D,
                   "shard_heads_q": hq, "shard_heads_kv": hkv, "causal": True, "ring_blocks": n_blk,
                   "step": "relayout q,k,v,dO -> fwd -> 4 partial fwd + merge -> bwd -> relayout o,dq,dk,dv"},
        "phases": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in kernels.items()},
        "gpu_kernels": gpu_kernels,
        "roofline": roofline,
        "device": torch.cuda.get_device_name(dev),
    }
    props = torch.cuda.get_device_properties(dev)
    out["device_info"] = {"name": props.name, "compute_units": props.multi_processor_count,
                          "arch": getattr(props, "gcnArchName", None), "hip": torch.version.hip}
    if not args.profile_steps:
        out["short_sequence_forward"] = short_forward(lc, torch, dev)
        # shard 0's heads read straight from the token-major input, no relayout
        qv = xs["q"].view(N, Hq, D)[:, :hq].permute(1, 0, 2).unsqueeze(0)
        kv_ = xs["k"].view(N, Hkv, D)[:, :hkv].permute(1, 0, 2).unsqueeze(0)
        vv = xs["v"].view(N, Hkv, D)[:, :hkv].permute(1, 0, 2).unsqueeze(0)
        o_tm = torch.empty((1, hq, N, D), dtype=torch.bfloat16, device=dev)
        ms = time_calls(torch, lambda: lc.attn_fwd_strided(qv, kv_, vv, causal=True, scale=scale, o=o_tm, lse=lse))
        out["token_major_forward"] = {"call": "attn_fwd_strided on shard 0's heads of the token-major input",
                                      "ms": round(ms, 4), "TFLOP/s": round(tflops(f_fwd, ms), 2),
                                      "frac_peak": round(tflops(f_fwd, ms) / PEAK_BF16_TFLOPS, 4)}
        # its backward the same way: Q, K, V, O, dO read and dQ, dK, dV written token-major
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
                                       "ms": round(ms, 4), "TFLOP/s": round(tflops(f_bwd, ms), 2),
                                       "frac_peak": round(tflops(f_bwd, ms) / PEAK_BF16_TFLOPS, 4)}
        del o_tmb, g_tm
        # the ring streamed into one running result (blocks one after another)
        o_acc = o_parts[0]
        q0, k0, v0 = (heads[n][0:1] for n in ("q", "k", "v"))

        def streamed():
            for i, a in enumerate(range(0, N, blk)):
                lc.attn_fwd_accumulate(q0, k0[:, :, a:a + blk], v0[:, :, a:a + blk], o_acc, lse_parts[0],
                                       first=(i == 0), causal=True, scale=scale, k_pos0=a,
                                       o_final=o_ring if a + blk >= N else None)
        ms = time_calls(torch, streamed)
        out["ring_streamed"] = {"call": f"{n_blk} x attn_fwd_accumulate (running fp32 O, LSE; bf16 O from the last)",
                                "ms": round(ms, 4), "TFLOP/s": round(tflops(f_ring, ms), 2),
                                "frac_peak": round(tflops(f_ring, ms) / PEAK_BF16_TFLOPS, 4)}
        # the ring's backward: Dv once, then one attn_bwd_block per KV block
        # (fp32 dQ accumulated in place, bf16 dQ from the last; each block's
        # dK, dV in bf16), against the same global LSE
        dq_acc = o_parts[1]
        delta = torch.empty_like(lse)
        ws_blk = torch.empty(max(16, lc.attn_bwd_block_workspace_size(1, hq, hkv, blk, D)), dtype=torch.uint8,
                             device=dev)
        do0 = heads["do"][0:1]

        def ring_backward():
            lc.attn_bwd_delta(o, do0, delta=delta)
            for i, a in enumerate(range(0, N, blk)):
                lc.attn_bwd_block(q0, k0[:, :, a:a + blk], v0[:, :, a:a + blk], do0, lse, delta, causal=True,
                                  scale=scale, k_pos0=a, dq_acc=dq_acc, dq_accumulate=i > 0,
                                  dq=dq if a + blk >= N else None, dk=dk[:, :, a:a + blk], dv=dv[:, :, a:a + blk],
                                  workspace=ws_blk)
        ms = time_calls(torch, ring_backward)
        out["ring_backward"] = {"call": f"attn_bwd_delta + {n_blk} x attn_bwd_block (fp32 dQ accumulated)",
                                "ms": round(ms, 4), "TFLOP/s": round(tflops(2.5 * f_ring, ms), 2),
                                "frac_peak": round(tflops(2.5 * f_ring, ms) / PEAK_BF16_TFLOPS, 4)}
        out["ring_sharding"] = ring_sharding(lc, torch, dev, heads, hq, N, D, scale, f_fwd, tflops)
        out["long_shapes"] = long_shapes(lc, torch, dev)

    if not args.no_cpu_baseline and not args.profile_steps:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def ring_sharding(lc, torch, dev, heads, hq, N, D, scale, f_fwd, tflops, Pr=4):
    """Shard 0's causal attention as a Pr-rank ring over 2*Pr chunks, every
    rank's every step timed on this GPU: the ring waits for the slowest rank
    at each step, so its critical path is the sum over steps of the maximum
    over ranks.  Contiguous sharding against zigzag (rank r holds chunks r
    and 2*Pr-1-r)."""
    from long_context_attention_fwd_amd.ring import SCHEMES, rank_chunks, ring_forward
    C = N // (2 * Pr)
    q0, k0, v0 = (heads[n][0:1] for n in ("q", "k", "v"))
    cq = [q0[:, :, c * C:(c + 1) * C].contiguous() for c in range(2 * Pr)]
    ck = [k0[:, :, c * C:(c + 1) * C].contiguous() for c in range(2 * Pr)]
    cv = [v0[:, :, c * C:(c + 1) * C].contiguous() for c in range(2 * Pr)]
    o_acc = [torch.empty((1, hq, C, D), dtype=torch.float32, device=dev) for _ in range(2)]
    lse = [torch.empty((1, hq, C), dtype=torch.float32, device=dev) for _ in range(2)]
    o_fin = [torch.empty((1, hq, C, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    # one call after another: a chunk call fills a quarter of this GPU here,
    # so running the two chunks' calls side by side would measure launch
    # overlap rather than each rank's causal work
    res = {"ranks": Pr, "chunk_tokens": C,
           "call": "attn_fwd_accumulate per visible (query chunk, key chunk) pair, in sequence"}
    # "<scheme>_grouped": the calls of a step that read the same key/value
    # chunk (one per query chunk) as one attn_fwd_accumulate_group launch
    for scheme, grouped in [(sc, g) for g in (False, True) for sc in SCHEMES]:
        t = [[0.0] * Pr for _ in range(Pr)]
        for r in range(Pr):
            qs = [cq[c] for c in rank_chunks(r, Pr, scheme)]

            def kv(src, scheme=scheme):
                return tuple((ck[c], cv[c]) for c in rank_chunks(src, Pr, scheme))
            for st in range(Pr):
                t[r][st] = time_calls(torch, lambda: ring_forward(qs, kv, r, Pr, C, o_acc=o_acc, lse_acc=lse,
                                                                  o_final=o_fin, scheme=scheme, scale=scale,
                                                                  steps={st}, grouped=grouped))
        crit = sum(max(t[r][s] for r in range(Pr)) for s in range(Pr))
        # a real ring runs the ranks on Pr GPUs at once: aggregate over the
        # ranks, and per rank (one GPU)
        res[scheme + ("_grouped" if grouped else "")] = {
            "critical_path_ms": round(crit, 4), "ring_TFLOP/s": round(tflops(f_fwd, crit), 2),
            "per_rank_TFLOP/s": round(tflops(f_fwd, crit) / Pr, 2),
            "per_rank_ms": [round(sum(t[r]), 4) for r in range(Pr)],
            "per_step_max_ms": [round(max(t[r][s] for r in range(Pr)), 4) for s in range(Pr)]}
    return res


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


def short_forward(lc, torch, dev, iters=20):
    """The glossary example's forward shape ([1, 4, 4096, 64], causal), timed
    apart from the step: attn_fwd, and attn_fwd_splitkv with the library's
    choice of key ranges.  One workgroup per 256 query rows gives only 64
    workgroups here, so the longest row sets attn_fwd's time."""
    import numpy as np
    from long_context_attention_fwd_amd.inputs import WORKLOADS, make_workload_inputs
    w = WORKLOADS["listing_4k"]
    d = make_workload_inputs(w)
    q, k, v = (torch.from_numpy(d[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in "qkv")
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    ws = torch.empty(lc.attn_fwd_splitkv_workspace_size(B, Hq, Hkv, N, N, D, True, 0), dtype=torch.uint8,
                     device=dev)
    flops = fwd_flops(B, Hq, N, D)
    res = {"workload": w.name, "shape": [B, Hq, N, D], "causal": True}
    calls = {"attn_fwd": lambda: lc.attn_fwd(q, k, v, scale=w.scale, o=o, lse=lse),
             "attn_fwd_splitkv": lambda: lc.attn_fwd_splitkv(q, k, v, scale=w.scale, workspace=ws, o=o, lse=lse)}
    for name, fn in calls.items():
        ms = time_calls(torch, fn, iters, 5)
        res[name] = {"us": round(1e3 * ms, 2), "TFLOP/s": round(flops / ms / 1e9, 2),
                     "frac_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    return res


def long_shapes(lc, torch, dev):
    """The other two large workloads, timed apart from the step on inputs
    drawn on the GPU (seeded normal, bf16): the 64K training shape
    (8 heads, forward and backward) and the 512K-token forward of one
    Ulysses share (4 query heads on 1 key/value head, inputs 0.5 N(0,1))."""
    from long_context_attention_fwd_amd.inputs import WORKLOADS
    res = {}
    gen = torch.Generator(device=dev)

    def draw(shape, seed, amp=1.0):
        gen.manual_seed(seed)
        return (amp * torch.randn(shape, generator=gen, device=dev)).to(torch.bfloat16)

    w = WORKLOADS["train_64k"]
    q, k, v, do = (draw((w.B, h, w.N, w.D), w.seed * 10 + i) for i, h in enumerate((w.Hq, w.Hkv, w.Hkv, w.Hq)))
    o, lse = lc.attn_fwd(q, k, v, scale=w.scale)
    ws = torch.empty(lc.attn_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.D), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    f = fwd_flops(w.B, w.Hq, w.N, w.D)
    t_f = time_calls(torch, lambda: lc.attn_fwd(q, k, v, scale=w.scale, o=o, lse=lse), 3, 1)
    t_b = time_calls(torch, lambda: lc.attn_bwd(q, k, v, o, do, lse, scale=w.scale, workspace=ws, dq=dq, dk=dk,
                                                dv=dv), 3, 1)
    res[w.name] = {"shape": [w.B, w.Hq, w.N, w.D], "fwd_ms": round(t_f, 3), "fwd_TFLOP/s": round(f / t_f / 1e9, 1),
                   "bwd_ms": round(t_b, 3), "bwd_TFLOP/s": round(2.5 * f / t_b / 1e9, 1),
                   "bwd_frac_peak": round(2.5 * f / t_b / 1e9 / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, do, o, lse, ws, dq, dk, dv
    w = WORKLOADS["ulysses_512k"]
    q = draw((w.B, w.Hq, w.N, w.D), w.seed * 10, w.amp)
    k = draw((w.B, w.Hkv, w.N, w.D), w.seed * 10 + 1, w.amp)
    v = draw((w.B, w.Hkv, w.N, w.D), w.seed * 10 + 2, w.amp)
    o, lse = lc.attn_fwd(q, k, v, scale=w.scale)
    f = fwd_flops(w.B, w.Hq, w.N, w.D)
    t_f = time_calls(torch, lambda: lc.attn_fwd(q, k, v, scale=w.scale, o=o, lse=lse), 2, 1)
    res[w.name] = {"shape": [w.B, w.Hq, w.N, w.D], "kv_heads": w.Hkv, "fwd_ms": round(t_f, 2),
                   "fwd_TFLOP/s": round(f / t_f / 1e9, 1), "fwd_frac_peak": round(f / t_f / 1e9 / PEAK_BF16_TFLOPS, 4)}
    return res


def cpu_baseline(w, budget_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same shard:
    forward attention of the last rows of shard 0 (4 query heads, 1 KV head),
    in chunks of 256 rows until the time budget is spent."""
    import numpy as np

    import oracle
    from long_context_attention_fwd_amd.inputs import make_workload_inputs

    d = make_workload_inputs(w)
    ref = {n: oracle.seq_to_head(d[n], w.P)[0:1] for n in "qkv"}
    N, D, hq = w.N, w.D, w.Hq // w.P
    done_rows, flops, t_used = 0, 0.0, 0.0
    end = N
    while t_used < budget_s and end > 0:
        rows = np.arange(max(0, end - 256), end)
        t0 = time.perf_counter()
        oracle.attention_forward(ref["q"], ref["k"], ref["v"], w.scale, True, rows=rows)
        t_used += time.perf_counter() - t0
        flops += 4.0 * hq * D * float((rows + 1).sum())
        done_rows += len(rows)
        end -= 256
    cores = len(os.sched_getaffinity(0))
    return {"value": round(flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 forward of the last {done_rows} query rows x {hq} heads of shard 0 "
                      f"(N={N}, D={D}); {t_used:.1f} s of CPU work",
            "seconds": round(t_used, 2)}


if __name__ == "__main__":
    main()
