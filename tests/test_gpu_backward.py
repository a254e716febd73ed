"""GPU parity of attn_bwd against the fp64 oracle (through the C ABI).

Gradient gate: per tensor, max |dX_gpu - dX_ref| / max |dX_ref| <= 2e-2 over
the checked rows.  The forward's O and LSE that the GPU backward consumes come
from the GPU forward, as in training; the oracle computes its own.
"""

import math

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import WORKLOADS, make_qkv, make_workload_inputs, sample_rows

from gpu_util import GRAD_REL_TOL, check_forward, f64_of, grad_rel_err, poisoned, to_dev

pytestmark = pytest.mark.gpu


def sdpa_scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def gpu_fwd_bwd(q, k, v, do, scale, causal=True):
    import torch
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=scale)
    dq = poisoned(tuple(q.shape), torch.bfloat16)
    dk = poisoned(tuple(k.shape), torch.bfloat16)
    dv = poisoned(tuple(v.shape), torch.bfloat16)
    lc.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def check_grads(got, ref, what):
    errs = {n: grad_rel_err(f64_of(g), r) for n, g, r in zip(("dq", "dk", "dv"), got, ref)}
    for n, e in errs.items():
        assert np.isfinite(f64_of(got[("dq", "dk", "dv").index(n)])).all(), f"{what}: non-finite {n}"
        assert e <= GRAD_REL_TOL, f"{what}: {n} relative error {e} ({errs})"
    return errs


@pytest.mark.parametrize("N", [1, 63, 64, 65, 127, 128, 129, 257, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,causal", [(1, True), (2, True), (4, True), (2, False)])
def test_bwd_small_sweep(gpu, N, D, G, causal):
    Hkv = 2
    d = make_qkv(1, Hkv * G, Hkv, N, D, seed=200 + N + D + G, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, s, causal)
    O, L, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, causal)
    check_forward(f64_of(o), f64_of(lse), O, L, f"fwd N={N}")
    check_grads((dq, dk, dv), (dQ, dK, dV), f"N={N} D={D} G={G} causal={causal}")


@pytest.mark.parametrize("N,D", [(1500, 64), (2049, 128)])
@pytest.mark.parametrize("G,causal", [(1, True), (4, True), (2, False)])
def test_bwd_split_ranges(gpu, N, D, G, causal):
    """Small problems run the dK/dV pass over query ranges and the dQ pass over
    key ranges (fp32 partials summed by the reduce kernels): batch 2 and a
    ragged N put range edges inside the diagonal and tail tiles."""
    B, Hkv = 2, 1 if G != 2 else 2
    d = make_qkv(B, Hkv * G, Hkv, N, D, seed=900 + N + G, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, s, causal)
    O, L, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, causal)
    check_forward(f64_of(o), f64_of(lse), O, L, f"fwd N={N}")
    check_grads((dq, dk, dv), (dQ, dK, dV), f"split B={B} N={N} D={D} G={G} causal={causal}")


def test_bwd_full_1024(gpu):
    """B=1, H=8, D=128, N=1024: every row of O, LSE, dQ, dK and dV."""
    d = make_qkv(1, 8, 8, 1024, 128, seed=5, with_do=True)
    s = sdpa_scale(128)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, s)
    O, L, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s)
    check_forward(f64_of(o), f64_of(lse), O, L, "fwd N=1024")
    check_grads((dq, dk, dv), (dQ, dK, dV), "N=1024")


def test_bwd_listing_mean_square_loss(gpu):
    """The glossary example's loss, mean(O^2), on its [1, 4, 4096, 64] shape:
    dO = 2 O / numel, each side from its own forward."""
    import torch
    w = WORKLOADS["listing_4k"]
    d = make_workload_inputs(w)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    o, lse = lc.attn_fwd(q, k, v, causal=True, scale=w.scale)
    do = (2.0 * o.float() / o.numel()).to(torch.bfloat16)
    dq, dk, dv = lc.attn_bwd(q, k, v, o, do, lse, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    O, _ = oracle.attention_forward(d["q"], d["k"], d["v"], w.scale)
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], 2.0 * O / O.size, w.scale)
    check_grads((dq, dk, dv), (dQ, dK, dV), "mean(O^2)")


def test_bwd_deterministic(gpu):
    import torch
    d = make_qkv(1, 4, 1, 700, 128, seed=36, with_do=True)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    r1 = gpu_fwd_bwd(q, k, v, do, sdpa_scale(128))
    r2 = gpu_fwd_bwd(q, k, v, do, sdpa_scale(128))
    for a, b in zip(r1, r2):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_bwd_train_64k_sampled(gpu):
    """N = 65536, H = 8, D = 128.  (1) O and LSE at 128 sampled rows; (2) dQ at
    those rows with the full dO; (3) with dO zeroed outside the sampled rows,
    dK and dV at every key row (gradients are linear in dO, so the oracle's
    sums run over the sampled rows only)."""
    import torch
    w = WORKLOADS["train_64k"]
    d = make_workload_inputs(w)
    s = w.scale
    rows = sample_rows(w.N, w.seed, w.sampled_rows)
    idx = torch.from_numpy(rows).cuda()
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, s)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], s, True, rows=rows)
    check_forward(f64_of(o[:, :, idx]), f64_of(lse[:, :, idx]), O, L, "train_64k fwd")
    dq_s = f64_of(dq[:, :, idx])
    del dq, dk, dv
    # (3) dO restricted to the sampled rows
    do_r = torch.zeros_like(do)
    do_r[:, :, idx] = do[:, :, idx]
    dq2, dk2, dv2 = lc.attn_bwd(q, k, v, o, do_r, lse, causal=True, scale=s)
    torch.cuda.synchronize()
    do_np = oracle.bf16_bits_to_f64(d["do"])
    mask = np.zeros(w.N, dtype=bool)
    mask[rows] = True
    do_np[:, :, ~mask] = 0.0
    rq, rk, rv = oracle.attention_backward_row_support(d["q"], d["k"], d["v"], do_np, s, rows)
    e_dq = grad_rel_err(dq_s, rq)                      # (2): full dO, sampled rows
    e_dq2 = grad_rel_err(f64_of(dq2[:, :, idx]), rq)   # same rows, restricted dO
    e_dk = grad_rel_err(f64_of(dk2), rk)
    e_dv = grad_rel_err(f64_of(dv2), rv)
    assert max(e_dq, e_dq2, e_dk, e_dv) <= GRAD_REL_TOL, (e_dq, e_dq2, e_dk, e_dv)


def test_bwd_ulysses_shard_32k_sampled(gpu):
    """The bench step's backward at its full size: shard 0 of the 32K-token
    layer after the seq->head relayout (4 query heads on 1 key/value head, so
    the per-head dK/dV partials and their sum), dO drawn like the bench's.
    dQ at the sampled rows with the full dO; dK, dV at every key for a dO
    zeroed outside the sampled rows."""
    import torch
    from long_context_attention_fwd_amd.inputs import normal_bf16
    w = WORKLOADS["ulysses_shard_32k"]
    d = make_workload_inputs(w)
    d["do"] = normal_bf16(np.random.default_rng(w.seed + 17), (w.P, w.N // w.P, w.Hq, w.D))
    heads = {n: lc.seq_to_head_relayout(to_dev(d[n]), w.P)[0:1].contiguous() for n in ("q", "k", "v", "do")}
    ref = {n: oracle.seq_to_head(d[n], w.P)[0:1] for n in ("q", "k", "v", "do")}
    rows = sample_rows(w.N, w.seed, 64)
    idx = torch.from_numpy(rows).cuda()
    o, lse = lc.attn_fwd(heads["q"], heads["k"], heads["v"], causal=True, scale=w.scale)
    dq, _, _ = lc.attn_bwd(heads["q"], heads["k"], heads["v"], o, heads["do"], lse, causal=True, scale=w.scale)
    do_r = torch.zeros_like(heads["do"])
    do_r[:, :, idx] = heads["do"][:, :, idx]
    _, dk, dv = lc.attn_bwd(heads["q"], heads["k"], heads["v"], o, do_r, lse, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    do_np = oracle.bf16_bits_to_f64(ref["do"])
    mask = np.zeros(w.N, dtype=bool)
    mask[rows] = True
    do_np[:, :, ~mask] = 0.0
    rq, rk, rv = oracle.attention_backward_row_support(ref["q"], ref["k"], ref["v"], do_np, w.scale, rows)
    # dQ of a row depends only on that row's dO (and its LSE and Dv): the
    # restricted dO gives the sampled rows of the full dQ
    e_dq = grad_rel_err(f64_of(dq[:, :, idx]), rq)
    e_dk = grad_rel_err(f64_of(dk), rk)
    e_dv = grad_rel_err(f64_of(dv), rv)
    assert max(e_dq, e_dk, e_dv) <= GRAD_REL_TOL, (e_dq, e_dk, e_dv)


def test_bwd_train_64k_full_do(gpu):
    """N = 65536, H = 8, D = 128 with the full dO: dQ at the 128 sampled query
    rows and dK, dV at the key rows with the same 128 indices, against the
    oracle with its own fp64 LSE and Dv for every query row (each sampled key
    row is reached by its own query row and every later one, up to 65536
    terms per element of dK and dV).  Both dQ paths: the product of the
    stored dS and the recomputing pass."""
    import time
    import torch
    from gpu_util import oracle_full_lse_delta
    w = WORKLOADS["train_64k"]
    d = make_workload_inputs(w)
    s = w.scale
    rows = sample_rows(w.N, w.seed, w.sampled_rows)
    idx = torch.from_numpy(rows).cuda()
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, s)  # dq from the stored dS (the binding's default here)
    got = (f64_of(dq[:, :, idx]), f64_of(dk[:, :, idx]), f64_of(dv[:, :, idx]))
    # the recomputing dQ pass on the same values: dK, dV the same bits
    dq_r, dk_r, dv_r = lc.attn_bwd(q, k, v, o, do, lse, causal=True, scale=s, stored_ds=False)
    torch.cuda.synchronize()
    assert torch.equal(dk.view(torch.int16), dk_r.view(torch.int16))
    assert torch.equal(dv.view(torch.int16), dv_r.view(torch.int16))
    got_dq_r = f64_of(dq_r[:, :, idx])
    del q, k, v, do, o, lse, dq, dk, dv, dq_r, dk_r, dv_r
    f = {n: oracle.bf16_bits_to_f64(d[n]) for n in ("q", "k", "v", "do")}
    t0 = time.perf_counter()
    L, Dv = oracle_full_lse_delta(f["q"], f["k"], f["v"], f["do"], s)
    t1 = time.perf_counter()
    rq, rk, rv = oracle.attention_backward_sampled(f["q"], f["k"], f["v"], f["do"], s, rows, rows, True,
                                                   lse=L, dv=Dv)
    print(f"oracle: full fp64 LSE/Dv {t1 - t0:.1f} s, sampled gradients {time.perf_counter() - t1:.1f} s")
    errs = [grad_rel_err(g, r) for g, r in zip(got + (got_dq_r,), (rq, rk, rv, rq))]
    assert all(np.isfinite(g).all() for g in got + (got_dq_r,))
    assert max(errs) <= GRAD_REL_TOL, errs


def test_bwd_ulysses_shard_32k_full_do(gpu):
    """Shard 0 of the 32K-token layer (4 query heads on 1 key/value head: the
    per-query-head dK/dV partials and their sum) with the full dO: dQ at 64
    sampled rows, dK and dV at the key rows with the same indices, against the
    oracle with its own fp64 LSE and Dv for every query row."""
    import torch
    from gpu_util import oracle_full_lse_delta
    from long_context_attention_fwd_amd.inputs import normal_bf16
    w = WORKLOADS["ulysses_shard_32k"]
    d = make_workload_inputs(w)
    d["do"] = normal_bf16(np.random.default_rng(w.seed + 17), (w.P, w.N // w.P, w.Hq, w.D))
    heads = {n: lc.seq_to_head_relayout(to_dev(d[n]), w.P)[0:1].contiguous() for n in ("q", "k", "v", "do")}
    rows = sample_rows(w.N, w.seed, 64)
    idx = torch.from_numpy(rows).cuda()
    o, lse = lc.attn_fwd(heads["q"], heads["k"], heads["v"], causal=True, scale=w.scale)
    dq, dk, dv = lc.attn_bwd(heads["q"], heads["k"], heads["v"], o, heads["do"], lse, causal=True, scale=w.scale)
    # the recomputing dQ pass on the same values (the call above took the stored dS)
    dq_r, dk_r, dv_r = lc.attn_bwd(heads["q"], heads["k"], heads["v"], o, heads["do"], lse, causal=True,
                                   scale=w.scale, stored_ds=False)
    torch.cuda.synchronize()
    assert torch.equal(dk.view(torch.int16), dk_r.view(torch.int16))
    assert torch.equal(dv.view(torch.int16), dv_r.view(torch.int16))
    got = (f64_of(dq[:, :, idx]), f64_of(dk[:, :, idx]), f64_of(dv[:, :, idx]), f64_of(dq_r[:, :, idx]))
    f = {n: oracle.bf16_bits_to_f64(oracle.seq_to_head(d[n], w.P)[0:1]) for n in ("q", "k", "v", "do")}
    L, Dv = oracle_full_lse_delta(f["q"], f["k"], f["v"], f["do"], w.scale)
    rq, rk, rv = oracle.attention_backward_sampled(f["q"], f["k"], f["v"], f["do"], w.scale, rows, rows, True,
                                                   lse=L, dv=Dv)
    errs = [grad_rel_err(g, r) for g, r in zip(got, (rq, rk, rv, rq))]
    assert all(np.isfinite(g).all() for g in got)
    assert max(errs) <= GRAD_REL_TOL, errs


def test_bwd_side_stream_concurrent_callers(gpu):
    """Small backwards run their dQ pass on a side stream of the library's own,
    one per caller stream.  Calls issued concurrently from two caller streams,
    and a chain of accumulating block calls on a third, give the same bits as
    the same work done alone, one call at a time, on the default stream; the
    allocation-free entry point (single stream) agrees with both."""
    import torch
    D, N = 64, 4096
    ins = []
    for seed in (31, 32):
        d = make_qkv(1, 4, 4, N, D, seed=seed, with_do=True)
        q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
        o, lse = lc.attn_fwd(q, k, v, scale=sdpa_scale(D))
        ins.append((q, k, v, o, do, lse))
    torch.cuda.synchronize()

    def bwd(x):
        q, k, v, o, do, lse = x
        return lc.attn_bwd(q, k, v, o, do, lse, scale=sdpa_scale(D))
    ref = [bwd(x) for x in ins]
    torch.cuda.synchronize()
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    out = [None, None]
    for _ in range(3):
        ev = torch.cuda.Event()
        ev.record()
        for st in (s1, s2, s3):
            st.wait_event(ev)
        with torch.cuda.stream(s1):
            out[0] = bwd(ins[0])
        with torch.cuda.stream(s2):
            out[1] = bwd(ins[1])
        with torch.cuda.stream(s3):
            # four KV blocks of ins[0] accumulated into one fp32 dQ, in order
            q, k, v, o, do, lse = ins[0]
            delta = lc.attn_bwd_delta(o, do)
            dq_acc = torch.empty(tuple(q.shape), dtype=torch.float32, device="cuda")
            for i, a in enumerate(range(0, N, 1024)):
                lc.attn_bwd_block(q, k[:, :, a:a + 1024].contiguous(), v[:, :, a:a + 1024].contiguous(), do, lse, delta,
                                  scale=sdpa_scale(D), k_pos0=a, dq_acc=dq_acc, dq_accumulate=i > 0)
            dq_blocks = dq_acc.to(torch.bfloat16)
        torch.cuda.synchronize()
        for r, g in zip(ref, out):
            for x, y in zip(r, g):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16))
        # the block chain sums the same fp32 terms in another grouping: gate, not bits
        assert grad_rel_err(f64_of(dq_blocks), f64_of(ref[0][0])) <= GRAD_REL_TOL
    q, k, v, o, do, lse = ins[1]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lc.attn_bwd_noalloc(q, k, v, o, do, lse, scale=sdpa_scale(D), dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for x, y in zip(ref[1], (dq, dk, dv)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_graph_capture_replays(gpu):
    """Forward and backward of the glossary shape captured into one HIP graph
    (the backward forks its dQ pass onto its side stream and joins it back
    inside the capture) and replayed three times, with eager library calls on
    other inputs in between: every replay equals the eager result bit for bit."""
    import torch
    D, N = 64, 4096
    d = make_qkv(1, 4, 4, N, D, seed=41, with_do=True)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    s = sdpa_scale(D)
    o, lse = torch.empty_like(q), torch.empty((1, 4, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, lc.attn_bwd_workspace_size(1, 4, 4, N, D)), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        lc.attn_fwd(q, k, v, scale=s, o=o, lse=lse)
        lc.attn_bwd(q, k, v, o, do, lse, scale=s, workspace=ws, dq=dq, dk=dk, dv=dv)
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        step()  # the capture stream's side stream exists before the capture
    torch.cuda.synchronize()
    ref = [x.clone() for x in (o, lse, dq, dk, dv)]
    other = make_qkv(1, 4, 4, N, D, seed=42, with_do=True)
    oq, ok_, ov, odo = (to_dev(other[n]) for n in ("q", "k", "v", "do"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    for _ in range(3):
        for x in (o, lse, dq, dk, dv):
            x.zero_()
        g.replay()
        torch.cuda.synchronize()
        for r, x in zip(ref, (o, lse, dq, dk, dv)):
            assert torch.equal(r.view(torch.int16) if r.dtype == torch.bfloat16 else r.view(torch.int32),
                               x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32))
        # eager work of the library between replays
        oo, ol = lc.attn_fwd(oq, ok_, ov, scale=s)
        lc.attn_bwd(oq, ok_, ov, oo, odo, ol, scale=s)
        torch.cuda.synchronize()
