"""GPU parity of attn_fwd_accumulate: a ring over KV blocks streamed into one
running fp32 result must give full attention (the fp64 oracle, and the GPU's
own attn_fwd), whatever the block order."""

import math

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import WORKLOADS, make_qkv, make_workload_inputs, sample_rows

from gpu_util import check_forward, f64_of, poisoned, to_dev

pytestmark = pytest.mark.gpu


def sdpa_scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def stream_ring(q, k, v, blk, causal, scale, order=None):
    """Run the ring: one attn_fwd_accumulate per KV block; returns (o bf16, lse)."""
    import torch
    B, Hq, Nq, D = q.shape
    Nk = k.shape[2]
    starts = list(range(0, Nk, blk))
    if order is not None:
        starts = [starts[i] for i in order]
    o_acc = poisoned((B, Hq, Nq, D), torch.float32)
    lse_acc = poisoned((B, Hq, Nq), torch.float32)
    o = poisoned((B, Hq, Nq, D), torch.bfloat16)
    for i, a in enumerate(starts):
        e = min(a + blk, Nk)
        lc.attn_fwd_accumulate(q, k[:, :, a:e].contiguous(), v[:, :, a:e].contiguous(), o_acc, lse_acc,
                               first=(i == 0), causal=causal, scale=scale, k_pos0=a,
                               o_final=o if i == len(starts) - 1 else None)
    torch.cuda.synchronize()
    return o, lse_acc


@pytest.mark.parametrize("N,blk", [(200, 64), (1000, 256), (1000, 1000), (777, 100)])
@pytest.mark.parametrize("G,causal", [(1, True), (4, True), (2, False)])
def test_ring_stream_matches_oracle(gpu, N, blk, G, causal):
    d = make_qkv(1, 2 * G, 2, N, 128, seed=600 + N + blk + G)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    o, lse = stream_ring(q, k, v, blk, causal, sdpa_scale(128))
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(128), causal)
    check_forward(f64_of(o), f64_of(lse), O, L, f"stream N={N} blk={blk} G={G} causal={causal}")


def test_ring_stream_any_block_order(gpu):
    """The merge is symmetric: blocks in reverse or shuffled order (the first
    call may even be a block that no early query sees) give the same result."""
    d = make_qkv(1, 4, 1, 900, 64, seed=77)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(64), True)
    for order in ([3, 2, 1, 0], [2, 0, 3, 1]):
        o, lse = stream_ring(q, k, v, 225, True, sdpa_scale(64), order)
        check_forward(f64_of(o), f64_of(lse), O, L, f"order {order}")


def test_ring_stream_32k_blocks(gpu):
    """The ring workload: 8 heads, N = 32768, four 8192-key blocks streamed;
    against the GPU's full attn_fwd on every row and the oracle on sampled rows."""
    import torch
    w = WORKLOADS["ring_blocks_32k"]
    d = make_workload_inputs(w)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    o, lse = stream_ring(q, k, v, w.N // 4, True, w.scale)
    o_full, lse_full = lc.attn_fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    check_forward(f64_of(o), f64_of(lse), f64_of(o_full), f64_of(lse_full), "stream vs attn_fwd")
    rows = sample_rows(w.N, w.seed, 64, block=w.N // 4)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], w.scale, True, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    check_forward(f64_of(o[:, :, idx]), f64_of(lse[:, :, idx]), O, L, "stream vs oracle")


@pytest.mark.parametrize("scheme", ["zigzag", "contiguous"])
@pytest.mark.parametrize("P,C,G,causal", [(4, 256, 4, True), (2, 300, 1, True), (8, 64, 2, True), (4, 100, 2, False)])
def test_ring_sharding_schemes(gpu, scheme, P, C, G, causal):
    """Every rank's ring (its two chunks of the 2P, each chunk pair one
    attn_fwd_accumulate with global positions) against the oracle's full
    causal attention at that rank's rows."""
    import torch
    from long_context_attention_fwd_amd.ring import rank_chunks, ring_forward
    N, D, Hkv = 2 * P * C, 128, 1
    d = make_qkv(1, Hkv * G, Hkv, N, D, seed=700 + P + C + G)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    s = sdpa_scale(D)

    def chunk(t, c):
        return t[:, :, c * C:(c + 1) * C].contiguous()

    kv = {r: tuple((chunk(k, c), chunk(v, c)) for c in rank_chunks(r, P, scheme)) for r in range(P)}
    streams = [torch.cuda.Stream() for _ in range(2)]  # odd ranks run their two chunks side by side
    for r in range(P):
        mine = rank_chunks(r, P, scheme)
        qs = [chunk(q, c) for c in mine]
        o_acc = [poisoned((1, Hkv * G, C, D), torch.float32) for _ in mine]
        lse = [poisoned((1, Hkv * G, C), torch.float32) for _ in mine]
        o = [poisoned((1, Hkv * G, C, D), torch.bfloat16) for _ in mine]
        ring_forward(qs, lambda src: kv[src], r, P, C, o_acc=o_acc, lse_acc=lse, o_final=o, scheme=scheme, scale=s,
                     causal=causal, streams=streams if r % 2 else None)
        torch.cuda.synchronize()
        for i, c in enumerate(mine):
            rows = np.arange(c * C, (c + 1) * C)
            O, L = oracle.attention_forward(d["q"], d["k"], d["v"], s, causal, rows=rows)
            check_forward(f64_of(o[i]), f64_of(lse[i]), O, L, f"{scheme} P={P} rank {r} chunk {c}")


@pytest.mark.parametrize("scheme", ["zigzag", "contiguous"])
@pytest.mark.parametrize("P,C,G,causal,D", [(4, 256, 4, True, 128), (2, 300, 1, True, 64), (4, 100, 2, False, 128)])
def test_ring_grouped_launches_match_calls(gpu, scheme, P, C, G, causal, D):
    """One attn_fwd_accumulate_group launch per (step, key chunk) gives, bit
    for bit, what the calls made one by one give, for every rank."""
    import torch
    from long_context_attention_fwd_amd.ring import rank_chunks, ring_forward
    N, Hkv = 2 * P * C, 1
    d = make_qkv(1, Hkv * G, Hkv, N, D, seed=900 + P + C + G + D)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    s = sdpa_scale(D)

    def chunk(t, c):
        return t[:, :, c * C:(c + 1) * C].contiguous()

    kv = {r: tuple((chunk(k, c), chunk(v, c)) for c in rank_chunks(r, P, scheme)) for r in range(P)}
    for r in range(P):
        mine = rank_chunks(r, P, scheme)
        qs = [chunk(q, c) for c in mine]
        outs = []
        for grouped in (False, True):
            o_acc = [poisoned((1, Hkv * G, C, D), torch.float32) for _ in mine]
            lse = [poisoned((1, Hkv * G, C), torch.float32) for _ in mine]
            o = [poisoned((1, Hkv * G, C, D), torch.bfloat16) for _ in mine]
            ring_forward(qs, lambda src: kv[src], r, P, C, o_acc=o_acc, lse_acc=lse, o_final=o, scheme=scheme,
                         scale=s, causal=causal, grouped=grouped)
            torch.cuda.synchronize()
            outs.append((o, lse, o_acc))
        for i in range(2):
            for a, b in zip(outs[0], outs[1]):
                assert torch.equal(a[i].view(torch.int32) if a[i].dtype == torch.float32 else a[i].view(torch.int16),
                                   b[i].view(torch.int32) if b[i].dtype == torch.float32 else b[i].view(torch.int16)), \
                    f"{scheme} P={P} rank {r} chunk {i}"
        for i, c in enumerate(mine):
            rows = np.arange(c * C, (c + 1) * C)
            O, L = oracle.attention_forward(d["q"], d["k"], d["v"], s, causal, rows=rows)
            check_forward(f64_of(outs[1][0][i]), f64_of(outs[1][1][i]), O, L, f"grouped {scheme} rank {r} chunk {c}")


@pytest.mark.parametrize("B", [1, 2])
def test_accumulate_group_uneven_calls(gpu, B):
    """Calls of different lengths and positions in one launch (the grid covers
    the longest): each equal to its own attn_fwd_accumulate."""
    import torch
    D, G = 128, 4
    d = make_qkv(B, G, 1, 1500, D, seed=77 + B)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    s = sdpa_scale(D)
    spec = [(0, 700, 0, 900), (700, 1500, 300, 1200), (1400, 1500, 0, 1500)]  # (q0, q1, k0, k1)
    ref, grp = [], []
    for q0, q1, k0, k1 in spec:
        args = dict(q=q[:, :, q0:q1].contiguous(), k=k[:, :, k0:k1].contiguous(), v=v[:, :, k0:k1].contiguous(),
                    q_pos0=q0, k_pos0=k0)
        o1 = poisoned((B, G, q1 - q0, D), torch.float32)
        l1 = poisoned((B, G, q1 - q0), torch.float32)
        lc.attn_fwd_accumulate(args["q"], args["k"], args["v"], o1, l1, first=True, scale=s, q_pos0=q0, k_pos0=k0)
        ref.append((o1, l1))
        o2 = poisoned((B, G, q1 - q0, D), torch.float32)
        l2 = poisoned((B, G, q1 - q0), torch.float32)
        grp.append(dict(args, o_acc=o2, lse_acc=l2, first=True))
    lc.attn_fwd_accumulate_group(grp, scale=s)
    torch.cuda.synchronize()
    for (o1, l1), g in zip(ref, grp):
        assert torch.equal(o1.view(torch.int32), g["o_acc"].view(torch.int32))
        assert torch.equal(l1.view(torch.int32), g["lse_acc"].view(torch.int32))


def stream_ring_split(q, k, v, blk, causal, scale, n_splits, order=None):
    """The ring of stream_ring, each block's call split into n_splits key
    ranges (attn_fwd_accumulate_group_split with one call)."""
    import torch
    B, Hq, Nq, D = q.shape
    Nk = k.shape[2]
    starts = list(range(0, Nk, blk))
    if order is not None:
        starts = [starts[i] for i in order]
    o_acc = poisoned((B, Hq, Nq, D), torch.float32)
    lse_acc = poisoned((B, Hq, Nq), torch.float32)
    o = poisoned((B, Hq, Nq, D), torch.bfloat16)
    ws = torch.empty(lc.attn_fwd_accumulate_workspace_size(B, Hq, Nq, D, n_splits), dtype=torch.uint8, device="cuda")
    for i, a in enumerate(starts):
        e = min(a + blk, Nk)
        lc.attn_fwd_accumulate_group_split(
            [dict(q=q, k=k[:, :, a:e].contiguous(), v=v[:, :, a:e].contiguous(), o_acc=o_acc, lse_acc=lse_acc,
                  first=(i == 0), k_pos0=a, o_final=o if i == len(starts) - 1 else None, workspace=ws)],
            n_splits=n_splits, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse_acc, o_acc


@pytest.mark.parametrize("N,blk,n_splits", [(200, 64, 2), (1000, 256, 3), (1000, 1000, 5), (777, 100, 1),
                                            (1000, 1000, 64)])
@pytest.mark.parametrize("G,causal,D", [(1, True, 128), (4, True, 64), (2, False, 128)])
def test_ring_stream_split_matches_oracle(gpu, N, blk, n_splits, G, causal, D):
    """Each block's keys in n_splits ranges side by side, merged with the
    running result: the oracle's attention over every block (also with more
    ranges than key tiles, where most ranges see nothing)."""
    d = make_qkv(1, 2 * G, 2, N, D, seed=700 + N + blk + G + n_splits)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    o, lse, o_acc = stream_ring_split(q, k, v, blk, causal, sdpa_scale(D), n_splits)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(D), causal)
    check_forward(f64_of(o), f64_of(lse), O, L, f"split stream N={N} blk={blk} S={n_splits} G={G} causal={causal}")
    check_forward(f64_of(o_acc), f64_of(lse), O, L, f"split stream fp32 N={N} blk={blk} S={n_splits}")


def test_ring_stream_split_any_order_and_empty_blocks(gpu):
    """Blocks in shuffled order, the first one seen by no early query; a block
    past every query leaves the running result bit for bit as it was."""
    import torch
    d = make_qkv(1, 4, 1, 900, 64, seed=78)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(64), True)
    o, lse, o_acc = stream_ring_split(q, k, v, 225, True, sdpa_scale(64), 3, order=[3, 0, 2, 1])
    check_forward(f64_of(o), f64_of(lse), O, L, "split stream shuffled")
    before_o, before_l = o_acc.clone(), lse.clone()
    kb = to_dev(make_qkv(1, 4, 1, 300, 64, seed=79)["k"])
    vb = to_dev(make_qkv(1, 4, 1, 300, 64, seed=80)["v"])
    ws = torch.empty(lc.attn_fwd_accumulate_workspace_size(1, 4, 900, 64, 4), dtype=torch.uint8, device="cuda")
    lc.attn_fwd_accumulate_group_split([dict(q=q, k=kb, v=vb, o_acc=o_acc, lse_acc=lse, first=False, k_pos0=900,
                                             workspace=ws)], n_splits=4, scale=sdpa_scale(64))
    torch.cuda.synchronize()
    assert torch.equal(o_acc.view(torch.int32), before_o.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), before_l.view(torch.int32))


@pytest.mark.parametrize("B", [1, 2])
def test_accumulate_group_split_uneven_calls(gpu, B):
    """Calls of different lengths and positions, split and merged in one
    launch each way: each within the gate of the oracle over its block, and
    close to its own unsplit attn_fwd_accumulate."""
    import torch
    D, G = 128, 4
    d = make_qkv(B, G, 1, 1500, D, seed=87 + B)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    s = sdpa_scale(D)
    spec = [(0, 700, 0, 900), (700, 1500, 300, 1200), (1400, 1500, 0, 1500)]  # (q0, q1, k0, k1)
    grp, ref = [], []
    for q0, q1, k0, k1 in spec:
        args = dict(q=q[:, :, q0:q1].contiguous(), k=k[:, :, k0:k1].contiguous(), v=v[:, :, k0:k1].contiguous(),
                    q_pos0=q0, k_pos0=k0)
        o1 = poisoned((B, G, q1 - q0, D), torch.float32)
        l1 = poisoned((B, G, q1 - q0), torch.float32)
        lc.attn_fwd_accumulate(args["q"], args["k"], args["v"], o1, l1, first=True, scale=s, q_pos0=q0, k_pos0=k0)
        ref.append((o1, l1))
        grp.append(dict(args, o_acc=poisoned((B, G, q1 - q0, D), torch.float32),
                        lse_acc=poisoned((B, G, q1 - q0), torch.float32), first=True,
                        o_final=poisoned((B, G, q1 - q0, D), torch.bfloat16)))
    lc.attn_fwd_accumulate_group_split(grp, n_splits=3, scale=s)
    torch.cuda.synchronize()
    for (q0, q1, k0, k1), (o1, l1), g in zip(spec, ref, grp):
        qs = d["q"][:, :, q0:q1].copy()
        O, L = oracle.attention_forward(qs, d["k"][:, :, k0:k1].copy(), d["v"][:, :, k0:k1].copy(), s, True, q0, k0)
        check_forward(f64_of(g["o_final"]), f64_of(g["lse_acc"]), O, L, f"split group call q0={q0} k0={k0}")
        vis = torch.isfinite(l1)
        assert torch.equal(vis, torch.isfinite(g["lse_acc"]))
        assert torch.allclose(g["lse_acc"][vis], l1[vis], rtol=0, atol=1e-4)
        assert torch.allclose(g["o_acc"], o1, rtol=0, atol=2e-3)
        assert torch.equal(g["o_final"].view(torch.int16), g["o_acc"].to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("scheme", ["zigzag", "contiguous"])
@pytest.mark.parametrize("P,C,G,causal,D,S", [(4, 256, 4, True, 128, 4), (2, 300, 1, True, 64, 3),
                                              (4, 100, 2, False, 128, 2)])
def test_ring_grouped_split_matches_oracle(gpu, scheme, P, C, G, causal, D, S):
    """Every rank's ring with each step's grouped calls split into S key
    ranges (ring_forward(..., grouped=True, n_splits=S)): the oracle's rows of
    the rank's chunks."""
    import torch
    from long_context_attention_fwd_amd.ring import rank_chunks, ring_forward
    N, Hkv = 2 * P * C, 1
    d = make_qkv(1, Hkv * G, Hkv, N, D, seed=950 + P + C + G + D)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    s = sdpa_scale(D)

    def chunk(t, c):
        return t[:, :, c * C:(c + 1) * C].contiguous()

    kv = {r: tuple((chunk(k, c), chunk(v, c)) for c in rank_chunks(r, P, scheme)) for r in range(P)}
    wss = [torch.empty(lc.attn_fwd_accumulate_workspace_size(1, Hkv * G, C, D, S), dtype=torch.uint8, device="cuda")
           for _ in range(4)]
    for r in range(P):
        mine = rank_chunks(r, P, scheme)
        o_acc = [poisoned((1, Hkv * G, C, D), torch.float32) for _ in mine]
        lse = [poisoned((1, Hkv * G, C), torch.float32) for _ in mine]
        o = [poisoned((1, Hkv * G, C, D), torch.bfloat16) for _ in mine]
        ring_forward([chunk(q, c) for c in mine], lambda src: kv[src], r, P, C, o_acc=o_acc, lse_acc=lse, o_final=o,
                     scheme=scheme, scale=s, causal=causal, grouped=True, n_splits=S, workspaces=wss)
        torch.cuda.synchronize()
        for i, c in enumerate(mine):
            rows = np.arange(c * C, (c + 1) * C)
            O, L = oracle.attention_forward(d["q"], d["k"], d["v"], s, causal, rows=rows)
            check_forward(f64_of(o[i]), f64_of(lse[i]), O, L, f"split grouped {scheme} rank {r} chunk {c}")
