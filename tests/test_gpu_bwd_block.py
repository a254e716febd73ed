"""GPU parity of the ring-step backward (attn_bwd_delta + attn_bwd_block)
against the fp64 oracle, through the C ABI.

A ring over KV blocks accumulates dQ in fp32 and emits each block's dK, dV;
summed over the blocks this must give the full backward (the oracle's
attention_backward, itself pinned to torch autograd).  Each side computes its
own forward (O, LSE) and Dv.  Gradient gate as for attn_bwd.
"""

import math

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import WORKLOADS, make_qkv, sample_rows

from gpu_util import GRAD_REL_TOL, bits_of, f64_of, grad_rel_err, poisoned, to_dev

pytestmark = pytest.mark.gpu


def sdpa_scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def cuts_of(N, parts):
    """Block boundaries: parts of uneven size, one of them a single key."""
    c = {0, N}
    for f in parts:
        c.add(min(N, max(0, int(f * N))))
    if N > 2:
        c.update((N - 1,))
    return sorted(c)


def ring_backward(q, k, v, do, lse, delta, cuts, scale, causal=True, q_pos0=0, dq_acc=None, dk_acc=None,
                  dv_acc=None, dkv_accumulate=False, want_bf16_dkv=True):
    """KV blocks [cuts[i], cuts[i+1]) in order: dQ accumulated in fp32 (bf16
    copy on the last block); dK, dV per block (bf16, and/or into fp32
    accumulators that may already hold other shards' sums)."""
    import torch
    dq_acc = poisoned(tuple(q.shape), torch.float32) if dq_acc is None else dq_acc
    dq = poisoned(tuple(q.shape), torch.bfloat16)
    dk = poisoned(tuple(k.shape), torch.bfloat16)
    dv = poisoned(tuple(v.shape), torch.bfloat16)
    n = len(cuts) - 1
    for i, (c, e) in enumerate(zip(cuts[:-1], cuts[1:])):
        kb, vb = k[:, :, c:e].contiguous(), v[:, :, c:e].contiguous()
        dkb = poisoned(tuple(kb.shape), torch.bfloat16) if want_bf16_dkv else None
        dvb = poisoned(tuple(vb.shape), torch.bfloat16) if want_bf16_dkv else None
        ka = dk_acc[:, :, c:e] if dk_acc is not None else None
        va = dv_acc[:, :, c:e] if dv_acc is not None else None
        if ka is not None:
            assert ka.is_contiguous()  # B = Hkv = 1 in the tests that pass accumulators
        lc.attn_bwd_block(q, kb, vb, do, lse, delta, causal=causal, scale=scale, q_pos0=q_pos0, k_pos0=c,
                          dq_acc=dq_acc, dq_accumulate=i > 0, dq=dq if i == n - 1 else None,
                          dk_acc=ka, dv_acc=va, dkv_accumulate=dkv_accumulate, dk=dkb, dv=dvb)
        if want_bf16_dkv:
            dk[:, :, c:e] = dkb
            dv[:, :, c:e] = dvb
    torch.cuda.synchronize()
    return dq_acc, dq, dk, dv


def check(got, ref, what):
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        x = f64_of(g)
        assert np.isfinite(x).all(), f"{what}: non-finite {name}"
        errs[name] = grad_rel_err(x, r)
    assert max(errs.values()) <= GRAD_REL_TOL, f"{what}: {errs}"
    return errs


@pytest.mark.parametrize("N", [65, 300, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,causal", [(1, True), (4, True), (2, False)])
def test_ring_backward_equals_full(gpu, N, D, G, causal):
    Hkv = 2
    d = make_qkv(1, Hkv * G, Hkv, N, D, seed=600 + N + D + G, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=s)
    delta = lc.attn_bwd_delta(o, do)
    cuts = cuts_of(N, (0.2, 0.5))
    dq_acc, dq, dk, dv = ring_backward(q, k, v, do, lse, delta, cuts, s, causal)
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, causal)
    check((dq, dk, dv), (dQ, dK, dV), f"ring N={N} D={D} G={G} causal={causal} cuts={cuts}")
    assert grad_rel_err(f64_of(dq_acc), dQ) <= GRAD_REL_TOL
    # the bf16 dQ is the fp32 accumulator rounded
    import torch
    assert torch.equal(dq.view(torch.int16), dq_acc.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("causal", [True, False])
def test_ring_backward_batch(gpu, causal):
    """B = 3 with grouped heads: the batch index of every kernel of the block
    path (Dv, dK/dV with the per-head partials and their sum, dQ)."""
    B, Hkv, G, N, D = 3, 2, 2, 500, 128
    d = make_qkv(B, Hkv * G, Hkv, N, D, seed=650 + int(causal), with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=s)
    delta = lc.attn_bwd_delta(o, do)
    dq_acc, dq, dk, dv = ring_backward(q, k, v, do, lse, delta, [0, 128, 300, 500], s, causal)
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, causal)
    check((dq, dk, dv), (dQ, dK, dV), f"batch ring causal={causal}")


@pytest.mark.parametrize("G", [1, 4])
def test_single_block_is_attn_bwd_bit_for_bit(gpu, G):
    """One block over the whole sequence with bf16 outputs runs attn_bwd's
    kernels on the same values.  The shape gives the dK/dV pass 256 or more
    workgroups, so attn_bwd does not split its passes into ranges (a split
    sums the same terms in another grouping: see the next test); its minimal
    workspace keeps the recomputing dQ pass (with room for the stored dS,
    dK and dV are the same bits and dq agrees to rounding: the stored-dS
    tests)."""
    import torch
    d = make_qkv(2, 2 * G, 2, 8192 - 57, 128, seed=41 + G, with_do=True)
    s = sdpa_scale(128)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=True, scale=s)
    dq0, dk0, dv0 = lc.attn_bwd(q, k, v, o, do, lse, causal=True, scale=s, stored_ds=False)
    delta = lc.attn_bwd_delta(o, do)
    dq1, dk1, dv1 = lc.attn_bwd_block(q, k, v, do, lse, delta, causal=True, scale=s, stored_ds=False)
    torch.cuda.synchronize()
    for a, b in ((dq0, dq1), (dk0, dk1), (dv0, dv1)):
        assert np.array_equal(bits_of(a), bits_of(b))
    # with room for the stored dS both calls take the product pass: the same bits again
    dq2, dk2, dv2 = lc.attn_bwd(q, k, v, o, do, lse, causal=True, scale=s, stored_ds=True)
    dq3, dk3, dv3 = lc.attn_bwd_block(q, k, v, do, lse, delta, causal=True, scale=s, stored_ds=True)
    torch.cuda.synchronize()
    for a, b in ((dq2, dq3), (dk2, dk3), (dv2, dv3), (dk0, dk2), (dv0, dv2)):
        assert np.array_equal(bits_of(a), bits_of(b))


@pytest.mark.parametrize("G", [1, 4])
def test_single_block_matches_split_attn_bwd(gpu, G):
    """On a small problem attn_bwd splits its passes into query and key ranges
    (fp32 partials, summed by the reduce kernels); the unsplit block call
    agrees with it to rounding, and both with the oracle."""
    d = make_qkv(1, 2 * G, 2, 777, 128, seed=41 + G, with_do=True)
    s = sdpa_scale(128)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=True, scale=s)
    got0 = lc.attn_bwd(q, k, v, o, do, lse, causal=True, scale=s)
    delta = lc.attn_bwd_delta(o, do)
    got1 = lc.attn_bwd_block(q, k, v, do, lse, delta, causal=True, scale=s)
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, True)
    check(got0, (dQ, dK, dV), f"split attn_bwd G={G}")
    check(got1, (dQ, dK, dV), f"block call G={G}")


def test_query_shards_and_kv_blocks(gpu):
    """Two query shards (each its own forward over every key, at its global
    offset) against three KV blocks; dK, dV accumulate in fp32 across the
    shards, as a block's gradients do when it travels the ring.  Blocks after
    a shard's last query contribute nothing."""
    import torch
    N, D = 600, 128
    d = make_qkv(1, 4, 1, N, D, seed=43, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    dk_acc = poisoned(tuple(k.shape), torch.float32)
    dv_acc = poisoned(tuple(v.shape), torch.float32)
    dq = torch.empty_like(q)
    cuts = [0, 200, 450, 600]
    for si, (a, b) in enumerate(((0, 250), (250, 600))):
        qs, dos = q[:, :, a:b].contiguous(), do[:, :, a:b].contiguous()
        o, lse = lc.attn_fwd(qs, k, v, causal=True, scale=s, q_pos0=a)
        delta = lc.attn_bwd_delta(o, dos)
        _, dqs, _, _ = ring_backward(qs, k, v, dos, lse, delta, cuts, s, True, q_pos0=a, dk_acc=dk_acc,
                                     dv_acc=dv_acc, dkv_accumulate=si > 0, want_bf16_dkv=False)
        dq[:, :, a:b] = dqs
    torch.cuda.synchronize()
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, True)
    check((dq, dk_acc, dv_acc), (dQ, dK, dV), "two shards x three blocks")


def test_block_with_no_visible_key(gpu):
    """A block after every query: dK = dV = 0 and an accumulating dQ is left
    bit for bit as it was."""
    import torch
    d = make_qkv(1, 4, 2, 256, 64, seed=44, with_do=True)
    s = sdpa_scale(64)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=True, scale=s)
    delta = lc.attn_bwd_delta(o, do)
    kb = to_dev(make_qkv(1, 4, 2, 100, 64, seed=45)["k"])
    vb = to_dev(make_qkv(1, 4, 2, 100, 64, seed=46)["v"])
    acc = torch.randn(tuple(q.shape), dtype=torch.float32, device="cuda")
    before = acc.clone()
    dk = poisoned(tuple(kb.shape), torch.bfloat16)
    dv = poisoned(tuple(vb.shape), torch.bfloat16)
    lc.attn_bwd_block(q, kb, vb, do, lse, delta, causal=True, scale=s, q_pos0=0, k_pos0=256, dq_acc=acc,
                      dq_accumulate=True, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.equal(acc, before)
    assert not f64_of(dk).any() and not f64_of(dv).any()


def test_partially_visible_blocks_against_oracle_block(gpu):
    """Queries at positions 1000..1129 against two non-adjacent blocks
    (900..1049 and 1100..1169): each side merges its own two partial forwards
    into the global (O, LSE); then each block's gradients against the oracle's
    attention_backward_block."""
    import torch
    D, G = 128, 4
    Nq, q0 = 130, 1000
    blocks = ((900, 150), (1100, 70))
    dq_ = make_qkv(1, 2 * G, 2, Nq, D, seed=47, with_do=True)
    kv = [make_qkv(1, 2 * G, 2, n, D, seed=48 + i) for i, (_, n) in enumerate(blocks)]
    s = sdpa_scale(D)
    q, do = to_dev(dq_["q"]), to_dev(dq_["do"])
    ks = [to_dev(x["k"]) for x in kv]
    vs = [to_dev(x["v"]) for x in kv]
    # GPU forward: streamed over the two blocks
    o_acc = torch.empty(tuple(q.shape), dtype=torch.float32, device="cuda")
    lse = torch.empty(tuple(q.shape[:3]), dtype=torch.float32, device="cuda")
    o_fin = torch.empty_like(q)
    for i, (p0, _) in enumerate(blocks):
        lc.attn_fwd_accumulate(q, ks[i], vs[i], o_acc, lse, first=i == 0, causal=True, scale=s, q_pos0=q0,
                               k_pos0=p0, o_final=o_fin if i == len(blocks) - 1 else None)
    delta = lc.attn_bwd_delta(o_fin, do)
    got = []
    for i, (p0, _) in enumerate(blocks):
        got.append(lc.attn_bwd_block(q, ks[i], vs[i], do, lse, delta, causal=True, scale=s, q_pos0=q0, k_pos0=p0))
    torch.cuda.synchronize()
    # oracle: its own partial forwards, merge, Dv
    parts = [oracle.attention_forward(dq_["q"], x["k"], x["v"], s, True, q0, p0) for x, (p0, _) in zip(kv, blocks)]
    O, L = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    Dv = np.einsum("bhnd,bhnd->bhn", oracle.bf16_bits_to_f64(dq_["do"]), O)
    for i, (x, (p0, _)) in enumerate(zip(kv, blocks)):
        rq, rk, rv = oracle.attention_backward_block(dq_["q"], x["k"], x["v"], dq_["do"], L, Dv, s, True, q0, p0)
        check(got[i], (rq, rk, rv), f"block at {p0}")


def test_ring_backward_deterministic(gpu):
    import torch
    d = make_qkv(1, 8, 2, 1500, 128, seed=49, with_do=True)
    s = sdpa_scale(128)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=True, scale=s)
    delta = lc.attn_bwd_delta(o, do)
    cuts = [0, 512, 1000, 1500]
    r1 = ring_backward(q, k, v, do, lse, delta, cuts, s)
    r2 = ring_backward(q, k, v, do, lse, delta, cuts, s)
    for a, b in zip(r1, r2):
        assert np.array_equal(bits_of(a), bits_of(b))


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (4, 1)])
def test_ring_backward_32k_sampled(gpu, Hq, Hkv):
    """N = 32768 in four 8192-key blocks (the ring example's block size), D =
    128.  dO is zeroed outside the sampled rows, so the oracle's gradients run
    over those rows only: dQ at the rows and dK, dV at every key."""
    import torch
    w = WORKLOADS["ring_blocks_32k"]
    d = make_qkv(1, Hq, Hkv, w.N, w.D, seed=w.seed, with_do=True)
    rows = sample_rows(w.N, w.seed, 64, block=w.N // 4)
    idx = torch.from_numpy(rows).cuda()
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    do_r = torch.zeros_like(do)
    do_r[:, :, idx] = do[:, :, idx]
    o, lse = lc.attn_fwd(q, k, v, causal=True, scale=w.scale)
    delta = lc.attn_bwd_delta(o, do_r)
    cuts = [0, 8192, 16384, 24576, 32768]
    _, dq, dk, dv = ring_backward(q, k, v, do_r, lse, delta, cuts, w.scale)
    do_np = oracle.bf16_bits_to_f64(d["do"])
    mask = np.zeros(w.N, dtype=bool)
    mask[rows] = True
    do_np[:, :, ~mask] = 0.0
    rq, rk, rv = oracle.attention_backward_row_support(d["q"], d["k"], d["v"], do_np, w.scale, rows)
    check((dq[:, :, idx], dk, dv), (rq, rk, rv), f"32K ring Hq={Hq} Hkv={Hkv}")


def _block_call_inputs(Hq, Hkv, D, Nq, Nk, q_pos0, k_pos0, seed, B=1):
    """q, k, v, dO of one block call and finite LSE, Dv for it (from the
    forward of q against this block)."""
    import torch
    d = make_qkv(B, Hq, Hkv, max(Nq, Nk), D, seed=seed, with_do=True)
    q, do = (to_dev(d[n][:, :, :Nq].copy()) for n in ("q", "do"))
    k, v = (to_dev(d[n][:, :, :Nk].copy()) for n in ("k", "v"))
    o, lse = lc.attn_fwd(q, k, v, causal=False, scale=sdpa_scale(D))
    delta = lc.attn_bwd_delta(o, do)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, do=do, lse=lse, delta=delta, q_pos0=q_pos0, k_pos0=k_pos0)


@pytest.mark.parametrize("D,G,B", [(128, 1, 1), (128, 4, 1), (64, 2, 1), (128, 2, 2)])
def test_bwd_block_group_matches_calls(gpu, D, G, B):
    """Up to four independent block calls in one group launch give exactly the
    results of the same calls made one at a time: uneven lengths and global
    positions (a diagonal block, a block partly visible, one fully visible,
    one no query sees), fp32 accumulators overwritten or added to, bf16
    copies; B = 2 checks the grid's (call, batch) numbering."""
    import torch
    Hkv = 2
    Hq = Hkv * G
    specs = [(300, 200, 200, 0), (256, 512, 1024, 512), (100, 64, 0, 0), (192, 128, 0, 4096)]
    gen = torch.Generator(device="cuda").manual_seed(7)
    calls = []
    for i, (Nq, Nk, qp, kp) in enumerate(specs):
        c = _block_call_inputs(Hq, Hkv, D, Nq, Nk, qp, kp, seed=300 + i, B=B)
        acc = i % 2 == 1  # odd calls add into accumulators that already hold values
        c["dq_acc"] = torch.randn((B, Hq, Nq, D), generator=gen, device="cuda")
        c["dk_acc"] = torch.randn((B, Hkv, Nk, D), generator=gen, device="cuda")
        c["dv_acc"] = torch.randn((B, Hkv, Nk, D), generator=gen, device="cuda")
        c["dq_accumulate"] = acc
        c["dkv_accumulate"] = acc
        c["dq"] = poisoned((B, Hq, Nq, D), torch.bfloat16)
        c["dk"] = poisoned((B, Hkv, Nk, D), torch.bfloat16)
        c["dv"] = poisoned((B, Hkv, Nk, D), torch.bfloat16)
        calls.append(c)
    outs = ("dq_acc", "dk_acc", "dv_acc", "dq", "dk", "dv")
    for n in (2, 4):
        grp = [dict(c, **{o: c[o].clone() for o in outs}) for c in calls[:n]]
        one = [dict(c, **{o: c[o].clone() for o in outs}) for c in calls[:n]]
        lc.attn_bwd_block_group(grp, causal=True, scale=sdpa_scale(D))
        for c in one:
            kw = {x: c[x] for x in c if x not in ("q", "k", "v", "do", "lse", "delta")}
            lc.attn_bwd_block(c["q"], c["k"], c["v"], c["do"], c["lse"], c["delta"], causal=True,
                              scale=sdpa_scale(D), **kw)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(grp, one)):
            for o in outs:
                x, y = a[o], b[o]
                if x.dtype == torch.bfloat16:
                    x, y = x.view(torch.int16), y.view(torch.int16)
                assert torch.equal(x, y), f"group of {n}: call {i} {o} differs"


@pytest.mark.parametrize("scheme", ["zigzag", "contiguous"])
@pytest.mark.parametrize("P,C,G,D", [(2, 128, 1, 128), (4, 64, 4, 128), (4, 96, 2, 64)])
def test_ring_backward_schemes(gpu, scheme, P, C, G, D):
    """Every rank's ring backward on one GPU, grouped and one call at a time:
    the dQ of each rank's query chunks and the dK, dV accumulated in each
    key/value chunk (as they would travel around the ring) equal the oracle's
    full backward.  LSE and Dv come from the GPU's full forward."""
    import torch
    from long_context_attention_fwd_amd.ring import rank_chunks, ring_backward
    Hkv = 2
    Hq = Hkv * G
    N = 2 * P * C
    s = sdpa_scale(D)
    d = make_qkv(1, Hq, Hkv, N, D, seed=900 + P + C + G, with_do=True)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=True, scale=s)
    delta = lc.attn_bwd_delta(o, do)
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, True)

    def ch(x, c):
        return x[:, :, c * C:(c + 1) * C].contiguous()
    ws = [torch.empty(max(16, lc.attn_bwd_block_workspace_size(1, Hq, Hkv, C, D)), dtype=torch.uint8,
                      device="cuda") for _ in range(4)]
    for grouped in (False, True):
        dq_acc = [torch.zeros((1, Hq, C, D), device="cuda") for _ in range(2 * P)]
        dk_acc = [torch.zeros((1, Hkv, C, D), device="cuda") for _ in range(2 * P)]
        dv_acc = [torch.zeros((1, Hkv, C, D), device="cuda") for _ in range(2 * P)]
        for r in range(P):
            mine = rank_chunks(r, P, scheme)
            ring_backward([ch(q, c) for c in mine], [ch(do, c) for c in mine], [ch(lse, c) for c in mine],
                          [ch(delta, c) for c in mine],
                          lambda src: tuple((ch(k, c), ch(v, c)) for c in rank_chunks(src, P, scheme)),
                          r, P, C, dq_acc=[dq_acc[c] for c in mine],
                          dkv_acc=lambda src, ki: (dk_acc[rank_chunks(src, P, scheme)[ki]],
                                                   dv_acc[rank_chunks(src, P, scheme)[ki]]),
                          scheme=scheme, scale=s, grouped=grouped, workspaces=ws)
        torch.cuda.synchronize()
        got = [torch.cat(x, dim=2) for x in (dq_acc, dk_acc, dv_acc)]
        check(got, (dQ, dK, dV), f"{scheme} P={P} C={C} G={G} D={D} grouped={grouped}")
