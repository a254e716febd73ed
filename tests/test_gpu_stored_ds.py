"""GPU parity of attn_bwd's stored-dS path (dq as the product of the dS
blocks that the dK/dV pass writes, selected by a workspace of
attn_bwd_ds_workspace_size bytes) against the fp64 oracle and against the
recomputing dQ pass, through the C ABI.

dK and dV come from the same kernel arithmetic on both paths (the stored-dS
instance only adds the stores), so they must match bit for bit; dq is the
same sum over keys in the same order, with dS formed from P after its bf16
rounding, so it is checked against the oracle at the gradient gate."""

import math

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import make_qkv

from gpu_util import GRAD_REL_TOL, bits_of, f64_of, grad_rel_err, poisoned, to_dev

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, N, D, causal): every case has B * Hq * ceil(N / 128) >= 256,
# the sizes that have the path
CASES = [
    (2, 8, 8, 2048, 128, True),
    (2, 8, 2, 2101, 64, True),     # grouped heads, ragged last query and key tiles
    (1, 16, 8, 2053, 128, False),  # no mask: keys past N in the last tile masked by the product pass
    (4, 4, 4, 2048, 64, False),
    (1, 16, 16, 2111, 128, True),  # odd number of 64-row tiles (the last key-tile pair half empty)
]


def sdpa_scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def token_major(x):
    return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


def run_bwd(q, k, v, o, do, lse, causal, s, ws_bytes, strided=False):
    import torch
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    if strided:
        nan = lambda x: token_major(torch.full(x.shape, float("nan"), dtype=torch.bfloat16, device="cuda"))  # noqa
        dq, dk, dv = nan(q), nan(k), nan(v)
        lc.attn_bwd_strided(q, k, v, o, do, lse, causal=causal, scale=s, workspace=ws, dq=dq, dk=dk, dv=dv)
    else:
        dq = poisoned(tuple(q.shape), torch.bfloat16)
        dk = poisoned(tuple(k.shape), torch.bfloat16)
        dv = poisoned(tuple(v.shape), torch.bfloat16)
        lc.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=s, workspace=ws, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dq.contiguous(), dk.contiguous(), dv.contiguous()


@pytest.mark.parametrize("case", range(len(CASES)))
def test_stored_ds_matches_oracle_and_recompute(gpu, case):
    B, Hq, Hkv, N, D, causal = CASES[case]
    print(f"stored dS case {case}: B={B} Hq={Hq} Hkv={Hkv} N={N} D={D} causal={causal}", flush=True)
    big = lc.attn_bwd_ds_workspace_size(B, Hq, Hkv, N, D, causal)
    small = lc.attn_bwd_workspace_size(B, Hq, Hkv, N, D)
    assert big > small > 0
    d = make_qkv(B, Hq, Hkv, N, D, seed=9100 + case, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=s)
    dq_s, dk_s, dv_s = run_bwd(q, k, v, o, do, lse, causal, s, big)
    dq_r, dk_r, dv_r = run_bwd(q, k, v, o, do, lse, causal, s, small)
    assert np.array_equal(bits_of(dk_s), bits_of(dk_r)), "dk differs between the two paths"
    assert np.array_equal(bits_of(dv_s), bits_of(dv_r)), "dv differs between the two paths"
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, causal)
    for name, g, r in (("dq", dq_s, dQ), ("dk", dk_s, dK), ("dv", dv_s, dV)):
        gg = f64_of(g)
        assert np.isfinite(gg).all(), f"non-finite {name}"
        e = grad_rel_err(gg, r)
        assert e <= GRAD_REL_TOL, f"{name} relative error {e}"
    # the two dq agree to rounding (the paths differ only in P's bf16 rounding inside dS)
    e = grad_rel_err(f64_of(dq_s), f64_of(dq_r))
    assert e <= 1e-2, f"dq of the two paths: {e}"


def test_stored_ds_strided_matches_contiguous(gpu):
    """attn_bwd_strided with the stored-dS workspace on token-major views
    equals attn_bwd with it on the same values, bit for bit."""
    B, Hq, Hkv, N, D, causal = 1, 16, 4, 2048 + 40, 128, True
    big = lc.attn_bwd_ds_workspace_size(B, Hq, Hkv, N, D, causal)
    assert big > 0
    d = make_qkv(B, Hq, Hkv, N, D, seed=9200, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=s)
    ref = run_bwd(q, k, v, o, do, lse, causal, s, big)
    got = run_bwd(*(token_major(x) for x in (q, k, v, o, do)), lse, causal, s, big, strided=True)
    for a, b, n in zip(got, ref, ("dq", "dk", "dv")):
        assert np.array_equal(bits_of(a), bits_of(b)), n


def test_stored_ds_repeat_is_deterministic(gpu):
    """Two calls with one workspace (its dS blocks left over from the first)
    give the same bits."""
    import torch
    B, Hq, Hkv, N, D, causal = 1, 8, 8, 4096, 128, True
    big = lc.attn_bwd_ds_workspace_size(B, Hq, Hkv, N, D, causal)
    d = make_qkv(B, Hq, Hkv, N, D, seed=9300, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=s)
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    first = lc.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=s, workspace=ws)
    first = [bits_of(x) for x in first]
    second = lc.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=s, workspace=ws)
    torch.cuda.synchronize()
    for a, b, n in zip(first, second, ("dq", "dk", "dv")):
        assert np.array_equal(a, bits_of(b)), n


@pytest.mark.parametrize("D,causal", [(128, True), (64, False)])
def test_stored_ds_block_ring(gpu, D, causal):
    """attn_bwd_block over three uneven KV blocks (fp32 dQ accumulated, a bf16
    copy on the last block; bf16 dK, dV per block).  The two larger blocks
    have the stored-dS path (B * Hq * ceil(Nk / 128) >= 256), the last not.
    Against the oracle's full backward, and dK, dV the same bits as the same
    ring with the recomputing pass."""
    import torch
    B, Hq, Hkv, N = 2, 16, 4, 3000
    cuts = [0, 1100, 2300, 3000]
    assert lc.attn_bwd_block_ds_workspace_size(B, Hq, Hkv, N, 1100, D) > 0
    assert lc.attn_bwd_block_ds_workspace_size(B, Hq, Hkv, N, 700, D) == 0
    d = make_qkv(B, Hq, Hkv, N, D, seed=9400 + D, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=s)
    delta = lc.attn_bwd_delta(o, do)
    res = {}
    for stored in (True, False):
        dq_acc = poisoned((B, Hq, N, D), torch.float32)
        dq = poisoned((B, Hq, N, D), torch.bfloat16)
        dks, dvs = [], []
        for i, (c, e) in enumerate(zip(cuts[:-1], cuts[1:])):
            kb, vb = k[:, :, c:e].contiguous(), v[:, :, c:e].contiguous()
            dk = poisoned(tuple(kb.shape), torch.bfloat16)
            dv = poisoned(tuple(vb.shape), torch.bfloat16)
            lc.attn_bwd_block(q, kb, vb, do, lse, delta, causal=causal, scale=s, k_pos0=c, dq_acc=dq_acc,
                              dq_accumulate=i > 0, dq=dq if i == len(cuts) - 2 else None, dk=dk, dv=dv,
                              stored_ds=stored)
            dks.append(dk)
            dvs.append(dv)
        torch.cuda.synchronize()
        res[stored] = (dq, torch.cat(dks, dim=2), torch.cat(dvs, dim=2), dq_acc)
    for i, n in ((1, "dk"), (2, "dv")):
        assert np.array_equal(bits_of(res[True][i]), bits_of(res[False][i])), n
    assert np.array_equal(bits_of(res[True][0]), bits_of(res[True][3].to(torch.bfloat16))), "bf16 copy of dq_acc"
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, causal)
    for stored in (True, False):
        for name, g, r in (("dq", res[stored][0], dQ), ("dk", res[stored][1], dK), ("dv", res[stored][2], dV)):
            e = grad_rel_err(f64_of(g), r)
            assert e <= GRAD_REL_TOL, f"stored={stored} {name} relative error {e}"


def test_stored_ds_block_query_shard(gpu):
    """A query shard at global rows 1400..2047 against KV blocks before, across
    and after it (q_pos0 != k_pos0: irregular causal rows, query tiles that
    see no key of a block, a block that no query sees), with the stored-dS
    path, fp32 dQ overwritten then added to: against
    oracle.attention_backward_block for each block."""
    import torch
    B, Hq, Hkv, N, D = 1, 32, 8, 3072, 64
    q0, q1 = 1400, 2048
    d = make_qkv(B, Hq, Hkv, N, D, seed=9500, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=True, scale=s)
    delta = lc.attn_bwd_delta(o, do)
    qs, dos = q[:, :, q0:q1].contiguous(), do[:, :, q0:q1].contiguous()
    lses, deltas = lse[:, :, q0:q1].contiguous(), delta[:, :, q0:q1].contiguous()
    q_np, do_np = d["q"][:, :, q0:q1], d["do"][:, :, q0:q1]
    lse_np, delta_np = f64_of(lses), f64_of(deltas)
    blocks = [(0, 1024), (1024, 2048), (2048, 3072)]
    dq_acc = poisoned(tuple(qs.shape), torch.float32)
    want_dq = 0.0
    for i, (c, e) in enumerate(blocks):
        assert lc.attn_bwd_block_ds_workspace_size(B, Hq, Hkv, q1 - q0, e - c, D) > 0
        kb, vb = k[:, :, c:e].contiguous(), v[:, :, c:e].contiguous()
        dk = poisoned(tuple(kb.shape), torch.bfloat16)
        dv = poisoned(tuple(vb.shape), torch.bfloat16)
        lc.attn_bwd_block(qs, kb, vb, dos, lses, deltas, causal=True, scale=s, q_pos0=q0, k_pos0=c, dq_acc=dq_acc,
                          dq_accumulate=i > 0, dk=dk, dv=dv, stored_ds=True)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.attention_backward_block(q_np, d["k"][:, :, c:e], d["v"][:, :, c:e], do_np, lse_np,
                                                     delta_np, s, True, q0, c)
        want_dq = want_dq + rq
        for name, g, r in (("dk", dk, rk), ("dv", dv, rv)):
            e_ = grad_rel_err(f64_of(g), r)
            assert e_ <= GRAD_REL_TOL, f"block {i} {name} relative error {e_}"
        e_ = grad_rel_err(f64_of(dq_acc), want_dq)
        assert e_ <= GRAD_REL_TOL, f"dq after block {i}: relative error {e_}"


def test_stored_ds_graph_replays(gpu):
    """attn_bwd with the stored-dS workspace captured into a HIP graph and
    replayed three times, with eager library calls on other inputs in
    between: every replay equals the eager result bit for bit."""
    import torch
    B, Hq, Hkv, N, D = 1, 8, 8, 4096, 128
    big = lc.attn_bwd_ds_workspace_size(B, Hq, Hkv, N, D, True)
    assert big > 0
    d = make_qkv(B, Hq, Hkv, N, D, seed=9600, with_do=True)
    s = sdpa_scale(D)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=True, scale=s)
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        lc.attn_bwd(q, k, v, o, do, lse, causal=True, scale=s, workspace=ws, dq=dq, dk=dk, dv=dv)
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (dq, dk, dv)]
    other = make_qkv(B, Hq, Hkv, N, D, seed=9601, with_do=True)
    oq, ok_, ov, odo = (to_dev(other[n]) for n in ("q", "k", "v", "do"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    for _ in range(3):
        for x in (dq, dk, dv):
            x.zero_()
        g.replay()
        torch.cuda.synchronize()
        for r, x in zip(ref, (dq, dk, dv)):
            assert torch.equal(r.view(torch.int16), x.view(torch.int16))
        oo, ol = lc.attn_fwd(oq, ok_, ov, scale=s)
        lc.attn_bwd(oq, ok_, ov, oo, odo, ol, scale=s, stored_ds=True)
        torch.cuda.synchronize()


@pytest.mark.parametrize("causal", [True, False])
def test_stored_ds_block_ragged_tail_visible(gpu, causal):
    """A 70-key block (the last 64-key tile ragged) whose queries lie past
    it (q_pos0 - k_pos0 = 500): by position every padding key of the tile is
    visible, so their stored dS must be masked by the product pass.  LSE
    over this block only, so a padding key's weight would be about 1/70 of
    a row: an unmasked one shows far above the gate.  Against
    oracle.attention_backward_block."""
    B, Hq, Hkv, Nq, Nk, D = 4, 64, 16, 256, 70, 64
    q_pos0, k_pos0 = 1000, 500
    assert lc.attn_bwd_block_ds_workspace_size(B, Hq, Hkv, Nq, Nk, D) > 0
    dq_in = make_qkv(B, Hq, Hkv, Nq, D, seed=9700, with_do=True)
    dk_in = make_qkv(B, Hq, Hkv, Nk, D, seed=9701)
    s = sdpa_scale(D)
    q, do = to_dev(dq_in["q"]), to_dev(dq_in["do"])
    k, v = to_dev(dk_in["k"]), to_dev(dk_in["v"])
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=s, q_pos0=q_pos0, k_pos0=k_pos0)
    delta = lc.attn_bwd_delta(o, do)
    dq, dk, dv = lc.attn_bwd_block(q, k, v, do, lse, delta, causal=causal, scale=s, q_pos0=q_pos0, k_pos0=k_pos0,
                                   stored_ds=True)
    import torch
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward_block(dq_in["q"], dk_in["k"], dk_in["v"], dq_in["do"], f64_of(lse),
                                                 f64_of(delta), s, causal, q_pos0, k_pos0)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = grad_rel_err(f64_of(g), r)
        assert e <= GRAD_REL_TOL, f"{name} relative error {e}"
