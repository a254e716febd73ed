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
