"""GPU parity on seeded random shapes: batch, head grouping, ragged query and
key lengths, head dim, mask kind and global positions drawn together, so that
combinations no hand-picked sweep lists (a split-KV range edge inside a
diagonal tile of a batch-3 grouped call, a split backward with a ragged tail)
meet the oracle.  The draw is fixed by the seed; each case prints its shape
before it runs.
"""

import math

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import make_qkv

from gpu_util import GRAD_REL_TOL, check_forward, f64_of, grad_rel_err, poisoned, to_dev

pytestmark = pytest.mark.gpu


def draw_cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 4]))
        D = int(rng.choice([64, 128]))
        Nq = int(rng.integers(1, 1300))
        Nk = int(rng.integers(1, 1300))
        causal = bool(rng.integers(0, 2))
        k_pos0 = int(rng.integers(0, 700))
        q_pos0 = int(rng.integers(0, 700))
        n_splits = int(rng.integers(0, 10))
        cases.append((B, Hkv, G, D, Nq, Nk, causal, q_pos0, k_pos0, n_splits))
    return cases


CASES = draw_cases(20)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_forward_and_split(gpu, case):
    """attn_fwd and attn_fwd_splitkv (the drawn range count; 0: the library's
    choice) with global positions against the oracle."""
    import torch
    B, Hkv, G, D, Nq, Nk, causal, qp, kp, ns = CASES[case]
    print(f"case {case}: B={B} Hkv={Hkv} G={G} D={D} Nq={Nq} Nk={Nk} causal={causal} q_pos0={qp} k_pos0={kp} "
          f"n_splits={ns}", flush=True)
    Hq = Hkv * G
    dq = make_qkv(B, Hq, Hkv, max(Nq, Nk), D, seed=7000 + case)
    q_bits = dq["q"][:, :, :Nq].copy()
    k_bits, v_bits = dq["k"][:, :, :Nk].copy(), dq["v"][:, :, :Nk].copy()
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    s = float(np.float32(1.0 / math.sqrt(D)))
    O, L = oracle.attention_forward(q_bits, k_bits, v_bits, s, causal, qp, kp)
    o = poisoned((B, Hq, Nq, D), torch.bfloat16)
    lse = poisoned((B, Hq, Nq), torch.float32)
    lc.attn_fwd(q, k, v, causal=causal, scale=s, q_pos0=qp, k_pos0=kp, o=o, lse=lse)
    torch.cuda.synchronize()
    check_forward(f64_of(o), f64_of(lse), O, L, f"attn_fwd case {case}")
    o2 = poisoned((B, Hq, Nq, D), torch.bfloat16)
    lse2 = poisoned((B, Hq, Nq), torch.float32)
    lc.attn_fwd_splitkv(q, k, v, causal=causal, scale=s, q_pos0=qp, k_pos0=kp, n_splits=ns, o=o2, lse=lse2)
    torch.cuda.synchronize()
    check_forward(f64_of(o2), f64_of(lse2), O, L, f"attn_fwd_splitkv case {case}")


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_backward(gpu, case):
    """attn_bwd (split into ranges whenever the shape is small) on the drawn
    batch, grouping, head dim, mask kind and length (Nq = Nk = the drawn Nq)
    against the oracle."""
    import torch
    B, Hkv, G, D, N, _, causal, _, _, _ = CASES[case]
    print(f"case {case}: B={B} Hkv={Hkv} G={G} D={D} N={N} causal={causal} "
          f"workspace={lc.attn_bwd_workspace_size(B, Hkv * G, Hkv, N, D)}", flush=True)
    Hq = Hkv * G
    d = make_qkv(B, Hq, Hkv, N, D, seed=8000 + case, with_do=True)
    s = float(np.float32(1.0 / math.sqrt(D)))
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=s)
    dq = poisoned(tuple(q.shape), torch.bfloat16)
    dk = poisoned(tuple(k.shape), torch.bfloat16)
    dv = poisoned(tuple(v.shape), torch.bfloat16)
    lc.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=s, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, causal)
    for name, g, r in (("dq", dq, dQ), ("dk", dk, dK), ("dv", dv, dV)):
        gg = f64_of(g)
        assert np.isfinite(gg).all(), f"case {case}: non-finite {name}"
        e = grad_rel_err(gg, r)
        assert e <= GRAD_REL_TOL, f"case {case}: {name} relative error {e}"
