"""GPU parity of attn_fwd_splitkv (keys cut into ranges that run side by side,
then log-sum-exp merged) against the fp64 oracle, through the C ABI."""

import math

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import WORKLOADS, make_qkv, make_workload_inputs

from gpu_util import bits_of, check_forward, f64_of, poisoned, to_dev

pytestmark = pytest.mark.gpu


def sdpa_scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def run_split(d, causal=True, q_pos0=0, k_pos0=0, n_splits=0, scale=None):
    import torch
    q, k, v = (to_dev(d[n]) for n in "qkv")
    B, Hq, Nq, D = q.shape
    scale = sdpa_scale(D) if scale is None else scale
    o = poisoned((B, Hq, Nq, D), torch.bfloat16)
    lse = poisoned((B, Hq, Nq), torch.float32)
    need = lc.attn_fwd_splitkv_workspace_size(B, Hq, k.shape[1], Nq, k.shape[2], D, causal, n_splits)
    ws = poisoned((need // 4,), torch.float32)  # scratch starts as NaN: every part must be written
    lc.attn_fwd_splitkv(q, k, v, causal=causal, q_pos0=q_pos0, k_pos0=k_pos0, n_splits=n_splits, scale=scale,
                        workspace=ws, o=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("N", [1, 65, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,causal", [(1, True), (4, True), (2, False)])
@pytest.mark.parametrize("n_splits", [0, 3, 64])
def test_splitkv_sweep(gpu, N, D, G, causal, n_splits):
    Hkv = 2
    d = make_qkv(1, Hkv * G, Hkv, N, D, seed=300 + N + D + G + n_splits)
    o, lse = run_split(d, causal, n_splits=n_splits)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(D), causal)
    check_forward(f64_of(o), f64_of(lse), O, L, f"N={N} D={D} G={G} causal={causal} splits={n_splits}")


@pytest.mark.parametrize("Nq,Nk,q_pos0,k_pos0", [
    (300, 200, 0, 0),
    (200, 300, 100, 0),
    (256, 128, 0, 128),      # rows 0..127 see no key: o = 0, lse = -inf
    (96, 64, 0, 4096),       # no query sees any key
])
def test_splitkv_offsets(gpu, Nq, Nk, q_pos0, k_pos0):
    d = make_qkv(1, 4, 1, max(Nq, Nk), 128, seed=11 + Nq + Nk)
    d = {"q": d["q"][:, :, :Nq].copy(), "k": d["k"][:, :, :Nk].copy(), "v": d["v"][:, :, :Nk].copy()}
    o, lse = run_split(d, True, q_pos0, k_pos0, n_splits=4)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(128), True, q_pos0, k_pos0)
    check_forward(f64_of(o), f64_of(lse), O, L, "splitkv offsets")


@pytest.mark.parametrize("n_splits", [0, 5])
def test_splitkv_batch(gpu, n_splits):
    """B = 3: the grid carries batch and key range in one dimension."""
    d = make_qkv(3, 4, 2, 700, 128, seed=17 + n_splits)
    o, lse = run_split(d, True, n_splits=n_splits)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(128), True)
    check_forward(f64_of(o), f64_of(lse), O, L, f"splitkv B=3 splits={n_splits}")


def test_splitkv_listing_4k_full(gpu):
    """The glossary example's shape [1, 4, 4096, 64], every row and head, with
    the library's own choice of ranges."""
    w = WORKLOADS["listing_4k"]
    d = make_workload_inputs(w)
    o, lse = run_split(d, scale=w.scale)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], w.scale)
    check_forward(f64_of(o), f64_of(lse), O, L, "listing_4k splitkv")


def test_splitkv_agrees_with_attn_fwd(gpu):
    """Both are exact up to rounding: same gates against each other."""
    import torch
    d = make_qkv(1, 8, 2, 3000, 128, seed=41)
    o1, l1 = run_split(d, n_splits=5)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    o2, l2 = lc.attn_fwd(q, k, v, causal=True, scale=sdpa_scale(128))
    torch.cuda.synchronize()
    check_forward(f64_of(o1), f64_of(l1), f64_of(o2), f64_of(l2), "splitkv vs attn_fwd")


def test_splitkv_deterministic(gpu):
    d = make_qkv(1, 4, 4, 2048, 64, seed=42)
    o1, l1 = run_split(d)
    o2, l2 = run_split(d)
    assert np.array_equal(bits_of(o1), bits_of(o2))
    assert np.array_equal(f64_of(l1), f64_of(l2))
