"""GPU parity of attn_fwd_strided: attention read from, and written to,
token-major views (the layout the Ulysses exchange delivers) must equal
attn_fwd on the same values, bit for bit, and the fp64 oracle."""

import math

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import WORKLOADS, make_qkv, make_workload_inputs, sample_rows

from gpu_util import bits_of, check_forward, f64_of, to_dev

pytestmark = pytest.mark.gpu


def sdpa_scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def token_major(x):
    """[B, H, N, D] device tensor -> the same values as a [B, H, N, D] view of
    token-major [B, N, H, D] storage."""
    return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


@pytest.mark.parametrize("N", [1, 65, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,causal,out_f32", [(1, True, False), (4, True, True), (2, False, False)])
def test_strided_token_major(gpu, N, D, G, causal, out_f32):
    import torch
    d = make_qkv(2, 2 * G, 2, N, D, seed=500 + N + D + G)
    q, k, v = (to_dev(d[n]) for n in "qkv")
    qt, kt, vt = token_major(q), token_major(k), token_major(v)
    if N > 1:
        assert qt.stride()[2] == q.shape[1] * D  # token stride H*D: really token-major
    dt = torch.float32 if out_f32 else torch.bfloat16
    o_tok = token_major(torch.full(q.shape, float("nan"), dtype=dt, device="cuda"))
    o_s, lse_s = lc.attn_fwd_strided(qt, kt, vt, causal=causal, scale=sdpa_scale(D), out_dtype=dt, o=o_tok)
    o_c, lse_c = lc.attn_fwd(q, k, v, causal=causal, scale=sdpa_scale(D), out_dtype=dt)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(o_s.contiguous()), bits_of(o_c))
    assert np.array_equal(bits_of(lse_s), bits_of(lse_c))
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(D), causal)
    check_forward(f64_of(o_s.contiguous()), f64_of(lse_s), O, L, f"strided N={N} D={D} G={G}")


def test_strided_ulysses_shard_without_relayout(gpu):
    """Shard 0's 4 query heads and its key/value head read straight from the
    token-major [P, N/P, H, D] input (no seq->head pass): identical to
    attn_fwd on the relayouted tensors."""
    import torch
    w = WORKLOADS["ulysses_shard_32k"]
    d = make_workload_inputs(w)
    P, N, D, Hq, Hkv = w.P, w.N, w.D, w.Hq, w.Hkv
    hq, hkv = Hq // P, Hkv // P
    xq, xk, xv = (to_dev(d[n]) for n in "qkv")
    # heads [0, hq) of token-major [N, Hq, D] as a [1, hq, N, D] view
    qv = xq.view(N, Hq, D)[:, :hq].permute(1, 0, 2).unsqueeze(0)
    kv_ = xk.view(N, Hkv, D)[:, :hkv].permute(1, 0, 2).unsqueeze(0)
    vv = xv.view(N, Hkv, D)[:, :hkv].permute(1, 0, 2).unsqueeze(0)
    o_s, lse_s = lc.attn_fwd_strided(qv, kv_, vv, causal=True, scale=w.scale)
    qh = lc.seq_to_head_relayout(xq, P)[0:1]
    kh = lc.seq_to_head_relayout(xk, P)[0:1]
    vh = lc.seq_to_head_relayout(xv, P)[0:1]
    o_c, lse_c = lc.attn_fwd(qh, kh, vh, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(o_s), bits_of(o_c))
    assert np.array_equal(bits_of(lse_s), bits_of(lse_c))
    # and against the oracle on sampled rows of head 0..3
    rows = sample_rows(N, w.seed, 64)
    qn = oracle.seq_to_head(d["q"], P)[0:1]
    kn = oracle.seq_to_head(d["k"], P)[0:1]
    vn = oracle.seq_to_head(d["v"], P)[0:1]
    O, L = oracle.attention_forward(qn, kn, vn, w.scale, True, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    check_forward(f64_of(o_s[:, :, idx]), f64_of(lse_s[:, :, idx]), O, L, "strided ulysses shard")


# ---------------------------------------------------------------------------
# the backward on strided (token-major) tensors
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N", [1, 65, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,causal", [(1, True), (4, True), (2, False)])
def test_bwd_strided_token_major(gpu, N, D, G, causal):
    """attn_bwd_strided on token-major views (dq, dk, dv written token-major)
    equals attn_bwd on the same values bit for bit, and the fp64 oracle."""
    import torch
    from gpu_util import grad_rel_err
    from gpu_util import GRAD_REL_TOL
    d = make_qkv(2, 2 * G, 2, N, D, seed=700 + N + D + G, with_do=True)
    q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
    s = sdpa_scale(D)
    o, lse = lc.attn_fwd(q, k, v, causal=causal, scale=s)
    dq_c, dk_c, dv_c = lc.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=s)
    qt, kt, vt, ot, dot = (token_major(x) for x in (q, k, v, o, do))
    nan = lambda x: token_major(torch.full(x.shape, float("nan"), dtype=torch.bfloat16, device="cuda"))  # noqa: E731
    dq_s, dk_s, dv_s = lc.attn_bwd_strided(qt, kt, vt, ot, dot, lse, causal=causal, scale=s, dq=nan(q), dk=nan(k),
                                           dv=nan(v))
    torch.cuda.synchronize()
    if N > 1:
        assert dq_s.stride()[2] == q.shape[1] * D and dk_s.stride()[2] == k.shape[1] * D
    for a, b, n in ((dq_s, dq_c, "dq"), (dk_s, dk_c, "dk"), (dv_s, dv_c, "dv")):
        assert np.array_equal(bits_of(a.contiguous()), bits_of(b)), n
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s, causal)
    for g, r, n in ((dq_s, dQ, "dq"), (dk_s, dK, "dk"), (dv_s, dV, "dv")):
        assert grad_rel_err(f64_of(g.contiguous()), r) <= GRAD_REL_TOL, n


def test_bwd_strided_ulysses_shard_without_relayout(gpu):
    """The backward of shard 0 (4 query heads on 1 key/value head, N = 32768)
    read from, and written into, token-major [N, H, D] storage: identical to
    relayout + attn_bwd on head-major tensors."""
    import torch
    w = WORKLOADS["ulysses_shard_32k"]
    d = make_workload_inputs(w)
    P, N, D, Hq, Hkv = w.P, w.N, w.D, w.Hq, w.Hkv
    hq, hkv = Hq // P, Hkv // P
    xq, xk, xv = (to_dev(d[n]) for n in "qkv")
    rng = np.random.default_rng(w.seed + 17)
    from long_context_attention_fwd_amd.inputs import normal_bf16
    xdo = to_dev(normal_bf16(rng, (P, N // P, Hq, D)))

    def heads(x, H, n):  # heads [0, n) of token-major [N, H, D] as a [1, n, N, D] view
        return x.view(N, H, D)[:, :n].permute(1, 0, 2).unsqueeze(0)

    qv, kv_, vv, dov = heads(xq, Hq, hq), heads(xk, Hkv, hkv), heads(xv, Hkv, hkv), heads(xdo, Hq, hq)
    o_tok = torch.zeros((N, Hq, D), dtype=torch.bfloat16, device="cuda")
    ov, lse = lc.attn_fwd_strided(qv, kv_, vv, causal=True, scale=w.scale, o=heads(o_tok, Hq, hq))
    g_q = torch.full((N, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    g_k = torch.full((N, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    g_v = torch.full((N, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    dq_s, dk_s, dv_s = lc.attn_bwd_strided(qv, kv_, vv, ov, dov, lse, causal=True, scale=w.scale,
                                           dq=heads(g_q, Hq, hq), dk=heads(g_k, Hkv, hkv), dv=heads(g_v, Hkv, hkv))
    qh, kh, vh, doh = (lc.seq_to_head_relayout(x, P)[0:1] for x in (xq, xk, xv, xdo))
    oh, lse_c = lc.attn_fwd(qh, kh, vh, causal=True, scale=w.scale)
    dq_c, dk_c, dv_c = lc.attn_bwd(qh, kh, vh, oh, doh, lse_c, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(lse), bits_of(lse_c))
    for a, b, n in ((dq_s, dq_c, "dq"), (dk_s, dk_c, "dk"), (dv_s, dv_c, "dv")):
        assert np.array_equal(bits_of(a.contiguous()), bits_of(b)), n
    # the other heads' rows of the token-major gradient buffers are untouched
    assert torch.isnan(g_q[:, hq:].float()).all() and torch.isnan(g_k[:, hkv:].float()).all()
