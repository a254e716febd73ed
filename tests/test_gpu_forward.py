"""GPU parity of attn_fwd against the fp64 oracle (through the C ABI)."""

import math

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import WORKLOADS, make_qkv, make_workload_inputs, sample_rows

from gpu_util import bits_of, check_forward, f64_of, poisoned, to_dev

pytestmark = pytest.mark.gpu


def sdpa_scale(D):
    """SDPA's default 1/sqrt(D), as the fp32 value the kernel receives."""
    return float(np.float32(1.0 / math.sqrt(D)))


def run_fwd(d, causal=True, q_pos0=0, k_pos0=0, out_f32=False, scale=None):
    import torch
    q, k, v = (to_dev(d[n]) for n in "qkv")
    B, Hq, Nq, D = q.shape
    scale = sdpa_scale(D) if scale is None else scale
    o = poisoned((B, Hq, Nq, D), torch.float32 if out_f32 else torch.bfloat16)
    lse = poisoned((B, Hq, Nq), torch.float32)
    lc.attn_fwd(q, k, v, causal=causal, q_pos0=q_pos0, k_pos0=k_pos0, o=o, lse=lse,
                out_dtype=torch.float32 if out_f32 else torch.bfloat16, scale=scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 1000, 1024])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,causal", [(1, True), (2, True), (4, True), (1, False), (4, False)])
def test_fwd_small_sweep(gpu, N, D, G, causal):
    Hkv = 2
    d = make_qkv(1, Hkv * G, Hkv, N, D, seed=100 + N + D + G)
    o, lse = run_fwd(d, causal)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(D), causal)
    check_forward(f64_of(o), f64_of(lse), O, L, f"N={N} D={D} G={G} causal={causal}")


@pytest.mark.parametrize("Nq,Nk,q_pos0,k_pos0", [
    (300, 200, 0, 0),        # fewer keys than queries
    (200, 300, 100, 0),      # queries later in the sequence
    (256, 128, 0, 128),      # keys after the first queries: rows 0..127 see nothing
    (130, 70, 1000, 1100),   # block partially visible
    (96, 64, 0, 4096),       # no query sees any key
])
@pytest.mark.parametrize("G", [1, 4])
def test_fwd_partial_offsets(gpu, Nq, Nk, q_pos0, k_pos0, G):
    import torch
    rng = np.random.default_rng(7 + Nq + Nk)
    d = make_qkv(1, 2 * G, 2, max(Nq, Nk), 128, seed=int(rng.integers(1 << 30)))
    d = {"q": d["q"][:, :, :Nq].copy(), "k": d["k"][:, :, :Nk].copy(), "v": d["v"][:, :, :Nk].copy()}
    for f32 in (False, True):
        o, lse = run_fwd(d, True, q_pos0, k_pos0, out_f32=f32)
        O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(128), True, q_pos0, k_pos0)
        check_forward(f64_of(o), f64_of(lse), O, L, f"offsets f32={f32}")


def test_fwd_row0_is_v0_bit_exact(gpu):
    d = make_qkv(2, 8, 2, 300, 128, seed=31)
    o, lse = run_fwd(d)
    assert np.array_equal(bits_of(o)[:, :, 0], d["v"][:, np.repeat(np.arange(2), 4), 0])
    q0 = oracle.bf16_bits_to_f64(d["q"][:, :, 0])
    k0 = oracle.bf16_bits_to_f64(d["k"][:, np.repeat(np.arange(2), 4), 0])
    want = sdpa_scale(128) * (q0 * k0).sum(-1)
    assert np.abs(f64_of(lse)[:, :, 0] - want).max() < 1e-4


def test_fwd_zero_query_prefix_mean(gpu):
    """Q = 0: LSE_i = ln(i + 1) and O_i is the mean of V_0..V_i."""
    d = make_qkv(1, 4, 1, 777, 64, seed=32)
    d["q"][:] = 0
    o, lse = run_fwd(d)
    n = np.arange(777)
    assert np.abs(f64_of(lse)[0, :] - np.log(n + 1)[None]).max() < 1e-3
    v = oracle.bf16_bits_to_f64(d["v"])[0, 0]
    want = np.cumsum(v, axis=0) / (n + 1)[:, None]
    assert np.abs(f64_of(o)[0] - want[None]).max() < 1e-2


def test_fwd_peaky_softmax(gpu):
    """Q scaled by 8 forces frequent running-max moves and near one-hot rows,
    so O_i is close to single V rows with |O| up to ~4.5: the O gate allows
    the bf16 rounding of such outputs on top of 1e-2."""
    d = make_qkv(1, 4, 1, 1500, 128, seed=33)
    q = oracle.bf16_bits_to_f64(d["q"]) * 8.0
    d["q"] = oracle.f32_to_bf16_bits(q.astype(np.float32))
    o, lse = run_fwd(d)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], sdpa_scale(128))
    check_forward(f64_of(o), f64_of(lse), O, L, "peaky", out_rounding=True)
    # at this scale the reference's own bf16 rounding is 7.8e-3, so the plain
    # 1e-2 gate still holds; it fails if a row's largest weight is rounded
    # (a reference maximum that lags the true one)
    assert np.abs(f64_of(o) - O).max() <= 1e-2


def test_fwd_deterministic(gpu):
    d = make_qkv(1, 4, 1, 2000, 128, seed=34)
    o1, l1 = run_fwd(d)
    o2, l2 = run_fwd(d)
    assert np.array_equal(bits_of(o1), bits_of(o2))
    assert np.array_equal(f64_of(l1), f64_of(l2))


def test_fwd_listing_4k_full(gpu):
    """The glossary example's shape [1, 4, 4096, 64], every row and head."""
    w = WORKLOADS["listing_4k"]
    d = make_workload_inputs(w)
    o, lse = run_fwd(d, scale=w.scale)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], w.scale)
    check_forward(f64_of(o), f64_of(lse), O, L, "listing_4k")


def sampled_check(d, scale, rows, o, lse, what):
    """Compare the GPU output at the sampled query rows (every head)."""
    import torch
    idx = torch.from_numpy(rows).to(o.device)
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], scale, True, rows=rows)
    return check_forward(f64_of(o[:, :, idx]), f64_of(lse[:, :, idx]), O, L, what)


def test_fwd_ulysses_512k_sampled(gpu):
    """512K tokens, 4 query heads on 1 key/value head, inputs 0.5 * N(0,1)."""
    w = WORKLOADS["ulysses_512k"]
    d = make_workload_inputs(w)
    o, lse = run_fwd(d, scale=w.scale)
    rows = sample_rows(w.N, w.seed, w.sampled_rows)
    sampled_check(d, w.scale, rows, o, lse, w.name)


@pytest.mark.parametrize("shard", [0, 7])
def test_fwd_ulysses_shard_32k_sampled(gpu, shard):
    """Relayout on the GPU, then causal GQA attention on one shard (4 query
    heads, 1 key/value head, N = 32768).  The oracle does its own relayout of
    the same token-major input."""
    import torch
    w = WORKLOADS["ulysses_shard_32k"]
    d = make_workload_inputs(w)
    heads = {}
    for name in "qkv":
        y = lc.seq_to_head_relayout(to_dev(d[name]), w.P)
        heads[name] = y[shard:shard + 1].contiguous()     # [1, H/P, N, D]
    o, lse = lc.attn_fwd(heads["q"], heads["k"], heads["v"], causal=True, scale=w.scale)
    torch.cuda.synchronize()
    ref = {n: oracle.seq_to_head(d[n], w.P)[shard:shard + 1] for n in "qkv"}
    rows = sample_rows(w.N, w.seed, w.sampled_rows)
    sampled_check(ref, w.scale, rows, o, lse, f"ulysses shard {shard}")
