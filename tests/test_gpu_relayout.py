"""GPU parity of the sequence<->head relayout: bit-exact against the oracle."""

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import WORKLOADS, make_workload_inputs

from gpu_util import bits_of, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P,N,H,D", [(8, 64, 32, 128), (8, 64, 8, 128), (4, 1000, 4, 64), (2, 6, 6, 64),
                                     (1, 17, 3, 128), (8, 8, 8, 64)])
def test_relayout_small_bit_exact(gpu, P, N, H, D):
    import torch
    x = np.random.default_rng(P * N + H).integers(0, 1 << 16, size=(P, N // P, H, D), dtype=np.uint16)
    xd = to_dev(x)
    y = lc.seq_to_head_relayout(xd, P, out=torch.full((P, H // P, N, D), float("nan"), dtype=torch.bfloat16,
                                                       device="cuda"))
    back = lc.head_to_seq_relayout(y, P)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(y), oracle.seq_to_head(x, P))
    assert np.array_equal(bits_of(back), x)


def test_relayout_fp32_words(gpu):
    import torch
    x = torch.randn(4, 16, 8, 64, device="cuda")
    y = lc.seq_to_head_relayout(x, 4)
    torch.cuda.synchronize()
    want = oracle.seq_to_head(x.cpu().numpy(), 4)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_relayout_ulysses_shard_32k_full(gpu):
    """Q [8, 4096, 32, 128] and K, V [8, 4096, 8, 128] -> head shards; every
    element compared, then the inverse must give the input back."""
    import torch
    w = WORKLOADS["ulysses_shard_32k"]
    d = make_workload_inputs(w)
    for name, H in (("q", w.Hq), ("k", w.Hkv), ("v", w.Hkv)):
        xd = to_dev(d[name])
        y = lc.seq_to_head_relayout(xd, w.P)
        back = lc.head_to_seq_relayout(y, w.P)
        torch.cuda.synchronize()
        assert tuple(y.shape) == (w.P, H // w.P, w.N, w.D)
        assert np.array_equal(bits_of(y), oracle.seq_to_head(d[name], w.P)), name
        assert torch.equal(back.view(torch.int16), xd.view(torch.int16)), name
        del xd, y, back


def test_relayout_batch_ulysses_shard_32k_full(gpu):
    """Q, K, V and dO of the 32K layer moved to head shards in one launch and
    back in another: every element against the oracle, and the round trip."""
    import torch
    w = WORKLOADS["ulysses_shard_32k"]
    d = make_workload_inputs(w)
    d["do"] = np.random.default_rng(w.seed + 17).integers(0, 1 << 16, size=d["q"].shape, dtype=np.uint16)
    names = ("q", "k", "v", "do")
    xs = [to_dev(d[n]) for n in names]
    outs = [torch.full((w.P, x.shape[2] // w.P, w.N, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
            for x in xs]
    ys = lc.seq_to_head_relayout_batch(xs, w.P, outs=outs)
    backs = lc.head_to_seq_relayout_batch(ys, w.P)
    torch.cuda.synchronize()
    for n, x, y, b in zip(names, xs, ys, backs):
        assert y.data_ptr() == outs[names.index(n)].data_ptr()
        assert np.array_equal(bits_of(y), oracle.seq_to_head(d[n], w.P)), n
        assert torch.equal(b.view(torch.int16), x.view(torch.int16)), n


@pytest.mark.parametrize("P,T,heads,D,elem", [
    (8, 8, (32, 8, 8, 4, 2, 1, 16, 8), 128, 2),   # eight tensors, three of them replicated (H < P)
    (4, 25, (4, 8, 2), 64, 2),                     # ragged: 100 tokens, 64-dim rows
    (2, 3, (6, 2), 64, 4),                          # fp32 words
    (1, 17, (3,), 128, 2),                          # one tensor, one rank
])
def test_relayout_batch_matches_single_calls(gpu, P, T, heads, D, elem):
    import torch
    rng = np.random.default_rng(P * 1000 + T)
    dt = torch.bfloat16 if elem == 2 else torch.float32
    xs, hs = [], []
    for H in heads:
        x = rng.integers(0, 1 << (8 * elem), size=(P, T, H, D), dtype=np.uint16 if elem == 2 else np.uint32)
        xs.append(x)
        hs.append(torch.from_numpy(x.view(np.int16 if elem == 2 else np.int32)).cuda().view(dt))
    ys = lc.seq_to_head_relayout_batch(hs, P)
    torch.cuda.synchronize()
    it = torch.int16 if elem == 2 else torch.int32
    for x, h, y in zip(xs, hs, ys):
        single = lc.seq_to_head_relayout(h, P)
        torch.cuda.synchronize()
        assert torch.equal(y.view(it), single.view(it))
        want = oracle.seq_to_head(x, P)
        assert np.array_equal(y.cpu().view(it).numpy().view(want.dtype), want)
    plain = [i for i, H in enumerate(heads) if H >= P and H % P == 0]
    if plain:
        backs = lc.head_to_seq_relayout_batch([ys[i] for i in plain], P)
        torch.cuda.synchronize()
        for i, b in zip(plain, backs):
            assert np.array_equal(b.cpu().view(it).numpy().view(xs[i].dtype), xs[i])


# ---------------------------------------------------------------------------
# fewer key/value heads than ranks: replication out, summed gradients back
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("P,N,H,D,elem", [(8, 4096, 4, 128, 2), (8, 4096, 2, 128, 2), (8, 1024, 1, 64, 2),
                                          (4, 100, 2, 128, 4)])
def test_relayout_replicates_shared_heads(gpu, P, N, H, D, elem):
    import torch
    if elem == 2:
        x = np.random.default_rng(N + H).integers(0, 1 << 16, size=(P, N // P, H, D), dtype=np.uint16)
        xd = to_dev(x)
        got = lambda y: bits_of(y)  # noqa: E731
    else:
        x = np.random.default_rng(N + H).standard_normal((P, N // P, H, D)).astype(np.float32)
        xd = torch.from_numpy(x).cuda()
        got = lambda y: y.cpu().numpy()  # noqa: E731
    dt = torch.bfloat16 if elem == 2 else torch.float32
    y = lc.seq_to_head_relayout(xd, P, out=torch.full((P, 1, N, D), float("nan"), dtype=dt, device="cuda"))
    torch.cuda.synchronize()
    want = oracle.seq_to_head(x, P)
    assert np.array_equal(got(y).view(np.uint16 if elem == 2 else np.uint32),
                          want.view(np.uint16 if elem == 2 else np.uint32))


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("P,N,H,D,f32", [(8, 4096, 4, 128, False), (8, 4096, 2, 128, True), (8, 512, 1, 64, False),
                                         (4, 1000, 8, 128, True), (4, 1000, 8, 128, False)])
def test_head_to_seq_reduce(gpu, P, N, H, D, f32):
    """Sum of the P/H replicas of each head (fp32 adds, one bf16 rounding):
    within one bf16 spacing of the exact sum plus the fp32 additions' own
    bound (R * 2^-24 * sum of |terms|, which matters where terms cancel); a
    single term (H >= P) is the bf16 rounding of the input exactly."""
    import torch
    R = max(1, P // H)
    rng = np.random.default_rng(N + H + int(f32))
    if f32:
        y = rng.standard_normal((P, max(1, H // P), N, D)).astype(np.float32)
        yd = torch.from_numpy(y).cuda()
    else:
        y = oracle.f32_to_bf16_bits(rng.standard_normal((P, max(1, H // P), N, D)).astype(np.float32))
        yd = to_dev(y)
    out = lc.head_to_seq_reduce(yd, P, H, out=torch.full((P, N // P, H, D), float("nan"), dtype=torch.bfloat16,
                                                          device="cuda"))
    torch.cuda.synchronize()
    exact = oracle.head_to_seq_sum(y, P, H)
    g = oracle.bf16_bits_to_f64(bits_of(out))
    if R == 1:
        assert np.array_equal(bits_of(out), oracle.f32_to_bf16_bits(exact.astype(np.float32)))
    else:
        mag = oracle.head_to_seq_sum(np.abs(oracle.bf16_bits_to_f64(y) if not f32 else y.astype(np.float64)), P, H)
        bound = bf16_ulp(exact) + R * 2.0 ** -24 * mag
        assert np.all(np.abs(g - exact) <= bound), float(np.max(np.abs(g - exact) / bound))


@pytest.mark.parametrize("via_block", [False, True])
def test_ulysses_with_shared_kv_heads_end_to_end(gpu, via_block):
    """16 query heads on 2 key/value heads over P = 8 ranks: each rank gets 2
    query heads and a replica of the key/value head they read; forward and
    backward per rank; O and dQ come back by the inverse relayout, dK and dV
    by summing the 4 ranks that shared each head (bf16 per-rank gradients
    from attn_bwd, or fp32 ones from attn_bwd_block).  Against the oracle's
    full-model forward and backward."""
    import torch
    from gpu_util import GRAD_REL_TOL, check_forward, f64_of, grad_rel_err
    from long_context_attention_fwd_amd.inputs import make_qkv
    P, N, Hq, Hkv, D = 8, 512, 16, 2, 128
    scale = float(np.float32(1.0 / np.sqrt(D)))
    d = make_qkv(1, Hq, Hkv, N, D, seed=61, with_do=True)
    tok = {n: np.ascontiguousarray(np.transpose(d[n][0], (1, 0, 2))).reshape(P, N // P, -1, D)
           for n in ("q", "k", "v", "do")}  # token-major [P, N/P, H, D]
    heads = {n: lc.seq_to_head_relayout(to_dev(tok[n]), P) for n in tok}
    hq = Hq // P
    o = torch.empty((P, hq, N, D), dtype=torch.bfloat16, device="cuda")
    dq = torch.empty_like(o)
    dk = torch.empty((P, 1, N, D), dtype=torch.float32 if via_block else torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    for r in range(P):
        q_, k_, v_, do_ = (heads[n][r:r + 1] for n in ("q", "k", "v", "do"))
        o_r, lse_r = lc.attn_fwd(q_, k_, v_, causal=True, scale=scale)
        o[r:r + 1] = o_r
        if via_block:
            delta = lc.attn_bwd_delta(o_r, do_)
            lc.attn_bwd_block(q_, k_, v_, do_, lse_r, delta, causal=True, scale=scale, dq=dq[r:r + 1],
                              dk_acc=dk[r:r + 1], dv_acc=dv[r:r + 1])
        else:
            lc.attn_bwd(q_, k_, v_, o_r, do_, lse_r, causal=True, scale=scale, dq=dq[r:r + 1], dk=dk[r:r + 1],
                        dv=dv[r:r + 1])
    o_tok = lc.head_to_seq_relayout(o, P)
    dq_tok = lc.head_to_seq_relayout(dq, P)
    dk_tok = lc.head_to_seq_reduce(dk, P, Hkv)
    dv_tok = lc.head_to_seq_reduce(dv, P, Hkv)
    torch.cuda.synchronize()

    def head_major(t):  # token-major [P, N/P, H, D] -> [1, H, N, D]
        return np.transpose(f64_of(t).reshape(N, -1, D), (1, 0, 2))[None]

    O, L, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], scale, True)
    check_forward(head_major(o_tok), np.zeros((1, Hq, N)), O, np.zeros((1, Hq, N)), "O through the exchange")
    for name, g, ref in (("dq", dq_tok, dQ), ("dk", dk_tok, dK), ("dv", dv_tok, dV)):
        e = grad_rel_err(head_major(g), ref)
        assert e <= GRAD_REL_TOL, (name, e)
