"""Pins of the fp64 oracle against things other than itself (CPU only).

Each check below fails for a plausible slip in the oracle: a dropped scale, a
flipped mask, a wrong GQA head map, a transposed operand, a wrong sign in the
backward, a broken merge weight or a wrong relayout index.  The planted-mistake
tests at the end run the same checks against deliberately broken copies of the
oracle's pieces to show that they would catch each slip.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from long_context_attention_fwd_amd.inputs import make_qkv, sample_rows, WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# bf16 codec: facts of the bf16 format (the upper 16 bits of binary32)
# ---------------------------------------------------------------------------
BF16_CASES = [
    (0x3F800000, 0x3F80),  # 1.0
    (0x3F808000, 0x3F80),  # exact tie, kept lsb even -> down
    (0x3F818000, 0x3F82),  # exact tie, kept lsb odd -> up to even
    (0x3F808001, 0x3F81),  # just above the tie -> up
    (0x3F807FFF, 0x3F80),  # just below the tie -> down
    (0x7F7F0000, 0x7F7F),  # largest finite bf16
    (0x7F7FFFFF, 0x7F80),  # largest finite binary32 rounds to +inf
    (0x80000000, 0x8000),  # -0.0
    (0x7F800000, 0x7F80),  # +inf
    (0x7FC00000, 0x7FC0),  # quiet NaN
    (0x7F800001, 0x7FC0),  # signalling NaN comes out quiet
    (0x00010000, 0x0001),  # smallest bf16 subnormal
]


def test_bf16_codec_known_patterns():
    f32 = np.array([c[0] for c in BF16_CASES], dtype=np.uint32).view(np.float32)
    got = oracle.f32_to_bf16_bits(f32)
    want = np.array([c[1] for c in BF16_CASES], dtype=np.uint16)
    assert np.array_equal(got, want), [hex(x) for x in got]


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3E00, 0x7F80, 0x0000, 0x8000], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert list(got[:3]) == [1.0, -2.0, 0.125]
    assert got[3] == np.inf and got[4] == 0.0 and np.signbit(got[5])


def test_bf16_codec_matches_torch_rne():
    torch = pytest.importorskip("torch")
    x = _rng(7).standard_normal(10000).astype(np.float32) * np.float32(37.0)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), want)


def test_input_generator_is_seeded_bf16():
    a = make_qkv(1, 2, 1, 16, 8, seed=11)
    b = make_qkv(1, 2, 1, 16, 8, seed=11)
    assert all(np.array_equal(a[n], b[n]) for n in "qkv")
    assert a["q"].dtype == np.uint16 and a["k"].shape == (1, 1, 16, 8)
    # the generator's encoding agrees with the oracle's codec
    x = _rng(11).standard_normal((1, 2, 16, 8), dtype=np.float32)
    assert np.array_equal(a["q"], oracle.f32_to_bf16_bits(x))


def test_listing_workload_matches_pages():
    with open(os.path.join(GOLDEN, "listing_example.json")) as f:
        g = json.load(f)
    w = WORKLOADS["listing_4k"]
    assert [w.B, w.Hq, w.N, w.D] == g["shape"] and w.Hkv == w.Hq
    assert w.causal == g["is_causal"] and w.amp == 1.0
    assert w.scale == 1.0 / math.sqrt(g["shape"][3])


# ---------------------------------------------------------------------------
# forward: hand cases, closed forms, brute force, library routine
# ---------------------------------------------------------------------------
def check_single_key():
    """N = 1: the only visible key has weight 1."""
    q = np.array([0.5, -1.0, 2.0])
    k = np.array([1.5, 0.25, -0.75])
    v = np.array([3.0, -4.0, 0.125])
    s = 0.3
    O, L = oracle.attention_forward(q.reshape(1, 1, 1, 3), k.reshape(1, 1, 1, 3),
                                    v.reshape(1, 1, 1, 3), s)
    want_l = s * (0.5 * 1.5 - 1.0 * 0.25 - 2.0 * 0.75)
    return max(np.abs(O[0, 0, 0] - v).max(), abs(L[0, 0, 0] - want_l))


def check_hand_two_tokens():
    """N = 2, D = 1, scale 1: q = (1, 2), k = (0.5, -1), v = (3, 5).
    Row 0 sees key 0 only: O = 3, LSE = 0.5.  Row 1 has scores 1 and -2:
    LSE = 1 + ln(1 + e^-3), O = (3 + 5 e^-3) / (1 + e^-3)."""
    q = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    k = np.array([0.5, -1.0]).reshape(1, 1, 2, 1)
    v = np.array([3.0, 5.0]).reshape(1, 1, 2, 1)
    O, L = oracle.attention_forward(q, k, v, 1.0)
    e3 = math.exp(-3.0)
    want_o = [3.0, (3.0 + 5.0 * e3) / (1.0 + e3)]
    want_l = [0.5, 1.0 + math.log1p(e3)]
    return max(np.abs(O[0, 0, :, 0] - want_o).max(), np.abs(L[0, 0] - want_l).max())


def check_zero_query_prefix_mean(Hq=4, Hkv=2, N=37, D=5, q_pos0=0, k_pos0=0, causal=True):
    """Q = 0 makes every visible score 0: LSE_i = ln(#visible keys) and O_i is
    the mean of the visible V rows (a prefix mean when causal)."""
    v = _rng(3).standard_normal((2, Hkv, N, D))
    k = _rng(4).standard_normal((2, Hkv, N, D))
    q = np.zeros((2, Hq, N, D))
    O, L = oracle.attention_forward(q, k, v, 0.7, causal, q_pos0, k_pos0)
    G = Hq // Hkv
    err = 0.0
    for h in range(Hq):
        for i in range(N):
            if causal:
                nvis = int(np.clip(q_pos0 + i - k_pos0 + 1, 0, N))
            else:
                nvis = N
            if nvis == 0:
                assert np.all(O[:, h, i] == 0) and np.all(np.isneginf(L[:, h, i]))
                continue
            want = v[:, h // G, :nvis].mean(axis=1)
            err = max(err, np.abs(O[:, h, i] - want).max(), np.abs(L[:, h, i] - math.log(nvis)).max())
    return err


def _brute_force(q, k, v, scale, causal, q_pos0, k_pos0):
    """Pure-Python loops: scores, max, exp, sums and weighted rows."""
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Hq, Nq, D))
    L = np.full((B, Hq, Nq), -math.inf)
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            for i in range(Nq):
                sc = []
                for j in range(Nk):
                    if causal and k_pos0 + j > q_pos0 + i:
                        continue
                    dot = 0.0
                    for d in range(D):
                        dot += float(q[b, h, i, d]) * float(k[b, kh, j, d])
                    sc.append((j, scale * dot))
                if not sc:
                    continue
                m = max(x for _, x in sc)
                z = sum(math.exp(x - m) for _, x in sc)
                L[b, h, i] = m + math.log(z)
                for j, x in sc:
                    w = math.exp(x - m) / z
                    for d in range(D):
                        O[b, h, i, d] += w * float(v[b, kh, j, d])
    return O, L


@pytest.mark.parametrize("causal,q_pos0,k_pos0", [(True, 0, 0), (False, 0, 0), (True, 9, 4), (True, 0, 5)])
def test_forward_brute_force(causal, q_pos0, k_pos0):
    r = _rng(21)
    q = r.standard_normal((1, 4, 7, 3))
    k = r.standard_normal((1, 2, 9, 3))
    v = r.standard_normal((1, 2, 9, 3))
    O, L = oracle.attention_forward(q, k, v, 0.45, causal, q_pos0, k_pos0)
    Ob, Lb = _brute_force(q, k, v, 0.45, causal, q_pos0, k_pos0)
    assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    assert np.abs(L[fin] - Lb[fin]).max() < 1e-12
    assert np.abs(O - Ob).max() < 1e-12


def test_single_key():
    assert check_single_key() < 1e-15


def test_hand_two_tokens():
    assert check_hand_two_tokens() < 1e-15


@pytest.mark.parametrize("q_pos0,k_pos0,causal", [(0, 0, True), (0, 0, False), (10, 3, True), (0, 20, True)])
def test_zero_query_prefix_mean(q_pos0, k_pos0, causal):
    assert check_zero_query_prefix_mean(q_pos0=q_pos0, k_pos0=k_pos0, causal=causal) < 1e-13


def test_probability_rows_sum_to_one():
    d = make_qkv(1, 4, 2, 50, 16, seed=5)
    P = oracle.attention_probabilities(d["q"], d["k"], 0.25, causal=True)
    assert np.abs(P.sum(axis=-1) - 1.0).max() < 1e-12
    assert np.all(np.triu(P[0, 0], 1) == 0.0)        # no weight above the diagonal
    assert np.all(P >= 0)


def check_against_torch_sdpa(Hq=4, Hkv=2, N=33, D=16, causal=True, seed=6):
    """The call the glossary example makes, in float64 on the CPU."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    d = make_qkv(2, Hq, Hkv, N, D, seed=seed)
    q, k, v = (oracle.bf16_bits_to_f64(d[n]) for n in "qkv")
    O, L = oracle.attention_forward(q, k, v, 1.0 / math.sqrt(D), causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    To = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, enable_gqa=True).numpy()
    # LSE from torch's own logsumexp on the masked scaled scores
    G = Hq // Hkv
    s = (tq @ tk.repeat_interleave(G, dim=1).transpose(-1, -2)) / math.sqrt(D)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    TL = torch.logsumexp(s, dim=-1).numpy()
    return max(np.abs(O - To).max(), np.abs(L - TL).max())


@pytest.mark.parametrize("Hq,Hkv,N,D,causal", [(4, 2, 33, 16, True), (4, 4, 20, 8, False), (8, 1, 17, 64, True)])
def test_forward_matches_torch_sdpa(Hq, Hkv, N, D, causal):
    assert check_against_torch_sdpa(Hq, Hkv, N, D, causal) < 1e-12


# ---------------------------------------------------------------------------
# merge: the ring result equals full attention over the whole sequence
# ---------------------------------------------------------------------------
def check_merge_partition(seed=8, N=40, Nk=57, n_parts=4, q_pos0=10, with_empty=True):
    r = _rng(seed)
    q = r.standard_normal((1, 2, N, 6))
    k = r.standard_normal((1, 1, Nk, 6))
    v = r.standard_normal((1, 1, Nk, 6))
    O, L = oracle.attention_forward(q, k, v, 0.4, True, q_pos0, 0)
    cuts = np.sort(r.choice(np.arange(1, Nk), size=n_parts - 1, replace=False))
    if with_empty:
        cuts = np.concatenate([cuts, [Nk]])          # an empty last part
    bounds = np.concatenate([[0], cuts, [Nk]])
    Os, Ls = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b > a:
            o, l = oracle.attention_forward(q, k[:, :, a:b], v[:, :, a:b], 0.4, True, q_pos0, int(a))
        else:
            o, l = np.zeros_like(O), np.full_like(L, -np.inf)
        Os.append(o)
        Ls.append(l)
    Om, Lm = oracle.lse_merge(np.stack(Os), np.stack(Ls))
    return max(np.abs(Om - O).max(), np.abs(Lm - L).max())


@pytest.mark.parametrize("seed,n_parts", [(8, 2), (9, 3), (10, 5)])
def test_merge_equals_full_attention(seed, n_parts):
    assert check_merge_partition(seed=seed, n_parts=n_parts) < 1e-12


def test_merge_all_empty_rows_stay_zero():
    o = np.zeros((3, 2, 4))
    l = np.full((3, 2), -np.inf)
    o[1, 1] = 5.0
    l[1, 1] = 0.3
    Om, Lm = oracle.lse_merge(o, l)
    assert np.all(Om[0] == 0) and np.isneginf(Lm[0]).all()
    assert np.allclose(Om[1], 5.0) and Lm[1] == pytest.approx(0.3)
    assert np.isfinite(Om).all()


# ---------------------------------------------------------------------------
# backward: library autograd and central finite differences
# ---------------------------------------------------------------------------
def check_backward_vs_torch(Hq=4, Hkv=2, N=24, D=8, causal=True, seed=12):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    d = make_qkv(1, Hq, Hkv, N, D, seed=seed, with_do=True)
    q, k, v, do = (oracle.bf16_bits_to_f64(d[n]) for n in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(D)
    _, _, dQ, dK, dV = oracle.attention_backward(q, k, v, do, s, causal)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, enable_gqa=True)
    (o * torch.from_numpy(do)).sum().backward()
    return max(np.abs(dQ - tq.grad.numpy()).max(), np.abs(dK - tk.grad.numpy()).max(),
               np.abs(dV - tv.grad.numpy()).max())


@pytest.mark.parametrize("Hq,Hkv,causal", [(4, 2, True), (2, 2, False), (4, 1, True)])
def test_backward_matches_torch_autograd(Hq, Hkv, causal):
    assert check_backward_vs_torch(Hq, Hkv, causal=causal) < 1e-12


def check_backward_finite_differences(loss="dot", seed=13, n_probe=6):
    """Central differences (h = 1e-6) of L = sum(O * dO), or of the glossary
    example's L = mean(O^2) whose dO is 2 O / numel."""
    r = _rng(seed)
    q = r.standard_normal((1, 2, 9, 4))
    k = r.standard_normal((1, 1, 9, 4))
    v = r.standard_normal((1, 1, 9, 4))
    s = 0.5
    O, _ = oracle.attention_forward(q, k, v, s)
    do = r.standard_normal(O.shape) if loss == "dot" else 2.0 * O / O.size

    def L(qq, kk, vv):
        o, _ = oracle.attention_forward(qq, kk, vv, s)
        return float((o * do).sum()) if loss == "dot" else float((o ** 2).mean())

    _, _, dQ, dK, dV = oracle.attention_backward(q, k, v, do, s)
    worst = 0.0
    h = 1e-6
    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        for _ in range(n_probe):
            idx = tuple(r.integers(0, n) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (L(args_p["q"], args_p["k"], args_p["v"]) - L(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            worst = max(worst, abs(fd - g[idx]) / max(1e-3, abs(g[idx])))
    return worst


@pytest.mark.parametrize("loss", ["dot", "mean_square"])
def test_backward_finite_differences(loss):
    assert check_backward_finite_differences(loss) < 1e-6


def test_backward_sampled_matches_full():
    d = make_qkv(1, 4, 2, 70, 8, seed=14, with_do=True)
    s = 1.0 / math.sqrt(8)
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s)
    rows = np.array([0, 5, 31, 69])
    sq, sk, sv = oracle.attention_backward_sampled(d["q"], d["k"], d["v"], d["do"], s, rows, rows)
    assert np.abs(sq - dQ[:, :, rows]).max() < 1e-12
    assert np.abs(sk - dK[:, :, rows]).max() < 1e-12
    assert np.abs(sv - dV[:, :, rows]).max() < 1e-12


def test_backward_row_support_matches_full_with_masked_do():
    d = make_qkv(1, 4, 2, 90, 8, seed=16, with_do=True)
    support = np.array([0, 3, 40, 41, 89])
    do = oracle.bf16_bits_to_f64(d["do"])
    mask = np.zeros(90, dtype=bool)
    mask[support] = True
    do[:, :, ~mask] = 0.0
    s = 1.0 / math.sqrt(8)
    _, _, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], do, s)
    rq, rk, rv = oracle.attention_backward_row_support(d["q"], d["k"], d["v"], do, s, support)
    assert np.abs(rq - dQ[:, :, support]).max() < 1e-12
    assert np.abs(rk - dK).max() < 1e-12 and np.abs(rv - dV).max() < 1e-12
    with pytest.raises(ValueError):
        oracle.attention_backward_row_support(d["q"], d["k"], d["v"], d["do"], s, support)


# ---------------------------------------------------------------------------
# backward of one ring step: gradients through one KV block
# ---------------------------------------------------------------------------
def check_block_backward_vs_torch(Hq=4, Hkv=2, N=30, D=8, causal=True, shards=(0, 11, 30), blocks=(0, 7, 19, 30),
                                  seed=21):
    """Query shards against KV blocks, each block a separate leaf of torch's
    autograd over SDPA with an explicit mask of global positions: the oracle's
    per-(shard, block) gradients must sum to torch's gradients of each shard's
    loss, and a block's dK/dV from one shard must equal torch's gradient of
    that shard's loss with respect to that block."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    d = make_qkv(1, Hq, Hkv, N, D, seed=seed, with_do=True)
    q, k, v, do = (oracle.bf16_bits_to_f64(d[n]) for n in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(D)
    G = Hq // Hkv
    worst = 0.0
    for a, b in zip(shards[:-1], shards[1:]):
        O, L = oracle.attention_forward(q, k, v, s, causal, rows=np.arange(a, b))
        Dv = np.einsum("bhnd,bhnd->bhn", do[:, :, a:b], O)
        tq = torch.from_numpy(q[:, :, a:b].copy()).requires_grad_()
        tk = [torch.from_numpy(k[:, :, c:e].copy()).requires_grad_() for c, e in zip(blocks[:-1], blocks[1:])]
        tv = [torch.from_numpy(v[:, :, c:e].copy()).requires_grad_() for c, e in zip(blocks[:-1], blocks[1:])]
        kk = torch.cat(tk, dim=2).repeat_interleave(G, dim=1)
        vv = torch.cat(tv, dim=2).repeat_interleave(G, dim=1)
        mask = None
        if causal:
            mask = torch.arange(N)[None, :] <= torch.arange(a, b)[:, None]
        o = F.scaled_dot_product_attention(tq, kk, vv, attn_mask=mask, scale=s)
        (o * torch.from_numpy(do[:, :, a:b].copy())).sum().backward()
        dq_sum = np.zeros_like(q[:, :, a:b])
        for i, (c, e) in enumerate(zip(blocks[:-1], blocks[1:])):
            bq, bk, bv = oracle.attention_backward_block(q[:, :, a:b], k[:, :, c:e], v[:, :, c:e], do[:, :, a:b], L,
                                                         Dv, s, causal, q_pos0=a, k_pos0=c)
            dq_sum += bq
            worst = max(worst, np.abs(bk - tk[i].grad.numpy()).max(), np.abs(bv - tv[i].grad.numpy()).max())
        worst = max(worst, np.abs(dq_sum - tq.grad.numpy()).max())
    return worst


@pytest.mark.parametrize("Hq,Hkv,causal", [(4, 2, True), (2, 2, False), (4, 1, True)])
def test_block_backward_matches_torch_autograd(Hq, Hkv, causal):
    assert check_block_backward_vs_torch(Hq, Hkv, causal=causal) < 1e-12


def test_block_backward_sums_to_full_backward():
    """Every (query shard, KV block) pair: dQ summed over blocks and dK, dV
    summed over shards give attention_backward's gradients."""
    d = make_qkv(2, 4, 2, 77, 8, seed=22, with_do=True)
    q, k, v, do = (oracle.bf16_bits_to_f64(d[n]) for n in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(8)
    O, L, dQ, dK, dV = oracle.attention_backward(q, k, v, do, s)
    Dv = np.einsum("bhnd,bhnd->bhn", do, O)
    cuts = [0, 13, 40, 64, 77]
    gq, gk, gv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for a, b in zip(cuts[:-1], cuts[1:]):          # query shard
        for c, e in zip(cuts[:-1], cuts[1:]):      # KV block
            bq, bk, bv = oracle.attention_backward_block(q[:, :, a:b], k[:, :, c:e], v[:, :, c:e], do[:, :, a:b],
                                                         L[:, :, a:b], Dv[:, :, a:b], s, True, a, c)
            if c > b - 1:                          # block entirely after the shard: no gradient
                assert not bq.any() and not bk.any() and not bv.any()
            gq[:, :, a:b] += bq
            gk[:, :, c:e] += bk
            gv[:, :, c:e] += bv
    assert np.abs(gq - dQ).max() < 1e-12
    assert np.abs(gk - dK).max() < 1e-12 and np.abs(gv - dV).max() < 1e-12


def test_block_backward_whole_sequence_is_full_backward():
    d = make_qkv(1, 2, 1, 40, 8, seed=23, with_do=True)
    s = 0.3
    O, L, dQ, dK, dV = oracle.attention_backward(d["q"], d["k"], d["v"], d["do"], s)
    Dv = np.einsum("bhnd,bhnd->bhn", oracle.bf16_bits_to_f64(d["do"]), O)
    bq, bk, bv = oracle.attention_backward_block(d["q"], d["k"], d["v"], d["do"], L, Dv, s)
    assert np.abs(bq - dQ).max() < 1e-12 and np.abs(bk - dK).max() < 1e-12 and np.abs(bv - dV).max() < 1e-12


def test_planted_block_backward_mistakes_are_caught(monkeypatch):
    orig = oa.attention_backward_block

    def local_lse(q, k, v, do, lse, dv, scale, causal=True, q_pos0=0, k_pos0=0):
        # the block's own LSE instead of the global one
        _, lb = oa.attention_forward(q, k, v, scale, causal, q_pos0, k_pos0)
        return orig(q, k, v, do, lb, dv, scale, causal, q_pos0, k_pos0)

    def shifted(q, k, v, do, lse, dv, scale, causal=True, q_pos0=0, k_pos0=0):
        return orig(q, k, v, do, lse, dv, scale, causal, q_pos0, k_pos0 + 1)   # off-by-one block position

    for bad in (local_lse, shifted):
        monkeypatch.setattr(oracle, "attention_backward_block", bad)
        assert check_block_backward_vs_torch() > 1e-3


# ---------------------------------------------------------------------------
# relayout: a transpose of the flattened token and head indices
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("P,N,H,D", [(8, 64, 32, 4), (8, 64, 8, 4), (4, 12, 4, 2), (2, 6, 6, 3)])
def test_relayout_is_transpose_and_round_trips(P, N, H, D):
    x = _rng(15).integers(0, 1 << 16, size=(P, N // P, H, D), dtype=np.uint16)
    y = oracle.seq_to_head(x, P)
    want = np.transpose(x.reshape(N, H, D), (1, 0, 2)).reshape(P, H // P, N, D)
    assert np.array_equal(y, want)
    assert np.array_equal(oracle.head_to_seq(y, P), x)


@pytest.mark.parametrize("P,N,H,D", [(8, 64, 4, 4), (8, 64, 1, 4), (4, 12, 2, 2), (8, 64, 2, 8)])
def test_relayout_replicates_shared_heads(P, N, H, D):
    """H < P: every head goes to the P/H ranks after one another (np.repeat
    of the transpose), i.e. rank r gets the key/value head its query heads
    h = r*(Hq/P) .. read under the grouped-query map h // (Hq/H)."""
    x = _rng(16).integers(0, 1 << 16, size=(P, N // P, H, D), dtype=np.uint16)
    y = oracle.seq_to_head(x, P)
    want = np.repeat(np.transpose(x.reshape(N, H, D), (1, 0, 2)), P // H, axis=0)[:, None]
    assert np.array_equal(y, want)
    Hq = 4 * P  # 4 query heads per rank
    for r in range(P):
        assert all((r * 4 + j) // (Hq // H) == r // (P // H) for j in range(4))


def adjoint_gap(P, N, H, D, seed=17):
    r = _rng(seed)
    x = r.standard_normal((P, N // P, H, D))
    y = r.standard_normal((P, max(1, H // P), N, D))
    lhs = float((oracle.seq_to_head(x, P) * y).sum())
    rhs = float((x * oracle.head_to_seq_sum(y, P, H)).sum())
    return abs(lhs - rhs) / max(1.0, abs(lhs))


@pytest.mark.parametrize("P,N,H,D", [(8, 64, 4, 4), (8, 64, 1, 4), (4, 12, 8, 2), (2, 6, 6, 3)])
def test_head_to_seq_sum_is_adjoint_of_seq_to_head(P, N, H, D):
    """<seq_to_head(x), y> = <x, head_to_seq_sum(y)> for all x, y: the sum is
    the transpose of the (replicating) exchange, which is what the gradient
    of a shared head needs; for H >= P it is the inverse relayout."""
    assert adjoint_gap(P, N, H, D) < 1e-9
    if H >= P:
        y = _rng(19).standard_normal((P, H // P, N, D))
        assert np.array_equal(oracle.head_to_seq_sum(y, P, H), oracle.head_to_seq(y, P))


def test_head_to_seq_sum_planted_mistake_is_caught(monkeypatch):
    """Replicas summed from the wrong ranks (interleaved r % H instead of
    r // (P/H)) must break the adjoint identity."""
    def bad(y, P, H):
        y = np.asarray(y, dtype=np.float64)
        T = y.shape[2] // P
        out = np.zeros((P, T, H, y.shape[3]))
        for p in range(P):
            for h in range(H):
                for i in range(P // H):
                    out[p, :, h] += y[i * H + h, 0, p * T:(p + 1) * T]
        return out

    assert adjoint_gap(8, 16, 2, 2) < 1e-9
    monkeypatch.setattr(oracle, "head_to_seq_sum", bad)
    assert adjoint_gap(8, 16, 2, 2) > 1e-6


def test_sample_rows_contains_boundaries():
    r = sample_rows(32768, seed=3, count=256, block=8192)
    assert len(r) == 256 and len(np.unique(r)) == 256
    for must in (0, 127, 128, 8191, 8192, 16383, 16384, 24575, 24576, 32767):
        assert must in r


# ---------------------------------------------------------------------------
# planted mistakes: each broken copy must fail at least one of the checks
# ---------------------------------------------------------------------------
def _bad_scores_no_scale(q_rows, k, scale, causal, q_pos, k_pos0=0):
    return _orig_scores(q_rows, k, 1.0, causal, q_pos, k_pos0)


def _bad_scores_flipped_mask(q_rows, k, scale, causal, q_pos, k_pos0=0):
    s = _orig_scores(q_rows, k, scale, False, q_pos, k_pos0)
    if causal:
        kp = np.int64(k_pos0) + np.arange(np.asarray(k).shape[0])
        s[kp[None, :] < np.asarray(q_pos)[:, None]] = -np.inf
    return s


def _bad_scores_strict_mask(q_rows, k, scale, causal, q_pos, k_pos0=0):
    s = _orig_scores(q_rows, k, scale, causal, q_pos, k_pos0)
    if causal:
        kp = np.int64(k_pos0) + np.arange(np.asarray(k).shape[0])
        s[kp[None, :] == np.asarray(q_pos)[:, None]] = -np.inf
    return s


_orig_scores = oa.scores


def _all_forward_checks():
    errs = [check_single_key(), check_hand_two_tokens(), check_zero_query_prefix_mean(),
            check_zero_query_prefix_mean(q_pos0=10, k_pos0=3)]
    try:
        errs.append(check_against_torch_sdpa())
    except Exception:
        errs.append(np.inf)
    return max(errs)


@pytest.mark.parametrize("bad", [_bad_scores_no_scale, _bad_scores_flipped_mask, _bad_scores_strict_mask])
def test_planted_forward_mistakes_are_caught(monkeypatch, bad):
    assert _all_forward_checks() < 1e-12
    monkeypatch.setattr(oa, "scores", bad)
    assert _all_forward_checks() > 1e-3


def test_planted_gqa_map_mistake_is_caught(monkeypatch):
    # a head map h % Hkv instead of h // G (interleaved instead of grouped)
    orig = oa.attention_forward

    def bad(q, k, v, scale, causal=True, q_pos0=0, k_pos0=0, rows=None):
        q = oa._as_f64(q)
        Hq, Hkv = q.shape[1], np.asarray(k).shape[1]
        G = Hq // Hkv
        perm = [(h % Hkv) * G + h // Hkv for h in range(Hq)]
        inv = np.argsort(perm)
        O, L = orig(q[:, perm], k, v, scale, causal, q_pos0, k_pos0, rows)
        return O[:, inv], L[:, inv]

    monkeypatch.setattr(oracle, "attention_forward", bad)
    assert check_against_torch_sdpa(Hq=4, Hkv=2) > 1e-3


def test_planted_merge_mistake_is_caught(monkeypatch):
    def bad(o_parts, lse_parts):            # forgets to renormalise by the total
        lse_parts = np.asarray(lse_parts)
        M = lse_parts.max(axis=0)
        w = np.exp(lse_parts - M[None])
        return (w[..., None] * o_parts).sum(axis=0), M

    monkeypatch.setattr(oracle, "lse_merge", bad)
    assert check_merge_partition() > 1e-3


def test_planted_backward_mistakes_are_caught(monkeypatch):
    orig = oa.attention_backward

    def bad_sign(q, k, v, do, scale, causal=True):
        O, L, dQ, dK, dV = orig(q, k, v, do, scale, causal)
        return O, L, dQ, -dK, dV                 # a sign slip in dS^T Q

    def bad_transpose(q, k, v, do, scale, causal=True):
        O, L, dQ, dK, dV = orig(q, k, v, do, scale, causal)
        return O, L, dQ, dK, dV[:, :, ::-1]      # rows of dV attributed to the wrong keys

    for bad in (bad_sign, bad_transpose):
        monkeypatch.setattr(oracle, "attention_backward", bad)
        assert check_backward_finite_differences() > 1e-3
        assert check_backward_vs_torch() > 1e-3
