"""GPU parity of partial attention + attn_partial_merge (the ring form)."""

import math

import numpy as np
import pytest

import oracle
import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import WORKLOADS, make_qkv, make_workload_inputs, sample_rows

from gpu_util import check_forward, f64_of, poisoned, to_dev

pytestmark = pytest.mark.gpu


def ring_partials(q, k, v, bounds, scale, part_dtype):
    """One attn_fwd per KV block [a, b) with its global key offset."""
    import torch
    B, H, N, D = q.shape
    n = len(bounds) - 1
    o_parts = poisoned((n, B, H, N, D), part_dtype)
    lse_parts = poisoned((n, B, H, N), torch.float32)
    for i in range(n):
        a, b = bounds[i], bounds[i + 1]
        lc.attn_fwd(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), causal=True, k_pos0=a, scale=scale,
                    out_dtype=part_dtype, o=o_parts[i], lse=lse_parts[i])
    return o_parts, lse_parts


@pytest.mark.parametrize("N,bounds,G", [(300, [0, 100, 200, 300], 1), (517, [0, 64, 65, 300, 517], 4),
                                        (256, [0, 256], 1), (1024, [0, 128, 512, 1000, 1024], 2)])
@pytest.mark.parametrize("f32", [True, False])
def test_merge_small(gpu, N, bounds, G, f32):
    import torch
    d = make_qkv(1, 2 * G, 2, N, 128, seed=40 + N)
    q, k, v = (to_dev(d[x]) for x in "qkv")
    s = float(np.float32(1 / math.sqrt(128)))
    dt = torch.float32 if f32 else torch.bfloat16
    o_parts, lse_parts = ring_partials(q, k, v, bounds, s, dt)
    o = poisoned(tuple(q.shape), torch.bfloat16)
    lse = poisoned(tuple(q.shape[:3]), torch.float32)
    lc.attn_partial_merge(o_parts, lse_parts, o=o, lse=lse)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], s, True)
    check_forward(f64_of(o), f64_of(lse), O, L, f"merge N={N} f32={f32}")
    # the oracle's merge of the GPU's own fp32 partials agrees as well
    if f32:
        Om, Lm = oracle.lse_merge(f64_of(o_parts), f64_of(lse_parts))
        assert np.abs(f64_of(o) - Om).max() < 1e-2 and np.abs(f64_of(lse) - Lm).max() < 1e-5


def test_merge_all_parts_empty(gpu):
    import torch
    o_parts = torch.zeros(3, 1, 2, 10, 64, device="cuda")
    lse_parts = torch.full((3, 1, 2, 10), float("-inf"), device="cuda")
    o, lse = lc.attn_partial_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_ring_blocks_32k(gpu):
    """N = 32768, H = 8, D = 128: four 8192-key partials (fp32) merged, against
    the GPU's full forward on every row and the oracle on 256 rows x 8 heads."""
    import torch
    w = WORKLOADS["ring_blocks_32k"]
    d = make_workload_inputs(w)
    q, k, v = (to_dev(d[x]) for x in "qkv")
    blk = w.N // w.kv_blocks
    bounds = [i * blk for i in range(w.kv_blocks + 1)]
    o_parts, lse_parts = ring_partials(q, k, v, bounds, w.scale, torch.float32)
    o, lse = lc.attn_partial_merge(o_parts, lse_parts)
    of, lf = lc.attn_fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    # merged vs the GPU's full forward, every row
    diff = (o.float() - of.float()).abs().max().item()
    ldiff = (lse - lf).abs().max().item()
    assert diff <= 1e-2 and ldiff <= 1e-3, (diff, ldiff)
    # both vs the oracle on the sampled rows
    rows = sample_rows(w.N, w.seed, w.sampled_rows, block=blk)
    idx = torch.from_numpy(rows).cuda()
    O, L = oracle.attention_forward(d["q"], d["k"], d["v"], w.scale, True, rows=rows)
    check_forward(f64_of(o[:, :, idx]), f64_of(lse[:, :, idx]), O, L, "ring merged")
    check_forward(f64_of(of[:, :, idx]), f64_of(lf[:, :, idx]), O, L, "ring full")
    # the oracle's merge of its own per-block partials on those rows (invariant)
    parts = [oracle.attention_forward(d["q"], d["k"][:, :, a:b], d["v"][:, :, a:b], w.scale, True, 0, a, rows=rows)
             for a, b in zip(bounds[:-1], bounds[1:])]
    Om, Lm = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.abs(Om - O).max() < 1e-12 and np.abs(Lm - L).max() < 1e-12


def test_ring_blocks_32k_grouped_partials(gpu):
    """The four 8192-key partials of the ring workload from one
    attn_fwd_accumulate_group launch (the bench step's ring leg): bit-identical
    to four attn_fwd calls, and merged within the gates of the full forward."""
    import torch
    w = WORKLOADS["ring_blocks_32k"]
    d = make_workload_inputs(w)
    q, k, v = (to_dev(d[x]) for x in "qkv")
    blk = w.N // w.kv_blocks
    bounds = [i * blk for i in range(w.kv_blocks + 1)]
    o_ref, lse_ref = ring_partials(q, k, v, bounds, w.scale, torch.float32)
    o_parts = poisoned(tuple(o_ref.shape), torch.float32)
    lse_parts = poisoned(tuple(lse_ref.shape), torch.float32)
    lc.attn_fwd_accumulate_group(
        [dict(q=q, k=k[:, :, a:b].contiguous(), v=v[:, :, a:b].contiguous(), o_acc=o_parts[i], lse_acc=lse_parts[i],
              first=True, k_pos0=a) for i, (a, b) in enumerate(zip(bounds[:-1], bounds[1:]))], scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_parts.view(torch.int32), o_ref.view(torch.int32))
    assert torch.equal(lse_parts.view(torch.int32), lse_ref.view(torch.int32))
