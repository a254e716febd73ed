"""attn_bwd_noalloc (the library's own per-GPU scratch instead of a caller
workspace) against attn_bwd on the same inputs, through the C ABI: three calls
in a row, each smaller than the one before, so that later calls run over
scratch left by bigger ones.  The same kernels run either way, so the
gradients must agree bit for bit."""

import math

import numpy as np
import pytest

import long_context_attention_fwd_amd as lc
from long_context_attention_fwd_amd.inputs import make_qkv

from gpu_util import poisoned, to_dev

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, N, D): the 32K Ulysses shard (Dv + per-head dK/dV partials,
# 128.5 MiB of the 160 MiB scratch), a smaller grouped-query case, a D = 64
# case without partials
CASES = [(1, 4, 1, 32768, 128), (1, 8, 2, 3000, 128), (2, 4, 4, 700, 64)]


def test_bwd_noalloc_matches_attn_bwd(gpu):
    import torch
    for i, (B, Hq, Hkv, N, D) in enumerate(CASES):
        print(f"case {i}: B={B} Hq={Hq} Hkv={Hkv} N={N} D={D}", flush=True)
        d = make_qkv(B, Hq, Hkv, N, D, seed=4000 + i, with_do=True)
        q, k, v, do = (to_dev(d[n]) for n in ("q", "k", "v", "do"))
        s = float(np.float32(1.0 / math.sqrt(D)))
        o, lse = lc.attn_fwd(q, k, v, causal=True, scale=s)
        # attn_bwd with its minimal workspace (the recomputing dQ pass, the
        # kernels the allocation-free form runs)
        ref = lc.attn_bwd(q, k, v, o, do, lse, causal=True, scale=s, stored_ds=False)
        got = tuple(poisoned(tuple(t.shape), torch.bfloat16) for t in (q, k, v))
        lc.attn_bwd_noalloc(q, k, v, o, do, lse, causal=True, scale=s, dq=got[0], dk=got[1], dv=got[2])
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g.view(torch.int16), r.view(torch.int16)), f"case {i}: {name} differs from attn_bwd"
