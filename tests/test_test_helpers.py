"""CPU checks of the test-side helpers that drive the oracle (no GPU)."""

import numpy as np

import oracle
from long_context_attention_fwd_amd.inputs import make_qkv

from gpu_util import oracle_full_lse_delta


def test_threaded_full_lse_delta_equals_direct_oracle():
    """The (head, row chunk) thread pool gives exactly the oracle's own LSE
    and Dv of a direct full call (rows are independent; same arithmetic)."""
    d = make_qkv(1, 4, 2, 300, 64, seed=5, with_do=True)
    f = {n: oracle.bf16_bits_to_f64(d[n]) for n in d}
    s = 0.125
    L, Dv = oracle_full_lse_delta(f["q"], f["k"], f["v"], f["do"], s, workers=3, chunk=64)
    O_ref, L_ref = oracle.attention_forward(f["q"], f["k"], f["v"], s, True)
    assert np.allclose(L, L_ref, rtol=0, atol=1e-12)
    assert np.allclose(Dv, np.einsum("bhnd,bhnd->bhn", f["do"], O_ref), rtol=0, atol=1e-12)
