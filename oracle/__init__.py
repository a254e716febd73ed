"""fp64 CPU oracle for causal scaled-dot-product attention on one GPU's share.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code with the HIP library
(no kernels, headers, helpers or constant tables); its only common ground with
the GPU side is the seeded input generator, which holds no attention arithmetic.

Every function is the plain definition of the operation written out in float64
with NumPy; see ``oracle/attention.py`` for the citations.
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    f32_to_bf16_bits,
    scores,
    attention_forward,
    attention_probabilities,
    lse_merge,
    attention_backward,
    attention_backward_sampled,
    attention_backward_row_support,
    attention_backward_block,
    seq_to_head,
    head_to_seq,
    head_to_seq_sum,
)
