"""Host logic of the ring schedules (CPU only): every causal (query chunk,
key chunk) pair is visited exactly once per rank, and the zigzag sharding
gives every rank the same work at every step."""

import pytest

from long_context_attention_fwd_amd.ring import rank_chunks, ring_schedule


@pytest.mark.parametrize("scheme", ["contiguous", "zigzag"])
@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_chunks_partition_the_sequence(scheme, P):
    owned = sorted(c for r in range(P) for c in rank_chunks(r, P, scheme))
    assert owned == list(range(2 * P))


@pytest.mark.parametrize("scheme", ["contiguous", "zigzag"])
@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_every_visible_pair_once(scheme, P, causal):
    for r in range(P):
        mine = rank_chunks(r, P, scheme)
        seen = []
        for step, src, qi, ki in ring_schedule(r, P, scheme, causal):
            assert src == (r - step) % P
            seen.append((mine[qi], rank_chunks(src, P, scheme)[ki]))
        want = sorted((qc, kc) for qc in mine for kc in range(2 * P) if not causal or kc <= qc)
        assert sorted(seen) == want


def work(P, scheme, C=1):
    """Causal score entries per (rank, step): a key chunk before the query
    chunk is C*C, the same chunk C*(C+1)/2."""
    w = [[0] * P for _ in range(P)]
    for r in range(P):
        mine = rank_chunks(r, P, scheme)
        for step, src, qi, ki in ring_schedule(r, P, scheme):
            qc, kc = mine[qi], rank_chunks(src, P, scheme)[ki]
            w[r][step] += C * C if kc < qc else C * (C + 1) // 2
    return w


@pytest.mark.parametrize("P", [2, 4, 8])
def test_zigzag_balances_every_step(P):
    C = 64
    z = work(P, "zigzag", C)
    for step in range(P):
        assert len({z[r][step] for r in range(P)}) == 1
    c = work(P, "contiguous", C)
    total = sum(map(sum, z))
    assert total == sum(map(sum, c)) == (2 * P * C) * (2 * P * C + 1) // 2
    # the ring waits for the busiest rank at every step
    crit_z = sum(max(z[r][s] for r in range(P)) for s in range(P))
    crit_c = sum(max(c[r][s] for r in range(P)) for s in range(P))
    assert crit_z * P == total
    assert crit_c > crit_z
