"""Ring schedules over the library's calls (host-side ordering only; every
piece of arithmetic runs in the library's kernels).

Ring attention ("Context Parallelism", Ultralytics glossary, section "So
funktioniert Kontextparallelität"): every rank keeps its queries and, over P
steps, receives every rank's key/value block; the partial attention of its
queries against each block is merged into a running result.  Here the
sequence is cut into 2P chunks of C tokens and a rank holds two of them:

* ``contiguous``: rank r holds chunks 2r and 2r+1.  Under the causal mask
  rank P-1 attends to every earlier chunk and rank 0 to its own only, so the
  ring's steps wait for the busiest rank.
* ``zigzag``: rank r holds chunks r and 2P-1-r, one early and one late, so
  every rank does the same causal work at every step (the load-balanced
  sharding named as the ring's next step).

A step's calls are the (query chunk, key chunk) pairs with at least one
visible key; each is one ``attn_fwd_accumulate`` with the chunks' global
positions, so the kernel's own mask handles the rest.
"""

from __future__ import annotations

SCHEMES = ("contiguous", "zigzag")


def rank_chunks(rank: int, P: int, scheme: str = "zigzag") -> tuple[int, int]:
    """The two chunk indices (of 2P) that rank ``rank`` holds, in order."""
    if not 0 <= rank < P:
        raise ValueError(f"rank {rank} out of [0, {P})")
    if scheme == "zigzag":
        return (rank, 2 * P - 1 - rank)
    if scheme == "contiguous":
        return (2 * rank, 2 * rank + 1)
    raise ValueError(f"scheme must be one of {SCHEMES}")


def ring_schedule(rank: int, P: int, scheme: str = "zigzag", causal: bool = True):
    """The calls of one rank's ring in order: tuples (step, src, qi, ki) --
    at ``step`` the rank holds the key/value chunks of rank ``src`` =
    (rank - step) mod P, and query chunk ``qi`` (0 or 1 of its own pair)
    attends to key chunk ``ki`` of src's pair.  Pairs whose keys all lie
    after the queries (causal) are left out."""
    mine = rank_chunks(rank, P, scheme)
    calls = []
    for step in range(P):
        src = (rank - step) % P
        theirs = rank_chunks(src, P, scheme)
        for qi, qc in enumerate(mine):
            for ki, kc in enumerate(theirs):
                if not causal or kc <= qc:
                    calls.append((step, src, qi, ki))
    return calls


def ring_groups(rank: int, P: int, scheme: str = "zigzag", causal: bool = True):
    """The launches of one rank's ring when the calls of a step that read the
    same key/value chunk go out together: a list of groups in launch order,
    each a list of (index into ring_schedule's calls, call).  A group holds at
    most one call per query chunk (their running results are distinct, so the
    calls are independent), and every query chunk's calls keep their order."""
    calls = ring_schedule(rank, P, scheme, causal)
    groups = []
    for step in range(P):
        for ki in (0, 1):
            g = [(i, c) for i, c in enumerate(calls) if c[0] == step and c[3] == ki]
            if g:
                groups.append(g)
    return groups


def ring_forward(q_chunks, kv_chunks, rank: int, P: int, C: int, *, o_acc, lse_acc, o_final=None,
                 scheme: str = "zigzag", causal: bool = True, scale: float | None = None, steps=None,
                 streams=None, grouped: bool = False, n_splits: int = 1, workspaces=None):
    """Run rank ``rank``'s ring on this GPU.

    q_chunks: the rank's two query chunks, [B, Hq, C, D] bf16 each.
    kv_chunks(src): ((k, v), (k, v)) of rank src's two chunks, [B, Hkv, C, D].
    o_acc, lse_acc: per query chunk, the fp32 running (O, LSE); o_final (per
    query chunk, optional) receives the bf16 O on that chunk's last call.
    steps: restrict to these ring steps (for timing one step); None = all.
    streams: two torch streams (default priority); the calls of query chunk
    i go to streams[i], so the two chunks' calls of a step run side by side
    (each chunk's calls stay in order: they update the same running result).
    The caller's stream waits for both at the end.
    grouped: the calls of a step that read the same key/value chunk (one per
    query chunk: independent running results) go out as one
    ``attn_fwd_accumulate_group`` launch instead (streams is then unused).
    n_splits > 1 (grouped only): each call's keys in that many ranges side by
    side, merged into the running result (``attn_fwd_accumulate_group_split``;
    ``attn_fwd_split_suggest`` gives the library's choice); workspaces: one
    uint8 tensor per call of a group, each of at least
    ``attn_fwd_accumulate_workspace_size(B, Hq, C, D, n_splits)`` bytes
    (allocated per call when None).
    """
    import torch

    from . import attn_fwd_accumulate

    calls = ring_schedule(rank, P, scheme, causal)
    mine = rank_chunks(rank, P, scheme)
    last = {qi: max(i for i, c in enumerate(calls) if c[2] == qi) for qi in (0, 1)}
    first_call = {qi: min(i for i, c in enumerate(calls) if c[2] == qi) for qi in (0, 1)}
    if grouped:
        from . import attn_fwd_accumulate_group
        for g in ring_groups(rank, P, scheme, causal):
            if steps is not None and g[0][1][0] not in steps:
                continue
            group = []
            for i, (step, src, qi, ki) in g:
                k, v = kv_chunks(src)[ki]
                kc = rank_chunks(src, P, scheme)[ki]
                group.append(dict(q=q_chunks[qi], k=k, v=v, o_acc=o_acc[qi], lse_acc=lse_acc[qi],
                                  first=(i == first_call[qi]), q_pos0=mine[qi] * C, k_pos0=kc * C,
                                  o_final=(o_final[qi] if o_final is not None and i == last[qi] else None)))
            if n_splits > 1:
                from . import attn_fwd_accumulate_group_split
                if workspaces is not None:
                    for slot, c in enumerate(group):
                        c["workspace"] = workspaces[slot]
                attn_fwd_accumulate_group_split(group, n_splits=n_splits, causal=causal, scale=scale)
            else:
                attn_fwd_accumulate_group(group, causal=causal, scale=scale)
        return
    if n_splits > 1:
        raise ValueError("n_splits > 1 needs grouped=True")
    caller = torch.cuda.current_stream(q_chunks[0].device)
    if streams is not None:
        fork = torch.cuda.Event()
        fork.record(caller)
        for st in streams:
            st.wait_event(fork)
    for i, (step, src, qi, ki) in enumerate(calls):
        if steps is not None and step not in steps:
            continue
        k, v = kv_chunks(src)[ki]
        kc = rank_chunks(src, P, scheme)[ki]
        with torch.cuda.stream(streams[qi] if streams is not None else caller):
            attn_fwd_accumulate(q_chunks[qi], k, v, o_acc[qi], lse_acc[qi], first=(i == first_call[qi]),
                                causal=causal, scale=scale, q_pos0=mine[qi] * C, k_pos0=kc * C,
                                o_final=(o_final[qi] if o_final is not None and i == last[qi] else None))
    if streams is not None:
        for st in streams:
            join = torch.cuda.Event()
            join.record(st)
            caller.wait_event(join)


def ring_backward_groups(rank: int, P: int, scheme: str = "zigzag", causal: bool = True):
    """The launches of one rank's ring backward when a step's calls go out
    together: a call adds into the dQ of its query chunk and into the dK, dV of
    its key/value chunk, so calls that share neither chunk are independent.
    Each step's calls are packed greedily in schedule order into groups of
    such calls; returns the groups in launch order, each a list of (index into
    ring_schedule's calls, call).  With two chunks on each side a step needs
    at most two launches: (q1, k1) with (q2, k2), and (q1, k2) with (q2, k1)."""
    calls = ring_schedule(rank, P, scheme, causal)
    groups = []
    for step in range(P):
        pending = [(i, c) for i, c in enumerate(calls) if c[0] == step]
        while pending:
            g, rest, used_q, used_k = [], [], set(), set()
            for i, c in pending:
                if c[2] in used_q or c[3] in used_k:
                    rest.append((i, c))
                    continue
                g.append((i, c))
                used_q.add(c[2])
                used_k.add(c[3])
            groups.append(g)
            pending = rest
    return groups


def ring_backward(q_chunks, do_chunks, lse_chunks, delta_chunks, kv_chunks, rank: int, P: int, C: int, *,
                  dq_acc, dkv_acc, scheme: str = "zigzag", causal: bool = True, scale: float | None = None,
                  steps=None, grouped: bool = False, workspaces=None):
    """Run rank ``rank``'s ring backward on this GPU: every visible (query
    chunk, key/value chunk) pair of ``ring_schedule`` as one attn_bwd_block
    call with the chunks' global positions, adding into fp32 accumulators.

    q_chunks, do_chunks: the rank's two query chunks and their output
    gradients, [B, Hq, C, D] bf16; lse_chunks, delta_chunks: their global LSE
    and Dv, [B, Hq, C] float.  kv_chunks(src): ((k, v), (k, v)) of rank src's
    chunks.  dq_acc: per query chunk, an fp32 dQ accumulator; dkv_acc(src, ki):
    the fp32 (dK, dV) accumulators of rank src's key/value chunk ki (on a ring
    they travel with the chunk).  All accumulators are added to, so the caller
    zeroes them first.  steps: restrict to these ring steps (for timing one
    step).  grouped: each group of ``ring_backward_groups`` goes out as one
    ``attn_bwd_block_group``.  workspaces: up to four workspace tensors (one
    per call of a group; needed for grouped-query attention)."""
    from . import attn_bwd_block, attn_bwd_block_group

    calls = ring_schedule(rank, P, scheme, causal)
    mine = rank_chunks(rank, P, scheme)

    def fields(step, src, qi, ki, slot):
        k, v = kv_chunks(src)[ki]
        dk_acc, dv_acc = dkv_acc(src, ki)
        kc = rank_chunks(src, P, scheme)[ki]
        d = dict(q=q_chunks[qi], k=k, v=v, do=do_chunks[qi], lse=lse_chunks[qi], delta=delta_chunks[qi],
                 q_pos0=mine[qi] * C, k_pos0=kc * C, dq_acc=dq_acc[qi], dq_accumulate=True, dk_acc=dk_acc,
                 dv_acc=dv_acc, dkv_accumulate=True)
        if workspaces is not None:
            d["workspace"] = workspaces[slot]
        return d

    if grouped:
        for g in ring_backward_groups(rank, P, scheme, causal):
            if steps is not None and g[0][1][0] not in steps:
                continue
            attn_bwd_block_group([fields(*c, slot) for slot, (_, c) in enumerate(g)], causal=causal, scale=scale)
        return
    for step, src, qi, ki in calls:
        if steps is not None and step not in steps:
            continue
        d = fields(step, src, qi, ki, 0)
        q, k, v, do, lse, delta = (d.pop(n) for n in ("q", "k", "v", "do", "lse", "delta"))
        attn_bwd_block(q, k, v, do, lse, delta, causal=causal, scale=scale, **d)
