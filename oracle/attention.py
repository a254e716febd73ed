"""Plain float64 definitions of the attention hot path (oracle; test infrastructure only).

Sources (web pages; the oracle restates them, it copies nothing):

* "Context Parallelism" (Ultralytics glossary, German edition), section
  "Praktische Anwendung und Kompromisse": its example program runs PyTorch's
  scaled-dot-product attention with ``is_causal=True`` on bf16 tensors laid out
  ``[batch, heads, sequence, head_dim]`` (sequence is dimension 2) and back-
  propagates the mean of the squared output.  The pages never print the
  formula; the oracle takes the textbook reading
  ``O = softmax(s * Q K^T + causal mask) V`` with ``s = 1/sqrt(D)`` (SDPA's
  default scale), plus the per-row log-sum-exp (natural log) of the scaled,
  masked scores.
* Same page, section "So funktioniert Kontextparallelität": ring attention
  computes partial attention of local queries against one KV block at a time
  and the combined result equals attention over the whole sequence up to the
  usual rounding differences.  The combine rule is not printed; the oracle
  uses the log-sum-exp merge, which follows from the definition of softmax
  over a disjoint union of key sets (see ``lse_merge``).
* "Million-Token-Kontexte im Training: Sequence Parallelism als
  Schlüsseltechnik für Long-Context-Modelle", section "Ulysses: Die Sequenz als
  Verteilungseinheit", and "Ulysses Sequence Parallelism: как тренировать
  модели с контекстом в миллион токенов", section "Как работает Ulysses:
  технические детали": the sequence is split into equal contiguous parts and an
  all-to-all exchange gives each GPU the full sequence for a subset of heads.
  ``seq_to_head`` / ``head_to_seq`` are that exchange's data movement on one
  GPU, with contiguous token shards and contiguous head groups.

Readings where the pages are silent (each is listed in the design notes):
causal alignment uses global positions (key ``k_pos0+j`` is visible to query
``q_pos0+i`` iff ``k_pos0+j <= q_pos0+i``); a row with no visible key has
``O = 0`` and ``LSE = -inf``; grouped-query attention maps query head ``h`` to
key/value head ``h // (Hq // Hkv)``.

Evaluation order: query rows are independent under the definition, so rows
are processed in batches to bound memory.  Keys are never tiled: every row's
scores, maximum, sum and output are formed over all of its keys at once.
Masked scores are exactly ``-inf`` and contribute exactly zero, so for causal
rows the keys past the batch's last visible position are not multiplied out.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "f32_to_bf16_bits",
    "scores",
    "attention_forward",
    "attention_probabilities",
    "lse_merge",
    "attention_backward",
    "attention_backward_sampled",
    "attention_backward_row_support",
    "attention_backward_block",
    "seq_to_head",
    "head_to_seq",
    "head_to_seq_sum",
]

_ROW_BATCH_ELEMS = 1 << 25  # score elements per batch of rows (256 MiB in fp64)


# ----------------------------------------------------------------------------
# bf16 storage codec.  bf16 is the upper half of an IEEE binary32 word.
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly: shift into the high half of a
    binary32 word, reinterpret, widen to float64."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 bit patterns must be uint16")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round binary32 values to bf16, round-to-nearest-even (integer method):
    add 0x7FFF plus the lowest kept bit, drop the low 16 bits.  NaNs stay NaN
    (quiet bit set)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    rne = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = np.where(is_nan, (u >> 16) | 0x0040, rne)
    return (out & 0xFFFF).astype(np.uint16)


# ----------------------------------------------------------------------------
# helpers on shapes
# ----------------------------------------------------------------------------
def _as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64, copy=False)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, Hq, _, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k, v must be [B, Hkv, Nk, D] matching q")
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, D


def _row_batches(rows: np.ndarray, nk: int):
    step = max(1, _ROW_BATCH_ELEMS // max(1, nk))
    for s in range(0, len(rows), step):
        yield rows[s:s + step]


# ----------------------------------------------------------------------------
# scores, probabilities, forward
# ----------------------------------------------------------------------------
def scores(q_rows, k, scale, causal, q_pos, k_pos0=0) -> np.ndarray:
    """S[i, j] = scale * <q_i, k_j>, or -inf where key position k_pos0+j lies
    after query position q_pos[i] (causal).  q_rows [R, D], k [Nk, D]."""
    q_rows = _as_f64(q_rows)
    k = _as_f64(k)
    s = np.float64(scale) * (q_rows @ k.T)
    if causal:
        kp = np.int64(k_pos0) + np.arange(k.shape[0], dtype=np.int64)
        masked = kp[None, :] > np.asarray(q_pos, dtype=np.int64)[:, None]
        s[masked] = -np.inf
    return s


def _softmax_rows(s: np.ndarray):
    """Per-row log-sum-exp (natural log) and probabilities of a score block.
    A row whose scores are all -inf has LSE = -inf and probabilities 0."""
    m = s.max(axis=1)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    tot = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(tot))
    p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, tot)[:, None])
    return lse, p


def attention_probabilities(q, k, scale, causal=True, q_pos0=0, k_pos0=0):
    """Full probability matrices P [B, Hq, Nq, Nk] (small inputs only)."""
    q = _as_f64(q)
    k = _as_f64(k)
    B, Hq, Hkv, D = _check_shapes(q, k, k)
    G = Hq // Hkv
    Nq, Nk = q.shape[2], k.shape[2]
    out = np.zeros((B, Hq, Nq, Nk))
    qpos = np.int64(q_pos0) + np.arange(Nq, dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            s = scores(q[b, h], k[b, h // G], scale, causal, qpos, k_pos0)
            out[b, h] = _softmax_rows(s)[1]
    return out


def _visible_keys(causal, q_pos_max, k_pos0, nk):
    """Number of leading keys that can be unmasked for queries at positions
    <= q_pos_max (all of them when not causal)."""
    if not causal:
        return nk
    return int(min(nk, max(0, q_pos_max - k_pos0 + 1)))


def attention_forward(q, k, v, scale, causal=True, q_pos0=0, k_pos0=0, rows=None):
    """Causal (or full) scaled-dot-product attention with per-row LSE.

    q [B, Hq, Nq, D]; k, v [B, Hkv, Nk, D] (float or bf16 bit patterns).
    Returns (O [B, Hq, R, D], LSE [B, Hq, R]) for the query rows ``rows``
    (all rows by default), both float64.  LSE is the natural log of the sum of
    exp of the scaled, masked scores; rows with no visible key give O = 0,
    LSE = -inf.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Hq, Hkv, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    Nq, Nk = q.shape[2], k.shape[2]
    rows = np.arange(Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((B, Hq, len(rows), D))
    L = np.full((B, Hq, len(rows)), -np.inf)
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            pos = 0
            for rb in _row_batches(rows, Nk):
                qpos = np.int64(q_pos0) + rb
                nvis = _visible_keys(causal, int(qpos.max()), k_pos0, Nk)
                sl = slice(pos, pos + len(rb))
                pos += len(rb)
                if nvis == 0:
                    continue
                s = scores(q[b, h, rb], k[b, kh, :nvis], scale, causal, qpos, k_pos0)
                lse, p = _softmax_rows(s)
                O[b, h, sl] = p @ v[b, kh, :nvis]
                L[b, h, sl] = lse
    return O, L


# ----------------------------------------------------------------------------
# merge of partial results over a partition of the keys
# ----------------------------------------------------------------------------
def lse_merge(o_parts, lse_parts):
    """Combine partial attention results computed over disjoint key blocks.

    For one query row, block b gives O_b = sum_{j in b} e^{S_j} V_j / Z_b and
    LSE_b = ln Z_b.  Softmax over the union of the blocks renormalises by
    Z = sum_b Z_b, so LSE = ln sum_b e^{LSE_b} and O = sum_b (Z_b / Z) O_b =
    sum_b e^{LSE_b - LSE} O_b.  The sum is evaluated after factoring out
    M = max_b LSE_b.  Blocks with LSE_b = -inf (no visible key) weigh zero;
    a row empty in every block stays O = 0, LSE = -inf.

    o_parts [n, ..., D], lse_parts [n, ...]; returns (O [..., D], LSE [...]).
    """
    o_parts = _as_f64(o_parts)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    empty = np.isneginf(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.exp(lse_parts - M_safe[None])          # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, M_safe + np.log(np.where(empty, 1.0, tot)))
    wn = np.where(empty[None], 0.0, w / np.where(empty, 1.0, tot)[None])
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, lse


# ----------------------------------------------------------------------------
# backward (analytic gradients of sum(O * dO))
# ----------------------------------------------------------------------------
def attention_backward(q, k, v, do, scale, causal=True):
    """Gradients of L = sum(O * dO) with respect to q, k, v (Nq = Nk = N,
    equal position offsets).

    Dv_i = <dO_i, O_i>;  dP_ij = <dO_i, V_j>;  dS_ij = P_ij (dP_ij - Dv_i);
    dQ_i = s sum_j dS_ij K_j;  dK_j = s sum_i dS_ij Q_i;  dV_j = sum_i P_ij dO_i.
    For grouped-query attention dK and dV of a key/value head sum over the
    query heads that read it.  Returns (O, LSE, dQ, dK, dV), float64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, Hq, Hkv, D = _check_shapes(q, k, v)
    if do.shape != q.shape or q.shape[2] != k.shape[2]:
        raise ValueError("backward needs Nq == Nk and dO shaped like q")
    G = Hq // Hkv
    N = q.shape[2]
    O, L = attention_forward(q, k, v, scale, causal)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    rows = np.arange(N, dtype=np.int64)
    s = np.float64(scale)
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            Dv = np.einsum("nd,nd->n", do[b, h], O[b, h])
            for rb in _row_batches(rows, N):
                nvis = _visible_keys(causal, int(rb.max()), 0, N)
                S = scores(q[b, h, rb], k[b, kh, :nvis], scale, causal, rb, 0)
                P = np.exp(S - L[b, h, rb][:, None])
                dP = do[b, h, rb] @ v[b, kh, :nvis].T
                dS = P * (dP - Dv[rb][:, None])
                dQ[b, h, rb] = s * (dS @ k[b, kh, :nvis])
                dK[b, kh, :nvis] += s * (dS.T @ q[b, h, rb])
                dV[b, kh, :nvis] += P.T @ do[b, h, rb]
    return O, L, dQ, dK, dV


def attention_backward_sampled(q, k, v, do, scale, q_rows, kv_rows, causal=True,
                               lse=None, dv=None):
    """Exact gradients at a subset of rows (large N).

    dQ at query rows ``q_rows`` needs only those rows' LSE and Dv.  dK, dV at
    key rows ``kv_rows`` need LSE and Dv of every query row that sees them;
    pass ``lse`` / ``dv`` [B, Hq, N] if already known (else they are computed
    here with a full forward).  Returns (dQ [B,Hq,|q_rows|,D],
    dK [B,Hkv,|kv_rows|,D], dV [B,Hkv,|kv_rows|,D]).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, Hq, Hkv, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    N = q.shape[2]
    s = np.float64(scale)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    kv_rows = np.asarray(kv_rows, dtype=np.int64)
    if lse is None or dv is None:
        O, lse = attention_forward(q, k, v, scale, causal)
        dv = np.einsum("bhnd,bhnd->bhn", do, O)
    dQ = np.zeros((B, Hq, len(q_rows), D))
    dK = np.zeros((B, Hkv, len(kv_rows), D))
    dV = np.zeros((B, Hkv, len(kv_rows), D))
    all_rows = np.arange(N, dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            # dQ at the sampled query rows
            pos = 0
            for rb in _row_batches(q_rows, N):
                nvis = _visible_keys(causal, int(rb.max()), 0, N)
                S = scores(q[b, h, rb], k[b, kh, :nvis], scale, causal, rb, 0)
                P = np.exp(S - lse[b, h, rb][:, None])
                dS = P * (do[b, h, rb] @ v[b, kh, :nvis].T - dv[b, h, rb][:, None])
                dQ[b, h, pos:pos + len(rb)] = s * (dS @ k[b, kh, :nvis])
                pos += len(rb)
            # dK, dV at the sampled key rows: every query row that sees them
            first = int(kv_rows.min()) if causal else 0
            for rb in _row_batches(all_rows[first:], len(kv_rows)):
                S = scores(q[b, h, rb], k[b, kh, kv_rows], scale, False, rb, 0)
                if causal:
                    S[kv_rows[None, :] > rb[:, None]] = -np.inf
                P = np.exp(S - lse[b, h, rb][:, None])
                dS = P * (do[b, h, rb] @ v[b, kh, kv_rows].T - dv[b, h, rb][:, None])
                dK[b, kh] += s * (dS.T @ q[b, h, rb])
                dV[b, kh] += P.T @ do[b, h, rb]
    return dQ, dK, dV


def attention_backward_block(q, k, v, do, lse, dv, scale, causal=True, q_pos0=0, k_pos0=0):
    """Gradients through one KV block of the attention of a query shard (the
    backward of one step of the ring of "So funktioniert Kontextparallelität").

    q, do [B, Hq, Nq, D]: the shard's queries at global positions
    q_pos0 .. q_pos0+Nq-1 and their output gradients.  k, v [B, Hkv, Nk, D]:
    one KV block at positions k_pos0 .. k_pos0+Nk-1.  lse, dv [B, Hq, Nq]: the
    shard's LSE over every key of the sequence and Dv_i = <dO_i, O_i> of its
    final output.  Softmax over a disjoint union of key sets shares one
    normaliser, so over this block P_ij = exp(s q_i.k_j - LSE_i) with the
    global LSE, dS_ij = P_ij (<dO_i, V_j> - Dv_i), and
    dQ_i = s sum_j dS_ij K_j (this block's term), dK_j = s sum_i dS_ij Q_i,
    dV_j = sum_i P_ij dO_i.  Returns (dQ, dK, dV), float64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    lse = np.asarray(lse, dtype=np.float64)
    dv = np.asarray(dv, dtype=np.float64)
    B, Hq, Hkv, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    Nq, Nk = q.shape[2], k.shape[2]
    if do.shape != q.shape or lse.shape != (B, Hq, Nq) or dv.shape != (B, Hq, Nq):
        raise ValueError("do like q; lse and dv [B, Hq, Nq]")
    s = np.float64(scale)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    rows = np.arange(Nq, dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            for rb in _row_batches(rows, Nk):
                qpos = np.int64(q_pos0) + rb
                nvis = _visible_keys(causal, int(qpos.max()), k_pos0, Nk)
                if nvis == 0:
                    continue
                S = scores(q[b, h, rb], k[b, kh, :nvis], scale, causal, qpos, k_pos0)
                with np.errstate(invalid="ignore"):
                    P = np.exp(S - lse[b, h, rb][:, None])
                P[np.isneginf(S)] = 0.0  # masked entries (also rows whose LSE is -inf)
                dS = P * (do[b, h, rb] @ v[b, kh, :nvis].T - dv[b, h, rb][:, None])
                dQ[b, h, rb] = s * (dS @ k[b, kh, :nvis])
                dK[b, kh, :nvis] += s * (dS.T @ q[b, h, rb])
                dV[b, kh, :nvis] += P.T @ do[b, h, rb]
    return dQ, dK, dV


def attention_backward_row_support(q, k, v, do, scale, support, kv_rows=None, causal=True):
    """Exact gradients when dO is zero outside the query rows ``support``.

    Gradients are linear in dO, and a row i with dO_i = 0 has Dv_i = 0 and
    dP_ij = 0, so it adds nothing to any of dQ, dK, dV.  Every sum then runs
    over the support rows only, which need only their own LSE and Dv.
    Returns (dQ [B,Hq,|support|,D], dK [B,Hkv,R,D], dV [B,Hkv,R,D]) with R the
    key rows ``kv_rows`` (all keys by default).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, Hq, Hkv, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    N = q.shape[2]
    support = np.asarray(support, dtype=np.int64)
    outside = np.ones(N, dtype=bool)
    outside[support] = False
    if np.any(do[:, :, outside] != 0):
        raise ValueError("dO must be zero outside the support rows")
    kv_rows = np.arange(N, dtype=np.int64) if kv_rows is None else np.asarray(kv_rows, dtype=np.int64)
    s = np.float64(scale)
    O, L = attention_forward(q, k, v, scale, causal, rows=support)
    dQ = np.zeros((B, Hq, len(support), D))
    dK = np.zeros((B, Hkv, len(kv_rows), D))
    dV = np.zeros((B, Hkv, len(kv_rows), D))
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            dor = do[b, h, support]
            Dv = np.einsum("nd,nd->n", dor, O[b, h])
            S = scores(q[b, h, support], k[b, kh], scale, causal, support, 0)
            P = np.exp(S - L[b, h][:, None])
            dS = P * (dor @ v[b, kh].T - Dv[:, None])
            dQ[b, h] = s * (dS @ k[b, kh])
            dK[b, kh] += s * (dS[:, kv_rows].T @ q[b, h, support])
            dV[b, kh] += P[:, kv_rows].T @ dor
    return dQ, dK, dV


# ----------------------------------------------------------------------------
# sequence <-> head relayout (the all-to-all's data movement on one GPU)
# ----------------------------------------------------------------------------
def seq_to_head(x, P: int) -> np.ndarray:
    """in [P, N/P, H, D] (shard p holds tokens p*N/P ...) -> out [P, H/P, N, D]
    (rank r holds heads r*H/P ...):  out[r, h', n, :] =
    in[n // (N/P), n mod (N/P), r*(H/P) + h', :].  Bit copy (any dtype).

    Fewer heads than ranks (H < P, H | P; key/value heads of grouped-query
    attention): rank r's query heads read head r // (P/H), so that head is
    what it receives: out [P, 1, N, D], out[r, 0, n, :] =
    in[n // (N/P), n mod (N/P), r // (P/H), :]."""
    x = np.asarray(x)
    Pp, T, H, D = x.shape
    if Pp != P or (H % P if H >= P else P % H):
        raise ValueError("shape must be [P, N/P, H, D] with P | H or H | P")
    N = P * T
    n = np.arange(N)
    src_p, src_t = n // T, n % T
    if H < P:
        R = P // H
        out = np.empty((P, 1, N, D), dtype=x.dtype)
        for r in range(P):
            out[r, 0] = x[src_p, src_t, r // R]
        return out
    Hp = H // P
    out = np.empty((P, Hp, N, D), dtype=x.dtype)
    for r in range(P):
        for hh in range(Hp):
            out[r, hh] = x[src_p, src_t, r * Hp + hh]
    return out


def head_to_seq(y, P: int) -> np.ndarray:
    """Inverse of ``seq_to_head``: in [P, H/P, N, D] -> out [P, N/P, H, D],
    out[p, t, h, :] = in[h // (H/P), h mod (H/P), p*(N/P) + t, :]."""
    y = np.asarray(y)
    Pp, Hp, N, D = y.shape
    if Pp != P or N % P:
        raise ValueError("shape must be [P, H/P, N, D] with P | N")
    T = N // P
    H = P * Hp
    out = np.empty((P, T, H, D), dtype=y.dtype)
    t = np.arange(T)
    for p in range(P):
        for h in range(H):
            out[p, :, h] = y[h // Hp, h % Hp, p * T + t]
    return out


def head_to_seq_sum(y, P: int, H: int) -> np.ndarray:
    """Inverse exchange of gradients (float64 values): in [P, max(1, H/P), N, D]
    -> out [P, N/P, H, D].  For H >= P it is ``head_to_seq`` on the values.
    For H < P each head was replicated to R = P/H ranks (``seq_to_head``), so
    its gradient is the sum of theirs: out[p, t, h, :] = sum over i < R of
    in[h*R + i, 0, p*(N/P) + t, :]."""
    y = _as_f64(y)
    Pp, Hr, N, D = y.shape
    if Pp != P or N % P or (H % P if H >= P else P % H) or Hr != max(1, H // P):
        raise ValueError("shape must be [P, max(1, H/P), N, D] with P | N and P | H or H | P")
    if H >= P:
        return head_to_seq(y, P)
    R = P // H
    T = N // P
    out = np.zeros((P, T, H, D))
    t = np.arange(T)
    for p in range(P):
        for h in range(H):
            for i in range(R):
                out[p, :, h] += y[h * R + i, 0, p * T + t]
    return out
