"""Seeded synthetic inputs shared by the parity tests, the bench and the oracle checks.

This module holds no attention arithmetic: it draws i.i.d. normal numbers from
NumPy's PCG64 generator and stores them as bf16 bit patterns (uint16).  The
GPU side receives the same bit patterns the oracle decodes, so both start from
identical data.

Recipe for every workload: ``numpy.random.default_rng(seed)``, then
``standard_normal(shape, float32)`` drawn in the order q, k, v, dO, each in its
logical layout, multiplied by ``amp`` (a power of two, so exact), and rounded
to bf16 with round-to-nearest-even.

The workloads mirror the shapes the pages use: the glossary example's
``[1, 4, 4096, 64]`` causal bf16 call ("Context Parallelism", Ultralytics
glossary, "Praktische Anwendung und Kompromisse"), a Llama-3-8B-shaped
Ulysses shard (32 query / 8 key-value heads, D=128) split P=8 ways over 32768
tokens, a 32768-token ring split into four contiguous 8192-token KV blocks (the
glossary's "So funktioniert Kontextparallelität" example splits 32,000 tokens
over four GPUs), the 512K-token scale the Ulysses pages quote, and a 65536-token
training backward.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even storage encoding (the synthetic data never holds NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, amp: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, amp^2) values stored as bf16 bit patterns."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if amp != 1.0:
        x *= np.float32(amp)
    return _f32_to_bf16_bits(x)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, distribution and seed."""
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    amp: float = 1.0
    causal: bool = True
    P: int = 1                 # Ulysses shards (relayout workloads)
    kv_blocks: int = 1         # ring KV blocks (partial + merge workloads)
    sampled_rows: int = 0      # 0: every row is checked against the oracle
    backward: bool = False
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        # SDPA's default 1/sqrt(D), as the fp32 value handed to the kernel
        return float(np.float32(1.0 / np.sqrt(float(self.D))))


WORKLOADS = {
    "listing_4k": Workload(
        "listing_4k", seed=1, B=1, Hq=4, Hkv=4, N=4096, D=64,
        notes="causal SDPA forward on the glossary example's [1,4,4096,64] bf16 shape"),
    "ulysses_shard_32k": Workload(
        "ulysses_shard_32k", seed=2, B=1, Hq=32, Hkv=8, N=32768, D=128, P=8, sampled_rows=256,
        notes="seq->head relayout of a P=8 Llama-3-8B-shaped layer, then causal GQA attention "
              "on one shard's 4 query heads and 1 KV head over 32768 tokens"),
    "ring_blocks_32k": Workload(
        "ring_blocks_32k", seed=3, B=1, Hq=8, Hkv=8, N=32768, D=128, kv_blocks=4, sampled_rows=256,
        notes="four 8192-key partial forwards merged by log-sum-exp, against full attention"),
    "ulysses_512k": Workload(
        "ulysses_512k", seed=4, B=1, Hq=4, Hkv=1, N=524288, D=128, amp=0.5, sampled_rows=256,
        notes="512K-token causal GQA forward on one Ulysses share"),
    "train_64k": Workload(
        "train_64k", seed=5, B=1, Hq=8, Hkv=8, N=65536, D=128, sampled_rows=128, backward=True,
        notes="causal forward + backward; dQ, dK, dV emitted as bf16"),
}


def make_qkv(B, Hq, Hkv, N, D, seed, amp=1.0, with_do=False, q_tokens_major=False):
    """Draw q, k, v (and dO) as bf16 bit patterns.

    Default layout is head-major ``[B, H, N, D]``.  With ``q_tokens_major`` the
    tensors are drawn token-major ``[N, H, D]`` per batch (``[B, N, H, D]``),
    the layout the sequence->head relayout consumes.
    """
    rng = np.random.default_rng(seed)
    if q_tokens_major:
        shp_q, shp_kv = (B, N, Hq, D), (B, N, Hkv, D)
    else:
        shp_q, shp_kv = (B, Hq, N, D), (B, Hkv, N, D)
    q = normal_bf16(rng, shp_q, amp)
    k = normal_bf16(rng, shp_kv, amp)
    v = normal_bf16(rng, shp_kv, amp)
    out = {"q": q, "k": k, "v": v}
    if with_do:
        out["do"] = normal_bf16(rng, shp_q, 1.0)
    return out


def make_workload_inputs(w: Workload):
    """Inputs of a named workload.  Relayout workloads (P > 1) come token-major
    and sharded: q [P, N/P, Hq, D], k and v [P, N/P, Hkv, D]."""
    if w.P > 1:
        rng = np.random.default_rng(w.seed)
        T = w.N // w.P
        q = normal_bf16(rng, (w.P, T, w.Hq, w.D), w.amp)
        k = normal_bf16(rng, (w.P, T, w.Hkv, w.D), w.amp)
        v = normal_bf16(rng, (w.P, T, w.Hkv, w.D), w.amp)
        return {"q": q, "k": k, "v": v}
    return make_qkv(w.B, w.Hq, w.Hkv, w.N, w.D, w.seed, w.amp, with_do=w.backward)


def sample_rows(N: int, seed: int, count: int = 256, tile: int = 128, block: int = 0) -> np.ndarray:
    """Sorted query-row indices for sampled checks at large N.

    Always contains the first and last row, each tile-boundary pair
    (tile-1, tile) and every KV-block boundary pair when ``block`` > 0; the
    rest are uniform draws without replacement from ``default_rng(seed+1000)``.
    The same set is used for every head.
    """
    forced = {0, N - 1}
    if N > tile:
        forced.update((tile - 1, tile))
    if block and N > block:
        for b in range(block, N, block):
            forced.update((b - 1, b))
    forced = {r for r in forced if 0 <= r < N}
    rng = np.random.default_rng(seed + 1000)
    rest = np.setdiff1d(np.arange(N), np.fromiter(forced, dtype=np.int64))
    need = max(0, min(count, N) - len(forced))
    pick = rng.choice(rest, size=need, replace=False) if need else np.empty(0, np.int64)
    return np.sort(np.concatenate([np.fromiter(forced, dtype=np.int64), pick.astype(np.int64)]))
