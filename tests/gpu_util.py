"""Helpers shared by the GPU parity tests: host<->device transfer of bf16 bit
patterns, NaN-poisoned outputs and the tolerance checks.

Tolerances (floating point, per tensor over every checked element):
  O        max |O_gpu - O_ref|                     <= 1e-2
  LSE      max |LSE_gpu - LSE_ref| (finite rows)   <= 1e-3, -inf rows must match
  O rows   max_i ||O_gpu,i - O_ref,i|| / ||O_ref,i|| <= 2e-2 (rows with ||O_ref,i|| > 0)
  grads    max |dX_gpu - dX_ref| / max |dX_ref|    <= 2e-2
The per-row relative check guards the late rows of long sequences, whose
entries are much smaller than 1e-2.
"""

from __future__ import annotations

import numpy as np

import oracle

O_ABS_TOL = 1e-2
LSE_ABS_TOL = 1e-3
ROW_REL_TOL = 2e-2
GRAD_REL_TOL = 2e-2


def to_dev(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bits_of(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(bits_of(t))
    return t.detach().cpu().double().numpy()


def poisoned(shape, dtype, device="cuda"):
    """An output buffer filled with NaN so that unwritten elements show."""
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device=device)


def check_forward(o_gpu, lse_gpu, o_ref, lse_ref, what="", out_rounding=False):
    """Assert the forward gates; returns a dict of the observed errors.

    ``out_rounding`` widens the O gate element-wise by 2^-8 |O_ref|, the
    largest relative error of rounding a value to bf16 (half an ulp).  It is
    used only for inputs built to have |O| above ~2.5, where a bf16 output
    cannot meet a 1e-2 absolute bound even when exactly rounded."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN LSE"
    empty_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty_ref), f"{what}: empty-row pattern differs"
    slack = 2.0 ** -8 * np.abs(o_ref) if out_rounding else 0.0
    o_err = float((np.abs(o_gpu - o_ref) - slack).max()) if o_ref.size else 0.0
    fin = ~empty_ref
    lse_err = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    ref_norm = np.linalg.norm(o_ref, axis=-1)
    err_norm = np.linalg.norm(o_gpu - o_ref, axis=-1)
    nz = ref_norm > 0
    row_rel = float((err_norm[nz] / ref_norm[nz]).max()) if nz.any() else 0.0
    if (~nz).any():
        assert np.all(o_gpu[~nz] == 0), f"{what}: empty rows must be zero"
    assert o_err <= O_ABS_TOL, f"{what}: O max abs err {o_err}"
    assert lse_err <= LSE_ABS_TOL, f"{what}: LSE max abs err {lse_err}"
    assert row_rel <= ROW_REL_TOL, f"{what}: O row relative err {row_rel}"
    return {"o_abs": o_err, "lse_abs": lse_err, "o_row_rel": row_rel}


def grad_rel_err(g_gpu, g_ref) -> float:
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    den = float(np.abs(g_ref).max())
    return float(np.abs(g_gpu - g_ref).max()) / (den if den > 0 else 1.0)


def oracle_full_lse_delta(q, k, v, do, scale, causal=True, workers=None, chunk=2048):
    """The oracle's fp64 LSE and Dv_i = <dO_i, O_i> for every query row of
    every head, from ``oracle.attention_forward`` run over (head, row chunk)
    tasks in a thread pool (rows are independent under the definition).
    BLAS is held to one thread per task so the tasks run side by side.
    q, k, v, do: float64 arrays [B, H, N, D] (decoded once by the caller).
    Returns (lse [B, Hq, N], dv [B, Hq, N])."""
    import concurrent.futures as cf
    import os
    from threadpoolctl import threadpool_limits

    B, Hq, N, _ = q.shape
    G = Hq // k.shape[1]
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    tasks = [(b, h, r0) for b in range(B) for h in range(Hq) for r0 in range(0, N, chunk)]
    tasks.sort(key=lambda t: -t[2])  # longest causal rows first
    lse = np.empty((B, Hq, N))
    dv = np.empty((B, Hq, N))

    def run(t):
        b, h, r0 = t
        rows = np.arange(r0, min(N, r0 + chunk))
        kh = h // G
        O, L = oracle.attention_forward(q[b:b + 1, h:h + 1], k[b:b + 1, kh:kh + 1], v[b:b + 1, kh:kh + 1],
                                        scale, causal, rows=rows)
        lse[b, h, rows] = L[0, 0]
        dv[b, h, rows] = np.einsum("nd,nd->n", do[b, h, rows], O[0, 0])

    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(run, tasks))
    return lse, dv
