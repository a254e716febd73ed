"""MI355X-native long-context causal attention: Python binding of ``libattn.so``.

The binding only marshals arguments: it checks dtypes, shapes, contiguity and
devices of torch tensors, allocates outputs with torch when the caller did not
pass them, and calls the C ABI declared in ``include/attn.h`` on torch's
current HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no fallback path.  If the library is missing, every call
raises.

Layouts follow the PyTorch call on the "Context Parallelism" glossary page
(Ultralytics, "Praktische Anwendung und Kompromisse"): ``[B, H, N, D]`` with
the sequence on dimension 2.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = [
    "attn_fwd",
    "attn_fwd_strided",
    "attn_fwd_accumulate",
    "attn_fwd_accumulate_group",
    "attn_fwd_split_suggest",
    "attn_fwd_accumulate_workspace_size",
    "attn_fwd_accumulate_group_split",
    "attn_fwd_splitkv",
    "attn_fwd_splitkv_workspace_size",
    "attn_partial_merge",
    "attn_bwd",
    "attn_bwd_workspace_size",
    "attn_bwd_ds_workspace_size",
    "attn_bwd_strided",
    "attn_bwd_delta",
    "attn_bwd_block",
    "attn_bwd_block_group",
    "attn_bwd_block_workspace_size",
    "attn_bwd_block_ds_workspace_size",
    "seq_to_head_relayout",
    "head_to_seq_relayout",
    "seq_to_head_relayout_batch",
    "head_to_seq_relayout_batch",
    "head_to_seq_reduce",
    "trace_enable",
    "trace_collect",
    "AttnError",
    "lib",
    "LIB_PATH",
    "ATTN_BF16",
    "ATTN_FP32",
    "STATUS",
]

# the library built next to this file; LCATTN_LIBRARY names another build of
# the same sources (e.g. the host-sanitizer build of the validation layer)
LIB_PATH = os.environ.get("LCATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_BF16, ATTN_FP32 = 0, 1
STATUS = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL",
    2: "ATTN_ERR_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_ALIGN",
    5: "ATTN_ERR_ALIAS",
    6: "ATTN_ERR_WORKSPACE",
    7: "ATTN_ERR_HIP",
}

_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_F = ctypes.c_float
class AccumulateCall(ctypes.Structure):
    """One entry of attn_fwd_accumulate_group (mirrors attn_accumulate_call)."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o_acc", ctypes.c_void_p), ("lse_acc", ctypes.c_void_p), ("o_final", ctypes.c_void_p),
                ("Nq", ctypes.c_int64), ("Nk", ctypes.c_int64), ("q_pos0", ctypes.c_int64),
                ("k_pos0", ctypes.c_int64), ("first", ctypes.c_int)]


class AccumulateSplitCall(ctypes.Structure):
    """One entry of attn_fwd_accumulate_group_split (mirrors attn_accumulate_split_call)."""
    _fields_ = [("call", AccumulateCall), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class BwdBlockCall(ctypes.Structure):
    """One entry of attn_bwd_block_group (mirrors attn_bwd_block_call)."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("d_o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("delta", ctypes.c_void_p),
                ("dq_acc", ctypes.c_void_p), ("dk_acc", ctypes.c_void_p), ("dv_acc", ctypes.c_void_p),
                ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("Nq", ctypes.c_int64), ("Nk", ctypes.c_int64), ("q_pos0", ctypes.c_int64),
                ("k_pos0", ctypes.c_int64), ("dq_accumulate", ctypes.c_int), ("dkv_accumulate", ctypes.c_int)]


_SIGS = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _L, _L, _I, _F, _I, _L, _L, _P]),
    "attn_fwd_strided": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _L, _L, _I, _F, _I, _L, _L, _P, _P, _P, _P]),
    "attn_fwd_accumulate": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _I, _F, _I, _L, _L, _I, _P]),
    "attn_fwd_accumulate_group": (_I, [_P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_fwd_split_suggest": (_I, [_I, _I, _I, _L, _L, _I, _I]),
    "attn_fwd_accumulate_workspace_size": (ctypes.c_size_t, [_I, _I, _L, _I, _I]),
    "attn_fwd_accumulate_group_split": (_I, [_P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "attn_fwd_splitkv_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _L, _L, _I, _I, _I]),
    "attn_fwd_splitkv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _I, _F, _I, _L, _L, _I, _P, ctypes.c_size_t,
                              _P]),
    "attn_partial_merge": (_I, [_P, _I, _P, _I, _P, _P, _I, _I, _L, _I, _P]),
    "attn_bwd_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _L, _I]),
    "attn_bwd_ds_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _L, _I, _I]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _L, _I, _F, _I, _P]),
    "attn_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _L, _I, _F, _I, _P]),
    "attn_bwd_noalloc_max_scratch": (ctypes.c_size_t, []),
    "attn_bwd_delta": (_I, [_P, _P, _P, _I, _I, _L, _I, _P]),
    "attn_bwd_strided": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _L, _I, _F, _I,
                              _P, _P, _P]),
    "head_to_seq_reduce": (_I, [_P, _I, _P, _I, _L, _I, _I, _P]),
    "attn_bwd_block_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _L, _I]),
    "attn_bwd_block_ds_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _L, _L, _I]),
    "attn_bwd_block_group": (_I, [_P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_block": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                            _I, _I, _I, _L, _L, _I, _F, _I, _L, _L, _I, _I, _P]),
    "seq_to_head_relayout": (_I, [_P, _P, _I, _L, _I, _I, _I, _P]),
    "head_to_seq_relayout": (_I, [_P, _P, _I, _L, _I, _I, _I, _P]),
    "seq_to_head_relayout_batch": (_I, [_I, _P, _P, _P, _I, _L, _I, _I, _P]),
    "head_to_seq_relayout_batch": (_I, [_I, _P, _P, _P, _I, _L, _I, _I, _P]),
    "attn_trace_enable": (_I, [_I]),
    "attn_trace_collect": (_I, [ctypes.c_char_p, _I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I), _I]),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_last_error": (ctypes.c_char_p, []),
}


class AttnError(RuntimeError):
    """A nonzero status returned by the library."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


def lib() -> ctypes.CDLL:
    """The loaded library with argument types set (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m long_context_attention_fwd_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def _check(status: int):
    if status != 0:
        raise AttnError(status, lib().attn_last_error().decode())


def _torch():
    import torch
    return torch


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, name, dtype=None, dims=None, strided=False):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if strided:
        if t.dim() >= 1 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got shape {tuple(t.shape)}")


def attn_fwd(q, k, v, *, causal: bool = True, scale: float | None = None, q_pos0: int = 0, k_pos0: int = 0,
             out_dtype=None, o=None, lse=None):
    """Causal attention forward: returns (o [B,Hq,Nq,D], lse [B,Hq,Nq] float32).

    q [B, Hq, Nq, D] bf16; k, v [B, Hkv, Nk, D] bf16.  ``out_dtype`` is
    bfloat16 (default) or float32 (unrounded partials for the merge).
    """
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Hkv, Nk, D] matching q")
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    if o is None:
        o = torch.empty((B, Hq, Nq, D), dtype=out_dtype, device=q.device)
    _need(o, "o", out_dtype, 4)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, 3)
    if tuple(o.shape) != (B, Hq, Nq, D) or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("o / lse have the wrong shape")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          ATTN_FP32 if out_dtype == torch.float32 else ATTN_BF16, lse.data_ptr(),
                          B, Hq, Hkv, Nq, Nk, D, scale, 1 if causal else 0, q_pos0, k_pos0, _stream(q)))
    return o, lse


def attn_fwd_strided(q, k, v, *, causal: bool = True, scale: float | None = None, q_pos0: int = 0,
                     k_pos0: int = 0, out_dtype=None, o=None, lse=None):
    """attn_fwd on [B, H, N, D] views with any batch / head / token strides
    (the last dimension contiguous), e.g. heads of a token-major [N, H, D]
    shard; returns (o, lse).  ``o`` may be such a view too (default: a new
    contiguous tensor)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4, strided=True)
    _need(k, "k", torch.bfloat16, 4, strided=True)
    _need(v, "v", torch.bfloat16, 4, strided=True)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Hkv, Nk, D] matching q")
    if tuple(v.stride()) != tuple(k.stride()):
        raise ValueError("k and v must have the same strides")
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    if o is None:
        o = torch.empty((B, Hq, Nq, D), dtype=out_dtype, device=q.device)
    _need(o, "o", out_dtype, 4, strided=True)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, 3)
    if tuple(o.shape) != (B, Hq, Nq, D) or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("o / lse have the wrong shape")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    arr = ctypes.c_int64 * 3
    qs, ks, os_ = arr(*q.stride()[:3]), arr(*k.stride()[:3]), arr(*o.stride()[:3])
    _check(lib().attn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  ATTN_FP32 if out_dtype == torch.float32 else ATTN_BF16, lse.data_ptr(),
                                  B, Hq, Hkv, Nq, Nk, D, scale, 1 if causal else 0, q_pos0, k_pos0,
                                  qs, ks, os_, _stream(q)))
    return o, lse


def attn_fwd_accumulate(q, k, v, o_acc, lse_acc, *, first: bool, causal: bool = True, scale: float | None = None,
                        q_pos0: int = 0, k_pos0: int = 0, o_final=None):
    """One streaming-ring step: attention of q against the KV block (k, v)
    merged in place into the running fp32 (o_acc, lse_acc) (overwritten when
    ``first``); ``o_final`` (bf16, optional) also receives the merged O."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(o_acc, "o_acc", torch.float32, 4)
    _need(lse_acc, "lse_acc", torch.float32, 3)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Hkv, Nk, D] matching q")
    if tuple(o_acc.shape) != (B, Hq, Nq, D) or tuple(lse_acc.shape) != (B, Hq, Nq):
        raise ValueError("o_acc / lse_acc have the wrong shape")
    if o_final is not None:
        _need(o_final, "o_final", torch.bfloat16, 4)
        if tuple(o_final.shape) != (B, Hq, Nq, D):
            raise ValueError("o_final has the wrong shape")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().attn_fwd_accumulate(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_acc.data_ptr(), lse_acc.data_ptr(),
                                     None if o_final is None else o_final.data_ptr(), B, Hq, Hkv, Nq, Nk, D, scale,
                                     1 if causal else 0, q_pos0, k_pos0, 1 if first else 0, _stream(q)))
    return o_acc, lse_acc


def _accumulate_calls(calls):
    """Checks of a group of accumulate calls; returns (AccumulateCall array,
    B, Hq, Hkv, D)."""
    torch = _torch()
    if not 1 <= len(calls) <= 4:
        raise ValueError("a group holds 1 to 4 calls")
    B, Hq, _, D = calls[0]["q"].shape
    Hkv = calls[0]["k"].shape[1]
    arr = (AccumulateCall * len(calls))()
    for i, c in enumerate(calls):
        q, k, v, o_acc, lse_acc = c["q"], c["k"], c["v"], c["o_acc"], c["lse_acc"]
        _need(q, "q", torch.bfloat16, 4)
        _need(k, "k", torch.bfloat16, 4)
        _need(v, "v", torch.bfloat16, 4)
        _need(o_acc, "o_acc", torch.float32, 4)
        _need(lse_acc, "lse_acc", torch.float32, 3)
        Nq, Nk = q.shape[2], k.shape[2]
        if (q.shape[0], q.shape[1], q.shape[3]) != (B, Hq, D) or tuple(k.shape) != (B, Hkv, Nk, D) \
                or tuple(v.shape) != tuple(k.shape):
            raise ValueError("the calls of a group share B, Hq, Hkv and D")
        if tuple(o_acc.shape) != (B, Hq, Nq, D) or tuple(lse_acc.shape) != (B, Hq, Nq):
            raise ValueError("o_acc / lse_acc have the wrong shape")
        of = c.get("o_final")
        if of is not None:
            _need(of, "o_final", torch.bfloat16, 4)
            if tuple(of.shape) != (B, Hq, Nq, D):
                raise ValueError("o_final has the wrong shape")
        arr[i] = AccumulateCall(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_acc.data_ptr(), lse_acc.data_ptr(),
                                None if of is None else of.data_ptr(), Nq, Nk, int(c.get("q_pos0", 0)),
                                int(c.get("k_pos0", 0)), 1 if c["first"] else 0)
    return arr, B, Hq, Hkv, D


def attn_fwd_accumulate_group(calls, *, causal: bool = True, scale: float | None = None):
    """Independent attn_fwd_accumulate calls (1 to 4) in one launch.  calls:
    dicts with q, k, v, o_acc, lse_acc, first and optionally o_final,
    q_pos0, k_pos0 (meanings as in attn_fwd_accumulate); B, Hq, Hkv, D are
    shared.  The calls must not write what another call reads or writes."""
    calls = list(calls)
    arr, B, Hq, Hkv, D = _accumulate_calls(calls)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().attn_fwd_accumulate_group(arr, len(calls), B, Hq, Hkv, D, scale, 1 if causal else 0,
                                           _stream(calls[0]["q"])))


def attn_fwd_split_suggest(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, causal: bool = True, n_calls: int = 1) -> int:
    """The library's choice of key ranges for n_calls accumulate calls of this
    size run side by side (1: no split)."""
    return int(lib().attn_fwd_split_suggest(B, Hq, Hkv, Nq, Nk, 1 if causal else 0, n_calls))


def attn_fwd_accumulate_workspace_size(B: int, Hq: int, Nq: int, D: int, n_splits: int) -> int:
    return int(lib().attn_fwd_accumulate_workspace_size(B, Hq, Nq, D, n_splits))


def attn_fwd_accumulate_group_split(calls, *, n_splits: int, causal: bool = True, scale: float | None = None):
    """attn_fwd_accumulate_group with each call's keys in n_splits ranges side
    by side, then one merge per call into its running result.  calls: as
    attn_fwd_accumulate_group's, each with a "workspace" (uint8 device tensor
    of >= attn_fwd_accumulate_workspace_size bytes; allocated when absent)."""
    torch = _torch()
    calls = list(calls)
    arr, B, Hq, Hkv, D = _accumulate_calls(calls)
    sarr = (AccumulateSplitCall * len(calls))()
    keep = []
    for i, c in enumerate(calls):
        need = attn_fwd_accumulate_workspace_size(B, Hq, c["q"].shape[2], D, n_splits)
        ws = c.get("workspace")
        if ws is None:
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=c["q"].device)
        keep.append(ws)
        sarr[i] = AccumulateSplitCall(arr[i], ws.data_ptr(), ws.numel() * ws.element_size())
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().attn_fwd_accumulate_group_split(sarr, len(calls), B, Hq, Hkv, D, scale, 1 if causal else 0,
                                                 int(n_splits), _stream(calls[0]["q"])))
    del keep  # the launches are enqueued: the stream orders any reuse after them


def attn_fwd_splitkv_workspace_size(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, D: int, causal: bool = True,
                                    n_splits: int = 0) -> int:
    return int(lib().attn_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, D, 1 if causal else 0, n_splits))


def attn_fwd_splitkv(q, k, v, *, causal: bool = True, scale: float | None = None, q_pos0: int = 0,
                     k_pos0: int = 0, n_splits: int = 0, workspace=None, o=None, lse=None):
    """attn_fwd with the keys split into ranges that run side by side (for
    short sequences); returns (o bf16 [B,Hq,Nq,D], lse [B,Hq,Nq] float32).
    ``n_splits`` <= 0 lets the library choose the number of ranges."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Hkv, Nk, D] matching q")
    if o is None:
        o = torch.empty((B, Hq, Nq, D), dtype=torch.bfloat16, device=q.device)
    _need(o, "o", torch.bfloat16, 4)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, 3)
    if tuple(o.shape) != (B, Hq, Nq, D) or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("o / lse have the wrong shape")
    need = attn_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, D, causal, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, Hq, Hkv, Nq, Nk, D, scale, 1 if causal else 0, q_pos0, k_pos0, n_splits,
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q)))
    return o, lse


def attn_partial_merge(o_parts, lse_parts, *, o=None, lse=None):
    """Merge partials over disjoint key blocks: o_parts [n,B,H,N,D] (bf16 or
    float32), lse_parts [n,B,H,N] float32 -> (o [B,H,N,D] bf16, lse [B,H,N])."""
    torch = _torch()
    _need(o_parts, "o_parts", (torch.bfloat16, torch.float32), 5)
    _need(lse_parts, "lse_parts", torch.float32, 4)
    n, B, H, N, D = o_parts.shape
    if tuple(lse_parts.shape) != (n, B, H, N):
        raise ValueError("lse_parts must be [n, B, H, N] matching o_parts")
    if o is None:
        o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    _need(o, "o", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    pd = ATTN_FP32 if o_parts.dtype == torch.float32 else ATTN_BF16
    _check(lib().attn_partial_merge(o_parts.data_ptr(), pd, lse_parts.data_ptr(), n, o.data_ptr(), lse.data_ptr(),
                                    B, H, N, D, _stream(o_parts)))
    return o, lse


def attn_bwd_workspace_size(B: int, Hq: int, Hkv: int, N: int, D: int) -> int:
    return int(lib().attn_bwd_workspace_size(B, Hq, Hkv, N, D))


def attn_bwd_ds_workspace_size(B: int, Hq: int, Hkv: int, N: int, D: int, causal: bool = True) -> int:
    """Workspace bytes with which attn_bwd forms dq from stored dS (0: not
    available for this shape)."""
    return int(lib().attn_bwd_ds_workspace_size(B, Hq, Hkv, N, D, 1 if causal else 0))


# the largest stored-dS workspace the backward allocates by itself
# (stored_ds=None): the 64K-token training shape at 8 heads needs 32 GiB
STORED_DS_AUTO_BYTES = 64 << 30


def _bwd_workspace(B, Hq, Hkv, N, D, causal, stored_ds, device):
    torch = _torch()
    need = 0
    if stored_ds is not False:
        need = attn_bwd_ds_workspace_size(B, Hq, Hkv, N, D, causal)
        if stored_ds is None and need > STORED_DS_AUTO_BYTES:
            need = 0
    if need == 0:
        need = attn_bwd_workspace_size(B, Hq, Hkv, N, D)
    return torch.empty(max(need, 16), dtype=torch.uint8, device=device)


def attn_bwd(q, k, v, o, do, lse, *, causal: bool = True, scale: float | None = None, workspace=None,
             dq=None, dk=None, dv=None, stored_ds: bool | None = None):
    """Gradients of sum(o * do): returns (dq, dk, dv) as bf16, shaped like q, k, v.
    The library picks the dq path by the workspace's size.  Without a
    workspace one is allocated: with room for the stored dS (dq as a product
    of it, attn_bwd_ds_workspace_size) when the shape has that path and
    stored_ds is True, or None and the room is at most STORED_DS_AUTO_BYTES;
    else the minimal one (dq recomputed)."""
    torch = _torch()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _need(t, name, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if tuple(o.shape) != tuple(q.shape) or tuple(do.shape) != tuple(q.shape):
        raise ValueError("o and do must be shaped like q")
    if tuple(k.shape) != (B, Hkv, N, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, N, D]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = _bwd_workspace(B, Hq, Hkv, N, D, causal, stored_ds, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), B, Hq, Hkv, N, D, scale,
                          1 if causal else 0, _stream(q)))
    return dq, dk, dv


def attn_bwd_noalloc_max_scratch() -> int:
    """Bytes of scratch attn_bwd_noalloc holds per GPU (its size limit)."""
    return int(lib().attn_bwd_noalloc_max_scratch())


def attn_bwd_noalloc(q, k, v, o, do, lse, *, causal: bool = True, scale: float | None = None,
                     dq=None, dk=None, dv=None):
    """attn_bwd with no workspace: the library's own per-GPU scratch serves
    its kernels, so the call allocates nothing when dq, dk, dv are given
    (usable under graph capture).  Calls that may overlap on one GPU share
    that scratch and must be serialised.  Returns (dq, dk, dv)."""
    torch = _torch()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _need(t, name, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if tuple(o.shape) != tuple(q.shape) or tuple(do.shape) != tuple(q.shape):
        raise ValueError("o and do must be shaped like q")
    if tuple(k.shape) != (B, Hkv, N, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, N, D]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _need(t, name, torch.bfloat16, 4)
        if tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{name} has the wrong shape")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, D,
                                  scale, 1 if causal else 0, _stream(q)))
    return dq, dk, dv


def attn_bwd_strided(q, k, v, o, do, lse, *, causal: bool = True, scale: float | None = None, workspace=None,
                     dq=None, dk=None, dv=None, stored_ds: bool | None = None):
    """attn_bwd on [B, H, N, D] views with any batch / head / token strides
    (the last dimension contiguous), e.g. heads of token-major [N, H, D]
    shards: q, o, do (and dq) share one stride set, k, v (and dk, dv)
    another.  dq, dk, dv default to new tensors with the strides of q and k.
    Returns (dq, dk, dv)."""
    torch = _torch()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _need(t, name, torch.bfloat16, 4, strided=True)
    _need(lse, "lse", torch.float32, 3)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if tuple(o.shape) != tuple(q.shape) or tuple(do.shape) != tuple(q.shape):
        raise ValueError("o and do must be shaped like q")
    if tuple(k.shape) != (B, Hkv, N, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, N, D]")
    if tuple(o.stride()) != tuple(q.stride()) or tuple(do.stride()) != tuple(q.stride()):
        raise ValueError("o and do must have the strides of q")
    if tuple(v.stride()) != tuple(k.stride()):
        raise ValueError("k and v must have the same strides")
    dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device) if dv is None else dv
    for t, name, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", k)):
        _need(t, name, torch.bfloat16, 4, strided=True)
        if tuple(t.shape) != tuple(ref.shape) or tuple(t.stride()) != tuple(ref.stride()):
            raise ValueError(f"{name} must have the shape and strides of {'q' if ref is q else 'k'}")
    if workspace is None:
        workspace = _bwd_workspace(B, Hq, Hkv, N, D, causal, stored_ds, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    arr = ctypes.c_int64 * 3
    qs, ks = arr(*q.stride()[:3]), arr(*k.stride()[:3])
    _check(lib().attn_bwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), B, Hq, Hkv, N, D, scale,
                                  1 if causal else 0, qs, ks, _stream(q)))
    return dq, dk, dv


def attn_bwd_delta(o, do, *, delta=None):
    """Dv = <do_i, o_i> per query row (fp32 [B, Hq, Nq]) for attn_bwd_block."""
    torch = _torch()
    _need(o, "o", torch.bfloat16, 4)
    _need(do, "do", torch.bfloat16, 4)
    if tuple(do.shape) != tuple(o.shape):
        raise ValueError("do must be shaped like o")
    B, Hq, Nq, D = o.shape
    delta = torch.empty((B, Hq, Nq), dtype=torch.float32, device=o.device) if delta is None else delta
    _need(delta, "delta", torch.float32, 3)
    if tuple(delta.shape) != (B, Hq, Nq):
        raise ValueError("delta must be [B, Hq, Nq]")
    _check(lib().attn_bwd_delta(o.data_ptr(), do.data_ptr(), delta.data_ptr(), B, Hq, Nq, D, _stream(o)))
    return delta


def attn_bwd_block_workspace_size(B: int, Hq: int, Hkv: int, Nk: int, D: int) -> int:
    return int(lib().attn_bwd_block_workspace_size(B, Hq, Hkv, Nk, D))


def attn_bwd_block_ds_workspace_size(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, D: int) -> int:
    """Workspace bytes with which attn_bwd_block forms dq from stored dS (0:
    not available for this shape)."""
    return int(lib().attn_bwd_block_ds_workspace_size(B, Hq, Hkv, Nq, Nk, D))


def _bwd_block_prepare(q, k, v, do, lse, delta, q_pos0, k_pos0, dq_acc, dq_accumulate, dk_acc, dv_acc,
                       dkv_accumulate, dq, dk, dv, workspace, stored_ds=False):
    """Checks of one block-backward call; allocates the default outputs and
    workspace.  Returns (BwdBlockCall, (B, Hq, Hkv, D), outputs, workspace):
    the caller holds the workspace until the launch is enqueued, or its memory
    could go to the next allocation (another call of the same group)."""
    torch = _torch()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
        _need(t, name, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(delta, "delta", torch.float32, 3)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(do.shape) != tuple(q.shape):
        raise ValueError("do must be shaped like q")
    if tuple(k.shape) != (B, Hkv, Nk, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, Nk, D]")
    if tuple(lse.shape) != (B, Hq, Nq) or tuple(delta.shape) != (B, Hq, Nq):
        raise ValueError("lse and delta must be [B, Hq, Nq]")
    for t, name, dt, shape in ((dq_acc, "dq_acc", torch.float32, q.shape), (dq, "dq", torch.bfloat16, q.shape),
                               (dk_acc, "dk_acc", torch.float32, k.shape), (dv_acc, "dv_acc", torch.float32, k.shape),
                               (dk, "dk", torch.bfloat16, k.shape), (dv, "dv", torch.bfloat16, k.shape)):
        if t is not None:
            _need(t, name, dt, 4)
            if tuple(t.shape) != tuple(shape):
                raise ValueError(f"{name} has the wrong shape")
    if dq_acc is None and dq is None:
        dq = torch.empty_like(q)
    if dk_acc is None and dk is None:
        dk = torch.empty_like(k)
        dv = torch.empty_like(v) if dv is None else dv
    need = attn_bwd_block_workspace_size(B, Hq, Hkv, Nk, D)
    if stored_ds is not False:
        big = attn_bwd_block_ds_workspace_size(B, Hq, Hkv, Nq, Nk, D)
        if big and (stored_ds is True or big <= STORED_DS_AUTO_BYTES):
            need = big
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)

    def ptr(t):
        return t.data_ptr() if t is not None else None

    call = BwdBlockCall(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(), delta.data_ptr(),
                        ptr(dq_acc), ptr(dk_acc), ptr(dv_acc), ptr(dq), ptr(dk), ptr(dv), ptr(workspace),
                        workspace.numel() * workspace.element_size() if workspace is not None else 0, Nq, Nk,
                        int(q_pos0), int(k_pos0), 1 if dq_accumulate else 0, 1 if dkv_accumulate else 0)
    outs = (dq_acc if dq_acc is not None else dq, dk_acc if dk_acc is not None else dk,
            dv_acc if dv_acc is not None else dv)
    return call, (B, Hq, Hkv, D), outs, workspace


def attn_bwd_block(q, k, v, do, lse, delta, *, causal: bool = True, scale: float | None = None,
                   q_pos0: int = 0, k_pos0: int = 0, dq_acc=None, dq_accumulate: bool = False,
                   dk_acc=None, dv_acc=None, dkv_accumulate: bool = False, dq=None, dk=None, dv=None,
                   workspace=None, stored_ds: bool | None = None):
    """Gradients through one KV block (k, v at global position k_pos0) of the
    attention of q, given the global lse and Dv (attn_bwd_delta).  fp32
    accumulators are overwritten, or added to with the *_accumulate flags;
    bf16 dq / dk / dv, when given, receive rounded copies.  The library picks
    the dq path by the workspace's size; without a workspace one is
    allocated with room for stored dS as attn_bwd does (stored_ds).  Returns
    (dq_acc or dq, dk_acc or dk, dv_acc or dv)."""
    c, (B, Hq, Hkv, D), outs, ws = _bwd_block_prepare(q, k, v, do, lse, delta, q_pos0, k_pos0, dq_acc, dq_accumulate,
                                                  dk_acc, dv_acc, dkv_accumulate, dq, dk, dv, workspace, stored_ds)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().attn_bwd_block(c.q, c.k, c.v, c.d_o, c.lse, c.delta, c.dq_acc, c.dk_acc, c.dv_acc, c.dq, c.dk, c.dv,
                                c.workspace, c.workspace_bytes, B, Hq, Hkv, c.Nq, c.Nk, D, scale, 1 if causal else 0,
                                c.q_pos0, c.k_pos0, c.dq_accumulate, c.dkv_accumulate, _stream(q)))
    return outs


def attn_bwd_block_group(calls, *, causal: bool = True, scale: float | None = None):
    """Independent attn_bwd_block calls (1 to 4) in one dK/dV and one dQ
    launch.  calls: dicts with q, k, v, do, lse, delta and optionally q_pos0,
    k_pos0, dq_acc, dq_accumulate, dk_acc, dv_acc, dkv_accumulate, dq, dk, dv,
    workspace (meanings as in attn_bwd_block); B, Hq, Hkv, D are shared.  No
    call may write what another call reads or writes.  Returns, per call,
    (dq_acc or dq, dk_acc or dk, dv_acc or dv)."""
    calls = list(calls)
    if not 1 <= len(calls) <= 4:
        raise ValueError("a group holds 1 to 4 calls")
    arr = (BwdBlockCall * len(calls))()
    outs, dims, keep = [], None, []
    for i, c in enumerate(calls):
        arr[i], d, o, ws = _bwd_block_prepare(c["q"], c["k"], c["v"], c["do"], c["lse"], c["delta"], c.get("q_pos0", 0),
                                          c.get("k_pos0", 0), c.get("dq_acc"), c.get("dq_accumulate", False),
                                          c.get("dk_acc"), c.get("dv_acc"), c.get("dkv_accumulate", False),
                                          c.get("dq"), c.get("dk"), c.get("dv"), c.get("workspace"))
        if dims is not None and d != dims:
            raise ValueError("the calls of a group share B, Hq, Hkv and D")
        dims = d
        outs.append(o)
        keep.append(ws)
    B, Hq, Hkv, D = dims
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().attn_bwd_block_group(arr, len(calls), B, Hq, Hkv, D, scale, 1 if causal else 0,
                                      _stream(calls[0]["q"])))
    del keep  # the launches are enqueued: the stream orders any reuse after them
    return outs


def _relayout_shape(x, P, out, to_head):
    """(N, H, D, element bytes, out) of one relayout operand, allocating out
    when it is None."""
    torch = _torch()
    _need(x, "x", None, 4)
    if x.dtype not in (torch.bfloat16, torch.float16, torch.float32, torch.int16):
        raise TypeError("relayout supports 2- and 4-byte elements")
    eb = x.element_size()
    if to_head:
        Pp, T, H, D = x.shape
        N = Pp * T
        shape = (Pp, max(1, H // Pp) if Pp else 0, N, D)  # H < P: one replicated head per rank
    else:
        Pp, Hp, N, D = x.shape
        H = Pp * Hp
        shape = (Pp, N // Pp if Pp else 0, H, D)
    if Pp != P:
        raise ValueError(f"leading dimension must be P={P}")
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    _need(out, "out", x.dtype, 4)
    return N, H, D, eb, out


def _relayout(fn_name, x, P, out, to_head):
    N, H, D, eb, out = _relayout_shape(x, P, out, to_head)
    _check(getattr(lib(), fn_name)(x.data_ptr(), out.data_ptr(), P, N, H, D, eb, _stream(x)))
    return out


def _relayout_batch(fn_name, xs, P, outs, to_head):
    xs = list(xs)
    if not 1 <= len(xs) <= 8:
        raise ValueError("a batch holds 1 to 8 tensors")
    outs = [None] * len(xs) if outs is None else list(outs)
    if len(outs) != len(xs):
        raise ValueError("outs must have one entry per input")
    shapes = [_relayout_shape(x, P, o, to_head) for x, o in zip(xs, outs)]
    N, _, D, eb, _ = shapes[0]
    if any((n, d, e) != (N, D, eb) for n, _, d, e, _ in shapes):
        raise ValueError("the tensors of a batch share N, D and the element size")
    n = len(xs)
    ins = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    ptrs = (ctypes.c_void_p * n)(*[s[4].data_ptr() for s in shapes])
    heads = (ctypes.c_int * n)(*[s[1] for s in shapes])
    _check(getattr(lib(), fn_name)(n, ins, ptrs, heads, P, N, D, eb, _stream(xs[0])))
    return [s[4] for s in shapes]


def seq_to_head_relayout(x, P: int, *, out=None):
    """[P, N/P, H, D] -> [P, H/P, N, D] (bit copy)."""
    return _relayout("seq_to_head_relayout", x, P, out, True)


def head_to_seq_relayout(y, P: int, *, out=None):
    """[P, H/P, N, D] -> [P, N/P, H, D] (bit copy)."""
    return _relayout("head_to_seq_relayout", y, P, out, False)


def seq_to_head_relayout_batch(xs, P: int, *, outs=None):
    """seq_to_head_relayout of every tensor of xs (1 to 8, same N, D and
    element size, any H) in one launch; returns the outputs."""
    return _relayout_batch("seq_to_head_relayout_batch", xs, P, outs, True)


def head_to_seq_relayout_batch(ys, P: int, *, outs=None):
    """head_to_seq_relayout of every tensor of ys in one launch."""
    return _relayout_batch("head_to_seq_relayout_batch", ys, P, outs, False)


def head_to_seq_reduce(y, P: int, H: int, *, out=None):
    """[P, max(1, H/P), N, D] (bf16 or fp32) -> [P, N/P, H, D] bf16, summing
    the P/H replicas of each head when H < P (gradients of shared key/value
    heads)."""
    torch = _torch()
    _need(y, "y", (torch.bfloat16, torch.float32), 4)
    Pp, Hr, N, D = y.shape
    if Pp != P:
        raise ValueError(f"leading dimension must be P={P}")
    if Hr != max(1, H // P):
        raise ValueError(f"dimension 1 must be max(1, H/P) = {max(1, H // P)}")
    if out is None:
        out = torch.empty((P, N // P if P else 0, H, D), dtype=torch.bfloat16, device=y.device)
    _need(out, "out", torch.bfloat16, 4)
    if tuple(out.shape) != (P, N // P, H, D):
        raise ValueError("out must be [P, N/P, H, D]")
    dt = ATTN_FP32 if y.dtype == torch.float32 else ATTN_BF16
    _check(lib().head_to_seq_reduce(y.data_ptr(), dt, out.data_ptr(), P, N, H, D, _stream(y)))
    return out


def trace_enable(on: bool = True) -> None:
    """Bracket every kernel the library launches with HIP events (measurement only)."""
    _check(lib().attn_trace_enable(1 if on else 0))


def trace_collect(max_kernels: int = 64) -> dict:
    """Per-kernel {name: (total_ms, calls)} of the launches recorded since the
    last collect; waits for their events."""
    name_len = 64
    names = ctypes.create_string_buffer(name_len * max_kernels)
    tot = (ctypes.c_double * max_kernels)()
    calls = (ctypes.c_int * max_kernels)()
    n = lib().attn_trace_collect(names, name_len, tot, calls, max_kernels)
    if n < 0:
        raise AttnError(-n, "trace events could not be read")
    out = {}
    for i in range(n):
        nm = names.raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out[nm] = (tot[i], calls[i])
    return out
