"""The C ABI: the library loads, exports every function include/attn.h declares,
and rejects bad arguments on the host before touching the GPU (CPU only)."""

import ctypes
import os
import re

import pytest

import long_context_attention_fwd_amd as lc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

A = 0x100000  # 16-byte aligned fake device addresses: never dereferenced on error paths
B_ = 0x10000000
C_ = 0x20000000
D_ = 0x30000000
E_ = 0x40000000
F_ = 0x50000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lc.LIB_PATH):
        pytest.fail("libattn.so is not built (python -m long_context_attention_fwd_amd.build)")
    return lc.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("attn_fwd", "attn_fwd_strided", "attn_fwd_accumulate", "attn_fwd_splitkv", "attn_fwd_splitkv_workspace_size", "attn_bwd",
              "attn_bwd_workspace_size", "attn_bwd_ds_workspace_size", "attn_bwd_delta", "attn_bwd_block", "attn_bwd_block_workspace_size",
              "attn_partial_merge", "head_to_seq_reduce",
              "attn_bwd_strided", "attn_bwd_noalloc", "attn_bwd_block_group", "attn_bwd_noalloc_max_scratch", "attn_fwd_accumulate_group", "attn_fwd_accumulate_group_split",
              "attn_fwd_accumulate_workspace_size", "attn_fwd_split_suggest", "seq_to_head_relayout", "head_to_seq_relayout", "seq_to_head_relayout_batch",
              "head_to_seq_relayout_batch", "attn_status_string", "attn_last_error"):
        assert n in names, names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_status_strings(L):
    assert L.attn_status_string(0) == b"ok"
    for s in range(1, 8):
        assert L.attn_status_string(s) and L.attn_status_string(s) != b"unknown status"
    assert L.attn_status_string(99) == b"unknown status"


def fwd(L, **kw):
    args = dict(q=A, k=B_, v=C_, o=D_, o_dtype=0, lse=E_, B=1, Hq=4, Hkv=1, Nq=128, Nk=128, D=128,
                scale=0.125, causal=1, q_pos0=0, k_pos0=0, stream=None)
    args.update(kw)
    return L.attn_fwd(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(lse=None), 1),
    (dict(B=0), 2), (dict(Nq=0), 2), (dict(Nk=-1), 2), (dict(Hq=4, Hkv=3), 2), (dict(q_pos0=-1), 2),
    (dict(D=96), 3), (dict(D=256), 3), (dict(o_dtype=7), 3), (dict(scale=0.0), 3), (dict(scale=float("nan")), 3),
    (dict(q=A + 8), 4), (dict(lse=E_ + 4), 4),
    (dict(o=A), 5), (dict(lse=B_ + 64), 5), (dict(o=E_ + 16), 5),
])
def test_fwd_rejects(L, kw, status):
    assert fwd(L, **kw) == status
    assert L.attn_last_error()


def splitkv(L, **kw):
    args = dict(q=A, k=B_, v=C_, o=D_, lse=E_, B=1, Hq=4, Hkv=1, Nq=128, Nk=128, D=128, scale=0.125, causal=1,
                q_pos0=0, k_pos0=0, n_splits=2, ws=F_, ws_bytes=1 << 24, stream=None)
    args.update(kw)
    return L.attn_fwd_splitkv(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(B=0), 2), (dict(Hq=4, Hkv=3), 2), (dict(D=96), 3), (dict(n_splits=65), 3),
    (dict(ws=None), 6), (dict(ws_bytes=100), 6), (dict(ws=F_ + 8), 4), (dict(ws=A), 5), (dict(o=A), 5),
    (dict(B=2000, n_splits=64), 3),
])
def test_splitkv_rejects(L, kw, status):
    assert splitkv(L, **kw) == status
    assert L.attn_last_error()


def test_splitkv_workspace_size(L):
    # n ranges of fp32 partial O and LSE: n * B*Hq*Nq*(D+1) floats
    assert L.attn_fwd_splitkv_workspace_size(1, 4, 1, 128, 128, 128, 1, 2) == 2 * 4 * 128 * 129 * 4
    assert L.attn_fwd_splitkv_workspace_size(1, 4, 1, 128, 128, 128, 1, 65) == 0
    assert L.attn_fwd_splitkv_workspace_size(1, 4, 3, 128, 128, 128, 1, 2) == 0
    auto = L.attn_fwd_splitkv_workspace_size(1, 4, 4, 4096, 4096, 64, 1, 0)
    per_range = 4 * 4096 * 65 * 4
    assert auto % per_range == 0 and 1 <= auto // per_range <= 64


def strided(L, qs=(0, 128, 4096), ks=(0, 128, 512), os_=(0, 128, 512), **kw):
    arr = ctypes.c_int64 * 3
    args = dict(q=A, k=B_, v=C_, o=D_, o_dtype=0, lse=E_, B=1, Hq=4, Hkv=1, Nq=128, Nk=128, D=128,
                scale=0.125, causal=1, q_pos0=0, k_pos0=0, qs=arr(*qs) if qs else None,
                ks=arr(*ks) if ks else None, os_=arr(*os_) if os_ else None, stream=None)
    args.update(kw)
    return L.attn_fwd_strided(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(qs=None), 1), (dict(os_=None), 1), (dict(qs=(0, -128, 4096)), 2), (dict(qs=(0, 128, 4100)), 4),
    (dict(ks=(0, 0, 64)), 2), (dict(ks=(0, 0, 1 << 24)), 3), (dict(os_=(0, 64, 512)), 5),
    (dict(os_=(0, 128, 128)), 5), (dict(o=A + 256), 5), (dict(D=96), 3),
])
def test_strided_rejects(L, kw, status):
    assert strided(L, **kw) == status
    assert L.attn_last_error()


def group_call(L, calls, n=None, B=1, Hq=4, Hkv=1, D=128, scale=0.125, causal=1):
    arr = (lc.AccumulateCall * max(1, len(calls)))(*[lc.AccumulateCall(*c) for c in calls])
    return L.attn_fwd_accumulate_group(arr if calls else None, len(calls) if n is None else n, B, Hq, Hkv, D, scale,
                                       causal, None)


def test_accumulate_group_rejects(L):
    # call: q, k, v, o_acc, lse_acc, o_final, Nq, Nk, q_pos0, k_pos0, first (Nq = Nk = 128: q, o_acc 256 KiB apart)
    c0 = (A, B_, C_, D_, E_, None, 128, 128, 0, 0, 1)
    c1 = (A + (1 << 20), B_, C_, D_ + (1 << 20), E_ + (1 << 20), None, 128, 128, 128, 0, 0)
    assert group_call(L, []) == 1
    assert group_call(L, [c0], n=0) == 2
    assert group_call(L, [c0] * 5) == 2
    assert group_call(L, [c0, (None,) + c1[1:]]) == 1
    assert b"call 1" in L.attn_last_error()
    assert group_call(L, [c0, c1[:3] + (D_ + 64,) + c1[4:]]) == 5          # o_acc of call 1 overlaps call 0's
    assert group_call(L, [c0, c1[:3] + (A + 512,) + c1[4:]]) == 5          # o_acc of call 1 overlaps q of call 0
    assert group_call(L, [c0, c1[:5] + (F_ + 8,) + c1[6:]]) == 4           # misaligned o_final
    assert group_call(L, [c0], D=96) == 3
    assert group_call(L, [c0] * 4, B=20000) == 3                           # grid z = B * n too large


W_ = 0x60000000  # fake workspace address


def split_group_call(L, calls, n=None, n_splits=2, B=1, Hq=4, Hkv=1, D=128, scale=0.125, causal=1):
    arr = (lc.AccumulateSplitCall * max(1, len(calls)))(
        *[lc.AccumulateSplitCall(lc.AccumulateCall(*c), ws, wb) for c, ws, wb in calls])
    return L.attn_fwd_accumulate_group_split(arr if calls else None, len(calls) if n is None else n, B, Hq, Hkv, D,
                                             scale, causal, n_splits, None)


def test_accumulate_workspace_size_and_suggestion(L):
    assert L.attn_fwd_accumulate_workspace_size(1, 4, 128, 128, 2) == 2 * 4 * 128 * (128 + 1) * 4
    assert L.attn_fwd_accumulate_workspace_size(1, 4, 128, 128, 0) == 0
    assert L.attn_fwd_accumulate_workspace_size(1, 4, 128, 128, 65) == 0
    assert L.attn_fwd_split_suggest(1, 4, 1, 4096, 4096, 1, 2) >= 1
    assert L.attn_fwd_split_suggest(1, 4, 3, 4096, 4096, 1, 2) == 1  # Hkv does not divide Hq: no split
    # long rows fill the GPU without a split
    assert L.attn_fwd_split_suggest(1, 8, 8, 1 << 16, 1 << 16, 1, 1) == 1


def test_accumulate_group_split_rejects(L):
    """Every case fails validation (nothing is launched)."""
    need = L.attn_fwd_accumulate_workspace_size(1, 4, 128, 128, 2)
    c0 = ((A, B_, C_, D_, E_, None, 128, 128, 0, 0, 1), W_, need)
    c1 = ((A + (1 << 20), B_, C_, D_ + (1 << 20), E_ + (1 << 20), None, 128, 128, 128, 0, 0), W_ + (1 << 24), need)
    assert split_group_call(L, []) == 1
    assert split_group_call(L, [c0], n=0) == 2
    assert split_group_call(L, [c0] * 5) == 2
    assert split_group_call(L, [c0], n_splits=0) == 3
    assert split_group_call(L, [c0], n_splits=65) == 3
    assert split_group_call(L, [c0, c1], B=20000, n_splits=4) == 3        # grid z = B * n * splits too large
    assert split_group_call(L, [c0, ((None,) + c1[0][1:], c1[1], c1[2])]) == 1
    assert b"call 1" in L.attn_last_error()
    assert split_group_call(L, [(c0[0], None, need)]) == 6                 # no workspace
    assert split_group_call(L, [(c0[0], W_, need - 16)]) == 6              # workspace too small
    assert split_group_call(L, [(c0[0], W_ + 8, need)]) == 4               # misaligned workspace
    assert split_group_call(L, [(c0[0], A + 256, need)]) == 5              # workspace overlaps q
    assert split_group_call(L, [c0, (c1[0], W_ + 1024, need)]) == 5        # workspaces of two calls overlap
    assert split_group_call(L, [c0, (c1[0], D_ + (1 << 20) + 64, need)]) == 5  # workspace overlaps call 1's o_acc
    assert split_group_call(L, [c0, (c1[0][:3] + (D_ + 64,) + c1[0][4:], c1[1], c1[2])]) == 5  # outputs overlap


def bwd_strided(L, qs=(0, 128, 1024), ks=(0, 128, 256), **kw):
    """Token-major shard of 8 query heads on 2 key/value heads, N = 1024, D = 128:
    q, o, d_o, dq rows 2 KiB apart, k, v, dk, dv rows 512 B apart (each tensor
    spans 2 MiB or 512 KiB from its base)."""
    arr = ctypes.c_int64 * 3
    n = 1 << 22
    args = dict(q=A, k=A + n, v=A + 2 * n, o=A + 3 * n, do=A + 4 * n, lse=A + 5 * n, dq=A + 6 * n, dk=A + 7 * n,
                dv=A + 8 * n, ws=A + 9 * n, ws_bytes=L.attn_bwd_workspace_size(1, 8, 2, 1024, 128), B=1, Hq=8,
                Hkv=2, N=1024, D=128, scale=0.088, causal=1, qs=arr(*qs) if qs else None,
                ks=arr(*ks) if ks else None, stream=None)
    args.update(kw)
    return L.attn_bwd_strided(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(qs=None), 1), (dict(ks=None), 1), (dict(dq=None), 1),
    (dict(qs=(0, -128, 1024)), 2),            # negative stride
    (dict(qs=(0, 128, 1028)), 4),             # rows not 16-byte aligned
    (dict(ks=(0, 0, 64)), 2),                 # token stride < D
    (dict(ks=(0, 128, 1 << 24)), 3),          # token stride beyond the kernels' offsets
    (dict(qs=(0, 64, 1024)), 5),              # dq rows of neighbouring heads overlap
    (dict(ks=(0, 0, 256)), 5),                # dk rows of the two heads coincide
    (dict(dq=A + (1 << 22) + 4096), 5),       # dq overlaps k
    (dict(dv=A + (7 << 22) + 256), 5),        # dv overlaps dk
    (dict(ws=None), 6), (dict(D=96), 3), (dict(Hkv=3), 2),
])
def test_bwd_strided_rejects(L, kw, status):
    assert bwd_strided(L, **kw) == status
    assert L.attn_last_error()


def accumulate(L, **kw):
    args = dict(q=A, k=B_, v=C_, o=D_, lse=E_, o_final=F_, B=1, Hq=4, Hkv=1, Nq=128, Nk=128, D=128, scale=0.125,
                causal=1, q_pos0=0, k_pos0=0, first=0, stream=None)
    args.update(kw)
    return L.attn_fwd_accumulate(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(Nk=0), 2), (dict(D=96), 3), (dict(o_final=F_ + 8), 4),
    (dict(o_final=A + 1024), 5), (dict(o=A), 5),
])
def test_accumulate_rejects(L, kw, status):
    assert accumulate(L, **kw) == status
    assert L.attn_last_error()


def merge(L, **kw):
    args = dict(o_parts=A, part_dtype=1, lse_parts=B_, n_parts=4, o=C_, lse=D_, B=1, H=8, N=1024, D=128, stream=None)
    args.update(kw)
    return L.attn_partial_merge(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(o_parts=None), 1), (dict(n_parts=0), 2), (dict(N=0), 2), (dict(D=80), 3), (dict(part_dtype=5), 3),
    (dict(o=C_ + 2), 4), (dict(o=A + 4096), 5), (dict(lse=B_), 5),
])
def test_merge_rejects(L, kw, status):
    assert merge(L, **kw) == status


def test_bwd_workspace_size(L):
    assert L.attn_bwd_workspace_size(1, 8, 8, 65536, 128) >= 8 * 65536 * 4
    # the glossary example's backward splits its passes: 4 query ranges of dK,
    # dV partials and 8 key ranges of dQ partials (fp32), then Dv
    assert L.attn_bwd_workspace_size(1, 4, 4, 4096, 64) == (2 * 4 + 8) * 4 * 4096 * 64 * 4 + 4 * 4096 * 4
    assert L.attn_bwd_workspace_size(1, 8, 3, 1024, 128) == 0
    assert L.attn_bwd_workspace_size(0, 8, 8, 1024, 128) == 0


def test_bwd_ds_workspace_size(L):
    # the 64K training shape: Dv (8 heads x 65536 rows, fp32) then, for each
    # head, the dS blocks at or left of the diagonal in pairs of key tiles:
    # query tile qt (of 1024) has 2 (qt // 2) + 2 blocks of 64 x 64 bf16
    blocks = sum(2 * (qt // 2) + 2 for qt in range(1024))
    assert blocks == 2 * 512 * 513
    assert L.attn_bwd_ds_workspace_size(1, 8, 8, 65536, 128, 1) == 8 * 65536 * 4 + 8 * blocks * 8192
    # without the mask every block of the 1024 x 1024 grid
    assert L.attn_bwd_ds_workspace_size(1, 8, 8, 65536, 128, 0) == 8 * 65536 * 4 + 8 * 1024 * 1024 * 8192
    # grouped heads: the per-query-head dK, dV partials sit before the blocks
    # (Dv 4 x 32768 floats, partials 2 x 4 x 32768 x 128 floats)
    blocks = sum(2 * (qt // 2) + 2 for qt in range(512))
    assert L.attn_bwd_ds_workspace_size(1, 4, 1, 32768, 128, 1) == (4 * 32768 + 2 * 4 * 32768 * 128) * 4 + \
        4 * blocks * 8192
    # ragged N: an odd number of query tiles (33), rows of key-tile pairs;
    # the first part padded to 256 bytes (Dv of 2 x 8 x 2100 rows, 64-float padded)
    first = (2 * 8 * 2100 + 63) // 64 * 64 * 4
    first = (first + 255) // 256 * 256
    assert L.attn_bwd_ds_workspace_size(2, 8, 8, 2100, 64, 1) == first + 2 * 8 * sum(2 * (qt // 2) + 2 for qt in
                                                                                    range(33)) * 8192
    # small problems (fewer than 256 dK/dV workgroups) have no such path
    assert L.attn_bwd_ds_workspace_size(1, 4, 4, 4096, 64, 1) == 0
    assert L.attn_bwd_ds_workspace_size(1, 8, 8, 4096, 128, 1) > 0  # 8 x 32 workgroups
    assert L.attn_bwd_ds_workspace_size(1, 8, 8, 3968, 128, 1) == 0  # 8 x 31
    assert L.attn_bwd_ds_workspace_size(1, 8, 3, 65536, 128, 1) == 0
    assert L.attn_bwd_ds_workspace_size(1, 8, 8, 65536, 96, 1) == 0


def test_bwd_block_ds_workspace_size(L):
    # grouped heads: the per-query-head dK, dV partials (2 B Hq Nk D floats),
    # padded to 256 bytes, then ceil(Nq / 64) rows of 2 ceil(Nk / 128)
    # blocks of 64 x 64 bf16 per batch and query head
    part = 2 * 2 * 16 * 1100 * 128 * 4
    assert part % 256 == 0
    assert L.attn_bwd_block_ds_workspace_size(2, 16, 4, 3000, 1100, 128) == part + 2 * 16 * 47 * 18 * 8192
    # no grouped heads: no partials
    assert L.attn_bwd_block_ds_workspace_size(1, 32, 32, 648, 1024, 64) == 32 * 11 * 16 * 8192
    # fewer than 256 dK/dV workgroups, bad sizes
    assert L.attn_bwd_block_ds_workspace_size(2, 16, 4, 3000, 700, 128) == 0
    assert L.attn_bwd_block_ds_workspace_size(2, 16, 3, 3000, 1100, 128) == 0
    assert L.attn_bwd_block_ds_workspace_size(2, 16, 4, 0, 1100, 128) == 0
    assert L.attn_bwd_block_ds_workspace_size(2, 16, 4, 3000, 1100, 96) == 0


def test_bwd_ds_workspace_selects_path(L):
    """A workspace between the two sizes is accepted (recomputing path); one
    below the minimum is refused."""
    need = L.attn_bwd_workspace_size(1, 8, 8, 4096, 128)
    big = L.attn_bwd_ds_workspace_size(1, 8, 8, 4096, 128, 1)
    assert big > need > 0
    n = 1 << 24
    common = (A, A + n, A + 2 * n, A + 3 * n, A + 4 * n, A + 5 * n, A + 6 * n, A + 7 * n, A + 8 * n, A + 9 * n)
    # null stream pointer on a machine without a GPU: validation runs first,
    # so a too-small workspace is reported before any launch
    rc = L.attn_bwd(*common, need - 16, 1, 8, 8, 4096, 128, 0.088, 1, None)
    assert rc == 6  # ATTN_ERR_WORKSPACE


def bwd(L, **kw):
    n = 1 << 22
    args = dict(q=A, k=A + n, v=A + 2 * n, o=A + 3 * n, do=A + 4 * n, lse=A + 5 * n, dq=A + 6 * n, dk=A + 7 * n,
                dv=A + 8 * n, ws=A + 9 * n, ws_bytes=L.attn_bwd_workspace_size(1, 8, 8, 1024, 128), B=1, Hq=8,
                Hkv=8, N=1024, D=128, scale=0.088, causal=1, stream=None)
    args.update(kw)
    return L.attn_bwd(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(dq=None), 1), (dict(N=0), 2), (dict(Hkv=3), 2), (dict(D=32), 3), (dict(scale=-1.0), 3),
    (dict(ws=None), 6), (dict(ws_bytes=100), 6), (dict(dk=A + 8), 4), (dict(dq=A), 5),
])
def test_bwd_rejects(L, kw, status):
    assert bwd(L, **kw) == status


def bwd_noalloc(L, **kw):
    n = 1 << 22
    args = dict(q=A, k=A + n, v=A + 2 * n, o=A + 3 * n, do=A + 4 * n, lse=A + 5 * n, dq=A + 6 * n, dk=A + 7 * n,
                dv=A + 8 * n, B=1, Hq=8, Hkv=8, N=1024, D=128, scale=0.088, causal=1, stream=None)
    args.update(kw)
    return L.attn_bwd_noalloc(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(dq=None), 1), (dict(N=0), 2), (dict(Hkv=3), 2), (dict(D=32), 3), (dict(scale=-1.0), 3),
    (dict(dk=A + 8), 4), (dict(dq=A), 5),
    # scratch beyond the library's per-GPU array: Dv + fp32 partials of 4 x 16 query heads
    (dict(B=4, Hq=16, Hkv=4, N=32768), 6),
])
def test_bwd_noalloc_rejects(L, kw, status):
    """Every check runs on the host before the scratch lookup (the first GPU
    call), so bad arguments fail here without a GPU."""
    assert bwd_noalloc(L, **kw) == status


def test_bwd_noalloc_limit(L):
    cap = L.attn_bwd_noalloc_max_scratch()
    assert cap == 160 << 20
    # the two backward shapes of the workloads fit: the 64K training shape
    # (8 heads, Dv only) and the 32K Ulysses shard (4 query heads on 1 KV head)
    assert L.attn_bwd_workspace_size(1, 8, 8, 65536, 128) <= cap
    assert L.attn_bwd_workspace_size(1, 4, 1, 32768, 128) <= cap
    assert L.attn_bwd_workspace_size(4, 16, 4, 32768, 128) > cap
    assert bwd_noalloc(L, B=4, Hq=16, Hkv=4, N=32768) == 6
    assert b"scratch" in L.attn_last_error()


@pytest.mark.parametrize("args,status", [
    ((None, B_, C_, 1, 8, 1024, 128), 1), ((A, B_, C_, 1, 8, 0, 128), 2), ((A, B_, C_, 1, 8, 1024, 96), 3),
    ((A, B_, C_ + 4, 1, 8, 1024, 128), 4), ((A, B_, A + 1024, 1, 8, 1024, 128), 5),
])
def test_bwd_delta_rejects(L, args, status):
    assert L.attn_bwd_delta(*args, None) == status


def test_bwd_block_workspace_size(L):
    assert L.attn_bwd_block_workspace_size(1, 8, 8, 4096, 128) == 0          # no group: no partials
    assert L.attn_bwd_block_workspace_size(1, 8, 2, 4096, 128) == 2 * 8 * 4096 * 128 * 4
    assert L.attn_bwd_block_workspace_size(1, 8, 3, 4096, 128) == 0
    assert L.attn_bwd_block_workspace_size(1, 8, 8, 0, 128) == 0


def bwd_block(L, **kw):
    n = 1 << 24
    args = dict(q=A, k=A + n, v=A + 2 * n, do=A + 3 * n, lse=A + 4 * n, delta=A + 5 * n, dq_acc=A + 6 * n,
                dk_acc=A + 7 * n, dv_acc=A + 8 * n, dq=A + 9 * n, dk=A + 10 * n, dv=A + 11 * n, ws=A + 12 * n,
                ws_bytes=1 << 24, B=1, Hq=8, Hkv=2, Nq=1024, Nk=512, D=128, scale=0.088, causal=1, q_pos0=512,
                k_pos0=0, dq_accumulate=1, dkv_accumulate=0, stream=None)
    args.update(kw)
    return L.attn_bwd_block(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(delta=None), 1),
    (dict(dq_acc=None, dq=None), 1),
    (dict(dk_acc=None), 1),                                   # dk_acc and dv_acc come together
    (dict(dk=None), 1),
    (dict(dk_acc=None, dv_acc=None, dk=None, dv=None), 1),
    (dict(dq_acc=None), 1),                                   # accumulate without the fp32 dQ
    (dict(Nk=0), 2), (dict(Hkv=3), 2), (dict(q_pos0=-1), 2),
    (dict(D=32), 3), (dict(scale=0.0), 3), (dict(Nq=1 << 30), 3),
    (dict(ws=None), 6), (dict(ws_bytes=1000), 6),
    (dict(dv=A + (11 << 24) + 8), 4),
    (dict(dq_acc=A + (1 << 24) + 64), 5),                    # dq_acc overlaps k
    (dict(dk=A + (7 << 24)), 5),                              # dk overlaps dk_acc
])
def test_bwd_block_rejects(L, kw, status):
    assert bwd_block(L, **kw) == status
    assert L.attn_last_error()


def bwd_group_call(base, **kw):
    """One attn_bwd_block_call with its own 13 fake buffers (16 MiB apart) from base."""
    n = 1 << 24
    f = dict(q=base, k=base + n, v=base + 2 * n, d_o=base + 3 * n, lse=base + 4 * n, delta=base + 5 * n,
             dq_acc=base + 6 * n, dk_acc=base + 7 * n, dv_acc=base + 8 * n, dq=base + 9 * n, dk=base + 10 * n,
             dv=base + 11 * n, workspace=base + 12 * n, workspace_bytes=1 << 24, Nq=1024, Nk=512, q_pos0=512,
             k_pos0=0, dq_accumulate=1, dkv_accumulate=1)
    f.update(kw)
    return lc.BwdBlockCall(**f)


def bwd_group(L, calls, n=None, **kw):
    arr = (lc.BwdBlockCall * max(1, len(calls)))(*calls)
    args = dict(calls=arr, n=len(calls) if n is None else n, B=1, Hq=8, Hkv=2, D=128, scale=0.088, causal=1,
                stream=None)
    args.update(kw)
    return L.attn_bwd_block_group(*args.values())


def test_bwd_block_group_rejects(L):
    """The group validates every call as attn_bwd_block (the error names the
    call) and rejects calls that write what another call reads or writes."""
    c0 = bwd_group_call(A)
    c1 = bwd_group_call(A + (16 << 24))
    assert bwd_group(L, [c0], n=0) == 2 and bwd_group(L, [c0] * 5, n=5) == 2
    assert L.attn_bwd_block_group(None, 1, 1, 8, 2, 128, 0.088, 1, None) == 1
    bad = bwd_group_call(A + (16 << 24), delta=None)
    assert bwd_group(L, [c0, bad]) == 1 and b"call 1" in L.attn_last_error()
    assert bwd_group(L, [c0, bwd_group_call(A + (16 << 24), Nk=0)]) == 2
    assert bwd_group(L, [c0, bwd_group_call(A + (16 << 24), workspace=None)]) == 6
    # the second call adds into the first call's dQ accumulator
    shared_dq = bwd_group_call(A + (16 << 24), dq_acc=A + 6 * (1 << 24))
    assert bwd_group(L, [c0, shared_dq]) == 5 and b"overlap" in L.attn_last_error()
    # the second call writes its dK into the first call's q
    writes_input = bwd_group_call(A + (16 << 24), dk=A)
    assert bwd_group(L, [c0, writes_input]) == 5
    assert bwd_group(L, [c0, c1], B=65535) == 3


@pytest.mark.parametrize("fn", ["seq_to_head_relayout", "head_to_seq_relayout"])
@pytest.mark.parametrize("args,status", [
    ((None, B_, 8, 4096, 32, 128, 2), 1),
    ((A, B_, 8, 4095, 32, 128, 2), 2),
    ((A, B_, 8, 4096, 12, 128, 2), 2),
    ((A, B_, 8, 4096, 32, 128, 3), 3),
    ((A, B_, 8, 4096, 32, 12, 2), 3),
    ((A + 2, B_, 8, 4096, 32, 128, 2), 4),
    ((A, A + 1024, 8, 4096, 32, 128, 2), 5),
])
def test_relayout_rejects(L, fn, args, status):
    assert getattr(L, fn)(*args, None) == status


def test_relayout_shared_heads(L):
    # H < P: replication is valid for seq->head only when H divides P; the
    # plain inverse refuses replicated heads (their gradients must be summed)
    assert L.seq_to_head_relayout(A, B_, 8, 4096, 3, 128, 2, None) == 2
    assert L.seq_to_head_relayout(A + 4 * 4096 * 256 - 16, A, 8, 4096, 4, 128, 2, None) == 5  # replicated out reaches in
    assert L.head_to_seq_relayout(A, B_, 8, 4096, 4, 128, 2, None) == 3


def batch_call(L, fn, ins, outs, heads, P=8, N=4096, D=128, eb=2):
    n = len(ins)
    arr = lambda t, xs: (t * max(1, n))(*xs) if xs is not None else None
    return getattr(L, fn)(n, arr(ctypes.c_void_p, ins), arr(ctypes.c_void_p, outs), arr(ctypes.c_int, heads),
                          P, N, D, eb, None)


MiB = 1 << 20


@pytest.mark.parametrize("fn", ["seq_to_head_relayout_batch", "head_to_seq_relayout_batch"])
def test_relayout_batch_rejects(L, fn):
    # tensors of [8, 512, H, 128] bf16: 1 MiB per 8 heads
    ins, outs, heads = [A, B_, C_], [D_, E_, F_], [32, 8, 8]
    assert getattr(L, fn)(3, None, None, None, 8, 4096, 128, 2, None) == 1
    assert batch_call(L, fn, [], [], [], ) == 2                          # n = 0
    assert batch_call(L, fn, [A] * 9, [B_] * 9, [32] * 9) == 2            # n > 8
    assert batch_call(L, fn, [A, None], [D_, E_], [32, 8]) == 1           # a null tensor
    assert batch_call(L, fn, ins, outs, [32, 12, 8]) == 2                 # P does not divide H of tensor 1
    assert b"tensor 1" in L.attn_last_error()
    assert batch_call(L, fn, [A, B_ + 2], [D_, E_], [32, 8]) == 4         # misaligned
    assert batch_call(L, fn, [A, B_], [D_, A + 64], [32, 8]) == 5         # output 1 overlaps input 0
    assert batch_call(L, fn, [A, B_], [D_, D_ + 2 * MiB], [32, 8]) == 5   # outputs 0 and 1 overlap
    assert batch_call(L, fn, [A], [B_], [32], N=4095) == 2
    assert batch_call(L, fn, [A], [B_], [32], eb=3) == 3


def test_relayout_batch_shared_heads(L):
    # replication only on the way to heads; the inverse refuses it as the single call does
    assert batch_call(L, "seq_to_head_relayout_batch", [A, B_], [D_, E_], [32, 3]) == 2
    assert batch_call(L, "head_to_seq_relayout_batch", [A, B_], [D_, E_], [32, 4]) == 3


@pytest.mark.parametrize("args,status", [
    ((None, 0, B_, 8, 4096, 4, 128), 1),
    ((A, 0, B_, 8, 4095, 4, 128), 2),
    ((A, 0, B_, 8, 4096, 3, 128), 2),
    ((A, 0, B_, 8, 4096, 12, 128), 2),
    ((A, 2, B_, 8, 4096, 4, 128), 3),
    ((A, 0, B_, 8, 4096, 4, 12), 3),
    ((A + 8, 0, B_, 8, 4096, 4, 128), 4),
    ((A, 1, A + 1024, 8, 4096, 4, 128), 5),
])
def test_head_to_seq_reduce_rejects(L, args, status):
    assert L.head_to_seq_reduce(*args, None) == status


def test_binding_raises_on_missing_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lc.attn_fwd(x, x, x)


def test_trace_hook_without_launches(L):
    assert L.attn_trace_enable(1) == 0
    assert lc.trace_collect() == {}
    assert L.attn_trace_enable(0) == 0
