"""Build step of the HIP library: compile every source for gfx950 and link
``libattn.so`` next to this file.

Usage: ``python -m long_context_attention_fwd_amd.build`` (or call ``build()``).
Flags: -O3, C++17, wave64 gfx950 code only, and packed fp32 arithmetic turned
off in device code (``-packed-fp32-ops``)."""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["api.cpp", "trace.cpp", "sizes.cpp", "relayout.hip", "merge.hip", "attn_fwd.hip", "attn_bwd.hip",
           "attn_bwd_ds.hip", "attn_bwd_dkdv_recompute.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]
# The forward's row maximum is a chain of fmaxf; without NaN semantics the
# compiler drops the quieting of each operand.  The row maximum may then skip
# a NaN score, but the NaN still reaches the row through exp2, the row sum and
# the products, and the epilogue decides whether a row is empty from key
# positions, never from the (then NaN) sum; the GPU tests feed NaN and Inf
# inputs.  Without signed zeros the compiler drops the 0 + x that starts each
# partial row sum (the sign of a zero sum does not matter: a row's sum is
# positive or the row is empty).
# The dK/dV kernel instances that store dS (D = 128, contiguous tensors;
# attn_bwd_ds.hip) are scheduled by the backend's iterative ILP strategy: the
# same results, measured 1.7% faster on the dK/dV pass of a 64K-token causal
# backward and 4.4% on a 32K-token 4-head shard (the max-ILP, min-register
# and max-occupancy strategies measured the same or slower).  The rest of the
# backward keeps the default: there the same strategy makes the recomputing
# path's dK/dV instance spill (140 bytes per lane) and run 25% slower, and
# the strided instances spill too; the forward gains nothing from any of them.
# The recomputing path's dense dK/dV instances (attn_bwd_dkdv_recompute.hip)
# take the max-ILP strategy: 1.2% faster at 64K tokens and 5.5% on the shard,
# same results (on the whole file it adds spills to eleven kernels).
PER_FILE = {"attn_fwd.hip": ["-fno-honor-nans", "-fno-signed-zeros"],
            "attn_bwd_ds.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
            "attn_bwd_dkdv_recompute.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *DEVICE, *PER_FILE.get(src, []), "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-x", "c++", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources (always) and link libattn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
