"""The C ABI's argument-validation layer (api.cpp, trace.cpp, sizes.cpp)
built for the host with AddressSanitizer and UndefinedBehaviorSanitizer
(device launchers replaced by tests/asan/launch_stubs.cpp), and
tests/test_abi.py run against that build (CPU only, no GPU code)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_attention_fwd_amd", "csrc")
ROCM = "/opt/rocm"


def test_abi_under_host_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("g++ and the ROCm runtime are needed for the host sanitizer build")
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan is not installed")
    lib = str(tmp_path / "libattn_sanitized.so")
    srcs = [os.path.join(CSRC, f) for f in ("api.cpp", "trace.cpp", "sizes.cpp")]
    srcs.append(os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"))
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", *srcs, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
           "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=asan, LCATTN_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
    assert " passed" in r.stdout, out
