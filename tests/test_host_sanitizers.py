"""The C ABI (api.cpp) and the host planners (plan.cpp) under AddressSanitizer
and UndefinedBehaviorSanitizer: both built with g++ for the host only, linked
against launcher stand-ins that run no kernel (tests/sanitize/launch_stubs.cpp),
and the ABI test suite (argument checks, size queries, workspace sweeps, launch
plans) run on that library in a subprocess.  Any sanitizer report fails the
test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_attention_08_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _runtime(gxx, name):
    p = subprocess.run([gxx, "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_abi_suite_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    asan = _runtime(gxx, "libasan.so")
    if asan is None:
        pytest.skip("no libasan")
    so = str(tmp_path / "libdsv4attn_host_san.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           "-o", so, "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=asan, DSV4ATTN_LIB=so,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=97",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, out
    assert " passed" in r.stdout, out
