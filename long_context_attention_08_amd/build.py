"""Build libdsv4attn.so for gfx950 with hipcc (in-tree, next to this file).

    python long_context_attention_08_amd/build.py
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libdsv4attn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "plan.cpp", "compress.hip", "indexer.hip", "topk.hip", "attn.hip", "normrope.hip", "gemm.hip",
           "stream.hip"]
ARCH = os.environ.get("DSV4_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay disabled in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
]


# Per-file additions.  The indexer's ReLU epilogue is the bulk of its VALU
# work; with IEEE mode off a max needs no operand quieting first (its inputs
# are finite MFMA results), which halves the epilogue.
FILE_FLAGS = {"indexer.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found")
    return h


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + FLAGS + FILE_FLAGS.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if verbose and msg.strip():
        print(msg)
    return obj


def build(verbose=False):
    """Compile every HIP source for gfx950 and link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
