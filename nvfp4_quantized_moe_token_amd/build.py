"""Build the nvfp4moe HIP library (gfx950) in-tree.

    python -m nvfp4_quantized_moe_token_amd.build

compiles every ``csrc/*.hip`` with hipcc for gfx950 and links
``nvfp4_quantized_moe_token_amd/libnvfp4moe.so``.  Fast math stays off and
floating-point contraction is disabled: the quantizer's bit-exactness
depends on IEEE fp32 division and unfused arithmetic.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libnvfp4moe.so")
BUILD_DIR = os.path.join(PKG_DIR, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the nvfp4moe library)")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("command failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    return res


def build(verbose=False):
    """Compile all HIP sources and link the shared library.  Always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources under %s" % CSRC)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
        _run([hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj])
        if verbose:
            print("compiled", os.path.relpath(src, PKG_DIR), flush=True)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("linked", LIB_PATH, flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
