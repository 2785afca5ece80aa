"""Build libcowa.so (C ABI + gfx950 HIP kernels) in-tree with hipcc.

    python -m structured_sparse_attention_plan_amd.build        # or build.build()

Every source is compiled for gfx950 with packed-fp32 instructions disabled, then linked
into ``structured_sparse_attention_plan_amd/libcowa.so``.  Object files go to
``_build/`` at the repository root.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcowa.so")

SOURCES = ["planner.cpp", "capi.cpp", "fwd_bf16.hip", "fwd_f32.hip", "bwd_bf16.hip",
           "decode_bf16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file additions.  The forward kernel takes running maxima of scores that are finite
# or -inf, never NaN: without NaN semantics max(max(a, b), c) becomes one v_max3_f32 (IEEE
# NaN rules otherwise keep it as two v_max_f32 per element).
FILE_FLAGS = {
    "fwd_bf16.hip": ["-fno-honor-nans"],
}


def _compile(src):
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose=False):
    """Compile every source and link libcowa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
