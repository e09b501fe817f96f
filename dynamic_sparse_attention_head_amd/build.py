"""Build libmmsa.so (gfx950 only) in-tree with hipcc.

    python -m dynamic_sparse_attention_head_amd.build

Each .hip source under csrc/ is compiled to an object in parallel, then the
objects are linked into dynamic_sparse_attention_head_amd/libmmsa.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmmsa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
# Per-source additions.  The attention kernel never sees a NaN (masked logits are
# -inf, never NaN), so its max/min need no NaN quieting: IEEE mode off lets them
# map to single v_max/v_max3 instructions.
FILE_FLAGS = {
    "k_attention.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
}


def hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return h


def _compile(src, obj, extra):
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False, extra=()):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        futs = []
        for s in srcs:
            obj = os.path.join(BUILD, s[:-4] + ".o")
            futs.append(ex.submit(_compile, os.path.join(CSRC, s), obj, list(extra)))
        for f in futs:
            objs.append(f.result())
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
