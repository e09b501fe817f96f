"""Build libmmsa.so (gfx950 only) in-tree with hipcc.

    python -m dynamic_sparse_attention_head_amd.build

Each .hip source under csrc/ is compiled to an object in parallel, then the
objects are linked into dynamic_sparse_attention_head_amd/libmmsa.so.  Also
built: the host-AddressSanitizer variant of the library (_build/asan/) and
the peak microbenchmarks (libmmsa_probe.so, probe/peaks.hip).
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


ASAN_LIB = os.path.join(BUILD, "asan", "libmmsa_asan.so")
PROBE_SRC = os.path.join(PKG, "probe", "peaks.hip")
PROBE_LIB = os.path.join(PKG, "libmmsa_probe.so")


def build_probe(verbose=False):
    """The peak microbenchmarks (an MFMA loop and a streaming copy) that
    bench.py --peaks times; a library of their own, outside libmmsa."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


def asan_runtime():
    """Path of the compiler's AddressSanitizer runtime (to preload into the
    host process that loads the ASan build), or None."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def build_asan(objs, verbose=False):
    """The same library with its host layer (argument validation, workspace
    layout, table building: csrc/mmsa_api.hip) built under AddressSanitizer.
    Only host code is instrumented (-Xarch_host); the kernels are the regular
    objects.  Loaded by the ABI tests through MMSA_LIB with the ASan runtime
    preloaded."""
    os.makedirs(os.path.dirname(ASAN_LIB), exist_ok=True)
    obj = os.path.join(os.path.dirname(ASAN_LIB), "mmsa_api_asan.o")
    host_asan = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()
    cmd = [hipcc(), *HIPCC_FLAGS, "-g", *host_asan, "-c", os.path.join(CSRC, "mmsa_api.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (host ASan) failed:\n{r.stdout}\n{r.stderr}")
    others = [o for o in objs if os.path.basename(o) != "mmsa_api.o"]
    tmp = ASAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *"-Xarch_host -fsanitize=address".split(),
           "-shared-libsan", "-o", tmp, obj, *others]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (host ASan) failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


def build(verbose=False, extra=(), asan=True):
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
    if asan:
        build_asan(objs, verbose=verbose)
    build_probe(verbose=verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
