"""The host-side ABI tests again, against the build of the library whose host
layer (argument validation, workspace layout, table building) is compiled
with AddressSanitizer: an out-of-bounds access or use-after-free in the host
code fails this test.  CPU only; skipped when the ASan build is absent."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from dynamic_sparse_attention_head_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_asan():
    if not os.path.exists(B.ASAN_LIB):
        pytest.skip("host-ASan build absent (python -m dynamic_sparse_attention_head_amd.build)")
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("ASan runtime not found")
    env = dict(os.environ, MMSA_LIB=B.ASAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=23")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert "AddressSanitizer" not in r.stderr, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
