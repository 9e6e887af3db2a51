"""The host-only ABI checks of tests/test_capi_host.py, run against
libjano_asan.so: the same library with its host code (argument validation,
geometry planning, launch set-up) built with AddressSanitizer. Any invalid
host memory access on those paths aborts the run with an ASan report. No GPU
is touched: every call in those checks returns before a launch."""
import os
import subprocess
import sys

import pytest

from token_sparse_attention_block_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_checks_under_asan():
    if not os.path.exists(B.ASAN_LIB):
        pytest.skip("libjano_asan.so not built (run __graft_entry__.build())")
    env = dict(os.environ, LD_PRELOAD=B.asan_runtime(), JANO_LIB=B.ASAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_capi_host.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and "skipped" not in out.split("\n")[-2], out[-2000:]
