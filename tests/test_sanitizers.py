"""The host code and the oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host sources (argument checks, the batch planner, workspace
sizing, the request planner) and the fp64 oracle are rebuilt with both
sanitizers, and the CPU tests that exercise them -- the C-ABI validation
(test_host_abi.py), the request planner (test_processor.py) and every oracle
pin (test_oracle_pins.py) -- run again in a child process with the clang
sanitizer runtime preloaded.  An out-of-bounds access, use after free,
integer overflow or other undefined behaviour aborts that child, and this test
fails with its output.  No GPU is used: the validation paths return before any
HIP call.
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle as o
from patch_merge_mlp_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_host_code_and_oracle_under_sanitizers(tmp_path):
    lib = b.build_sanitized(str(tmp_path))
    orc = o.build_sanitized(str(tmp_path))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": b.sanitizer_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:new_delete_type_mismatch=0:"
                        "alloc_dealloc_mismatch=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "VLBRIDGE_LIB": lib,
        "VLB_ORACLE_LIB": orc,
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           "tests/test_host_abi.py", "tests/test_processor.py", "tests/test_oracle_pins.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
