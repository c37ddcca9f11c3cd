"""The library's host code (argument checks, workspace carving, status strings) under
AddressSanitizer, on the CPU: a host-only build with ASan on the host code
(build.build_asan()) runs every check of tests/test_abi.py in a child process with the ASan
runtime preloaded; an invalid read or write in those paths aborts the child with a report."""

import os
import subprocess
import sys

import pytest

from block_sparse_linear_02_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_address_sanitizer():
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_asan()
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["SLA_TEST_LIB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
