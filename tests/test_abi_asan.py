"""The C layer's host code under AddressSanitizer: test_abi.py runs again, in a child process,
against libbsg_asan.so (host code built with -fsanitize=address, device code as usual) with
the sanitizer runtime preloaded.  No GPU is needed: like test_abi.py it only makes calls that
fail validation or are pure host queries."""
import os
import subprocess
import sys

import pytest

from block_sparse_gqa_pool_amd import build as bld

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_pass_under_asan():
    try:
        runtime = bld.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = bld.lib_path("asan")
    if bld.is_stale("asan"):
        bld.build(variant="asan")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms, "the asan variant is not instrumented"
    env = dict(os.environ, LD_PRELOAD=runtime, BSG_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "AddressSanitizer" not in r.stderr
    assert " passed" in r.stdout
