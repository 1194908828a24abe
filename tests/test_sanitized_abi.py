"""The boundary's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with its host side instrumented and the argument,
refusal and export tests of the C ABI run against it in a child process with
the clang ASan runtime preloaded (no GPU is touched: every call there fails
before device work).  Any invalid access or undefined behaviour in the host
checks aborts the child.
"""
import glob
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

RUNTIMES = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

CHILD = """
import sys
sys.path.insert(0, {root!r})
from conditional_draft_tree_dominotree_amd import binding
binding.library_path = lambda: {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {tests!r}]))
"""


@pytest.mark.skipif(not RUNTIMES, reason="no clang ASan runtime in this image")
def test_abi_checks_under_asan_and_ubsan(tmp_path):
    from conditional_draft_tree_dominotree_amd import _build
    lib = _build.build_host_sanitized(str(tmp_path))
    env = dict(os.environ, LD_PRELOAD=RUNTIMES[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = CHILD.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert re.search(r"\b\d+ passed\b", r.stdout) and not re.search(r"\b\d+ (failed|errors?)\b", r.stdout), tail
