"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library is built with the sanitizers on the host side only (the device code
is compiled as in the product build) and tests/test_abi.py runs against it in a
child process that preloads the clang sanitizer runtime.  Those tests drive every
argument check, size query, overlap check and error path of the C ABI without a
GPU, so an out-of-bounds access, use after free or undefined operation in that
code stops the child with a sanitizer report.
"""
import os
import shutil
import subprocess
import sys

import pytest

from linear_rnn_sequence_wkv7_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import ctypes, os, sys
sys.path.insert(0, {root!r})
os.chdir({root!r})
# The sanitizer runtime must be live in this process.
ctypes.CDLL(None).__asan_init
from linear_rnn_sequence_wkv7_amd import wkv7 as W
W.lib_path = lambda: {lib!r}
import pytest
sys.exit(pytest.main(["tests/test_abi.py", "-q", "-p", "no:cacheprovider"]))
"""


@pytest.mark.timeout(900)
def test_abi_under_host_sanitizers(tmp_path):
    try:
        runtime = B.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if runtime is None:
        pytest.skip("no clang sanitizer runtime in the toolchain")
    lib = B.build_host_sanitized(str(tmp_path / "hostsan"))
    if shutil.which("nm"):
        syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
        assert "__asan_" in syms and "__ubsan_" in syms, "the host code is not instrumented"
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=lib)], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout and "failed" not in r.stdout, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
