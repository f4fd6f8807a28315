"""The host-side ABI tests (argument checks, workspace sizing, status strings,
exported symbols) run again against a copy of the library whose host code is
built with AddressSanitizer and UndefinedBehaviorSanitizer.  No GPU is needed:
every call these tests make is rejected or answered on the host before any
device work, so the sanitizers see the whole of that path."""
import os
import shutil
import subprocess
import sys

import pytest

from fp4_kv_cache_layer_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RUNNER = """
import sys
sys.path.insert(0, {root!r})
from fp4_kv_cache_layer_amd import _lib
_lib.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                      {tests!r}]))
"""


def test_abi_under_host_sanitizers(tmp_path):
    rt = B.asan_runtime()
    if rt is None or shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()):
        pytest.skip("no hipcc or no clang AddressSanitizer runtime")
    lib = B.build_sanitized(str(tmp_path / "san"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    # leaks: the Python interpreter's own allocations are not this library's;
    # link order: the runtime is preloaded into an interpreter not built with it
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    code = RUNNER.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=str(tmp_path), capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert " passed" in out, out[-2000:]
