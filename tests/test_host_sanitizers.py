"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of the library is built with both sanitizers on its host code (device
code unchanged) and the C-ABI host tests (spec validation, arena and
workspace sizing, argument errors: every path that runs without a GPU) are run
against it in a child process with the sanitizer runtime preloaded.  Any
sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

from weight_shared_rank_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RUNNER = """
import sys
sys.path.insert(0, {root!r})
from weight_shared_rank_amd import binding
binding.LIBPATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {tests!r}]))
"""


@pytest.mark.timeout(900)
def test_abi_host_paths_clean_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc is not installed")
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    lib = build.build_host_sanitized()
    runner = tmp_path / "run_abi_tests.py"
    runner.write_text(RUNNER.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_cpu.py")))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, str(runner)], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=800)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
