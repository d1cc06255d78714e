"""The library's host code (argument checks, partition planning, pointer queries, launch paths)
built with AddressSanitizer and UndefinedBehaviorSanitizer, and driven through every C entry point
by tests/test_abi.py in a child process that preloads the sanitizer runtime. CPU only: the ABI
cases never reach a kernel launch. Any sanitizer report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

from paged_kv_cache_384_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_abi_cases_under_host_sanitizers(tmp_path):
    if not os.path.exists(_build.hipcc()) or shutil.which("nm") is None:
        pytest.skip("hipcc or nm missing")
    runtime = _build.asan_runtime()
    if not os.path.exists(runtime):
        pytest.skip("no ASan runtime next to hipcc's clang")
    lib = _build.build(extra_flags=_build.HOST_SANITIZE_FLAGS,
                       out=str(tmp_path / "libpa_sanitized.so"))
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True,
                               text=True, check=True).stdout
    assert "__asan_report" in undefined and "__ubsan_handle" in undefined  # instrumented
    env = dict(os.environ, LD_PRELOAD=runtime, PA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-s", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout and "skipped" not in r.stdout.splitlines()[-1], r.stdout[-2000:]
