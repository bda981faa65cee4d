"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is rebuilt with its host code
instrumented (device code unchanged), and the ABI tests -- exports, every
validation path, per-thread error messages -- run against it in a fresh
process with the sanitizer runtime preloaded.  Any report fails the run.
Host only: no kernel is launched."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "query_aware_kv_amd")


def test_abi_tests_clean_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, PKG)
    try:
        import build
    finally:
        sys.path.remove(PKG)
    if not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not installed")
    lib = build.build_sanitized()
    runtime = build.sanitizer_runtime()
    assert os.path.exists(runtime), runtime
    logs = tmp_path / "san"
    env = dict(os.environ,
               LD_PRELOAD=runtime, QUEST_LIB=lib,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(p.read_text() for p in tmp_path.glob("san*"))
    assert r.returncode == 0 and not reports, (r.stdout[-2000:], reports[:4000])
    assert " passed" in r.stdout
