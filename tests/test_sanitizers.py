"""The host planner, geometry validation and C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is rebuilt with its host code instrumented and
tests/test_abi.py runs against it in a child process that preloads the ASan runtime. Any
sanitizer report ends the child with a failure. No GPU is used."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sparse_attention_frame_amd import build as B  # noqa: E402


def test_abi_suite_under_asan_and_ubsan():
    try:
        B.hipcc()
        runtime = B.asan_runtime()
    except RuntimeError as e:  # pragma: no cover
        pytest.skip(f"no sanitizer toolchain: {e}")
    lib = B.build_sanitized()
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "the host code is not instrumented"
    env = dict(os.environ)
    env.update(SFA_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
