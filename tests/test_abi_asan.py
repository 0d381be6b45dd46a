"""The C ABI's host-side code under AddressSanitizer, on the CPU: tests/test_abi.py (argument
checks, status codes, workspace sizes, the host planner arithmetic, the no-alloc entry point's
host checks) run in a child process against libspecdec_asan.so -- the same sources with the host
code built with -fsanitize=address, the device code as usual -- with the sanitizer's runtime
preloaded.  The sanitized library is rebuilt when it is missing or older than a source.  Skipped
where the runtime is absent, or where the environment already preloads a library (the sanitizer
must come first, and this test replaces nobody's preload)."""
import os
import pathlib
import subprocess
import sys

import pytest

from speculative_decoding_verification_specdec_amd import build as B

ROOT = pathlib.Path(__file__).resolve().parents[1]


def _stale() -> bool:
    out = B.ASAN_OUTPUT
    if not out.exists():
        return True
    t = out.stat().st_mtime
    return any(p.stat().st_mtime > t for p in [*B.SOURCES, *B.HEADERS])


def test_abi_under_address_sanitizer():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a library is already preloaded here")
    try:
        rt = B.asan_runtime()
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("no compiler to locate the AddressSanitizer runtime")
    if not os.path.isfile(rt):
        pytest.skip("no AddressSanitizer runtime")
    if _stale():
        B.build_library(verbose=False, asan=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               SPECDEC_LIBRARY=str(B.ASAN_OUTPUT), HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", str(ROOT / "tests" / "test_abi.py")],
                       cwd=str(ROOT), env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr, out
    assert " passed" in r.stdout and " failed" not in r.stdout, out
