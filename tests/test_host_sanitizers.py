"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/test_abi_host.py (the C ABI's argument checks, dispatch, sizes and
environment overrides) runs in a subprocess against a build of libq4 whose
host code is instrumented, and tests/test_oracle_pins.py against an
instrumented build of the oracle.  Any sanitizer report ends that subprocess
with an error.  The builds are made on first use (a few minutes) and reused
while the sources are unchanged.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_asan_and_ubsan():
    from gemv_q4_affine_amd import build as hb
    import oracle

    if not os.path.exists(hb.SAN_RUNTIME):
        pytest.skip(f"no sanitizer runtime at {hb.SAN_RUNTIME}")
    lib = hb.build_host_sanitized()
    olib = oracle.build_sanitized(os.path.join(hb.SAN_DIR, "liboracle_san.so"))
    for path in (lib, olib):
        syms = subprocess.run(["nm", "-D", path], capture_output=True, text=True, check=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, f"{path} is not instrumented"
    env = dict(os.environ,
               LD_PRELOAD=hb.SAN_RUNTIME,
               ASAN_OPTIONS="detect_leaks=0",            # the interpreter's own allocations
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               Q4_LIB_PATH=lib,
               Q4_ORACLE_LIB=olib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi_host.py", "tests/test_oracle_pins.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    assert " passed" in r.stdout
