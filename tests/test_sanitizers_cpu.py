"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer: the fp64 oracle driven on
edge shapes, and libxv's host-side argument checks (every entry point with arguments that
break one check; nothing launches).  Each program exits 0 only with no sanitizer report."""
import os
import shutil
import subprocess

import pytest


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    import oracle
    exe = oracle.build_sanitized(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer run: ok" in r.stdout


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_library_host_checks_under_sanitizers(tmp_path):
    from bit_exact_speculative_amd import build
    exe = build.build_sanitized_host_checks(str(tmp_path))
    rc, out = _run(exe)
    assert rc == 0, out
    assert "libxv host checks under the sanitizers: ok" in out
