"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle and the library's host side (argument checks, planner, status
strings) are built with the sanitizers and driven by C self-tests; any
out-of-bounds access, overflow or undefined operation ends the run with a
sanitizer report ("membound", section "Build, run, profile": warnings as
errors and a smoke run; here also the sanitizers).  Leak detection stays on
for the oracle; the HIP runtime the library links keeps allocations for the
life of the process, so the library's run leaves it off.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))


@pytest.fixture(scope="module")
def out_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    proc = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = proc.stdout + proc.stderr
    assert proc.returncode == 0 and "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out
    return out


def test_oracle_under_sanitizers(out_dir):
    import build

    exe = build.build_oracle_selftest(out_dir)
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=1", "OMP_NUM_THREADS": "2"})
    assert "all checks passed" in out


def test_library_host_code_under_sanitizers(out_dir):
    import build

    exe = build.build_host_selftest(out_dir)
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
    assert "every argument check passed" in out
