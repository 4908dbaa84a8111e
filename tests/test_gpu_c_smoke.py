"""Runs the C-only smoke program of the C ABI (tests/c_smoke/c_abi_smoke.c):
plain C calling every format through include/*.h, checked against the
oracle library.  The program is built by __graft_entry__.build()."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_smoke", "c_abi_smoke")


def test_c_abi_smoke(gpu):
    assert os.path.exists(BIN), "C smoke program not built: run __graft_entry__.build()"
    print("[c-smoke] running", BIN, flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c-smoke PASSED" in r.stdout
