"""GPU checks of the entry points under HIP graph capture and on concurrent
streams: a captured sequence replayed several times, with eager work and
synchronisations between the replays, must give the eager result on every
replay (no entry point records a memset or allocates); calls on two streams
at once must each give their own result."""
import numpy as np
import pytest
import torch

from memory_bound_gemv_row_amd import binding, inputs

from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def test_graph_replays_match_eager(gpu):
    M, N = 2048, 4096
    f16 = inputs.make("f16", M, N, seed=1)
    q8 = inputs.make("q8", M, N, seed=2)
    q4 = inputs.make("q4", M, N, seed=3)
    W = dev(inputs.make_weights(512, 4096, seed=4))
    X = dev(inputs.make_logits(256, 8192, seed=5))
    A16, x16 = dev(f16["A"]), dev(f16["x"])
    A8, s8, x8 = dev(q8["A"]), dev(q8["scale"]), dev(q8["x"])
    A4, s4, x4 = dev(q4["A"]), dev(q4["scale"]), dev(q4["x"])
    y16, y8, y4 = (torch.empty(M, device="cuda") for _ in range(3))
    qw = torch.empty((512, 4096), dtype=torch.int8, device="cuda")
    sw = torch.empty(512, dtype=torch.float16, device="cuda")
    ew = torch.empty(512, dtype=torch.float32, device="cuda")
    ys = torch.empty_like(X)

    def work():
        h = torch.cuda.current_stream().cuda_stream
        assert binding.gemv_f16_ptr(A16.data_ptr(), x16.data_ptr(), y16.data_ptr(), M, N, h) == 0
        assert binding.gemv_q8_ptr(A8.data_ptr(), s8.data_ptr(), x8.data_ptr(), y8.data_ptr(), M, N, h) == 0
        assert binding.gemv_q4_ptr(A4.data_ptr(), s4.data_ptr(), x4.data_ptr(), y4.data_ptr(), M, N, h) == 0
        assert binding.quantize_q8_ptr(W.data_ptr(), qw.data_ptr(), sw.data_ptr(), ew.data_ptr(), 512, 4096, h) == 0
        assert binding.softmax_f16_ptr(X.data_ptr(), ys.data_ptr(), 256, 8192, h) == 0

    outs = (y16, y8, y4, qw, sw, ew, ys)
    say("[graph] eager")
    work()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    say("[graph] capture")
    g = _capture(work)
    for r in range(4):
        for o in outs:
            o.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        say(f"[graph] replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), r


def test_two_streams_at_once(gpu, oracle_mod):
    from oracle.metrics import GATES, parity_error

    a = inputs.make("f16", 4096, 8192, seed=6)
    b = inputs.make("q4", 4096, 8192, seed=7)
    Aa, xa = dev(a["A"]), dev(a["x"])
    Ab, sb, xb = dev(b["A"]), dev(b["scale"]), dev(b["x"])
    ya, yb = torch.empty(4096, device="cuda"), torch.empty(4096, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    say("[streams]")
    for _ in range(20):
        with torch.cuda.stream(s1):
            binding.gemv_f16(Aa, xa, out=ya)
        with torch.cuda.stream(s2):
            binding.gemv_q4(Ab, sb, xb, out=yb)
    torch.cuda.synchronize()
    assert parity_error(ya.cpu().numpy(), oracle_mod.gemv_f16(a["A"], a["x"])) <= GATES["f16"]
    assert parity_error(yb.cpu().numpy(), oracle_mod.gemv_q4(b["A"], b["scale"], b["x"])) <= GATES["q4"]


_FIRST_CALL_CAPTURED = r"""
import sys
import torch
from memory_bound_gemv_row_amd import binding, inputs

M, N = 1024, 4096
f16 = inputs.make("f16", M, N, seed=8)
A = torch.from_numpy(f16["A"]).cuda()
x = torch.from_numpy(f16["x"]).cuda()
W = torch.from_numpy(inputs.make_weights(256, 4096, seed=9)).cuda()
X = torch.from_numpy(inputs.make_logits(64, 8192, seed=10)).cuda()
y = torch.empty(M, device="cuda")
qw = torch.empty((256, 4096), dtype=torch.int8, device="cuda")
sw = torch.empty(256, dtype=torch.float16, device="cuda")
ew = torch.empty(256, dtype=torch.float32, device="cuda")
ys = torch.empty_like(X)
outs = (y, qw, sw, ew, ys)
torch.cuda.synchronize()

def work():
    h = torch.cuda.current_stream().cuda_stream
    rc = (binding.gemv_f16_ptr(A.data_ptr(), x.data_ptr(), y.data_ptr(), M, N, h),
          binding.quantize_q8_ptr(W.data_ptr(), qw.data_ptr(), sw.data_ptr(), ew.data_ptr(), 256, 4096, h),
          binding.softmax_f16_ptr(X.data_ptr(), ys.data_ptr(), 64, 8192, h))
    assert rc == (0, 0, 0), rc

# the process's first library calls are recorded into a graph
g = torch.cuda.CUDAGraph()
s = torch.cuda.Stream()
s.wait_stream(torch.cuda.current_stream())
with torch.cuda.stream(s):
    with torch.cuda.graph(g, stream=s):
        work()
torch.cuda.current_stream().wait_stream(s)
torch.cuda.synchronize()
g.replay()
torch.cuda.synchronize()
got = [o.clone() for o in outs]
for o in outs:
    o.zero_()
work()
torch.cuda.synchronize()
assert all(torch.equal(a, b) for a, b in zip(got, outs))
print("first-call capture ok", flush=True)
"""


def test_first_call_inside_graph_capture(gpu):
    # A fresh process whose first calls of the library (which reads the
    # device's CU count and LDS size once) are captured into a graph: the
    # capture must succeed and the replay match eager calls.
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("[graph] first call captured, fresh process")
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_CAPTURED], cwd=root, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "first-call capture ok" in r.stdout
