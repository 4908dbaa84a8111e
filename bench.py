#!/usr/bin/env python3
"""Benchmark of row-major GEMV on one MI355X.

One step is one GEMV call, y = A . x, on FP16 A[8192, 8192] and x[8192]
with FP32 accumulation and output: the FP16 decode-projection workload of the
"membound" page (section "Results").  Weights rotate through >= 1 GiB of
device copies, so that no launch is served by the 256 MB Infinity Cache or
the L2 ("membound", section "Two gotchas the numbers caught", gotcha 1); x
and y stay fixed.  The same run measures a pure-read probe over the same
ring, before and after the GEMV, and keeps the higher rate as the
denominator ("membound", section "Why GEMV, and why MBU", and gotcha 2).

Prints ONE JSON line.  ``value`` is the achieved algorithmic HBM bandwidth
(bytes of A + x + y per call / time per call).  Extra fields:
``roofline`` (the GEMV kernel against the 8 TB/s datasheet), ``probe``
(the same-run pure-read ceiling and the %-of-probe), ``cpu_baseline`` (the
CPU oracle timed on the host cores on the same inputs; its result also
gates the GPU result, and the run aborts on a parity failure, as the pages
do), ``detail`` (the other FP16 shapes, FP16 weights with FP32 x, FP16
accumulation, and the INT8/INT4 speed-ups over FP16, timed in interleaved
rounds), ``quantiser`` (the FP32 -> INT8/INT4 weight quantiser and the
RMSE of its codes), ``softmax`` (the row softmax against the
streaming-copy ceiling) and ``roofline_study`` (every GEMV point and a
library GEMM reference against min(peak, AI x bandwidth);
``--plot-roofline FILE`` draws it).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMV achieved HBM GB/s and % of pure-read roofline (fp16 8192² and 4096×14336)"
HBM_PEAK_GBPS = 8000.0
RING_BYTES = 1 << 30

def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--kind", default="f16", choices=["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
    ap.add_argument("--M", type=int, default=8192)
    ap.add_argument("--N", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target wall time of the CPU-baseline leg")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--op", choices=["quant_q8", "quant_q4", "softmax"],
                    help="time (or, with --profile, launch once) the quantiser or the softmax at --M x --N "
                         "instead of the GEMV bench line")
    ap.add_argument("--plot-roofline", metavar="BENCH_JSON",
                    help="print an ASCII roofline chart from a saved bench line and exit (no GPU needed)")
    ap.add_argument("--plan-sweep", type=int, default=0, metavar="COUNT",
                    help="time the library's plan on COUNT seeded random shapes per format against the "
                         "same-size pure-read probe, instead of the bench line")
    ap.add_argument("--plan-search", type=int, default=0, metavar="COUNT",
                    help="time every plan the library holds a kernel for (gemv_launch_plan) on COUNT seeded "
                         "random shapes per format against the library's own plan, instead of the bench line")
    ap.add_argument("--seed", type=int, default=0, help="seed of --plan-sweep's and --plan-search's shapes")
    ap.add_argument("--plan-search-named", action="store_true",
                    help="the plan search of --plan-search on the named workloads and the shard shapes "
                         "(every shape and format of the detail table) instead of random shapes")
    ap.add_argument("--profile", action="store_true",
                    help="launch each kernel exactly once after a cold flush (for counter collection)")
    return ap.parse_args()


# ---------------------------------------------------------------- device workload
class Ring:
    """>= 1 GiB of identical weight copies in one allocation, plus x and y."""

    def __init__(self, kind, M, N, ops, min_bytes=RING_BYTES):
        import numpy as np
        import torch

        from memory_bound_gemv_row_amd import accounting

        self.kind, self.M, self.N = kind, M, N
        wbytes = accounting.weight_bytes(kind, M, N)
        abytes = ops["A"].nbytes
        sbytes = ops["scale"].nbytes if "scale" in ops else 0
        self.abytes = -(-abytes // 256) * 256          # scales start on a 256-byte boundary
        self.slot = -(-(self.abytes + sbytes) // 256) * 256
        assert wbytes == abytes + sbytes
        self.copies = accounting.ring_copies(kind, M, N, min_bytes)
        self.buf = torch.empty(self.copies * self.slot, dtype=torch.uint8, device="cuda")
        src = torch.zeros(self.slot, dtype=torch.uint8, device="cuda")
        src[:abytes] = torch.from_numpy(np.ascontiguousarray(ops["A"]).view(np.uint8).ravel()).cuda()
        if sbytes:
            src[self.abytes:self.abytes + sbytes] = torch.from_numpy(
                np.ascontiguousarray(ops["scale"]).view(np.uint8).ravel()).cuda()
        for c in range(self.copies):
            self.buf[c * self.slot:(c + 1) * self.slot].copy_(src)
        del src
        self.x = torch.from_numpy(np.ascontiguousarray(ops["x"]).view(np.uint8).ravel()).cuda()
        self.y = torch.empty(M, dtype=torch.float32, device="cuda")
        self.base = self.buf.data_ptr()
        torch.cuda.synchronize()

    def a_ptr(self, c):
        return self.base + (c % self.copies) * self.slot

    def s_ptr(self, c):
        return self.a_ptr(c) + self.abytes

    def launch(self, c, stream):
        from memory_bound_gemv_row_amd import binding

        k, M, N, y, x = self.kind, self.M, self.N, self.y.data_ptr(), self.x.data_ptr()
        if k == "f32":
            rc = binding.gemv_f32_ptr(self.a_ptr(c), x, y, M, N, stream)
        elif k == "f16":
            rc = binding.gemv_f16_ptr(self.a_ptr(c), x, y, M, N, stream)
        elif k == "f16x32":
            rc = binding.gemv_f16x32_ptr(self.a_ptr(c), x, y, M, N, stream)
        elif k == "f16_acc16":
            rc = binding.gemv_f16_acc16_ptr(self.a_ptr(c), x, y, M, N, stream)
        elif k == "q8":
            rc = binding.gemv_q8_ptr(self.a_ptr(c), self.s_ptr(c), x, y, M, N, stream)
        else:
            rc = binding.gemv_q4_ptr(self.a_ptr(c), self.s_ptr(c), x, y, M, N, stream)
        if rc != 0:
            raise RuntimeError(f"gemv_{k} returned status {rc} ({binding.status_string(rc)})")

    def launch_plan(self, c, stream, plan):
        """One launch with an explicit plan (gemv_launch_plan)."""
        from memory_bound_gemv_row_amd import binding

        scale = self.s_ptr(c) if self.kind in ("q8", "q4") else 0
        rc = binding.launch_plan_ptr(self.kind, self.a_ptr(c), scale, self.x.data_ptr(), self.y.data_ptr(),
                                     self.M, self.N, plan, stream)
        if rc != 0:
            raise RuntimeError(f"gemv_launch_plan {self.kind} {plan} returned status {rc}")

    def free(self):
        self.buf = self.x = self.y = None


def time_eager(ring, steps, warmup):
    """Warm up, then time exactly `steps` launches with HIP events on the
    stream the kernels run on.  Returns seconds per launch."""
    import torch

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for i in range(warmup):
        ring.launch(i, sh)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        ring.launch(warmup + i, sh)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3 / steps


def graph_of(ring, launches, first=0):
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(launches):
                ring.launch(first + i, torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_graph(g, launches, replays=1):
    import torch

    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3 / (launches * replays)


def launch_floor_us(launches=1000):
    """Per-launch floor: back-to-back launches of the pure-read probe over 16
    bytes (one workgroup), eager, between events on the launch stream."""
    import torch

    from memory_bound_gemv_row_amd import binding

    buf = torch.zeros(16, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for _ in range(50):
        binding.probe_read_ptr(buf.data_ptr(), 16, sink.data_ptr(), 0xA5A5A5A5, sh)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(launches):
        binding.probe_read_ptr(buf.data_ptr(), 16, sink.data_ptr(), 0xA5A5A5A5, sh)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / launches


def probe_gbps(buf, reps=20):
    """Best pure-read rate over `reps` full passes of `buf`."""
    import torch

    from memory_bound_gemv_row_amd import binding

    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    nbytes = buf.numel() * buf.element_size()
    sh = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for r in range(reps + 2):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        rc = binding.probe_read_ptr(buf.data_ptr(), nbytes, sink.data_ptr(), 0xA5A5A5A5, sh)
        end.record()
        if rc != 0:
            raise RuntimeError(f"gemv_probe_read returned {rc}")
        torch.cuda.synchronize()
        if r >= 2:
            best = max(best, nbytes / (start.elapsed_time(end) * 1e-3) / 1e9)
    return best


# ---------------------------------------------------------------- CPU baseline leg
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"

def cpu_baseline(kind, ops, y_gpu, seconds):
    """Time the oracle (as it stands) on the host cores and check the GPU result
    against it.  Returns (record, parity report)."""
    import numpy as np

    import oracle
    from memory_bound_gemv_row_amd import accounting

    oracle.build(force=False)
    fn = {"f32": lambda: oracle.gemv_f32(ops["A"], ops["x"]),
          "f16": lambda: oracle.gemv_f16(ops["A"], ops["x"]),
          "f16x32": lambda: oracle.gemv_f16x32(ops["A"], ops["x"]),
          "f16_acc16": lambda: oracle.gemv_f16(ops["A"], ops["x"]),
          "q8": lambda: oracle.gemv_q8(ops["A"], ops["scale"], ops["x"]),
          "q4": lambda: oracle.gemv_q4(ops["A"], ops["scale"], ops["x"])}[kind]
    def timed(budget):
        times = []
        t_end = time.perf_counter() + budget
        while len(times) < 3 or (time.perf_counter() < t_end and len(times) < 200):
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), len(times)

    ref = fn()                                    # warm run; also the parity reference
    cores = oracle.num_threads()
    t, calls = timed(seconds)
    oracle.set_threads(1)
    t1, calls1 = timed(min(seconds, 5.0))
    oracle.set_threads(cores)
    M, N = ops["A"].shape[0], (ops["A"].shape[1] * (2 if kind == "q4" else 1))
    nbytes = accounting.alg_bytes(kind, M, N)
    rec = {"value": accounting.gbps(nbytes, t), "unit": "GB/s",
           "cores": cores, "kind": "oracle",
           "ms_per_call": t * 1e3, "calls": calls, "gflops": accounting.flops(M, N) / t / 1e9,
           "one_thread": {"value": accounting.gbps(nbytes, t1), "ms_per_call": t1 * 1e3, "calls": calls1},
           "cpu_model": cpu_model(),
           "sample": f"the full {kind} {M}x{N} workload (same seeded inputs), {calls} oracle calls on "
                     f"{cores} threads, median (then {calls1} calls on one thread)"}
    rep = oracle.parity_report(y_gpu, ref)
    if kind == "f16_acc16":
        # lossy path: gated by its derived componentwise bound (ratio <= 1)
        A64 = np.abs(ops["A"].astype(np.float64))
        rep["acc16_ratio"] = oracle.acc16_ratio(y_gpu, ref, A64 @ np.abs(ops["x"].astype(np.float64)), N)
        rep["ok"] = rep["acc16_ratio"] <= 1.0
    else:
        rep["gate"] = oracle.GATES[kind]
        rep["ok"] = rep["floored_rel"] <= rep["gate"]
    return rec, rep


# ---------------------------------------------------------------- traffic from counters
def traffic_record(kind, M, N):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or it was taken on other kernel sources."""
    from memory_bound_gemv_row_amd import profiling

    got = profiling.read_traffic(os.path.join(ROOT, "profiles", f"gemv_{kind}_{M}x{N}_traffic.txt"))
    if got is None or got[1] != profiling.kernel_source_hash():
        return None
    return got[0]


# ---------------------------------------------------------------- interleaved detail
DETAIL_SHAPES = [
    ("8192x8192", 8192, 8192, ("f16", "q8", "f16x32", "f16_acc16")),
    ("14336x4096", 14336, 4096, ("f16", "q8", "q4", "f16x32")),
    ("4096x14336", 4096, 14336, ("f16", "q4", "f16x32")),
    ("4096x4096", 4096, 4096, ("f16",)),
    # the FP32 square sweep: small-M grid fill against large-n bandwidth
    ("1024x1024", 1024, 1024, ("f32",)),
    ("2048x2048", 2048, 2048, ("f32",)),
    ("4096x4096", 4096, 4096, ("f32",)),
    ("8192x8192", 8192, 8192, ("f32",)),
    # one GPU's share of 14336x4096 split over 8 GPUs: by rows, by columns
    ("1792x4096", 1792, 4096, ("f16", "q8", "q4")),
    ("14336x512", 14336, 512, ("f16", "q8", "q4")),
]


def probe_slice_graph(ring, launches):
    """HIP graph of `launches` pure-read probes, each over one ring slot's
    weight bytes (rotating slots): a pure read of exactly what one GEMV
    launch streams, launched the same way."""
    import torch

    from memory_bound_gemv_row_amd import accounting, binding

    nbytes = accounting.weight_bytes(ring.kind, ring.M, ring.N) // 16 * 16
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(launches):
                rc = binding.probe_read_ptr(ring.a_ptr(i), nbytes, sink.data_ptr(), 0xA5A5A5A5,
                                            torch.cuda.current_stream().cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"gemv_probe_read returned {rc}")
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g._sink = sink
    return g, nbytes


def detail(rounds, launches=256):
    """Other shapes and formats, in interleaved rounds (best round per
    kernel).  Besides each GEMV, a pure-read probe over the same weight bytes
    is timed the same way; its time is the floor for that launch, and the
    ratio of those floors bounds the INT8/INT4 speed-ups over FP16."""
    import torch

    from memory_bound_gemv_row_amd import accounting, inputs

    out = {}
    for name, M, N, kinds in DETAIL_SHAPES:
        rings, graphs, pgraphs = {}, {}, {}
        for k in kinds:
            rings[k] = Ring(k, M, N, inputs.make(k, M, N, seed=0))
            graphs[k] = graph_of(rings[k], launches)
            graphs[k].replay()
            pgraphs[k] = probe_slice_graph(rings[k], launches)
            pgraphs[k][0].replay()
        probe_buf = rings[kinds[0]].buf
        torch.cuda.synchronize()
        best = {k: float("inf") for k in kinds}
        pbest = {k: float("inf") for k in kinds}
        per_round = {k: [] for k in kinds}
        probe_best = 0.0
        for _ in range(rounds):
            for k in kinds:
                t = time_graph(graphs[k], launches)
                per_round[k].append(t)
                best[k] = min(best[k], t)
                pbest[k] = min(pbest[k], time_graph(pgraphs[k][0], launches))
            probe_best = max(probe_best, probe_gbps(probe_buf, reps=3))
        rec = {"probe_gbps": probe_best}
        for k in kinds:
            gb = accounting.gbps(accounting.alg_bytes(k, M, N), best[k])
            rec[k] = {"us": best[k] * 1e6, "us_median": sorted(per_round[k])[len(per_round[k]) // 2] * 1e6,
                      "gbps": gb, "pct_of_probe": 100 * gb / max(probe_best, gb),
                      "pct_of_8tbs": 100 * gb / HBM_PEAK_GBPS,
                      "same_size_probe_us": pbest[k] * 1e6,
                      "pct_of_same_size_probe": 100 * pbest[k] / best[k]}
        for k in kinds:
            if k != "f16" and "f16" in kinds:
                rec[k]["x_f16"] = best["f16"] / best[k]
                rec[k]["x_f16_same_size_probe_ceiling"] = pbest["f16"] / pbest[k]
        out.setdefault(name, {}).update(rec)
        out[name]["probe_gbps"] = max(out[name].get("probe_gbps", 0.0), probe_best)
        for k in kinds:
            rings[k].free()
        del graphs, rings, pgraphs
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- plan sweep
SWEEP_KINDS = ("f32", "f16", "f16x32", "q8", "q4")
SWEEP_MAX_WEIGHT_BYTES = 512 << 20


def sweep_shapes(count, seed):
    """`count` seeded shapes per format: M log-uniform on [256, 65536], N
    log-uniform on [256, 32768] rounded to a multiple of 128 (INT4's group),
    weights at most 512 MiB (redrawn otherwise)."""
    import numpy as np

    from memory_bound_gemv_row_amd import accounting

    rng = np.random.default_rng(seed)
    out = []
    for kind in SWEEP_KINDS:
        got = 0
        while got < count:
            M = int(round(2 ** rng.uniform(8, 16)))
            N = max(128, int(round(2 ** rng.uniform(8, 15) / 128)) * 128)
            if accounting.weight_bytes(kind, M, N) > SWEEP_MAX_WEIGHT_BYTES:
                continue
            out.append((kind, M, N))
            got += 1
    return out


def zero_operands(kind, M, N):
    """Operands of the right dtypes and shapes, all zero: the timing of the
    streaming kernels does not depend on the values."""
    import numpy as np

    a = {"f32": (np.float32, N), "f16": (np.float16, N), "f16x32": (np.float16, N), "f16_acc16": (np.float16, N),
         "q8": (np.int8, N), "q4": (np.uint8, N // 2)}[kind]
    ops = {"A": np.zeros((M, a[1]), a[0]),
           "x": np.zeros(N, np.float32 if kind in ("f32", "f16x32") else np.float16)}
    if kind == "q8":
        ops["scale"] = np.zeros(M, np.float16)
    elif kind == "q4":
        ops["scale"] = np.zeros((M, N // 128), np.float16)
    return ops


def plan_sweep(count, seed, rounds=3, launches=64):
    """The library's own plan on seeded random shapes (sweep_shapes), each
    against the pure-read probe over the same weight bytes launched the same
    way (graph of `launches` launches over a >= 1 GiB ring, best of `rounds`):
    how far each shape's plan sits from the floor of a launch that reads the
    same bytes.  Prints one JSON line per shape and a per-format summary."""
    import torch

    from memory_bound_gemv_row_amd import binding

    rows = []
    for kind, M, N in sweep_shapes(count, seed):
        ring = Ring(kind, M, N, zero_operands(kind, M, N))
        g = graph_of(ring, launches)
        pg, _ = probe_slice_graph(ring, launches)
        g.replay()
        pg.replay()
        torch.cuda.synchronize()
        tg = min(time_graph(g, launches) for _ in range(rounds))
        tp = min(time_graph(pg, launches) for _ in range(rounds))
        info = binding.describe_launch(kind, M, N, True)
        row = {"kind": kind, "M": M, "N": N, "us": round(tg * 1e6, 3), "same_size_probe_us": round(tp * 1e6, 3),
               "pct_of_same_size_probe": round(100 * tp / tg, 1), "plan": info}
        rows.append(row)
        print(json.dumps(row), flush=True)
        ring.free()
        del g, pg
        torch.cuda.empty_cache()
    summary = {}
    for kind in SWEEP_KINDS:
        r = sorted((x for x in rows if x["kind"] == kind), key=lambda x: x["pct_of_same_size_probe"])
        if r:
            summary[kind] = {"shapes": len(r), "worst_pct": r[0]["pct_of_same_size_probe"],
                             "median_pct": r[len(r) // 2]["pct_of_same_size_probe"],
                             "worst_shape": f"{r[0]['M']}x{r[0]['N']}"}
    print(json.dumps({"plan_sweep": summary, "seed": seed, "count": count}), flush=True)


def plan_candidates(kind, N):
    """Every explicit plan (variant, waves, units in flight, rows per wave,
    stage order, cap) the library holds a kernel for at row length N, over
    the ranges its planner chooses from; gemv_check_plan_for drops those that
    do not fit a given shape and device."""
    epc = {"f32": 4, "f16": 8, "f16_acc16": 8, "f16x32": 8, "q8": 16, "q4": 32}[kind]
    nchunks = N // epc
    P = -(-nchunks // 64)
    fp = kind in ("f32", "f16", "f16_acc16")
    out = []
    if P == 1:
        out += [(5, w, d, r, -1, cap) for w in (4, 8) for d in (1, 2) for r in (1, 2) for cap in (0, 3)]
    elif P == 2:
        out += [(5, 4, 2, 1, -1, cap) for cap in (0, 3, 6)]
    elif P == 3:
        out += [(5, w, 3, 1, -1, cap) for w in (4, 8) for cap in (0, 3)]
    if kind in ("q8", "q4") and nchunks <= 32:
        out += [(4, 8, d, r, -1, 0) for d, r in ((1, 1), (1, 2), (2, 2), (2, 4), (1, 4))]
    out += [(2, w, d, r, -1, 0) for w in (4, 8) for d in (2, 4, 8) for r in ((1, 2, 4) if fp else (1, 2))]
    if not fp:
        out += [(1, w, d, r, stg, cap) for w in (4, 8) for d in (2, 4, 8) for stg in (0, 1, 2)
                for r, cap in ((1, 0), (2, 0), (1, 1), (1, 2), (1, 3), (1, 4))]
        if kind == "q8":
            out += [(1, 4, 5, 1, 2, cap) for cap in (0, 2, 3)]
        if kind == "q4":
            out += [(1, 4, d, 1, 1, cap) for d in (3, 5) for cap in (0, 2, 3)]
    if kind != "f16_acc16":
        out += [(6, S, d, 1, -1, 0) for S in (2, 4, 8, 16) if 2 * S <= P for d in (2, 4)]
    if kind in ("q8", "q4", "f16x32"):
        # row slabs: S waves own P / S passes each (one or two)
        for S in sorted({P, P // 2}):
            if not (1 <= S <= 16 and P % S == 0 and P // S <= 2):
                continue
            out += [(7, S, d, r, -1, cap) for d in (4, 8) for r in (4, 8) for cap in sorted({0, max(1, 32 // S)})
                    if (r * (P // S)) % d == 0]
    return out


def plan_search(count, seed, rounds=3, launches=48, shapes=None):
    """Brute force over the plans: on each seeded random shape
    (sweep_shapes), every candidate plan that fits (plan_candidates,
    gemv_check_plan_for) and the library's own plan, each as a graph of
    `launches` launches over a >= 1 GiB ring, best of `rounds`.  Prints one
    JSON line per shape (the library's plan, the fastest candidate, their
    ratio, every candidate's time) and a per-format summary: how far the
    planner's choice sits from the best plan the library could have
    launched.  `shapes` replaces the random shapes when given."""
    import math

    import torch

    from memory_bound_gemv_row_amd import binding

    props = torch.cuda.get_device_properties(0)
    cus, lds_max = props.multi_processor_count, props.shared_memory_per_block
    rows = []
    for kind, M, N in shapes or sweep_shapes(count, seed):
        ring = Ring(kind, M, N, zero_operands(kind, M, N))
        sh = torch.cuda.current_stream().cuda_stream
        for i in range(16):   # warm the clocks before the first timing
            ring.launch(i, sh)
        torch.cuda.synchronize()

        def timed(launch_one):
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for i in range(launches):
                        launch_one(i, torch.cuda.current_stream().cuda_stream)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            return min(time_graph(g, launches) for _ in range(rounds))

        t_lib = timed(ring.launch)
        cands = []
        for plan in plan_candidates(kind, N):
            if binding.check_plan_for(kind, M, N, cus, lds_max, plan) is None:
                continue
            cands.append((timed(lambda i, h, plan=plan: ring.launch_plan(i, h, plan)), plan))
        t_lib = min(t_lib, timed(ring.launch))   # again after the candidates: the better of the two
        best_t, best_plan = min(cands)
        info = binding.describe_launch(kind, M, N, True)
        row = {"kind": kind, "M": M, "N": N, "lib_us": round(t_lib * 1e6, 3), "best_us": round(best_t * 1e6, 3),
               "lib_over_best": round(t_lib / best_t, 4), "lib_plan": info, "best_plan": list(best_plan),
               "candidates": len(cands), "all_us": [[list(p), round(t * 1e6, 3)] for t, p in cands]}
        rows.append(row)
        print(json.dumps(row), flush=True)
        ring.free()
        torch.cuda.empty_cache()
    summary = {}
    for kind in dict.fromkeys(x["kind"] for x in rows):
        r = sorted((x for x in rows if x["kind"] == kind), key=lambda x: x["lib_over_best"])
        if r:
            geo = math.exp(sum(math.log(x["lib_over_best"]) for x in r) / len(r))
            summary[kind] = {"shapes": len(r), "geomean_lib_over_best": round(geo, 4),
                             "median_lib_over_best": r[len(r) // 2]["lib_over_best"],
                             "worst_lib_over_best": r[-1]["lib_over_best"], "worst_shape": f"{r[-1]['M']}x{r[-1]['N']}"}
    print(json.dumps({"plan_search": summary, "seed": None if shapes else seed, "count": len(rows)}), flush=True)


# ---------------------------------------------------------------- quantiser
def quant_detail(rounds, launches=64, shapes=None):
    """The weight quantiser (FP32 -> INT8 / INT4 + per-row squared error) on
    the INT8/INT4 GEMV shapes.  Each slot of a >= 1 GiB ring holds a copy of
    the weights and its own outputs (codes, scales, row errors), so that
    neither the reads nor the writes of one launch can be served by a cache
    that the previous launch filled; launches are captured in a HIP graph,
    best of `rounds`.  Two floors are timed the same way: a pure read of the
    FP32 weights (the bytes that must be read), and a streaming copy moving
    the same total bytes (half read, half written, into a rotating
    destination); the quantiser's mix (8:1 or 4:1 read:write) lies between.
    Also reports the RMSE of the GPU's codes ("membound", dequant section:
    2.3e-3 / 4.1e-2 on U[-1,1])."""
    import numpy as np
    import torch

    from memory_bound_gemv_row_amd import accounting, binding, inputs

    def up(n):
        return -(-n // 256) * 256

    out = {}
    for kind, M, N in (shapes or inputs.QUANT_WORKLOADS):
        wbytes = 4 * M * N
        qbytes = M * N if kind == "q8" else M * N // 2
        sbytes = 2 * M if kind == "q8" else 2 * M * (N // 128)
        offs = [0, up(wbytes), up(wbytes) + up(qbytes), up(wbytes) + up(qbytes) + up(sbytes)]
        slot = offs[3] + up(4 * M)
        copies = max(1, -(-RING_BYTES // slot))
        ring = torch.empty((copies, slot), dtype=torch.uint8, device="cuda")
        W = torch.from_numpy(inputs.make_weights(M, N, seed=0).view(np.uint8).ravel()).cuda()
        for c in range(copies):
            ring[c, :wbytes].copy_(W)
        del W
        nbytes = accounting.quant_bytes(kind, M, N)
        half = nbytes // 2 // 16 * 16             # a copy of this many bytes moves nbytes in total
        cdst = torch.empty((copies, up(half)), dtype=torch.uint8, device="cuda")
        fn = binding.quantize_q8_ptr if kind == "q8" else binding.quantize_q4_ptr
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        graphs = []
        for which in ("quant", "probe", "copy"):
            g = torch.cuda.CUDAGraph()
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                with torch.cuda.graph(g, stream=st):
                    for i in range(launches):
                        h = torch.cuda.current_stream().cuda_stream
                        base = ring[i % copies].data_ptr()
                        if which == "quant":
                            rc = fn(base, base + offs[1], base + offs[2], base + offs[3], M, N, h)
                        elif which == "probe":
                            rc = binding.probe_read_ptr(base, wbytes, sink.data_ptr(), 0xA5A5A5A5, h)
                        else:
                            rc = binding.probe_copy_ptr(base, cdst[i % copies].data_ptr(), half, h)
                        if rc != 0:
                            raise RuntimeError(f"{which} returned {rc}")
            torch.cuda.current_stream().wait_stream(st)
            torch.cuda.synchronize()
            g.replay()
            graphs.append(g)
        best = [float("inf")] * 3
        for _ in range(rounds):
            for j in range(3):
                best[j] = min(best[j], time_graph(graphs[j], launches))
        gb = nbytes / best[0] / 1e9
        e = ring[0, offs[3]:offs[3] + 4 * M].view(torch.float32)
        rmse = float(np.sqrt(e.double().sum().item() / (M * N)))
        out[f"{kind}_{M}x{N}"] = {
            "us": best[0] * 1e6, "alg_bytes": nbytes, "gbps": gb, "pct_of_8tbs": 100 * gb / HBM_PEAK_GBPS,
            "read_probe_us": best[1] * 1e6,
            "pct_of_read_probe_time": 100 * best[1] / best[0],
            "equal_bytes_copy_us": best[2] * 1e6,
            "pct_of_equal_bytes_copy_time": 100 * best[2] / best[0],
            "rmse": rmse,
        }
        del graphs, ring, cdst
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- softmax
def softmax_detail(rounds, launches=32, shapes=None):
    """Row softmax on the "membound" softmax shapes (binary16 in and out):
    (x, y) slot pairs rotate through >= 1 GiB, launches captured in a HIP
    graph, best of `rounds`.  The ceiling is the streaming-copy probe moving
    the same bytes (read 2MN, write 2MN) the same way: the traffic mix of
    softmax is one read and one write per element, so a pure-read ceiling
    would flatter it (section "Bonus kernel: online softmax")."""
    import torch

    from memory_bound_gemv_row_amd import binding, inputs

    out = {}
    for M, N in (shapes or inputs.SOFTMAX_WORKLOADS):
        nbytes = 2 * M * N
        slots = max(1, -(-RING_BYTES // (2 * nbytes)))
        x = torch.from_numpy(inputs.make_logits(M, N, seed=0)).cuda()
        xs = torch.empty((slots, M, N), dtype=torch.float16, device="cuda")
        xs[:] = x
        ys = torch.empty((slots, M, N), dtype=torch.float16, device="cuda")
        del x
        graphs = []
        for which in ("softmax", "copy"):
            g = torch.cuda.CUDAGraph()
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                with torch.cuda.graph(g, stream=st):
                    for i in range(launches):
                        h = torch.cuda.current_stream().cuda_stream
                        a, b = xs[i % slots].data_ptr(), ys[i % slots].data_ptr()
                        rc = (binding.softmax_f16_ptr(a, b, M, N, h) if which == "softmax"
                              else binding.probe_copy_ptr(a, b, nbytes, h))
                        if rc != 0:
                            raise RuntimeError(f"{which} returned {rc}")
            torch.cuda.current_stream().wait_stream(st)
            torch.cuda.synchronize()
            g.replay()
            graphs.append(g)
        best = [float("inf"), float("inf")]
        for _ in range(rounds):
            for j in range(2):
                best[j] = min(best[j], time_graph(graphs[j], launches))
        gb = 2 * nbytes / best[0] / 1e9
        out[f"{M}x{N}"] = {"us": best[0] * 1e6, "alg_bytes": 2 * nbytes, "gbps": gb,
                           "pct_of_8tbs": 100 * gb / HBM_PEAK_GBPS,
                           "copy_probe_us": best[1] * 1e6, "copy_probe_gbps": 2 * nbytes / best[1] / 1e9,
                           "pct_of_copy_ceiling": 100 * best[1] / best[0]}
        del graphs, xs, ys
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- roofline study
PEAK_TFLOPS = {"f32": 157.3, "f16": 2500.0}     # MI355X dense: FP32 vector/MFMA, FP16 MFMA


def gemm_reference(n=8192, reps=20):
    """Library GEMM reference points (torch.matmul -> hipBLASLt / rocBLAS) on
    square n x n x n operands, FP16 and FP32: the compute-bound end of the
    roofline that "cuda-gemv-optimization" names as its next comparison
    (section "What I'd explore next").  Returns one point per dtype."""
    import torch

    pts = []
    for name, dt in (("f16", torch.float16), ("f32", torch.float32)):
        g = torch.Generator(device="cuda").manual_seed(0)
        a = torch.randn((n, n), dtype=dt, device="cuda", generator=g)
        b = torch.randn((n, n), dtype=dt, device="cuda", generator=g)
        for _ in range(3):
            c = torch.matmul(a, b)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            c = torch.matmul(a, b)
        end.record()
        torch.cuda.synchronize()
        t = start.elapsed_time(end) * 1e-3 / reps
        elt = a.element_size()
        flops = 2 * n ** 3
        nbytes = elt * 3 * n * n                    # A, B read once, C written once
        pts.append({"kernel": f"gemm_{name}_{n}^3 (library)", "dtype": name, "ai": flops / nbytes,
                    "tflops": flops / t / 1e12, "us": t * 1e6, "peak_tflops": PEAK_TFLOPS[name]})
        del a, b, c
    torch.cuda.empty_cache()
    return pts


def roofline_study(rec):
    """Points (arithmetic intensity, achieved TFLOP/s) for every GEMV kernel
    the bench timed and for the GEMM reference, with the attainable bound
    min(P_peak, AI * B) ("Making GEMV Fast", section "Arithmetic
    intensity"), B = the same-run pure-read probe."""
    from memory_bound_gemv_row_amd import accounting

    bw = rec["probe"]["gbps"] * 1e9
    pts = []

    def gemv_point(kind, M, N, us):
        f = accounting.flops(M, N)
        ai = f / accounting.alg_bytes(kind, M, N)
        peak = PEAK_TFLOPS["f32"]                    # GEMV arithmetic is FP32 (or FP16-in, FP32-out dot2)
        tf = f / (us * 1e-6) / 1e12
        return {"kernel": f"gemv_{kind}_{M}x{N}", "dtype": kind, "ai": ai, "tflops": tf, "us": us,
                "peak_tflops": peak}

    M, N, kind = rec["config"]["M"], rec["config"]["N"], rec["dtype"]
    pts.append(gemv_point(kind, M, N, rec["roofline"]["kernel_us"]))
    for shape, d in rec.get("detail", {}).items():
        m, n = (int(v) for v in shape.split("x"))
        for k, v in d.items():
            if isinstance(v, dict) and not (k == kind and m == M and n == N):
                pts.append(gemv_point(k, m, n, v["us"]))
    pts.extend(gemm_reference())
    for p in pts:
        p["attainable_tflops"] = min(p["peak_tflops"], p["ai"] * bw / 1e12)
        p["pct_of_attainable"] = 100 * p["tflops"] / p["attainable_tflops"]
        p["bound"] = "hbm" if p["ai"] * bw / 1e12 < p["peak_tflops"] else "compute"
    return {"bandwidth_gbps": bw / 1e9, "points": pts}


def ascii_roofline(study, width=72, height=22):
    """Log-log text chart: the FP16-MFMA and FP32 roofs against the measured
    bandwidth, and every point of the study (G = GEMV, M = GEMM)."""
    import math

    bw = study["bandwidth_gbps"] * 1e9
    x0, x1, y0, y1 = -1.0, 4.0, -1.0, 3.6          # log10 AI (FLOP/B) and log10 TFLOP/s
    grid = [[" "] * width for _ in range(height)]

    def cell(ai, tf):
        cx = int(round((math.log10(ai) - x0) / (x1 - x0) * (width - 1)))
        cy = int(round((math.log10(tf) - y0) / (y1 - y0) * (height - 1)))
        return min(max(cx, 0), width - 1), min(max(height - 1 - cy, 0), height - 1)

    for peak, ch in ((PEAK_TFLOPS["f16"], "="), (PEAK_TFLOPS["f32"], "-")):
        for i in range(width):
            ai = 10 ** (x0 + (x1 - x0) * i / (width - 1))
            cx, cy = cell(ai, min(peak, ai * bw / 1e12))
            if grid[cy][cx] == " ":
                grid[cy][cx] = ch
    for p in study["points"]:
        cx, cy = cell(p["ai"], p["tflops"])
        grid[cy][cx] = "M" if p["kernel"].startswith("gemm") else "G"
    lines = [f"TFLOP/s (log)  roofs: '=' FP16 MFMA {PEAK_TFLOPS['f16']:.0f}, '-' FP32 {PEAK_TFLOPS['f32']:.0f}, "
             f"slope = {study['bandwidth_gbps']:.0f} GB/s"]
    for r, row in enumerate(grid):
        ylab = 10 ** (y1 - (y1 - y0) * r / (height - 1))
        lines.append(f"{ylab:9.1f} |" + "".join(row))
    lines.append(" " * 10 + "+" + "-" * width)
    lines.append(" " * 11 + "".join(f"{10 ** (x0 + i):<{width // 5}g}" for i in range(5)) + "  AI (FLOP/byte, log)")
    return "\n".join(lines)


# ---------------------------------------------------------------- quantiser / softmax on their own
def op_main(args):
    """--op: the quantiser or the softmax at one shape.  With --profile: one
    cold launch after a >= 1 GiB flush read, then the calibration probes
    (1 GiB read, 256 MiB copy), for counter collection; otherwise the timed
    record of quant_detail / softmax_detail for that shape."""
    import torch

    from memory_bound_gemv_row_amd import binding, inputs

    M, N = args.M, args.N
    if not args.profile:
        if args.op == "softmax":
            rec = softmax_detail(args.rounds, shapes=[(M, N)])
        else:
            rec = quant_detail(args.rounds, shapes=[(args.op[-2:], M, N)])
        print(json.dumps({"op": args.op, "M": M, "N": N, "record": rec}), flush=True)
        return
    flush = torch.empty(RING_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    if args.op == "softmax":
        x = torch.from_numpy(inputs.make_logits(M, N, seed=0)).cuda()
        y = torch.empty_like(x)
        launch = lambda: binding.softmax_f16_ptr(x.data_ptr(), y.data_ptr(), M, N, sh)
    else:
        W = torch.from_numpy(inputs.make_weights(M, N, seed=0)).cuda()
        q8 = args.op == "quant_q8"
        q = torch.empty((M, N if q8 else N // 2), dtype=torch.uint8, device="cuda")
        sc = torch.empty(M if q8 else M * (N // 128), dtype=torch.float16, device="cuda")
        e = torch.empty(M, dtype=torch.float32, device="cuda")
        fn = binding.quantize_q8_ptr if q8 else binding.quantize_q4_ptr
        launch = lambda: fn(W.data_ptr(), q.data_ptr(), sc.data_ptr(), e.data_ptr(), M, N, sh)
    torch.cuda.synchronize()
    binding.probe_read_ptr(flush.data_ptr(), RING_BYTES, sink.data_ptr(), 0xA5A5A5A5, sh)
    if launch() != 0:
        raise RuntimeError(f"{args.op} launch failed")
    binding.probe_read_ptr(flush.data_ptr(), RING_BYTES, sink.data_ptr(), 0xA5A5A5A5, sh)
    binding.probe_copy_ptr(flush.data_ptr(), flush.data_ptr() + (512 << 20), 256 << 20, sh)
    torch.cuda.synchronize()
    print(json.dumps({"profile": f"{args.op}_{M}x{N}", "launches": 1}), flush=True)


# ---------------------------------------------------------------- main
def main():
    args = parse()
    if args.plot_roofline:
        with open(args.plot_roofline) as f:
            rec = json.loads(f.read().strip().splitlines()[-1])
        print(ascii_roofline(rec["roofline_study"]))
        for p in rec["roofline_study"]["points"]:
            print(f"{p['kernel']:<34} AI {p['ai']:8.2f}  {p['tflops']:8.2f} TFLOP/s  "
                  f"attainable {p['attainable_tflops']:8.2f}  ({p['pct_of_attainable']:5.1f} %, {p['bound']})")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this GEMV library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from memory_bound_gemv_row_amd import accounting, binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    if args.op:
        return op_main(args)
    if args.plan_sweep:
        return plan_sweep(args.plan_sweep, args.seed)
    if args.plan_search:
        return plan_search(args.plan_search, args.seed)
    if args.plan_search_named:
        named = [(k, M, N) for _, M, N, kinds in DETAIL_SHAPES for k in kinds]
        return plan_search(0, None, rounds=5, launches=64, shapes=named)
    kind, M, N = args.kind, args.M, args.N
    ops = inputs.make(kind, M, N, seed=0)
    ring = Ring(kind, M, N, ops)
    nbytes = accounting.alg_bytes(kind, M, N)

    if args.profile:
        # one cold launch per kernel, each after a >= 1 GiB flush read
        flush = torch.empty(RING_BYTES, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        sh = torch.cuda.current_stream().cuda_stream
        binding.probe_read_ptr(flush.data_ptr(), RING_BYTES, sink.data_ptr(), 0xA5A5A5A5, sh)
        ring.launch(0, sh)
        binding.probe_read_ptr(flush.data_ptr(), RING_BYTES, sink.data_ptr(), 0xA5A5A5A5, sh)
        binding.probe_copy_ptr(ring.buf.data_ptr(), flush.data_ptr(), 256 << 20, sh)
        torch.cuda.synchronize()
        print(json.dumps({"profile": f"{kind}_{M}x{N}", "launches": 1}), flush=True)
        return

    launch_floor = launch_floor_us()
    probe_before = probe_gbps(ring.buf)
    t = time_eager(ring, args.steps, args.warmup)
    probe_after = probe_gbps(ring.buf)
    y_gpu = ring.y.cpu().numpy()
    value = accounting.gbps(nbytes, t)
    probe = max(probe_before, probe_after)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": t * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": kind, "data": "synthetic",
        "config": {"workload": f"{kind}_{M}x{N}", "M": M, "N": N,
                   "accumulate": "f16 (lossy)" if kind == "f16_acc16" else "f32", "seed": 0,
                   "ring_copies": ring.copies, "ring_bytes": ring.copies * ring.slot,
                   "launch": binding.describe_launch(kind, M, N, True)},
    }
    rec["probe"] = {"gbps": round(probe, 2), "before": round(probe_before, 2), "after": round(probe_after, 2),
                    "launch_floor_us": round(launch_floor, 3),
                    "pct_of_probe": round(100 * value / max(probe, value), 2),
                    "pct_of_8tbs": round(100 * probe / HBM_PEAK_GBPS, 2)}
    traffic = traffic_record(kind, M, N)
    rec["roofline"] = {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": traffic,
                       "alg_bytes_per_launch": nbytes, "kernel_us": round(t * 1e6, 3),
                       "gflops": round(accounting.flops(M, N) / t / 1e9, 1)}
    ring.free()
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(kind, ops, y_gpu, args.cpu_seconds)
        rec["cpu_baseline"] = cpu
        rec["parity"] = parity
        if not parity["ok"]:
            print(json.dumps({"error": "parity failure: GPU result disagrees with the oracle", "parity": parity}),
                  flush=True)
            sys.exit(3)
    else:
        rec["cpu_baseline"] = None

    if not args.no_detail:
        rec["detail"] = detail(args.rounds)
        rec["quantiser"] = quant_detail(args.rounds)
        rec["softmax"] = softmax_detail(args.rounds)
        rec["roofline_study"] = roofline_study(rec)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
