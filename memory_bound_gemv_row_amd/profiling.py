"""Summaries of rocprofv3 runs of ``bench.py`` (kernel trace and counters).

Usage (after the rocprofv3 runs named in each summary's header)::

    python -m memory_bound_gemv_row_amd.profiling trace  <kernel_stats.csv> <out.txt> <command>
    python -m memory_bound_gemv_row_amd.profiling counters <counter_collection.csv> <out.txt> <command>
    python -m memory_bound_gemv_row_amd.profiling traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <workload> <out.txt> <fetch command> <write command>

Traffic calibration: ``bench.py --profile`` launches, in order, a 1 GiB
pure-read probe, the GEMV once, the probe again, and a 256 MiB copy.  The
FETCH_SIZE reading of the probe (known to read 1 GiB) and the WRITE_SIZE
reading of the copy (known to write 256 MiB) give the factors that turn
each counter's KiB into bytes; the GEMV's readings times those factors are
its HBM bytes per launch.
"""
from __future__ import annotations

import csv
import hashlib
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_CSRC = "memory_bound_gemv_row_amd/csrc/"
# the device properties the plans read are part of every operation's code
KERNEL_SOURCES = (_CSRC + "gemv_kernels.hpp", _CSRC + "gemv_api.hip", _CSRC + "device_info.hpp")
OP_SOURCES = {
    "gemv": KERNEL_SOURCES,
    "quant": (_CSRC + "quant_kernels.hpp", _CSRC + "quant_api.hip", _CSRC + "device_info.hpp"),
    "softmax": (_CSRC + "softmax_kernels.hpp", _CSRC + "softmax_api.hip", _CSRC + "device_info.hpp"),
}
PROBE_READ_BYTES = 1 << 30
PROBE_COPY_BYTES = 256 << 20


_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed (string and
    character literals kept), so that editing a comment does not change
    the hash below."""
    kept = _TOKENS.sub(lambda m: " " if m.group(0).startswith("/") else m.group(0), text)
    return " ".join(kept.split())


def kernel_source_hash(op: str = "gemv") -> str:
    """Hash of the code (comments aside) of one operation's kernel sources
    (the GEMV by default): a traffic summary is valid only for the code it
    was taken on."""
    h = hashlib.sha256()
    for rel in OP_SOURCES[op]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _counter(rows, name, kernel_substr):
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == name and kernel_substr in r["Kernel_Name"]]
    if not vals:
        raise ValueError(f"no {name} reading for a kernel matching {kernel_substr!r}")
    return vals


# kernel-name substring of each profiled operation's kernels
KERNEL_MATCH = {"gemv": "gemv_", "quant": "quantize_", "softmax": "softmax_f16"}


def traffic(fetch_csv, write_csv, match="gemv_"):
    """Per-launch HBM bytes of the profiled kernel (the GEMV unless `match`
    names another), with the calibration used."""
    fr, wr = _rows(fetch_csv), _rows(write_csv)
    probe_fetch_kib = max(_counter(fr, "FETCH_SIZE", "probe_read_kernel"))
    copy_write_kib = _counter(wr, "WRITE_SIZE", "probe_copy_kernel")[0]
    fetch_factor = PROBE_READ_BYTES / (probe_fetch_kib * 1024)
    write_factor = PROBE_COPY_BYTES / (copy_write_kib * 1024)
    g_fetch = _counter(fr, "FETCH_SIZE", match)
    g_write = _counter(wr, "WRITE_SIZE", match)
    kname = next(r["Kernel_Name"] for r in fr if match in r["Kernel_Name"] and r["Counter_Name"] == "FETCH_SIZE")
    fetch_b = sum(g_fetch) / len(g_fetch) * 1024 * fetch_factor
    write_b = sum(g_write) / len(g_write) * 1024 * write_factor
    return {"kernel": kname, "fetch_kib_raw": sum(g_fetch) / len(g_fetch), "write_kib_raw": sum(g_write) / len(g_write),
            "probe_fetch_kib_raw": probe_fetch_kib, "copy_write_kib_raw": copy_write_kib,
            "fetch_factor": fetch_factor, "write_factor": write_factor,
            "fetch_bytes": fetch_b, "write_bytes": write_b, "bytes_per_launch": fetch_b + write_b}


def write_traffic_summary(fetch_csv, write_csv, workload, out, fetch_cmd, write_cmd):
    """workload: '<kind>_<M>x<N>' for a GEMV kind, 'quant_q8_<M>x<N>',
    'quant_q4_<M>x<N>' or 'softmax_<M>x<N>'."""
    from memory_bound_gemv_row_amd import accounting

    name, shape = workload.rsplit("_", 1)
    M, N = (int(v) for v in shape.split("x"))
    if name.startswith("quant_"):
        op = "quant"
        t = traffic(fetch_csv, write_csv, KERNEL_MATCH[op])
        alg, what = accounting.quant_bytes(name[-2:], M, N), "quantiser"
    elif name == "softmax":
        op = "softmax"
        t = traffic(fetch_csv, write_csv, KERNEL_MATCH[op])
        alg, what = accounting.softmax_bytes(M, N), "softmax"
    else:
        op = "gemv"
        t = traffic(fetch_csv, write_csv)
        alg, what = accounting.alg_bytes(name, M, N), "GEMV"
    lines = [
        f"# HBM traffic of one {workload} {what} launch (rocprofv3 counters)",
        f"fetch command: {fetch_cmd}",
        f"write command: {write_cmd}",
        f"kernel: {t['kernel']}",
        f"kernel_source_hash: {kernel_source_hash(op)}",
        f"probe_read 1 GiB FETCH_SIZE raw KiB: {t['probe_fetch_kib_raw']:.1f} -> fetch factor {t['fetch_factor']:.4f}",
        f"probe_copy 256 MiB WRITE_SIZE raw KiB: {t['copy_write_kib_raw']:.1f} -> write factor {t['write_factor']:.4f}",
        f"kernel FETCH_SIZE raw KiB: {t['fetch_kib_raw']:.3f} -> {t['fetch_bytes']:.0f} bytes",
        f"kernel WRITE_SIZE raw KiB: {t['write_kib_raw']:.3f} -> {t['write_bytes']:.0f} bytes",
        f"bytes_per_launch: {t['bytes_per_launch']:.0f}",
        f"algorithmic_bytes: {alg}",
        f"traffic / algorithmic: {t['bytes_per_launch'] / alg:.4f}",
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return t


def write_trace_summary(stats_csv, out, command):
    rows = _rows(stats_csv)
    lines = [f"# rocprofv3 --kernel-trace --stats summary", f"command: {command}",
             "calls  avg_us  min_us  max_us  share%  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):5d} {float(r['AverageNs']) / 1e3:8.3f} {float(r['MinNs']) / 1e3:7.3f} "
                     f"{float(r['MaxNs']) / 1e3:7.3f} {float(r['Percentage']):6.2f}  {r['Name'][:150]}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_counter_summary(csv_path, out, command):
    """Every counter reading of the GEMV and probe dispatches, plus the L2
    (TCC) hit rate where both TCC_HIT_sum and TCC_MISS_sum were collected."""
    rows = [r for r in _rows(csv_path) if "gemv" in r["Kernel_Name"]]
    by_dispatch = {}
    for r in rows:
        d = by_dispatch.setdefault(r["Dispatch_Id"], {"kernel": r["Kernel_Name"][:110]})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    lines = ["# rocprofv3 counter readings per dispatch", f"command: {command}",
             f"kernel_source_hash: {kernel_source_hash()}"]
    for did, d in sorted(by_dispatch.items(), key=lambda kv: int(kv[0])):
        extra = ""
        if "TCC_HIT_sum" in d and "TCC_MISS_sum" in d:
            tot = d["TCC_HIT_sum"] + d["TCC_MISS_sum"]
            extra = f"  L2 hit rate {100 * d['TCC_HIT_sum'] / tot:.1f}%" if tot else ""
        vals = "  ".join(f"{k}={v:.0f}" for k, v in d.items() if k != "kernel")
        lines.append(f"dispatch {did}: {d['kernel']}\n    {vals}{extra}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path):
    """(bytes_per_launch, kernel_source_hash) from a traffic summary, or None."""
    try:
        with open(path) as f:
            kv = dict(line.split(": ", 1) for line in f.read().splitlines() if ": " in line)
        return float(kv["bytes_per_launch"]), kv["kernel_source_hash"].strip()
    except (OSError, KeyError, ValueError):
        return None


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        write_trace_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "counters":
        write_counter_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        print(write_traffic_summary(*sys.argv[2:8]))
    else:
        raise SystemExit(__doc__)
