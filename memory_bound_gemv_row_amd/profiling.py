"""Summaries of rocprofv3 runs of ``bench.py`` (kernel trace and counters).

Usage (after the rocprofv3 runs named in each summary's header)::

    python -m memory_bound_gemv_row_amd.profiling trace  <kernel_stats.csv> <out.txt> <command>
    python -m memory_bound_gemv_row_amd.profiling counters <counter_collection.csv> <out.txt> <command>
    python -m memory_bound_gemv_row_amd.profiling traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <workload> <out.txt> <fetch command> <write command>
    python -m memory_bound_gemv_row_amd.profiling table <workload> <out.txt> \
        <run dir> <command> [<run dir> <command> ...]
    python -m memory_bound_gemv_row_amd.profiling search <plan-search jsonl> <seed|named> <out.txt>
    python -m memory_bound_gemv_row_amd.profiling sweep <plan-sweep jsonl> <seed> <out.txt>

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
import json
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


def _traced_op(names):
    """The operation a trace profiles, from its kernel names."""
    if any("quantize_" in n for n in names):
        return "quant"
    if any("softmax_f16" in n for n in names):
        return "softmax"
    return "gemv"


def write_trace_summary(stats_csv, out, command):
    rows = _rows(stats_csv)
    op = _traced_op([r["Name"] for r in rows])
    lines = [f"# rocprofv3 --kernel-trace --stats summary", f"command: {command}",
             f"kernel_source_hash: {kernel_source_hash(op)}",
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


def _agent(agent_csv):
    """Num_Xcc, Cu_Count, Simd_Count and Max_Waves_Per_Cu of the profiled GPU."""
    for r in _rows(agent_csv):
        if r.get("Agent_Type", "").upper() == "GPU":
            a = {k: int(r[k]) for k in ("Num_Xcc", "Cu_Count", "Simd_Count", "Max_Waves_Per_Cu", "Cu_Per_Engine")}
            a["Shader_Engines"] = a["Cu_Count"] // a["Cu_Per_Engine"]
            return a
    raise ValueError(f"no GPU agent in {agent_csv}")


def _mean_dispatches(csv_path, match, skip, largest=False):
    """Mean of each counter over the dispatches whose kernel name contains
    `match`, after the first `skip` of them (warm launches only); with
    `largest`, only the dispatches of the largest grid (the full-size
    probe, not the one-workgroup launch-floor probes)."""
    per, grid = {}, {}
    for r in _rows(csv_path):
        if match in r["Kernel_Name"]:
            i = int(r["Dispatch_Id"])
            per.setdefault(i, {})[r["Counter_Name"]] = float(r["Counter_Value"])
            per[i]["_kernel"] = r["Kernel_Name"]
            grid[i] = int(r["Grid_Size"])
    ids = sorted(per)
    if largest and ids:
        g = max(grid.values())
        ids = [i for i in ids if grid[i] == g]
    ids = ids[skip:]
    if not ids:
        raise ValueError(f"no dispatch of {match!r} after the first {skip} in {csv_path}")
    keys = [k for k in per[ids[0]] if k != "_kernel"]
    return {k: sum(per[i][k] for i in ids) / len(ids) for k in keys}, per[ids[0]]["_kernel"], len(ids)


def derived_counters(c, agent):
    """Figures from SQ/TCC readings of one dispatch.  SQ_BUSY_CYCLES is
    summed over the shader engines (Cu_Count / Cu_Per_Engine of them), so the
    kernel's busy cycles are T = SQ_BUSY_CYCLES / engines (GRBM_GUI_ACTIVE /
    Num_Xcc also counts the dispatch's set-up, long next to a short kernel);
    SQ_WAVE_CYCLES, SQ_ACTIVE_INST_VALU and SQ_WAIT_INST_ANY count in units
    of four cycles (a wave64 VALU instruction occupies its SIMD for four),
    summed over the CUs:
      waves per CU  4 SQ_WAVE_CYCLES / (Cu_Count T)   (occupancy; max Max_Waves_Per_Cu)
      VALU busy     4 SQ_ACTIVE_INST_VALU / (Simd_Count T)
      wait to issue SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of wave time waiting for an instruction to issue)
      L2 hit rate   TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)"""
    out = {}
    if c.get("SQ_BUSY_CYCLES"):
        T = c["SQ_BUSY_CYCLES"] / agent["Shader_Engines"]
    else:
        T = c.get("GRBM_GUI_ACTIVE", 0) / agent["Num_Xcc"]
    if T and "SQ_WAVE_CYCLES" in c:
        out["waves_per_cu"] = 4 * c["SQ_WAVE_CYCLES"] / (agent["Cu_Count"] * T)
    if T and "SQ_ACTIVE_INST_VALU" in c:
        out["valu_busy"] = 4 * c["SQ_ACTIVE_INST_VALU"] / (agent["Simd_Count"] * T)
    if c.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in c:
        out["waiting"] = c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]
    if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c and c["TCC_HIT_sum"] + c["TCC_MISS_sum"] > 0:
        out["l2_hit"] = c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
    if c.get("SQ_WAVES") and "SQ_INSTS_VALU" in c:
        out["valu_per_wave"] = c["SQ_INSTS_VALU"] / c["SQ_WAVES"]
    if c.get("SQ_WAVES") and "SQ_INSTS_LDS" in c:
        out["lds_per_wave"] = c["SQ_INSTS_LDS"] / c["SQ_WAVES"]
    out["busy_us_at_2.4GHz"] = T / 2.4e3
    return out


def _fmt_derived(d, agent):
    parts = []
    if "waves_per_cu" in d:
        parts.append(f"waves per CU {d['waves_per_cu']:.1f} of {agent['Max_Waves_Per_Cu']}")
    if "valu_busy" in d:
        parts.append(f"VALU busy {100 * d['valu_busy']:.1f}%")
    if "waiting" in d:
        parts.append(f"wait to issue {100 * d['waiting']:.1f}%")
    if "l2_hit" in d:
        parts.append(f"L2 hit rate {100 * d['l2_hit']:.1f}%")
    if "valu_per_wave" in d:
        parts.append(f"VALU per wave {d['valu_per_wave']:.0f}")
    if "lds_per_wave" in d:
        parts.append(f"LDS instr per wave {d['lds_per_wave']:.1f}")
    parts.append(f"busy {d['busy_us_at_2.4GHz']:.2f} us at 2.4 GHz")
    return "; ".join(parts)


def write_counter_table(workload, out, passes, skip=4):
    """One workload's counter passes (rocprofv3 --pmc of a short bench.py
    run, each GEMV launch a dispatch of its own), averaged over the warm GEMV
    dispatches, with derived figures (derived_counters), and the same figures
    for the run's pure-read probe as a reference.

    passes: [(run directory holding *counter_collection.csv and
    *agent_info.csv, command), ...]."""
    import glob

    lines = [f"# rocprofv3 counters of the {workload} GEMV (mean over warm launches) and the same run's probe",
             f"kernel_source_hash: {kernel_source_hash()}"]
    gemv, probe, kname, n, agent = {}, {}, None, 0, None
    for d, cmd in passes:
        csv_path = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
        agent = _agent(glob.glob(os.path.join(d, "*agent_info.csv"))[0])
        vals, kname, n = _mean_dispatches(csv_path, "gemv_stream", skip) if "gemv_stream" in open(csv_path).read() \
            else _mean_dispatches(csv_path, "gemv_", skip)
        pvals, _, _ = _mean_dispatches(csv_path, "probe_read_kernel", 0, largest=True)
        gemv.update(vals)
        probe.update(pvals)
        lines.append(f"command: {cmd}")
    lines.append(f"agent: {agent}")
    lines.append(f"kernel: {kname}  (mean of {n} warm dispatches)")
    lines.append("readings: " + "  ".join(f"{k}={v:.0f}" for k, v in sorted(gemv.items())))
    lines.append("derived: " + _fmt_derived(derived_counters(gemv, agent), agent))
    lines.append("probe readings: " + "  ".join(f"{k}={v:.0f}" for k, v in sorted(probe.items())))
    lines.append("probe derived: " + _fmt_derived(derived_counters(probe, agent), agent))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _bench_lines(src, key):
    rows, summary = [], None
    with open(src) as f:
        for line in f:
            if not line.startswith("{"):
                continue
            d = json.loads(line)
            if key in d:
                summary = d[key]
            else:
                rows.append(d)
    return rows, summary


def write_search_summary(src, seed, out):
    """Text summary of `bench.py --plan-search 24 --seed <seed>` output (JSON
    lines in `src`): per shape the library's plan against the fastest of
    every plan the library holds a kernel for."""
    rows, summ = _bench_lines(src, "plan_search")
    named = seed == "named"
    with open(out, "w") as f:
        f.write("# bench.py --plan-search: the library's plan against every plan it holds a kernel for "
                f"(gemv_launch_plan), graph-timed, best of {5 if named else 3}\n")
        run = "--plan-search-named" if named else f"--plan-search 24 --seed {seed}"
        f.write(f"command: python3 bench.py {run} > {os.path.basename(src)}\n")
        f.write(f"summary by: python3 -m memory_bound_gemv_row_amd.profiling search {os.path.basename(src)} {seed} "
                f"{os.path.basename(out)}\n")
        f.write(f"kernel_source_hash: {kernel_source_hash()}\n")
        f.write("summary (library plan / fastest candidate: geometric mean, median, worst): " + "; ".join(
            f"{k} {v['geomean_lib_over_best']:.3f} / {v['median_lib_over_best']:.3f} / {v['worst_lib_over_best']:.3f} "
            f"(worst {v['worst_shape']})" for k, v in summ.items()) + "\n")
        f.write("kind    M       N     lib_us   best_us  lib/best  candidates  library plan (variant grid block "
                "in-flight stage)  fastest (variant waves in-flight rows stage cap)\n")
        for r in sorted(rows, key=lambda r: (r["kind"], r["lib_over_best"])):
            p = r["lib_plan"]
            f.write(f"{r['kind']:6s} {r['M']:6d} {r['N']:6d} {r['lib_us']:9.3f} {r['best_us']:9.3f} "
                    f"{r['lib_over_best']:7.3f} {r['candidates']:6d}      {p['variant']} {p['grid']} {p['block']} "
                    f"{p['units_in_flight']} {p['stage_order']}      {' '.join(map(str, r['best_plan']))}\n")


def write_sweep_summary(src, seed, out):
    """Text summary of `bench.py --plan-sweep 24 --seed <seed>` output: each
    shape's plan against the pure-read probe over the same bytes."""
    rows, summ = _bench_lines(src, "plan_sweep")
    with open(out, "w") as f:
        f.write("# bench.py --plan-sweep: each shape's plan against the pure-read probe over the same bytes "
                "(graph-timed, best of 3)\n")
        f.write(f"command: python3 bench.py --plan-sweep 24 --seed {seed} > {os.path.basename(src)}\n")
        f.write(f"summary by: python3 -m memory_bound_gemv_row_amd.profiling sweep {os.path.basename(src)} {seed} "
                f"{os.path.basename(out)}\n")
        f.write(f"kernel_source_hash: {kernel_source_hash()}\n")
        f.write("summary (worst / median % of the same-size probe): " + "; ".join(
            f"{k} {v['worst_pct']} / {v['median_pct']} (worst {v['worst_shape']})" for k, v in summ.items()) + "\n")
        f.write("kind    M       N        us   probe_us  %probe  variant grid block units_in_flight stage\n")
        for r in sorted(rows, key=lambda r: (r["kind"], r["pct_of_same_size_probe"])):
            p = r["plan"]
            f.write(f"{r['kind']:6s} {r['M']:6d} {r['N']:6d} {r['us']:9.3f} {r['same_size_probe_us']:9.3f} "
                    f"{r['pct_of_same_size_probe']:6.1f}  {p['variant']} {p['grid']} {p['block']} "
                    f"{p['units_in_flight']} {p['stage_order']}\n")


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
    elif sys.argv[1] == "table":
        # table <workload> <out.txt> <run dir 1> <cmd 1> [<run dir 2> <cmd 2> ...]
        a = sys.argv[4:]
        write_counter_table(sys.argv[2], sys.argv[3], list(zip(a[0::2], a[1::2])))
    elif sys.argv[1] == "search":
        write_search_summary(sys.argv[2], sys.argv[3], sys.argv[4])   # <bench jsonl> <seed> <out.txt>
    elif sys.argv[1] == "sweep":
        write_sweep_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    else:
        raise SystemExit(__doc__)
