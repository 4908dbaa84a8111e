"""CPU checks of the rocprofv3 summary helpers: the counter calibration that
turns FETCH_SIZE / WRITE_SIZE readings into bytes, the byte models they are
compared with, and the round trip of the committed summary format."""
import csv
import os

import pytest

from memory_bound_gemv_row_amd import accounting, profiling


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


@pytest.mark.parametrize("workload,match,alg", [
    ("f16_8192x8192", "void gemv::gemv_stream<1, 8, 8, true, true, 0>", accounting.alg_bytes("f16", 8192, 8192)),
    ("quant_q4_4096x14336", "void gquant::quantize_q4_kernel<4, 4, true>", accounting.quant_bytes("q4", 4096, 14336)),
    ("softmax_1024x131072", "void gsoftmax::softmax_f16_kernel<16, 16>", accounting.softmax_bytes(1024, 131072)),
])
def test_traffic_calibration_and_summary(tmp_path, workload, match, alg):
    # the probe reads 1 GiB but FETCH_SIZE shows half (factor 2); the copy
    # writes 256 MiB and WRITE_SIZE shows it exactly; the kernel's readings
    # are chosen so that calibrated traffic equals the algorithmic bytes
    fetch_kib = alg * 0.75 / 1024 / 2          # three quarters of the bytes are reads
    write_kib = alg * 0.25 / 1024
    fr, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counters(fr, [("void gemv::probe_read_kernel<4, true>", "FETCH_SIZE", (1 << 30) / 1024 / 2),
                         (match, "FETCH_SIZE", fetch_kib),
                         ("void gemv::probe_read_kernel<4, true>", "FETCH_SIZE", (1 << 30) / 1024 / 2)])
    _write_counters(wr, [(match, "WRITE_SIZE", write_kib),
                         ("void gemv::probe_copy_kernel<4, true>", "WRITE_SIZE", (256 << 20) / 1024)])
    out = tmp_path / "summary.txt"
    t = profiling.write_traffic_summary(str(fr), str(wr), workload, str(out), "fetch cmd", "write cmd")
    assert t["fetch_factor"] == pytest.approx(2.0)
    assert t["write_factor"] == pytest.approx(1.0)
    assert t["bytes_per_launch"] == pytest.approx(alg, rel=1e-9)
    text = out.read_text()
    assert "traffic / algorithmic: 1.0000" in text
    got = profiling.read_traffic(str(out))
    op = "quant" if workload.startswith("quant") else ("softmax" if workload.startswith("softmax") else "gemv")
    assert got == (pytest.approx(alg, rel=1e-6), profiling.kernel_source_hash(op))


def test_byte_models():
    assert accounting.quant_bytes("q8", 8192, 8192) == 4 * 8192 * 8192 + 8192 * 8192 + 6 * 8192
    assert accounting.quant_bytes("q4", 4096, 14336) == 4 * 4096 * 14336 + 4096 * 7168 + 2 * 4096 * 112 + 4 * 4096
    assert accounting.softmax_bytes(1024, 131072) == 4 * 1024 * 131072


def test_committed_summaries_parse():
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
    for f in os.listdir(root):
        if f.endswith("_traffic.txt"):
            got = profiling.read_traffic(os.path.join(root, f))
            assert got is not None and got[0] > 0, f


def test_source_hash_ignores_comments_not_code():
    src = 'int f(int a) { // add one\n  return a + 1; /* done */ }\nconst char* s = "a // b";\n'
    same = 'int f(int a) {\n  // a different comment\n  return a + 1; }\nconst char* s = "a // b";\n'
    other = 'int f(int a) { return a + 2; }\nconst char* s = "a // b";\n'
    assert profiling.code_only(src) == profiling.code_only(same)
    assert profiling.code_only(src) != profiling.code_only(other)
    assert '"a // b"' in profiling.code_only(src)   # string literals are code
