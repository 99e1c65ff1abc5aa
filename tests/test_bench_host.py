"""Host logic of bench.py (no GPU): the comment-blind source hash that keys
the committed profile records, the kernel-trace and counter summaries that
turn rocprofv3 CSV files into those records, and the refusal of more than
one GPU."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

PREFILL = "void (anonymous namespace)::intra_kernel<false, true>((anonymous namespace)::Params)"
CARRY = "void (anonymous namespace)::inter_kernel<32>((anonymous namespace)::Params)"
REPAIR = "void (anonymous namespace)::inter_kernel<16>((anonymous namespace)::Params)"
CLEAR = "(anonymous namespace)::clear_flags_kernel(int*, long)"
DECODE = ("void (anonymous namespace)::decode_kernel<(anonymous namespace)::SplitInputs>"
          "((anonymous namespace)::SplitInputs, unsigned short*, long, long, int const*, int)")


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "kda_gated_delta_amd" / "csrc"
    src.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (src / "k.hip").write_text("// header\nint f(int x) {  // body\n  return x + 1;\n}\n")
    h0 = bench.source_hash("k.hip")
    (src / "k.hip").write_text("/* a block\n comment */\n\nint f(int x) {\n  return x + 1;   // changed note\n}\n")
    assert bench.source_hash("k.hip") == h0, "a comment or blank-line edit changed the hash"
    (src / "k.hip").write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_hash("k.hip") != h0, "a code edit left the hash unchanged"


def test_kernel_trace_summary(tmp_path):
    """Per-kernel averages from the stats file; the prefill call's span runs
    from its first kernel's start to its last kernel's end, and the decode
    (or anything else) ends a call."""
    stats = tmp_path / "run_kernel_stats.csv"
    _write_csv(stats, ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"], [
        {"Name": PREFILL, "Calls": 2, "AverageNs": 690000.0},
        {"Name": CARRY, "Calls": 2, "AverageNs": 680000.0},
        {"Name": REPAIR, "Calls": 2, "AverageNs": 4500.0},
        {"Name": CLEAR, "Calls": 2, "AverageNs": 2500.0},
        {"Name": DECODE, "Calls": 2, "AverageNs": 32000.0},
    ])
    trace = []
    for base, end_carry in ((0, 715000), (1000000, 1725000)):
        trace += [
            {"Kernel_Name": CLEAR, "Start_Timestamp": base, "End_Timestamp": base + 3000},
            {"Kernel_Name": PREFILL, "Start_Timestamp": base + 12000, "End_Timestamp": base + 700000},
            {"Kernel_Name": CARRY, "Start_Timestamp": base + 18000, "End_Timestamp": end_carry},
            {"Kernel_Name": REPAIR, "Start_Timestamp": base + 726000, "End_Timestamp": base + 730000},
            {"Kernel_Name": DECODE, "Start_Timestamp": base + 740000, "End_Timestamp": base + 772000},
        ]
    _write_csv(tmp_path / "run_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    out = tmp_path / "rec.json"
    bench.kernel_trace_summary(str(stats), str(out))
    rec = json.load(open(out))
    assert rec["prefill_calls"] == 2
    assert rec["prefill_call_span_us"] == pytest.approx(730.0)
    k = rec["kernels_us"]
    assert k["intra_kernel<false, true>"] == pytest.approx(690.0)
    assert k["inter_kernel<32>"] == pytest.approx(680.0)
    assert k["clear_flags_kernel"] == pytest.approx(2.5)
    assert k["decode_kernel"] == pytest.approx(32.0)
    assert rec["prefill_code_sha256_16"] == bench.source_hash("prefill.hip")


def test_traffic_summary(tmp_path):
    """Bytes per dispatch = counter KiB / (what the counter reads per KiB of
    a plain copy) x 1024, summed over the prefill's kernels; the repair
    launch is left out beside the 32-column carry."""
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    fetch = [{"Kernel_Name": n, "Counter_Name": "FETCH_SIZE", "Counter_Value": v}
             for n, v in ((PREFILL, 400.0), (PREFILL, 402.0), (CARRY, 500.0), (REPAIR, 170.0), (CLEAR, 1.0))]
    write = [{"Kernel_Name": n, "Counter_Name": "WRITE_SIZE", "Counter_Value": v}
             for n, v in ((PREFILL, 800.0), (CARRY, 200.0), (REPAIR, 130.0), (CLEAR, 2.0))]
    _write_csv(tmp_path / "f.csv", fields, fetch)
    _write_csv(tmp_path / "w.csv", fields, write)
    copy_bytes = 1 << 20    # 1024 KiB copied
    _write_csv(tmp_path / "cf.csv", fields, [{"Kernel_Name": "copy", "Counter_Name": "FETCH_SIZE", "Counter_Value": 512.0}])
    _write_csv(tmp_path / "cw.csv", fields, [{"Kernel_Name": "copy", "Counter_Name": "WRITE_SIZE", "Counter_Value": 1024.0}])
    out = tmp_path / "t.json"
    bench.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                          str(tmp_path / "cw.csv"), copy_bytes, str(out))
    rec = json.load(open(out))
    assert rec["fetch_scale"] == pytest.approx(0.5) and rec["write_scale"] == pytest.approx(1.0)
    assert "inter_kernel<16>" not in rec["kernels"]
    expect = ((401.0 + 500.0 + 1.0) / 0.5 + (800.0 + 200.0 + 2.0)) * 1024.0
    assert rec["hbm_bytes_per_launch"] == pytest.approx(expect)
    assert rec["kernels"]["intra_kernel<false, true>"]["fetch_bytes"] == pytest.approx(401.0 / 0.5 * 1024.0)


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout.strip() == ""
