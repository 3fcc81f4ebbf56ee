"""Host-side logic of bench.py (no GPU): the one-GPU refusal and the source
hash that keys the stored HBM counter readings to the FFN kernels' code."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup",
                        "0"], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int a) {\n  return a + 1; // add one\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "FFN_SOURCES", ("k.hip",))
    h0 = bench.ffn_source_hash()
    src.write_text("/* header */\nint f(int a)\n{\n    return a + 1;   // one more\n}\n")
    assert bench.ffn_source_hash() == h0
    src.write_text("int f(int a) {\n  return a + 2;\n}\n")
    assert bench.ffn_source_hash() != h0


def test_prefill_mfma_summary_from_counters(tmp_path):
    # one gate/up dispatch of the 16384-token leg, 1,000 us: 1.0 G busy SIMD
    # cycles (2.0 G MOPS, 1,024 flops per busy cycle) at MfmaUtil 54.25 % put
    # one XCD's GUI-active count at 1.0e9 / (0.5425 * 1024) = 1.80 M cycles,
    # a 1.80 GHz clock; 1.5 TFLOP of algorithmic work in 1 ms is 0.6 of the
    # 2.5 PFLOP/s peak and 0.8 of the peak at 1.80 GHz
    import csv
    busy, util, us = 1.0e9, 54.2534722, 1000.0  # 1e9 / (0.542534722 * 1024) = 1.80 M cycles over 1 ms
    name = "void (anonymous namespace)::k_pf_wide<0>((anonymous namespace)::PfArgs)"
    grid = 8 * 33 * 12 * 256
    tr = tmp_path / "kt"
    tr.mkdir()
    with open(tr / "x_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, ["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp", "Dispatch_Id"])
        w.writeheader()
        w.writerow({"Kernel_Name": name, "Grid_Size_X": grid, "Start_Timestamp": 0, "End_Timestamp": int(us * 1e3),
                    "Dispatch_Id": 1})
    mf = tmp_path / "mfma"
    mf.mkdir()
    with open(mf / "x_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("GRBM_GUI_ACTIVE", 8 * 1.8e6), ("MfmaUtil", util),
                     ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 2 * busy)):
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": c, "Counter_Value": v})
    flops = 1.5e12
    legs = [(16384, [("k_pf_wide<0>", 1.0, flops, grid)])]

    def pick(rows, kname, g, key):
        return [r for r in rows if bench._short(r["Kernel_Name"]) == kname and int(r[key]) == g]

    trace = bench._csv_rows(str(tr), "kernel_trace.csv")
    lines = bench._prefill_mfma_lines(str(mf), trace, legs, pick)
    row = [l for l in lines if "k_pf_wide<0>" in l]
    assert len(row) == 1
    f = row[0].split()
    # busy %, clock, MFMA TFLOP (2e9 MOPS * 512), alg TFLOP, ratio, TFLOP/s, of peak, at clock
    assert f[1] == "54.3%" and f[2] == "1.80"
    assert f[3] == "1.02" and f[4] == "1.50" and f[5] == "0.68"
    assert f[6] == "1500.0" and f[7] == "0.600" and f[8] == "0.800"
