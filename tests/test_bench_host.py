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
