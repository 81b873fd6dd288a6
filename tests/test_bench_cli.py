"""The bench's command-line contract on the CPU: more than one GPU is refused with a message (the layer path is
single-GPU), and the traffic file's source hash ignores comments.  No GPU is touched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    csrc = tmp_path / "post_weight_quantization_09_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (csrc / "k.hip").write_text("int f() { return 1; }  // one\n\n// note\nint g();\n")
    h1 = bench.source_hash("k.hip")
    (csrc / "k.hip").write_text("// header\nint f() { return 1; }  // other\nint g();   \n")
    assert bench.source_hash("k.hip") == h1
    (csrc / "k.hip").write_text("int f() { return 2; }\nint g();\n")
    assert bench.source_hash("k.hip") != h1


def test_traffic_is_keyed_by_workload(tmp_path, monkeypatch):
    """The HBM traffic of a kernel is read only from the summary of the same workload and source."""
    import json
    sys.path.insert(0, ROOT)
    import bench
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"workload": "c5_down_proj_70b", "source_hash": "abc", "bytes_per_launch": 123.0}
    (tmp_path / "profiles" / "gram_bf16_c5_down_proj_70b_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("gram_bf16", "c5_down_proj_70b", "abc") == 123.0
    assert bench.measured_traffic("gram_bf16", "c5_down_proj_70b", "other") is None
    assert bench.measured_traffic("gram_bf16", "c2_q_proj_8b", "abc") is None
    (tmp_path / "profiles" / "gram_bf16_c2_q_proj_8b_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("gram_bf16", "c2_q_proj_8b", "abc") is None   # a file naming another workload
