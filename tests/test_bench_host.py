"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the source hash
that keeps counter records attached to unchanged kernels, and the workload
labels of the JSON line."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout and "--gpus 2" in r.stdout


def test_source_sha_ignores_comments_and_blank_lines(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n    return x + 1;\n}\n")
    b.write_text("// header\n\nint f(int x) {  /* inline\n note */\n    return x + 1;  // trailing\n}\n\n")
    c.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert bench.source_sha(str(a)) == bench.source_sha(str(b))
    assert bench.source_sha(str(a)) != bench.source_sha(str(c))


def test_workload_labels_name_shape_and_adapters():
    up = bench.workload_label(workloads.config("llama_up"))
    assert "4096x14336" in up and "32_adapters" in up
    for name in ("qwen_q", "llama_sq", "longtail"):
        label = bench.workload_label(workloads.config(name))
        wl = workloads.config(name)
        assert "%dx%d" % (wl.d_in, wl.d_out) in label
