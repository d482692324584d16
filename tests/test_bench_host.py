"""Host logic of bench.py that runs without a GPU: the one-GPU guard and the tie between the
committed HBM counter record and the kernel source it was taken on."""
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_hash_ignores_comments_and_whitespace(tmp_path):
    src = os.path.join(ROOT, "fp8_compression_tensor_amd", "csrc")
    copy = tmp_path / "csrc"
    shutil.copytree(src, copy)
    h0 = bench.kernel_source_hash(str(copy))
    assert h0 == bench.kernel_source_hash(src)
    f = copy / "tfp8_kernels.hip"
    text = f.read_text()
    f.write_text("// a new comment\n/* and a block\n comment */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash(str(copy)) == h0
    f.write_text(text + "\nstatic const int one_more_constant = 1;\n")
    assert bench.kernel_source_hash(str(copy)) != h0


def test_traffic_record_applies_only_to_its_source(tmp_path):
    src = os.path.join(ROOT, "fp8_compression_tensor_amd", "csrc")
    rec = {"fetch_bytes_per_launch": 1.5e9, "write_bytes_per_launch": 1.0e9,
           "kernel_source_sha256": bench.kernel_source_hash(src)}
    p = tmp_path / "rec.json"
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p), src) == 2.5e9
    rec["kernel_source_sha256"] = "0" * 64
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p), src) is None
    assert bench.measured_traffic(str(tmp_path / "missing.json"), src) is None



def test_cpu_model_names_the_host_cpu():
    # taken from lscpu (before the bench touches the GPU), else /proc/cpuinfo
    m = bench.cpu_model()
    assert isinstance(m, str) and m and m != "unknown"
    if shutil.which("lscpu"):
        assert "lscpu: vendor" in m
