"""bench.py's contract checks that need no GPU: more than one GPU is refused
with a message and a non-zero exit, and the committed traffic summary parses
into the fields the JSON line's roofline reads."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_summary_has_the_roofline_fields():
    kv = {}
    with open(os.path.join(ROOT, "profiles", "sparse_gemm_2048x4096x4096_traffic.txt")) as f:
        for line in f:
            if not line.startswith("#") and ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    for key in ("hbm_read_bytes_per_launch", "hbm_write_bytes_per_launch", "hbm_bytes_per_launch",
                "algorithmic_bytes_per_launch", "kernel_source_sha256"):
        assert key in kv, key
    assert float(kv["hbm_bytes_per_launch"]) == float(kv["hbm_read_bytes_per_launch"]) + float(
        kv["hbm_write_bytes_per_launch"])
    assert len(kv["kernel_source_sha256"]) == 64
