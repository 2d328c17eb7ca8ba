"""Host-side checks of bench.py's command-line contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    # the benchmark runs on one GPU; asking for more exits with status 2 and a message,
    # before touching any device
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_bench_workload_constants_match_the_metric_config():
    sys.path.insert(0, ROOT)
    import bench
    assert (bench.M, bench.K, bench.N, bench.R) == (4096, 3072, 3072, 32)
    assert bench.WORKLOAD == "attn_4096x3072x3072_r32"
    # the recorded traffic file names the GEMM sources it was taken on
    text = open(os.path.join(ROOT, bench.TRAFFIC_FILE)).read()
    assert "sources_sha256_16:" in text and "hbm_bytes_per_launch:" in text
