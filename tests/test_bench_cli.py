"""CPU checks of bench.py's contract that need no GPU: more than one GPU is
refused with a message (one GPU is measured), and the algorithmic byte count
of a projection call follows its definition."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_call_bytes_definition():
    sys.path.insert(0, ROOT)
    import bench
    # weight K*N, column scales 4N, fp32 activations 4MK, fp32 output 4MN
    assert bench.call_bytes(16, 1024, 2048) == 2301952
    assert bench.call_bytes(1, 3072, 1024) == 3072 * 1024 + 4 * 1024 + 4 * 3072 + 4 * 1024
