"""bench.py's command line on the CPU: it measures one GPU only and says so
before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU only" in proc.stderr


def test_help_lists_the_workloads():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0
    for w in ("llama3_8b_decode", "long_split_decode", "large_ragged_decode", "ragged_prefill", "kv_append"):
        assert w in proc.stdout
