"""bench.py's command line on the CPU: more than one GPU is refused with a
message before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_per_config_rejects_the_headline_workload():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "2",
                        "--per-config", "1,2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--per-config" in r.stderr
    assert r.stdout == ""
