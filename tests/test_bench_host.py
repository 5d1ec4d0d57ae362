"""Host-side checks of bench.py that need no GPU: the single-GPU contract
(any --gpus other than 1 exits with status 2 and says why, before touching a
device) and the workload table."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_workloads_listed():
    sys.path.insert(0, ROOT)
    import bench
    assert {"opt6.7b", "attn6.7b", "robust8192", "decode70b", "opt175b", "ln8192"} <= set(bench.WORKLOADS)
