"""Host-side checks of bench.py (no GPU): the one-GPU contract."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_source_hash_is_stable():
    sys.path.insert(0, ROOT)
    import bench

    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
