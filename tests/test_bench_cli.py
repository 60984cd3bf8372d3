"""bench.py's command line on the CPU: it runs on one GPU only, and says so.

The driver may ask for --gpus N with N > 1; the bench then exits with status
2 and a message naming the limit, before it touches a GPU.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_world_size_above_one_exits_with_a_message():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr
