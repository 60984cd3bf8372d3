"""bench.py on the CPU: it runs on one GPU only, and says so; its counts of
the work a pass executes match a count over the cells themselves.

The driver may ask for --gpus N with N > 1; the bench then exits with status
2 and a message naming the limit, before it touches a GPU.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

BK = 64


@pytest.mark.parametrize("n,batch", [(64, 1), (65, 3), (300, 2), (517, 1)])
def test_executed_triples_count_the_upper_band_pairs(n, batch):
    band = np.arange(n) // BK
    kept = band[:, None] <= band[None, :]          # quadrants (A, B), A <= B
    assert bench.executed_triples(n, batch) == int(kept.sum()) * n * batch


@pytest.mark.parametrize("n,ahead,W", [(300, 0, 1), (300, 1, 1), (517, 2, 2), (700, 2, 3),
                                       (130, 1, 1)])
def test_bulk_triples_count_the_stored_cells(n, ahead, W):
    band = np.arange(n) // BK
    TB = int(band[-1]) + 1
    stored = dense = 0
    for K in range(0, TB, W):
        live = (band < K) | (band >= min(TB, K + W * (1 + ahead)))
        atoms = int(((band >= K) & (band < K + W)).sum())
        cells = live[:, None] & live[None, :]
        stored += int((cells & (band[:, None] <= band[None, :])).sum()) * atoms
        dense += int(cells.sum()) * atoms
    assert bench.tiles_units_per_pass(n, 2, ahead, W) == (2 * stored, 2 * dense)


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
