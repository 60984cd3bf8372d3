"""The synthetic inputs have the shapes, structure and guarantees they claim."""
import numpy as np
import pytest

import pins
from distance_geometry_bound_amd import gen
from oracle import check


def test_deterministic():
    a = gen.make_molecule(200, seed=3)
    b = gen.make_molecule(200, seed=3)
    assert np.array_equal(a.U, b.U) and np.array_equal(a.L, b.L) and np.array_equal(a.X, b.X)
    c = gen.make_molecule(200, seed=4)
    assert not np.array_equal(a.U, c.U)


def test_walk_geometry():
    X = gen.walk_chain(300, seed=9)
    steps = np.sqrt(((X[1:] - X[:-1]) ** 2).sum(-1))
    assert np.allclose(steps, gen.STEP, atol=1e-9)
    d = gen.true_distances(X)
    np.fill_diagonal(d, np.inf)
    assert d.min() >= gen.EXCL


def test_sphere_geometry():
    X = gen.sphere_chains(6, 64, 25.0, seed=5)
    assert X.shape == (384, 3)
    assert np.sqrt((X ** 2).sum(-1)).max() <= 25.0 + 1e-9
    d = gen.true_distances(X)
    np.fill_diagonal(d, np.inf)
    assert d.min() >= gen.EXCL
    for c in range(6):
        Y = X[c * 64:(c + 1) * 64]
        assert np.allclose(np.sqrt(((Y[1:] - Y[:-1]) ** 2).sum(-1)), gen.STEP, atol=1e-9)


@pytest.mark.parametrize("name", ["n128", "n1024", "b64n500", "n4096", "n12288"])
def test_workload_contract(name):
    W = gen.make_workload(name, batch=4 if name == "b64n500" else None)
    assert W.U.shape == (W.batch, W.n, W.n) and W.U.dtype == np.float32
    if name != "n12288":
        assert check.flags(W.U, W.L) == 0
    for b in range(W.batch):
        U, L = W.U[b], W.L[b]
        assert np.array_equal(U, U.T) and np.array_equal(L, L.T)
        assert np.all(np.diag(U) == 0) and np.all(np.diag(L) == 0)
        assert np.all(L <= U) and np.all(L >= 0)
        assert np.all(U * 64 == np.round(U * 64)) and np.all(L * 64 == np.round(L * 64))
        assert pins.sound(U, L, W.X[b])
        # bonded neighbours are known to within one grid step
        i = np.arange(W.n - 1)
        if name in ("n4096", "n12288"):
            i = i[(i % 256) != 255]
        assert np.all(U[i, i + 1] - L[i, i + 1] <= 2.0 / 64)


def test_workload_rules():
    W = gen.make_workload("n4096")
    U, L = W.U[0], W.L[0]
    off = ~np.eye(W.n, dtype=bool)
    assert set(np.unique(U[off & (U > 7.0)])) == {120.0}
    assert L[off].min() == 1.0
    W = gen.make_workload("n12288")
    U = W.U[0]
    assert U.max() == 180.0
    frac_known = np.count_nonzero(U < 180.0) / U.size
    assert 1e-4 < frac_known < 1e-2


def test_random_generators_contract():
    U, L = gen.random_bounds(30, seed=1)
    assert np.array_equal(U, U.T) and np.all(L <= U) and np.all(np.diag(U) == 0)
    U, L, X = gen.random_sound_bounds(30, seed=2)
    assert pins.sound(U, L, X) and check.flags(U, L) == 0
    U, L = gen.random_directed_bounds(12, seed=3)
    assert not np.array_equal(U, U.T) and np.all(L <= U)
