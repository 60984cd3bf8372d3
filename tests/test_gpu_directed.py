"""Directed-rounding passes on the GPU against the CPU oracle (needs an MI355X).

Directed rounding rounds sums of upper bounds up and differences of lower
bounds down (the notes on GPU Gems 2, Ch. 43 say the smoothing is sensitive
to precision, §6).  The inputs here are off the 2^-6 grid, so rounding matters.

  * Per-round and single-workgroup kernels: bit for bit the oracle's directed
    rounds, in the same order, including partial ranges.
  * Every algorithm on grid inputs: every operation is exact there, so the
    bits are those of the plain pass.
  * Blocked pass on inputs off the grid: it groups the roundings differently.
    It must lie within the derived rounding bound of the oracle's directed
    result (see tests/test_directed_pins.py): U within a factor
    (1 + 2^-23)^(n-2) either way, L within delta.  It must also be sound
    against the true distances, and give L <= U.
"""
import numpy as np
import pytest
import torch

import distance_geometry_bound_amd as dgb
import oracle
from distance_geometry_bound_amd import gen
from oracle import steps

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
EPS = 2.0 ** -23


def dev(A):
    return torch.from_numpy(np.ascontiguousarray(A)).to(DEV)


def host(T):
    torch.cuda.synchronize(DEV)
    return T.cpu().numpy()


def bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint32),
                          np.ascontiguousarray(b).view(np.uint32))


def unquantised(n, batch, seed):
    U, L, _ = gen.random_unquantised_bounds(n, seed=seed, batch=batch, box=6.0 + n / 8,
                                            slack=0.0 if seed % 2 else 1.0, known=0.5)
    return U, L


def within_bound(Ug, Lg, Uo, Lo, L0):
    """The derived rounding bound between two directed results of one input."""
    n = Uo.shape[-1]
    grow = (1.0 + EPS) ** max(n - 2, 0) * (1.0 + 4 * EPS)   # + float64 slack of this check
    U64, Uo64 = Ug.astype(np.float64), Uo.astype(np.float64)
    fin = np.isfinite(Uo64)
    ok_u = np.array_equal(np.isfinite(U64), fin) and \
        np.all(U64[fin] <= Uo64[fin] * grow) and np.all(U64[fin] * grow >= Uo64[fin])
    umax = float(Uo64[fin].max()) if fin.any() else 0.0
    lmax = float(np.asarray(L0, dtype=np.float64).max())
    delta = 2 * umax * (grow - 1) + 2 * n * EPS * (lmax + 2 * umax)
    ok_l = np.all(np.abs(Lg.astype(np.float64) - Lo.astype(np.float64)) <= delta)
    return ok_u and ok_l


# ---------------------------------------------------------------- bit-exact paths
@pytest.mark.parametrize("n,batch,algo", [
    (1, 1, "perk"), (2, 2, "perk"), (7, 2, "lds"), (7, 2, "perk"), (64, 1, "lds"),
    (65, 3, "lds"), (101, 2, "perk"), (130, 2, "lds"), (176, 1, "lds"), (176, 1, "auto"),
    (257, 1, "perk"), (300, 2, "perk"),
])
def test_directed_matches_oracle_bit_for_bit(n, batch, algo):
    U0, L0 = unquantised(n, batch, seed=n + batch)
    Ue, Le = oracle.smooth_directed(U0, L0)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, algo=algo)
    assert bits_equal(host(U), Ue) and bits_equal(host(L), Le), (n, batch, algo)


@pytest.mark.parametrize("n", [40, 130])
def test_directed_line_matches_oracle_and_is_sound(n):
    U0, L0, X = gen.unquantised_line(n, seed=n)
    d = gen.true_distances(X)
    Ue, Le = oracle.smooth_directed(U0, L0)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L)
    Ug, Lg = host(U), host(L)
    assert bits_equal(Ug, Ue) and bits_equal(Lg, Le)
    assert np.all(Ug.astype(np.float64) >= d) and np.all(Lg.astype(np.float64) <= d)


@pytest.mark.parametrize("n,cuts,algo", [
    (150, [0, 1, 50, 149, 150], "lds"),
    (150, [0, 37, 150], "perk"),
    (300, [0, 1, 63, 64, 100, 300], "perk"),
])
def test_directed_ranges_match_oracle(n, cuts, algo):
    U0, L0 = unquantised(n, 2, seed=n + len(cuts))
    U, L = dev(U0), dev(L0)
    Ue, Le = U0, L0
    for a, b in zip(cuts[:-1], cuts[1:]):
        dgb.smooth_directed_range(U, L, a, b, algo=algo)
        Ue, Le = oracle.rounds_directed(Ue, Le, a, b)
        assert bits_equal(host(U), Ue) and bits_equal(host(L), Le), (algo, a, b)


@pytest.mark.parametrize("n,batch", [(7, 2), (130, 1), (260, 1)])
def test_directed_packed_small_and_per_round_match_oracle(n, batch):
    # n <= 176: single workgroup; n = 260 with a ragged range: per-round kernel
    U0, L0 = unquantised(n, batch, seed=3 * n)
    P = dgb.pack(dev(U0), dev(L0))
    if n <= 176:
        dgb.smooth_packed_directed(P)
        Ue, Le = oracle.smooth_directed(U0, L0)
    else:
        dgb.smooth_packed_directed(P, 0, 37)
        Ue, Le = oracle.rounds_directed(U0, L0, 0, 37)
    assert bits_equal(host(P), steps.pack(Ue, Le))


# ---------------------------------------------------------------- grid inputs
@pytest.mark.parametrize("n,batch", [(177, 1), (300, 2), (700, 1)])
def test_directed_blocked_on_grid_equals_plain_pass(n, batch):
    U0, L0, _ = gen.random_sound_bounds(n, seed=n, batch=batch, box=6.0 + n / 8)
    Ue, Le = oracle.smooth(U0, L0)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, algo="blocked")
    assert bits_equal(host(U), Ue) and bits_equal(host(L), Le)
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed_directed(P)
    assert bits_equal(host(P), steps.pack(Ue, Le))


def test_directed_blocked_on_grid_workload_n4096():
    W = gen.make_workload("n4096")
    Ue, Le = oracle.smooth(W.U, W.L)
    U, L = dev(W.U), dev(W.L)
    dgb.smooth_directed(U, L)
    assert bits_equal(host(U), Ue) and bits_equal(host(L), Le)


# ---------------------------------------------------------------- off the grid, blocked
@pytest.mark.parametrize("n,batch", [(177, 2), (300, 1), (700, 1), (1024, 1)])
def test_directed_blocked_within_rounding_bound(n, batch):
    U0, L0 = unquantised(n, batch, seed=n)
    Ue, Le = oracle.smooth_directed(U0, L0)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, algo="blocked")
    Ug, Lg = host(U), host(L)
    assert within_bound(Ug, Lg, Ue, Le, L0)
    assert np.all(Lg <= Ug)
    # the packed layout runs the same kernels in the same order
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed_directed(P)
    assert bits_equal(host(P), steps.pack(Ug, Lg))


@pytest.mark.parametrize("n,batch,bands,blocks,lead", [
    (700, 1, 2, 2, None), (700, 1, 2, 4, None), (700, 1, 1, 3, None), (385, 2, 2, 4, None),
    (700, 1, 0, 1, True), (385, 3, 0, 1, True)])
def test_directed_steps_within_rounding_bound(n, batch, bands, blocks, lead):
    # steps of several k-blocks, and the lead schedule's products, group the
    # roundings differently again; every path sum still takes at most n - 2
    # roundings, so the same bound holds
    U0, L0 = unquantised(n, batch, seed=3 * n + blocks)
    Ue, Le = oracle.smooth_directed(U0, L0)
    kw = dict(lookahead=bands, step_blocks=blocks, lead=lead)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, algo="blocked", **kw)
    Ug, Lg = host(U), host(L)
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed_directed(P, **kw)
    Pg = host(P)
    assert within_bound(Ug, Lg, Ue, Le, L0)
    assert np.all(Lg <= Ug)
    if bands == 2:
        # two steps ahead the dense layout builds its panels as the closure of
        # the diagonal tile and a product, the packed one by the 64-round
        # phase 1-2 launch: another grouping of the roundings, in the bound
        Up, Lp = steps.unpack(Pg)
        assert within_bound(Up, Lp, Ue, Le, L0)
        assert np.all(Lp <= Up)
    else:
        # the packed layout runs the same kernels in the same order
        assert bits_equal(Pg, steps.pack(Ug, Lg))


@pytest.mark.parametrize("lead", [None, True])
@pytest.mark.parametrize("n", [300, 700])
def test_directed_blocked_sound_on_line(n, lead):
    U0, L0, X = gen.unquantised_line(n, seed=n)
    d = gen.true_distances(X)
    Ue, Le = oracle.smooth_directed(U0, L0)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, algo="blocked", lead=lead)
    Ug, Lg = host(U), host(L)
    assert np.all(Ug.astype(np.float64) >= d) and np.all(Lg.astype(np.float64) <= d)
    assert np.all(Lg <= Ug)
    assert within_bound(Ug, Lg, Ue, Le, L0)
    # the plain pass is not sound on this input: the directed one is needed
    Un, Ln = dev(U0), dev(L0)
    dgb.smooth(Un, Ln, algo="blocked")
    assert np.any(host(Un).astype(np.float64) < d) or np.any(host(Ln).astype(np.float64) > d)


# ---------------------------------------------------------------- full size
def _n12288_sampled_checks(W, Ug, Lg, tag):
    """Four shortest-path rows against a textbook Dijkstra, L at every pair of
    those atoms against the closed form, symmetry, L <= U and soundness."""
    import pins
    rng = np.random.default_rng(12288)
    src = sorted(rng.choice(W.n, size=4, replace=False).tolist())
    D = pins.sssp_dense(W.U[0], src)
    for a, s in enumerate(src):
        assert np.array_equal(Ug[s].astype(np.float64), D[a]), f"{tag}: U row {s}"
    for a in range(len(src)):
        for b in range(a, len(src)):
            want = pins.lower_pair(W.L[0], D[a], D[b])
            assert float(Lg[src[a], src[b]]) == want, (tag, src[a], src[b])
    assert np.array_equal(Ug.view(np.uint32), Ug.T.view(np.uint32))
    assert np.array_equal(Lg.view(np.uint32), Lg.T.view(np.uint32))
    assert np.all(Lg <= Ug) and pins.sound(Ug, Lg, W.X[0])


def test_directed_n12288_on_grid_sampled():
    # the n12288 workload is on the 2^-6 grid, so the directed pass must reach
    # the exact result, checked at sampled rows and pairs
    W = gen.make_workload("n12288")
    U, L = dev(W.U[0]), dev(W.L[0])
    dgb.smooth_directed(U, L)
    _n12288_sampled_checks(W, host(U), host(L), "directed n12288")


def test_packed_n12288_sampled():
    W = gen.make_workload("n12288")
    P = dgb.pack(dev(W.U[0]), dev(W.L[0]))
    dgb.smooth_packed(P)
    U, L = dgb.unpack(P)
    _n12288_sampled_checks(W, host(U), host(L), "packed n12288")
