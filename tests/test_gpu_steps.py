"""Bit-exact parity of the steps around a pass with the CPU oracle (needs an
MI355X): restraint lists to dense bounds, partial passes over a range of
rounds (every algorithm), and the tightened-cell mask."""
import numpy as np
import pytest
import torch

import distance_geometry_bound_amd as dgb
import oracle
from distance_geometry_bound_amd import gen
from oracle import steps

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def dev(A):
    return torch.from_numpy(np.ascontiguousarray(A)).to(DEV)


def host(T):
    torch.cuda.synchronize(DEV)
    return T.cpu().numpy()


def bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint32),
                          np.ascontiguousarray(b).view(np.uint32))


def random_restraints(n, batch, m, seed, bad=True):
    rng = np.random.default_rng(seed)
    mol = rng.integers(0, batch, m).astype(np.int32)
    ia = rng.integers(0, n, m).astype(np.int32)
    ja = rng.integers(0, n, m).astype(np.int32)
    lo = rng.uniform(-1.0, 20.0, m).astype(np.float32)
    hi = (lo + rng.uniform(0.0, 15.0, m)).astype(np.float32)
    if bad and m >= 6:                        # a few invalid entries of each kind
        k = rng.choice(m, 6, replace=False)
        ia[k[0]] = n
        mol[k[1]] = batch
        lo[k[2]] = np.nan
        hi[k[3]] = lo[k[3]] - 1.0
        hi[k[4]] = np.inf
        ja[k[5]] = -1
    return mol, ia, ja, lo, hi


# ---------------------------------------------------------------- restraints
@pytest.mark.parametrize("n,batch,m", [(1, 1, 3), (7, 3, 50), (100, 3, 4000), (257, 2, 20000),
                                       (260, 1, 5000)])
def test_restraints_match_oracle(n, batch, m):
    mol, ia, ja, lo, hi = random_restraints(n, batch, m, seed=n + m)
    Ue, Le, ste = steps.bounds_from_restraints(n, batch, 0.25, 40.0, ia, ja, lo, hi, mol=mol)
    U, L, st = dgb.bounds_from_restraints(n, dev(ia), dev(ja), dev(lo), dev(hi), 0.25, 40.0,
                                          mol=dev(mol), batch=batch)
    assert bits_equal(host(U), Ue) and bits_equal(host(L), Le)
    assert st == ste


def test_restraints_empty_list_and_misaligned_output():
    n = 12
    empty_i = torch.zeros(0, dtype=torch.int32, device=DEV)
    empty_f = torch.zeros(0, dtype=torch.float32, device=DEV)
    bu = torch.zeros(n * n + 1, device=DEV)
    bl = torch.zeros(n * n + 1, device=DEV)
    out = (bu[1:].view(1, n, n), bl[1:].view(1, n, n))
    U, L, st = dgb.bounds_from_restraints(n, empty_i, empty_i, empty_f, empty_f, 1.0, 9.0,
                                          out=out)
    Ue, Le, _ = steps.bounds_from_restraints(n, 1, 1.0, 9.0, [], [], [], [])
    assert st == 0 and bits_equal(host(U), Ue) and bits_equal(host(L), Le)


@pytest.mark.parametrize("name,batch", [("n1024", None), ("b64n500", 8), ("n12288", None)])
def test_restraints_workloads(name, batch):
    mol, ia, ja, lo, hi, ul, uu, n, nb = gen.workload_restraints(name, batch=batch)
    Ue, Le, ste = steps.bounds_from_restraints(n, nb, ul, uu, ia, ja, lo, hi, mol=mol)
    U, L, st = dgb.bounds_from_restraints(n, dev(ia), dev(ja), dev(lo), dev(hi), ul, uu,
                                          mol=dev(mol), batch=nb)
    assert st == ste == 0
    assert bits_equal(host(U), Ue) and bits_equal(host(L), Le)


def test_restraints_then_smooth():
    mol, ia, ja, lo, hi, ul, uu, n, nb = gen.workload_restraints("b64n500", batch=3)
    Ue, Le, _ = steps.bounds_from_restraints(n, nb, ul, uu, ia, ja, lo, hi, mol=mol)
    Ue, Le = oracle.smooth(Ue, Le)
    U, L, _ = dgb.bounds_from_restraints(n, dev(ia), dev(ja), dev(lo), dev(hi), ul, uu,
                                         mol=dev(mol), batch=nb)
    dgb.smooth(U, L)
    assert bits_equal(host(U), Ue) and bits_equal(host(L), Le)


# ---------------------------------------------------------------- ranges
def sound(n, batch, seed):
    U0, L0, _ = gen.random_sound_bounds(n, seed=seed, batch=batch, box=6.0 + n / 8)
    return U0, L0


@pytest.mark.parametrize("n,cuts,algo", [
    (300, [0, 64, 192, 256, 300], "blocked"),
    (300, [0, 64, 192, 256, 300], "auto"),
    (257, [0, 128, 257], "auto"),
    (300, [0, 1, 63, 64, 100, 300], "auto"),      # unaligned ends take the per-round path
    (300, [0, 37, 300], "perk"),
    (150, [0, 1, 50, 149, 150], "lds"),
    (150, [0, 64, 150], "blocked"),
])
def test_range_pieces_match_oracle(n, cuts, algo):
    U0, L0 = sound(n, 2, seed=n + len(cuts))
    U, L = dev(U0), dev(L0)
    Ue, Le = U0, L0
    for a, b in zip(cuts[:-1], cuts[1:]):
        dgb.smooth_range(U, L, a, b, algo=algo)
        Ue, Le = oracle.rounds(Ue, Le, a, b)
        assert bits_equal(host(U), Ue) and bits_equal(host(L), Le), (algo, a, b)


def test_range_rejects_unaligned_blocked():
    U0, L0 = sound(300, 1, seed=1)
    U, L = dev(U0), dev(L0)
    with pytest.raises(ValueError):
        dgb.smooth_range(U, L, 10, 64, algo="blocked")
    with pytest.raises(ValueError):
        dgb.smooth_range(U, L, 0, 301)
    U, L = dev(U0[0]), dev(L0[0])
    with pytest.raises(ValueError):
        dgb.smooth_range(U, L, 0, 64, algo="lds")


# ---------------------------------------------------------------- mask
@pytest.mark.parametrize("n,batch", [(5, 1), (130, 3), (1001, 1)])
def test_tightened_matches_oracle(n, batch):
    U0, L0 = sound(n, batch, seed=n)
    U1, L1 = oracle.rounds(U0, L0, 0, min(n, 3))
    m = dgb.tightened(dev(U0), dev(L0), dev(U1), dev(L1))
    assert np.array_equal(host(m), steps.tightened(U0, L0, U1, L1))


# ---------------------------------------------------------------- packed storage
@pytest.mark.parametrize("n,batch", [(1, 1), (2, 2), (5, 1), (63, 1), (64, 2), (65, 1),
                                     (130, 3), (257, 1), (260, 1)])
def test_pack_unpack_match_oracle(n, batch):
    U0, L0 = sound(n, batch, seed=3 * n)
    P = dgb.pack(dev(U0), dev(L0))
    assert bits_equal(host(P), steps.pack(U0, L0))
    U, L = dgb.unpack(P)
    assert bits_equal(host(U), U0) and bits_equal(host(L), L0)


@pytest.mark.parametrize("n,batch", [(3, 1), (7, 2), (64, 1), (65, 2), (129, 1), (130, 3)])
def test_packed_each_round_matches_oracle(n, batch):
    U0, L0 = sound(n, batch, seed=5 * n)
    P = dgb.pack(dev(U0), dev(L0))
    Ue, Le = U0, L0
    for k in range(n):
        dgb.smooth_packed(P, k, k + 1)
        Ue, Le = oracle.rounds(Ue, Le, k, k + 1)
        assert bits_equal(host(P), steps.pack(Ue, Le)), (n, batch, k)


@pytest.mark.parametrize("name,batch", [("n128", None), ("n1024", None), ("b64n500", 4)])
def test_packed_full_pass_workloads(name, batch):
    W = gen.make_workload(name, batch=batch)
    Ue, Le = oracle.smooth(W.U, W.L)
    P = dgb.pack(dev(W.U), dev(W.L))
    dgb.smooth_packed(P)
    assert bits_equal(host(P), steps.pack(Ue, Le))
    U, L = dgb.unpack(P)
    assert bits_equal(host(U), Ue) and bits_equal(host(L), Le)


def test_packed_misaligned_and_ragged():
    n = 260
    U0, L0, _ = gen.random_sound_bounds(n, seed=8, box=40.0)
    Ue, Le = oracle.smooth(U0, L0)
    buf = torch.zeros(n * n + 1, device=DEV)
    P = buf[1:].view(n, n)
    dgb.pack(dev(U0), dev(L0), out=P)
    assert P.data_ptr() % 16 != 0
    dgb.smooth_packed(P)
    assert bits_equal(host(P), steps.pack(Ue, Le))


@pytest.mark.parametrize("n,batch", [(177, 1), (191, 2), (192, 1), (193, 1), (255, 1),
                                     (257, 2), (320, 1), (383, 1), (385, 1), (700, 1)])
def test_packed_blocked_full_pass(n, batch):
    U0, L0 = sound(n, batch, seed=7 * n)
    Ue, Le = oracle.smooth(U0, L0)
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed(P)
    assert bits_equal(host(P), steps.pack(Ue, Le))


def test_packed_ranges_mix_per_round_and_blocked():
    n = 257
    U0, L0 = sound(n, 2, seed=11)
    P = dgb.pack(dev(U0), dev(L0))
    Ue, Le = U0, L0
    for a, b in ((0, 1), (1, 64), (64, 128), (128, 200), (200, 257)):
        dgb.smooth_packed(P, a, b)
        Ue, Le = oracle.rounds(Ue, Le, a, b)
        assert bits_equal(host(P), steps.pack(Ue, Le)), (a, b)


@pytest.mark.parametrize("n,batch,slots", [
    (1, 1, [((0, 0), 1.0)]),
    (5, 2, []),
    (5, 2, [((1, 3, 1), -1.0)]),
    (63, 1, [((62, 0), 99.0)]),
    (64, 1, [((0, 63), np.nan)]),
    (65, 3, [((2, 64, 64), 1.0), ((1, 10, 64), 0.001)]),
    (130, 2, [((1, 129, 3), 2.0 ** 17), ((0, 3, 129), -0.0)]),
    (200, 1, [((150, 140), 1e9), ((140, 150), np.inf)]),
])
def test_check_packed_matches_definitions(n, batch, slots):
    from oracle import check as check_defs
    U0, L0 = sound(n, batch, seed=n)
    P = steps.pack(U0, L0)
    for s, v in slots:
        P[s if batch > 1 or len(s) == 3 else (0,) + s] = v
    assert dgb.check_packed(dev(P)) == check_defs.flags_packed(P)
