"""Bit-exact parity of every HIP path with the CPU oracle (needs an MI355X).

Inputs are on the 2^-6 grid, so every candidate is exact in fp32 and the
tolerance is zero: results are compared as raw 32-bit patterns.  Sizes span
several tiles and ragged tails (n mod 4, n mod 64, n mod 128), batches, and
the five benchmark workloads.  At n = 12288, where the oracle needs many
minutes, the blocked pass (as the benchmark runs it) is checked on sampled
outputs from the closed form (shortest-path rows and lower-bound pairs) and
on properties that hold at any size; the per-round kernel is compared with
the oracle over a prefix of rounds on the full matrix.
"""
import functools

import numpy as np
import pytest
import torch

import distance_geometry_bound_amd as dgb
import oracle
import pins
from distance_geometry_bound_amd import gen
from oracle import check as check_defs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def dev(A):
    return torch.from_numpy(np.ascontiguousarray(A)).to(DEV)


def host(T):
    torch.cuda.synchronize(DEV)
    return T.cpu().numpy()


def assert_bits(Ug, Lg, Ue, Le, tag):
    du = np.flatnonzero(Ug.view(np.uint32).ravel() != Ue.view(np.uint32).ravel())
    dl = np.flatnonzero(Lg.view(np.uint32).ravel() != Le.view(np.uint32).ravel())
    if du.size or dl.size:
        first = du[0] if du.size else dl[0]
        raise AssertionError(f"{tag}: {du.size} U and {dl.size} L entries differ "
                             f"(first flat index {first}: gpu U {Ug.ravel()[first]} "
                             f"L {Lg.ravel()[first]}, oracle U {Ue.ravel()[first]} "
                             f"L {Le.ravel()[first]})")


def gpu_pass(U0, L0, algo, **kw):
    U, L = dev(U0), dev(L0)
    dgb.smooth(U, L, algo=algo, **kw)
    return host(U), host(L)


def sound_input(n, batch, seed):
    U0, L0, _ = gen.random_sound_bounds(n, seed=seed, batch=batch, box=6.0 + n / 8)
    return U0, L0


TAIL_N = [1, 2, 3, 4, 5, 7, 8, 13, 31, 63, 64, 65, 127, 128, 129, 176, 177, 191, 192, 193,
          255, 257, 320]


# -------------------------------------------------------------- per round
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 13, 31, 63, 64, 65, 127, 128, 129, 257])
@pytest.mark.parametrize("batch", [1, 3])
def test_each_round_matches_oracle(n, batch):
    """After every round k the in-place per-round kernel equals the oracle's
    front/back-buffer round, cell by cell."""
    U0, L0 = sound_input(n, batch, seed=10 * n + batch)
    U, L = dev(U0), dev(L0)
    Ue, Le = U0, L0
    for k in range(n):
        dgb.smooth_round(U, L, k)
        Ue, Le = oracle.rounds(Ue, Le, k, k + 1)
        assert_bits(host(U), host(L), Ue, Le, f"n={n} batch={batch} round {k}")


@pytest.mark.parametrize("n", [500, 501, 502, 503])
def test_rounds_ragged_n(n):
    U0, L0 = sound_input(n, 2, seed=n)
    U, L = dev(U0), dev(L0)
    Ue, Le = U0, L0
    for a, b in ((0, 1), (1, 2), (2, 7), (7, 250), (250, 251), (251, n)):
        dgb.smooth_rounds(U, L, a, b)
        Ue, Le = oracle.rounds(Ue, Le, a, b)
        assert_bits(host(U), host(L), Ue, Le, f"n={n} rounds {a}..{b}")


# -------------------------------------------------------------- full pass
@pytest.mark.parametrize("n", TAIL_N)
@pytest.mark.parametrize("batch", [1, 3])
def test_full_pass_every_algorithm(n, batch):
    U0, L0 = sound_input(n, batch, seed=1000 + 7 * n + batch)
    Ue, Le = oracle.smooth(U0, L0)
    algos = ["auto", "blocked", "perk"] + (["lds"] if n <= dgb.lib().dbs_lds_max_n() else [])
    for algo in algos:
        Ug, Lg = gpu_pass(U0, L0, algo)
        assert_bits(Ug, Lg, Ue, Le, f"{algo} n={n} batch={batch}")


@pytest.mark.parametrize("n", [383, 384, 385, 640, 700])
def test_full_pass_multi_tile(n):
    U0, L0 = sound_input(n, 1, seed=n)
    Ue, Le = oracle.smooth(U0, L0)
    for algo in ("blocked", "perk"):
        Ug, Lg = gpu_pass(U0, L0, algo)
        assert_bits(Ug, Lg, Ue, Le, f"{algo} n={n}")


@pytest.mark.parametrize("bands", [0, 1, 2])
@pytest.mark.parametrize("n,batch", [(129, 2), (300, 1), (385, 2), (700, 1)])
def test_every_lookahead_depth(n, batch, bands):
    # the automatic choice runs these sizes without a second stream; forcing
    # each depth covers the one- and two-step schedules (steps of one and of
    # two k-blocks) at small sizes, on the dense, directed and packed passes
    # and on ranges of whole k-blocks
    from oracle import steps
    U0, L0 = sound_input(n, batch, seed=31 * n + bands)
    Ue, Le = oracle.smooth(U0, L0)
    assert dgb.schedule(n, batch, lookahead=bands)[0] == bands
    kw = dict(algo="blocked", lookahead=bands)
    Ug, Lg = gpu_pass(U0, L0, **kw)
    assert_bits(Ug, Lg, Ue, Le, f"blocked n={n} batch={batch} bands={bands}")
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, **kw)
    assert_bits(host(U), host(L), Ue, Le, f"directed n={n} bands={bands}")
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed(P, **kw)
    assert np.array_equal(host(P).view(np.uint32), steps.pack(Ue, Le).view(np.uint32))
    U, L = dev(U0), dev(L0)
    Ur, Lr = oracle.rounds(U0, L0, 0, 128)
    dgb.smooth_range(U, L, 0, 128, **kw)
    assert_bits(host(U), host(L), Ur, Lr, f"range 0..128 n={n} bands={bands}")
    dgb.smooth_range(U, L, 128, n, **kw)
    assert_bits(host(U), host(L), Ue, Le, f"range 128..n n={n} bands={bands}")
    # ranges that start at an odd k-block (two steps ahead pairs the blocks
    # from the range's first one, so the pairs fall differently)
    U, L = dev(U0), dev(L0)
    cuts = sorted({0, 64, min(n, 320), n})
    for a, b in zip(cuts[:-1], cuts[1:]):
        dgb.smooth_range(U, L, a, b, **kw)
    assert_bits(host(U), host(L), Ue, Le, f"ranges 0,64,320,n n={n} bands={bands}")


@pytest.mark.parametrize("blocks", [1, 2, 3, 4])
@pytest.mark.parametrize("bands", [0, 1, 2])
@pytest.mark.parametrize("n,batch", [(385, 2), (700, 1)])
def test_every_step_width(n, batch, bands, blocks):
    # steps of 1..4 k-blocks (the pass picks 1 or 2) at every look-ahead
    # depth, on the dense, directed and packed passes and on ranges that
    # start inside a step
    from oracle import steps
    U0, L0 = sound_input(n, batch, seed=97 * n + 7 * bands + blocks)
    Ue, Le = oracle.smooth(U0, L0)
    assert dgb.schedule(n, batch, lookahead=bands, step_blocks=blocks)[1] == blocks
    kw = dict(algo="blocked", lookahead=bands, step_blocks=blocks)
    tag = f"n={n} batch={batch} bands={bands} blocks={blocks}"
    Ug, Lg = gpu_pass(U0, L0, **kw)
    assert_bits(Ug, Lg, Ue, Le, "blocked " + tag)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, **kw)
    assert_bits(host(U), host(L), Ue, Le, "directed " + tag)
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed(P, **kw)
    assert np.array_equal(host(P).view(np.uint32), steps.pack(Ue, Le).view(np.uint32)), tag
    U, L = dev(U0), dev(L0)
    for a, b in ((0, 192), (192, n)):
        dgb.smooth_range(U, L, a, b, **kw)
    assert_bits(host(U), host(L), Ue, Le, "ranges 0,192,n " + tag)


@pytest.mark.parametrize("lead", [None, False])
@pytest.mark.parametrize("n,batch", [(130, 129), (200, 87), (257, 86)])
def test_split_batch(n, batch, lead):
    # more than 256 phase 1-2 workgroups: automatically the lead schedule on
    # one stream; without it (lead=False) the batch splits into two unequal
    # halves (batch // 2 and the rest), one per stream.  Dense, directed and
    # packed passes, and ranges that cut the pass at k-block boundaries
    from oracle import steps
    assert (-(-n // 64) - 1) * batch > 256 and dgb.lookahead_bands(n, batch) == 0
    assert dgb.schedule(n, batch, lead=lead)[2] == (0 if lead is False else 1)
    U0, L0 = sound_input(n, batch, seed=11 * n + batch)
    Ue, Le = oracle.smooth(U0, L0)
    tag = f"n={n} batch={batch} lead={lead}"
    kw = dict(algo="blocked", lead=lead)
    Ug, Lg = gpu_pass(U0, L0, **kw)
    assert_bits(Ug, Lg, Ue, Le, "blocked " + tag)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, **kw)
    assert_bits(host(U), host(L), Ue, Le, "directed " + tag)
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed(P, **kw)
    assert np.array_equal(host(P).view(np.uint32), steps.pack(Ue, Le).view(np.uint32)), tag
    U, L = dev(U0), dev(L0)
    Ur, Lr = oracle.rounds(U0, L0, 0, 64)
    dgb.smooth_range(U, L, 0, 64, **kw)
    assert_bits(host(U), host(L), Ur, Lr, "range 0..64 " + tag)
    dgb.smooth_range(U, L, 64, n, **kw)
    assert_bits(host(U), host(L), Ue, Le, "range 64..n " + tag)


@pytest.mark.parametrize("n", [65, 127, 128, 129, 191, 192, 257, 300, 385, 503, 700])
@pytest.mark.parametrize("batch", [1, 3])
def test_lead_schedule(n, batch):
    # the lead schedule forced on (phase 2 as a product with the closed
    # diagonal tile; phase 3 of each k-block beside phase 1 of the next, in
    # one launch) at sizes with ragged last k-blocks and tiles: dense,
    # directed and packed passes, and ranges that start inside the pass
    from oracle import steps
    assert dgb.schedule(n, batch, lead=True) == (0, 1, 1)
    U0, L0 = sound_input(n, batch, seed=17 * n + batch)
    Ue, Le = oracle.smooth(U0, L0)
    kw = dict(algo="blocked", lead=True)
    tag = f"lead n={n} batch={batch}"
    Ug, Lg = gpu_pass(U0, L0, **kw)
    assert_bits(Ug, Lg, Ue, Le, "blocked " + tag)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, **kw)
    assert_bits(host(U), host(L), Ue, Le, "directed " + tag)
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed(P, **kw)
    assert np.array_equal(host(P).view(np.uint32), steps.pack(Ue, Le).view(np.uint32)), tag
    U, L = dev(U0), dev(L0)
    cuts = sorted({0, 64, min(n, 192), n})
    for a, b in zip(cuts[:-1], cuts[1:]):
        dgb.smooth_range(U, L, a, b, **kw)
        Ur, Lr = oracle.rounds(U0, L0, 0, b)
        assert_bits(host(U), host(L), Ur, Lr, f"range 0..{b} " + tag)
    P = dgb.pack(dev(U0), dev(L0))
    for a, b in zip(cuts[:-1], cuts[1:]):
        dgb.smooth_packed(P, a, b, **kw)
    assert np.array_equal(host(P).view(np.uint32), steps.pack(Ue, Le).view(np.uint32)), tag


@pytest.mark.parametrize("n,batch", [(2048, 1), (700, 12), (1500, 2), (130, 128), (1536, 1),
                                     (500, 8), (300, 16), (300, 100), (700, 40)])
def test_automatic_lead_window(n, batch):
    # from 64 phase-3 tiles (times molecules) the automatic schedule of a
    # dense blocked pass is the lead one, up to 512 tiles for one molecule
    # and 1024 for a batch, whether or not the phase 1-2 launch would fill
    # the chip; the packed layout takes it from 256 to 512 tiles, or where
    # that launch fills the chip: dense, directed and packed blocked passes
    # against the oracle
    from oracle import steps
    assert dgb.schedule(n, batch) == (0, 1, 1)
    T = -(-n // 128)
    tiles = T * (T + 1) // 2 * batch
    assert dgb.schedule(n, batch, packed=True)[2] == (1 if 256 <= tiles < 512 or
                                                      (-(-n // 64) - 1) * batch > 256 else 0)
    U0, L0 = sound_input(n, batch, seed=5 * n + batch)
    Ue, Le = oracle.smooth(U0, L0)
    tag = f"automatic n={n} batch={batch}"
    Ug, Lg = gpu_pass(U0, L0, "blocked")
    assert_bits(Ug, Lg, Ue, Le, "dense " + tag)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, algo="blocked")
    assert_bits(host(U), host(L), Ue, Le, "directed " + tag)
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed(P, algo="blocked")
    assert np.array_equal(host(P).view(np.uint32), steps.pack(Ue, Le).view(np.uint32)), tag


@pytest.mark.parametrize("n,batch,width", [(300, 171, 1), (500, 103, 1), (300, 300, 2)])
def test_automatic_two_ahead_for_batches(n, batch, width):
    # a dense batch from 1024 phase-3 tiles runs two steps ahead in steps of
    # one k-block, from 1600 tiles of two: dense, directed and packed passes
    # (the packed layout keeps its own widths) against the oracle
    from oracle import steps
    assert dgb.schedule(n, batch) == (2, width, 0)
    assert dgb.schedule(n, batch, packed=True)[0] == 2
    U0, L0 = sound_input(n, batch, seed=13 * n + batch)
    Ue, Le = oracle.smooth(U0, L0)
    tag = f"two ahead n={n} batch={batch}"
    Ug, Lg = gpu_pass(U0, L0, "blocked")
    assert_bits(Ug, Lg, Ue, Le, "dense " + tag)
    U, L = dev(U0), dev(L0)
    dgb.smooth_directed(U, L, algo="blocked")
    assert_bits(host(U), host(L), Ue, Le, "directed " + tag)
    P = dgb.pack(dev(U0), dev(L0))
    dgb.smooth_packed(P, algo="blocked")
    assert np.array_equal(host(P).view(np.uint32), steps.pack(Ue, Le).view(np.uint32)), tag


def test_walk_molecules_batched():
    W = gen.make_workload("b64n500", batch=5)
    Ue, Le = oracle.smooth(W.U, W.L)
    Ug, Lg = gpu_pass(W.U, W.L, "auto")
    assert_bits(Ug, Lg, Ue, Le, "auto b5n500")


@functools.lru_cache(maxsize=1)
def workload_expected(name):
    W = gen.make_workload(name)
    Ue, Le = oracle.smooth(W.U, W.L)
    return W, Ue, Le


@pytest.mark.parametrize("name,algo", [(w, a) for w in ("n128", "n1024", "b64n500", "n4096")
                                       for a in ("auto", "perk")])
def test_workloads(name, algo):
    W, Ue, Le = workload_expected(name)
    print(f"{name}: oracle done", flush=True)
    Ug, Lg = gpu_pass(W.U, W.L, algo)
    assert_bits(Ug, Lg, Ue, Le, f"{algo} {name}")
    assert check_defs.flags(Ug, Lg) == 0


# -------------------------------------------------------------- n = 12288
@functools.lru_cache(maxsize=1)
def big():
    W = gen.make_workload("n12288")
    U, L = dev(W.U[0]), dev(W.L[0])
    dgb.smooth(U, L)                       # the benchmark's path (auto -> blocked)
    return W, U, L


def test_n12288_perk_prefix_matches_oracle():
    W = gen.make_workload("n12288")
    R = 6
    Ue, Le = oracle.rounds(W.U[0], W.L[0], 0, R)
    U, L = dev(W.U[0]), dev(W.L[0])
    dgb.smooth_rounds(U, L, 0, R)
    assert_bits(host(U), host(L), Ue, Le, f"perk n12288 rounds 0..{R}")


def test_n12288_closed_form_samples():
    W, U, L = big()
    Ug, Lg = host(U), host(L)
    rng = np.random.default_rng(12288)
    src = sorted(rng.choice(W.n, size=4, replace=False).tolist())
    D = pins.sssp_dense(W.U[0], src)
    print("n12288: shortest-path rows done", flush=True)
    for a, s in enumerate(src):
        assert np.array_equal(Ug[s].astype(np.float64), D[a]), f"U row {s}"
    for a in range(len(src)):
        for b in range(a, len(src)):
            want = pins.lower_pair(W.L[0], D[a], D[b])
            assert float(Lg[src[a], src[b]]) == want, (src[a], src[b])
            assert float(Lg[src[b], src[a]]) == want, (src[b], src[a])


def test_n12288_invariants():
    W, U, L = big()
    Ug, Lg = host(U), host(L)
    U0, L0 = W.U[0], W.L[0]
    assert np.array_equal(Ug.view(np.uint32), Ug.T.view(np.uint32))
    assert np.array_equal(Lg.view(np.uint32), Lg.T.view(np.uint32))
    assert np.all(np.diag(Ug).view(np.uint32) == 0) and np.all(np.diag(Lg).view(np.uint32) == 0)
    assert np.all(Ug <= U0) and np.all(Lg >= L0) and np.all(Lg <= Ug)
    assert pins.sound(Ug, Lg, W.X[0])
    print("n12288: global invariants done", flush=True)
    rng = np.random.default_rng(5)
    u, lo = Ug.astype(np.float64), Lg
    for _ in range(20):
        i = rng.integers(0, W.n, 200_000)
        j = rng.integers(0, W.n, 200_000)
        k = rng.integers(0, W.n, 200_000)
        assert np.all(u[i, j] <= u[i, k] + u[k, j])
        assert np.all(lo[i, j] >= lo[i, k].astype(np.float64) - u[k, j])
        assert np.all(lo[i, j] >= lo[k, j].astype(np.float64) - u[i, k])
    # a second pass over a finished result changes nothing
    U2, L2 = U.clone(), L.clone()
    dgb.smooth(U2, L2)
    assert torch.equal(U2.view(torch.int32), U.view(torch.int32))
    assert torch.equal(L2.view(torch.int32), L.view(torch.int32))


def test_n12288_schedule_independent():
    # every schedule of the pass reaches the same bits (exact arithmetic on
    # the grid): the benchmark's schedule (two steps ahead, steps of four
    # k-blocks) against one stream with one-block steps, over the whole
    # matrix, and the packed pass against the packed form of that result
    W, U, L = big()
    assert dgb.lookahead_bands(W.n) == 2 and dgb.step_blocks(W.n) == 4
    U1, L1 = dev(W.U[0]), dev(W.L[0])
    dgb.smooth(U1, L1, algo="blocked", lookahead=0, step_blocks=1)
    torch.cuda.synchronize(DEV)
    assert torch.equal(U1.view(torch.int32), U.view(torch.int32))
    assert torch.equal(L1.view(torch.int32), L.view(torch.int32))
    del U1, L1
    P = dgb.pack(dev(W.U[0]), dev(W.L[0]))
    dgb.smooth_packed(P)
    assert torch.equal(P.view(torch.int32), dgb.pack(U, L).view(torch.int32))


# -------------------------------------------------------------- contract
def test_deterministic_and_side_stream():
    U0, L0 = sound_input(1000, 1, seed=77)
    Ue, Le = oracle.smooth(U0, L0)
    s = torch.cuda.Stream(DEV)
    with torch.cuda.stream(s):
        U, L = dev(U0), dev(L0)
        dgb.smooth(U, L, algo="blocked")
    s.synchronize()
    assert_bits(U.cpu().numpy(), L.cpu().numpy(), Ue, Le, "side stream")
    Ug, Lg = gpu_pass(U0, L0, "blocked")
    assert_bits(Ug, Lg, Ue, Le, "repeat")


def test_unaligned_rows_take_the_scalar_path():
    n = 260                                   # n % 4 == 0, base misaligned by 4 bytes
    U0, L0, _ = gen.random_sound_bounds(n, seed=9, box=40.0)
    Ue, Le = oracle.smooth(U0, L0)
    for algo in ("blocked", "perk"):
        bu = torch.zeros(n * n + 1, device=DEV)
        bl = torch.zeros(n * n + 1, device=DEV)
        U = bu[1:].view(n, n)
        L = bl[1:].view(n, n)
        U.copy_(dev(U0))
        L.copy_(dev(L0))
        assert U.data_ptr() % 16 != 0
        dgb.smooth(U, L, algo=algo)
        assert_bits(host(U), host(L), Ue, Le, f"{algo} misaligned")


def test_inconsistent_bounds_upper_exact_and_flagged():
    U0, L0 = gen.random_bounds(150, seed=3, batch=2, umax_units=200)
    Ue, _ = oracle.smooth(U0, L0)
    for algo in ("blocked", "lds", "perk"):
        U, L = dev(U0), dev(L0)
        dgb.smooth(U, L, algo=algo)
        Ug = host(U)
        assert np.array_equal(Ug.view(np.uint32), Ue.view(np.uint32)), algo
        assert dgb.check(U, L) & dgb.CHECK_FLAGS["l_gt_u"]


@pytest.mark.parametrize("case", ["clean", "asym", "diag", "nan", "inf", "lgtu", "lneg",
                                  "unq", "range", "negzero"])
def test_check_matches_definitions(case):
    U, L, _ = gen.random_sound_bounds(37, seed=5, batch=2)
    U, L = U.copy(), L.copy()
    if case == "asym":
        U[1, 1, 2] += 1.0
    elif case == "diag":
        L[0, 3, 3] = 1.0
    elif case == "nan":
        U[1, 4, 2] = U[1, 2, 4] = np.nan
    elif case == "inf":
        L[0, 4, 2] = L[0, 2, 4] = np.inf
    elif case == "lgtu":
        L[1, 5, 6] = L[1, 6, 5] = U[1, 5, 6] + 1.0
    elif case == "lneg":
        L[0, 5, 6] = L[0, 6, 5] = -1.0
    elif case == "unq":
        U[0, 7, 8] = U[0, 8, 7] = U[0, 7, 8] + 0.001
    elif case == "range":
        U[1, 7, 8] = U[1, 8, 7] = 2.0 ** 17
    elif case == "negzero":
        L[0, 7, 8] = L[0, 8, 7] = -0.0
    assert dgb.check(dev(U), dev(L)) == check_defs.flags(U, L)


def test_empty_and_trivial_shapes():
    for n in (0, 1):
        U = torch.zeros(2, n, n, device=DEV)
        L = torch.zeros(2, n, n, device=DEV)
        dgb.smooth(U, L)
        torch.cuda.synchronize(DEV)
    with pytest.raises(ValueError):
        dgb.smooth(torch.zeros(4, 5, device=DEV), torch.zeros(4, 5, device=DEV))
    U = torch.zeros(8, 8, device=DEV)
    with pytest.raises(ValueError):
        dgb.smooth(U, U)                       # U and L overlap


def test_single_round_entry_and_smooth_check_option():
    U0, L0, _ = gen.random_sound_bounds(70, seed=70, batch=2)
    U, L = dev(U0), dev(L0)
    Ue, Le = U0, L0
    for k in (0, 1, 69):
        dgb.smooth_round(U, L, k)
        Ue, Le = oracle.rounds(Ue, Le, k, k + 1)
        assert_bits(host(U), host(L), Ue, Le, f"round {k}")
    with pytest.raises(ValueError):
        dgb.smooth_round(U, L, 70)
    U, L = dev(U0), dev(L0)
    dgb.smooth(U, L, check=True)
    assert_bits(host(U), host(L), *oracle.smooth(U0, L0), "checked pass")
    Ub = U0.copy()
    Ub[0, 1, 2] = Ub[0, 2, 1] = Ub[0, 1, 2] + 0.001   # off the grid
    with pytest.raises(ValueError, match="unquant"):
        dgb.smooth(dev(Ub), dev(L0), check=True)


# -------------------------------------------------------------- caller streams
def _expected_pair(n, batch, seed):
    U0, L0 = sound_input(n, batch, seed=seed)
    return U0, L0, *oracle.smooth(U0, L0)


@pytest.mark.parametrize("kw", [dict(lookahead=2, step_blocks=2), dict(lookahead=1),
                                dict()])
def test_passes_on_two_caller_streams(kw):
    # two passes in flight at once on two caller streams, each with the
    # library's second stream of its own (forced look-ahead at these sizes;
    # the last case is (130, 129), a batch split over the two streams)
    cases = [(700, 1, 71), (385, 2, 72)] if kw else [(130, 129, 73), (200, 87, 74)]
    data = [_expected_pair(*c) for c in cases]
    streams = [torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)]
    out = []
    for (U0, L0, _, _), s in zip(data, streams):
        s.wait_stream(torch.cuda.current_stream(DEV))
        with torch.cuda.stream(s):
            U, L = dev(U0), dev(L0)
            for _ in range(2):                 # the second pass changes nothing
                dgb.smooth(U, L, algo="blocked", **kw)
        out.append((U, L))
    for (U, L), (_, _, Ue, Le), c in zip(out, data, cases):
        assert_bits(host(U), host(L), Ue, Le, f"stream pass {c} {kw}")


def test_passes_from_two_host_threads():
    # host threads enqueue passes concurrently, each on its own stream, and
    # also both on one shared stream (the library serialises the enqueue of
    # the passes that share its second stream)
    import threading
    cases = [(700, 1, 81), (640, 1, 82), (385, 2, 83), (520, 1, 84)]
    data = [_expected_pair(*c) for c in cases]
    shared = torch.cuda.Stream(DEV)
    own = [torch.cuda.Stream(DEV) for _ in cases]
    results, errors = [None] * len(cases), []

    def work(i):
        try:
            U0, L0, _, _ = data[i]
            s = shared if i % 2 else own[i]
            with torch.cuda.stream(s):
                U, L = dev(U0), dev(L0)
                for _ in range(3):
                    dgb.smooth(U, L, algo="blocked", lookahead=2, step_blocks=1 + i % 3)
                s.synchronize()
                results[i] = (U.cpu().numpy(), L.cpu().numpy())
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (Ug, Lg), (_, _, Ue, Le), c in zip(results, data, cases):
        assert_bits(Ug, Lg, Ue, Le, f"thread pass {c}")
