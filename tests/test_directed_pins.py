"""Pins of the oracle's directed-rounding pass.

Directed rounding rounds every upper-bound sum toward +inf and every
lower-bound difference toward -inf.  The notes on GPU Gems 2, Ch. 43 (§6)
call the smoothing precision-sensitive.  On inputs off the 2^-6 grid,
round-to-nearest can move a bound past the value it stands for.

What fixes the directed result, independently of the oracle's code:
  * hand-derived cases (tests/golden/directed_cases.txt), for both modes;
  * on grid inputs every operation is exact, so both modes give the same bits;
  * the exact closure, computed in rational arithmetic by path enumeration,
    brackets it: U >= U* and L <= L* exactly, and within a bound derived from
    the rounding error (below);
  * soundness with respect to the true distances, on a construction where
    round-to-nearest provably is not sound;
  * planted mistakes (wrong direction, mode not restored, flag ignored) fail.

Derived tolerance.  Write e = 2^-23.  A directed sum of positive terms is at
most (1 + e) times the exact sum, and a path of h <= n - 1 edges is summed
in at most n - 2 levels.  So U <= U* (1 + e)^(n-2).  A lower-bound candidate
is L_kl minus such sums, with at most 2n rounded subtractions, each of which
loses at most e times the magnitude it handles (<= Lmax + 2 Umax*).  So
L >= L* - delta with
    delta = 2 Umax* ((1 + e)^(n-2) - 1) + 2 n e (Lmax + 2 Umax*),
where Umax* is the largest finite U* and Lmax the largest L.
"""
import itertools
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from distance_geometry_bound_amd import gen
from test_oracle_pins import bits_equal

GOLDEN = __file__.replace("test_directed_pins.py", "golden/directed_cases.txt")
EPS = Fraction(1, 2 ** 23)


def _num(tok):
    return float.fromhex(tok) if tok.lstrip("-").startswith("0x") else float(tok)


def read_directed_cases(path=GOLDEN):
    cases, cur, key = {}, None, None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("case "):
            cur, key = {"name": line.split()[1]}, None
        elif line == "end":
            name = cur.pop("name")
            cases[name] = {k: np.array(v, dtype=np.float32) for k, v in cur.items()}
        elif line in ("U0", "L0", "U1", "L1", "UN", "LN"):
            key = line
            cur[key] = []
        else:
            cur[key].append([_num(t) for t in line.split()])
    return cases


CASES = read_directed_cases()


@pytest.mark.parametrize("name", sorted(CASES))
def test_directed_hand_cases(name):
    c = CASES[name]
    U, L = oracle.smooth_directed(c["U0"], c["L0"])
    assert bits_equal(U, c["U1"]) and bits_equal(L, c["L1"])
    U, L = oracle.smooth(c["U0"], c["L0"])
    assert bits_equal(U, c["UN"]) and bits_equal(L, c["LN"])
    # the two modes differ on every case, and only by rounding direction
    assert not (bits_equal(c["U1"], c["UN"]) and bits_equal(c["L1"], c["LN"]))
    assert np.all(c["U1"] >= c["UN"]) and np.all(c["L1"] <= c["LN"])


def test_directed_equals_nearest_on_the_grid():
    U0, L0, _ = gen.random_sound_bounds(60, seed=4, batch=2, box=15.0)
    assert bits_equal(oracle.smooth_directed(U0, L0)[0], oracle.smooth(U0, L0)[0])
    assert bits_equal(oracle.smooth_directed(U0, L0)[1], oracle.smooth(U0, L0)[1])
    W = gen.make_workload("n128")
    Ud, Ld = oracle.smooth_directed(W.U, W.L)
    Un, Ln = oracle.smooth(W.U, W.L)
    assert bits_equal(Ud, Un) and bits_equal(Ld, Ln)


def test_directed_rounds_compose():
    U0, L0, _ = gen.random_unquantised_bounds(40, seed=2, slack=0.0, known=0.5)
    Ua, La = oracle.rounds_directed(U0, L0, 0, 17)
    Ua, La = oracle.rounds_directed(Ua, La, 17, 40)
    Ub, Lb = oracle.smooth_directed(U0, L0)
    assert bits_equal(Ua, Ub) and bits_equal(La, Lb)


# ----------------------------------------------------------------- exact closure
def exact_closure(U, L):
    """U* by enumerating simple paths, L*_ij = max_{k,l} L_kl - U*_ik - U*_lj,
    in exact rational arithmetic (n <= 8)."""
    n = U.shape[0]
    u = [[Fraction(float(U[i, j])) for j in range(n)] for i in range(n)]
    us = [[None] * n for _ in range(n)]
    for i in range(n):
        for j in range(n):
            if i == j:
                us[i][j] = Fraction(0)
                continue
            best = u[i][j]
            others = [m for m in range(n) if m not in (i, j)]
            for r in range(1, len(others) + 1):
                for mid in itertools.permutations(others, r):
                    path = (i,) + mid + (j,)
                    s = sum((u[a][b] for a, b in zip(path, path[1:])), Fraction(0))
                    if s < best:
                        best = s
            us[i][j] = best
    ls = [[max(Fraction(float(L[k, l])) - us[i][k] - us[l][j]
               for k in range(n) for l in range(n)) for j in range(n)] for i in range(n)]
    return us, ls


def bracket(U, L, us, ls, Lin):
    """(exact sides hold, derived tolerance holds) for a result U, L."""
    n = U.shape[0]
    umax = max(x for row in us for x in row)
    lmax = max(Fraction(float(x)) for x in Lin.ravel())
    grow = (1 + EPS) ** max(n - 2, 0)
    delta = 2 * umax * (grow - 1) + 2 * n * EPS * (lmax + 2 * umax)
    exact = tol = True
    for i in range(n):
        for j in range(n):
            u, l = Fraction(float(U[i, j])), Fraction(float(L[i, j]))
            exact &= u >= us[i][j] and l <= ls[i][j]
            tol &= u <= us[i][j] * grow and l >= ls[i][j] - delta
    return exact, tol


def _small_cases():
    out = []
    for seed in range(12):
        n = 5 + seed % 3
        U, L, _ = gen.random_unquantised_bounds(n, seed=seed, box=8.0, known=0.6,
                                                slack=0.0 if seed % 2 else 1.0)
        out.append((U, L))
    for n in (5, 6, 7, 8):
        U, L, _ = gen.unquantised_line(n, seed=n)
        out.append((U, L))
    return out


def test_directed_brackets_the_exact_closure():
    nearest_fails = 0
    for U0, L0 in _small_cases():
        us, ls = exact_closure(U0, L0)
        U, L = oracle.smooth_directed(U0, L0)
        exact, tol = bracket(U, L, us, ls, L0)
        assert exact and tol
        Un, Ln = oracle.smooth(U0, L0)
        nearest_fails += not bracket(Un, Ln, us, ls, L0)[0]
    # the cases are stringent enough that round-to-nearest leaves the bracket
    assert nearest_fails > 0


# ----------------------------------------------------------------- soundness
@pytest.mark.parametrize("n", [50, 200])
def test_directed_is_sound_where_nearest_is_not(n):
    U0, L0, X = gen.unquantised_line(n, seed=n)
    d = gen.true_distances(X)
    U, L = oracle.smooth_directed(U0, L0)
    assert np.all(U.astype(np.float64) >= d) and np.all(L.astype(np.float64) <= d)
    assert np.all(L <= U)
    Un, Ln = oracle.smooth(U0, L0)
    assert np.any(Un.astype(np.float64) < d) and np.any(Ln.astype(np.float64) > d)


def test_directed_is_sound_on_random_molecules():
    U0, L0, Xs = gen.random_unquantised_bounds(90, seed=9, batch=2, slack=0.0, known=0.5)
    U, L = oracle.smooth_directed(U0, L0)
    for b in range(2):
        d = gen.true_distances(Xs[b])
        assert np.all(U[b].astype(np.float64) >= d) and np.all(L[b].astype(np.float64) <= d)


# ----------------------------------------------------------------- planted mistakes
MUTANTS = {
    "upper_rounded_down": ("fesetround(FE_UPWARD);", "fesetround(FE_DOWNWARD);"),
    "lower_rounded_up": ("fesetround(FE_DOWNWARD);", "fesetround(FE_UPWARD);"),
    "lower_to_nearest": ("fesetround(FE_DOWNWARD);", "fesetround(FE_TONEAREST);"),
    "mode_not_restored": ("fesetround(FE_TONEAREST);", ";"),
    "flag_ignored": ("threads, 1);", "threads, 0);"),
}


def _build(src, tmp_path, name):
    import ctypes
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-frounding-math",
                    str(c), "-lm", "-o", str(so)], check=True)
    lib = ctypes.CDLL(str(so))
    f32p = ctypes.POINTER(ctypes.c_float)
    for f in ("dbs_oracle_rounds", "dbs_oracle_rounds_directed"):
        getattr(lib, f).argtypes = [f32p, f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int]
        getattr(lib, f).restype = ctypes.c_int

    def run(fname, U, L):
        U = np.array(U, dtype=np.float32, copy=True)
        L = np.array(L, dtype=np.float32, copy=True)
        n = U.shape[-1]
        b = 1 if U.ndim == 2 else U.shape[0]
        assert getattr(lib, fname)(U.ctypes.data_as(f32p), L.ctypes.data_as(f32p), n, b, 0, n,
                                   2) == 0
        return U, L
    return run


def _battery(run):
    for c in CASES.values():
        U, L = run("dbs_oracle_rounds_directed", c["U0"], c["L0"])
        if not (bits_equal(U, c["U1"]) and bits_equal(L, c["L1"])):
            return False
        U, L = run("dbs_oracle_rounds", c["U0"], c["L0"])
        if not (bits_equal(U, c["UN"]) and bits_equal(L, c["LN"])):
            return False
    U0, L0, X = gen.unquantised_line(50, seed=50)
    d = gen.true_distances(X)
    U, L = run("dbs_oracle_rounds_directed", U0, L0)
    return bool(np.all(U.astype(np.float64) >= d) and np.all(L.astype(np.float64) <= d))


@pytest.mark.parametrize("name", [None] + sorted(MUTANTS))
def test_directed_pins_reject_mutants(name, tmp_path):
    src = open(oracle.SRC).read()
    if name:
        old, new = MUTANTS[name]
        assert src.count(old) == 1, name
        src = src.replace(old, new)
    assert _battery(_build(src, tmp_path, name or "original")) == (name is None), name
