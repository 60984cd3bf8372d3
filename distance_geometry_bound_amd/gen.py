"""Seeded synthetic inputs for distance-bound triangle smoothing.

This module builds the dense bound matrices that both the GPU library and the
CPU reference consume.  It holds none of the smoothing arithmetic: it places
atoms (self-avoiding random-walk chains), measures their true distances, and
turns a subset of them into [lower, upper] intervals, with wide placeholders
for every pair the "experiment" did not measure.  The placeholders follow the
GPU Gems 2 Ch. 43 notes, §1 (unknown edges start at the molecular diameter for
the upper bound and at about zero for the lower bound).

Every value is rounded outward to the 2^-6 Angstrom grid (lower bounds down,
upper bounds up) in float64 and then stored as float32, which is exact for
|x| < 2^17.  On that grid every sum and difference of two bounds is exact in
fp32, so the smoothed result does not depend on the order of operations.

Named workloads (sizes and rules are those of the benchmark suite):

    n128      one chain, n=128, kept pairs d<5 A at p=0.5 as [d-0.5, d+0.5]
    n1024     one chain, n=1024, kept pairs d<6 A at p=0.3, half-width U(0.25,1)
    b64n500   64 chains of n=500 (seeds 3000+b), rules of n128
    n4096     16 chains x 256 in a sphere of radius 60 A, d<6 A at p=0.2,
              +-0.5 A; unknown pairs get L=1.0, U=120
    n12288    48 chains x 256 in a sphere of radius 90 A, d<5 A at p=0.1,
              +-0.5 A; unknown pairs get L=0, U=180
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GRID = 64.0            # values are multiples of 1/GRID Angstrom
STEP = 3.8             # bond length of the walk (A)
EXCL = 3.0             # minimum distance to any earlier atom (A)
MAX_TRIES = 1000       # failed placements before a chain restarts

__all__ = [
    "Molecule", "Workload", "WORKLOADS", "round_down", "round_up",
    "walk_chain", "sphere_chains", "restraints_from_coords", "bounds_from_coords",
    "make_molecule", "molecule_restraints", "make_workload", "workload_restraints", "random_bounds", "random_sound_bounds",
    "random_directed_bounds", "true_distances",
]


def round_down(x):
    """Largest multiple of 2^-6 that is <= x (float64 in, float64 out)."""
    return np.floor(np.asarray(x, dtype=np.float64) * GRID) / GRID


def round_up(x):
    """Smallest multiple of 2^-6 that is >= x (float64 in, float64 out)."""
    return np.ceil(np.asarray(x, dtype=np.float64) * GRID) / GRID


class _CellGrid:
    """Uniform hash grid with cell size EXCL for the exclusion test."""

    def __init__(self, h: float = EXCL):
        self.h = h
        self.cells: dict[tuple[int, int, int], list[int]] = {}
        self.pts: list[tuple[float, float, float]] = []

    def key(self, p):
        h = self.h
        return (math.floor(p[0] / h), math.floor(p[1] / h), math.floor(p[2] / h))

    def clear_from(self, start: int) -> None:
        """Forget atoms start..end (a chain that restarts)."""
        for idx in range(start, len(self.pts)):
            self.cells[self.key(self.pts[idx])].remove(idx)
        del self.pts[start:]

    def add(self, p) -> None:
        self.pts.append((float(p[0]), float(p[1]), float(p[2])))
        self.cells.setdefault(self.key(p), []).append(len(self.pts) - 1)

    def free(self, p, r2: float = EXCL * EXCL) -> bool:
        cx, cy, cz = self.key(p)
        px, py, pz = float(p[0]), float(p[1]), float(p[2])
        pts, cells = self.pts, self.cells
        for dx in (-1, 0, 1):
            for dy in (-1, 0, 1):
                for dz in (-1, 0, 1):
                    lst = cells.get((cx + dx, cy + dy, cz + dz))
                    if not lst:
                        continue
                    for q in lst:
                        a = pts[q]
                        ex, ey, ez = a[0] - px, a[1] - py, a[2] - pz
                        if ex * ex + ey * ey + ez * ez < r2:
                            return False
        return True


def _direction(rng) -> np.ndarray:
    v = rng.standard_normal(3)
    nv = float(np.sqrt(v @ v))
    while nv == 0.0:
        v = rng.standard_normal(3)
        nv = float(np.sqrt(v @ v))
    return v / nv


def _grow(rng, grid: _CellGrid, start: np.ndarray, length: int,
          radius: float | None) -> bool:
    """Append one chain of `length` atoms starting at `start` to `grid`.

    Each step is STEP long in a uniformly random direction; a step closer than
    EXCL to any atom already placed (or outside the sphere, when `radius` is
    given) is redrawn.  Returns False after MAX_TRIES failures at one step.
    """
    grid.add(start)
    prev = start
    for _ in range(length - 1):
        for _try in range(MAX_TRIES):
            p = prev + STEP * _direction(rng)
            if radius is not None and float(p @ p) > radius * radius:
                continue
            if grid.free(p):
                break
        else:
            return False
        grid.add(p)
        prev = p
    return True


def walk_chain(n: int, seed: int) -> np.ndarray:
    """Self-avoiding random walk of n atoms starting at the origin, [n,3] f64."""
    rng = np.random.default_rng(seed)
    while True:
        grid = _CellGrid()
        if _grow(rng, grid, np.zeros(3), n, None):
            return np.asarray(grid.pts, dtype=np.float64).reshape(n, 3)


def sphere_chains(chains: int, length: int, radius: float, seed: int) -> np.ndarray:
    """`chains` self-avoiding walks of `length` atoms packed in a sphere.

    Chain starts are uniform in the sphere; the exclusion applies across all
    chains.  A chain that gets stuck is removed and restarted from a new start.
    Returns [chains*length, 3] f64, chain c occupying rows c*length..
    """
    rng = np.random.default_rng(seed)
    grid = _CellGrid()
    for _c in range(chains):
        while True:
            base = len(grid.pts)
            while True:
                s = rng.uniform(-radius, radius, 3)
                if float(s @ s) <= radius * radius and grid.free(s):
                    break
            if _grow(rng, grid, s, length, radius):
                break
            grid.clear_from(base)
    return np.asarray(grid.pts, dtype=np.float64)


def true_distances(X: np.ndarray, rows=None) -> np.ndarray:
    """Euclidean distances (float64) between rows `rows` of X and all of X."""
    X = np.asarray(X, dtype=np.float64)
    A = X if rows is None else X[rows]
    d2 = ((A[:, None, :] - X[None, :, :]) ** 2).sum(-1)
    return np.sqrt(d2)


@dataclass
class Molecule:
    U: np.ndarray            # [n,n] float32 upper bounds
    L: np.ndarray            # [n,n] float32 lower bounds
    X: np.ndarray            # [n,3] float64 true coordinates
    chain_len: int           # atoms per chain (neighbour pairs never cross chains)


def _pairs_within(X: np.ndarray, cutoff: float):
    """Unordered pairs (i<j) with true distance < cutoff, sorted (i, j)."""
    from scipy.spatial import cKDTree

    tree = cKDTree(X)
    pr = tree.query_pairs(r=cutoff, output_type="ndarray")
    if pr.size == 0:
        return np.zeros((0, 2), dtype=np.int64), np.zeros(0)
    pr = np.sort(pr.astype(np.int64), axis=1)
    order = np.lexsort((pr[:, 1], pr[:, 0]))
    pr = pr[order]
    d = np.sqrt(((X[pr[:, 0]] - X[pr[:, 1]]) ** 2).sum(-1))
    keep = d < cutoff
    return pr[keep], d[keep]


def _diameter(X: np.ndarray) -> float:
    n = X.shape[0]
    best = 0.0
    for s in range(0, n, 1024):
        best = max(best, float(true_distances(X, np.arange(s, min(n, s + 1024))).max()))
    return best


def restraints_from_coords(X: np.ndarray, chain_len: int, rng, *, cutoff: float, p: float,
                           halfwidth):
    """The measured pairs of a molecule, before rounding.

    * bonded neighbours (i, i+1) of one chain: the true distance d as [d, d];
    * other pairs with d < cutoff, each kept with probability p: [d-w, d+w]
      (w a number, or w ~ U(lo, hi) per pair when `halfwidth` is a pair).
    Random draws: one uniform per candidate pair for the keep decision, then
    one half-width per candidate when it is drawn, both in sorted pair order.
    Returns (ia, ja, lo, hi): int64 atom indices (i < j) and float64 bounds,
    kept pairs first, then the bonded neighbours.
    """
    n = X.shape[0]
    pr, d = _pairs_within(X, cutoff)
    bonded = (pr[:, 1] == pr[:, 0] + 1) & (pr[:, 0] // chain_len == pr[:, 1] // chain_len)
    cand, dc = pr[~bonded], d[~bonded]
    u = rng.random(len(cand))
    if isinstance(halfwidth, tuple):
        w = rng.uniform(halfwidth[0], halfwidth[1], len(cand))
    else:
        w = np.full(len(cand), float(halfwidth))
    kept = u < p
    bi = np.arange(n - 1)
    bi = bi[(bi // chain_len) == ((bi + 1) // chain_len)]
    bd = np.sqrt(((X[bi] - X[bi + 1]) ** 2).sum(-1))
    ia = np.concatenate([cand[kept, 0], bi])
    ja = np.concatenate([cand[kept, 1], bi + 1])
    lo = np.concatenate([dc[kept] - w[kept], bd])
    hi = np.concatenate([dc[kept] + w[kept], bd])
    return ia, ja, lo, hi


def bounds_from_coords(X: np.ndarray, chain_len: int, rng, *, cutoff: float,
                       p: float, halfwidth, unknown_L: float,
                       unknown_U: float | None) -> tuple[np.ndarray, np.ndarray]:
    """Dense symmetric [n,n] float32 (U, L) from coordinates.

    Every measured pair of restraints_from_coords gets its interval rounded
    outward (the lower end clipped at 0); every other pair gets
    [unknown_L, unknown_U], where unknown_U None means the molecular diameter
    (largest true distance) rounded up; the diagonal is 0.
    """
    n = X.shape[0]
    if unknown_U is None:
        unknown_U = float(round_up(_diameter(X))) if n > 1 else 0.0
    U = np.full((n, n), unknown_U, dtype=np.float32)
    L = np.full((n, n), unknown_L, dtype=np.float32)
    ia, ja, lo, hi = restraints_from_coords(X, chain_len, rng, cutoff=cutoff, p=p,
                                            halfwidth=halfwidth)
    lo = round_down(np.maximum(lo, 0.0)).astype(np.float32)
    hi = round_up(hi).astype(np.float32)
    U[ia, ja] = hi; U[ja, ia] = hi
    L[ia, ja] = lo; L[ja, ia] = lo
    idx = np.arange(n)
    U[idx, idx] = 0.0
    L[idx, idx] = 0.0
    return U, L


def _molecule_setup(n: int, seed: int, chains: int, radius):
    if chains == 1:
        return walk_chain(n, seed), max(n, 1)
    if n % chains:
        raise ValueError("n must be a multiple of chains")
    return sphere_chains(chains, n // chains, radius, seed), n // chains


def make_molecule(n: int, seed: int, *, cutoff: float = 5.0, p: float = 0.5,
                  halfwidth=0.5, unknown_L: float = 0.0,
                  unknown_U: float | None = None, chains: int = 1,
                  radius: float | None = None) -> Molecule:
    """One molecule of n atoms (a single walk, or `chains` walks in a sphere)."""
    X, chain_len = _molecule_setup(n, seed, chains, radius)
    rng = np.random.default_rng([seed, 0xB0])
    U, L = bounds_from_coords(X, chain_len, rng, cutoff=cutoff, p=p,
                              halfwidth=halfwidth, unknown_L=unknown_L,
                              unknown_U=unknown_U)
    return Molecule(U=U, L=L, X=X, chain_len=chain_len)


def molecule_restraints(n: int, seed: int, *, cutoff: float = 5.0, p: float = 0.5,
                        halfwidth=0.5, unknown_L: float = 0.0,
                        unknown_U: float | None = None, chains: int = 1,
                        radius: float | None = None):
    """The restraint list behind make_molecule (same arguments, same draws).

    Returns (ia, ja, lo, hi, unknown_L, unknown_U): the measured pairs with
    their unrounded float64 intervals, and the placeholders (unknown_U None
    becomes the molecular diameter, rounded up)."""
    X, chain_len = _molecule_setup(n, seed, chains, radius)
    rng = np.random.default_rng([seed, 0xB0])
    if unknown_U is None:
        unknown_U = float(round_up(_diameter(X))) if n > 1 else 0.0
    ia, ja, lo, hi = restraints_from_coords(X, chain_len, rng, cutoff=cutoff, p=p,
                                            halfwidth=halfwidth)
    return ia, ja, lo, hi, unknown_L, unknown_U


@dataclass
class Workload:
    name: str
    n: int
    batch: int
    U: np.ndarray            # [batch,n,n] float32
    L: np.ndarray            # [batch,n,n] float32
    X: list = field(default_factory=list)   # per molecule [n,3] float64


def _workload_spec(name: str):
    if name == "n128":
        return dict(n=128, batch=1, seeds=[1], kw=dict(cutoff=5.0, p=0.5, halfwidth=0.5))
    if name == "n1024":
        return dict(n=1024, batch=1, seeds=[2],
                    kw=dict(cutoff=6.0, p=0.3, halfwidth=(0.25, 1.0)))
    if name == "b64n500":
        return dict(n=500, batch=64, seeds=[3000 + b for b in range(64)],
                    kw=dict(cutoff=5.0, p=0.5, halfwidth=0.5))
    if name == "n4096":
        return dict(n=4096, batch=1, seeds=[4],
                    kw=dict(cutoff=6.0, p=0.2, halfwidth=0.5, unknown_L=1.0,
                            unknown_U=120.0, chains=16, radius=60.0))
    if name == "n12288":
        return dict(n=12288, batch=1, seeds=[5],
                    kw=dict(cutoff=5.0, p=0.1, halfwidth=0.5, unknown_L=0.0,
                            unknown_U=180.0, chains=48, radius=90.0))
    raise KeyError(f"unknown workload {name!r}")


WORKLOADS = ("n128", "n1024", "b64n500", "n4096", "n12288")


def make_workload(name: str, batch: int | None = None) -> Workload:
    """Build a named workload; `batch` may shrink a batched workload."""
    spec = _workload_spec(name)
    seeds = spec["seeds"] if batch is None else spec["seeds"][:batch]
    n = spec["n"]
    U = np.empty((len(seeds), n, n), dtype=np.float32)
    L = np.empty((len(seeds), n, n), dtype=np.float32)
    Xs = []
    for b, s in enumerate(seeds):
        m = make_molecule(n, s, **spec["kw"])
        U[b], L[b] = m.U, m.L
        Xs.append(m.X)
    return Workload(name=name, n=n, batch=len(seeds), U=U, L=L, X=Xs)


def workload_restraints(name: str, batch: int | None = None):
    """Restraint lists of a named workload (molecule b's list has mol == b).

    Returns (mol, ia, ja, lo, hi, unknown_L, unknown_U, n, nbatch) with int32
    indices and float32 intervals (the unrounded values cast to float32), the
    form the GPU library takes.  The placeholders must agree across the
    batch; for the diameter-placeholder workloads the largest diameter is
    used.
    """
    spec = _workload_spec(name)
    seeds = spec["seeds"] if batch is None else spec["seeds"][:batch]
    parts, uL, uU = [], None, 0.0
    for b, s in enumerate(seeds):
        ia, ja, lo, hi, ul, uu = molecule_restraints(spec["n"], s, **spec["kw"])
        parts.append((np.full(len(ia), b), ia, ja, lo, hi))
        uL = ul
        uU = max(uU, uu)
    cat = [np.concatenate([p_[k] for p_ in parts]) for k in range(5)]
    return (cat[0].astype(np.int32), cat[1].astype(np.int32), cat[2].astype(np.int32),
            cat[3].astype(np.float32), cat[4].astype(np.float32), float(uL), float(uU),
            spec["n"], len(seeds))


def random_bounds(n: int, seed: int, *, umax_units: int = 256, batch: int | None = None):
    """Arbitrary (not necessarily consistent) bounds on the 2^-6 grid.

    U is symmetric with off-diagonal entries uniform in [1, umax_units]/64,
    L is symmetric with 0 <= L <= U, and both diagonals are 0.  Smoothing
    such input tightens many entries and may leave L > U (infeasible bounds),
    which is what stresses every candidate of the update.
    Returns float32 [n,n] pairs, or [batch,n,n] when batch is given.
    """
    rng = np.random.default_rng(seed)
    shape = (1 if batch is None else batch, n, n)
    Ui = rng.integers(1, umax_units + 1, size=shape)
    Ui = np.triu(Ui, 1)
    Ui = Ui + np.transpose(Ui, (0, 2, 1))
    Li = np.floor(rng.random(shape) * (Ui + 1)).astype(np.int64)
    Li = np.minimum(Li, Ui)
    Li = np.triu(Li, 1)
    Li = Li + np.transpose(Li, (0, 2, 1))
    U = (Ui / GRID).astype(np.float32)
    L = (Li / GRID).astype(np.float32)
    if batch is None:
        return U[0], L[0]
    return U, L


def random_sound_bounds(n: int, seed: int, *, box: float = 20.0, known: float = 0.4,
                        slack: float = 2.0, batch: int | None = None):
    """Bounds that contain the true distances of random points (so consistent).

    Points are uniform in a cube of side `box`.  Each unordered pair is known
    with probability `known` as [d - a, d + b] with a, b ~ U(0, slack), and
    unknown otherwise as [0, 2*box] (an upper bound on every distance).
    Outward-rounded to the 2^-6 grid.  Returns float32 [n,n] (or [batch,n,n])
    pairs and the coordinates.
    """
    rng = np.random.default_rng(seed)
    nb = 1 if batch is None else batch
    U = np.empty((nb, n, n), dtype=np.float32)
    L = np.empty((nb, n, n), dtype=np.float32)
    Xs = []
    for b in range(nb):
        X = rng.uniform(0.0, box, size=(n, 3))
        d = true_distances(X)
        a = rng.uniform(0.0, slack, size=(n, n))
        c = rng.uniform(0.0, slack, size=(n, n))
        k = rng.random((n, n)) < known
        a, c, k = np.triu(a, 1), np.triu(c, 1), np.triu(k, 1)
        a, c, k = a + a.T, c + c.T, k | k.T
        lo = np.where(k, round_down(np.maximum(d - a, 0.0)), 0.0)
        hi = np.where(k, round_up(d + c), round_up(2.0 * box))
        np.fill_diagonal(lo, 0.0)
        np.fill_diagonal(hi, 0.0)
        U[b], L[b] = hi, lo
        Xs.append(X)
    if batch is None:
        return U[0], L[0], Xs[0]
    return U, L, Xs


def f32_down(x):
    """The largest float32 <= x (x float64), elementwise."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) > x, np.nextafter(f, np.float32(-np.inf)), f)


def f32_up(x):
    """The smallest float32 >= x (x float64), elementwise."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) < x, np.nextafter(f, np.float32(np.inf)), f)


def random_unquantised_bounds(n: int, seed: int, *, box: float = 20.0, known: float = 0.4,
                              slack: float = 2.0, batch: int | None = None):
    """random_sound_bounds without the 2^-6 grid: each known pair gets
    [d - a, d + b] (a, b ~ U(0, slack); slack 0 gives [d, d]) rounded outward
    to the neighbouring float32 values, so sums and differences of bounds
    are generally not exact in float32.  Unknown pairs get [0, 2*box]."""
    rng = np.random.default_rng([seed, 0xF32])
    nb = 1 if batch is None else batch
    U = np.empty((nb, n, n), dtype=np.float32)
    L = np.empty((nb, n, n), dtype=np.float32)
    Xs = []
    for b in range(nb):
        X = rng.uniform(0.0, box, size=(n, 3))
        d = true_distances(X)
        a = rng.uniform(0.0, slack, size=(n, n)) if slack > 0 else np.zeros((n, n))
        c = rng.uniform(0.0, slack, size=(n, n)) if slack > 0 else np.zeros((n, n))
        k = rng.random((n, n)) < known
        a, c, k = np.triu(a, 1), np.triu(c, 1), np.triu(k, 1)
        a, c, k = a + a.T, c + c.T, k | k.T
        lo = np.where(k, f32_down(np.maximum(d - a, 0.0)), 0.0)
        hi = np.where(k, f32_up(d + c), f32_up(2.0 * box))
        np.fill_diagonal(lo, 0.0)
        np.fill_diagonal(hi, 0.0)
        U[b], L[b] = hi, lo
        Xs.append(X)
    if batch is None:
        return U[0], L[0], Xs[0]
    return U, L, Xs


def unquantised_line(n: int, seed: int, *, spacing: tuple = (1.0, 4.0)):
    """Atoms on a line at random float64 positions (gaps ~ U(spacing)): each
    neighbour pair and the two end atoms known exactly, [d, d] rounded
    outward to float32, every other pair [0, total length + 1 rounded up].
    Along a line distances add, so the smoothed upper bounds are sums of many
    rounded terms, and the lower bounds (end-to-end length minus the rest)
    differences of them: a stringent case for the soundness of rounding.
    Returns (U, L, positions)."""
    rng = np.random.default_rng([seed, 0x11E])
    x = np.concatenate([[0.0], np.cumsum(rng.uniform(spacing[0], spacing[1], n - 1))])
    X = np.stack([x, np.zeros(n), np.zeros(n)], axis=1)
    U = np.full((n, n), f32_up(x[-1] - x[0] + 1.0), dtype=np.float32)
    L = np.zeros((n, n), dtype=np.float32)
    i = np.arange(n - 1)
    gap = x[1:] - x[:-1]
    U[i, i + 1] = U[i + 1, i] = f32_up(gap)
    L[i, i + 1] = L[i + 1, i] = f32_down(gap)
    if n > 2:
        U[0, n - 1] = U[n - 1, 0] = f32_up(x[-1] - x[0])
        L[0, n - 1] = L[n - 1, 0] = f32_down(x[-1] - x[0])
    np.fill_diagonal(U, 0.0)
    return U, L, X


def random_directed_bounds(n: int, seed: int, *, box: float = 12.0,
                           known: float = 0.5, slack: float = 3.0):
    """Asymmetric bounds around a symmetric metric (random points in a cube).

    Each ordered pair (i,j) is known with probability `known`, independently
    of (j,i), as [d - a, d + b] with a, b ~ U(0, slack) drawn per direction;
    unknown pairs get [0, 2*box].  The bounds contain the true distances, so
    they are consistent, but U and L are not symmetric.  Used only to exercise
    a reference implementation on directed input.  Returns float32 (U, L).
    """
    rng = np.random.default_rng(seed)
    X = rng.uniform(0.0, box, size=(n, 3))
    d = true_distances(X)
    a = rng.uniform(0.0, slack, size=(n, n))
    c = rng.uniform(0.0, slack, size=(n, n))
    k = rng.random((n, n)) < known
    lo = np.where(k, round_down(np.maximum(d - a, 0.0)), 0.0)
    hi = np.where(k, round_up(d + c), round_up(2.0 * box))
    np.fill_diagonal(lo, 0.0)
    np.fill_diagonal(hi, 0.0)
    return hi.astype(np.float32), lo.astype(np.float32)
