"""Independent checks that pin the CPU oracle (test code only).

None of these helpers shares code with the oracle or the GPU library.  They
compute what one smoothing pass must reach from its plain definitions, in
exact int64 units of 2^-6 A:

* the upper bounds after a full pass are the shortest-path lengths of the
  complete graph weighted by U (Floyd-Warshall is named as an all-pairs
  shortest-path algorithm in GPU Gems 2, Ch. 43 notes, §3);
* the lower bounds after a full pass are
      L*[i,j] = max over (k,l) of  L[k,l] - U*[i,k] - U*[l,j],
  i.e. two max-plus products.  Reason: the fused round of §2 is
  Floyd-Warshall on a 2n-vertex digraph (two copies of K_n weighted by U and
  one-way crossing edges i -> j' of weight -L[i,j]); with U >= 0 it has no
  negative cycle, so every vertex order, block partition or buffer scheme
  reaches the same shortest paths, and d(i, j') = -L*[i,j].
"""
from __future__ import annotations

import itertools

import numpy as np

GRID = 64


def units(A) -> np.ndarray:
    """float32 grid values -> exact int64 multiples of 2^-6."""
    A = np.asarray(A, dtype=np.float64)
    Q = A * GRID
    assert np.all(Q == np.round(Q)), "value off the 2^-6 grid"
    return np.round(Q).astype(np.int64)


def from_units(Q) -> np.ndarray:
    return (np.asarray(Q, dtype=np.float64) / GRID).astype(np.float32)


# ---------------------------------------------------------------- brute force
def brute_upper(Ui: np.ndarray) -> np.ndarray:
    """Shortest simple-path lengths by enumerating every simple path (n <= 8).

    Works for directed (asymmetric) weights too.  The trivial path gives 0 on
    the diagonal; a direct edge i->j is the path with no intermediate atom.
    """
    n = Ui.shape[0]
    best = np.empty_like(Ui)
    for i in range(n):
        for j in range(n):
            if i == j:
                best[i, j] = min(0, Ui[i, i])
                continue
            others = [v for v in range(n) if v != i and v != j]
            b = Ui[i, j]
            for m in range(1, len(others) + 1):
                for mid in itertools.permutations(others, m):
                    path = (i,) + mid + (j,)
                    s = 0
                    for a, c in zip(path[:-1], path[1:]):
                        s += Ui[a, c]
                    if s < b:
                        b = s
            best[i, j] = b
    return best


def brute_lower(Li: np.ndarray, Us: np.ndarray) -> np.ndarray:
    """max over (k,l) of L[k,l] - U*[i,k] - U*[l,j], by direct enumeration."""
    n = Li.shape[0]
    out = np.empty_like(Li)
    for i in range(n):
        for j in range(n):
            out[i, j] = max(Li[k, l] - Us[i, k] - Us[l, j]
                            for k in range(n) for l in range(n))
    return out


# ------------------------------------------------------------- library / algebra
def apsp_scipy(U: np.ndarray) -> np.ndarray:
    """All-pairs shortest paths with scipy (float64; exact on the grid)."""
    from scipy.sparse.csgraph import shortest_path

    U = np.asarray(U, dtype=np.float64)
    off = ~np.eye(U.shape[0], dtype=bool)
    # dense scipy input reads a 0 weight as "no edge"; our off-diagonals are > 0
    assert np.all(U[off] > 0)
    return shortest_path(U, method="FW", directed=True)


def maxplus(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C[i,j] = max_k A[i,k] + B[k,j] (int64, exact)."""
    C = A[:, :1] + B[:1, :]
    for k in range(1, A.shape[1]):
        np.maximum(C, A[:, k:k + 1] + B[k:k + 1, :], out=C)
    return C


def closed_lower(Li: np.ndarray, Us: np.ndarray) -> np.ndarray:
    """L* = max_{k,l} L[k,l] - U*[i,k] - U*[l,j] as two max-plus products."""
    M = maxplus(Li, -Us)            # M[k,j] = max_l L[k,l] - U*[l,j]
    return maxplus(-Us, M)          # L*[i,j] = max_k -U*[i,k] + M[k,j]


# ------------------------------------------------------------------ invariants
def triangle_violations(Ui: np.ndarray) -> int:
    """Count (i,j,k) with U[i,j] > U[i,k] + U[k,j] (0 for a closed U)."""
    bad = 0
    for k in range(Ui.shape[0]):
        bad += int(np.count_nonzero(Ui > Ui[:, k:k + 1] + Ui[k:k + 1, :]))
    return bad


def lower_closure_violations(Li: np.ndarray, Ui: np.ndarray) -> int:
    """Count (i,j,k) with L[i,j] < L[i,k] - U[k,j] or < L[k,j] - U[i,k]."""
    bad = 0
    for k in range(Li.shape[0]):
        bad += int(np.count_nonzero(Li < Li[:, k:k + 1] - Ui[k:k + 1, :]))
        bad += int(np.count_nonzero(Li < Li[k:k + 1, :] - Ui[:, k:k + 1]))
    return bad


def sound(U, L, X) -> bool:
    """True distances (float64) of coordinates X lie inside [L, U]."""
    X = np.asarray(X, dtype=np.float64)
    n = X.shape[0]
    for s in range(0, n, 512):
        r = slice(s, min(n, s + 512))
        d = np.sqrt(((X[r, None, :] - X[None, :, :]) ** 2).sum(-1))
        if np.any(d < L[r].astype(np.float64)) or np.any(d > U[r].astype(np.float64)):
            return False
    return True


# ---------------------------------------------------------- algorithm variants
def variant_inplace_cells(Ui: np.ndarray, Li: np.ndarray):
    """One pass, in place, cell by cell: U then L of each cell (int64)."""
    U, L = Ui.copy(), Li.copy()
    n = U.shape[0]
    for k in range(n):
        for i in range(n):
            for j in range(n):
                U[i, j] = min(U[i, j], U[i, k] + U[k, j])
                L[i, j] = max(L[i, j], L[i, k] - U[k, j], L[k, j] - U[i, k])
    return U, L


def variant_two_pass(Ui: np.ndarray, Li: np.ndarray):
    """A whole upper pass first, then a whole lower pass on the final U."""
    U, L = Ui.copy(), Li.copy()
    n = U.shape[0]
    for k in range(n):
        U = np.minimum(U, U[:, k:k + 1] + U[k:k + 1, :])
    for k in range(n):
        L = np.maximum(L, np.maximum(L[:, k:k + 1] - U[k:k + 1, :],
                                     L[k:k + 1, :] - U[:, k:k + 1]))
    return U, L


def _fused_block(U, L, rows, cols, ks):
    """Relax the (rows x cols) block of U/L with intermediates ks, round by round."""
    for k in ks:
        U[np.ix_(rows, cols)] = np.minimum(U[np.ix_(rows, cols)],
                                           U[rows, k][:, None] + U[k, cols][None, :])
        L[np.ix_(rows, cols)] = np.maximum(
            L[np.ix_(rows, cols)],
            np.maximum(L[rows, k][:, None] - U[k, cols][None, :],
                       L[k, cols][None, :] - U[rows, k][:, None]))


def variant_blocked(Ui: np.ndarray, Li: np.ndarray, B: int):
    """Three-phase blocked Floyd-Warshall with block size B (int64, dense)."""
    U, L = Ui.copy(), Li.copy()
    n = U.shape[0]
    blocks = [np.arange(s, min(n, s + B)) for s in range(0, n, B)]
    for K in blocks:
        _fused_block(U, L, K, K, K)                       # diagonal tile
        for J in blocks:                                  # row and column panels
            if J[0] == K[0]:
                continue
            _fused_block(U, L, K, J, K)
            _fused_block(U, L, J, K, K)
        # remaining tiles: panels are final, so rounds can be merged
        for I in blocks:
            if I[0] == K[0]:
                continue
            for J in blocks:
                if J[0] == K[0]:
                    continue
                cu = U[np.ix_(I, K)]; cl = L[np.ix_(I, K)]
                ru = U[np.ix_(K, J)]; rl = L[np.ix_(K, J)]
                blk = np.ix_(I, J)
                U[blk] = np.minimum(U[blk], (cu[:, :, None] + ru[None, :, :]).min(1))
                L[blk] = np.maximum(L[blk], np.maximum(
                    (cl[:, :, None] - ru[None, :, :]).max(1),
                    (rl[None, :, :] - cu[:, :, None]).max(1)))
    return U, L


def sssp_dense(U, sources) -> np.ndarray:
    """Textbook O(n^2) Dijkstra from each source over the dense weights U.

    float64 (exact on the grid); returns [len(sources), n] shortest-path
    lengths.  All sources advance together, one settled vertex per step.
    """
    W = np.asarray(U)
    n = W.shape[0]
    S = len(sources)
    dist = np.full((S, n), np.inf)
    done = np.zeros((S, n), dtype=bool)
    rows = np.arange(S)
    dist[rows, list(sources)] = 0.0
    for _ in range(n):
        cand = np.where(done, np.inf, dist)
        u = cand.argmin(axis=1)
        done[rows, u] = True
        np.minimum(dist, dist[rows, u][:, None] + W[u].astype(np.float64), out=dist)
    return dist


def lower_pair(L, Us_i, Us_j) -> float:
    """L*[i,j] = max_{k,l} L[k,l] - U*[i,k] - U*[l,j] for one pair, from the
    shortest-path rows of i and j (U* symmetric).  float64, exact on the grid."""
    best = -np.inf
    n = L.shape[0]
    for s in range(0, n, 2048):
        blk = L[s:s + 2048].astype(np.float64) - Us_i[s:s + 2048, None] - Us_j[None, :]
        best = max(best, float(blk.max()))
    return best
