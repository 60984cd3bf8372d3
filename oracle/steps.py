"""Plain definitions of the steps around a smoothing pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bounds_from_restraints follows GPU Gems 2, Ch. 43 notes, §1: a molecule's
bound matrices start from placeholders (the molecular diameter above, about
zero below) and every measured pair carries its interval; values are rounded
outward to the 2^-6 grid so that the bounds stay sound and the later
smoothing is exact in 32-bit floats (§6).  tightened marks the cells whose
bounds changed, as the notes' §5 experiment colours the tightened entries.
Written as plain loops over the restraints, in float64.
"""
import numpy as np

GRID = 64.0
INDEX, VALUE = 1, 2      # status bits of a skipped restraint


def round_down(x):
    return np.floor(np.float64(x) * GRID) / GRID


def round_up(x):
    return np.ceil(np.float64(x) * GRID) / GRID


def bounds_from_restraints(n, batch, unknown_L, unknown_U, ia, ja, lo, hi, mol=None):
    """Dense float32 [batch,n,n] (U, L) and the status bits of skipped restraints.

    Placeholders off the diagonal (L rounded down, U rounded up), zeros on it;
    then each valid restraint (b, i, j, lo, hi) with i != j sets, for (i,j) and
    (j,i), L = max(L, round_down(max(lo, 0))) and U = min(U, round_up(hi)).
    A restraint is skipped, and flagged, when an index is out of range
    (INDEX) or when a value is not finite, lo > hi, hi < 0, |lo| >= 2^17 or
    the rounded hi >= 2^17 (VALUE).
    """
    U = np.full((batch, n, n), round_up(unknown_U), dtype=np.float64)
    L = np.full((batch, n, n), round_down(unknown_L), dtype=np.float64)
    for b in range(batch):
        np.fill_diagonal(U[b], 0.0)
        np.fill_diagonal(L[b], 0.0)
    status = 0
    for r in range(len(ia)):
        b = int(mol[r]) if mol is not None else 0
        i, j = int(ia[r]), int(ja[r])
        l, h = np.float64(lo[r]), np.float64(hi[r])
        bad = 0
        if not (0 <= b < batch and 0 <= i < n and 0 <= j < n):
            bad |= INDEX
        finite = np.isfinite(l) and np.isfinite(h)
        hr = round_up(h) if finite else np.nan
        if not finite or l > h or h < 0 or abs(l) >= 2.0 ** 17 or hr >= 2.0 ** 17:
            bad |= VALUE
        if bad:
            status |= bad
            continue
        if i == j:
            continue
        lr = round_down(max(l, 0.0))
        for (x, y) in ((i, j), (j, i)):
            U[b, x, y] = min(U[b, x, y], hr)
            L[b, x, y] = max(L[b, x, y], lr)
    return U.astype(np.float32), L.astype(np.float32), status


def tightened(U0, L0, U1, L1):
    """uint8 mask: 1 where U or L differs bit for bit between the two states."""
    a = [np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) for x in (U0, L0, U1, L1)]
    return ((a[0] != a[2]) | (a[1] != a[3])).astype(np.uint8)


def pack(U, L):
    """One-buffer storage of a molecule's bounds (GPU Gems 2, Ch. 43 notes, §6
    keeps the two symmetric matrices as two triangles): P[i,j] = U[i,j] above
    the diagonal, L[i,j] below it, and U[i,i] on it.  [..., n, n] float32."""
    U = np.asarray(U, dtype=np.float32)
    L = np.asarray(L, dtype=np.float32)
    n = U.shape[-1]
    iu = np.triu(np.ones((n, n), dtype=bool), 1)
    il = np.tril(np.ones((n, n), dtype=bool), -1)
    P = np.where(iu, U, np.where(il, L, U))
    return P.astype(np.float32)


def unpack(P):
    """Inverse of pack for symmetric bounds: U[i,j] = P[min,max],
    L[i,j] = P[max,min], U[i,i] = L[i,i] = P[i,i]."""
    P = np.asarray(P, dtype=np.float32)
    n = P.shape[-1]
    iu = np.triu(np.ones((n, n), dtype=bool), 1)
    Pt = np.swapaxes(P, -1, -2)
    U = np.where(iu, P, Pt)                       # upper part, mirrored
    L = np.where(iu, Pt, P)                       # lower part, mirrored
    d = np.arange(n)
    U[..., d, d] = P[..., d, d]
    L[..., d, d] = P[..., d, d]
    return U.astype(np.float32), L.astype(np.float32)
