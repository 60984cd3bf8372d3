"""Plain definitions of the input checks reported by the library's validator.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The smoothing update is exact only for inputs that meet its preconditions:
bound matrices of a molecule are symmetric with a zero diagonal (GPU Gems 2,
Ch. 43 notes, §1), 0 <= L <= U, finite, and on the 2^-6 grid with
|x| < 2^17 so that every sum and difference is exact in fp32 (the notes' §6
puts the arithmetic in 32-bit IEEE float).  Each flag below is one of those
conditions, evaluated over a whole [batch,n,n] input.
"""
import numpy as np

ASYM = 1          # U or L not bit-for-bit symmetric
DIAG = 2          # a diagonal entry of U or L is not +0.0
NONFINITE = 4     # NaN or +-Inf anywhere
L_GT_U = 8        # L[i,j] > U[i,j] somewhere
L_NEG = 16        # L[i,j] < 0 somewhere
UNQUANT = 32      # a value that is not a multiple of 2^-6
RANGE = 64        # |x| >= 2^17
NEGZERO = 128     # a -0.0 anywhere


def flags(U, L) -> int:
    U = np.asarray(U, dtype=np.float32)
    L = np.asarray(L, dtype=np.float32)
    if U.ndim == 2:
        U, L = U[None], L[None]
    f = 0
    ub, lb = U.view(np.uint32), L.view(np.uint32)
    if not (np.array_equal(ub, ub.transpose(0, 2, 1)) and
            np.array_equal(lb, lb.transpose(0, 2, 1))):
        f |= ASYM
    du = np.diagonal(ub, axis1=1, axis2=2)
    dl = np.diagonal(lb, axis1=1, axis2=2)
    if np.any(du != 0) or np.any(dl != 0):
        f |= DIAG
    fin_u, fin_l = np.isfinite(U), np.isfinite(L)
    if not (fin_u.all() and fin_l.all()):
        f |= NONFINITE
    with np.errstate(invalid="ignore"):
        if np.any(L > U):
            f |= L_GT_U
        if np.any(L < 0):
            f |= L_NEG
        for A, fin in ((U, fin_u), (L, fin_l)):
            a = A[fin].astype(np.float64)
            if np.any(a * 64.0 != np.floor(a * 64.0)):
                f |= UNQUANT
            if np.any(np.abs(a) >= 2.0 ** 17):
                f |= RANGE
    if np.any(ub == 0x80000000) or np.any(lb == 0x80000000):
        f |= NEGZERO
    return f


def flags_packed(P) -> int:
    """The checks of a packed buffer (U strictly above the diagonal, L strictly
    below, the shared zero diagonal on it; GPU Gems 2, Ch. 43 notes, §6 on
    keeping one triangle of each symmetric matrix): by definition those of the
    dense pair it stands for, U[i,j] = P[min,max] and L[i,j] = P[max,min].
    That pair is symmetric by construction, so ASYM never appears."""
    P = np.asarray(P, dtype=np.float32)
    if P.ndim == 2:
        P = P[None]
    n = P.shape[-1]
    upper = np.triu(np.ones((n, n), dtype=bool), 1)
    lower = upper.T
    Pt = P.transpose(0, 2, 1)
    U = np.where(lower, Pt, P)           # P[min, max]
    L = np.where(upper, Pt, P)           # P[max, min]
    return flags(U, L)
