"""The input-check definitions flag exactly the violated precondition."""
import numpy as np
import pytest

from distance_geometry_bound_amd import gen
from oracle import check


def _base(n=9):
    U, L, _ = gen.random_sound_bounds(n, seed=5)
    return U.copy(), L.copy()


def test_clean_input():
    U, L = _base()
    assert check.flags(U, L) == 0


@pytest.mark.parametrize("case,flag", [
    ("asym", check.ASYM), ("diag", check.DIAG), ("nan", check.NONFINITE),
    ("inf", check.NONFINITE), ("lgtu", check.L_GT_U), ("lneg", check.L_NEG),
    ("unq", check.UNQUANT), ("range", check.RANGE), ("negzero", check.NEGZERO),
])
def test_single_violation(case, flag):
    U, L = _base()
    if case == "asym":
        U[1, 2] += 1.0
    elif case == "diag":
        U[3, 3] = 1.0
    elif case == "nan":
        U[1, 2] = U[2, 1] = np.nan
    elif case == "inf":
        U[1, 2] = U[2, 1] = np.inf
    elif case == "lgtu":
        L[1, 2] = L[2, 1] = U[1, 2] + 1.0
    elif case == "lneg":
        L[1, 2] = L[2, 1] = -1.0
    elif case == "unq":
        U[1, 2] = U[2, 1] = U[1, 2] + 0.001
    elif case == "range":
        U[1, 2] = U[2, 1] = 2.0 ** 17
    elif case == "negzero":
        L[1, 2] = L[2, 1] = -0.0
    f = check.flags(U, L)
    assert f & flag
    # no other flag may fire
    assert f == flag, (case, f)
