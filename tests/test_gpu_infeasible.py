"""The infeasibility option of a pass on the GPU (needs an MI355X).

A pass given per-molecule words ORs DBS_INFEASIBLE_END into the word of a
molecule whose output has some L > U, and, in the blocked pass,
DBS_INFEASIBLE_EARLY where phase 1 closes a diagonal tile that has L > U
(GPU Gems 2, Ch. 43 notes, §2: the lower bounds only rise and the upper bounds
only fall, so L > U at any step means inconsistent bounds, and on
inconsistent ones the finished pass shows L > U somewhere).

  * Consistent bounds (sound ones built from coordinates, and the workloads):
    no word is ever set, for every algorithm, layout and schedule.
  * Inconsistent bounds: END is set exactly for the molecules whose oracle
    result has L > U, in a batch that mixes both kinds.
  * A violation planted in the first diagonal tile sets EARLY in every
    blocked schedule (phase 1 of the first k-block sees it); EARLY never
    comes without END.
"""
import numpy as np
import pytest
import torch

import distance_geometry_bound_amd as dgb
import oracle
from distance_geometry_bound_amd import gen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
EARLY, END = dgb.INFEASIBLE_EARLY, dgb.INFEASIBLE_END

SCHEDULES = [dict(algo="perk"), dict(algo="auto"), dict(algo="blocked", lookahead=0),
             dict(algo="blocked", lookahead=1), dict(algo="blocked", lookahead=2),
             dict(algo="blocked", lookahead=2, step_blocks=3),
             dict(algo="blocked", lookahead=0, lead=True),
             dict(algo="blocked", lookahead=0, lead=False)]


def dev(A):
    return torch.from_numpy(np.ascontiguousarray(A)).to(DEV)


def run(U0, L0, packed, **kw):
    """One pass with the option; returns the words (host)."""
    batch = U0.shape[0]
    words = torch.zeros(batch, dtype=torch.int32, device=DEV)
    if packed:
        P = dgb.pack(dev(U0), dev(L0))
        dgb.smooth_packed(P, infeasible=words, **kw)
    else:
        dgb.smooth(dev(U0), dev(L0), infeasible=words, **kw)
    torch.cuda.synchronize(DEV)
    return words.cpu().numpy().astype(np.uint32)


def lds_ok(n, kw):
    return kw.get("algo") != "lds" or n <= dgb.lib().dbs_lds_max_n()


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("n,batch", [(65, 2), (129, 1), (300, 2), (700, 1)])
def test_consistent_bounds_set_no_word(n, batch, packed):
    U0, L0, _ = gen.random_sound_bounds(n, seed=n + batch, batch=batch, box=6.0 + n / 8)
    for kw in SCHEDULES + ([dict(algo="lds")] if n <= 176 else []):
        assert not run(U0, L0, packed, **kw).any(), (n, batch, packed, kw)


def test_workloads_set_no_word():
    for name in ("n128", "n1024", "b64n500"):
        W = gen.make_workload(name)
        assert not run(W.U, W.L, False).any(), name
        assert not run(W.U, W.L, True).any(), name


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("n", [150, 385])
def test_end_marks_exactly_the_inconsistent_molecules(n, packed):
    # molecule 0 sound, molecules 1 and 2 arbitrary (mostly inconsistent)
    Us, Ls, _ = gen.random_sound_bounds(n, seed=n, batch=1, box=6.0 + n / 8)
    Ur, Lr = gen.random_bounds(n, seed=n + 1, batch=2, umax_units=200)
    U0, L0 = np.concatenate([Us, Ur]), np.concatenate([Ls, Lr])
    Ue, Le = oracle.smooth(U0, L0)
    want = [bool(np.any(Le[b] > Ue[b])) for b in range(3)]
    assert want[0] is False and any(want)
    for kw in SCHEDULES:
        got = run(U0, L0, packed, **kw)
        assert [bool(w & END) for w in got] == want, (n, packed, kw, got)
        assert all(not (w & EARLY) or (w & END) for w in got), (n, packed, kw, got)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("n", [200, 520])
def test_a_violation_in_the_first_diagonal_tile_is_seen_early(n, packed):
    U0, L0, _ = gen.random_sound_bounds(n, seed=2 * n, batch=2, box=6.0 + n / 8)
    U0, L0 = U0.copy(), L0.copy()
    L0[1, 3, 5] = L0[1, 5, 3] = U0[1, 3, 5] + 1.0   # molecule 1 only
    for kw in SCHEDULES[2:]:
        got = run(U0, L0, packed, **kw)
        assert got[0] == 0 and got[1] == EARLY | END, (n, packed, kw, got)


def test_a_range_tests_its_own_output():
    n = 300
    U0, L0, _ = gen.random_sound_bounds(n, seed=7, batch=1, box=6.0 + n / 8)
    U, L = dev(U0), dev(L0)
    words = torch.zeros(1, dtype=torch.int32, device=DEV)
    dgb.smooth_range(U, L, 0, 128, infeasible=words)
    torch.cuda.synchronize(DEV)
    assert int(words.item()) == 0
    L[0, 200, 201] = L[0, 201, 200] = U[0, 200, 201] + 1.0   # outside the tiles closed next
    dgb.smooth_range(U, L, 128, 192, infeasible=words)
    torch.cuda.synchronize(DEV)
    assert int(words.item()) & END


def test_words_are_validated():
    U, L = torch.zeros(2, 8, 8, device=DEV), torch.zeros(2, 8, 8, device=DEV)
    with pytest.raises(ValueError):
        dgb.smooth(U, L, infeasible=torch.zeros(1, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        dgb.smooth(U, L, infeasible=torch.zeros(2, dtype=torch.float32, device=DEV))
