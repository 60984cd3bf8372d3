"""Seeded random sweep of shapes and options against the CPU oracle (needs an MI355X).

Each case draws n (including k-block and tile tails), a batch, an algorithm (on either layout),
the layout (dense or packed), the rounding entry point (plain or directed; on grid inputs both must give the plain
pass's bits), a look-ahead depth (automatic or forced 0, 1, 2), a step width (automatic or
forced 1..4 k-blocks) and the lead schedule (automatic, off or on). It runs one full pass, or a
pass split at a k-block boundary, and compares every entry with the oracle bit for bit. The draws
are fixed by the seed, so a failure names a reproducible case.
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


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    n = int(rng.choice([int(rng.integers(2, 200)), int(rng.integers(200, 900)),
                        64 * int(rng.integers(2, 12)) + int(rng.integers(-1, 2))]))
    batch = int(rng.integers(1, 4))
    algo = str(rng.choice(["auto", "blocked", "blocked", "perk"] + (["lds"] if n <= 176 else [])))
    packed = bool(rng.integers(0, 2))
    directed = bool(rng.integers(0, 2))
    depth = int(rng.choice([-1, 0, 1, 2]))
    split = bool(rng.integers(0, 2)) and n > 128
    blocks = int(rng.choice([-1, 1, 2, 3, 4]))
    lead = [None, False, True][int(rng.integers(0, 3))]
    return n, batch, algo, packed, directed, depth, split, blocks, lead


def _run(U0, L0, n, algo, packed, directed, depth, split, blocks, lead):
    kw = dict(algo=algo, lookahead=None if depth < 0 else depth,
              step_blocks=None if blocks < 0 else blocks, lead=lead)
    cuts = [0, 128, n] if split else [0, n]
    if packed:
        P = dgb.pack(torch.from_numpy(U0).to(DEV), torch.from_numpy(L0).to(DEV))
        for a, b in zip(cuts[:-1], cuts[1:]):
            (dgb.smooth_packed_directed if directed else dgb.smooth_packed)(P, a, b, **kw)
        torch.cuda.synchronize(DEV)
        return P.cpu().numpy(), None
    U = torch.from_numpy(U0).to(DEV)
    L = torch.from_numpy(L0).to(DEV)
    for a, b in zip(cuts[:-1], cuts[1:]):
        if directed:
            dgb.smooth_directed_range(U, L, a, b, **kw)
        else:
            dgb.smooth_range(U, L, a, b, **kw)
    torch.cuda.synchronize(DEV)
    return U.cpu().numpy(), L.cpu().numpy()


@pytest.mark.parametrize("seed", range(64))
def test_random_case_matches_oracle(seed):
    n, batch, algo, packed, directed, depth, split, blocks, lead = _case(seed)
    tag = (f"seed={seed} n={n} batch={batch} algo={algo} packed={packed} "
           f"directed={directed} depth={depth} split={split} blocks={blocks} lead={lead}")
    U0, L0, _ = gen.random_sound_bounds(n, seed=seed, batch=batch, box=6.0 + n / 8)
    Ue, Le = oracle.smooth(U0, L0)
    A, B = _run(U0, L0, n, algo, packed, directed, depth, split, blocks, lead)
    if packed:
        assert np.array_equal(A.view(np.uint32), steps.pack(Ue, Le).view(np.uint32)), tag
    else:
        assert np.array_equal(A.view(np.uint32), Ue.view(np.uint32)), tag
        assert np.array_equal(B.view(np.uint32), Le.view(np.uint32)), tag


def _batch_case(seed):
    # many small molecules: 100 to 4000 phase-3 tiles x molecules, across the
    # automatic choices for batches (lead below 1024 tiles, then two steps
    # ahead in steps of one, two or four k-blocks)
    rng = np.random.default_rng(7000 + seed)
    n = int(rng.integers(65, 330))
    T = -(-n // 128)
    tiles = T * (T + 1) // 2
    batch = int(rng.integers(max(2, 100 // tiles), 4000 // tiles + 1))
    batch = min(batch, 1200)
    packed = bool(rng.integers(0, 2))
    directed = bool(rng.integers(0, 2))
    return n, batch, packed, directed


@pytest.mark.parametrize("seed", range(16))
def test_random_batch_matches_oracle(seed):
    n, batch, packed, directed = _batch_case(seed)
    sched = dgb.schedule(n, batch, packed=packed)
    tag = f"seed={seed} n={n} batch={batch} packed={packed} directed={directed} schedule={sched}"
    U0, L0, _ = gen.random_sound_bounds(n, seed=seed, batch=batch, box=6.0 + n / 8)
    Ue, Le = oracle.smooth(U0, L0)
    A, B = _run(U0, L0, n, "auto", packed, directed, -1, False, -1, None)
    if packed:
        assert np.array_equal(A.view(np.uint32), steps.pack(Ue, Le).view(np.uint32)), tag
    else:
        assert np.array_equal(A.view(np.uint32), Ue.view(np.uint32)), tag
        assert np.array_equal(B.view(np.uint32), Le.view(np.uint32)), tag


def test_single_molecule_two_ahead_in_one_block_steps():
    # n = 5120 (820 phase-3 tiles): a single dense molecule runs two steps
    # ahead in steps of one k-block; every entry against the oracle
    n = 5120
    assert dgb.schedule(n, 1) == (2, 1, 0)
    U0, L0, _ = gen.random_sound_bounds(n, seed=n, batch=1, box=6.0 + n / 8)
    Ue, Le = oracle.smooth(U0, L0)
    A, B = _run(U0, L0, n, "auto", False, False, -1, False, -1, None)
    assert np.array_equal(A.view(np.uint32), Ue.view(np.uint32))
    assert np.array_equal(B.view(np.uint32), Le.view(np.uint32))
