"""CPU model of the blocked pass's schedule (test code only).

The GPU pass (csrc/blocked.hip) runs, per k-block K of BK = 64 atoms,
  phases 1+2  the rounds of band K over the diagonal tile (K,K) and, in the
           same loop, over each panel tile of band K (one workgroup per
           panel tile), panel tiles read from their fresh orientation (upper
           TILE x TILE region) and written in both orientations;
  phase 3  band K+1 first (the strip, on a second stream, followed there by
           phases 1-2 of K+1), and every other live cell of the upper
           TILE x TILE tiles (the bulk, on the caller's stream, as BK x BK
           quadrants: a quadrant in band K or K+1 is skipped whole, which
           leaves exactly the live cells modelled here);
and mirrors the upper tiles into the lower ones at the end.

This model re-implements that data flow in plain Python on exact int64 units
(one cell at a time, no shared code with the kernels or the oracle) and checks
  * that it reaches the oracle's result bit for bit, and
  * that the two streams of one k-block touch disjoint cells: nothing the
    side stream writes is read or written by the bulk, and nothing the bulk
    writes is read by the side stream -- in the dense layout, and in the
    packed one-buffer layout (where cell (i,j) occupies P[i][j] and P[j][i]).
The GPU parity tests then check the kernels themselves against the oracle.
"""
import numpy as np
import pytest

import oracle
import pins
from distance_geometry_bound_amd import gen

BK, TILE = 64, 128
RATIO = TILE // BK


def fresh(a, b):
    return a // RATIO <= b // RATIO


class Model:
    def __init__(self, U0, L0, depth=2, skip_second=True):
        self.depth = depth                # bands run ahead on the side stream
        self.skip_second = skip_second    # False plants an overlap (self-test)
        self.n = U0.shape[0]
        self.U = pins.units(U0).copy()
        self.L = pins.units(L0).copy()
        self.TB = -(-self.n // BK)
        self.T = -(-self.n // TILE)

    def band(self, K):
        return list(range(K * BK, min(self.n, K * BK + BK)))

    def relax(self, i, j, k, U, L):
        """One round k on cell (i, j), reading row k for both operands
        (U[i,k] = U[k,i] by symmetry)."""
        u = min(U[i, j], U[k, i] + U[k, j])
        l = max(L[i, j], L[k, i] - U[k, j], L[k, j] - U[k, i])
        return u, l

    def phase12(self, K):
        """Phases 1 and 2 in one launch (k_diag_panel): every panel workgroup
        runs the rounds m of band K in order over the diagonal tile D and its
        panel tile R, each round reading row m of both as they stand before
        the round (D's column m is its row m by symmetry).  Panel tiles are
        read from their fresh orientation and written in both; D is written
        as a full square."""
        reads, writes = set(), set()
        kb = self.band(K)
        U, L = self.U, self.L
        D = {(a, b): (U[a, b], L[a, b]) for a in kb for b in kb}
        reads |= set(D)
        R = {}
        for J in range(self.TB):
            if J == K:
                continue
            for a in kb:
                for c in self.band(J):
                    src = (a, c) if fresh(K, J) else (c, a)
                    R[(a, c)] = (U[src], L[src])
                    reads.add(src)
        for m in kb:
            def rel(cell, row):
                (u, l), (cu, cl), (ru, rl) = cell, D[(m, row[0])], row[1]
                return min(u, cu + ru), max(l, cl - ru, rl - cu)
            newD = {(a, b): rel(D[(a, b)], (a, D[(m, b)])) for (a, b) in D}
            newR = {(a, c): rel(R[(a, c)], (a, R[(m, c)])) for (a, c) in R}
            D, R = newD, newR
        for (a, b), (u, l) in D.items():
            U[a, b], L[a, b] = u, l
            writes.add((a, b))
        for (a, c), (u, l) in R.items():
            U[a, c] = U[c, a] = u
            L[a, c] = L[c, a] = l
            writes |= {(a, c), (c, a)}
        return reads, writes

    def strip(self, K, A, skip):
        """Phase 3 of block K on row band A only: blocks (A, J) for every
        column band J other than K and `skip`, each in its fresh orientation."""
        reads, writes = set(), set()
        kb, ab = self.band(K), self.band(A)
        for J in range(self.TB):
            if J == K or J == skip:
                continue
            jb = self.band(J)
            reads |= {(k, x) for k in kb for x in ab + jb}
            for a in ab:
                for c in jb:
                    dst = (a, c) if fresh(A, J) else (c, a)
                    u, l = self.U[dst], self.L[dst]
                    reads.add(dst)
                    for k in kb:
                        u = min(u, self.U[k, a] + self.U[k, c])
                        l = max(l, self.L[k, a] - self.U[k, c], self.L[k, c] - self.U[k, a])
                    self.U[dst], self.L[dst] = u, l
                    writes.add(dst)
        return reads, writes

    def bulk(self, K, skip_bands):
        """Phase 3 of block K on the BK x BK quadrants of the upper TILE x TILE
        tiles, a quadrant in band K or in a skipped band left whole."""
        n = self.n
        reads, writes = set(), set()
        dead = set(self.band(K))
        for b in skip_bands:
            dead |= set(self.band(b))
        kb = self.band(K)
        new = {}
        for J in range(self.T):
            for I in range(J + 1):
                rows = [i for i in range(I * TILE, min(n, I * TILE + TILE)) if i not in dead]
                cols = [j for j in range(J * TILE, min(n, J * TILE + TILE)) if j not in dead]
                reads |= {(k, x) for k in kb for x in rows + cols}
                for i in rows:
                    for j in cols:
                        u, l = self.U[i, j], self.L[i, j]
                        reads.add((i, j))
                        for k in kb:
                            u = min(u, self.U[k, i] + self.U[k, j])
                            l = max(l, self.L[k, i] - self.U[k, j], self.L[k, j] - self.U[k, i])
                        new[(i, j)] = (u, l)
                        writes.add((i, j))
        for (i, j), (u, l) in new.items():
            self.U[i, j], self.L[i, j] = u, l
        return reads, writes

    def run(self):
        """The pass as the two streams issue it.  Two bands ahead:
          main  per K: [wait ready(K)] bulk(K) skipping bands K, K+1, K+2
          side  per K: strip(K, band K+1), phases 1-2 of K+1,
                       [wait bulk(K-1)] strip(K, band K+2 without band K+1),
                       record ready(K+1)
        One band ahead:
          main  per K: [wait ready(K)] bulk(K) skipping bands K, K+1
          side  per K: [wait bulk(K-1)] strip(K, band K+1), phases 1-2 of K+1,
                       record ready(K+1)
        Side work that bulk(K) may overlap is everything after ready(K) and
        before the side's wait for bulk(K); each such footprint must be
        disjoint from bulk(K)'s."""
        TB, deep = self.TB, self.depth == 2
        self.phase12(0)
        side = []          # (iteration, kind, reads, writes) in side-stream order
        bulks = {}
        ready_at = {}      # K -> index into `side` after which ready(K) is recorded
        wait_at = {}       # K -> index into `side` at which the side waits for bulk(K)
        for K in range(TB):
            # the model executes in an order consistent with both streams: the
            # side work of iteration K (it only reads state bulk(K) leaves alone)
            if K + 1 < TB:
                if not deep:
                    wait_at[K - 1] = len(side)
                side.append((K, "strip1", *self.strip(K, K + 1, None)))
                side.append((K, "phase12", *self.phase12(K + 1)))
            if deep and K + 2 < TB:
                wait_at[K - 1] = len(side)
                side.append((K, "strip2", *self.strip(K, K + 2, K + 1)))
            if K + 1 < TB:
                ready_at[K + 1] = len(side)
            ahead = (K + 1, K + 2) if deep and self.skip_second else (K + 1,)
            bulks[K] = self.bulk(K, [b for b in ahead if b < TB])
        sym = lambda cells: cells | {(j, i) for (i, j) in cells}
        for K, (br, bw) in bulks.items():
            lo = ready_at.get(K, 0)
            hi = wait_at.get(K, len(side))
            for it, kind, sr, sw in side[lo:hi]:
                tag = f"bulk({K}) vs {kind}({it})"
                assert not (sw & (br | bw)), tag + ": side writes what the bulk touches"
                assert not (bw & sr), tag + ": bulk writes what the side reads"
                # packed storage: a logical cell (i,j) lives in P[min][max] (U)
                # and P[max][min] (L), so a footprint becomes its symmetric closure
                assert not (sym(sw) & sym(br | bw)), tag + ": packed overlap (writes)"
                assert not (sym(bw) & sym(sr)), tag + ": packed overlap (reads)"
        n = self.n
        for i in range(n):
            for j in range(n):
                if (i // BK) // RATIO > (j // BK) // RATIO:
                    self.U[i, j], self.L[i, j] = self.U[j, i], self.L[j, i]
        return self.U, self.L


@pytest.mark.parametrize("n,depth", [(65, 2), (130, 2), (200, 2), (257, 2), (330, 2),
                                     (130, 1), (257, 1)])
def test_schedule_model_matches_oracle_and_streams_are_disjoint(n, depth):
    U0, L0, _ = gen.random_sound_bounds(n, seed=n, box=6.0 + n / 8)
    Ue, Le = oracle.smooth(U0, L0)
    Um, Lm = Model(U0, L0, depth=depth).run()
    assert np.array_equal(Um, pins.units(Ue))
    assert np.array_equal(Lm, pins.units(Le))


def test_schedule_model_detects_a_planted_overlap():
    # a bulk that forgets to leave band K+2 alone overlaps the side stream's
    # second strip: the footprint check must say so
    U0, L0, _ = gen.random_sound_bounds(200, seed=1, box=30.0)
    with pytest.raises(AssertionError, match="side writes what the bulk touches"):
        Model(U0, L0, skip_second=False).run()
