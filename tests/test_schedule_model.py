"""CPU model of the blocked pass's schedule (test code only).

The GPU pass (csrc/blocked.hip) runs in steps of W k-blocks of BK = 64
atoms (W = 1 one step ahead, 2 to 4 two steps ahead, any of 1..4 when forced),
per step
  panel    the rows of the step's bands made final for all of its rounds:
           for each block b+j of the step in turn, phases 1+2 of it (the
           rounds of band b+j over the diagonal tile and, in the same loop,
           over each panel tile of the band, one workgroup per panel tile,
           panel tiles read from their fresh orientation (upper TILE x TILE
           region) and written in both orientations), then block b+j on the
           step's other bands (one strip; the bands before b+j, which are
           panel rows already, in both orientations);
  phase 3  the bands of the next steps first (strips, on a second stream,
           followed there by the next step's panel), and every other live
           cell of the upper TILE x TILE tiles (the bulk, on the caller's
           stream, as BK x BK quadrants: a quadrant in a band of the step or
           of a step run ahead is skipped whole, which leaves exactly the
           live cells modelled here);
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
    """Band pair (a, b) is kept current: a quadrant of an upper TILE x TILE
    tile, or an upper or diagonal quadrant of a diagonal tile (tiles are
    RATIO whole bands wide, so these are the pairs a <= b)."""
    return a // RATIO < b // RATIO or (a // RATIO == b // RATIO and a <= b)


def stale_cells(n):
    """Cells whose band pair is not kept current (mirrored at the end)."""
    band = np.arange(n) // BK
    return band[:, None] > band[None, :]


def test_fresh_quadrants_are_the_upper_band_pairs():
    # the kernels test freshness as a <= b on band indices; the tile form
    # above and the stale set of the final mirror say the same
    for a in range(4 * RATIO + 1):
        for b in range(4 * RATIO + 1):
            assert fresh(a, b) == (a <= b), (a, b)
    n = 5 * BK + 7
    band = np.arange(n) // BK
    fr = np.array([[fresh(a, b) for b in band] for a in band])
    assert np.array_equal(stale_cells(n), ~fr)


class Model:
    """Footprints are boolean n x n masks of the cells a launch reads or
    writes.  Within a launch the relaxations are evaluated per block with
    numpy; the values are exact int64 units, so a min or max over a block's
    candidates does not depend on their order."""

    def __init__(self, U0, L0, depth=2, skip_second=True, W=None, fresh_read=True,
                 product_panels=None):
        self.depth = depth                # steps run ahead on the side stream
        self.W = W if W else (2 if depth == 2 else 1)   # k-blocks per step
        self.skip_second = skip_second    # False plants an overlap (self-test)
        self.fresh_read = fresh_read      # False plants a stale read (self-test)
        # two steps ahead (dense layout), phases 1-2 of a block are the
        # closure of its diagonal tile and a product launch; else one
        # k_diag_panel launch
        self.product_panels = depth == 2 if product_panels is None else product_panels
        self.n = U0.shape[0]
        self.U = pins.units(U0).copy()
        self.L = pins.units(L0).copy()
        self.TB = -(-self.n // BK)
        self.T = -(-self.n // TILE)

    def band(self, K):
        return np.arange(K * BK, min(self.n, K * BK + BK))

    def mask(self):
        return np.zeros((self.n, self.n), dtype=bool)

    def phase12(self, K):
        """Phases 1 and 2 in one launch (k_diag_panel): every panel workgroup
        runs the rounds m of band K in order over the diagonal tile D and its
        panel tile R, each round reading row m of both as they stand before
        the round (D's column m is its row m by symmetry).  Panel tiles are
        read from their fresh orientation and written in both; D is written
        as a full square."""
        reads, writes = self.mask(), self.mask()
        kb = self.band(K)
        U, L = self.U, self.L
        ix = np.ix_(kb, kb)
        Du, Dl = U[ix].copy(), L[ix].copy()
        reads[ix] = True
        cols, Ru, Rl = [], [], []
        for J in range(self.TB):
            if J == K:
                continue
            jb = self.band(J)
            if fresh(K, J):
                Ru.append(U[np.ix_(kb, jb)]), Rl.append(L[np.ix_(kb, jb)])
                reads[np.ix_(kb, jb)] = True
            else:
                Ru.append(U[np.ix_(jb, kb)].T), Rl.append(L[np.ix_(jb, kb)].T)
                reads[np.ix_(jb, kb)] = True
            cols.append(jb)
        cols = np.concatenate(cols)
        Ru, Rl = np.concatenate(Ru, axis=1), np.concatenate(Rl, axis=1)
        for m in range(len(kb)):
            du, dl = Du[m].copy(), Dl[m].copy()      # D[m][*] = D[*][m]
            ru, rl = Ru[m].copy(), Rl[m].copy()      # R[m][*]
            Du = np.minimum(Du, du[:, None] + du[None, :])
            Dl = np.maximum(Dl, np.maximum(dl[:, None] - du[None, :], dl[None, :] - du[:, None]))
            Ru = np.minimum(Ru, du[:, None] + ru[None, :])
            Rl = np.maximum(Rl, np.maximum(dl[:, None] - ru[None, :], rl[None, :] - du[:, None]))
        U[ix], L[ix] = Du, Dl
        writes[ix] = True
        U[np.ix_(kb, cols)], L[np.ix_(kb, cols)] = Ru, Rl
        U[np.ix_(cols, kb)], L[np.ix_(cols, kb)] = Ru.T, Rl.T
        writes[np.ix_(kb, cols)] = True
        writes[np.ix_(cols, kb)] = True
        return reads, writes

    def close(self, Z):
        """The rounds of band Z over the diagonal tile (Z,Z) alone, in order
        (phase 1; one workgroup per molecule): (reads, writes)."""
        reads, writes = self.mask(), self.mask()
        zb = self.band(Z)
        ix = np.ix_(zb, zb)
        reads[ix] = True
        Du, Dl = self.U[ix].copy(), self.L[ix].copy()
        for m in range(len(zb)):
            du, dl = Du[m].copy(), Dl[m].copy()
            Du = np.minimum(Du, du[:, None] + du[None, :])
            Dl = np.maximum(Dl, np.maximum(dl[:, None] - du[None, :], dl[None, :] - du[:, None]))
        self.U[ix], self.L[ix] = Du, Dl
        writes[ix] = True
        return reads, writes

    def product(self, K, Kend=None):
        """Phase 2 of K from the closed diagonal tile: (reads, writes) per
        panel workgroup (Kend: the end of the pass or range)."""
        Kend = self.TB if Kend is None else Kend
        kb = self.band(K)
        dix = np.ix_(kb, kb)
        Du, Dl = self.U[dix].copy(), self.L[dix].copy()
        parts, new = [], []
        for J in range(self.TB):
            if J == K:
                continue
            reads, writes = self.mask(), self.mask()
            reads[dix] = True
            jb = self.band(J)
            if fresh(K, J) or not self.fresh_read:
                Ru, Rl = self.U[np.ix_(kb, jb)].copy(), self.L[np.ix_(kb, jb)].copy()
                reads[np.ix_(kb, jb)] = True
            else:
                Ru, Rl = self.U[np.ix_(jb, kb)].T.copy(), self.L[np.ix_(jb, kb)].T.copy()
                reads[np.ix_(jb, kb)] = True
            # min / max over the atoms m: D*[a][m] with R[m][c] as read
            bu = (Du[:, :, None] + Ru[None, :, :]).min(1)
            bl = np.maximum((Dl[:, :, None] - Ru[None, :, :]).max(1),
                            (Rl[None, :, :] - Du[:, :, None]).max(1))
            nu, nl = np.minimum(Ru, bu), np.maximum(Rl, bl)
            new.append((kb, jb, nu, nl, J))
            writes[np.ix_(kb, jb)] = True
            writes[np.ix_(jb, kb)] = True
            parts.append((f"product({K}) tile {J}", reads, writes))
        for kb_, jb, nu, nl, J in new:
            self.U[np.ix_(kb_, jb)], self.L[np.ix_(kb_, jb)] = nu, nl
            # right of the diagonal the other copy stays stale until the
            # panel of J rewrites it (a range ending before J writes it here)
            if J < K or J >= Kend:
                self.U[np.ix_(jb, kb_)], self.L[np.ix_(jb, kb_)] = nu.T, nl.T
        return parts

    def mirror(self, excl=()):
        """The last launch's mirror: the stale cells of the quadrants that
        launch computes (every band but `excl`, the bands of its own step)
        take their transposes.  The stale cells of the `excl` bands keep what
        the panels wrote: they must be current already."""
        stale = stale_cells(self.n)
        band = np.arange(self.n) // BK
        inx = np.isin(band, list(excl))
        stale &= ~(inx[:, None] | inx[None, :])
        self.U[stale], self.L[stale] = self.U.T[stale], self.L.T[stale]
        return self.U, self.L

    @staticmethod
    def disjoint(parts):
        sym = lambda m: m | m.T
        for i, (ta, ra, wa) in enumerate(parts):
            for tb, rb, wb in parts[i + 1:]:
                tag = f"{ta} vs {tb}"
                assert not np.any(wa & (rb | wb)), tag + ": overlap"
                assert not np.any(wb & ra), tag + ": overlap"
                assert not np.any(sym(wa) & sym(rb | wb)), tag + ": packed overlap"
                assert not np.any(sym(wb) & sym(ra)), tag + ": packed overlap"

    def _phase3(self, kb, rows, cols):
        """Candidates of the atoms kb for the cells rows x cols, from the
        atom rows (U[i,k] = U[k,i]): (best U, best L) blocks."""
        Ur, Uc = self.U[np.ix_(kb, rows)], self.U[np.ix_(kb, cols)]
        Lr, Lc = self.L[np.ix_(kb, rows)], self.L[np.ix_(kb, cols)]
        bu = (Ur[:, :, None] + Uc[:, None, :]).min(0)
        bl = np.maximum((Lr[:, :, None] - Uc[:, None, :]).max(0),
                        (Lc[:, None, :] - Ur[:, :, None]).max(0))
        return bu, bl

    def strip(self, Ks, A, excl, both=False):
        """Phase 3 of the blocks Ks (their atoms in order) on row band A only:
        blocks (A, J) for every column band J outside `excl`, each in its
        fresh orientation, and with `both` in the other one too."""
        reads, writes = self.mask(), self.mask()
        kb = np.concatenate([self.band(K) for K in Ks])
        ab = self.band(A)
        for J in range(self.TB):
            if J in excl:
                continue
            jb = self.band(J)
            reads[np.ix_(kb, np.concatenate([ab, jb]))] = True
            bu, bl = self._phase3(kb, ab, jb)
            dst = np.ix_(ab, jb) if fresh(A, J) else np.ix_(jb, ab)
            cur_u, cur_l = (self.U[dst], self.L[dst]) if fresh(A, J) else (self.U[dst].T, self.L[dst].T)
            reads[dst] = True
            nu, nl = np.minimum(cur_u, bu), np.maximum(cur_l, bl)
            if fresh(A, J):
                self.U[dst], self.L[dst] = nu, nl
            else:
                self.U[dst], self.L[dst] = nu.T, nl.T
            writes[dst] = True
            if both:
                other = np.ix_(jb, ab) if fresh(A, J) else np.ix_(ab, jb)
                if fresh(A, J):
                    self.U[other], self.L[other] = nu.T, nl.T
                else:
                    self.U[other], self.L[other] = nu, nl
                writes[other] = True
        return reads, writes

    def bulk(self, Ks, skip_bands):
        """Phase 3 of the blocks Ks on the BK x BK quadrants kept current (of
        the upper TILE x TILE tiles, less the lower-left one of each diagonal
        tile), a quadrant in a band of Ks or in a skipped band left whole."""
        n = self.n
        reads, writes = self.mask(), self.mask()
        live = np.ones(n, dtype=bool)
        for b in list(Ks) + list(skip_bands):
            live[self.band(b)] = False
        kb = np.concatenate([self.band(K) for K in Ks])
        new = []
        for B in range(self.TB):
            for A in range(self.TB):
                if not fresh(A, B):
                    continue
                ta, tb = self.band(A), self.band(B)
                rows, cols = ta[live[ta]], tb[live[tb]]
                if len(rows) == 0 or len(cols) == 0:
                    continue
                reads[np.ix_(kb, np.concatenate([rows, cols]))] = True
                cell = np.ix_(rows, cols)
                reads[cell] = True
                bu, bl = self._phase3(kb, rows, cols)
                new.append((cell, np.minimum(self.U[cell], bu), np.maximum(self.L[cell], bl)))
                writes[cell] = True
        for cell, nu, nl in new:
            self.U[cell], self.L[cell] = nu, nl
        return reads, writes

    def block_panel(self, K):
        """Phases 1-2 of block K as (kind, reads, writes) launches: the
        closure of the diagonal tile, then the product launch (whose panel
        workgroups must be disjoint), or one k_diag_panel launch."""
        if not self.product_panels:
            return [("phase12", *self.phase12(K))]
        out = [("close", *self.close(K))]
        parts = self.product(K)
        self.disjoint(parts)
        reads, writes = self.mask(), self.mask()
        for _, r, w in parts:
            reads |= r
            writes |= w
        out.append(("product", reads, writes))
        return out

    def step_panel(self, Ks):
        """The rows of the step's bands Ks final for all of its rounds, as
        (kind, reads, writes) launches.  On the GPU each block's strip over
        the other bands is one launch (row band Ks[r] leaves out the columns
        of the bands before it, whose blocks those rows hold)."""
        out = []
        for K in Ks:
            out.extend(self.block_panel(K))
            for r, A in enumerate(Ks):
                if A != K:
                    out.append(("panel-strip",
                                *self.strip([K], A, set(Ks[:r]) | {K}, both=A < K)))
        return out

    def run(self):
        """The pass as the two streams issue it, in steps of W k-blocks (W = 2
        two steps ahead, else 1); S(t) = the bands of step t.  Two steps ahead:
          main  per t: [wait ready(t)] bulk(t) skipping S(t), S(t+1), S(t+2)
          side  per t: strip(t, rows S(t+1)), panel of step t+1,
                       [wait bulk(t-1)] strip(t, rows S(t+2) without
                       columns S(t+1)), record ready(t+1)
        One step ahead:
          main  per t: [wait ready(t)] bulk(t) skipping S(t), S(t+1)
          side  per t: [wait bulk(t-1)] strip(t, rows S(t+1)), panel of
                       step t+1, record ready(t+1)
        A strip over the two row bands of a step leaves the first band out of
        the second's columns (those cells are the first band's).  Side work
        that bulk(t) may overlap is everything after ready(t) and before the
        side's wait for bulk(t); each such footprint must be disjoint from
        bulk(t)'s."""
        TB, deep, W = self.TB, self.depth == 2, self.W
        steps = [list(range(b, min(b + W, TB))) for b in range(0, TB, W)]
        NS = len(steps)
        self.step_panel(steps[0])
        side = []          # (iteration, kind, reads, writes) in side-stream order
        bulks = {}
        ready_at = {}      # t -> index into `side` after which ready(t) is recorded
        wait_at = {}       # t -> index into `side` at which the side waits for bulk(t)

        def strip_rows(t, rows, excl_to):
            for r, A in enumerate(rows):
                excl = set(range(steps[t][0], excl_to + r))
                side.append((t, "strip", *self.strip(steps[t], A, excl)))

        for t in range(NS):
            # the model executes in an order consistent with both streams: the
            # side work of iteration t (it only reads state bulk(t) leaves alone)
            if t + 1 < NS:
                if not deep:
                    wait_at[t - 1] = len(side)
                strip_rows(t, steps[t + 1], steps[t][-1] + 1)
                side.extend((t, kind, r, w) for kind, r, w in self.step_panel(steps[t + 1]))
            if deep and t + 2 < NS:
                wait_at[t - 1] = len(side)
                strip_rows(t, steps[t + 2], steps[t + 1][-1] + 1)
            if t + 1 < NS:
                ready_at[t + 1] = len(side)
            ahead = steps[t + 1:t + 3] if deep and self.skip_second else steps[t + 1:t + 2]
            bulks[t] = self.bulk(steps[t], [b for s_ in ahead for b in s_])
        sym = lambda m: m | m.T
        for t, (br, bw) in bulks.items():
            lo = ready_at.get(t, 0)
            hi = wait_at.get(t, len(side))
            for it, kind, sr, sw in side[lo:hi]:
                tag = f"bulk({t}) vs {kind}({it})"
                assert not np.any(sw & (br | bw)), tag + ": side writes what the bulk touches"
                assert not np.any(bw & sr), tag + ": bulk writes what the side reads"
                # packed storage: a logical cell (i,j) lives in P[min][max] (U)
                # and P[max][min] (L), so a footprint becomes its symmetric closure
                assert not np.any(sym(sw) & sym(br | bw)), tag + ": packed overlap (writes)"
                assert not np.any(sym(bw) & sym(sr)), tag + ": packed overlap (reads)"
        return self.mirror(steps[-1])


@pytest.mark.parametrize("n,depth,W", [(65, 2, None), (130, 2, None), (200, 2, None),
                                       (257, 2, None), (330, 2, None), (130, 1, None),
                                       (257, 1, None), (330, 2, 3), (330, 2, 4), (257, 1, 3),
                                       (200, 1, 2), (520, 2, 3), (520, 2, 4), (700, 2, 4),
                                       (520, 1, 4), (257, 2, 1), (330, 2, 1), (520, 2, 1)])
def test_schedule_model_matches_oracle_and_streams_are_disjoint(n, depth, W):
    U0, L0, _ = gen.random_sound_bounds(n, seed=n, box=6.0 + n / 8)
    Ue, Le = oracle.smooth(U0, L0)
    Um, Lm = Model(U0, L0, depth=depth, W=W).run()
    assert np.array_equal(Um, pins.units(Ue))
    assert np.array_equal(Lm, pins.units(Le))


@pytest.mark.parametrize("n,W", [(200, None), (330, 3), (520, 4)])
def test_schedule_model_two_ahead_with_round_panels(n, W):
    # the packed layout's two-step look-ahead keeps the 64-round phase 1-2
    # launch; the footprint checks are the same
    U0, L0, _ = gen.random_sound_bounds(n, seed=n + 1, box=6.0 + n / 8)
    Ue, Le = oracle.smooth(U0, L0)
    Um, Lm = Model(U0, L0, depth=2, W=W, product_panels=False).run()
    assert np.array_equal(Um, pins.units(Ue))
    assert np.array_equal(Lm, pins.units(Le))


def test_schedule_model_detects_a_planted_overlap():
    # a bulk that forgets to leave the bands of step t+2 alone overlaps the
    # side stream's second strip: the footprint check must say so
    # (n = 260: five k-blocks, so step 0 has a step two ahead)
    U0, L0, _ = gen.random_sound_bounds(260, seed=1, box=36.0)
    with pytest.raises(AssertionError, match="side writes what the bulk touches"):
        Model(U0, L0, skip_second=False).run()


def test_schedule_model_detects_a_missing_panel_orientation():
    # the panel of a block must leave its atom rows current: the bulk and the
    # strips read them, and a product that writes only the fresh orientation
    # leaves the row orientation of the tiles left of the diagonal stale
    class Broken(Model):
        def product(self, K):
            U, L = self.U.copy(), self.L.copy()
            parts = super().product(K)
            kb = self.band(K)
            for J in range(self.TB):
                if J != K:
                    jb = self.band(J)
                    old = np.ix_(jb, kb) if fresh(K, J) else np.ix_(kb, jb)
                    self.U[old], self.L[old] = U[old], L[old]
            return parts

    U0, L0, _ = gen.random_sound_bounds(520, seed=520, box=6.0 + 520 / 8)
    Ue, Le = oracle.smooth(U0, L0)
    Um, Lm = Broken(U0, L0, depth=2, W=4).run()
    assert not (np.array_equal(Um, pins.units(Ue)) and np.array_equal(Lm, pins.units(Le)))


@pytest.mark.parametrize("lead", [False, True])
def test_schedule_model_detects_a_tile_level_mirror(lead):
    # the bulk leaves the lower-left quadrant of each diagonal tile to the
    # final mirror; a mirror of whole tiles only keeps those quadrants as
    # their own bands' panels left them, which misses the oracle
    def tile_mirror(self, excl=()):
        band = np.arange(self.n) // BK
        tile = band // RATIO
        inx = np.isin(band, list(excl))
        stale = (tile[:, None] > tile[None, :]) & ~(inx[:, None] | inx[None, :])
        self.U[stale], self.L[stale] = self.U.T[stale], self.L.T[stale]
        return self.U, self.L

    base = LeadModel if lead else Model
    Broken = type("Broken", (base,), {"mirror": tile_mirror})
    U0, L0, _ = gen.random_sound_bounds(330, seed=331, box=6.0 + 330 / 8)
    Ue, Le = oracle.smooth(U0, L0)
    Um, Lm = Broken(U0, L0).run()
    assert not (np.array_equal(Um, pins.units(Ue)) and np.array_equal(Lm, pins.units(Le)))


def test_schedule_model_detects_a_product_before_its_closure():
    # two steps ahead the panel of a block is the product from its closed
    # diagonal tile; a product from the tile as it stood misses the oracle
    class Broken(Model):
        def block_panel(self, K):
            self.product(K)
            return [("product", self.mask(), self.mask()), ("close", *self.close(K))]

    U0, L0, _ = gen.random_sound_bounds(330, seed=330, box=6.0 + 330 / 8)
    Ue, Le = oracle.smooth(U0, L0)
    Um, Lm = Broken(U0, L0, depth=2).run()
    assert not (np.array_equal(Um, pins.units(Ue)) and np.array_equal(Lm, pins.units(Le)))


class LeadModel(Model):
    """The one-stream lead schedule (one k-block per step), per k-block K:
      product(K)  phase 2 of K with the diagonal tile (K,K) already closed:
                  every panel tile (K,J), J != K, read from its fresh
                  orientation, becomes the min/max over the atoms m of band K
                  of D*[a][m] (+/-) R[m][c] with R as read (one workgroup per
                  tile), written in its row orientation and, for J < K, in
                  the other (its fresh one) too;
      lead(K, Z)  in one launch: phase 3 of K on every quadrant outside band
                  K and outside the diagonal tile (Z,Z), Z = K + 1 (the bulk
                  workgroups), and phase 3 of K on (Z,Z) followed by the
                  rounds of band Z over it (the closure workgroup);
    after a first launch that closes (K0,K0) alone.  Checked: the oracle's
    result, and that within a launch no workgroup writes what another one
    reads or writes (the two parts of a lead launch, and the panel tiles of a
    product launch), in the dense layout and under the packed layout's
    symmetric closure of the footprints."""

    def __init__(self, U0, L0, skip_diag=True, fresh_read=True):
        super().__init__(U0, L0, depth=0, W=1, fresh_read=fresh_read)
        self.skip_diag = skip_diag      # False plants an overlap (self-test)

    def closure_part(self, K, Z):
        reads, writes = self.mask(), self.mask()
        zb = self.band(Z)
        ix = np.ix_(zb, zb)
        reads[ix] = True
        if K >= 0:
            kb = self.band(K)
            reads[np.ix_(kb, zb)] = True
            bu, bl = self._phase3(kb, zb, zb)
            self.U[ix], self.L[ix] = np.minimum(self.U[ix], bu), np.maximum(self.L[ix], bl)
        self.close(Z)
        writes[ix] = True
        return reads, writes

    def bulk_part(self, K, Z):
        """Phase 3 of K on the quadrants of the upper tiles outside band K and
        outside (Z,Z), as separate quadrant workgroups."""
        reads, writes = self.mask(), self.mask()
        kb = self.band(K)
        new = []
        for A in range(self.TB):
            for B in range(self.TB):
                if not fresh(A, B) or A == K or B == K:
                    continue
                if self.skip_diag and A == Z and B == Z:
                    continue
                ab, jb = self.band(A), self.band(B)
                reads[np.ix_(kb, np.concatenate([ab, jb]))] = True
                cell = np.ix_(ab, jb)
                reads[cell] = True
                bu, bl = self._phase3(kb, ab, jb)
                new.append((cell, np.minimum(self.U[cell], bu), np.maximum(self.L[cell], bl)))
                writes[cell] = True
        for cell, nu, nl in new:
            self.U[cell], self.L[cell] = nu, nl
        return reads, writes

    def run(self, K0=0, K1=None):
        """The k-blocks K0 .. K1-1 (a whole pass by default)."""
        K1 = self.TB if K1 is None else K1
        self.closure_part(-1, K0)
        for K in range(K0, K1):
            self.disjoint(self.product(K, K1))
            Z = K + 1 if K + 1 < K1 else -1
            parts = [(f"bulk({K})", *self.bulk_part(K, Z))]
            if Z >= 0:
                # the closure workgroup computes from the state before the
                # launch, as the bulk part does; the model runs it after the
                # bulk part, which is equivalent when the two are disjoint
                parts.append((f"closure({Z})", *self.closure_part(K, Z)))
            self.disjoint(parts)
        return self.mirror({K1 - 1})


@pytest.mark.parametrize("n", [65, 127, 128, 129, 200, 257, 330, 450])
def test_lead_schedule_matches_oracle_and_launches_are_disjoint(n):
    U0, L0, _ = gen.random_sound_bounds(n, seed=3 * n, box=6.0 + n / 8)
    Ue, Le = oracle.smooth(U0, L0)
    Um, Lm = LeadModel(U0, L0).run()
    assert np.array_equal(Um, pins.units(Ue))
    assert np.array_equal(Lm, pins.units(Le))


@pytest.mark.parametrize("n,K0,K1", [(200, 0, 1), (200, 0, 2), (200, 1, 3), (330, 0, 2),
                                      (330, 2, 4), (330, 1, 6), (450, 3, 5)])
def test_lead_ranges_match_oracle(n, K0, K1):
    # a range of k-blocks K0 .. K1-1 from the state after the rounds before
    # it: the result, both copies of every cell, equals the oracle's rounds
    # (a product leaves the stale copy of (K, J), K < J, only where J is
    # inside the range)
    U0, L0, _ = gen.random_sound_bounds(n, seed=5 * n + K0, box=6.0 + n / 8)
    Us, Ls = oracle.rounds(U0, L0, 0, K0 * BK)
    Ue, Le = oracle.rounds(U0, L0, 0, min(n, K1 * BK))
    Um, Lm = LeadModel(Us, Ls).run(K0, K1)
    assert np.array_equal(Um, pins.units(Ue)) and np.array_equal(Lm, pins.units(Le))


def test_lead_model_detects_a_range_that_leaves_a_copy_stale():
    # a product that skips the other copy of every tile right of the
    # diagonal, also where the range ends before that tile's band is a
    # panel, leaves a stale copy in the range's result
    class Broken(LeadModel):
        def product(self, K, Kend=None):
            return super().product(K, self.TB)

    n = 330
    U0, L0, _ = gen.random_sound_bounds(n, seed=9, box=6.0 + n / 8)
    Ue, Le = oracle.rounds(U0, L0, 0, 2 * BK)
    Um, Lm = Broken(U0, L0).run(0, 2)
    assert not (np.array_equal(Um, pins.units(Ue)) and np.array_equal(Lm, pins.units(Le)))


def test_lead_model_detects_a_planted_overlap():
    # a lead launch whose bulk part also takes the next diagonal tile writes
    # what the closure workgroup reads and writes
    U0, L0, _ = gen.random_sound_bounds(200, seed=2, box=31.0)
    with pytest.raises(AssertionError, match="overlap"):
        LeadModel(U0, L0, skip_diag=False).run()


def test_lead_model_detects_a_stale_panel_read():
    # a product that reads panel tiles in the row orientation even where the
    # symmetric schedule left that copy stale misses the oracle
    U0, L0, _ = gen.random_sound_bounds(330, seed=4, box=47.0)
    Ue, Le = oracle.smooth(U0, L0)
    Um, Lm = LeadModel(U0, L0, fresh_read=False).run()
    assert not (np.array_equal(Um, pins.units(Ue)) and np.array_equal(Lm, pins.units(Le)))
