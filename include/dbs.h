/*
 * dbs.h -- C ABI of libdbs: distance-bound triangle smoothing on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (GPU Gems 2, Ch. 43 "GPU Computing for Protein Structure
 * Prediction", study notes):
 *   - §1: a molecule of n atoms is the complete graph K_n.  Pair (i,j) has
 *     an upper bound U[i,j] and a lower bound L[i,j] on its distance; the
 *     two bounds live in two dense n x n matrices.
 *   - §2: through an intermediate atom k the bounds tighten as
 *         U[i,j] <- min(U[i,j], U[i,k] + U[k,j])
 *         L[i,j] <- max(L[i,j], L[i,k] - U[k,j], L[k,j] - U[i,k])
 *     with the upper bounds tightened before the lower bounds read them.
 *   - §3: Floyd-Warshall order: rounds k = 0..n-1 in sequence, all pairs of
 *     a round independent, each round seeing the whole previous round.
 * One "pass" is all n rounds.  The library runs a pass on a batch of
 * independent molecules, in place.
 *
 * Data layout (all entry points): U and L are device pointers to
 * [batch][n][n] float32, row-major, contiguous, batch stride n*n.  The
 * caller allocates and owns them (e.g. torch tensors); the library keeps no
 * reference after a call returns and allocates no device memory.  U and L
 * must not overlap.  4-byte alignment is enough; 16-byte aligned rows take
 * vector loads.
 *
 * Preconditions for exact results (dbs_check tests the per-entry ones on
 * the device; none is tested by the smoothing calls):
 *   - U and L bit-for-bit symmetric, both diagonals +0.0;
 *   - every value finite, 0 <= L, a multiple of 2^-6 with |x| < 2^17, and
 *     no -0.0.  On that grid every sum and difference of two bounds is
 *     exact in fp32 (32-bit IEEE float, as in the notes' §6), so every
 *     schedule reaches the same bits;
 *   - the bounds are consistent: no L[i,j] exceeds the shortest-path upper
 *     bound between i and j.  Sound bounds (ones that contain the distances
 *     of some real coordinates) are always consistent.  A pass over
 *     inconsistent bounds still returns the exact shortest-path upper
 *     bounds, leaves L > U somewhere (which dbs_check on the result
 *     reports), and leaves the lower bounds unspecified.
 * Violating a precondition never causes an out-of-bounds access.
 *
 * Execution: every call validates its arguments on the host, then enqueues
 * kernels on `stream` (a hipStream_t; NULL means the null stream) and
 * returns without synchronising.  Faults of enqueued kernels surface at the
 * caller's next synchronisation, as usual in HIP.  Calls that touch the same
 * matrices must be ordered by the caller.  The library is thread-safe and
 * keeps no settings between calls: every choice a pass makes comes from its
 * arguments (dbs_options below).
 *
 * A blocked pass may also run part of its work on a second stream that the
 * library owns (see dbs_schedule): one such stream per device and caller
 * stream, created on the first pass enqueued on that caller stream and kept
 * for the life of the process, forked from and joined back into the caller's
 * stream with events.  Passes on different caller streams therefore share
 * no library stream and run independently.  (Past 64 caller streams on one
 * device, further streams get no second stream of their own and their
 * passes run on the caller's stream alone, with the same results.)  A pass
 * enqueued on a stream that is being captured into a HIP graph brings the
 * second stream into that capture and joins it back before returning.
 *
 * Status codes (every int-returning entry point):
 */
#ifndef DBS_H
#define DBS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DBS_OK 0           /* success                                         */
#define DBS_EINVAL (-1)    /* bad argument; nothing was enqueued              */
#define DBS_EDEVICE (-2)   /* no HIP device, or the current device is not gfx950 */
#define DBS_ELAUNCH (-3)   /* the HIP runtime rejected a launch               */
#define DBS_EUNSUPPORTED (-4) /* the requested algorithm cannot run this shape */

/* Algorithms for dbs_smooth_algo.  All of them produce the same bits. */
#define DBS_ALGO_AUTO 0    /* dbs_auto_algo: mostly LDS when it fits, else
                              BLOCKED                                         */
#define DBS_ALGO_PERK 1    /* one launch per round k (the notes' §3-§4 round
                              structure, in place instead of front/back buffers) */
#define DBS_ALGO_LDS 2     /* one workgroup per molecule runs the whole pass;
                              n <= dbs_lds_max_n()                            */
#define DBS_ALGO_BLOCKED 3 /* three-phase blocked pass (diagonal tile, panel,
                              remaining tiles), symmetric tile schedule       */

/*
 * Per-call options of a pass (dbs_smooth_opts, dbs_smooth_packed_opts,
 * dbs_smooth_profiled, dbs_schedule).  A NULL pointer means the defaults,
 * which dbs_options_init also writes:
 *   algo         DBS_ALGO_* (default DBS_ALGO_AUTO);
 *   directed     0: round to nearest (default); 1: directed rounding, see
 *                dbs_smooth_directed_range;
 *   lookahead    DBS_AUTO (default), or 0, 1, 2: force that look-ahead depth
 *                of a blocked pass (dbs_schedule);
 *   step_blocks  DBS_AUTO (default), or 1 .. 4: force that many k-blocks per
 *                step of a blocked pass.
 *   lead         DBS_AUTO (default), 0 or 1: where a blocked pass runs on the
 *                caller's stream alone in steps of one k-block, 1 takes the
 *                lead schedule and 0 the plain one (see dbs_schedule).
 *   infeasible   NULL (default), or a device pointer to `batch` uint32 words,
 *                one per molecule, owned by the caller (who clears them):
 *                the pass ORs DBS_INFEASIBLE_* bits into the word of a
 *                molecule whose bounds it finds inconsistent, that is, with
 *                L[i,j] > U[i,j] for some pair (the notes' §2: L and U only
 *                approach each other, so on consistent bounds L <= U holds
 *                at every step, and on inconsistent ones the output of a
 *                whole pass has L > U somewhere):
 *     DBS_INFEASIBLE_EARLY  seen during a blocked pass, where the diagonal
 *                tile of a k-block is closed (phase 1): some cell of that
 *                tile has L > U after the rounds of its k-block;
 *     DBS_INFEASIBLE_END    seen in the output of the call: some cell has
 *                L > U (a test of every cell, enqueued after the pass).
 *                For a whole pass it is set exactly for the inconsistent
 *                molecules; EARLY is never set without END.
 * The schedule fields only reorder independent cell updates: every value
 * gives the same results.  They exist for tests and tuning.  Any other value
 * of a field makes the call return DBS_EINVAL.  The options are read during
 * the call; the library keeps no pointer to them.
 */
#define DBS_AUTO (-1)
#define DBS_INFEASIBLE_EARLY 1u
#define DBS_INFEASIBLE_END 2u
typedef struct dbs_options {
  int32_t algo;
  int32_t directed;
  int32_t lookahead;
  int32_t step_blocks;
  int32_t lead;
  uint32_t *infeasible;
} dbs_options;

void dbs_options_init(dbs_options *opts);

/*
 * dbs_smooth_opts -- rounds k_begin..k_end-1 of a pass on U, L in place with
 * the given options: the general form of dbs_smooth, dbs_smooth_algo,
 * dbs_smooth_range, dbs_smooth_directed and dbs_smooth_directed_range
 * (which are this call with the matching options).  Arguments, algorithm
 * rules and errors as dbs_smooth_range; DBS_EINVAL for invalid options.
 *
 * dbs_smooth_packed_opts -- the same on the packed one-buffer layout P (see
 * dbs_smooth_packed_range): DBS_ALGO_PERK, DBS_ALGO_LDS and DBS_ALGO_BLOCKED
 * follow the rules of dbs_smooth_range; DBS_ALGO_AUTO takes the choice of
 * dbs_auto_algo (the packed layout and directed rounding: LDS whenever it
 * fits) when both ends are on k-block boundaries, else LDS when it fits,
 * else PERK.
 */
int dbs_smooth_opts(float *U, float *L, int64_t n, int64_t batch, int64_t k_begin,
                    int64_t k_end, void *stream, const dbs_options *opts);
int dbs_smooth_packed_opts(float *P, int64_t n, int64_t batch, int64_t k_begin,
                           int64_t k_end, void *stream, const dbs_options *opts);

/*
 * dbs_smooth -- one full smoothing pass (rounds k = 0..n-1) on every molecule,
 * in place.  Same as dbs_smooth_algo(..., DBS_ALGO_AUTO).
 *   U, L   device pointers, [batch][n][n] float32, read and written.
 *   n      atoms per molecule, >= 1 (n = 1 is a no-op).
 *   batch  number of molecules, >= 1.
 *   stream hipStream_t to enqueue on (NULL = null stream).
 * Returns DBS_OK, DBS_EINVAL (null pointer, n < 1, batch < 1, a size that
 * overflows 64-bit byte counts, n >= 2^26 (no such matrix fits in device
 * memory), or overlapping U/L), DBS_EDEVICE or DBS_ELAUNCH.
 */
int dbs_smooth(float *U, float *L, int64_t n, int64_t batch, void *stream);

/*
 * dbs_smooth_algo -- dbs_smooth with an explicit algorithm (DBS_ALGO_*).
 * DBS_EUNSUPPORTED if `algo` is DBS_ALGO_LDS and n > dbs_lds_max_n();
 * DBS_EINVAL for an unknown `algo`.
 */
int dbs_smooth_algo(float *U, float *L, int64_t n, int64_t batch, void *stream,
                    int algo);

/*
 * dbs_rounds -- rounds k_begin..k_end-1 of a pass on every molecule, one
 * launch per round (the per-round state after round k_end-1 equals that of
 * the notes' §4 front/back-buffer scheme).  0 <= k_begin <= k_end <= n,
 * else DBS_EINVAL.  k_begin == k_end enqueues nothing.
 */
int dbs_rounds(float *U, float *L, int64_t n, int64_t batch, int64_t k_begin,
               int64_t k_end, void *stream);

/*
 * dbs_round -- the single round k (the notes' §3-§4: one render pass per
 * intermediate atom), in place on every molecule.  0 <= k < n, else
 * DBS_EINVAL.  Equivalent to dbs_rounds(U, L, n, batch, k, k + 1, stream).
 */
int dbs_round(float *U, float *L, int64_t n, int64_t batch, int64_t k, void *stream);

/*
 * dbs_check -- test the per-entry preconditions on the device in O(n^2).
 * ORs DBS_CHECK_* bits into *d_flags (a device pointer to one uint32 that
 * the caller zeroes beforehand and reads after synchronising).  Run it on
 * the output of a pass to detect inconsistent bounds (DBS_CHECK_L_GT_U).
 * Same argument errors as dbs_smooth (d_flags must be non-null).
 */
int dbs_check(const float *U, const float *L, int64_t n, int64_t batch, void *stream,
              uint32_t *d_flags);

#define DBS_CHECK_ASYM 1u        /* U or L not bit-for-bit symmetric          */
#define DBS_CHECK_DIAG 2u        /* a diagonal entry is not +0.0              */
#define DBS_CHECK_NONFINITE 4u   /* NaN or infinity                           */
#define DBS_CHECK_L_GT_U 8u      /* L[i,j] > U[i,j]                           */
#define DBS_CHECK_L_NEG 16u      /* L[i,j] < 0                                */
#define DBS_CHECK_UNQUANT 32u    /* not a multiple of 2^-6                    */
#define DBS_CHECK_RANGE 64u      /* |x| >= 2^17                               */
#define DBS_CHECK_NEGZERO 128u   /* -0.0                                      */

/*
 * dbs_smooth_profiled -- one full pass as dbs_smooth_opts(U, L, n, batch, 0,
 * n, stream, opts), with every kernel launch bracketed by a HIP event pair
 * on the stream it is launched on; waits for the pass to finish and fills,
 * per kernel kind DBS_PROF_*, the number of launches (counts[kind]) and their
 * summed device time in milliseconds (ms[kind]).
 *   counts, ms  host arrays of DBS_PROF_KINDS elements, written by the call.
 * Same argument errors as dbs_smooth_opts; DBS_EINVAL if counts or ms is
 * null.  The events add a few microseconds per launch; for measurement only.
 */
int dbs_smooth_profiled(float *U, float *L, int64_t n, int64_t batch, void *stream,
                        const struct dbs_options *opts, int64_t *counts, double *ms);

#define DBS_PROF_ROUND 0   /* per-round kernel                                 */
#define DBS_PROF_SMALL 1   /* single-workgroup pass (whole molecule or diagonal tile) */
#define DBS_PROF_PANEL 2   /* blocked phase 2: panel tiles                     */
#define DBS_PROF_TILES 3   /* blocked phase 3: the bulk (every upper tile, less
                              the current and the next k-block's bands)       */
#define DBS_PROF_MIRROR 4  /* reserved, always 0: the last phase-3 launch of a
                              blocked pass writes the stale transposed copies */
#define DBS_PROF_STRIP 5   /* blocked phase 3 on the next k-block's band, run
                              ahead on a second stream                        */
#define DBS_PROF_FILL 6    /* restraints: placeholder fill                     */
#define DBS_PROF_SCATTER 7 /* restraints: interval scatter                     */
#define DBS_PROF_KINDS 8

/*
 * dbs_smooth_range -- rounds k_begin..k_end-1 of a pass, in place: the state
 * after the first rounds of a pass, or the rest of a pass resumed from it
 * (the notes' §5 experiment steps the number of finished rounds).
 * 0 <= k_begin <= k_end <= n, else DBS_EINVAL; k_begin == k_end is a no-op.
 * `algo`: DBS_ALGO_PERK runs one launch per round; DBS_ALGO_LDS (n <=
 * dbs_lds_max_n()) runs the range in one workgroup per molecule;
 * DBS_ALGO_BLOCKED needs both ends on k-block boundaries (multiples of
 * dbs_block_rounds(), or k_end == n; else DBS_EUNSUPPORTED); DBS_ALGO_AUTO
 * takes LDS when it fits, else BLOCKED when the ends allow it, else PERK.
 * Every algorithm gives the same bits.  The input must meet the
 * preconditions above (it does when it is the output of earlier ranges).
 */
int dbs_smooth_range(float *U, float *L, int64_t n, int64_t batch, int64_t k_begin,
                     int64_t k_end, void *stream, int algo);

/* Rounds per k-block of the blocked algorithm (64). */
int dbs_block_rounds(void);

/*
 * dbs_tightened -- which cells a smoothing step changed (the notes' §5 marks
 * the entries tightened relative to the initial bounds).  mask[b][i][j] = 1
 * if U1 or L1 differs bit for bit from U0 or L0 at (b,i,j), else 0.
 *   U0, L0, U1, L1  device [batch][n][n] float32, read only.
 *   mask            device [batch][n][n] uint8, written.
 * Same argument errors as dbs_smooth (mask must be non-null; the four inputs
 * may alias each other but not mask).
 */
int dbs_tightened(const float *U0, const float *L0, const float *U1, const float *L1,
                  int64_t n, int64_t batch, uint8_t *mask, void *stream);

/*
 * dbs_bounds_from_restraints -- dense bound matrices from a list of distance
 * restraints, the input the notes describe in §1: the experiment gives an
 * interval for some pairs; every other pair starts at a placeholder (the
 * molecular diameter above, about zero below).  For every molecule b:
 *   off the diagonal  L = unknown_L rounded down, U = unknown_U rounded up;
 *   on the diagonal   L = U = +0;
 *   then each restraint r of molecule b on the pair (i,j), i != j, tightens
 *   both (i,j) and (j,i):  L = max(L, round_down(max(lo[r], 0))),
 *                          U = min(U, round_up(hi[r])).
 * Rounding is outward to multiples of 2^-6 (down for lower bounds, up for
 * upper bounds), so the bounds stay sound and exactly representable.
 * Duplicate restraints of a pair combine to the tightest interval, in any
 * order.  Restraints with i == j are ignored.
 *   U, L        device [batch][n][n] float32, written (every entry).
 *   unknown_L, unknown_U  host values, finite, 0 <= unknown_L <= unknown_U
 *               < 2^17, else DBS_EINVAL.
 *   mol         device int32[count]: molecule of each restraint; may be NULL
 *               when batch == 1.
 *   ia, ja      device int32[count]: the two atoms of each restraint.
 *   lo, hi      device float32[count]: the interval of each restraint.
 *   count       number of restraints, >= 0 (0: placeholders only).
 *   d_status    device uint32 into which the kernel ORs DBS_RESTRAINT_* bits
 *               (caller zeroes; may be NULL).  A flagged restraint is skipped.
 * DBS_EINVAL for a null U, L, ia, ja, lo or hi (with count > 0), for a null
 * mol with batch > 1 and count > 0, or for the size checks of dbs_smooth.
 */
int dbs_bounds_from_restraints(float *U, float *L, int64_t n, int64_t batch,
                               float unknown_L, float unknown_U, const int32_t *mol,
                               const int32_t *ia, const int32_t *ja, const float *lo,
                               const float *hi, int64_t count, uint32_t *d_status,
                               void *stream);

#define DBS_RESTRAINT_INDEX 1u  /* molecule or atom index out of range        */
#define DBS_RESTRAINT_VALUE 2u  /* NaN or infinite value, lo > hi, hi < 0, or
                                   |value| >= 2^17                            */

/*
 * Directed rounding (the notes' §6: the smoothing is sensitive to the
 * precision of its float arithmetic).  On bounds that are not on the 2^-6
 * grid a sum or difference of two bounds is generally not representable in
 * float32, and round-to-nearest can move a bound past the value it stands
 * for (a shortened upper bound, a raised lower bound: an unsound result,
 * and even L > U on consistent input).  These entry points round every
 * upper-bound sum toward +inf and every lower-bound difference toward
 * -inf, so that each result is an upper (lower) bound on the exact value of
 * the path it comes from, and sound bounds stay sound.
 *
 * dbs_smooth_directed_range -- as dbs_smooth_range, with directed rounding.
 *   With DBS_ALGO_PERK and DBS_ALGO_LDS the result is bit for bit that of
 *   the rounds k_begin..k_end-1 in plain order with sums rounded up and
 *   differences rounded down.  DBS_ALGO_BLOCKED groups the same candidates
 *   differently, so its bits may differ from the plain order within the
 *   rounding error (relative 2^-23 per addition along a path); it is sound
 *   in the same sense.  On grid inputs (every operation exact) all
 *   algorithms give the bits of dbs_smooth_range.
 * dbs_smooth_directed -- a full pass, algorithm as dbs_smooth except that
 *   DBS_ALGO_AUTO keeps DBS_ALGO_LDS wherever it fits.
 * dbs_smooth_packed_directed_range -- dbs_smooth_packed_range with directed
 *   rounding (same algorithm choice, same remarks).
 * Preconditions and argument errors as dbs_smooth, except that values need
 * not lie on the 2^-6 grid (finite, 0 <= L, symmetric, zero diagonal).
 */
int dbs_smooth_directed(float *U, float *L, int64_t n, int64_t batch, void *stream);
int dbs_smooth_directed_range(float *U, float *L, int64_t n, int64_t batch, int64_t k_begin,
                              int64_t k_end, void *stream, int algo);
int dbs_smooth_packed_directed_range(float *P, int64_t n, int64_t batch, int64_t k_begin,
                                     int64_t k_end, void *stream);

/*
 * Packed storage (the notes' §6 keeps the two symmetric matrices as two
 * triangles): one [batch][n][n] float32 buffer P with P[i,j] = U[i,j] for
 * i < j, L[i,j] for i > j, and U[i,i] (= L[i,i] = 0) on the diagonal.  It
 * needs half the memory of the U, L pair.
 *
 * dbs_pack    -- P from symmetric U, L (reads U above and L below the diagonal).
 * dbs_unpack  -- U, L from P (U[i,j] = P[min,max], L[i,j] = P[max,min]).
 *   U, L, P device pointers, caller-owned; P may overlap neither U nor L.
 * dbs_smooth_packed_range -- rounds k_begin..k_end-1 of a pass on P in place;
 *   the result equals pack(smoothed U, L) bit for bit.  Algorithm as
 *   dbs_smooth_range with DBS_ALGO_AUTO: one workgroup per molecule for
 *   n <= dbs_lds_max_n(), else the blocked pass when both ends are on
 *   k-block boundaries (or k_end == n), else one launch per round.
 *   0 <= k_begin <= k_end <= n, else DBS_EINVAL.
 * dbs_smooth_packed -- a full pass (k = 0..n-1) on P.
 * dbs_check_packed -- dbs_check of the U, L pair that P stands for, without
 *   unpacking it: ORs DBS_CHECK_* bits into *d_flags (device pointer, zeroed
 *   by the caller).  DBS_CHECK_ASYM never appears (the pair is symmetric by
 *   construction); DBS_CHECK_DIAG means P[i][i] is not +0.0.
 * Same argument errors and preconditions as dbs_smooth (on the unpacked
 * U, L: the packed form is symmetric by construction).
 */
int dbs_pack(const float *U, const float *L, float *P, int64_t n, int64_t batch, void *stream);
int dbs_unpack(const float *P, float *U, float *L, int64_t n, int64_t batch, void *stream);
int dbs_smooth_packed(float *P, int64_t n, int64_t batch, void *stream);
int dbs_smooth_packed_range(float *P, int64_t n, int64_t batch, int64_t k_begin, int64_t k_end,
                            void *stream);
int dbs_check_packed(const float *P, int64_t n, int64_t batch, void *stream, uint32_t *d_flags);

/*
 * dbs_schedule -- the schedule a blocked pass (DBS_ALGO_BLOCKED) on the dense
 * layout takes for this shape under `opts` (NULL: the defaults);
 * dbs_schedule_packed the same for the packed layout (dbs_smooth_packed and
 * its variants).  The rules below are the packed layout's; the dense layout
 * differs where noted [dense]:
 *   *lookahead    how many steps it updates ahead on its second stream:
 *     0  no look-ahead: a single k-block or phase-3 tile; fewer than 256
 *        phase-3 tiles x molecules (the bulk launch is shorter than the band
 *        strip it would hide); more than 256 phase 1-2 workgroups (the
 *        panel launch fills the chip by itself); or, below 1024 tiles x
 *        molecules, where the pass takes the lead schedule (below).  Without look-ahead, a
 *        batch of two or more molecules with more than 256 phase 1-2
 *        workgroups ((k-blocks - 1) x molecules) splits into two halves, one
 *        on the caller's stream and one on the second stream, so that one
 *        half's phase 1-2 launches run beside the other half's phase 3;
 *        otherwise the pass uses the caller's stream alone;
 *     1  otherwise, below 1024 tiles x molecules: steps of one k-block;
 *     2  from 1024 tiles x molecules [dense: and for a single molecule from
 *        800 tiles].  In the dense layout phase 1 of a block is then the
 *        closure of its diagonal tile alone (one workgroup per molecule)
 *        and phase 2 a product from it, both on the second stream.
 *   *step_blocks  k-blocks per step: where it runs two steps ahead, 4 from
 *     3000 phase-3 tiles x molecules, 3 from 1800, else 2 [dense: a single
 *     molecule below 1024 tiles 1; a batch 1 below 1600 tiles, 2 below
 *     3000, else 4]; otherwise 1.  A
 *     step of w blocks is blocked Floyd-Warshall with 64w atoms per phase-3
 *     launch; its panel (the rows of the step's bands, final for all of its
 *     rounds) is built from the 64-wide phases 1-2 and phase-3 strips.
 *   *lead  1 where the pass takes the lead schedule, else 0.  It applies to
 *     a pass without look-ahead in steps of one k-block and n below 23 040
 *     (the phase-3 quadrants of a launch fit one grid dimension), and is
 *     chosen where a batch has more than 256 phase 1-2 workgroups
 *     ((k-blocks - 1) x molecules), and from 256 to 511 phase-3 tiles x
 *     molecules [dense: for a batch from 64 to 1023 tiles x molecules, for
 *     a single molecule from 64 to 511].  Per k-block K it runs two launches on the caller's stream:
 *     phase 2 of K as a product with K's diagonal tile, closed the launch
 *     before, and one launch that holds phase 3 of K and, beside it, phase 1
 *     of K + 1 (phase 3 of K on the diagonal tile of K + 1, then its
 *     closure).  A batch on the lead schedule does not split over two
 *     streams.
 * opts->lookahead, opts->step_blocks and opts->lead, when not DBS_AUTO,
 * replace these choices (the depth stays 0 for a single k-block or tile).
 * Every schedule gives the same results.  Any output pointer may be NULL.
 * Returns DBS_OK, or DBS_EINVAL for n < 1, batch < 1 or invalid options.
 */
int dbs_schedule(int64_t n, int64_t batch, const struct dbs_options *opts, int32_t *lookahead,
                 int32_t *step_blocks, int32_t *lead);
int dbs_schedule_packed(int64_t n, int64_t batch, const struct dbs_options *opts,
                        int32_t *lookahead, int32_t *step_blocks, int32_t *lead);

/* dbs_schedule's automatic look-ahead depth and step width for this shape
   (DBS_EINVAL for n < 1 or batch < 1). */
int dbs_lookahead_bands(int64_t n, int64_t batch);
int dbs_step_blocks(int64_t n, int64_t batch);

/* Largest n the LDS algorithm accepts. */
int dbs_lds_max_n(void);

/* The algorithm DBS_ALGO_AUTO picks for a whole round-to-nearest pass in the
 * dense layout of this shape (n, batch >= 1): BLOCKED from n = 128 with at
 * most 16 molecules and above dbs_lds_max_n(), else LDS (the packed layout
 * and directed rounding take LDS whenever it fits). */
int dbs_auto_algo(int64_t n, int64_t batch);

/* Static description of a status code (never NULL). */
const char *dbs_strerror(int status);

/* Library version, 0xMMmmpp. */
int dbs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DBS_H */
