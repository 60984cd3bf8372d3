/*
 * oracle.c -- CPU reference for distance-bound triangle smoothing.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent checker that the
 * GPU library is compared against.  Only the test-suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it; the GPU library never
 * includes, links or calls anything here, and this file shares no code with
 * it.
 *
 * What it computes follows GPU Gems 2, Ch. 43 "GPU Computing for Protein
 * Structure Prediction" (study notes):
 *   - §1: a molecule of n atoms is the complete graph K_n; edge (i,j) carries
 *     an upper bound U[i,j] and a lower bound L[i,j], stored as two dense
 *     n x n matrices.
 *   - §2: with an intermediate atom k the upper bound shrinks to
 *     min(U[i,j], U[i,k] + U[k,j]) and the lower bound grows to
 *     max(L[i,j], L[i,k] - U[k,j], L[k,j] - U[i,k]); the upper bounds are
 *     tightened before the lower bounds use them.
 *   - §3: Floyd-Warshall order: the rounds k = 0..n-1 run one after the
 *     other, every pair (i,j) of a round is independent, and a round sees the
 *     complete result of the previous one.
 *   - §4: a round reads the previous round's matrices and writes fresh ones
 *     (front/back buffers swapped after the round).
 *   - §6: arithmetic is 32-bit IEEE float, and the result is sensitive to
 *     its precision.
 *
 * So one round k is written out literally: first the upper sweep over every
 * pair, reading the front U; then the lower sweep over every pair, reading
 * the front L and the upper bounds the round has just produced.  Nothing is
 * reordered or fused.  OpenMP splits the rows of a sweep over threads, which
 * changes no arithmetic (every pair is computed by the same expression).
 *
 * Directed rounding (dbs_oracle_rounds_directed): the same rounds with every
 * upper-bound sum rounded toward +infinity and every lower-bound difference
 * toward -infinity (the C rounding mode of each sweep, set in every OpenMP
 * thread), so that, on inputs that are not on an exact grid, the results
 * stay sound bounds: an upper bound is never rounded below the sum it
 * stands for, a lower bound never above its difference.
 *
 * Layout: U and L are [batch][n][n] float32, row-major, batch stride n*n.
 * Return codes: 0 ok, -1 bad argument, -2 out of host memory.
 */
#include <fenv.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_VERSION 0x000100

static int nthreads(int threads)
{
#ifdef _OPENMP
    return threads > 0 ? threads : omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}

/* One Floyd-Warshall round with intermediate atom k (§2, §3, §4).
   directed: round the upper sweep's sums up and the lower sweep's
   differences down (each thread sets, then restores, its own mode). */
static void one_round(const float *Uf, const float *Lf, float *Ub, float *Lb,
                      int64_t n, int64_t k, int threads, int directed)
{
#pragma omp parallel num_threads(threads)
    {
        int64_t i, j;
        if (directed)
            fesetround(FE_UPWARD);
        /* upper bounds first: U[i,j] <- min(U[i,j], U[i,k] + U[k,j]) */
#pragma omp for schedule(static)
        for (i = 0; i < n; ++i) {
            for (j = 0; j < n; ++j) {
                float keep = Uf[i * n + j];
                float path = Uf[i * n + k] + Uf[k * n + j];
                Ub[i * n + j] = path < keep ? path : keep;
            }
        }
        /* (the loop's barrier: every upper bound of the round is written) */
        if (directed)
            fesetround(FE_DOWNWARD);
        /* then lower bounds, from this round's upper bounds:
           L[i,j] <- max(L[i,j], L[i,k] - U[k,j], L[k,j] - U[i,k]) */
#pragma omp for schedule(static)
        for (i = 0; i < n; ++i) {
            for (j = 0; j < n; ++j) {
                float best = Lf[i * n + j];
                float a = Lf[i * n + k] - Ub[k * n + j];
                float b = Lf[k * n + j] - Ub[i * n + k];
                if (a > best) best = a;
                if (b > best) best = b;
                Lb[i * n + j] = best;
            }
        }
        if (directed)
            fesetround(FE_TONEAREST);
    }
}

/* Rounds k_begin..k_end-1 of one pass, in place on every molecule. */
static int run_rounds(float *U, float *L, int64_t n, int64_t batch,
                      int64_t k_begin, int64_t k_end, int threads, int directed)
{
    if (!U || !L || n < 1 || batch < 1 || k_begin < 0 || k_end > n || k_begin > k_end)
        return -1;
    if (n > (int64_t)1 << 31)
        return -1;
    const size_t nn = (size_t)n * (size_t)n;
    int t = nthreads(threads);
    float *spare_u = (float *)malloc(nn * sizeof(float));
    float *spare_l = (float *)malloc(nn * sizeof(float));
    if (!spare_u || !spare_l) {
        free(spare_u);
        free(spare_l);
        return -2;
    }
    for (int64_t b = 0; b < batch; ++b) {
        float *Umol = U + (size_t)b * nn, *Lmol = L + (size_t)b * nn;
        float *fu = Umol, *fl = Lmol;           /* front: last finished round */
        float *bu = spare_u, *bl = spare_l;     /* back: the round being written */
        for (int64_t k = k_begin; k < k_end; ++k) {
            one_round(fu, fl, bu, bl, n, k, t, directed);
            float *tu = fu, *tl = fl;
            fu = bu; fl = bl;
            bu = tu; bl = tl;
        }
        if (fu != Umol) {
            memcpy(Umol, fu, nn * sizeof(float));
            memcpy(Lmol, fl, nn * sizeof(float));
        }
    }
    free(spare_u);
    free(spare_l);
    return 0;
}

int dbs_oracle_rounds(float *U, float *L, int64_t n, int64_t batch,
                      int64_t k_begin, int64_t k_end, int threads)
{
    return run_rounds(U, L, n, batch, k_begin, k_end, threads, 0);
}

/* The same rounds with directed rounding (sums up, differences down). */
int dbs_oracle_rounds_directed(float *U, float *L, int64_t n, int64_t batch,
                               int64_t k_begin, int64_t k_end, int threads)
{
    return run_rounds(U, L, n, batch, k_begin, k_end, threads, 1);
}

/* One full pass (rounds 0..n-1) on every molecule. */
int dbs_oracle_smooth(float *U, float *L, int64_t n, int64_t batch, int threads)
{
    return dbs_oracle_rounds(U, L, n, batch, 0, n, threads);
}

/* Number of threads a call with threads <= 0 uses. */
int dbs_oracle_max_threads(void) { return nthreads(0); }

int dbs_oracle_version(void) { return ORACLE_VERSION; }
