// small.hip -- a whole Floyd-Warshall pass over a small symmetric block in
// one workgroup.
//
// Works on dense U, L or on the packed one-buffer layout (PK; U == L == P).
// Used (a) for whole molecules with n <= kSmallMaxN, one workgroup per
// molecule (the batched path for many small molecules), and (b) for the
// diagonal tile of the blocked pass.  Rounds k run in order (GPU Gems 2,
// Ch. 43 notes, §3); every cell of a round is independent.
//
// Layout: the block is split into 4x4 cell tiles.  By symmetry only tiles on
// or above the diagonal are held, one per thread, in registers (32 values);
// tiles on the diagonal hold both halves.  Round k needs, for every cell
// (i,j), the values U/L[i,k] and U/L[k,j]; both are entries of row k
// (U[i,k] = U[k,i]).  The threads holding row k (tile row k/4) or, below the
// diagonal, column k (tile column k/4) publish it to a double-buffered LDS
// vector, one barrier later every thread reads its 4+4 operands from it and
// relaxes its 16 cells.  LDS traffic is O(n) per round; the cells never leave
// registers until the pass ends.
#include "dbs_internal.h"

namespace dbs {
namespace {

constexpr int kMaxG = kSmallMaxN / 4;  // tiles per side

template <bool kUseRow>
__device__ __forceinline__ void publish(float (&u)[4][4], float (&l)[4][4], int r, float *vu,
                                        float *vl) {
  // kUseRow: publish row r of the tile; else column r (cells (c, r)).
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    vu[c] = kUseRow ? u[r][c] : u[c][r];
    vl[c] = kUseRow ? l[r][c] : l[c][r];
  }
}

template <bool PK, bool RU>
__global__ __launch_bounds__(1024) void k_small(float *U, float *L, int64_t ld, int64_t mstride,
                                                int64_t off, int m, int k_lo, int k_hi,
                                                int64_t batch) {
  __shared__ float vu[2][4 * kMaxG];
  __shared__ float vl[2][4 * kMaxG];

  rounding_prologue<RU>();
  const int G = (m + 3) >> 2;
  const int tiles = G * (G + 1) / 2;
  const int t = threadIdx.x;
  const bool active = t < tiles;
  // t -> (ty, tx), ty <= tx, row-major over the upper triangle of tiles
  int ty = 0, rem = t;
  if (active) {
    while (rem >= G - ty) {
      rem -= G - ty;
      ++ty;
    }
  }
  const int tx = ty + rem;
  const int i0 = ty * 4, j0 = tx * 4;

  for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
    float *Ub = U + b * mstride + off;
    float *Lb = L + b * mstride + off;
    float u[4][4], l[4][4];
    if (active) {
      // element offsets from the row starts of the tile's rows and columns
      // (packed: U of (i,j) at row min(i,j), L at row max(i,j)); they fit
      // 32 bits (the launcher checks m * ld).  The tile corner is laundered
      // so that the offsets are formed per molecule, not hoisted out of the
      // molecule loop and kept live.
      int li0 = i0, lj0 = j0;
      asm volatile("" : "+v"(li0), "+v"(lj0));
      int ib[4], jb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ib[q] = (li0 + q) * (int)ld;
        jb[q] = (lj0 + q) * (int)ld;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = li0 + r, j = lj0 + c;
          const bool in = i < m && j < m;
          const int gu = !PK || i < j ? ib[r] + j : jb[c] + i;
          const int gl = !PK || i > j ? ib[r] + j : jb[c] + i;
          u[r][c] = in ? Ub[gu] : kInf;
          l[r][c] = in ? Lb[gl] : 0.0f;
        }
    }

    for (int kb = k_lo / 4; kb < G; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int k = kb * 4 + r;
        if (k >= k_hi) break;  // uniform across the workgroup
        if (k < k_lo) continue;
        const int buf = k & 1;
        if (active) {
          if (ty == kb)
            publish<true>(u, l, r, &vu[buf][j0], &vl[buf][j0]);
          else if (tx == kb)
            publish<false>(u, l, r, &vu[buf][i0], &vl[buf][i0]);
        }
        __syncthreads();
        if (active) {
          float cu[4], cl[4], ru[4], rl[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            cu[q] = vu[buf][i0 + q];
            cl[q] = vl[buf][i0 + q];
            ru[q] = vu[buf][j0 + q];
            rl[q] = vl[buf][j0 + q];
          }
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c)
              relax1<RU>(u[a][c], l[a][c], cu[a], cl[a], ru[c], rl[c]);
        }
      }
    }

    if (active) {
      // the store offsets are re-derived here (laundered tile corner), not
      // kept live through the rounds
      int wi0 = i0, wj0 = j0;
      asm volatile("" : "+v"(wi0), "+v"(wj0));
      int ib[4], jb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ib[q] = (wi0 + q) * (int)ld;
        jb[q] = (wj0 + q) * (int)ld;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = wi0 + r, j = wj0 + c;
          l[r][c] = lower_out<RU>(l[r][c]);
          if (PK) {
            // one slot each for U(i,j) and L(i,j); a diagonal tile holds both
            // (i,j) and (j,i) with the same values, the diagonal stays 0
            if (i < m && j < m && i != j) {
              Ub[i < j ? ib[r] + j : jb[c] + i] = u[r][c];
              Lb[i > j ? ib[r] + j : jb[c] + i] = l[r][c];
            }
          } else if (i < m && j < m) {
            Ub[ib[r] + j] = u[r][c];
            Lb[ib[r] + j] = l[r][c];
            if (wi0 != wj0) {
              Ub[jb[c] + i] = u[r][c];
              Lb[jb[c] + i] = l[r][c];
            }
          }
        }
    }
    // the LDS vectors are rewritten by the next molecule's first rounds only
    // after every thread has passed at least one more barrier
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_small_block(float *U, float *L, int64_t ld, int64_t mstride, int64_t off,
                              int m, int k_lo, int k_hi, int64_t batch, hipStream_t s,
                              Prof *prof, unsigned flags) {
  if (m <= 1 || k_lo >= k_hi) return hipSuccess;
  // the kernel's element offsets within a molecule are 32-bit
  if ((int64_t)m * (ld + 1) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int G = (m + 3) / 4;
  const int tiles = G * (G + 1) / 2;
  const int threads = (tiles + 63) / 64 * 64;
  const unsigned grid = (unsigned)(batch < 1048576 ? batch : 1048576);
  const bool pk = flags & kPacked, ru = flags & kDirected;
  auto kern = pk ? (ru ? k_small<true, true> : k_small<true, false>)
                 : (ru ? k_small<false, true> : k_small<false, false>);
  return launch(prof, kProfSmall, kern, dim3(grid), dim3(threads), s, U, L, ld, mstride, off, m,
                k_lo, k_hi, batch);
}

hipError_t launch_small(float *U, float *L, int64_t n, int64_t batch, int k_lo, int k_hi,
                        hipStream_t s, Prof *prof, unsigned flags) {
  return launch_small_block(U, L, n, n * n, 0, (int)n, k_lo, k_hi, batch, s, prof, flags);
}

}  // namespace dbs
