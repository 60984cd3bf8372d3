// blocked.hip -- one smoothing pass as blocked Floyd-Warshall in three
// phases per block of BK intermediate atoms.
//
// The pages give the per-round update (GPU Gems 2, Ch. 43 notes, §2-§3); the
// blocked order is ours.  Under the exactness preconditions it reaches the
// same bits as the plain round order: the fused round is Floyd-Warshall on a
// graph with no negative cycle, every candidate is exact on the 2^-6 grid, so
// any partition of the rounds into blocks yields the same shortest paths.
//
// For k-block K (atoms k0..k0+bK-1, "band K"):
//   phase 1  the diagonal tile (K,K): a full pass over it, rounds in order;
//   phase 2  every other tile of band K ("panel"): rounds in order, over
//            the diagonal tile's rows (phases 1 and 2 run together in
//            k_diag_panel, one workgroup per panel tile; or phase 1 as the
//            closure of the diagonal tile alone and phase 2 as a product
//            from it, k_lead and k_product);
//   phase 3  every remaining cell: all bK rounds at once from the finished
//            panel (k_quads / k_quads_packed: the bulk on 64x64 quadrants;
//            k_strip: given row bands alone, when running ahead or inside
//            a step's panel).  This is where 1 - O(BK/n) of the work is.
// A step of w k-blocks (launch_blocked) is the same with 64w atoms in
// phase 3; its panel is built from the phase 1-2 kernel and strips.
//
// Symmetric schedule.  U and L stay exactly symmetric, so only the cells of
// TILE x TILE tiles (I,J) with I < J, and of the upper and diagonal BK x BK
// quadrants of the tiles (I,I), are kept current ("fresh"); the rest goes
// stale and gets its final values from the last launch that writes its
// transposes (the last bulk launch of a pass writes each quadrant whose
// mirror is stale at both positions; the panels are written in both
// orientations anyway).  Phase 3 therefore does half the work of a dense
// schedule.  It
// reads its operands U/L[i,k] and U/L[k,j] from row k only (U[i,k] = U[k,i]),
// so phase 2 must leave all of row band K current: it updates each panel
// tile from whichever orientation is fresh and writes its row orientation
// and its fresh one (the products leave a stale copy right of the diagonal,
// which nothing reads before the panel of that band rewrites it).
//
// Phase 3: a 256-thread workgroup owns a 64x64 block, each thread a 4x4
// register tile (512 threads with 4x2 tiles when a launch has fewer blocks
// than CUs); the panel rows of the k-block are staged through LDS.  No
// matrix cores: min-plus is not a multiply-add contraction.
#include <map>
#include <memory>
#include <mutex>
#include <utility>

#include "dbs.h"
#include "dbs_internal.h"

namespace dbs {
namespace {

constexpr int BK = 64;          // atoms per k-block (phases 1 and 2 tile size)
constexpr int TILE = 128;       // freshness granularity: tiles I <= J are kept current
constexpr int RATIO = TILE / BK;
constexpr int KC = 16;          // atoms per LDS chunk in phase 3
// Phase-3 tiles (times molecules) from which the pass runs two steps ahead
// (the packed layout's crossover, and the dense one's for a batch, below
// which a dense batch takes the lead schedule; measured, one step ahead
// against two in two-block steps: n5632, 990 tiles, 9.78-9.80 against
// 10.14-10.17 ms; n6144, 1176 tiles, 12.15 against 11.59 ms).
constexpr int64_t kDeepTiles = 1024;
// A single molecule in the dense layout runs two steps ahead, in steps of
// one k-block, from this many tiles (measured, two steps of one block
// against one step: n5120, 820 tiles, 7.51-7.54 against 7.58-7.70 ms;
// n5376, 903 tiles, 8.07 against 8.36; n5632, 990 tiles, 9.06-9.14 against
// 9.54-9.58; n4864, 741 tiles, 7.07 against 6.54).
constexpr int64_t kDeepTilesSingle = 800;
// k-blocks per step when running two steps ahead: 4 from kStep4Tiles phase-3
// tiles (times molecules), 3 from kStep3Tiles, else 2.  Wider steps spread a
// bulk launch's fixed costs over more atoms but leave more bands to the
// strips and lengthen the side stream's chain (measured, dense ms, widths
// 2/3/4: n6144 11.8/13.2/14.0; n8192 25.5/24.9/25.8; n10240 49.5/47.8/47.0;
// n12288 73.9/72.6/71.1).
constexpr int64_t kStep4Tiles = 3000, kStep3Tiles = 1800;
// A batch in the dense layout takes narrower steps: one k-block below
// kStep2TilesBatch tiles, two below kStep4Tiles (measured, widths 1/2/3:
// 128 x n500, 1280 tiles, 1.50/1.59/-; 32 x n1024, 1152, 2.31/2.38/-;
// 8 x n2048, 1088, 3.78/4.02/-; 64 x n700, 1344, 1.82/1.97/-; 64 x n1024,
// 2304, 4.13/4.04/4.27; 16 x n2048, 2176, 7.24/6.72/7.20; 128 x n700, 2688,
// 3.37/3.26/3.38; 256 x n500, 2560, 2.85/2.79/2.76 ms).
constexpr int64_t kStep2TilesBatch = 1600;
// Below this many phase-3 tiles (times molecules) a bulk launch is too short
// to hide the band strip that running ahead puts on the critical path.
constexpr int64_t kAheadTiles = 256;
// Above this many phase 1-2 workgroups the panel launch fills the chip by
// itself, and running it beside the bulk gains nothing (one per CU).
constexpr int64_t kPanelFill = 256;
// Phase 1-2 workgroups (times molecules) up to which the dense phase 1-2
// launch splits each panel tile's columns over several workgroups.
constexpr int64_t kSplitPanelFill = 256;
// A batch in the dense layout takes the lead schedule from kLeadTilesMin up
// to kDeepTiles tiles (measured, lead against one step ahead: 4 x n2048, 544
// tiles, 2.32 against 2.50-2.52 ms; 8 x n1536, 624, 1.93 against 2.06; 16 x
// n1024, 576, 1.23 against 1.41-1.42; 2 x n3072, 600, 3.62 against 3.71-3.72;
// 6 x n2048, 816, 3.00 against 3.23).  Otherwise,
// between these many phase-3 tiles (times molecules) a one-stream pass takes
// the lead schedule even where its phase 1-2 launch would not fill the chip:
// there a bulk launch is long enough to hide the closure of the next
// diagonal tile, and the product is shorter than a phase 1-2 launch.
// Measured (median of 10 passes, lead against the plain or one-step
// schedule): n1024 (36 tiles) 1.09x, n1280 (55) 1.08x, 4 x n500 (40)
// 1.07x; 2 x n1024 (72) 0.95x, n1536 (78) 0.94x, 8 x n500 (80) 0.89x,
// 16 x n300 (96) 0.92x, n1792 (105) 0.95x, n2048 (136) 0.88x, n3072 (300)
// 0.81x, 32 x n500 (320) 0.76x; n4096 (528) 1.02x.  The packed layout, whose
// product keeps 4x4 cells, from kLeadTilesMinPacked (packed passes, lead
// against plain: n1536 (78) 1.26x, 32 x n256 (96) 1.21x, n2048 (136) 1.07x,
// 4 x n1024 (144) 1.08x, n2560 (210) 0.99x, n3072 (300) 0.94x, 8 x n1024
// (288) 0.90x).
constexpr int64_t kLeadTilesMin = 64, kLeadTilesMinPacked = 256, kLeadTilesMax = 512;
constexpr int kThreads = 256;

// The side-stream kernels (strips, and phases 1-2 of the next blocks) are
// on the critical path of a step whenever they share compute units with the
// bulk kernel: their waves take instruction-issue priority over its waves on
// the same SIMD (wave priority only; the streams keep the default priority).
__device__ __forceinline__ void critical_path_priority() { __builtin_amdgcn_s_setprio(2); }

// Quadrant (band a, band b) is fresh under the symmetric schedule: it lies in
// an upper TILE x TILE tile, or is an upper or diagonal quadrant of a diagonal
// tile; with tiles RATIO whole bands wide, that is a <= b
__device__ __forceinline__ bool fresh(int64_t a, int64_t b) { return a <= b; }

// The early test of the infeasibility option, where phase 1 has closed a
// diagonal tile (bZ atoms; thread (ty, tx) holds RT x CT of its cells): a
// cell with L > U marks the molecule's word with DBS_INFEASIBLE_EARLY.  On
// consistent bounds L <= U holds at every step (L only rises and U only
// falls towards the closure), so the mark is never wrong.
template <int RT, int CT>
__device__ __forceinline__ void flag_infeasible(uint32_t *word, int bZ, int ty, int tx,
                                                const float (&u)[RT][CT],
                                                const float (&l)[RT][CT]) {
  bool bad = false;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < CT; ++q)
      bad |= ty * RT + r < bZ && tx * CT + q < bZ && l[r][q] > u[r][q];
  if (bad) atomicOr(word, DBS_INFEASIBLE_EARLY);
}

// ---------------------------------------------------------------- helpers
// Four consecutive entries p[0..3]; entry q is used only if q < cnt, else the
// neutral value `fill`.  VEC: p is 16-byte aligned and cnt is 0 or >= 4.
// Branch-free: an entry that is not used is read from `safe` (any valid,
// 16-byte aligned address) and replaced afterwards, so that the compiler can
// issue a run of these loads back to back instead of one at a time.
template <bool VEC>
__device__ __forceinline__ float4 load4(const float *p, int cnt, float fill, const float *safe) {
  if (VEC) {
    const float4 v = *reinterpret_cast<const float4 *>(cnt >= 4 ? p : safe);
    return cnt >= 4 ? v : make_float4(fill, fill, fill, fill);
  }
  const float x0 = *(cnt > 0 ? p : safe), x1 = *(cnt > 1 ? p + 1 : safe);
  const float x2 = *(cnt > 2 ? p + 2 : safe), x3 = *(cnt > 3 ? p + 3 : safe);
  return make_float4(cnt > 0 ? x0 : fill, cnt > 1 ? x1 : fill, cnt > 2 ? x2 : fill,
                     cnt > 3 ? x3 : fill);
}

__device__ __forceinline__ int clamp4(int64_t left) { return left < 0 ? 0 : (left > 4 ? 4 : (int)left); }

// Two consecutive entries, as load4.  VEC: p is 8-byte aligned and cnt is 0
// or >= 2.
template <bool VEC>
__device__ __forceinline__ float2 load2(const float *p, int cnt, float fill, const float *safe) {
  if (VEC) {
    const float2 v = *reinterpret_cast<const float2 *>(cnt >= 2 ? p : safe);
    return cnt >= 2 ? v : make_float2(fill, fill);
  }
  const float x0 = *(cnt > 0 ? p : safe), x1 = *(cnt > 1 ? p + 1 : safe);
  return make_float2(cnt > 0 ? x0 : fill, cnt > 1 ? x1 : fill);
}

// S consecutive entries (S = 2 or 4) as an array.
template <int S>
struct Seg {
  float v[S];
};

template <bool VEC, int S>
__device__ __forceinline__ Seg<S> load_seg(const float *p, int64_t left, float fill,
                                           const float *safe) {
  Seg<S> r;
  const int cnt = left < 0 ? 0 : (left > S ? S : (int)left);
  if constexpr (S == 4) {
    const float4 x = load4<VEC>(p, cnt, fill, safe);
    r.v[0] = x.x; r.v[1] = x.y; r.v[2] = x.z; r.v[3] = x.w;
  } else {
    static_assert(S == 2, "segments of 2 or 4 entries");
    const float2 x = load2<VEC>(p, cnt, fill, safe);
    r.v[0] = x.x; r.v[1] = x.y;
  }
  return r;
}

// ---------------------------------------------------------------- packed blocks
// Packed layout: logical cell (i, j) has U at P[min][max] and L at P[max][min].
// A BK x BK block of logical cells (r0 + a, c0 + c), a < rows, c < cols, is
// read into u/l[S][S] of thread (ty, tx) (rows S*ty.., columns S*tx..) from
// the row segments P[r0+a][c0..] and the column segments P[c0+c][r0..], both
// as S-wide vectors.  Right of the diagonal (r0 < c0) the row segments hold U; left
// of it L; on a diagonal block (r0 == c0) it is decided per cell, and the
// diagonal itself reads P[i][i] for both.  Cells outside get the neutral
// values.
template <bool VEC, int S = 4>
__device__ __forceinline__ void packed_block_load(const float *P, int64_t n, int64_t r0,
                                                  int64_t c0, int rows, int cols, int ty, int tx,
                                                  float (&u)[S][S], float (&l)[S][S]) {
  // all 2S loads are issued before any value is unpacked
  Seg<S> x[S], y[S];
#pragma unroll
  for (int r = 0; r < S; ++r) {
    const int a = ty * S + r;
    x[r] = load_seg<VEC, S>(P + (r0 + a) * n + c0 + tx * S, a < rows ? cols - tx * S : 0, 0.0f,
                            P);
  }
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int c = tx * S + q;
    y[q] = load_seg<VEC, S>(P + (c0 + c) * n + r0 + ty * S, c < cols ? rows - ty * S : 0, 0.0f,
                            P);
  }
#pragma unroll
  for (int r = 0; r < S; ++r)
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const int a = ty * S + r, c = tx * S + q;
      const float d = x[r].v[q], t = y[q].v[r];  // P[r0+a][c0+c], P[c0+c][r0+a]
      const bool in = a < rows && c < cols;
      const bool upper = r0 < c0 || (r0 == c0 && a < c);
      const bool lower = r0 > c0 || (r0 == c0 && a > c);
      u[r][q] = in ? (lower ? t : d) : kInf;
      l[r][q] = in ? (upper ? t : d) : 0.0f;
    }
}

// The inverse of packed_block_load (the diagonal of a diagonal block is not
// written: its single slot holds U[i][i]).  On a diagonal block cells (a, c)
// and (c, a) write the same two slots with equal values.
// `bad` (may be null) accumulates whether a stored cell has L > U.
template <int S = 4>
__device__ __forceinline__ void packed_block_store(float *P, int64_t n, int64_t r0, int64_t c0,
                                                   int rows, int cols, int ty, int tx,
                                                   const float (&u)[S][S],
                                                   const float (&l)[S][S],
                                                   bool *bad = nullptr) {
#pragma unroll
  for (int r = 0; r < S; ++r)
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const int a = ty * S + r, c = tx * S + q;
      if (a >= rows || c >= cols || (r0 == c0 && a == c)) continue;
      if (bad) *bad |= l[r][q] > u[r][q];
      const bool upper = r0 < c0 || (r0 == c0 && a < c);
      P[(r0 + a) * n + c0 + c] = upper ? u[r][q] : l[r][q];
      P[(c0 + c) * n + r0 + a] = upper ? l[r][q] : u[r][q];
    }
}

// ---------------------------------------------------------------- phases 1 and 2
// Phases 1 and 2 of k-block K in one launch.  Workgroup J (one per k-block
// tile other than K; grid.y = molecules) holds the diagonal tile D = (K, K)
// and its panel tile R = (K, J) in registers and runs the rounds m of band K
// in order over both.  Row m of D and of R is published through LDS
// (double-buffered, one barrier per round); column m of D equals its row m
// by symmetry:
//   D[a][b] <- relax(D[a][b], D[a][m], D[m][b])
//   R[a][c] <- relax(R[a][c], D[a][m], R[m][c]).
// These are the plain rounds of the notes' §3 restricted to the rows of band
// K, so they reach the values of finishing D first and the panel from it
// (exactly, on the 2^-6 grid).  Every workgroup repeats D's rounds: that
// costs less than a launch of its own on the critical path of the pass.
// The last workgroup writes D back.  Cells outside the matrix start neutral and stay
// neutral (every candidate through them is +inf for U and <= 0 for L).
//
// Thread (ty, tx) owns an S x S cell block of D and of R (rows S*ty.., columns
// S*tx..), so the workgroup has (BK/S)^2 threads.  S = 2 (1024 threads, four
// waves per SIMD) hides the latency of the rounds best when the kernel has
// the chip to itself; S = 4 (256 threads, a footprint like a phase-3
// workgroup) gets compute units while the bulk of phase 3 runs (the packed
// layout's two-step look-ahead).
template <int S>
constexpr int panel_threads() { return (BK / S) * (BK / S); }

template <bool VEC, bool PK, bool RU, int S>
__global__ __launch_bounds__(panel_threads<S>()) void k_diag_panel(float *__restrict__ U,
                                                                   float *__restrict__ L,
                                                                   int64_t n, int64_t batch,
                                                                   int64_t K,
                                                                   uint32_t *infeasible) {
  constexpr int NT = BK / S;  // threads per side
  __shared__ __align__(16) float dvu[2][BK], dvl[2][BK];  // row m of D
  __shared__ __align__(16) float rvu[2][BK], rvl[2][BK];  // row m of R
  // With 1024 threads (S = 2) the panel tile's copy in the other orientation
  // is read and written through an LDS tile, as row segments instead of one
  // or two floats per lane down a column: tt[.][c][a] = R[a][c] (U and L;
  // packed, the one slot written there).  The 256-thread variant runs beside
  // the bulk of phase 3 and keeps its LDS footprint small.
  constexpr bool kStageT = S == 2;
  __shared__ float tt[kStageT ? (PK ? 1 : 2) : 1][kStageT ? BK : 1][kStageT ? BK + 1 : 1];

  rounding_prologue<RU>();
  critical_path_priority();
  const int tid = threadIdx.x, ty = tid / NT, tx = tid % NT;
  int64_t J = blockIdx.x;
  if (J >= K) ++J;
  const int64_t k0 = K * BK, j0 = J * BK;
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  const bool rowor = fresh(K, J);
  // the last workgroup of the molecule writes D back: every other one was
  // dispatched before it and reads D at its start, long before that
  // workgroup's 64 rounds are done
  const bool writes_d = blockIdx.x == gridDim.x - 1;
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = PK ? Ub : L + b * nn;

    float du[S][S], dl[S][S];  // D[S*ty + r][S*tx + q]
    float u[S][S], l[S][S];    // R[S*ty + r][S*tx + q] = cell (k0 + S*ty + r, j0 + S*tx + q)
    if (PK) {
      packed_block_load<VEC, S>(Ub, n, k0, k0, bK, bK, ty, tx, du, dl);
      packed_block_load<VEC, S>(Ub, n, k0, j0, bK, bJ, ty, tx, u, l);
    } else {
      // all loads are issued before any value is unpacked
      Seg<S> xu[S], xl[S], yu[S], yl[S];
#pragma unroll
      for (int r = 0; r < S; ++r) {
        const int a = ty * S + r;
        const int64_t g = (k0 + a) * n + k0 + tx * S;
        const int64_t left = a < bK ? bK - tx * S : 0;
        xu[r] = load_seg<VEC, S>(Ub + g, left, kInf, Ub);
        xl[r] = load_seg<VEC, S>(Lb + g, left, 0.0f, Lb);
      }
      // the panel tile from its fresh orientation: R[a][c] = M[k0+a][j0+c]
      // (row segments), else M[j0+c][k0+a] (column segments, or with S = 2
      // the rows of that copy, exchanged through LDS below)
      const bool swap = kStageT && !rowor;
#pragma unroll
      for (int r = 0; r < S; ++r) {
        int64_t left, g;
        if (rowor) {
          left = ty * S + r < bK ? bJ - tx * S : 0;
          g = (k0 + ty * S + r) * n + j0 + tx * S;
        } else if (swap) {
          left = ty * S + r < bJ ? bK - tx * S : 0;
          g = (j0 + ty * S + r) * n + k0 + tx * S;
        } else {
          left = tx * S + r < bJ ? bK - ty * S : 0;
          g = (j0 + tx * S + r) * n + k0 + ty * S;
        }
        yu[r] = load_seg<VEC, S>(Ub + g, left, kInf, Ub);
        yl[r] = load_seg<VEC, S>(Lb + g, left, 0.0f, Lb);
      }
#pragma unroll
      for (int r = 0; r < S; ++r)
#pragma unroll
        for (int q = 0; q < S; ++q) {
          du[r][q] = xu[r].v[q];
          dl[r][q] = xl[r].v[q];
          u[r][q] = rowor || swap ? yu[r].v[q] : yu[q].v[r];
          l[r][q] = rowor || swap ? yl[r].v[q] : yl[q].v[r];
        }
      if constexpr (kStageT) {
        if (swap) {  // uniform: u[r][q] holds M[j0 + ty*S + r][k0 + tx*S + q]
#pragma unroll
          for (int r = 0; r < S; ++r)
#pragma unroll
            for (int q = 0; q < S; ++q) {
              tt[0][ty * S + r][tx * S + q] = u[r][q];
              tt[PK ? 0 : 1][ty * S + r][tx * S + q] = l[r][q];
            }
          __syncthreads();
#pragma unroll
          for (int r = 0; r < S; ++r)
#pragma unroll
            for (int q = 0; q < S; ++q) {
              u[r][q] = tt[0][tx * S + q][ty * S + r];
              l[r][q] = tt[PK ? 0 : 1][tx * S + q][ty * S + r];
            }
        }
      }
    }

    for (int mb = 0; mb < NT; ++mb) {
#pragma unroll
      for (int r = 0; r < S; ++r) {
        const int m = mb * S + r;
        if (m >= bK) break;  // uniform
        const int buf = m & 1;
        if (ty == mb) {
#pragma unroll
          for (int q = 0; q < S; ++q) {
            dvu[buf][tx * S + q] = du[r][q];
            dvl[buf][tx * S + q] = dl[r][q];
            rvu[buf][tx * S + q] = u[r][q];
            rvl[buf][tx * S + q] = l[r][q];
          }
        }
        __syncthreads();
        float cu[S], cl[S], eu[S], el[S], ru[S], rl[S];
#pragma unroll
        for (int q = 0; q < S; ++q) {
          cu[q] = dvu[buf][ty * S + q];  // D[a][m] = D[m][a]
          cl[q] = dvl[buf][ty * S + q];
          eu[q] = dvu[buf][tx * S + q];  // D[m][b]
          el[q] = dvl[buf][tx * S + q];
          ru[q] = rvu[buf][tx * S + q];  // R[m][c]
          rl[q] = rvl[buf][tx * S + q];
        }
#pragma unroll
        for (int a = 0; a < S; ++a)
#pragma unroll
          for (int q = 0; q < S; ++q) {
            relax1<RU>(du[a][q], dl[a][q], cu[a], cl[a], eu[q], el[q]);
            relax1<RU>(u[a][q], l[a][q], cu[a], cl[a], ru[q], rl[q]);
          }
      }
    }

#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
      for (int q = 0; q < S; ++q) {
        l[r][q] = lower_out<RU>(l[r][q]);
        dl[r][q] = lower_out<RU>(dl[r][q]);
      }
    // R in both orientations (packed: the one slot of U and of L); D, which
    // lies in a fresh tile, as a full square
    const bool up = k0 < j0;  // R lies right of the diagonal
    if (PK) {
      if (kStageT) {
#pragma unroll
        for (int r = 0; r < S; ++r)
#pragma unroll
          for (int q = 0; q < S; ++q) {
            const int a = ty * S + r, c = tx * S + q;
            if (a < bK && c < bJ) Ub[(k0 + a) * n + j0 + c] = up ? u[r][q] : l[r][q];
          }
      } else {
        packed_block_store<S>(Ub, n, k0, j0, bK, bJ, ty, tx, u, l);
      }
    }
    // the early infeasibility test (as in flag_infeasible), on the cells of D
    // as they are stored, which keeps the test within the store's registers
    bool bad = false;
    if (PK && writes_d)
      packed_block_store<S>(Ub, n, k0, k0, bK, bK, ty, tx, du, dl, infeasible ? &bad : nullptr);
#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
      for (int q = 0; q < S; ++q) {
        const int a = ty * S + r, c = tx * S + q;
        if (!PK && a < bK && c < bJ) {
          Ub[(k0 + a) * n + j0 + c] = u[r][q];
          Lb[(k0 + a) * n + j0 + c] = l[r][q];
          if (!kStageT) {
            Ub[(j0 + c) * n + k0 + a] = u[r][q];
            Lb[(j0 + c) * n + k0 + a] = l[r][q];
          }
        }
        if (!PK && writes_d && a < bK && c < bK) {
          bad |= infeasible && dl[r][q] > du[r][q];
          Ub[(k0 + a) * n + k0 + c] = du[r][q];
          Lb[(k0 + a) * n + k0 + c] = dl[r][q];
        }
      }
    if constexpr (kStageT) {  // the copy in the other orientation, through tt
#pragma unroll
      for (int r = 0; r < S; ++r)
#pragma unroll
        for (int q = 0; q < S; ++q) {
          if (PK) {
            tt[0][tx * S + q][ty * S + r] = up ? l[r][q] : u[r][q];
          } else {
            tt[0][tx * S + q][ty * S + r] = u[r][q];
            tt[PK ? 0 : 1][tx * S + q][ty * S + r] = l[r][q];
          }
        }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < S; ++r)
#pragma unroll
        for (int q = 0; q < S; ++q) {
          const int c = ty * S + r, a = tx * S + q;
          if (c < bJ && a < bK) {
            Ub[(j0 + c) * n + k0 + a] = tt[0][c][a];
            if (!PK) Lb[(j0 + c) * n + k0 + a] = tt[PK ? 0 : 1][c][a];
          }
        }
    }
    if (bad) atomicOr(infeasible + b, DBS_INFEASIBLE_EARLY);
    __syncthreads();  // LDS reuse by the next molecule
  }
}

// Phases 1 and 2 of k-block K with each panel tile's columns split over P
// workgroups (where the launch is on the critical path):
// workgroup (J, h) (grid.x = P per k-block tile other than K, grid.y =
// molecules) holds the diagonal tile D, 2x2 cells per thread as
// k_diag_panel with S = 2 does, and the W = BK / P columns h*W .. of the
// panel tile R = (K, J), W / 16 cells per thread, and runs the rounds of
// band K in order over both.  Every workgroup repeats D's rounds; a round's
// arithmetic on one compute unit falls from D and R (8192 cells) to D and a
// P-th of R.  The slice is staged through an LDS tile for its loads and its
// stores in both orientations, so that the global accesses are row
// segments (packed: the row slots of R's cells hold U right of the diagonal
// and L left of it, the transposed slots the other).  The last workgroup of
// the molecule writes D back, as in k_diag_panel.
template <bool VEC, bool PK, bool RU, int P>
__global__ __launch_bounds__(1024) void k_diag_panel_split(float *__restrict__ U,
                                                          float *__restrict__ L, int64_t n,
                                                          int64_t batch, int64_t K,
                                                          uint32_t *infeasible) {
  static_assert(P == 2 || P == 4, "two or four column slices");
  constexpr int W = BK / P;   // columns of R per workgroup
  constexpr int NR = W / 16;  // R cells per thread: 2 (P = 2) or 1 (P = 4)
  __shared__ __align__(16) float dvu[2][BK], dvl[2][BK];  // row m of D
  __shared__ __align__(16) float rvu[2][W], rvl[2][W];    // row m of the slice
  __shared__ float sr[2][BK][W + 1];                      // the slice (U, L)

  rounding_prologue<RU>();
  critical_path_priority();
  const int tid = threadIdx.x, ty = tid >> 5, tx = tid & 31;
  // this thread's cells of the slice: column rc, rows 2ty + rr + i (i < NR)
  const int rc = P == 2 ? tx : (tx & 15);
  const int rr = P == 2 ? 0 : (tx >> 4);
  int64_t J = blockIdx.x / P;
  if (J >= K) ++J;
  const int64_t k0 = K * BK, c0 = J * BK + (blockIdx.x % P) * W;  // the slice's first column
  const bool up = K < J;  // R lies right of the diagonal
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int bW = (int)(n - c0 < W ? (n - c0 > 0 ? n - c0 : 0) : W);  // its columns inside
  const bool rowor = fresh(K, J);
  const bool writes_d = blockIdx.x == gridDim.x - 1;
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = PK ? Ub : L + b * nn;
    float du[2][2], dl[2][2];  // D[2ty + r][2tx + q]
    if constexpr (PK) {
      packed_block_load<VEC, 2>(Ub, n, k0, k0, bK, bK, ty, tx, du, dl);
      // the slice's row slots P[k0+a][c0+c] (lanes along c) and transposed
      // slots P[c0+c][k0+a] (lanes along a)
#pragma unroll
      for (int it = 0; it < BK * W / 1024; ++it) {
        const int e = tid + it * 1024;
        const int a = e / W, c = e % W, at = e % BK, ct = e / BK;
        const bool in = a < bK && c < bW, inT = at < bK && ct < bW;
        const float x = Ub[in ? (k0 + a) * n + c0 + c : 0];
        const float y = Ub[inT ? (c0 + ct) * n + k0 + at : 0];
        sr[up ? 0 : 1][a][c] = in ? x : (up ? kInf : 0.0f);
        sr[up ? 1 : 0][at][ct] = inT ? y : (up ? 0.0f : kInf);
      }
    } else {
      Seg<2> xu[2], xl[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int a = ty * 2 + r;
        const int64_t g = (k0 + a) * n + k0 + tx * 2;
        const int64_t left = a < bK ? bK - tx * 2 : 0;
        xu[r] = load_seg<VEC, 2>(Ub + g, left, kInf, Ub);
        xl[r] = load_seg<VEC, 2>(Lb + g, left, 0.0f, Lb);
      }
      // the slice from its fresh orientation: R[a][c] = M[k0+a][c0+c] (lanes
      // along c), else M[c0+c][k0+a] (lanes along a)
#pragma unroll
      for (int it = 0; it < BK * W / 1024; ++it) {
        const int e = tid + it * 1024;
        const int a = rowor ? e / W : e % BK, c = rowor ? e % W : e / BK;
        const bool in = a < bK && c < bW;
        const int64_t g = in ? (rowor ? (k0 + a) * n + c0 + c : (c0 + c) * n + k0 + a) : 0;
        const float xu = Ub[g], xl = Lb[g];
        sr[0][a][c] = in ? xu : kInf;
        sr[1][a][c] = in ? xl : 0.0f;
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          du[r][q] = xu[r].v[q];
          dl[r][q] = xl[r].v[q];
        }
    }
    __syncthreads();
    float ur[NR], lr[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      ur[i] = sr[0][2 * ty + rr + i][rc];
      lr[i] = sr[1][2 * ty + rr + i][rc];
    }

    // Row m of D and of the slice is published into dv/rv[m & 1] by its
    // owners during round m - 1, right after they relax it and before their
    // other cells, so that the LDS write overlaps that work instead of
    // preceding the barrier (buffer m & 1 was last read in round m - 2,
    // which every thread finished before round m - 1 began).
    auto publish = [&](int m, int buf, int a) {
      // this thread's cells of row m = 2ty + a (D) and of slice row m
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        dvu[buf][tx * 2 + q] = du[a][q];
        dvl[buf][tx * 2 + q] = dl[a][q];
      }
      if constexpr (P == 2) {
        rvu[buf][rc] = ur[a];
        rvl[buf][rc] = lr[a];
      } else if (rr == a) {
        rvu[buf][rc] = ur[0];
        rvl[buf][rc] = lr[0];
      }
    };
    if (ty == 0) publish(0, 0, 0);
    for (int mb = 0; mb < BK / 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int m = mb * 2 + r;
        if (m >= bK) break;  // uniform
        const int buf = m & 1;
        __syncthreads();
        float cu[2], cl[2], eu[2], el[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          cu[q] = dvu[buf][ty * 2 + q];  // D[a][m] = D[m][a]
          cl[q] = dvl[buf][ty * 2 + q];
          eu[q] = dvu[buf][tx * 2 + q];  // D[m][b]
          el[q] = dvl[buf][tx * 2 + q];
        }
        const float ru = rvu[buf][rc], rl = rvl[buf][rc];  // R[m][c]
        // row m + 1 (parity 1 - r) first: its owners publish it next
        const int r1 = 1 - r;  // the loop is unrolled: a constant per copy
        if constexpr (P == 2) {
          relax1<RU>(ur[r1], lr[r1], cu[r1], cl[r1], ru, rl);
        } else {
          relax1<RU>(ur[0], lr[0], rr ? cu[1] : cu[0], rr ? cl[1] : cl[0], ru, rl);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) relax1<RU>(du[r1][q], dl[r1][q], cu[r1], cl[r1], eu[q], el[q]);
        if (m + 1 < bK && ty == (r == 0 ? mb : mb + 1)) publish(m + 1, buf ^ 1, r1);
#pragma unroll
        for (int q = 0; q < 2; ++q) relax1<RU>(du[r][q], dl[r][q], cu[r], cl[r], eu[q], el[q]);
        if constexpr (P == 2) relax1<RU>(ur[r], lr[r], cu[r], cl[r], ru, rl);
      }
    }

    // the slice in both orientations, through sr (each thread rewrites the
    // entries it read; no other thread reads sr during the rounds)
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      sr[0][2 * ty + rr + i][rc] = ur[i];
      sr[1][2 * ty + rr + i][rc] = lower_out<RU>(lr[i]);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < BK * W / 1024; ++it) {
      const int e = tid + it * 1024;
      const int a = e / W, c = e % W;  // rows of band K, lanes along c
      if (a < bK && c < bW) {
        if (PK) {
          Ub[(k0 + a) * n + c0 + c] = sr[up ? 0 : 1][a][c];
        } else {
          Ub[(k0 + a) * n + c0 + c] = sr[0][a][c];
          Lb[(k0 + a) * n + c0 + c] = sr[1][a][c];
        }
      }
      const int at = e % BK, ct = e / BK;  // the other orientation, lanes along a
      if (at < bK && ct < bW) {
        if (PK) {
          Ub[(c0 + ct) * n + k0 + at] = sr[up ? 1 : 0][at][ct];
        } else {
          Ub[(c0 + ct) * n + k0 + at] = sr[0][at][ct];
          Lb[(c0 + ct) * n + k0 + at] = sr[1][at][ct];
        }
      }
    }
    // D (a fresh tile, as a full square) from the last workgroup, with the
    // early test of the infeasibility option on its cells as they are stored
    bool bad = false;
    if (PK && writes_d) {
      float dlo[2][2];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 2; ++q) dlo[r][q] = lower_out<RU>(dl[r][q]);
      packed_block_store<2>(Ub, n, k0, k0, bK, bK, ty, tx, du, dlo, infeasible ? &bad : nullptr);
    }
    if (!PK && writes_d) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int a = ty * 2 + r, c = tx * 2 + q;
          const float lo = lower_out<RU>(dl[r][q]);
          if (a < bK && c < bK) {
            bad |= infeasible && lo > du[r][q];
            Ub[(k0 + a) * n + k0 + c] = du[r][q];
            Lb[(k0 + a) * n + k0 + c] = lo;
          }
        }
    }
    if (bad) atomicOr(infeasible + b, DBS_INFEASIBLE_EARLY);
    __syncthreads();  // LDS reuse by the next molecule
  }
}

// ---------------------------------------------------------------- packed panel staging
// Packed layout: the panel values of band K at the 64 columns xh..xh+63 and
// rows k0+kc..k0+kc+KC-1 are U[k][x] = P[min(k,x)][max(k,x)] and
// L[k][x] = P[max(k,x)][min(k,x)].  Right of the band (x > k) U is a row
// segment of P and L a column segment; left of it the other way round.  A
// column segment is read as rows of P, four consecutive k per float4.  Each
// of the 256 threads loads one float4 of each kind.  `dead` (values no live
// cell uses) gives the neutral values.
struct HalfLoad {
  float4 direct, across;
};

template <bool VEC>
__device__ __forceinline__ HalfLoad packed_half_load(const float *P, int64_t n, int64_t k0,
                                                     int kc, int bK, int64_t xh, bool right,
                                                     bool dead, int tid) {
  HalfLoad h;
  {
    const int kk = tid / (BK / 4), x4 = tid % (BK / 4);
    const int64_t x = xh + 4 * x4;
    const int cnt = (!dead && kc + kk < bK) ? clamp4(n - x) : 0;
    h.direct = load4<VEC>(P + (k0 + kc + kk) * n + x, cnt, right ? kInf : 0.0f, P);
  }
  {
    const int xt = tid / (KC / 4), kq = tid % (KC / 4);
    const int64_t x = xh + xt;
    const int cnt = (!dead && x < n) ? clamp4(bK - (kc + 4 * kq)) : 0;
    h.across = load4<VEC>(P + x * n + k0 + kc + 4 * kq, cnt, right ? 0.0f : kInf, P);
  }
  return h;
}

// packed_half_load for a whole chunk of an interior block (no masks): the
// thread's offsets od (direct: its atom row within the chunk and column) and
// oa (across: its column's row and atom quad) are the same in every chunk,
// 32-bit (n is below 2^27); only the wave-uniform bases move.
__device__ __forceinline__ HalfLoad packed_half_load_whole(const float *P, int64_t n,
                                                           int64_t k, int64_t xh, uint32_t od,
                                                           uint32_t oa) {
  HalfLoad h;
  h.direct = *reinterpret_cast<const float4 *>(P + k * n + xh + od);
  h.across = *reinterpret_cast<const float4 *>(P + xh * n + k + oa);
  return h;
}

__device__ __forceinline__ uint32_t half_direct_offset(int64_t n, int tid) {
  return (uint32_t)((tid / (BK / 4)) * n + (tid % (BK / 4)) * 4);
}
__device__ __forceinline__ uint32_t half_across_offset(int64_t n, int tid) {
  return (uint32_t)((tid / (KC / 4)) * n + (tid % (KC / 4)) * 4);
}

// Store a HalfLoad into LDS arrays su, sl ([KC][stride] floats) at column col.
__device__ __forceinline__ void packed_half_store(const HalfLoad &h, bool right, float *su,
                                                  float *sl, int stride, int col, int tid) {
  float *dst_direct = right ? su : sl, *dst_across = right ? sl : su;
  {
    const int kk = tid / (BK / 4), x4 = tid % (BK / 4);
    *reinterpret_cast<float4 *>(dst_direct + kk * stride + col + 4 * x4) = h.direct;
  }
  {
    const int xt = tid / (KC / 4), kq = tid % (KC / 4);
    dst_across[(4 * kq + 0) * stride + col + xt] = h.across.x;
    dst_across[(4 * kq + 1) * stride + col + xt] = h.across.y;
    dst_across[(4 * kq + 2) * stride + col + xt] = h.across.z;
    dst_across[(4 * kq + 3) * stride + col + xt] = h.across.w;
  }
}

// ---------------------------------------------------------------- block write-back
// v[r][q] of thread (ty, tx) (a 4 x CT cell tile of a BK x BK block) to
// P[r0 + 4ty + r][c0 + CT*tx + q], rows < rows and columns < cols: one
// CT-float vector per row where the row segment is whole (VEC: aligned).
template <bool VEC, int CT = 4>
__device__ __forceinline__ void store_rows(float *P, int64_t n, int64_t r0, int64_t c0, int rows,
                                           int cols, int ty, int tx, const float (&v)[4][CT]) {
  static_assert(CT == 4 || CT == 2, "4 or 2 columns");
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int a = ty * 4 + r, c = tx * CT;
    if (a >= rows) continue;
    float *p = P + (r0 + a) * n + c0 + c;
    if (VEC && c + CT - 1 < cols) {
      if constexpr (CT == 4)
        *reinterpret_cast<float4 *>(p) = make_float4(v[r][0], v[r][1], v[r][2], v[r][3]);
      else
        *reinterpret_cast<float2 *>(p) = make_float2(v[r][0], v[r][1]);
    } else {
#pragma unroll
      for (int q = 0; q < CT; ++q)
        if (c + q < cols) p[q] = v[r][q];
    }
  }
}

// A diagonal block of the packed layout (r0 == c0) holds both (a, c) and
// (c, a), so its row segments alone cover every slot once: U of the cells
// right of the diagonal, L of those left of it and U on it (the relaxed value
// that the dense layout stores there).
template <bool VEC>
__device__ __forceinline__ void store_packed_diagonal(float *P, int64_t n, int64_t r0, int rows,
                                                      int ty, int tx, const float (&u)[4][4],
                                                      const float (&l)[4][4]) {
  float v[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) v[r][q] = ty * 4 + r > tx * 4 + q ? l[r][q] : u[r][q];
  store_rows<VEC>(P, n, r0, r0, rows, rows, ty, tx, v);
}

// The same cells to their transposed position P[c0 + CT*tx + q][r0 + 4ty + r]
// (the workgroup: (BK / 4) x (BK / CT) threads).  The block is turned around
// in the LDS tile `tr` first (stride BK + 1: the writes meet at most 8
// threads on a bank, the reads 2), so that the global writes are row
// segments, 16 threads to a 256-byte row.  Contains barriers: every thread of
// the workgroup must call it.
template <bool VEC, int CT = 4>
__device__ __forceinline__ void store_transposed(float *P, int64_t n, int64_t r0, int64_t c0,
                                                 int rows, int cols, int ty, int tx,
                                                 const float (&v)[4][CT],
                                                 float (*tr)[BK + 1]) {
  constexpr int NTH = (BK / 4) * (BK / CT);
  __syncthreads();  // tr free (a previous call may still be reading it)
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < CT; ++q) tr[tx * CT + q][ty * 4 + r] = v[r][q];
  __syncthreads();
  const int tid = ty * (BK / CT) + tx;
#pragma unroll
  for (int it = 0; it < BK * BK / 4 / NTH; ++it) {
    const int e = tid + it * NTH, c = e / (BK / 4), a = (e % (BK / 4)) * 4;
    if (c >= cols) continue;
    float *p = P + (c0 + c) * n + r0 + a;
    if (VEC && a + 3 < rows) {
      *reinterpret_cast<float4 *>(p) = make_float4(tr[c][a], tr[c][a + 1], tr[c][a + 2],
                                                    tr[c][a + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (a + i < rows) p[i] = tr[c][a + i];
    }
  }
}

// ---------------------------------------------------------------- phase 3

// Quadrant order of a bulk launch.  The upper TILE x TILE tiles are split
// into their four BK x BK quadrants (consecutive workgroups), and the
// hardware deals consecutive workgroups to the 8 XCDs in turn.
//  * Plain order: tiles column-major over the upper triangle, so at any
//    moment an XCD works on a few tile columns and on every 8th tile row of
//    them.
//  * XCD order: the tiles are grouped into super-blocks of SB x SB tiles,
//    numbered column-major over the upper triangle (a diagonal super-block
//    keeps its lower tiles, which exit at once); workgroup w takes
//    super-block 8 * (w / 8 / (4 SB^2)) + w % 8, so each XCD works through
//    every 8th super-block, four quadrants of a tile after another.  The
//    quadrants an XCD runs at once then share few panel row slices, which
//    stay in its L2: at n = 12288 with 256-atom steps a launch reads 1.26 GB
//    instead of 2.39 GB, at the same launch time.  It deals the work less
//    evenly among the XCDs, since the bands a launch leaves out empty some
//    super-blocks: that costs nothing where a launch runs many rounds of
//    workgroups, but 2 % at n = 4096 (about two rounds per launch).  Larger
//    super-blocks cut the reads a little further (SB = 4: 1.18 GB) and are
//    less even again (n = 12288 pass 69.4 against 68.6 ms); one contiguous
//    run per XCD is worse still (74 ms).
constexpr int64_t kSuperBlock = 2;
// Tiles per side from which a pass that runs two steps ahead takes the XCD
// order.
constexpr int64_t kXcdTiles = 64;

// Workgroups of a bulk launch over T x T tiles (the quadrants' grid.x).
inline int64_t bulk_workgroups(int64_t T, bool xcd) {
  if (!xcd) return 4 * (T * (T + 1) / 2);
  const int64_t NSB = ceil_div(T, kSuperBlock), nsp = NSB * (NSB + 1) / 2;
  return 8 * ceil_div(nsp, 8) * kSuperBlock * kSuperBlock * 4;
}

// The quadrant (row band A, column band B) of bulk workgroup w in the plain
// or XCD order, and whether it is the lower-left quadrant of a diagonal
// tile; false if the workgroup has no quadrant.
__device__ __forceinline__ bool bulk_quadrant(int64_t w, int64_t n, bool xcd, int64_t &A,
                                              int64_t &B, bool &lower_left) {
  int64_t I2, J2, qd;
  if (!xcd) {
    const int64_t p = w >> 2;
    qd = w & 3;
    J2 = tri_col(p);
    I2 = p - J2 * (J2 + 1) / 2;
  } else {
    constexpr int64_t SB = kSuperBlock, PER = SB * SB * 4;
    const int64_t T = (n + TILE - 1) / TILE, NSB = (T + SB - 1) / SB;
    const int64_t loc = w >> 3, sp = (loc / PER) * 8 + (w & 7);
    if (sp >= NSB * (NSB + 1) / 2) return false;
    const int64_t r = loc % PER, t = r >> 2;
    qd = r & 3;
    const int64_t SJ = tri_col(sp), SI = sp - SJ * (SJ + 1) / 2;
    I2 = SI * SB + t % SB;
    J2 = SJ * SB + t / SB;
    if (I2 > J2 || J2 >= T) return false;
  }
  A = RATIO * I2 + (qd >> 1);
  B = RATIO * J2 + (qd & 1);
  lower_left = I2 == J2 && qd == 2;
  return true;
}

// Phase 3 of the k-blocks K .. K+nk-1 (their atoms in order) on the row
// bands A0 + r, r < grid.z, other than the atoms' own, run ahead of the bulk
// on the second stream or inside a step's panel.  Row band A0 + r takes
// every column band outside [X0, X1 + r) and other than Y (< 0: none).  The
// callers put the atoms' own bands (whose rows are final) in that set, and
// X1 = A0 where grid.z > 1: then row band A0 + r leaves out the row bands
// before it (block (A0+r, A0+r') is block (A0+r', A0+r) of an earlier row
// band).  grid.x = the first row band's column bands, grid.y = molecules.
// Block (A, J) is read and written in its fresh orientation (dense) or as
// its U and L slots (packed); with `both` (dense), row bands before K write
// the other orientation too, so that their rows can serve as a panel
// afterwards.  Thread (ty, tx) owns a
// 4x4 cell tile.  The panel rows of the atoms are staged through LDS in
// chunks of KC atoms; the global loads of chunk c+1 are issued before chunk
// c is computed.  Per atom and cell the VALU does one add and one min for U,
// two subtracts and two max for L; pairs of atoms fold into 3-input min/max
// (4.5 instructions per cell and atom).  The strip is on the critical path
// of the look-ahead and raises its waves' issue priority.
template <bool VEC, bool PK, bool RU>
__global__ __launch_bounds__(kThreads) void k_strip(float *__restrict__ U, float *__restrict__ L,
                                                    int64_t n, int64_t batch, int64_t K,
                                                    int64_t nk, int64_t A0, int64_t X0,
                                                    int64_t X1, int64_t Y, int both) {
  __shared__ float4 scu[KC][BK / 4];
  __shared__ float4 scl[KC][BK / 4];
  __shared__ float4 sru[KC][BK / 4];
  __shared__ float4 srl[KC][BK / 4];
  __shared__ float tr[BK][BK + 1];  // write-back of transposed values

  rounding_prologue<RU>();
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  critical_path_priority();
  // row band A = A0 + blockIdx.z; column band B: the blockIdx.x-th band
  // outside [X0, X1 + blockIdx.z) and other than Y
  const int64_t TB = (n + BK - 1) / BK, A = A0 + blockIdx.z;
  const int64_t xe = X1 + blockIdx.z < TB ? X1 + blockIdx.z : TB;
  const int64_t y = Y >= xe && Y < TB ? Y : -1;
  int64_t B = blockIdx.x;
  // uniform over the workgroup, before any barrier
  if (B >= TB - (xe - X0) - (y >= 0) || (A >= K && A < K + nk)) return;
  if (B >= X0) B += xe - X0;
  if (y >= 0 && B >= y) ++B;
  const bool rowor = fresh(A, B);  // stored as (A, B), else as its transpose (B, A)
  const int64_t k0 = K * BK, a0 = A * BK, j0 = B * BK;
  const int bK = (int)(n - k0 < nk * BK ? n - k0 : nk * BK);
  const int bA = (int)(n - a0 < BK ? n - a0 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = PK ? Ub : L + b * nn;

    // logical cell (a, c) = (a0 + a, j0 + c); stored at (a0+a, j0+c) or (j0+c, a0+a)
    float u[4][4], l[4][4];
    if (PK) {
      packed_block_load<VEC>(Ub, n, a0, j0, bA, bJ, ty, tx, u, l);
    } else {
      float4 x[4], y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cnt = rowor ? (ty * 4 + r < bA ? clamp4(bJ - tx * 4) : 0)
                              : (tx * 4 + r < bJ ? clamp4(bA - ty * 4) : 0);
        const int64_t g = rowor ? (a0 + ty * 4 + r) * n + j0 + tx * 4
                                : (j0 + tx * 4 + r) * n + a0 + ty * 4;
        x[r] = load4<VEC>(Ub + g, cnt, kInf, Ub);
        y[r] = load4<VEC>(Lb + g, cnt, 0.0f, Lb);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float xr[4] = {x[r].x, x[r].y, x[r].z, x[r].w};
        const float yr[4] = {y[r].x, y[r].y, y[r].z, y[r].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          (rowor ? u[r][q] : u[q][r]) = xr[q];
          (rowor ? l[r][q] : l[q][r]) = yr[q];
        }
      }
    }

    // staged operands of one chunk: panel rows k0+kc.., columns of band A
    // (U/L[i,k] = U/L[k,i]) and of band B
    // a whole chunk of an interior block loads without masks, from offsets
    // that are the same in every chunk (see k_quads)
    const uint32_t od = half_direct_offset(n, tid), oa = half_across_offset(n, tid);
    const bool whole_rows = bA == BK && bJ == BK;
    auto fetch = [&](int kc, float4 (&st)[4], HalfLoad (&hl)[2]) {
      if (VEC && whole_rows && kc + KC <= bK) {
        if (PK) {
          hl[0] = packed_half_load_whole(Ub, n, k0 + kc, a0, od, oa);
          hl[1] = packed_half_load_whole(Ub, n, k0 + kc, j0, od, oa);
        } else {
          const float *cu = Ub + (k0 + kc) * n, *cl = Lb + (k0 + kc) * n;
          st[0] = *reinterpret_cast<const float4 *>(cu + a0 + od);
          st[1] = *reinterpret_cast<const float4 *>(cl + a0 + od);
          st[2] = *reinterpret_cast<const float4 *>(cu + j0 + od);
          st[3] = *reinterpret_cast<const float4 *>(cl + j0 + od);
        }
      } else if (PK) {
        // band A and band B each lie right or left of band K; the addresses
        // are re-derived per chunk (laundered thread index), not kept live
        int tf = tid;
        asm volatile("" : "+v"(tf));
        hl[0] = packed_half_load<VEC>(Ub, n, k0, kc, bK, a0, A > K, false, tf);
        hl[1] = packed_half_load<VEC>(Ub, n, k0, kc, bK, j0, B > K, false, tf);
      } else {
        // KC x BK/4 float4 per array: one of each per thread
        const int kk = tid / (BK / 4), x4 = tid % (BK / 4);
        const int64_t k = k0 + kc + kk;
        const bool kin = kc + kk < bK;
        const int ni = kin ? clamp4(bA - x4 * 4) : 0;
        const int nj = kin ? clamp4(bJ - x4 * 4) : 0;
        st[0] = load4<VEC>(Ub + k * n + a0 + x4 * 4, ni, kInf, Ub);
        st[1] = load4<VEC>(Lb + k * n + a0 + x4 * 4, ni, 0.0f, Lb);
        st[2] = load4<VEC>(Ub + k * n + j0 + x4 * 4, nj, kInf, Ub);
        st[3] = load4<VEC>(Lb + k * n + j0 + x4 * 4, nj, 0.0f, Lb);
      }
    };
    auto stage = [&](const float4 (&st)[4], const HalfLoad (&hl)[2]) {
      if (PK) {
        int ts = tid;
        asm volatile("" : "+v"(ts));
        packed_half_store(hl[0], A > K, reinterpret_cast<float *>(&scu[0][0]),
                          reinterpret_cast<float *>(&scl[0][0]), BK, 0, ts);
        packed_half_store(hl[1], B > K, reinterpret_cast<float *>(&sru[0][0]),
                          reinterpret_cast<float *>(&srl[0][0]), BK, 0, ts);
      } else {
        const int kk = tid / (BK / 4), x4 = tid % (BK / 4);
        scu[kk][x4] = st[0];
        scl[kk][x4] = st[1];
        sru[kk][x4] = st[2];
        srl[kk][x4] = st[3];
      }
    };

    float4 st[4];
    HalfLoad hl[2];
    fetch(0, st, hl);
    for (int kc = 0; kc < bK; kc += KC) {
      stage(st, hl);
      __syncthreads();
      if (kc + KC < bK) fetch(kc + KC, st, hl);  // in flight during this chunk
#pragma unroll 2
      for (int kk = 0; kk < KC; kk += 2) {
        const float4 a0v = scu[kk][ty], b0 = scl[kk][ty], c0 = sru[kk][tx], d0 = srl[kk][tx];
        const float4 a1 = scu[kk + 1][ty], b1v = scl[kk + 1][ty], c1 = sru[kk + 1][tx], d1 = srl[kk + 1][tx];
        const float cu0[4] = {a0v.x, a0v.y, a0v.z, a0v.w}, cl0[4] = {b0.x, b0.y, b0.z, b0.w};
        const float ru0[4] = {c0.x, c0.y, c0.z, c0.w}, rl0[4] = {d0.x, d0.y, d0.z, d0.w};
        const float cu1[4] = {a1.x, a1.y, a1.z, a1.w}, cl1[4] = {b1v.x, b1v.y, b1v.z, b1v.w};
        const float ru1[4] = {c1.x, c1.y, c1.z, c1.w}, rl1[4] = {d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            relax2<RU>(u[r][q], l[r][q], cu0[r], cl0[r], ru0[q], rl0[q], cu1[r], cl1[r], ru1[q],
                   rl1[q]);
      }
      __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) l[r][q] = lower_out<RU>(l[r][q]);
    // write-back as row segments: scattered single-float writes across rows
    // cost more than the LDS round trip of the transposed half.  The thread
    // index is re-derived here so that the write addresses are computed
    // after the k loop instead of being kept live through it.
    int tw = tid;
    asm volatile("" : "+v"(tw));
    const int wy = tw >> 4, wx = tw & 15;
    if (PK && a0 == j0) {
      store_packed_diagonal<VEC>(Ub, n, a0, bA, wy, wx, u, l);
    } else if (PK) {
      // one side of the diagonal: the row slots hold U right of it, L left
      if (a0 < j0) {
        store_rows<VEC>(Ub, n, a0, j0, bA, bJ, wy, wx, u);
        store_transposed<VEC>(Ub, n, a0, j0, bA, bJ, wy, wx, l, tr);
      } else {
        store_rows<VEC>(Ub, n, a0, j0, bA, bJ, wy, wx, l);
        store_transposed<VEC>(Ub, n, a0, j0, bA, bJ, wy, wx, u, tr);
      }
    } else if (rowor) {
      store_rows<VEC>(Ub, n, a0, j0, bA, bJ, wy, wx, u);
      store_rows<VEC>(Lb, n, a0, j0, bA, bJ, wy, wx, l);
    } else {
      store_transposed<VEC>(Ub, n, a0, j0, bA, bJ, wy, wx, u, tr);
      store_transposed<VEC>(Lb, n, a0, j0, bA, bJ, wy, wx, l, tr);
    }
    if (!PK && both && A < K && A != B) {
      // the other orientation too (uniform over the workgroup)
      if (rowor) {
        store_transposed<VEC>(Ub, n, a0, j0, bA, bJ, wy, wx, u, tr);
        store_transposed<VEC>(Lb, n, a0, j0, bA, bJ, wy, wx, l, tr);
      } else {
        store_rows<VEC>(Ub, n, a0, j0, bA, bJ, wy, wx, u);
        store_rows<VEC>(Lb, n, a0, j0, bA, bJ, wy, wx, l);
      }
    }
    __syncthreads();
  }
}

// One BK x BK block of the dense layout as phase 3 handles it: thread
// (ty, tx) owns RT x CT cells (rows a0 + RT*ty + r, columns j0 + CT*tx + q),
// and the panel rows of the atoms are staged through LDS, KCH atoms per
// chunk with the next chunk's loads in flight.  Used by the bulk (k_quads)
// and by the lead launch (k_lead).  Larger register tiles read fewer staged
// operand floats per cell but lose occupancy; 4x4 is the fastest measured
// for the bulk (kBulkRT below).
template <bool VEC, bool RU, int RT, int CT, int KCH>
struct Quad {
  static constexpr int NTX = BK / CT, NT = (BK / RT) * NTX;
  // operands and cells move as vectors of RW rows / CW columns (4, or 2 for
  // 2-wide tiles)
  static constexpr int RW = RT < 4 ? RT : 4, CW = CT < 4 ? CT : 4;
  static constexpr int RQ = RT / RW, CQ = CT / CW;
  static_assert(RW % 2 == 0 && CW % 2 == 0 && RT % RW == 0 && CT % CW == 0, "tile shape");
  static constexpr int ITER = KCH * (BK / 4) / NT;  // staged float4 per thread and array
  static_assert(ITER >= 1 && KCH * (BK / 4) % NT == 0, "staging split");
  struct Stage {
    float4 cu[KCH][BK / 4], cl[KCH][BK / 4], ru[KCH][BK / 4], rl[KCH][BK / 4];
  };

  // the block's cells of one molecule (neutral outside the matrix)
  static __device__ __forceinline__ void load(const float *Ub, const float *Lb, int64_t n,
                                              int64_t a0, int64_t j0, int bA, int bJ, int ty,
                                              int tx, float (&u)[RT][CT], float (&l)[RT][CT]) {
    Seg<CW> x[RT][CQ], y[RT][CQ];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int h = 0; h < CQ; ++h) {
        const int a = ty * RT + r, c = tx * CT + CW * h;
        const int64_t left = a < bA ? bJ - c : 0;
        const int64_t g = (a0 + a) * n + j0 + c;
        x[r][h] = load_seg<VEC, CW>(Ub + g, left, kInf, Ub);
        y[r][h] = load_seg<VEC, CW>(Lb + g, left, 0.0f, Lb);
      }
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int h = 0; h < CQ; ++h)
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          u[r][CW * h + i] = x[r][h].v[i];
          l[r][CW * h + i] = y[r][h].v[i];
        }
  }

  // The atoms k0 .. k0+bK-1 applied to the cells: the panel rows of the atoms
  // at the columns of band A (U/L[i,k] = U/L[k,i]) and of band B, staged
  // through sm.  Contains barriers: every thread of the workgroup calls it.
  static __device__ __forceinline__ void relax(Stage &sm, const float *Ub, const float *Lb,
                                               int64_t n, int64_t k0, int bK, int64_t a0,
                                               int64_t j0, int bA, int bJ, int tid, int ty,
                                               int tx, float (&u)[RT][CT], float (&l)[RT][CT]) {
    // Staging: this thread's float4 of each panel array sits at the same
    // offset from the chunk's first atom row in every chunk (32-bit: n is
    // below 2^27), so only the wave-uniform chunk base moves.  A whole chunk
    // of an interior block loads without masks.
    float4 st[ITER][4];
    uint32_t so[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int e = tid + it * NT;
      so[it] = (uint32_t)((e / (BK / 4)) * n + (e % (BK / 4)) * 4);
    }
    const bool interior = bA == BK && bJ == BK;
    auto fetch = [&](int kc) {
      const float *cu = Ub + (k0 + kc) * n, *cl = Lb + (k0 + kc) * n;
      if (VEC && interior && kc + KCH <= bK) {
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
          st[it][0] = *reinterpret_cast<const float4 *>(cu + a0 + so[it]);
          st[it][1] = *reinterpret_cast<const float4 *>(cl + a0 + so[it]);
          st[it][2] = *reinterpret_cast<const float4 *>(cu + j0 + so[it]);
          st[it][3] = *reinterpret_cast<const float4 *>(cl + j0 + so[it]);
        }
      } else {
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
          const int e = tid + it * NT, kk = e / (BK / 4), x4 = e % (BK / 4);
          const bool kin = kc + kk < bK;
          const int ni = kin ? clamp4(bA - x4 * 4) : 0;
          const int nj = kin ? clamp4(bJ - x4 * 4) : 0;
          st[it][0] = load4<VEC>(cu + a0 + so[it], ni, kInf, Ub);
          st[it][1] = load4<VEC>(cl + a0 + so[it], ni, 0.0f, Lb);
          st[it][2] = load4<VEC>(cu + j0 + so[it], nj, kInf, Ub);
          st[it][3] = load4<VEC>(cl + j0 + so[it], nj, 0.0f, Lb);
        }
      }
    };
    fetch(0);
    for (int kc = 0; kc < bK; kc += KCH) {
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int e = tid + it * NT, kk = e / (BK / 4), x4 = e % (BK / 4);
        sm.cu[kk][x4] = st[it][0];
        sm.cl[kk][x4] = st[it][1];
        sm.ru[kk][x4] = st[it][2];
        sm.rl[kk][x4] = st[it][3];
      }
      __syncthreads();
      if (kc + KCH < bK) fetch(kc + KCH);  // in flight during this chunk
#pragma unroll 2
      for (int kk = 0; kk < KCH; kk += 2) {
        float cu0[RT], cl0[RT], cu1[RT], cl1[RT], ru0[CT], rl0[CT], ru1[CT], rl1[CT];
        // W consecutive staged floats of atom row kk starting at float index i0
        auto vec = [&](float4 (*arr)[BK / 4], int kr, int i0, int W, float *out) {
          if (W == 4) {
            const float4 v = arr[kr][i0 / 4];
            out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
          } else {
            const float2 v = reinterpret_cast<const float2 *>(&arr[kr][0])[i0 / 2];
            out[0] = v.x; out[1] = v.y;
          }
        };
#pragma unroll
        for (int h = 0; h < RQ; ++h) {
          const int i0 = RT * ty + RW * h;
          vec(sm.cu, kk, i0, RW, cu0 + RW * h);
          vec(sm.cl, kk, i0, RW, cl0 + RW * h);
          vec(sm.cu, kk + 1, i0, RW, cu1 + RW * h);
          vec(sm.cl, kk + 1, i0, RW, cl1 + RW * h);
        }
#pragma unroll
        for (int h = 0; h < CQ; ++h) {
          const int i0 = CT * tx + CW * h;
          vec(sm.ru, kk, i0, CW, ru0 + CW * h);
          vec(sm.rl, kk, i0, CW, rl0 + CW * h);
          vec(sm.ru, kk + 1, i0, CW, ru1 + CW * h);
          vec(sm.rl, kk + 1, i0, CW, rl1 + CW * h);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int q = 0; q < CT; ++q)
            relax2<RU>(u[r][q], l[r][q], cu0[r], cl0[r], ru0[q], rl0[q], cu1[r], cl1[r], ru1[q],
                       rl1[q]);
      }
      __syncthreads();
    }
  }

  // write-back of the cells, one CW-float vector per row group.  The thread
  // index is re-derived here so that the write addresses are computed after
  // the k loop instead of being kept live through it.
  static __device__ __forceinline__ void store(float *Ub, float *Lb, int64_t n, int64_t a0,
                                               int64_t j0, int bA, int bJ, int tid,
                                               const float (&u)[RT][CT],
                                               const float (&l)[RT][CT]) {
    int tw = tid;
    asm volatile("" : "+v"(tw));
    const int wy = tw / NTX, wx = tw % NTX;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int a = wy * RT + r;
      if (a >= bA) continue;
#pragma unroll
      for (int h = 0; h < CQ; ++h) {
        const int c = wx * CT + CW * h;
        float *pu = Ub + (a0 + a) * n + j0 + c, *pl = Lb + (a0 + a) * n + j0 + c;
        float uv[CW], lv[CW];
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          uv[i] = u[r][CW * h + i];
          lv[i] = lower_out<RU>(l[r][CW * h + i]);
        }
        if (VEC && c + CW - 1 < bJ) {
          if constexpr (CW == 4) {
            *reinterpret_cast<float4 *>(pu) = make_float4(uv[0], uv[1], uv[2], uv[3]);
            *reinterpret_cast<float4 *>(pl) = make_float4(lv[0], lv[1], lv[2], lv[3]);
          } else {
            *reinterpret_cast<float2 *>(pu) = make_float2(uv[0], uv[1]);
            *reinterpret_cast<float2 *>(pl) = make_float2(lv[0], lv[1]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < CW; ++i)
            if (c + i < bJ) {
              pu[i] = uv[i];
              pl[i] = lv[i];
            }
        }
      }
    }
  }

  // The cells also at their transposed positions (j0 + c, a0 + a), for the
  // stale copy of an off-diagonal tile when this is the last launch of the
  // pass to write it.  Each matrix is turned around in the LDS tile `tr`
  // (stride BK + 1) so that the global writes are row segments.  Contains
  // barriers: every thread of the workgroup calls it.
  static __device__ __forceinline__ void store_transposed(float *Ub, float *Lb, int64_t n,
                                                          int64_t a0, int64_t j0, int bA, int bJ,
                                                          int tid, const float (&u)[RT][CT],
                                                          const float (&l)[RT][CT],
                                                          float (*tr)[BK + 1]) {
    int tw = tid;
    asm volatile("" : "+v"(tw));
    const int wy = tw / NTX, wx = tw % NTX;
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
      __syncthreads();  // tr free (the staging, or the previous matrix)
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int q = 0; q < CT; ++q)
          tr[wx * CT + q][wy * RT + r] = mat ? lower_out<RU>(l[r][q]) : u[r][q];
      __syncthreads();
      float *M = mat ? Lb : Ub;
      // row c of the transposed block: BK / 4 float4 per row, NT threads
#pragma unroll
      for (int it = 0; it < BK * BK / 4 / NT; ++it) {
        const int e = tw + it * NT, c = e / (BK / 4), a = (e % (BK / 4)) * 4;
        if (c >= bJ) continue;
        float *p = M + (j0 + c) * n + a0 + a;
        if (VEC && a + 3 < bA) {
          *reinterpret_cast<float4 *>(p) =
              make_float4(tr[c][a], tr[c][a + 1], tr[c][a + 2], tr[c][a + 3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (a + i < bA) p[i] = tr[c][a + i];
        }
      }
    }
  }
};

// Bulk of phase 3 for the dense layout: the atoms of k-blocks K .. K+nk-1 in
// order on every fresh cell outside the bands [X0, X1), as the four BK x BK
// quadrants of each upper TILE x TILE tile (grid.x = bulk_workgroups(T), in
// the order of bulk_quadrant; grid.y = molecules).  [X0, X1) starts with the atoms' own bands, whose rows are
// final, and goes on over the bands updated ahead on the other stream.  A
// quadrant in any of them is skipped whole (quadrants and bands are both BK
// wide): it is neither read nor written, and the panel columns of the bands
// run ahead are not read, since the other stream may be updating exactly
// those cells while this launch runs.  Each quadrant is a Quad block.  With
// MIR (the last launch of a pass) a quadrant of an off-diagonal tile is
// also written at its transposed position, which leaves the stale tiles
// final (measured, b64n500 / n1024 / n12288 pass: a separate transposed-copy
// kernel after the pass took 37 / 15 / 330 us).
template <bool VEC, bool RU, int RT, int CT, int KCH, bool MIR>
__global__ __launch_bounds__((BK / RT) * (BK / CT)) void k_quads(float *__restrict__ U,
                                                                 float *__restrict__ L,
                                                                 int64_t n, int64_t batch,
                                                                 int64_t K, int64_t nk,
                                                                 int64_t X0, int64_t X1,
                                                                 int xcd) {
  using Q = Quad<VEC, RU, RT, CT, KCH>;
  __shared__ union {
    typename Q::Stage sm;
    float tr[MIR ? BK : 1][BK + 1];  // the transposed write-back (MIR only)
  } lds;
  auto &sm = lds.sm;

  rounding_prologue<RU>();
  const int tid = threadIdx.x, ty = tid / Q::NTX, tx = tid % Q::NTX;
  int64_t A, B;
  bool lower_left;
  if (!bulk_quadrant(blockIdx.x, n, xcd, A, B, lower_left) || A * BK >= n || B * BK >= n ||
      (A >= X0 && A < X1) || (B >= X0 && B < X1) || lower_left)
    return;  // uniform over the workgroup, before any barrier
  const int64_t k0 = K * BK, a0 = A * BK, j0 = B * BK;
  const int bK = (int)(n - k0 < nk * BK ? n - k0 : nk * BK);
  const int bA = (int)(n - a0 < BK ? n - a0 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = L + b * nn;
    float u[RT][CT], l[RT][CT];
    Q::load(Ub, Lb, n, a0, j0, bA, bJ, ty, tx, u, l);
    Q::relax(sm, Ub, Lb, n, k0, bK, a0, j0, bA, bJ, tid, ty, tx, u, l);
    Q::store(Ub, Lb, n, a0, j0, bA, bJ, tid, u, l);
    if constexpr (MIR) {
      if (!fresh(B, A))  // uniform: the quadrant's mirror is stale
        Q::store_transposed(Ub, Lb, n, a0, j0, bA, bJ, tid, u, l, lds.tr);
    }
    __syncthreads();
  }
}

// Phase 1 of k-block Z on a Quad block's cells: the closure of the diagonal
// tile (Z, Z) over its own atoms, in order, by the plain rounds of the
// notes' §3 restricted to the tile.  Row m is published through LDS (dv,
// double-buffered, one barrier per round); column m equals row m by
// symmetry.  Cells outside the matrix are neutral and stay so.  Contains
// barriers: every thread of the workgroup calls it.
template <bool RU, int RT, int CT>
__device__ __forceinline__ void close_tile(float (*dv)[2][BK], int bZ, int ty, int tx,
                                           float (&u)[RT][CT], float (&l)[RT][CT]) {
  for (int mb = 0; mb * RT < bZ; ++mb) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int m = mb * RT + r;
      if (m >= bZ) break;  // uniform
      const int buf = m & 1;
      if (ty == mb) {
#pragma unroll
        for (int q = 0; q < CT; ++q) {
          dv[buf][0][tx * CT + q] = u[r][q];
          dv[buf][1][tx * CT + q] = l[r][q];
        }
      }
      __syncthreads();
      float cu[RT], cl[RT], eu[CT], el[CT];
#pragma unroll
      for (int a = 0; a < RT; ++a) {
        cu[a] = dv[buf][0][ty * RT + a];  // D[a][m] = D[m][a]
        cl[a] = dv[buf][1][ty * RT + a];
      }
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        eu[q] = dv[buf][0][tx * CT + q];  // D[m][b]
        el[q] = dv[buf][1][tx * CT + q];
      }
#pragma unroll
      for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int q = 0; q < CT; ++q) relax1<RU>(u[a][q], l[a][q], cu[a], cl[a], eu[q], el[q]);
    }
  }
}

// The lead launch of the one-stream schedule for k-block K: phase 3 of K on
// every cell outside band K and outside the diagonal tile (Z, Z) of the next
// k-block Z = K + 1 (the dense bulk, grid.y = 1 + 4 T(T+1)/2 quadrants), and,
// in workgroup y = 0 of each molecule, that diagonal tile: phase 3 of K on it
// (the atoms of K from their finished panel rows), then phase 1 of Z (its
// closure).  The two parts touch disjoint cells and read only band K, which
// neither writes, so phase 1 of the next k-block runs beside this one's bulk
// instead of after it.  With K < 0 the launch is the closure of tile Z alone
// (the first k-block); with Z < 0 it is the bulk alone (the last, which with
// MIR also writes the transposed copies, as k_quads does).  The
// closure is on the critical path: grid.x = molecules, so that workgroups
// dispatch x-fastest and every molecule's closure starts first, and its
// waves raise their issue priority.
template <bool VEC, bool RU, int RT, int CT, int KCH, bool MIR>
__global__ __launch_bounds__((BK / RT) * (BK / CT)) void k_lead(float *__restrict__ U,
                                                                float *__restrict__ L,
                                                                int64_t n, int64_t batch,
                                                                int64_t K, int64_t Z,
                                                                uint32_t *infeasible) {
  using Q = Quad<VEC, RU, RT, CT, KCH>;
  __shared__ union {
    typename Q::Stage sm;
    float tr[MIR ? BK : 1][BK + 1];  // the transposed write-back (MIR only)
  } lds;
  auto &sm = lds.sm;
  __shared__ __align__(16) float dv[2][2][BK];

  rounding_prologue<RU>();
  const int tid = threadIdx.x, ty = tid / Q::NTX, tx = tid % Q::NTX;
  const int64_t nn = n * n;
  if (blockIdx.y == 0) {
    if (Z < 0) return;  // uniform
    critical_path_priority();
    const int64_t z0 = Z * BK, k0 = K * BK;
    const int bZ = (int)(n - z0 < BK ? n - z0 : BK);
    const int bK = K < 0 ? 0 : (int)(n - k0 < BK ? n - k0 : BK);
    for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
      float *Ub = U + b * nn;
      float *Lb = L + b * nn;
      float u[RT][CT], l[RT][CT];
      Q::load(Ub, Lb, n, z0, z0, bZ, bZ, ty, tx, u, l);
      if (K >= 0) Q::relax(sm, Ub, Lb, n, k0, bK, z0, z0, bZ, bZ, tid, ty, tx, u, l);
      close_tile<RU>(dv, bZ, ty, tx, u, l);
      if (infeasible) flag_infeasible<RT, CT>(infeasible + b, bZ, ty, tx, u, l);
      Q::store(Ub, Lb, n, z0, z0, bZ, bZ, tid, u, l);
      __syncthreads();
    }
    return;
  }
  if (K < 0) return;
  const int64_t p = (blockIdx.y - 1) >> 2, qd = (blockIdx.y - 1) & 3;
  const int64_t J2 = tri_col(p), I2 = p - J2 * (J2 + 1) / 2;
  const int64_t A = RATIO * I2 + (qd >> 1), B = RATIO * J2 + (qd & 1);
  if (A * BK >= n || B * BK >= n || A == K || B == K || (A == Z && B == Z) ||
      (I2 == J2 && qd == 2))
    return;  // uniform over the workgroup, before any barrier
  const int64_t k0 = K * BK, a0 = A * BK, j0 = B * BK;
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int bA = (int)(n - a0 < BK ? n - a0 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
    float *Ub = U + b * nn;
    float *Lb = L + b * nn;
    float u[RT][CT], l[RT][CT];
    Q::load(Ub, Lb, n, a0, j0, bA, bJ, ty, tx, u, l);
    Q::relax(sm, Ub, Lb, n, k0, bK, a0, j0, bA, bJ, tid, ty, tx, u, l);
    Q::store(Ub, Lb, n, a0, j0, bA, bJ, tid, u, l);
    if constexpr (MIR) {
      if (!fresh(B, A))  // uniform: the quadrant's mirror is stale
        Q::store_transposed(Ub, Lb, n, a0, j0, bA, bJ, tid, u, l, lds.tr);
    }
    __syncthreads();
  }
}

// Phase 2 of k-block K with its diagonal tile D* = (K, K) already closed: the
// panel tile R = (K, J) (grid.x = the k-blocks J other than K, grid.y =
// molecules) becomes
//   R*[a][c] = min(R[a][c], min_m D*[a][m] + R[m][c])              (upper)
//   L*[a][c] = max(L[a][c], max_m L_D*[a][m] - U_R[m][c], L_R[m][c] - U_D*[a][m])
// over the atoms m of band K, with R as it was before this phase on the
// right-hand side.  In the graph view (the 2n-vertex digraph whose shortest
// paths the fused rounds compute) these are the paths from band K's vertices
// through band K to J's, split at the last atom of band K they visit, so on
// the 2^-6 grid this equals running the rounds of band K in order over the
// panel tile, which the phase 1-2 kernel does.  Unlike those rounds the
// products need no barrier per atom: D* and R are staged in LDS whole, and
// every thread relaxes its cells over the atoms as the bulk does.  R is
// read from its fresh orientation and written in its row orientation, which
// the bulk of K reads, and in the other one where that is fresh (J < K) or
// where block J is past the end Kend of the pass or range (dense).  For
// K < J < Kend the other copy stays stale: no launch reads it before the
// phase 2 of J rewrites tile (J, K).  Packed: as its U and L slots.
// Thread (ty, tx) owns 4 x CT cells of R.  CT = 4 (256 threads) runs beside
// the bulk (the two-step look-ahead); CT = 2 (512 threads, dense layout)
// where the launch has the chip to itself: D* and R take 64 KB of LDS, so a
// compute unit holds two workgroups, and 4x2 cells give its SIMDs four waves
// each instead of two to issue from.
template <int CT>
constexpr int product_threads() { return (BK / 4) * (BK / CT); }

template <bool VEC, bool PK, bool RU, int CT>
__global__ __launch_bounds__(product_threads<CT>()) void k_product(float *__restrict__ U,
                                                                   float *__restrict__ L,
                                                                   int64_t n, int64_t batch,
                                                                   int64_t K, int64_t Kend) {
  static_assert(CT == 4 || (CT == 2 && !PK), "4x4 cells, or 4x2 on the dense layout");
  constexpr int NTX = BK / CT, NTH = product_threads<CT>();
  __shared__ __align__(16) float su[2][BK][BK];  // D* rows: su[.][m][a] = U/L D*[m][a]
  __shared__ __align__(16) float sr[2][BK][BK];  // R rows:  sr[.][m][c] = U/L R[m][c]
  float(*tr)[BK + 1] = reinterpret_cast<float(*)[BK + 1]>(&su[0][0][0]);  // write-back

  rounding_prologue<RU>();
  // beside the bulk (two steps ahead) its waves take issue priority, as the
  // phase 1-2 kernel's do (n12288 pass 67.15-67.17 ms against 67.6-67.7)
  critical_path_priority();
  const int tid = threadIdx.x, ty = tid / NTX, tx = tid % NTX;
  int64_t J = blockIdx.x;
  if (J >= K) ++J;
  const int64_t k0 = K * BK, j0 = J * BK;
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  const bool rowor = fresh(K, J);
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = PK ? Ub : L + b * nn;

    // D* straight into LDS, one row segment of four at a time (rows of the
    // dense diagonal tile; the packed one through its logical cells)
    if constexpr (PK) {
      float du[4][4], dl[4][4];
      packed_block_load<VEC>(Ub, n, k0, k0, bK, bK, ty, tx, du, dl);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<float4 *>(&su[0][ty * 4 + r][tx * 4]) =
            make_float4(du[r][0], du[r][1], du[r][2], du[r][3]);
        *reinterpret_cast<float4 *>(&su[1][ty * 4 + r][tx * 4]) =
            make_float4(dl[r][0], dl[r][1], dl[r][2], dl[r][3]);
      }
    } else {
#pragma unroll
      for (int it = 0; it < BK * BK / 4 / NTH; ++it) {
        const int e = tid + it * NTH, a = e / (BK / 4), c = (e % (BK / 4)) * 4;
        const int64_t g = (k0 + a) * n + k0 + c;
        const int cnt = a < bK ? clamp4(bK - c) : 0;
        *reinterpret_cast<float4 *>(&su[0][a][c]) = load4<VEC>(Ub + g, cnt, kInf, Ub);
        *reinterpret_cast<float4 *>(&su[1][a][c]) = load4<VEC>(Lb + g, cnt, 0.0f, Lb);
      }
    }
    // this thread's 4 x CT cells of R, the logical cells (k0 + 4ty + r, j0 + CT*tx + q)
    float u[4][CT], l[4][CT];
    if constexpr (PK) {
      packed_block_load<VEC>(Ub, n, k0, j0, bK, bJ, ty, tx, u, l);
    } else if (rowor) {  // row segments M[k0 + a][j0 + c ..]
      Seg<CT> yu[4], yl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t left = ty * 4 + r < bK ? bJ - tx * CT : 0;
        const int64_t g = (k0 + ty * 4 + r) * n + j0 + tx * CT;
        yu[r] = load_seg<VEC, CT>(Ub + g, left, kInf, Ub);
        yl[r] = load_seg<VEC, CT>(Lb + g, left, 0.0f, Lb);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < CT; ++q) {
          u[r][q] = yu[r].v[q];
          l[r][q] = yl[r].v[q];
        }
    } else {  // column segments M[j0 + c][k0 + a ..] of the other orientation
      float4 yu[CT], yl[CT];
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        const int c = tx * CT + q;
        const int cnt = c < bJ ? clamp4(bK - ty * 4) : 0;
        const int64_t g = (j0 + c) * n + k0 + ty * 4;
        yu[q] = load4<VEC>(Ub + g, cnt, kInf, Ub);
        yl[q] = load4<VEC>(Lb + g, cnt, 0.0f, Lb);
      }
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        const float bu[4] = {yu[q].x, yu[q].y, yu[q].z, yu[q].w};
        const float bl[4] = {yl[q].x, yl[q].y, yl[q].z, yl[q].w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u[r][q] = bu[r];
          l[r][q] = bl[r];
        }
      }
    }
    // CT consecutive floats of an LDS row, as one vector
    auto put = [](float *p, const float *v) {
      if constexpr (CT == 4)
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
      else
        *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
    };
    auto get = [](const float *p, float *v) {
      if constexpr (CT == 4) {
        const float4 x = *reinterpret_cast<const float4 *>(p);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      } else {
        const float2 x = *reinterpret_cast<const float2 *>(p);
        v[0] = x.x; v[1] = x.y;
      }
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      put(&sr[0][ty * 4 + r][tx * CT], u[r]);
      put(&sr[1][ty * 4 + r][tx * CT], l[r]);
    }
    __syncthreads();

    // atoms past bK carry the neutral values (+inf above, 0 below), so the
    // loop may run over whole pairs
#pragma unroll 2
    for (int m = 0; m < bK; m += 2) {
      const float4 a0v = *reinterpret_cast<const float4 *>(&su[0][m][ty * 4]);
      const float4 b0v = *reinterpret_cast<const float4 *>(&su[1][m][ty * 4]);
      const float4 a1v = *reinterpret_cast<const float4 *>(&su[0][m + 1][ty * 4]);
      const float4 b1v = *reinterpret_cast<const float4 *>(&su[1][m + 1][ty * 4]);
      float ru0[CT], rl0[CT], ru1[CT], rl1[CT];
      get(&sr[0][m][tx * CT], ru0);
      get(&sr[1][m][tx * CT], rl0);
      get(&sr[0][m + 1][tx * CT], ru1);
      get(&sr[1][m + 1][tx * CT], rl1);
      const float cu0[4] = {a0v.x, a0v.y, a0v.z, a0v.w}, cl0[4] = {b0v.x, b0v.y, b0v.z, b0v.w};
      const float cu1[4] = {a1v.x, a1v.y, a1v.z, a1v.w}, cl1[4] = {b1v.x, b1v.y, b1v.z, b1v.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < CT; ++q)
          relax2<RU>(u[r][q], l[r][q], cu0[r], cl0[r], ru0[q], rl0[q], cu1[r], cl1[r], ru1[q],
                     rl1[q]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < CT; ++q) l[r][q] = lower_out<RU>(l[r][q]);

    // write-back (tr aliases su, free once every thread has left the loop,
    // which store_transposed's first barrier ensures)
    int tw = tid;
    asm volatile("" : "+v"(tw));
    const int wy = tw / NTX, wx = tw % NTX;
    if constexpr (PK) {
      // R lies on one side of the diagonal: its row slots hold U right of
      // it, L left of it
      if (k0 < j0) {
        store_rows<VEC>(Ub, n, k0, j0, bK, bJ, wy, wx, u);
        store_transposed<VEC>(Ub, n, k0, j0, bK, bJ, wy, wx, l, tr);
      } else {
        store_rows<VEC>(Ub, n, k0, j0, bK, bJ, wy, wx, l);
        store_transposed<VEC>(Ub, n, k0, j0, bK, bJ, wy, wx, u, tr);
      }
    } else {
      store_rows<VEC, CT>(Ub, n, k0, j0, bK, bJ, wy, wx, u);
      store_rows<VEC, CT>(Lb, n, k0, j0, bK, bJ, wy, wx, l);
      if (J < K || J >= Kend) {  // uniform: the other orientation is read
        store_transposed<VEC, CT>(Ub, n, k0, j0, bK, bJ, wy, wx, u, tr);
        store_transposed<VEC, CT>(Lb, n, k0, j0, bK, bJ, wy, wx, l, tr);
      }
    }
    __syncthreads();  // LDS reuse by the next molecule
  }
}

// Phase 2 of k-block K as k_product computes it (dense layout), with each
// panel tile's columns split over P workgroups: workgroup (J, h) stages D*
// whole and the W = BK / P columns h*W .. of R, and relaxes 4 x (W / 16)
// cells per thread on 256 threads.  Where a product launch has fewer
// workgroups than the chip has CUs, this spreads each tile over P of them.
// R's slice is staged through LDS from its fresh orientation (lanes along
// the slice's rows or columns, so both reads are row segments) and written
// back the same way, in its row orientation and, left of the diagonal, in
// the other one (as k_product).
template <bool VEC, bool RU, int P>
__global__ __launch_bounds__(256) void k_product_slice(float *__restrict__ U,
                                                      float *__restrict__ L, int64_t n,
                                                      int64_t batch, int64_t K, int64_t Kend) {
  static_assert(P == 2 || P == 4, "two or four column slices");
  constexpr int W = BK / P, CT = W / 16;  // slice columns, cells per thread along them
  __shared__ __align__(16) float su[2][BK][BK];  // D* rows: su[.][m][a] = U/L D*[m][a]
  __shared__ __align__(16) float sr[2][BK][W];   // the slice's rows: sr[.][m][c] = R[m][c]
  __shared__ float tt[2][W][BK + 1];             // the slice turned around for its copy

  rounding_prologue<RU>();
  critical_path_priority();
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  int64_t J = blockIdx.x / P;
  if (J >= K) ++J;
  const int64_t k0 = K * BK, c0 = J * BK + (blockIdx.x % P) * W;
  if (c0 >= n) return;  // uniform: a slice past the matrix
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int bW = (int)(n - c0 < W ? n - c0 : W);
  const bool rowor = fresh(K, J);
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = L + b * nn;
    // D* straight into LDS, one row segment of four at a time
#pragma unroll
    for (int it = 0; it < BK * BK / 4 / 256; ++it) {
      const int e = tid + it * 256, a = e / (BK / 4), c = (e % (BK / 4)) * 4;
      const int64_t g = (k0 + a) * n + k0 + c;
      const int cnt = a < bK ? clamp4(bK - c) : 0;
      *reinterpret_cast<float4 *>(&su[0][a][c]) = load4<VEC>(Ub + g, cnt, kInf, Ub);
      *reinterpret_cast<float4 *>(&su[1][a][c]) = load4<VEC>(Lb + g, cnt, 0.0f, Lb);
    }
    // the slice from its fresh orientation: R[a][c] = M[k0+a][c0+c] (lanes
    // along c), else M[c0+c][k0+a] (lanes along a)
#pragma unroll
    for (int it = 0; it < BK * W / 256; ++it) {
      const int e = tid + it * 256;
      const int a = rowor ? e / W : e % BK, c = rowor ? e % W : e / BK;
      const bool in = a < bK && c < bW;
      const int64_t g = in ? (rowor ? (k0 + a) * n + c0 + c : (c0 + c) * n + k0 + a) : 0;
      const float xu = Ub[g], xl = Lb[g];
      sr[0][a][c] = in ? xu : kInf;
      sr[1][a][c] = in ? xl : 0.0f;
    }
    __syncthreads();
    // this thread's cells: rows 4ty + r, columns CT*tx + q of the slice
    float u[4][CT], l[4][CT];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        u[r][q] = sr[0][ty * 4 + r][tx * CT + q];
        l[r][q] = sr[1][ty * 4 + r][tx * CT + q];
      }
    // atoms past bK carry the neutral values (+inf above, 0 below)
#pragma unroll 2
    for (int m = 0; m < bK; m += 2) {
      const float4 a0v = *reinterpret_cast<const float4 *>(&su[0][m][ty * 4]);
      const float4 b0v = *reinterpret_cast<const float4 *>(&su[1][m][ty * 4]);
      const float4 a1v = *reinterpret_cast<const float4 *>(&su[0][m + 1][ty * 4]);
      const float4 b1v = *reinterpret_cast<const float4 *>(&su[1][m + 1][ty * 4]);
      float ru0[CT], rl0[CT], ru1[CT], rl1[CT];
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        ru0[q] = sr[0][m][tx * CT + q];
        rl0[q] = sr[1][m][tx * CT + q];
        ru1[q] = sr[0][m + 1][tx * CT + q];
        rl1[q] = sr[1][m + 1][tx * CT + q];
      }
      const float cu0[4] = {a0v.x, a0v.y, a0v.z, a0v.w}, cl0[4] = {b0v.x, b0v.y, b0v.z, b0v.w};
      const float cu1[4] = {a1v.x, a1v.y, a1v.z, a1v.w}, cl1[4] = {b1v.x, b1v.y, b1v.z, b1v.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < CT; ++q)
          relax2<RU>(u[r][q], l[r][q], cu0[r], cl0[r], ru0[q], rl0[q], cu1[r], cl1[r], ru1[q],
                     rl1[q]);
    }
    // the slice's rows through sr, its other orientation through tt
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        const float lo = lower_out<RU>(l[r][q]);
        tt[0][tx * CT + q][ty * 4 + r] = u[r][q];
        tt[1][tx * CT + q][ty * 4 + r] = lo;
        l[r][q] = lo;
      }
    __syncthreads();  // every thread has left the loop: sr may be rewritten
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        sr[0][ty * 4 + r][tx * CT + q] = u[r][q];
        sr[1][ty * 4 + r][tx * CT + q] = l[r][q];
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < BK * W / 256; ++it) {
      const int e = tid + it * 256;
      const int a = e / W, c = e % W;  // rows of band K, lanes along c
      if (a < bK && c < bW) {
        Ub[(k0 + a) * n + c0 + c] = sr[0][a][c];
        Lb[(k0 + a) * n + c0 + c] = sr[1][a][c];
      }
      const int at = e % BK, ct = e / BK;  // the other orientation, lanes along a
      if ((J < K || J >= Kend) && at < bK && ct < bW) {  // (as k_product)
        Ub[(c0 + ct) * n + k0 + at] = tt[0][ct][at];
        Lb[(c0 + ct) * n + k0 + at] = tt[1][ct][at];
      }
    }
    __syncthreads();  // LDS reuse by the next molecule
  }
}

// One BK x BK block of the packed layout (one buffer P: U above the
// diagonal, L below) as phase 3 handles it, 4x4 cells per thread on 256
// threads.  An off-diagonal block (a0 < j0) reads its U as row segments
// P[a0+a][j0..] and its L as column segments P[j0+c][a0..] (float4 along a,
// turned around in registers), and writes them back the same way, the L half
// through an LDS tile so that the global writes are row segments.  A
// diagonal block (a0 == j0) loads the same segments, swaps U and L of its
// cells left of the diagonal, and writes its rows only (they cover both
// halves).  The panel rows of the atoms lie right or left of the diagonal,
// so each staged half is a row segment of P and a column segment read four
// atoms per float4 (packed_half_load).  Used by the packed bulk
// (k_quads_packed) and the packed lead launch (k_lead_packed).
template <bool VEC, bool RU>
struct PQuad {
  struct Stage {
    float4 cu[KC][BK / 4], cl[KC][BK / 4], ru[KC][BK / 4], rl[KC][BK / 4];
  };

  static __device__ __forceinline__ void load(const float *Pb, int64_t n, int64_t a0, int64_t j0,
                                              int bA, int bJ, int ty, int tx, bool diag,
                                              float (&u)[4][4], float (&l)[4][4]) {
    float4 x[4], y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = ty * 4 + r;
      x[r] = load4<VEC>(Pb + (a0 + a) * n + j0 + tx * 4, a < bA ? clamp4(bJ - tx * 4) : 0,
                        kInf, Pb);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tx * 4 + q;
      y[q] = load4<VEC>(Pb + (j0 + c) * n + a0 + ty * 4, c < bJ ? clamp4(bA - ty * 4) : 0,
                        0.0f, Pb);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float xr[4] = {x[r].x, x[r].y, x[r].z, x[r].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) u[r][q] = xr[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float yq[4] = {y[q].x, y[q].y, y[q].z, y[q].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) l[r][q] = yq[r];
    }
    if (diag) {
      // left of the diagonal the row segment holds L and the column one U
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (ty * 4 + r > tx * 4 + q) {
            const float t = u[r][q];
            u[r][q] = l[r][q];
            l[r][q] = t;
          }
    }
  }

  // The atoms k0 .. k0+bK-1 (band K's, or a step's from K on) applied to the
  // cells of block (A, B); A and B are outside the atoms' bands.  Contains
  // barriers: every thread of the workgroup calls it.
  static __device__ __forceinline__ void relax(Stage &sm, const float *Pb, int64_t n,
                                               int64_t k0, int bK, int64_t K, int64_t A,
                                               int64_t B, int64_t a0, int64_t j0, int tid,
                                               int ty, int tx, float (&u)[4][4],
                                               float (&l)[4][4]) {
    // the staging addresses are re-derived per chunk (laundered thread
    // index) rather than kept live through the k loop.  A whole interior
    // chunk loads from two 32-bit offsets without masks (73.1-73.8 ms per
    // packed pass at n12288, against 74.6-74.9 masked; with the offsets kept
    // live through the loop, as the dense bulk does, it was slower: 78.8 ms)
    HalfLoad hl[2];
    auto fetch = [&](int kc) {
      int tf = tid;
      asm volatile("" : "+v"(tf));
      if (VEC && kc + KC <= bK && a0 + BK <= n && j0 + BK <= n) {  // uniform
        const uint32_t od = half_direct_offset(n, tf), oa = half_across_offset(n, tf);
        hl[0] = packed_half_load_whole(Pb, n, k0 + kc, a0, od, oa);
        hl[1] = packed_half_load_whole(Pb, n, k0 + kc, j0, od, oa);
      } else {
        hl[0] = packed_half_load<VEC>(Pb, n, k0, kc, bK, a0, A > K, false, tf);
        hl[1] = packed_half_load<VEC>(Pb, n, k0, kc, bK, j0, B > K, false, tf);
      }
    };
    fetch(0);
    for (int kc = 0; kc < bK; kc += KC) {
      int ts = tid;
      asm volatile("" : "+v"(ts));
      packed_half_store(hl[0], A > K, reinterpret_cast<float *>(&sm.cu[0][0]),
                        reinterpret_cast<float *>(&sm.cl[0][0]), BK, 0, ts);
      packed_half_store(hl[1], B > K, reinterpret_cast<float *>(&sm.ru[0][0]),
                        reinterpret_cast<float *>(&sm.rl[0][0]), BK, 0, ts);
      __syncthreads();
      if (kc + KC < bK) fetch(kc + KC);  // in flight during this chunk
#pragma unroll 2
      for (int kk = 0; kk < KC; kk += 2) {
        const float4 a0v = sm.cu[kk][ty], b0 = sm.cl[kk][ty], c0 = sm.ru[kk][tx],
                     d0 = sm.rl[kk][tx];
        const float4 a1 = sm.cu[kk + 1][ty], b1 = sm.cl[kk + 1][ty], c1 = sm.ru[kk + 1][tx],
                     d1 = sm.rl[kk + 1][tx];
        const float cu0[4] = {a0v.x, a0v.y, a0v.z, a0v.w}, cl0[4] = {b0.x, b0.y, b0.z, b0.w};
        const float ru0[4] = {c0.x, c0.y, c0.z, c0.w}, rl0[4] = {d0.x, d0.y, d0.z, d0.w};
        const float cu1[4] = {a1.x, a1.y, a1.z, a1.w}, cl1[4] = {b1.x, b1.y, b1.z, b1.w};
        const float ru1[4] = {c1.x, c1.y, c1.z, c1.w}, rl1[4] = {d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            relax2<RU>(u[r][q], l[r][q], cu0[r], cl0[r], ru0[q], rl0[q], cu1[r], cl1[r], ru1[q],
                       rl1[q]);
      }
      __syncthreads();
    }
  }

  // write-back: the addresses are computed after the k loop, not kept live
  // in it.  Contains barriers: every thread of the workgroup calls it.
  static __device__ __forceinline__ void store(float *Pb, int64_t n, int64_t a0, int64_t j0,
                                               int bA, int bJ, int tid, bool diag,
                                               float (&u)[4][4], float (&l)[4][4],
                                               float (*tr)[BK + 1]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) l[r][q] = lower_out<RU>(l[r][q]);
    int tw = tid;
    asm volatile("" : "+v"(tw));
    const int wy = tw >> 4, wx = tw & 15;
    if (diag) {
      store_packed_diagonal<VEC>(Pb, n, a0, bA, wy, wx, u, l);
    } else {
      store_rows<VEC>(Pb, n, a0, j0, bA, bJ, wy, wx, u);
      store_transposed<VEC>(Pb, n, a0, j0, bA, bJ, wy, wx, l, tr);
    }
  }
};

// Bulk of phase 3 for the packed layout on the same quadrants as k_quads,
// each a PQuad block; the lower-left quadrant of a diagonal tile is left
// out, since its slots are the upper-right one's.
template <bool VEC, bool RU>
__global__ __launch_bounds__(kThreads) void k_quads_packed(float *__restrict__ P, int64_t n,
                                                           int64_t batch, int64_t K, int64_t nk,
                                                           int64_t X0, int64_t X1, int xcd) {
  using Q = PQuad<VEC, RU>;
  __shared__ typename Q::Stage sm;
  __shared__ float tr[BK][BK + 1];  // write-back of the L half

  rounding_prologue<RU>();
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  int64_t A, B;
  bool lower_left;
  if (!bulk_quadrant(blockIdx.x, n, xcd, A, B, lower_left) || A * BK >= n || B * BK >= n ||
      (A >= X0 && A < X1) || (B >= X0 && B < X1) || lower_left)
    return;  // uniform over the workgroup, before any barrier
  const int64_t k0 = K * BK, a0 = A * BK, j0 = B * BK;
  const int bK = (int)(n - k0 < nk * BK ? n - k0 : nk * BK);
  const int bA = (int)(n - a0 < BK ? n - a0 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  const bool diag = A == B;  // else A < B: every cell lies above the diagonal
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Pb = P + b * nn;
    float u[4][4], l[4][4];
    Q::load(Pb, n, a0, j0, bA, bJ, ty, tx, diag, u, l);
    Q::relax(sm, Pb, n, k0, bK, K, A, B, a0, j0, tid, ty, tx, u, l);
    Q::store(Pb, n, a0, j0, bA, bJ, tid, diag, u, l, tr);
    __syncthreads();  // tr and the staging arrays are reused by the next molecule
  }
}

// The lead launch of the one-stream schedule on the packed layout: k_lead
// with PQuad blocks (quadrants of the upper tiles, less the lower-left one
// of each diagonal tile; the closure workgroup's tile is a diagonal block).
template <bool VEC, bool RU>
__global__ __launch_bounds__(kThreads) void k_lead_packed(float *__restrict__ P, int64_t n,
                                                          int64_t batch, int64_t K, int64_t Z,
                                                          uint32_t *infeasible) {
  using Q = PQuad<VEC, RU>;
  __shared__ typename Q::Stage sm;
  __shared__ float tr[BK][BK + 1];
  __shared__ __align__(16) float dv[2][2][BK];

  rounding_prologue<RU>();
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t nn = n * n;
  if (blockIdx.y == 0) {
    if (Z < 0) return;  // uniform
    critical_path_priority();
    const int64_t z0 = Z * BK, k0 = K * BK;
    const int bZ = (int)(n - z0 < BK ? n - z0 : BK);
    const int bK = K < 0 ? 0 : (int)(n - k0 < BK ? n - k0 : BK);
    for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
      float *Pb = P + b * nn;
      float u[4][4], l[4][4];
      Q::load(Pb, n, z0, z0, bZ, bZ, ty, tx, true, u, l);
      if (K >= 0) Q::relax(sm, Pb, n, k0, bK, K, Z, Z, z0, z0, tid, ty, tx, u, l);
      close_tile<RU>(dv, bZ, ty, tx, u, l);
      if (infeasible) flag_infeasible<4, 4>(infeasible + b, bZ, ty, tx, u, l);
      Q::store(Pb, n, z0, z0, bZ, bZ, tid, true, u, l, tr);
      __syncthreads();
    }
    return;
  }
  if (K < 0) return;
  const int64_t p = (blockIdx.y - 1) >> 2, qd = (blockIdx.y - 1) & 3;
  const int64_t J2 = tri_col(p), I2 = p - J2 * (J2 + 1) / 2;
  const int64_t A = RATIO * I2 + (qd >> 1), B = RATIO * J2 + (qd & 1);
  if (A * BK >= n || B * BK >= n || A == K || B == K || (A == Z && B == Z) ||
      (I2 == J2 && qd == 2))
    return;  // uniform over the workgroup, before any barrier
  const int64_t k0 = K * BK, a0 = A * BK, j0 = B * BK;
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int bA = (int)(n - a0 < BK ? n - a0 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  const bool diag = A == B;
  for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
    float *Pb = P + b * nn;
    float u[4][4], l[4][4];
    Q::load(Pb, n, a0, j0, bA, bJ, ty, tx, diag, u, l);
    Q::relax(sm, Pb, n, k0, bK, K, A, B, a0, j0, tid, ty, tx, u, l);
    Q::store(Pb, n, a0, j0, bA, bJ, tid, diag, u, l, tr);
    __syncthreads();
  }
}

// The dense bulk's register tile.
// (measured at n12288, bulk launch: 4x4 419 us at 4 workgroups per CU; 4x8
// and 8x4 with 8-atom chunks 422-428 us at 3; 4x8, 8x4 with 16-atom chunks
// 484-494 us at 2; 8x8 needs more than 256 VGPRs)
constexpr int kBulkRT = 4, kBulkCT = 4, kBulkKC = 16;
// A bulk launch on one stream with few quadrant workgroups leaves its SIMDs
// one or two waves each: there each quadrant takes 512 threads with 4x2
// cells instead of 256 with 4x4.  Plain bulk launches, up to kSmallGrid
// quadrants (measured at n1024, 144 quadrants, bulk launch: 4x4 17.3 us,
// 2x2 15.6 us with the whole k-block staged at once, 2x4 13.3 us, 4x2
// 13.2 us; passes at 312 and 420 quadrants, n1536 and n1792, 2 % faster
// with 4x4).  Lead launches, up to kSmallLeadGrid quadrants, the 4x4
// workgroups the chip holds at once (passes, 4x2 against 4x4: n2048, 544
// quadrants, 1.26 against 1.44 ms; 64 x n256, 768, 0.199 against 0.225 ms;
// 24 x n500, 960, 0.427 against 0.435 ms; from 1088 quadrants 4x4 is
// faster: 2 x n2048 1.58 against 1.67 ms, n3072 2.35 against 2.48 ms).
constexpr int kSmallRT = 4, kSmallCT = 2, kSmallKC = 32;
constexpr int64_t kSmallGrid = 256, kSmallLeadGrid = 1024;

// The ordering events of a pass that runs part of its work on a second
// stream.  They only order the two streams of one device: the kernels they
// follow end with a device-scope release and the kernels that wait on them
// start with an acquire, so the events need no timing and no system-scope
// fence of their own (which writes back the caches and costs about 11 us per
// hop between the streams).
constexpr unsigned kOrderingEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

// A lane: the library's second stream for one caller stream on one device
// (default priority, non-blocking), and the events that order the two.  A
// lane is created on the first pass enqueued on that caller stream that needs
// it and kept for the life of the process; its mutex is held while a pass
// is enqueued through it, so that passes enqueued from several host threads
// on one caller stream do not interleave their event records.  Passes on
// different caller streams use different lanes and share nothing.
struct Lane {
  std::mutex mu;
  hipStream_t side = nullptr;
  // start: the fork from the caller's stream; bulk[t & 1]: bulk(t) done;
  // ready[t & 1]: the side stream's work that bulk(t) needs is done.  A
  // stream wait captures the event's state when it is enqueued, so the
  // events are re-recorded by every pass.
  hipEvent_t e[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  hipEvent_t &start() { return e[0]; }
  hipEvent_t &bulk(int64_t t) { return e[1 + (t & 1)]; }
  hipEvent_t &ready(int64_t t) { return e[3 + (t & 1)]; }
  bool init() {
    if (hipStreamCreateWithFlags(&side, hipStreamNonBlocking) != hipSuccess) {
      side = nullptr;
      return false;
    }
    for (auto &x : e)
      if (hipEventCreateWithFlags(&x, kOrderingEventFlags) != hipSuccess) return false;
    return true;
  }
};

// Lanes per device; passes on further caller streams run on one stream.
constexpr int kMaxLanes = 64;
constexpr int kMaxDevices = 64;

// The lane of caller stream `s` on the current device, locked; none (an
// unlocked guard) when no lane can be had.  A lane whose second stream is
// part of a graph capture that this pass does not belong to (a capture of
// another stream sharing the handle, still open) is not used either.
std::unique_lock<std::mutex> lock_lane(hipStream_t s, Lane **out) {
  *out = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return {};
  static std::mutex registry_mu;
  static std::map<std::pair<int, uintptr_t>, std::unique_ptr<Lane>> lanes;
  static int per_device[kMaxDevices];
  Lane *lane = nullptr;
  {
    std::lock_guard<std::mutex> g(registry_mu);
    const auto key = std::make_pair(dev, reinterpret_cast<uintptr_t>(s));
    auto it = lanes.find(key);
    if (it != lanes.end()) {
      lane = it->second.get();
    } else if (per_device[dev] < kMaxLanes) {
      auto fresh_lane = std::make_unique<Lane>();
      if (!fresh_lane->init()) return {};  // a half-made lane is dropped (its handles leak)
      lane = fresh_lane.get();
      lanes.emplace(key, std::move(fresh_lane));
      ++per_device[dev];
    }
  }
  if (!lane) return {};
  std::unique_lock<std::mutex> lk(lane->mu);
  hipStreamCaptureStatus cs_side = hipStreamCaptureStatusNone, cs_own = hipStreamCaptureStatusNone;
  unsigned long long id_side = 0, id_own = 0;
  if (hipStreamGetCaptureInfo(lane->side, &cs_side, &id_side) != hipSuccess ||
      hipStreamGetCaptureInfo(s, &cs_own, &id_own) != hipSuccess)
    return {};
  if (cs_side != hipStreamCaptureStatusNone &&
      (cs_own != hipStreamCaptureStatusActive || cs_side != hipStreamCaptureStatusActive ||
       id_own != id_side))
    return {};
  *out = lane;
  return lk;
}

}  // namespace

int step_blocks(int64_t n, int64_t batch, const Sched &sched) {
  if (sched.step_blocks > 0) return sched.step_blocks;
  if (lookahead_bands(n, batch, sched) != 2) return 1;
  const int64_t T = ceil_div(n, TILE), tiles = T * (T + 1) / 2 * batch;
  if (!sched.packed && batch > 1 && tiles >= kDeepTiles)
    return tiles >= kStep4Tiles ? 4 : tiles >= kStep2TilesBatch ? 2 : 1;
  if (!sched.packed && batch == 1 && tiles >= kDeepTilesSingle && tiles < kDeepTiles) return 1;
  return tiles >= kStep4Tiles ? 4 : tiles >= kStep3Tiles ? 3 : 2;
}

// The automatic choice of the lead schedule (for a one-stream pass of one
// k-block per step).
bool auto_lead(int64_t n, int64_t batch, bool packed) {
  const int64_t TB = ceil_div(n, BK), T = ceil_div(n, TILE);
  const int64_t tiles = T * (T + 1) / 2 * batch;
  if (!packed && batch >= 2 && tiles >= kLeadTilesMin && tiles < kDeepTiles) return true;
  // (molecules of one tile never run ahead: from kDeepTiles they keep this rule)
  return (batch >= 2 && (TB - 1) * batch > kPanelFill) ||
         (tiles >= (packed ? kLeadTilesMinPacked : kLeadTilesMin) && tiles < kLeadTilesMax);
}

bool lead_schedule(int64_t n, int64_t batch, const Sched &sched) {
  const int64_t TB = ceil_div(n, BK), T = ceil_div(n, TILE);
  // a lead launch's quadrants (and its closure) are one grid dimension
  if (TB <= 1 || 1 + 2 * T * (T + 1) > kMaxGridYZ || lookahead_bands(n, batch, sched) != 0 ||
      step_blocks(n, batch, sched) != 1)
    return false;
  if (sched.lead >= 0) return sched.lead == 1;
  return auto_lead(n, batch, sched.packed);
}

int lookahead_bands(int64_t n, int64_t batch, const Sched &sched) {
  const int64_t TB = ceil_div(n, BK), T = ceil_div(n, TILE);
  if (TB <= 1 || T <= 1) return 0;
  if (sched.lookahead >= 0) return sched.lookahead;
  const int64_t tiles = T * (T + 1) / 2 * batch;
  if (tiles >= kDeepTiles || (!sched.packed && batch == 1 && tiles >= kDeepTilesSingle)) return 2;
  // the lead schedule runs on one stream
  if (sched.step_blocks <= 1 &&
      (sched.lead == 1 || (sched.lead < 0 && auto_lead(n, batch, sched.packed))))
    return 0;
  // where one phase 1-2 launch fills the chip the batch splits over the two
  // streams instead (launch_blocked_on), in both layouts
  if (tiles < kAheadTiles || (TB - 1) * batch > kPanelFill) return 0;
  return 1;
}

// Enqueue one pass.  With more than one k-block the pass may run ahead on a
// second stream (lookahead_bands: by two steps when there are many phase-3
// tiles, one for a mid-sized bulk, none when the bulk is too short to hide a
// band strip or the phase 1-2 launch fills the chip; a batch then splits over
// the two streams).  A step is one
// k-block, or two when running two steps ahead: blocked Floyd-Warshall with
// 128 atoms per phase 3, whose panel (the rows of both bands, final for all
// 128 rounds) is built from the 64-wide phase 1-2 kernel and strips.  Per
// step t the caller's stream runs bulk(t): phase 3 of step t's blocks on
// everything but their bands and the bands run ahead.  Two steps ahead, the
// side stream runs phase 3 of step t on the bands of step t+1 (strip),
// step t+1's panel, then (once bulk(t-1) is done) phase 3 of step t on the
// bands of step t+2; bulk(t+1) waits only for the side stream's work before
// that, so step t+1's panel has all of bulk(t) to finish in.  One step
// ahead, the side stream waits for bulk(t-1), then runs the strip and the
// panel of step t+1 while bulk(t) runs.  The side work a bulk launch may
// overlap touches only bands it leaves alone and reads only panel rows it
// does not write; the CPU model of this schedule in the tests checks that
// cell by cell, for both depths.
namespace {
hipError_t launch_blocked_on(float *U, float *L, int64_t n, int64_t batch, int64_t K0, int64_t K1,
                             hipStream_t s, Prof *prof, unsigned flags, const Sched &sched,
                             bool half, uint32_t *infeasible);
}  // namespace

hipError_t launch_blocked(float *U, float *L, int64_t n, int64_t batch, int64_t K0, int64_t K1,
                          hipStream_t s, Prof *prof, unsigned flags, const Sched &sched,
                          uint32_t *infeasible) {
  Sched sc = sched;
  sc.packed = (flags & kPacked) != 0;
  return launch_blocked_on(U, L, n, batch, K0, K1, s, prof, flags, sc, false, infeasible);
}

namespace {
// `half`: one half of a split batch, run on one stream without look-ahead.
hipError_t launch_blocked_on(float *U, float *L, int64_t n, int64_t batch, int64_t K0, int64_t K1,
                             hipStream_t s, Prof *prof, unsigned flags, const Sched &sched,
                             bool half, uint32_t *infeasible) {
  static_assert(BK == kBlockRounds, "k-block size");
  const int64_t TB = ceil_div(n, BK);    // k-blocks
  if (K1 > TB) K1 = TB;
  if (n <= 1 || K0 >= K1) return hipSuccess;
  // the kernels' staging offsets are 32-bit (64 rows of n floats); such an
  // n would need more than 2^54 bytes per matrix
  if (n >= ((int64_t)1 << 26)) return hipErrorInvalidValue;
  const int64_t T = ceil_div(n, TILE);   // phase-3 tiles per side
  const bool packed = flags & kPacked, ru = flags & kDirected;
  const bool vec = (n % 4 == 0) && aligned16(U) && aligned16(L);
  const unsigned gy = (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ);
  const int64_t nn = n * n;
  if (packed) L = U;
  auto packed_kernel = ru ? (vec ? k_quads_packed<true, true> : k_quads_packed<false, true>)
                          : (vec ? k_quads_packed<true, false> : k_quads_packed<false, false>);
  // the dense bulk runs with larger register tiles
#define DBS_QUADS(R, C, KC, M)                                                               \
  (ru ? (vec ? k_quads<true, true, R, C, KC, M> : k_quads<false, true, R, C, KC, M>)          \
      : (vec ? k_quads<true, false, R, C, KC, M> : k_quads<false, false, R, C, KC, M>))
  auto quads_kernel = DBS_QUADS(kBulkRT, kBulkCT, kBulkKC, false);
  auto quads_last = DBS_QUADS(kBulkRT, kBulkCT, kBulkKC, true);
  unsigned quads_block = (BK / kBulkRT) * (BK / kBulkCT);
  auto strip_kernel =
      packed ? (ru ? (vec ? k_strip<true, true, true> : k_strip<false, true, true>)
                   : (vec ? k_strip<true, true, false> : k_strip<false, true, false>))
             : (ru ? (vec ? k_strip<true, false, true> : k_strip<false, false, true>)
                   : (vec ? k_strip<true, false, false> : k_strip<false, false, false>));
  // With many phase-3 tiles the bulk runs long enough to hide phases 1-2 of
  // the next blocks: they run two steps ahead, on 256-thread workgroups that
  // fit where phase-3 workgroups finish.  With fewer tiles they are the
  // critical path: one step ahead or none, on 1024-thread workgroups that
  // hide the latency of their rounds best.
  const int64_t pairs = T * (T + 1) / 2;
  const int ahead = half ? 0 : lookahead_bands(n, batch, sched);
  // A batch whose phase 1-2 launch fills the chip by itself splits into two
  // halves, one per stream: the molecules share nothing, so the phase 1-2
  // launches of one half run beside the bulk of the other.  With fewer
  // workgroups per launch the two halves only contend, and one stream in
  // order is faster.
  const int64_t W = step_blocks(n, batch, sched), NS = ceil_div(K1 - K0, W);
  // One stream, one k-block per step: the lead schedule.  Per
  // k-block K, phase 2 of K (k_product, its diagonal tile closed the launch
  // before), then one launch holding phase 3 of K and, beside it, phase 1 of
  // K + 1 (k_lead).  The chain per k-block is the longer of the two parts of
  // a lead launch plus a product launch, instead of a phase 1-2 launch (64
  // rounds over the diagonal tile and a panel tile) plus a bulk launch.
  const bool lead_sched = !half && lead_schedule(n, batch, sched);
  const bool split = ahead == 0 && !half && !lead_sched && batch >= 2 && TB > 1 && T > 1 &&
                     (TB - 1) * batch > kPanelFill;
  // the second stream of this caller stream, held (locked) until the whole
  // pass is enqueued
  Lane *lane = nullptr;
  std::unique_lock<std::mutex> lane_lock;
  if (split || (ahead > 0 && TB > 1)) lane_lock = lock_lane(s, &lane);
  if (split && lane) {
    const int64_t b1 = batch / 2;
    hipError_t e = hipEventRecord(lane->start(), s);
    if (e == hipSuccess) e = hipStreamWaitEvent(lane->side, lane->start(), 0);
    if (e == hipSuccess)
      e = launch_blocked_on(U, L, n, b1, K0, K1, s, prof, flags, sched, true, infeasible);
    if (e == hipSuccess)
      e = launch_blocked_on(U + b1 * nn, L + b1 * nn, n, batch - b1, K0, K1, lane->side, prof,
                            flags, sched, true, infeasible ? infeasible + b1 : nullptr);
    if (e == hipSuccess) e = hipEventRecord(lane->bulk(0), lane->side);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, lane->bulk(0), 0);
    return e;
  }
  const bool deep = ahead == 2;
  // Phase 1 of a k-block as the closure of its diagonal tile alone (a lead
  // launch with no bulk part), and phase 2 as a product from it: the lead
  // schedule's parts, also the panels of the two-step look-ahead.
#define DBS_LEAD(R, C, KC, M)                                                                \
  (ru ? (vec ? k_lead<true, true, R, C, KC, M> : k_lead<false, true, R, C, KC, M>)            \
      : (vec ? k_lead<true, false, R, C, KC, M> : k_lead<false, false, R, C, KC, M>))
  const bool small_lead = !packed && 4 * pairs * batch <= kSmallLeadGrid;
  auto lead_kernel = small_lead ? DBS_LEAD(kSmallRT, kSmallCT, kSmallKC, false)
                                : DBS_LEAD(kBulkRT, kBulkCT, kBulkKC, false);
  auto lead_last = small_lead ? DBS_LEAD(kSmallRT, kSmallCT, kSmallKC, true)
                              : DBS_LEAD(kBulkRT, kBulkCT, kBulkKC, true);
  const unsigned lead_block = small_lead ? (BK / kSmallRT) * (BK / kSmallCT)
                                         : (BK / kBulkRT) * (BK / kBulkCT);
#undef DBS_LEAD
  auto lead_packed = ru ? (vec ? k_lead_packed<true, true> : k_lead_packed<false, true>)
                        : (vec ? k_lead_packed<true, false> : k_lead_packed<false, false>);
  // (4x2 cells where the product launch runs alone: the lead schedule of
  // the dense layout)
  const bool wide_product = !packed && lead_sched;
#define DBS_PRODUCT(P, C)                                                                    \
  (ru ? (vec ? k_product<true, P, true, C> : k_product<false, P, true, C>)                    \
      : (vec ? k_product<true, P, false, C> : k_product<false, P, false, C>))
  auto product_kernel = packed ? DBS_PRODUCT(true, 4)
                               : (wide_product ? DBS_PRODUCT(false, 2) : DBS_PRODUCT(false, 4));
#undef DBS_PRODUCT
  const unsigned product_block =
      (unsigned)(wide_product ? product_threads<2>() : product_threads<4>());
  // ... and its columns split over four workgroups where four times its
  // workgroups still get a compute unit each (measured passes, against the
  // 4x2-cell product: n1536 0.860 / 0.930 ms, n2048 1.168 / 1.259, n3072
  // 2.239 / 2.359, 4 x n1024 0.639 / 0.682, 8 x n500 0.321 / 0.335; two
  // slices lost 1-2 %: 16 x n500 0.382 / 0.373, 32 x n256 0.186 / 0.184;
  // four slices where the launch has more workgroups than CUs lost 5-7 %:
  // 64 x n500 0.729 / 0.681, 16 x n1024 1.293 / 1.233, 40 x n700 1.128 /
  // 1.077)
  const int product_p = wide_product && 4 * (TB - 1) * batch <= kSplitPanelFill ? 4 : 1;
  auto product_slice = ru ? (vec ? k_product_slice<true, true, 4> : k_product_slice<false, true, 4>)
                          : (vec ? k_product_slice<true, false, 4> : k_product_slice<false, false, 4>);
  // phase 3 of K (none for K < 0) beside phase 1 of Z (none for Z < 0);
  // grid.x = molecules, grid.y = the closure and then the quadrants
  const unsigned mx = (unsigned)(batch < kMaxGridX ? batch : kMaxGridX);
  // (last: the last launch of the pass, which also writes the stale tiles'
  // copies; packed storage keeps one slot per value, so nothing goes stale)
  auto lead = [&](int64_t K, int64_t Z, hipStream_t st, bool last) -> hipError_t {
    const unsigned gq = (unsigned)(1 + (K >= 0 ? 4 * pairs : 0));
    const int kind = K >= 0 ? kProfTiles : kProfSmall;
    if (packed)
      return launch(prof, kind, lead_packed, dim3(mx, gq), dim3(kThreads), st, U, n, batch, K, Z,
                    infeasible);
    return launch(prof, kind, last ? lead_last : lead_kernel, dim3(mx, gq), dim3(lead_block), st,
                  U, L, n, batch, K, Z, infeasible);
  };
  auto product = [&](int64_t K, hipStream_t st) -> hipError_t {
    if (product_p > 1)
      return launch(prof, kProfPanel, product_slice, dim3((unsigned)((TB - 1) * product_p), gy),
                    dim3(256), st, U, L, n, batch, K, K1);
    return launch(prof, kProfPanel, product_kernel, dim3((unsigned)(TB - 1), gy),
                  dim3(product_block), st, U, L, n, batch, K, K1);
  };
  if (lead_sched) {
    hipError_t e = lead(-1, K0, s, false);
    for (int64_t K = K0; K < K1 && e == hipSuccess; ++K) {
      e = product(K, s);
      if (e == hipSuccess) e = lead(K, K + 1 < K1 ? K + 1 : -1, s, K + 1 == K1);
    }
    return e;
  }
  if (ahead == 0 && 4 * pairs * batch <= kSmallGrid) {
    quads_kernel = DBS_QUADS(kSmallRT, kSmallCT, kSmallKC, false);
    quads_last = DBS_QUADS(kSmallRT, kSmallCT, kSmallKC, true);
    quads_block = (BK / kSmallRT) * (BK / kSmallCT);
  }
#undef DBS_QUADS
#define DBS_PICK_PANEL(S)                                                                   \
  (packed ? (ru ? (vec ? k_diag_panel<true, true, true, S> : k_diag_panel<false, true, true, S>)   \
                : (vec ? k_diag_panel<true, true, false, S> : k_diag_panel<false, true, false, S>)) \
          : (ru ? (vec ? k_diag_panel<true, false, true, S> : k_diag_panel<false, false, true, S>)  \
                : (vec ? k_diag_panel<true, false, false, S> : k_diag_panel<false, false, false, S>)))
  // the packed layout's two-step look-ahead keeps the 64-round launch, on
  // 256-thread workgroups that fit where bulk workgroups retire
  const bool packed_deep = deep && packed;
  auto panel = packed_deep ? DBS_PICK_PANEL(4) : DBS_PICK_PANEL(2);
  const unsigned panel_block = packed_deep ? panel_threads<4>() : panel_threads<2>();
#undef DBS_PICK_PANEL
  // The phase 1-2 launch splits each panel tile's columns over P
  // workgroups where P times its workgroups still get a compute unit each:
  // four on the critical path of a one-stream pass, and in the dense layout
  // two beside the bulk one step ahead (measured passes, P = 1 / 2 / 4:
  // n1024 0.576 / 0.520 / 0.515 ms, n128 0.087 / 0.079 / 0.075 ms, 4 x n500
  // 0.310 / 0.285 / 0.284 ms; n4096, one step ahead, 4.24 / 4.12 / 4.56 ms;
  // packed, P = 1 / 4: n1024 0.688 / 0.627 ms, 4 x n500 0.364 / 0.337 ms,
  // and n4096 one step ahead 4.60 against 4.71 ms with P = 2).
  const int64_t panel_wgs = (TB - 1) * batch;
  const int split_p = deep || (packed && ahead > 0) ? 1
                      : ahead == 0 && 4 * panel_wgs <= kSplitPanelFill ? 4
                      : 2 * panel_wgs <= kSplitPanelFill ? 2
                                                          : 1;
#define DBS_PICK_SPLIT(K, P)                                                                 \
  (ru ? (vec ? k_diag_panel_split<true, K, true, P> : k_diag_panel_split<false, K, true, P>)  \
      : (vec ? k_diag_panel_split<true, K, false, P> : k_diag_panel_split<false, K, false, P>))
  auto panel_split = packed ? (split_p == 4 ? DBS_PICK_SPLIT(true, 4) : DBS_PICK_SPLIT(true, 2))
                            : (split_p == 4 ? DBS_PICK_SPLIT(false, 4) : DBS_PICK_SPLIT(false, 2));
#undef DBS_PICK_SPLIT

  // Phases 1 and 2 of block K (the diagonal tile alone when it is the only
  // block).  On the critical path (no look-ahead, or one step) as one launch
  // of 64 rounds over the diagonal tile and each panel tile, whose
  // 1024-thread workgroups hide the rounds' latency best.  Two steps ahead
  // they run beside the bulk, off the critical path, and take its compute
  // units: there, in the dense layout, as the closure of the diagonal tile
  // (one workgroup per molecule) and the product, which does not repeat the
  // diagonal tile's rounds in every panel workgroup (measured n12288 pass,
  // dense: 68.59 ms with the 64-round launch, 67.71-67.73 ms closure and
  // product; packed: 72.3 against 80.6 ms the other way round; at n4096,
  // one step ahead, 4.24 against 4.65-4.78 ms).
  auto phase12 = [&](int64_t K, hipStream_t st) -> hipError_t {
    if (TB == 1)
      return launch_small_block(U, L, n, nn, 0, (int)n, 0, (int)n, batch, st, prof, flags);
    if (deep && !packed) {
      const hipError_t r = lead(-1, K, st, false);
      return r == hipSuccess ? product(K, st) : r;
    }
    if (split_p > 1)
      return launch(prof, kProfPanel, panel_split, dim3((unsigned)((TB - 1) * split_p), gy),
                    dim3(1024), st, U, L, n, batch, K, infeasible);
    return launch(prof, kProfPanel, panel, dim3((unsigned)(TB - 1), gy), dim3(panel_block), st, U,
                  L, n, batch, K, infeasible);
  };
  // The pass advances by steps of W k-blocks: step t holds the blocks
  // [lo(t), hi(t)).  Two steps ahead the bulk takes several blocks per
  // launch, which spreads its fixed costs (the loads and stores of the
  // matrix, the launch's ramp and tail) over more atoms.
  auto lo = [&](int64_t t) { return K0 + t * W; };
  auto hi = [&](int64_t t) { return K0 + (t + 1) * W < K1 ? K0 + (t + 1) * W : K1; };

  // phase 3 of the blocks [K, K + nk) on the cells outside the bands [K, X1)
  // the XCD order where a bulk launch runs many rounds of workgroups
  // (measured pass ms, plain / XCD order: n6144 11.29-11.43 / 11.54, n8192
  // 24.09-24.10 / 24.02-24.13, n12288 68.63-68.84 / 68.41-68.76)
  const int xcd = deep && T >= kXcdTiles ? 1 : 0;
  const unsigned bulk_grid = (unsigned)bulk_workgroups(T, xcd);
  // (last: the last one of the pass, which also writes the stale tiles'
  // copies; packed storage keeps one slot per value, so nothing goes stale)
  auto phase3 = [&](int64_t K, int64_t nk, int64_t X1, hipStream_t st, bool last) -> hipError_t {
    if (!packed)
      return launch(prof, kProfTiles, last ? quads_last : quads_kernel, dim3(bulk_grid, gy),
                    dim3(quads_block), st, U, L, n, batch, K, nk, K, X1, xcd);
    return launch(prof, kProfTiles, packed_kernel, dim3(bulk_grid, gy),
                  dim3(kThreads), st, U, n, batch, K, nk, K, X1, xcd);
  };
  // phase 3 of the blocks [K, K + nk) on the nr row bands from A0: row band
  // A0 + r on every column band outside [X0, X1 + r) and other than Y
  auto strip = [&](int64_t K, int64_t nk, int64_t A0, int64_t nr, int64_t X0, int64_t X1,
                   int64_t Y, bool both, hipStream_t st) -> hipError_t {
    const int64_t xe = X1 < TB ? X1 : TB;
    const int64_t cols = TB - (xe - X0) - (Y >= xe && Y < TB ? 1 : 0);
    return launch(prof, kProfStrip, strip_kernel, dim3((unsigned)cols, gy, (unsigned)nr),
                  dim3(kThreads), st, U, L, n, batch, K, nk, A0, X0, X1, Y, (int)both);
  };
  // The rows of step t's bands final for all of its rounds, in both
  // orientations: per block b+j in turn, its phases 1-2, then the block on
  // the step's other bands (one strip; the bands before b+j, whose rows are
  // panel rows already, in both orientations).  This is the one-block
  // schedule restricted to the step's bands.
  auto step_panel = [&](int64_t t, hipStream_t st) -> hipError_t {
    const int64_t b = lo(t), w = hi(t) - b;
    hipError_t r = hipSuccess;
    for (int64_t j = 0; j < w && r == hipSuccess; ++j) {
      if ((r = phase12(b + j, st)) != hipSuccess) break;
      if (w > 1) r = strip(b + j, 1, b, w, b, b, b + j, true, st);
    }
    return r;
  };

  hipError_t e = step_panel(0, s);
  if (e != hipSuccess || TB == 1) return e;

  hipStream_t side = ahead > 0 && lane ? lane->side : nullptr;
  Lane *ev = lane;
  if (side == nullptr) {
    for (int64_t t = 0; t < NS && e == hipSuccess; ++t) {
      e = phase3(lo(t), hi(t) - lo(t), hi(t), s, t + 1 == NS);
      if (e == hipSuccess && t + 1 < NS) e = step_panel(t + 1, s);
    }
  } else {
    if ((e = hipEventRecord(ev->start(), s)) == hipSuccess)
      e = hipStreamWaitEvent(side, ev->start(), 0);
    for (int64_t t = 0; t < NS && e == hipSuccess; ++t) {
      const bool n1 = t + 1 < NS, n2 = deep && t + 2 < NS;
      const int64_t b = lo(t), w = hi(t) - b;
      if (t > 0 && (e = hipStreamWaitEvent(s, ev->ready(t), 0)) != hipSuccess) break;
      if ((e = phase3(b, w, n2 ? hi(t + 2) : n1 ? hi(t + 1) : hi(t), s, t + 1 == NS)) !=
          hipSuccess)
        break;
      if ((e = hipEventRecord(ev->bulk(t), s)) != hipSuccess) break;
      if (n1) {
        // one step ahead, step t+1's bands after step t-1 come from bulk(t-1)
        if (!deep && t > 0 && (e = hipStreamWaitEvent(side, ev->bulk(t - 1), 0)) != hipSuccess)
          break;
        if ((e = strip(b, w, lo(t + 1), hi(t + 1) - lo(t + 1), b, hi(t), -1, false, side)) !=
            hipSuccess)
          break;
        if ((e = step_panel(t + 1, side)) != hipSuccess) break;
      }
      if (n2) {
        if (t > 0 && (e = hipStreamWaitEvent(side, ev->bulk(t - 1), 0)) != hipSuccess) break;
        if ((e = strip(b, w, lo(t + 2), hi(t + 2) - lo(t + 2), b, hi(t + 1), -1, false,
                       side)) != hipSuccess)
          break;
      }
      if (n1 && (e = hipEventRecord(ev->ready(t + 1), side)) != hipSuccess) break;
    }
  }
  return e;
}
}  // namespace

}  // namespace dbs
