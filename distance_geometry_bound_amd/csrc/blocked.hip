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
//            k_diag_panel, one workgroup per panel tile);
//   phase 3  every remaining cell: all bK rounds at once from the finished
//            panel (k_tiles, plus k_strip for band K+1 when running ahead).
//            This is where 1 - O(BK/n) of the work is.
//
// Symmetric schedule.  U and L stay exactly symmetric, so only the cells of
// TILE x TILE tiles (I,J) with I <= J are kept current ("fresh"); tiles below
// the diagonal go stale and are rebuilt by one transposed copy at the end
// (k_mirror).  Phase 3 therefore does half the work of a dense schedule.  It
// reads its operands U/L[i,k] and U/L[k,j] from row k only (U[i,k] = U[k,i]),
// so phase 2 must leave all of row band K fresh: it updates each panel tile
// from whichever orientation is fresh and writes both orientations.
//
// Phase 3 bulk kernel: a 256-thread workgroup owns a 128x128 tile; each thread an
// 8x8 register tile (rows ty*4+{0..3} and 64+ty*4+{0..3}, same for columns,
// so the LDS reads of a wave are contiguous).  The panel rows of the k-block
// are staged through LDS in chunks of KC atoms.  Per atom and cell the VALU
// does one add and one min for U, two subtracts and two max for L; pairs of
// atoms fold into 3-input min/max.  No matrix cores: min-plus is not a
// multiply-add contraction.
#include <mutex>

#include "dbs_internal.h"

namespace dbs {
namespace {

constexpr int BK = 64;          // atoms per k-block (phases 1 and 2 tile size)
constexpr int TILE = 128;       // phase-3 tile size; fresh region is I <= J in these tiles
constexpr int RATIO = TILE / BK;
constexpr int KC = 16;          // atoms per LDS chunk in phase 3
constexpr int kThreads = 256;

// The side-stream kernels (band K+1 strip, then phases 1-2 of block K+1) are
// the critical path of a k-block whenever they share compute units with the
// bulk kernel: their waves take instruction-issue priority over its waves on
// the same SIMD (wave priority only; the streams keep the default priority).
__device__ __forceinline__ void critical_path_priority() { __builtin_amdgcn_s_setprio(2); }

// (k-block tile a, k-block tile b) is fresh under the symmetric schedule
__device__ __forceinline__ bool fresh(int64_t a, int64_t b) { return a / RATIO <= b / RATIO; }

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ float4 inf4() { return make_float4(kInf, kInf, kInf, kInf); }
__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

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
template <int S = 4>
__device__ __forceinline__ void packed_block_store(float *P, int64_t n, int64_t r0, int64_t c0,
                                                   int rows, int cols, int ty, int tx,
                                                   const float (&u)[S][S],
                                                   const float (&l)[S][S]) {
#pragma unroll
  for (int r = 0; r < S; ++r)
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const int a = ty * S + r, c = tx * S + q;
      if (a >= rows || c >= cols || (r0 == c0 && a == c)) continue;
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
// Workgroup 0 writes D back.  Cells outside the matrix start neutral and stay
// neutral (every candidate through them is +inf for U and <= 0 for L).
//
// The rounds are latency-bound (a barrier and LDS round trip each), so the
// workgroup is 1024 threads, four waves per SIMD to cover each other's
// stalls, and thread (ty, tx) owns a 2x2 cell block of D and of R: rows
// 2ty, 2ty+1 and columns 2tx, 2tx+1.
constexpr int kPanelThreads = 1024;
constexpr int PS = 2;  // cells per side and thread in k_diag_panel

template <bool VEC, bool PK, bool RU>
__global__ __launch_bounds__(kPanelThreads) void k_diag_panel(float *__restrict__ U,
                                                              float *__restrict__ L, int64_t n,
                                                              int64_t batch, int64_t K) {
  __shared__ float2 dvu[2][BK / PS], dvl[2][BK / PS];  // row m of D
  __shared__ float2 rvu[2][BK / PS], rvl[2][BK / PS];  // row m of R

  rounding_prologue<RU>();
  critical_path_priority();
  const int tid = threadIdx.x, ty = tid / (BK / PS), tx = tid % (BK / PS);
  int64_t J = blockIdx.x;
  if (J >= K) ++J;
  const int64_t k0 = K * BK, j0 = J * BK;
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  const bool rowor = fresh(K, J);
  const bool writes_d = blockIdx.x == 0;
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = PK ? Ub : L + b * nn;

    float du[PS][PS], dl[PS][PS];  // D[2ty + r][2tx + q]
    float u[PS][PS], l[PS][PS];    // R[2ty + r][2tx + q] = cell (k0 + 2ty + r, j0 + 2tx + q)
    if (PK) {
      packed_block_load<VEC, PS>(Ub, n, k0, k0, bK, bK, ty, tx, du, dl);
      packed_block_load<VEC, PS>(Ub, n, k0, j0, bK, bJ, ty, tx, u, l);
    } else {
      // all loads are issued before any value is unpacked
      Seg<PS> xu[PS], xl[PS], yu[PS], yl[PS];
#pragma unroll
      for (int r = 0; r < PS; ++r) {
        const int a = ty * PS + r;
        const int64_t g = (k0 + a) * n + k0 + tx * PS;
        const int64_t left = a < bK ? bK - tx * PS : 0;
        xu[r] = load_seg<VEC, PS>(Ub + g, left, kInf, Ub);
        xl[r] = load_seg<VEC, PS>(Lb + g, left, 0.0f, Lb);
      }
      // the panel tile from its fresh orientation: R[a][c] = M[k0+a][j0+c]
      // (row segments), else M[j0+c][k0+a] (column segments)
#pragma unroll
      for (int r = 0; r < PS; ++r) {
        const int64_t left = rowor ? (ty * PS + r < bK ? bJ - tx * PS : 0)
                                   : (tx * PS + r < bJ ? bK - ty * PS : 0);
        const int64_t g = rowor ? (k0 + ty * PS + r) * n + j0 + tx * PS
                                : (j0 + tx * PS + r) * n + k0 + ty * PS;
        yu[r] = load_seg<VEC, PS>(Ub + g, left, kInf, Ub);
        yl[r] = load_seg<VEC, PS>(Lb + g, left, 0.0f, Lb);
      }
#pragma unroll
      for (int r = 0; r < PS; ++r)
#pragma unroll
        for (int q = 0; q < PS; ++q) {
          du[r][q] = xu[r].v[q];
          dl[r][q] = xl[r].v[q];
          u[r][q] = rowor ? yu[r].v[q] : yu[q].v[r];
          l[r][q] = rowor ? yl[r].v[q] : yl[q].v[r];
        }
    }

    for (int mb = 0; mb < BK / PS; ++mb) {
#pragma unroll
      for (int r = 0; r < PS; ++r) {
        const int m = mb * PS + r;
        if (m >= bK) break;  // uniform
        const int buf = m & 1;
        if (ty == mb) {
          dvu[buf][tx] = make_float2(du[r][0], du[r][1]);
          dvl[buf][tx] = make_float2(dl[r][0], dl[r][1]);
          rvu[buf][tx] = make_float2(u[r][0], u[r][1]);
          rvl[buf][tx] = make_float2(l[r][0], l[r][1]);
        }
        __syncthreads();
        const float2 cu = dvu[buf][ty], cl = dvl[buf][ty];  // D[a][m] = D[m][a]
        const float2 eu = dvu[buf][tx], el = dvl[buf][tx];  // D[m][b]
        const float2 ru = rvu[buf][tx], rl = rvl[buf][tx];  // R[m][c]
        const float cuv[2] = {cu.x, cu.y}, clv[2] = {cl.x, cl.y};
        const float euv[2] = {eu.x, eu.y}, elv[2] = {el.x, el.y};
        const float ruv[2] = {ru.x, ru.y}, rlv[2] = {rl.x, rl.y};
#pragma unroll
        for (int a = 0; a < PS; ++a)
#pragma unroll
          for (int q = 0; q < PS; ++q) {
            relax1<RU>(du[a][q], dl[a][q], cuv[a], clv[a], euv[q], elv[q]);
            relax1<RU>(u[a][q], l[a][q], cuv[a], clv[a], ruv[q], rlv[q]);
          }
      }
    }

#pragma unroll
    for (int r = 0; r < PS; ++r)
#pragma unroll
      for (int q = 0; q < PS; ++q) {
        l[r][q] = lower_out<RU>(l[r][q]);
        dl[r][q] = lower_out<RU>(dl[r][q]);
      }
    // R in both orientations (packed: the one slot of U and of L); D, which
    // lies in a fresh tile, as a full square
    if (PK) {
      packed_block_store<PS>(Ub, n, k0, j0, bK, bJ, ty, tx, u, l);
      if (writes_d) packed_block_store<PS>(Ub, n, k0, k0, bK, bK, ty, tx, du, dl);
    }
#pragma unroll
    for (int r = 0; r < PS; ++r)
#pragma unroll
      for (int q = 0; q < PS; ++q) {
        const int a = ty * PS + r, c = tx * PS + q;
        if (!PK && a < bK && c < bJ) {
          Ub[(k0 + a) * n + j0 + c] = u[r][q];
          Lb[(k0 + a) * n + j0 + c] = l[r][q];
          Ub[(j0 + c) * n + k0 + a] = u[r][q];
          Lb[(j0 + c) * n + k0 + a] = l[r][q];
        }
        if (!PK && writes_d && a < bK && c < bK) {
          Ub[(k0 + a) * n + k0 + c] = du[r][q];
          Lb[(k0 + a) * n + k0 + c] = dl[r][q];
        }
      }
    __syncthreads();  // LDS reuse by the next molecule
  }
}

// ---------------------------------------------------------------- packed panel staging
// Packed layout: the panel values of band K at the 64 columns xh..xh+63 and
// rows k0+kc..k0+kc+KC-1 are U[k][x] = P[min(k,x)][max(k,x)] and
// L[k][x] = P[max(k,x)][min(k,x)].  Right of the band (x > k) U is a row
// segment of P and L a column segment; left of it the other way round.  A
// column segment is read as rows of P, four consecutive k per float4.  Each
// of the 256 threads loads one float4 of each kind.  `dead` (band K, band
// K+1 or beyond n: values no live cell uses) gives the neutral values.
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

// ---------------------------------------------------------------- phase 3

// Tiles are numbered column-major over the upper triangle.  The hardware
// deals consecutive workgroups to the 8 XCDs in turn, so at any moment an
// XCD works on a few tile columns and on every 8th tile row of them: the
// panel slices it needs fit its L2.  (Giving each XCD a contiguous run of
// tiles instead makes it sweep every row slice of the panel, and is slower.)

// Bulk of phase 3.  grid.x = T(T+1)/2 tiles (I <= J), grid.y = molecules.
// Cells in band K (final after phase 2) and in band s1 (the next k-block's
// band, updated ahead by k_strip; s1 < 0 for none) are neither read nor
// written, and band s1's panel columns are not read: while this kernel runs,
// another stream may be updating exactly those cells.
template <bool VEC, bool PK, bool RU>
__global__ __launch_bounds__(kThreads, 2) void k_tiles(float *__restrict__ U,
                                                       float *__restrict__ L, int64_t n,
                                                       int64_t batch, int64_t K, int64_t s1) {
  __shared__ float4 scu[KC][TILE / 4];
  __shared__ float4 scl[KC][TILE / 4];
  __shared__ float4 sru[KC][TILE / 4];
  __shared__ float4 srl[KC][TILE / 4];

  rounding_prologue<RU>();
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t p = blockIdx.x;
  const int64_t J = tri_col(p);
  const int64_t I = p - J * (J + 1) / 2;
  const int64_t i0 = I * TILE, j0 = J * TILE;
  const int64_t k0 = K * BK;
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int64_t e1 = s1 < 0 ? -1 : (s1 + BK < n ? s1 + BK : n);
  const int64_t nn = n * n;
  // x is live: in range and outside both bands (band edges are multiples of 4)
  auto live = [&](int64_t x) { return x < n && (x < k0 || x >= k0 + bK) && (x < s1 || x >= e1); };
  auto in_s1 = [&](int64_t x) { return x >= s1 && x < e1; };

  // rows of this thread: i0 + rofs(r), r < 8; columns likewise with tx
  auto rofs = [](int t, int r) { return (r < 4 ? 0 : TILE / 2 - 4) + t * 4 + r; };
  // liveness of the thread's 8 rows and 8 columns, one bit each
  unsigned rmask = 0, cmask = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    rmask |= (unsigned)live(i0 + rofs(ty, r)) << r;
    cmask |= (unsigned)live(j0 + rofs(tx, r)) << r;
  }

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = PK ? Ub : L + b * nn;

    // U (and dense L) at (i, j); packed U is P tile (I, J) itself
    float u[8][8], l[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t i = i0 + rofs(ty, r);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t j = j0 + rofs(tx, h * 4);
        const bool on = ((rmask >> r) & (cmask >> (h * 4)) & 1u) != 0;
        const int cnt = on ? (VEC ? 4 : clamp4(n - j)) : 0;
        const float4 x = load4<VEC>(Ub + i * n + j, cnt, kInf, Ub);
        u[r][h * 4 + 0] = x.x; u[r][h * 4 + 1] = x.y; u[r][h * 4 + 2] = x.z; u[r][h * 4 + 3] = x.w;
        if (!PK) {
          const float4 y = load4<VEC>(Lb + i * n + j, cnt, 0.0f, Lb);
          l[r][h * 4 + 0] = y.x; l[r][h * 4 + 1] = y.y; l[r][h * 4 + 2] = y.z; l[r][h * 4 + 3] = y.w;
        }
      }
    }
    if (PK) {
      // packed L(i,j) = P[j][i] (tile (J, I) read across): for each column j
      // two float4 along i
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int64_t j = j0 + rofs(tx, c);
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
          const int64_t i = i0 + rofs(ty, hr * 4);
          const bool on = ((cmask >> c) & (rmask >> (hr * 4)) & 1u) != 0;
          const int cnt = on ? (VEC ? 4 : clamp4(n - i)) : 0;
          const float4 t = load4<VEC>(Ub + j * n + i, cnt, 0.0f, Ub);
          l[hr * 4 + 0][c] = t.x; l[hr * 4 + 1][c] = t.y; l[hr * 4 + 2][c] = t.z; l[hr * 4 + 3][c] = t.w;
        }
      }
      if (I == J) {
        // a diagonal tile: below the diagonal P[i][j] is L(i,j) and P[j][i] is U(i,j)
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const int64_t i = i0 + rofs(ty, r), j = j0 + rofs(tx, c);
            if (i > j) {
              const float t = u[r][c];
              u[r][c] = l[r][c];
              l[r][c] = t;
            } else if (i == j) {
              l[r][c] = u[r][c];
            }
          }
      }
    }

    for (int kc = 0; kc < bK; kc += KC) {
      // stage panel rows k0+kc .. k0+kc+KC-1, columns of I and of J: every
      // global load of the chunk is issued before the first LDS store
      if (PK) {
        // addresses recomputed per chunk (not hoisted out of the k loop)
        int tl = tid;
        asm volatile("" : "+v"(tl));
        HalfLoad hl[4];
        bool right[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t xh = (q < 2 ? i0 : j0) + (q & 1) * (TILE / 2);
          right[q] = xh > k0;
          const bool dead = xh == k0 || xh == s1 || xh >= n;
          hl[q] = packed_half_load<VEC>(Ub, n, k0, kc, bK, xh, right[q], dead, tl);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          packed_half_store(hl[q], right[q],
                            reinterpret_cast<float *>(q < 2 ? &scu[0][0] : &sru[0][0]),
                            reinterpret_cast<float *>(q < 2 ? &scl[0][0] : &srl[0][0]), TILE,
                            (q & 1) * (TILE / 2), tl);
      } else {
      constexpr int kIter = KC * (TILE / 4) / kThreads;
      float4 st[kIter][4];
#pragma unroll
      for (int it = 0; it < kIter; ++it) {
        const int e = tid + it * kThreads;
        const int kk = e / (TILE / 4), x4 = e % (TILE / 4);
        const int64_t k = k0 + kc + kk;
        const bool kin = kc + kk < bK;
        const int64_t ci = i0 + x4 * 4, cj = j0 + x4 * 4;
        const int ni = (kin && !in_s1(ci)) ? clamp4(n - ci) : 0;
        const int nj = (kin && !in_s1(cj)) ? clamp4(n - cj) : 0;
        st[it][0] = load4<VEC>(Ub + k * n + ci, ni, kInf, Ub);
        st[it][1] = load4<VEC>(Lb + k * n + ci, ni, 0.0f, Lb);
        st[it][2] = load4<VEC>(Ub + k * n + cj, nj, kInf, Ub);
        st[it][3] = load4<VEC>(Lb + k * n + cj, nj, 0.0f, Lb);
      }
#pragma unroll
      for (int it = 0; it < kIter; ++it) {
        const int e = tid + it * kThreads;
        const int kk = e / (TILE / 4), x4 = e % (TILE / 4);
        scu[kk][x4] = st[it][0];
        scl[kk][x4] = st[it][1];
        sru[kk][x4] = st[it][2];
        srl[kk][x4] = st[it][3];
      }
      }
      __syncthreads();

#pragma unroll 2
      for (int kk = 0; kk < KC; kk += 2) {
        float cu0[8], cl0[8], ru0[8], rl0[8], cu1[8], cl1[8], ru1[8], rl1[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int xi = h * (TILE / 8) + ty, xj = h * (TILE / 8) + tx;
          const float4 a0 = scu[kk][xi], b0 = scl[kk][xi], c0 = sru[kk][xj], d0 = srl[kk][xj];
          const float4 a1 = scu[kk + 1][xi], b1 = scl[kk + 1][xi], c1 = sru[kk + 1][xj], d1 = srl[kk + 1][xj];
          cu0[h * 4 + 0] = a0.x; cu0[h * 4 + 1] = a0.y; cu0[h * 4 + 2] = a0.z; cu0[h * 4 + 3] = a0.w;
          cl0[h * 4 + 0] = b0.x; cl0[h * 4 + 1] = b0.y; cl0[h * 4 + 2] = b0.z; cl0[h * 4 + 3] = b0.w;
          ru0[h * 4 + 0] = c0.x; ru0[h * 4 + 1] = c0.y; ru0[h * 4 + 2] = c0.z; ru0[h * 4 + 3] = c0.w;
          rl0[h * 4 + 0] = d0.x; rl0[h * 4 + 1] = d0.y; rl0[h * 4 + 2] = d0.z; rl0[h * 4 + 3] = d0.w;
          cu1[h * 4 + 0] = a1.x; cu1[h * 4 + 1] = a1.y; cu1[h * 4 + 2] = a1.z; cu1[h * 4 + 3] = a1.w;
          cl1[h * 4 + 0] = b1.x; cl1[h * 4 + 1] = b1.y; cl1[h * 4 + 2] = b1.z; cl1[h * 4 + 3] = b1.w;
          ru1[h * 4 + 0] = c1.x; ru1[h * 4 + 1] = c1.y; ru1[h * 4 + 2] = c1.z; ru1[h * 4 + 3] = c1.w;
          rl1[h * 4 + 0] = d1.x; rl1[h * 4 + 1] = d1.y; rl1[h * 4 + 2] = d1.z; rl1[h * 4 + 3] = d1.w;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c)
            relax2<RU>(u[r][c], l[r][c], cu0[r], cl0[r], ru0[c], rl0[c], cu1[r], cl1[r], ru1[c],
                   rl1[c]);
      }
      __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) l[r][c] = lower_out<RU>(l[r][c]);
    // the store addresses are recomputed here rather than kept live across
    // the k loop from the loads
    int ts = tid;
    asm volatile("" : "+v"(ts));
    const int sy = ts >> 4, sx = ts & 15;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (!((rmask >> r) & 1u)) continue;
      const int64_t i = i0 + rofs(sy, r);
      float *pu = Ub + i * n + j0;
      float *pl = Lb + i * n + j0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (!((cmask >> c) & 1u)) continue;
        const int64_t j = j0 + rofs(sx, c);
        if (!PK) {
          pu[rofs(sx, c)] = u[r][c];
          pl[rofs(sx, c)] = l[r][c];
        } else if (I != J) {
          Ub[i * n + j] = u[r][c];
          Ub[j * n + i] = l[r][c];
        } else if (i != j) {
          Ub[i * n + j] = i < j ? u[r][c] : l[r][c];
        }
      }
    }
    __syncthreads();
  }
}

// Phase 3 on band K+1 only, run ahead of the bulk: the cells (i, j) with i in
// band K+1 and j outside band K, each kept in its fresh orientation.
// grid.x = k-block tiles J other than K (one BK x BK tile each),
// grid.y = molecules.  Thread (ty, tx) owns a 4x4 cell tile.
template <bool VEC, bool PK, bool RU>
__global__ __launch_bounds__(kThreads) void k_strip(float *__restrict__ U, float *__restrict__ L,
                                                    int64_t n, int64_t batch, int64_t K) {
  __shared__ float4 scu[KC][BK / 4];
  __shared__ float4 scl[KC][BK / 4];
  __shared__ float4 sru[KC][BK / 4];
  __shared__ float4 srl[KC][BK / 4];

  rounding_prologue<RU>();
  critical_path_priority();
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  int64_t J = blockIdx.x;
  if (J >= K) ++J;
  const int64_t k0 = K * BK, s1 = (K + 1) * BK, j0 = J * BK;
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int b1 = (int)(n - s1 < BK ? n - s1 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  const bool rowor = fresh(K + 1, J);
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = PK ? Ub : L + b * nn;

    // logical cell (a, c) = (s1 + a, j0 + c); stored at (s1+a, j0+c) or (j0+c, s1+a)
    float u[4][4], l[4][4];
    if (PK) {
      packed_block_load<VEC>(Ub, n, s1, j0, b1, bJ, ty, tx, u, l);
    } else if (rowor) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = ty * 4 + r;
        const int cnt = a < b1 ? clamp4(bJ - tx * 4) : 0;
        const int64_t g = (s1 + a) * n + j0 + tx * 4;
        const float4 x = load4<VEC>(Ub + g, cnt, kInf, Ub), y = load4<VEC>(Lb + g, cnt, 0.0f, Lb);
        u[r][0] = x.x; u[r][1] = x.y; u[r][2] = x.z; u[r][3] = x.w;
        l[r][0] = y.x; l[r][1] = y.y; l[r][2] = y.z; l[r][3] = y.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tx * 4 + q;
        const int cnt = c < bJ ? clamp4(b1 - ty * 4) : 0;
        const int64_t g = (j0 + c) * n + s1 + ty * 4;
        const float4 x = load4<VEC>(Ub + g, cnt, kInf, Ub), y = load4<VEC>(Lb + g, cnt, 0.0f, Lb);
        u[0][q] = x.x; u[1][q] = x.y; u[2][q] = x.z; u[3][q] = x.w;
        l[0][q] = y.x; l[1][q] = y.y; l[2][q] = y.z; l[3][q] = y.w;
      }
    }

    for (int kc = 0; kc < bK; kc += KC) {
      if (PK) {
        // band K+1 lies right of band K; band J right or left of it
        const HalfLoad hc = packed_half_load<VEC>(Ub, n, k0, kc, bK, s1, true, false, tid);
        const HalfLoad hr = packed_half_load<VEC>(Ub, n, k0, kc, bK, j0, J > K, false, tid);
        packed_half_store(hc, true, reinterpret_cast<float *>(&scu[0][0]),
                          reinterpret_cast<float *>(&scl[0][0]), BK, 0, tid);
        packed_half_store(hr, J > K, reinterpret_cast<float *>(&sru[0][0]),
                          reinterpret_cast<float *>(&srl[0][0]), BK, 0, tid);
      } else {
        // KC x BK/4 float4 per array: one of each per thread
        const int kk = tid / (BK / 4), x4 = tid % (BK / 4);
        const int64_t k = k0 + kc + kk;
        const bool kin = kc + kk < bK;
        const int ni = kin ? clamp4(b1 - x4 * 4) : 0;
        const int nj = kin ? clamp4(bJ - x4 * 4) : 0;
        scu[kk][x4] = load4<VEC>(Ub + k * n + s1 + x4 * 4, ni, kInf, Ub);
        scl[kk][x4] = load4<VEC>(Lb + k * n + s1 + x4 * 4, ni, 0.0f, Lb);
        sru[kk][x4] = load4<VEC>(Ub + k * n + j0 + x4 * 4, nj, kInf, Ub);
        srl[kk][x4] = load4<VEC>(Lb + k * n + j0 + x4 * 4, nj, 0.0f, Lb);
      }
      __syncthreads();
#pragma unroll 2
      for (int kk = 0; kk < KC; kk += 2) {
        const float4 a0 = scu[kk][ty], b0 = scl[kk][ty], c0 = sru[kk][tx], d0 = srl[kk][tx];
        const float4 a1 = scu[kk + 1][ty], b1v = scl[kk + 1][ty], c1 = sru[kk + 1][tx], d1 = srl[kk + 1][tx];
        const float cu0[4] = {a0.x, a0.y, a0.z, a0.w}, cl0[4] = {b0.x, b0.y, b0.z, b0.w};
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
    if (PK) packed_block_store(Ub, n, s1, j0, b1, bJ, ty, tx, u, l);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int a = ty * 4 + r, c = tx * 4 + q;
        if (!PK && a < b1 && c < bJ) {
          const int64_t g = rowor ? (s1 + a) * n + j0 + c : (j0 + c) * n + s1 + a;
          Ub[g] = u[r][q];
          Lb[g] = l[r][q];
        }
      }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- mirror
// grid.x = TB*TB k-block tiles (a = x / TB, b = x % TB), grid.y = molecules.
// Stale tiles (a,b) (a/RATIO > b/RATIO) are overwritten with the transpose
// of the fresh tile (b,a).
__global__ __launch_bounds__(kThreads) void k_mirror(float *__restrict__ U, float *__restrict__ L,
                                                     int64_t n, int64_t batch, int64_t TB) {
  __shared__ float su[BK][BK + 1];
  __shared__ float sl[BK][BK + 1];
  const int64_t a = blockIdx.x / TB, bt = blockIdx.x % TB;
  if (fresh(a, bt)) return;  // uniform: whole workgroup leaves
  const int tid = threadIdx.x;
  const int64_t nn = n * n;
  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = L + b * nn;
    // read fresh tile (bt, a): rows bt*BK + r, columns a*BK + c
    for (int e = tid; e < BK * BK; e += kThreads) {
      const int r = e / BK, c = e % BK;
      const int64_t i = bt * BK + r, j = a * BK + c;
      if (i < n && j < n) {
        su[r][c] = Ub[i * n + j];
        sl[r][c] = Lb[i * n + j];
      }
    }
    __syncthreads();
    for (int e = tid; e < BK * BK; e += kThreads) {
      const int r = e / BK, c = e % BK;
      const int64_t i = a * BK + r, j = bt * BK + c;
      if (i < n && j < n) {
        Ub[i * n + j] = su[c][r];
        Lb[i * n + j] = sl[c][r];
      }
    }
    __syncthreads();
  }
}

// Side stream for the lookahead (one per device, default priority, created
// on first use and kept for the life of the process).
hipStream_t side_stream() {
  static std::mutex mu;
  static hipStream_t streams[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev]) {
    hipStream_t st = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess) streams[dev] = st;
  }
  return streams[dev];
}

// Ordering events of the lookahead: one set per host thread and device,
// created on first use and re-recorded by every pass (a stream wait captures
// the event's state when it is enqueued, so re-recording is safe).
struct Events {
  hipEvent_t e[3] = {nullptr, nullptr, nullptr};  // e[0] unused
  bool ready = false;
  bool init() {
    if (ready) return true;
    for (auto &x : e)
      if (!x && hipEventCreateWithFlags(&x, hipEventDisableTiming) != hipSuccess) return false;
    ready = true;
    return true;
  }
  ~Events() {
    for (auto &x : e)
      if (x) (void)hipEventDestroy(x);
  }
};

Events *thread_events() {
  thread_local Events per_device[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  return per_device[dev].init() ? &per_device[dev] : nullptr;
}

}  // namespace

// Enqueue one pass.  With more than one k-block the pass runs ahead: phase 3
// of block K is split into band K+1 (k_strip) and everything else (k_tiles).
// The side stream runs strip(K), then phases 1 and 2 of block K+1, while the
// caller's stream runs tiles(K); so the short, latency-bound phases hide
// under the long one.  Everything on the side stream reads and writes only
// band K+1 cells and band K's panel rows, which tiles(K) neither writes nor
// (for band K+1) reads.  Events order strip(K) after tiles(K-1), and
// tiles(K+1) after phase 2 of K+1.
hipError_t launch_blocked(float *U, float *L, int64_t n, int64_t batch, int64_t K0, int64_t K1,
                          hipStream_t s, Prof *prof, unsigned flags) {
  static_assert(BK == kBlockRounds, "k-block size");
  const int64_t TB = ceil_div(n, BK);    // k-blocks
  if (K1 > TB) K1 = TB;
  if (n <= 1 || K0 >= K1) return hipSuccess;
  const int64_t T = ceil_div(n, TILE);   // phase-3 tiles per side
  const bool packed = flags & kPacked, ru = flags & kDirected;
  const bool vec = (n % 4 == 0) && aligned16(U) && aligned16(L);
  const unsigned gy = (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ);
  const int64_t nn = n * n;
  if (packed) L = U;
#define DBS_PICK(K)                                                                   \
  (packed ? (ru ? (vec ? K<true, true, true> : K<false, true, true>)                  \
                : (vec ? K<true, true, false> : K<false, true, false>))               \
          : (ru ? (vec ? K<true, false, true> : K<false, false, true>)                \
                : (vec ? K<true, false, false> : K<false, false, false>)))
  auto panel = DBS_PICK(k_diag_panel);
  auto tiles = DBS_PICK(k_tiles);
  auto strip = DBS_PICK(k_strip);
#undef DBS_PICK

  // phases 1 and 2 of block K: one launch (the diagonal tile alone when it is
  // the only block)
  auto phase12 = [&](int64_t K, hipStream_t st) -> hipError_t {
    if (TB == 1)
      return launch_small_block(U, L, n, nn, 0, (int)n, 0, (int)n, batch, st, prof, flags);
    return launch(prof, kProfPanel, panel, dim3((unsigned)(TB - 1), gy), dim3(kPanelThreads), st,
                  U, L, n, batch, K);
  };
  // s1: first atom of the band the bulk launch must leave alone (-1: none)
  auto phase3 = [&](int64_t K, int64_t s1, hipStream_t st) -> hipError_t {
    return launch(prof, kProfTiles, tiles, dim3((unsigned)(T * (T + 1) / 2), gy), dim3(kThreads),
                  st, U, L, n, batch, K, s1);
  };

  hipError_t e = phase12(K0, s);
  if (e != hipSuccess || TB == 1) return e;

  hipStream_t side = T > 1 ? side_stream() : nullptr;
  Events *ev = side ? thread_events() : nullptr;
  const bool ahead = side != nullptr && ev != nullptr;
  for (int64_t K = K0; K < K1 && e == hipSuccess; ++K) {
    if (K + 1 == K1) {
      e = phase3(K, -1, s);
    } else if (!ahead) {
      e = phase3(K, -1, s);
      if (e == hipSuccess) e = phase12(K + 1, s);
    } else {
      if ((e = hipEventRecord(ev->e[1], s)) != hipSuccess) break;
      if ((e = hipStreamWaitEvent(side, ev->e[1], 0)) != hipSuccess) break;
      if ((e = launch(prof, kProfStrip, strip, dim3((unsigned)(TB - 1), gy), dim3(kThreads), side,
                      U, L, n, batch, K)) != hipSuccess)
        break;
      if ((e = phase12(K + 1, side)) != hipSuccess) break;
      if ((e = hipEventRecord(ev->e[2], side)) != hipSuccess) break;
      if ((e = phase3(K, (K + 1) * BK, s)) != hipSuccess) break;
      e = hipStreamWaitEvent(s, ev->e[2], 0);
    }
  }
  // packed storage keeps one slot per value: nothing goes stale
  if (e == hipSuccess && T > 1 && !packed)
    e = launch(prof, kProfMirror, k_mirror, dim3((unsigned)(TB * TB), gy), dim3(kThreads), s, U,
               L, n, batch, TB);
  return e;
}

}  // namespace dbs
