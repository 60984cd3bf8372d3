// blocked.hip -- one smoothing pass as blocked Floyd-Warshall in three
// phases per block of BK intermediate atoms.
//
// The pages give the per-round update (GPU Gems 2, Ch. 43 notes, §2-§3); the
// blocked order is ours.  Under the exactness preconditions it reaches the
// same bits as the plain round order: the fused round is Floyd-Warshall on a
// graph with no negative cycle, every candidate is exact on the 2^-6 grid, so
// any partition of the rounds into blocks yields the same shortest paths.
//
// For k-block K (atoms k0..k0+bK-1):
//   phase 1  the diagonal tile (K,K): a full pass over it, rounds in order
//            (k_small, one workgroup per molecule);
//   phase 2  every other tile on row K ("panel"): rounds in order, reading
//            the final diagonal tile (k_panel, one workgroup per tile);
//   phase 3  every remaining tile: all bK rounds at once from the finished
//            panel (k_tiles).  This is where 1 - O(BK/n) of the work is.
//
// Symmetric schedule.  U and L stay exactly symmetric, so only the cells of
// TILE x TILE tiles (I,J) with I <= J are kept current ("fresh"); tiles below
// the diagonal go stale and are rebuilt by one transposed copy at the end
// (k_mirror).  Phase 3 therefore does half the work of a dense schedule.  It
// reads its operands U/L[i,k] and U/L[k,j] from row k only (U[i,k] = U[k,i]),
// so phase 2 must leave all of row band K fresh: it updates each panel tile
// from whichever orientation is fresh and writes both orientations.
//
// Phase 3 kernel: a 256-thread workgroup owns a 128x128 tile; each thread an
// 8x8 register tile (rows ty*4+{0..3} and 64+ty*4+{0..3}, same for columns,
// so the LDS reads of a wave are contiguous).  The panel rows of the k-block
// are staged through LDS in chunks of KC atoms.  Per atom and cell the VALU
// does one add and one min for U, two subtracts and two max for L; pairs of
// atoms fold into 3-input min/max.  No matrix cores: min-plus is not a
// multiply-add contraction.
#include "dbs_internal.h"

namespace dbs {
namespace {

constexpr int BK = 64;          // atoms per k-block (phases 1 and 2 tile size)
constexpr int TILE = 128;       // phase-3 tile size; fresh region is I <= J in these tiles
constexpr int RATIO = TILE / BK;
constexpr int KC = 16;          // atoms per LDS chunk in phase 3
constexpr int kThreads = 256;

// (k-block tile a, k-block tile b) is fresh under the symmetric schedule
__device__ __forceinline__ bool fresh(int64_t a, int64_t b) { return a / RATIO <= b / RATIO; }

// ---------------------------------------------------------------- phase 2
// grid.x = k-block tiles on row K other than K itself, grid.y = molecules.
// Thread (ty, tx) owns rows a = ty*4+{0..3}, columns c = tx*4+{0..3} of the
// panel tile R = (K, J) seen in row orientation.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_panel(float *__restrict__ U, float *__restrict__ L,
                                                    int64_t n, int64_t batch, int64_t K) {
  __shared__ float du[BK][BK];
  __shared__ float dl[BK][BK];
  __shared__ float vu[2][BK];
  __shared__ float vl[2][BK];

  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  int64_t J = blockIdx.x;
  if (J >= K) ++J;
  const int64_t k0 = K * BK, j0 = J * BK;
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int bJ = (int)(n - j0 < BK ? n - j0 : BK);
  const bool rowor = fresh(K, J);
  const int64_t nn = n * n;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = L + b * nn;

    // the finished diagonal tile (both halves current after phase 1)
    for (int e = tid; e < BK * BK; e += kThreads) {
      const int m = e / BK, a = e % BK;
      const bool in = m < bK && a < bK;
      const int64_t g = (k0 + m) * n + k0 + a;
      du[m][a] = in ? Ub[g] : kInf;
      dl[m][a] = in ? Lb[g] : 0.0f;
    }

    float u[4][4], l[4][4];
    if (rowor) {
      // R[a][c] = M[k0+a][j0+c]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = ty * 4 + r;
        const int64_t g = (k0 + a) * n + j0 + tx * 4;
        if (VEC) {
          const bool in = a < bK && tx * 4 < bJ;
          const float4 x = in ? *reinterpret_cast<const float4 *>(Ub + g) : make_float4(kInf, kInf, kInf, kInf);
          const float4 y = in ? *reinterpret_cast<const float4 *>(Lb + g) : make_float4(0.f, 0.f, 0.f, 0.f);
          u[r][0] = x.x; u[r][1] = x.y; u[r][2] = x.z; u[r][3] = x.w;
          l[r][0] = y.x; l[r][1] = y.y; l[r][2] = y.z; l[r][3] = y.w;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool in = a < bK && tx * 4 + q < bJ;
            u[r][q] = in ? Ub[g + q] : kInf;
            l[r][q] = in ? Lb[g + q] : 0.0f;
          }
        }
      }
    } else {
      // R[a][c] = M[j0+c][k0+a]
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tx * 4 + q;
        const int64_t g = (j0 + c) * n + k0 + ty * 4;
        if (VEC) {
          const bool in = c < bJ && ty * 4 < bK;
          const float4 x = in ? *reinterpret_cast<const float4 *>(Ub + g) : make_float4(kInf, kInf, kInf, kInf);
          const float4 y = in ? *reinterpret_cast<const float4 *>(Lb + g) : make_float4(0.f, 0.f, 0.f, 0.f);
          u[0][q] = x.x; u[1][q] = x.y; u[2][q] = x.z; u[3][q] = x.w;
          l[0][q] = y.x; l[1][q] = y.y; l[2][q] = y.z; l[3][q] = y.w;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool in = c < bJ && ty * 4 + r < bK;
            u[r][q] = in ? Ub[g + r] : kInf;
            l[r][q] = in ? Lb[g + r] : 0.0f;
          }
        }
      }
    }
    __syncthreads();

    for (int mb = 0; mb < BK / 4; ++mb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mb * 4 + r;
        if (m >= bK) break;  // uniform
        const int buf = m & 1;
        if (ty == mb) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            vu[buf][tx * 4 + q] = u[r][q];
            vl[buf][tx * 4 + q] = l[r][q];
          }
        }
        __syncthreads();
        float ru[4], rl[4], cu[4], cl[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ru[q] = vu[buf][tx * 4 + q];
          rl[q] = vl[buf][tx * 4 + q];
          cu[q] = du[m][ty * 4 + q];  // U[i,k] = D[a][m] = D[m][a]
          cl[q] = dl[m][ty * 4 + q];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) relax1(u[a][q], l[a][q], cu[a], cl[a], ru[q], rl[q]);
      }
    }

    // write both orientations
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int a = ty * 4 + r, c = tx * 4 + q;
        if (a < bK && c < bJ) {
          Ub[(k0 + a) * n + j0 + c] = u[r][q];
          Lb[(k0 + a) * n + j0 + c] = l[r][q];
          Ub[(j0 + c) * n + k0 + a] = u[r][q];
          Lb[(j0 + c) * n + k0 + a] = l[r][q];
        }
      }
    __syncthreads();  // LDS reuse by the next molecule
  }
}

// ---------------------------------------------------------------- phase 3
__device__ __forceinline__ int64_t tri_col(int64_t p) {
  // p -> J with J(J+1)/2 <= p < (J+1)(J+2)/2
  int64_t J = (int64_t)((sqrt(8.0 * (double)p + 1.0) - 1.0) * 0.5);
  while (J * (J + 1) / 2 > p) --J;
  while ((J + 1) * (J + 2) / 2 <= p) ++J;
  return J;
}

// grid.x = T(T+1)/2 tiles (I <= J, column-major over the upper triangle),
// grid.y = molecules.
template <bool VEC>
__global__ __launch_bounds__(kThreads, 2) void k_tiles(float *__restrict__ U,
                                                       float *__restrict__ L, int64_t n,
                                                       int64_t batch, int64_t K) {
  __shared__ float4 scu[KC][TILE / 4];
  __shared__ float4 scl[KC][TILE / 4];
  __shared__ float4 sru[KC][TILE / 4];
  __shared__ float4 srl[KC][TILE / 4];

  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t p = blockIdx.x;
  const int64_t J = tri_col(p);
  const int64_t I = p - J * (J + 1) / 2;
  const int64_t i0 = I * TILE, j0 = J * TILE;
  const int64_t k0 = K * BK;
  const int bK = (int)(n - k0 < BK ? n - k0 : BK);
  const int64_t nn = n * n;

  // rows of this thread: i0 + rofs(r), r < 8; columns likewise with tx
  auto rofs = [](int t, int r) { return (r < 4 ? 0 : TILE / 2 - 4) + t * 4 + r; };

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    float *Ub = U + b * nn;
    float *Lb = L + b * nn;

    float u[8][8], l[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t i = i0 + rofs(ty, r);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t j = j0 + rofs(tx, h * 4);
        const int64_t g = i * n + j;
        if (VEC) {
          const bool in = i < n && j < n;
          const float4 x = in ? *reinterpret_cast<const float4 *>(Ub + g) : make_float4(kInf, kInf, kInf, kInf);
          const float4 y = in ? *reinterpret_cast<const float4 *>(Lb + g) : make_float4(0.f, 0.f, 0.f, 0.f);
          u[r][h * 4 + 0] = x.x; u[r][h * 4 + 1] = x.y; u[r][h * 4 + 2] = x.z; u[r][h * 4 + 3] = x.w;
          l[r][h * 4 + 0] = y.x; l[r][h * 4 + 1] = y.y; l[r][h * 4 + 2] = y.z; l[r][h * 4 + 3] = y.w;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool in = i < n && j + q < n;
            u[r][h * 4 + q] = in ? Ub[g + q] : kInf;
            l[r][h * 4 + q] = in ? Lb[g + q] : 0.0f;
          }
        }
      }
    }

    for (int kc = 0; kc < bK; kc += KC) {
      // stage panel rows k0+kc .. k0+kc+KC-1, columns of I and of J
      for (int e = tid; e < KC * (TILE / 4); e += kThreads) {
        const int kk = e / (TILE / 4), x4 = e % (TILE / 4);
        const int64_t k = k0 + kc + kk;
        const bool kin = kc + kk < bK;
        const int64_t ci = i0 + x4 * 4, cj = j0 + x4 * 4;
        float4 a, c, d, f;
        if (VEC) {
          const bool ini = kin && ci < n, inj = kin && cj < n;
          a = ini ? *reinterpret_cast<const float4 *>(Ub + k * n + ci) : make_float4(kInf, kInf, kInf, kInf);
          c = ini ? *reinterpret_cast<const float4 *>(Lb + k * n + ci) : make_float4(0.f, 0.f, 0.f, 0.f);
          d = inj ? *reinterpret_cast<const float4 *>(Ub + k * n + cj) : make_float4(kInf, kInf, kInf, kInf);
          f = inj ? *reinterpret_cast<const float4 *>(Lb + k * n + cj) : make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
          float ta[4], tc[4], td[4], tf[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool ini = kin && ci + q < n, inj = kin && cj + q < n;
            ta[q] = ini ? Ub[k * n + ci + q] : kInf;
            tc[q] = ini ? Lb[k * n + ci + q] : 0.0f;
            td[q] = inj ? Ub[k * n + cj + q] : kInf;
            tf[q] = inj ? Lb[k * n + cj + q] : 0.0f;
          }
          a = make_float4(ta[0], ta[1], ta[2], ta[3]);
          c = make_float4(tc[0], tc[1], tc[2], tc[3]);
          d = make_float4(td[0], td[1], td[2], td[3]);
          f = make_float4(tf[0], tf[1], tf[2], tf[3]);
        }
        scu[kk][x4] = a;
        scl[kk][x4] = c;
        sru[kk][x4] = d;
        srl[kk][x4] = f;
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
            relax2(u[r][c], l[r][c], cu0[r], cl0[r], ru0[c], rl0[c], cu1[r], cl1[r], ru1[c],
                   rl1[c]);
      }
      __syncthreads();
    }

    // store, except the k-block's own rows and columns (final after phase 2)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t i = i0 + rofs(ty, r);
      const bool row_ok = i < n && (i < k0 || i >= k0 + bK);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int64_t j = j0 + rofs(tx, c);
        if (row_ok && j < n && (j < k0 || j >= k0 + bK)) {
          Ub[i * n + j] = u[r][c];
          Lb[i * n + j] = l[r][c];
        }
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

}  // namespace

hipError_t launch_blocked(float *U, float *L, int64_t n, int64_t batch, hipStream_t s,
                          Prof *prof) {
  if (n <= 1) return hipSuccess;
  const int64_t TB = ceil_div(n, BK);    // k-blocks
  const int64_t T = ceil_div(n, TILE);   // phase-3 tiles per side
  const bool vec = (n % 4 == 0) && aligned16(U) && aligned16(L);
  const unsigned gy = (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ);
  const int64_t nn = n * n;
  hipError_t e = hipSuccess;
  for (int64_t K = 0; K < TB && e == hipSuccess; ++K) {
    const int64_t k0 = K * BK;
    const int bK = (int)(n - k0 < BK ? n - k0 : BK);
    e = launch_small_block(U, L, n, nn, k0 * n + k0, bK, batch, s, prof);
    if (e != hipSuccess || TB == 1) break;
    const dim3 g2((unsigned)(TB - 1), gy);
    e = launch(prof, kProfPanel, vec ? k_panel<true> : k_panel<false>, g2, dim3(kThreads), s, U,
               L, n, batch, K);
    if (e != hipSuccess) break;
    const dim3 g3((unsigned)(T * (T + 1) / 2), gy);
    e = launch(prof, kProfTiles, vec ? k_tiles<true> : k_tiles<false>, g3, dim3(kThreads), s, U,
               L, n, batch, K);
  }
  if (e == hipSuccess && T > 1)
    e = launch(prof, kProfMirror, k_mirror, dim3((unsigned)(TB * TB), gy), dim3(kThreads), s, U,
               L, n, batch, TB);
  return e;
}

}  // namespace dbs
