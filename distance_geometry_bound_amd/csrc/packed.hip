// packed.hip -- the bounds of a molecule in one n x n buffer.
//
// GPU Gems 2, Ch. 43 notes, §6: U and L are symmetric, so one triangle of
// each suffices; the chapter keeps the two triangles.  Here one buffer P
// holds both: P[i,j] = U[i,j] above the diagonal, L[i,j] below it, and the
// (zero) diagonal on it.  That halves the memory of a molecule.
//
// A round k in this layout: every cell of P is either an upper bound
// (i < j) or a lower bound (i > j), and relaxes from round k's vectors
//   u[x] = U[k,x] = P[min(k,x), max(k,x)],  l[x] = L[k,x] = P[max(k,x), min(k,x)],
// which are row k and column k of P:
//   i < j:  P[i,j] = min(P[i,j], u[i] + u[j])
//   i > j:  P[i,j] = max(P[i,j], l[i] - u[j], l[j] - u[i])
// (the update of the notes' §2 with U[i,k] = u[i], L[k,j] = l[j], ...).
// Row k and column k do not change in round k, so the round runs in place.
// One workgroup owns a 64 x 64 tile of P: it gathers the 4 x 64 vector
// entries it needs once (the column-k part is a strided read that stays in
// cache), then streams the tile (16 bytes per cell pair read and written
// once per round: HBM-bound).
#include "dbs_internal.h"

namespace dbs {
namespace {

constexpr int kThreads = 256;
constexpr int PT = 64;  // tile side

// Pack and unpack stream through HBM once: four-column vectors, and stores
// with the non-temporal hint.
typedef float vf4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void put4(float *p, vf4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<vf4 *>(p));
}

// grid = (tiles per side, tiles per side, molecules); thread (ty, tx) owns
// rows 4ty..4ty+3 and columns 4tx..4tx+3 of the tile.
template <bool VEC, bool RU>
__global__ __launch_bounds__(kThreads) void k_round_packed(float *__restrict__ P, int64_t n,
                                                           int64_t batch, int64_t k) {
  __shared__ float su[2][PT], sl[2][PT];  // [0]: rows of the tile, [1]: columns
  rounding_prologue<RU>();
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t i0 = (int64_t)blockIdx.y * PT, j0 = (int64_t)blockIdx.x * PT;
  const int64_t nn = n * n;
  for (int64_t b = blockIdx.z; b < batch; b += gridDim.z) {
    float *Pb = P + b * nn;
    if (tid < 2 * PT) {
      const int side = tid / PT, x = tid % PT;
      const int64_t g = (side ? j0 : i0) + x;
      float u = kInf, l = 0.0f;
      if (g < n) {
        const int64_t lo = g < k ? g : k, hi = g < k ? k : g;
        u = Pb[lo * n + hi];
        l = Pb[hi * n + lo];
      }
      su[side][x] = u;
      sl[side][x] = l;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = ty * 4 + r;
      const int64_t i = i0 + a;
      if (i >= n || i == k) continue;
      const float ui = su[0][a], li = sl[0][a];
      float *row = Pb + i * n + j0 + tx * 4;
      float v[4];
      const int64_t jb = j0 + tx * 4;
      if (VEC && jb + 3 < n) {
        const float4 x = *reinterpret_cast<const float4 *>(row);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = jb + q < n ? row[q] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t j = jb + q;
        const float uj = su[1][tx * 4 + q], lj = sl[1][tx * 4 + q];
        if (i < j)
          v[q] = fminf(v[q], ui + uj);
        else if (i > j)
          v[q] = RU ? lower_out<RU>(fmaxf(fmaxf(v[q], -(uj - li)), -(ui - lj)))
                    : fmaxf(fmaxf(v[q], li - uj), lj - ui);
      }
      // column k is unchanged by round k; rewriting it with the same value
      // would race with other workgroups' reads of it, so it is skipped
      if (VEC && jb + 3 < n && (k < jb || k > jb + 3)) {
        *reinterpret_cast<float4 *>(row) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (jb + q < n && jb + q != k) row[q] = v[q];
      }
    }
    __syncthreads();
  }
}

// P[i,j] = U[i,j] (i < j), L[i,j] (i > j), U[i,i] (i == j); grid = (column
// groups, rows, molecules), VEC: 4 columns per thread (n % 4 == 0, all
// buffers 16-byte aligned), else one.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_pack(const float *__restrict__ U,
                                                   const float *__restrict__ L,
                                                   float *__restrict__ P, int64_t n,
                                                   int64_t batch) {
  const int64_t j = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * (VEC ? 4 : 1);
  if (j >= n) return;
  const int64_t nn = n * n;
  for (int64_t b = blockIdx.z; b < batch; b += gridDim.z)
    for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
      const int64_t g = b * nn + i * n + j;
      if constexpr (VEC) {
        // columns j..j+3 all above the diagonal (U), all below it (L), or
        // across it
        vf4 v;
        if (j >= i) {
          v = *reinterpret_cast<const vf4 *>(U + g);
        } else if (j + 3 < i) {
          v = *reinterpret_cast<const vf4 *>(L + g);
        } else {
          const vf4 u = *reinterpret_cast<const vf4 *>(U + g);
          const vf4 l = *reinterpret_cast<const vf4 *>(L + g);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = i > j + q ? l[q] : u[q];
        }
        put4(P + g, v);
      } else {
        P[g] = i > j ? L[g] : U[g];
      }
    }
}

// U[i,j] = P[min,max], L[i,j] = P[max,min], both P[i,i] on the diagonal.
// grid = (tiles, tiles, molecules); workgroup (J, I) with I <= J reads the
// tiles A = P(I, J) and B = P(J, I) once, through LDS, and writes
// U(I, J) = A, L(I, J) = B^T, U(J, I) = A^T, L(J, I) = B (a diagonal tile:
// each cell from A or A^T by its side of the diagonal), so P is read once.
// VEC (n % 4 == 0, all buffers 16-byte aligned): rows move as four-column
// vectors.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_unpack(const float *__restrict__ P,
                                                     float *__restrict__ U,
                                                     float *__restrict__ L, int64_t n,
                                                     int64_t batch) {
  __shared__ float ta[PT][PT + 1], tb[PT][PT + 1];
  if (blockIdx.y > blockIdx.x) return;  // uniform: the pair's other workgroup
  const int tid = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.y * PT, j0 = (int64_t)blockIdx.x * PT;
  const bool diag = i0 == j0;
  const int64_t nn = n * n;
  constexpr int V = VEC ? 4 : 1;
  // tile (r0, c0) of P into t (rows r < n - r0, columns c < n - c0)
  auto load = [&](const float *Pb, int64_t r0, int64_t c0, float (*t)[PT + 1]) {
    for (int e = tid; e < PT * PT / V; e += kThreads) {
      const int r = e / (PT / V), c = (e % (PT / V)) * V;
      const int64_t gi = r0 + r, gj = c0 + c;
      if (gi >= n || gj >= n) continue;
      if constexpr (VEC) {
        const vf4 x = *reinterpret_cast<const vf4 *>(Pb + gi * n + gj);
#pragma unroll
        for (int q = 0; q < 4; ++q) t[r][c + q] = x[q];
      } else {
        t[r][c] = Pb[gi * n + gj];
      }
    }
  };
  // rows of the output tile (r0, c0) of M from t (transposed when T)
  auto store = [&](float *Mb, int64_t r0, int64_t c0, float (*t)[PT + 1], bool T) {
    for (int e = tid; e < PT * PT / V; e += kThreads) {
      const int r = e / (PT / V), c = (e % (PT / V)) * V;
      const int64_t gi = r0 + r, gj = c0 + c;
      if (gi >= n || gj >= n) continue;
      if constexpr (VEC) {
        vf4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = T ? t[c + q][r] : t[r][c + q];
        put4(Mb + gi * n + gj, v);
      } else {
        Mb[gi * n + gj] = T ? t[c][r] : t[r][c];
      }
    }
  };
  for (int64_t b = blockIdx.z; b < batch; b += gridDim.z) {
    const float *Pb = P + b * nn;
    float *Ub = U + b * nn, *Lb = L + b * nn;
    load(Pb, i0, j0, ta);
    if (!diag) load(Pb, j0, i0, tb);
    __syncthreads();
    if (diag) {
      // U from the upper triangle, L from the lower, mirrored across
      for (int e = tid; e < PT * PT; e += kThreads) {
        const int r = e / PT, c = e % PT;
        const int64_t gi = i0 + r, gj = i0 + c;
        if (gi >= n || gj >= n) continue;
        Ub[gi * n + gj] = r <= c ? ta[r][c] : ta[c][r];
        Lb[gi * n + gj] = r >= c ? ta[r][c] : ta[c][r];
      }
    } else {
      store(Ub, i0, j0, ta, false);
      store(Lb, i0, j0, tb, true);
      store(Ub, j0, i0, ta, true);
      store(Lb, j0, i0, tb, false);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_round_packed(float *P, int64_t n, int64_t batch, int64_t k, hipStream_t s,
                               Prof *prof, unsigned flags) {
  const bool vec = n % 4 == 0 && aligned16(P), ru = flags & kDirected;
  const unsigned tiles = (unsigned)ceil_div(n, PT);
  const dim3 g(tiles, tiles, (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ));
  auto kern = vec ? (ru ? k_round_packed<true, true> : k_round_packed<true, false>)
                  : (ru ? k_round_packed<false, true> : k_round_packed<false, false>);
  return launch(prof, kProfRound, kern, g, dim3(kThreads), s, P, n, batch, k);
}

hipError_t launch_pack(const float *U, const float *L, float *P, int64_t n, int64_t batch,
                       hipStream_t s) {
  const bool vec = n % 4 == 0 && aligned16(U) && aligned16(L) && aligned16(P);
  const dim3 g((unsigned)ceil_div(n, vec ? 4 * kThreads : kThreads),
               (unsigned)(n < kMaxGridYZ ? n : kMaxGridYZ),
               (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ));
  return launch(nullptr, 0, vec ? k_pack<true> : k_pack<false>, g, dim3(kThreads), s, U, L, P,
                n, batch);
}

hipError_t launch_unpack(const float *P, float *U, float *L, int64_t n, int64_t batch,
                         hipStream_t s) {
  const bool vec = n % 4 == 0 && aligned16(P) && aligned16(U) && aligned16(L);
  const unsigned tiles = (unsigned)ceil_div(n, PT);
  const dim3 g(tiles, tiles, (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ));
  return launch(nullptr, 0, vec ? k_unpack<true> : k_unpack<false>, g, dim3(kThreads), s, P, U,
                L, n, batch);
}

}  // namespace dbs
