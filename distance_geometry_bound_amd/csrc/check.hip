// check.hip -- device-side test of the per-entry preconditions of a pass.
//
// The update of GPU Gems 2, Ch. 43 notes, §2 is exact here only for bound
// matrices that are symmetric with a zero diagonal (the notes' §1 keeps
// D[i,j] = D[j,i] and a zero diagonal), finite, 0 <= L, and on the 2^-6 grid
// with |x| < 2^17 (fp32, the notes' §6).  Each thread tests some entries and
// ORs what it finds into one device word.  Run on the output of a pass,
// DBS_CHECK_L_GT_U reveals inconsistent bounds.
#include "dbs.h"
#include "dbs_internal.h"

namespace dbs {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t entry_flags(float x) {
  uint32_t f = 0;
  const uint32_t bits = __float_as_uint(x);
  if (bits == 0x80000000u) f |= DBS_CHECK_NEGZERO;
  if (!isfinite(x)) return f | DBS_CHECK_NONFINITE;
  const float s = x * 64.0f;  // exact: scaling by a power of two
  if (s != floorf(s)) f |= DBS_CHECK_UNQUANT;
  if (fabsf(x) >= 131072.0f) f |= DBS_CHECK_RANGE;
  return f;
}

__global__ __launch_bounds__(kThreads) void k_check(const float *__restrict__ U,
                                                    const float *__restrict__ L, int64_t n,
                                                    int64_t batch, uint32_t *__restrict__ flags) {
  const int64_t nn = n * n;
  const int64_t total = nn * batch;
  uint32_t f = 0;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t b = e / nn, r = e % nn, i = r / n, j = r % n;
    const float u = U[e], l = L[e];
    f |= entry_flags(u) | entry_flags(l);
    const int64_t t = b * nn + j * n + i;
    if (__float_as_uint(U[t]) != __float_as_uint(u) || __float_as_uint(L[t]) != __float_as_uint(l))
      f |= DBS_CHECK_ASYM;
    if (i == j && (__float_as_uint(u) != 0u || __float_as_uint(l) != 0u)) f |= DBS_CHECK_DIAG;
    if (l > u) f |= DBS_CHECK_L_GT_U;
    if (l < 0.0f) f |= DBS_CHECK_L_NEG;
  }
  if (f) atomicOr(flags, f);
}

// Packed buffer: U[i,j] = P[min,max], L[i,j] = P[max,min].  The tile pairs
// (I <= J) of PT x PT tiles are dealt to the workgroups of grid.x; for each,
// a workgroup tests the entries of tile (I, J) and of its mirror (J, I)
// (read transposed through LDS so that both reads are row-contiguous), and
// the pair conditions L <= U and 0 <= L on the cells of tile (I, J) above the
// diagonal.
constexpr int PT = 64;

__global__ __launch_bounds__(kThreads) void k_check_packed(const float *__restrict__ P, int64_t n,
                                                           int64_t batch,
                                                           uint32_t *__restrict__ flags) {
  __shared__ float t[PT][PT + 1];
  const int tid = threadIdx.x;
  const int64_t T = ceil_div(n, PT), pairs = T * (T + 1) / 2, nn = n * n;
  uint32_t f = 0;
  for (int64_t p = blockIdx.x; p < pairs; p += gridDim.x) {
    const int64_t J = tri_col(p), I = p - J * (J + 1) / 2;
    const int64_t i0 = I * PT, j0 = J * PT;
    for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
      const float *Pb = P + b * nn;
      for (int e = tid; e < PT * PT; e += kThreads) {
        const int r = e / PT, c = e % PT;
        const int64_t gi = j0 + r, gj = i0 + c;  // P[j0 + r][i0 + c]
        if (gi < n && gj < n) t[r][c] = Pb[gi * n + gj];
      }
      __syncthreads();
      for (int e = tid; e < PT * PT; e += kThreads) {
        const int r = e / PT, c = e % PT;
        const int64_t i = i0 + r, j = j0 + c;
        if (i >= n || j >= n) continue;
        const float d = Pb[i * n + j];  // P[i][j]
        const float m = t[c][r];        // P[j][i]
        f |= entry_flags(d);
        if (I != J) f |= entry_flags(m);
        if (i < j) {
          if (m > d) f |= DBS_CHECK_L_GT_U;
          if (m < 0.0f) f |= DBS_CHECK_L_NEG;
        } else if (i == j && __float_as_uint(d) != 0u) {
          f |= DBS_CHECK_DIAG;
        }
      }
      __syncthreads();
    }
  }
  if (f) atomicOr(flags, f);
}

// The infeasibility option's test of a pass's output (dense): words[b] gets
// DBS_INFEASIBLE_END when a cell of molecule b has L > U.  grid.y =
// molecules; each workgroup ORs the result of its cells once.
__global__ __launch_bounds__(kThreads) void k_infeasible(const float *__restrict__ U,
                                                         const float *__restrict__ L, int64_t n,
                                                         int64_t batch,
                                                         uint32_t *__restrict__ words) {
  const int64_t nn = n * n;
  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    const float *Ub = U + b * nn, *Lb = L + b * nn;
    int bad = 0;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < nn;
         e += (int64_t)gridDim.x * kThreads)
      bad |= Lb[e] > Ub[e];
    if (__syncthreads_or(bad) && threadIdx.x == 0) atomicOr(&words[b], DBS_INFEASIBLE_END);
  }
}

// The same on the packed buffer: for i < j, L = P[j][i] against U = P[i][j].
// The tile pairs (I <= J) of PT x PT tiles are dealt to the workgroups of
// grid.x; a workgroup reads tile (J, I) transposed through LDS, so that both
// reads are row-contiguous.
__global__ __launch_bounds__(kThreads) void k_infeasible_packed(const float *__restrict__ P,
                                                                int64_t n, int64_t batch,
                                                                uint32_t *__restrict__ words) {
  __shared__ float t[PT][PT + 1];
  const int tid = threadIdx.x;
  const int64_t T = ceil_div(n, PT), pairs = T * (T + 1) / 2, nn = n * n;
  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    const float *Pb = P + b * nn;
    int bad = 0;
    for (int64_t p = blockIdx.x; p < pairs; p += gridDim.x) {
      const int64_t J = tri_col(p), I = p - J * (J + 1) / 2;
      const int64_t i0 = I * PT, j0 = J * PT;
      for (int e = tid; e < PT * PT; e += kThreads) {
        const int r = e / PT, c = e % PT;
        const int64_t gi = j0 + r, gj = i0 + c;  // P[j0 + r][i0 + c]
        if (gi < n && gj < n) t[r][c] = Pb[gi * n + gj];
      }
      __syncthreads();
      for (int e = tid; e < PT * PT; e += kThreads) {
        const int r = e / PT, c = e % PT;
        const int64_t i = i0 + r, j = j0 + c;
        if (i < j && j < n) bad |= t[c][r] > Pb[i * n + j];  // L(i,j) > U(i,j)
      }
      __syncthreads();
    }
    if (__syncthreads_or(bad) && tid == 0) atomicOr(&words[b], DBS_INFEASIBLE_END);
  }
}

}  // namespace

hipError_t launch_infeasible(const float *U, const float *L, int64_t n, int64_t batch,
                             uint32_t *words, hipStream_t s) {
  int64_t blocks = ceil_div(n * n, kThreads);
  if (blocks > 1024) blocks = 1024;
  const dim3 g((unsigned)blocks, (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ));
  return launch(nullptr, 0, k_infeasible, g, dim3(kThreads), s, U, L, n, batch, words);
}

hipError_t launch_infeasible_packed(const float *P, int64_t n, int64_t batch, uint32_t *words,
                                    hipStream_t s) {
  const int64_t T = ceil_div(n, PT), pairs = T * (T + 1) / 2;
  const dim3 g((unsigned)(pairs < 1024 ? pairs : 1024),
               (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ));
  return launch(nullptr, 0, k_infeasible_packed, g, dim3(kThreads), s, P, n, batch, words);
}

hipError_t launch_check_packed(const float *P, int64_t n, int64_t batch, uint32_t *flags,
                               hipStream_t s) {
  const int64_t T = ceil_div(n, PT), pairs = T * (T + 1) / 2;
  const dim3 g((unsigned)(pairs < (1 << 20) ? pairs : (1 << 20)),
               (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ));
  return launch(nullptr, 0, k_check_packed, g, dim3(kThreads), s, P, n, batch, flags);
}

hipError_t launch_check(const float *U, const float *L, int64_t n, int64_t batch,
                        uint32_t *flags, hipStream_t s) {
  const int64_t total = n * n * batch;
  int64_t blocks = ceil_div(total, kThreads);
  if (blocks > 65536) blocks = 65536;
  return launch(nullptr, 0, k_check, dim3((unsigned)blocks), dim3(kThreads), s, U, L, n, batch,
                flags);
}

}  // namespace dbs
