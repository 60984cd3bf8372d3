// restraints.hip -- dense bound matrices from a restraint list, and the mask
// of cells a smoothing step changed.
//
// GPU Gems 2, Ch. 43 notes, §1: the experiment supplies an interval for some
// atom pairs; every other pair starts at a placeholder (the molecular
// diameter as its upper bound, about zero as its lower bound).  k_fill writes
// the placeholders (HBM-bound: 8 bytes per cell), k_scatter tightens the
// measured pairs with outward rounding to the 2^-6 grid.  Duplicate
// restraints of a pair combine through atomic min (upper) and max (lower) on
// the bit patterns, which order like the values for non-negative floats.
//
// k_tightened marks the cells whose bounds differ between two states (the
// notes' §5 experiment colours the entries tightened so far).
#include "dbs.h"
#include "dbs_internal.h"

namespace dbs {
namespace {

constexpr int kThreads = 256;
// The fill and the mask stream through HBM once: their stores (and the
// mask's loads) carry the non-temporal hint.  Measured at n12288, fill and
// scatter 0.217-0.224 ms against 0.226-0.228 without the hint, mask
// 0.449-0.453 ms against 0.486 (and 0.493-0.503 before it took two steps'
// loads at once).
constexpr bool kStreamFill = true, kStreamMask = true;

typedef float vf4 __attribute__((ext_vector_type(4)));
typedef uint32_t vu4 __attribute__((ext_vector_type(4)));

template <bool NT, typename T>
__device__ __forceinline__ void put(T *p, T v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}
template <bool NT, typename T>
__device__ __forceinline__ T get(const T *p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// Outward rounding to the 2^-6 grid; exact in fp32 for |x| < 2^17 (scaling
// by a power of two and floor/ceil introduce no rounding).
__device__ __forceinline__ float grid_down(float x) { return floorf(x * 64.0f) * 0.015625f; }
__device__ __forceinline__ float grid_up(float x) { return ceilf(x * 64.0f) * 0.015625f; }

// grid = (column groups of 4*kThreads, rows, molecules); 4 columns per thread.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_fill(float *__restrict__ U, float *__restrict__ L,
                                                   int64_t n, int64_t batch, float lo, float hi) {
  const int64_t j = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (j >= n) return;
  const int64_t nn = n * n;
  for (int64_t b = blockIdx.z; b < batch; b += gridDim.z)
    for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
      float *pu = U + b * nn + i * n + j;
      float *pl = L + b * nn + i * n + j;
      if (VEC) {
        vf4 u = {hi, hi, hi, hi}, l = {lo, lo, lo, lo};
        if (i >= j && i < j + 4) {
          u[i - j] = 0.0f;
          l[i - j] = 0.0f;
        }
        put<kStreamFill>(reinterpret_cast<vf4 *>(pu), u);
        put<kStreamFill>(reinterpret_cast<vf4 *>(pl), l);
      } else {
        for (int q = 0; q < 4 && j + q < n; ++q) {
          pu[q] = (i == j + q) ? 0.0f : hi;
          pl[q] = (i == j + q) ? 0.0f : lo;
        }
      }
    }
}

__global__ __launch_bounds__(kThreads) void k_scatter(float *__restrict__ U, float *__restrict__ L,
                                                      int64_t n, int64_t batch,
                                                      const int32_t *__restrict__ mol,
                                                      const int32_t *__restrict__ ia,
                                                      const int32_t *__restrict__ ja,
                                                      const float *__restrict__ lo,
                                                      const float *__restrict__ hi, int64_t count,
                                                      uint32_t *__restrict__ status) {
  const int64_t nn = n * n;
  uint32_t bad_all = 0;
  for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < count;
       r += (int64_t)gridDim.x * kThreads) {
    const int64_t b = mol ? mol[r] : 0, i = ia[r], j = ja[r];
    const float l = lo[r], h = hi[r];
    uint32_t bad = 0;
    if (b < 0 || b >= batch || i < 0 || i >= n || j < 0 || j >= n) bad |= DBS_RESTRAINT_INDEX;
    const float lr = grid_down(fmaxf(l, 0.0f)), hr = grid_up(h);
    if (!(isfinite(l) && isfinite(h)) || l > h || h < 0.0f || fabsf(l) >= 131072.0f ||
        hr >= 131072.0f)
      bad |= DBS_RESTRAINT_VALUE;
    if (bad) {
      bad_all |= bad;
      continue;
    }
    if (i == j) continue;
    unsigned int *Ub = reinterpret_cast<unsigned int *>(U + b * nn);
    unsigned int *Lb = reinterpret_cast<unsigned int *>(L + b * nn);
    atomicMin(Ub + i * n + j, __float_as_uint(hr));
    atomicMin(Ub + j * n + i, __float_as_uint(hr));
    atomicMax(Lb + i * n + j, __float_as_uint(lr));
    atomicMax(Lb + j * n + i, __float_as_uint(lr));
  }
  if (bad_all && status) atomicOr(status, bad_all);
}

// VEC: total % 4 == 0, the float arrays 16-byte and the mask 4-byte aligned;
// each thread then handles 4 consecutive cells a step, two steps' loads in
// flight at once.
__device__ __forceinline__ uint32_t changed4(vu4 a, vu4 b, vu4 c, vu4 d) {
  return (uint32_t)(a.x != b.x || c.x != d.x) | (uint32_t)(a.y != b.y || c.y != d.y) << 8 |
         (uint32_t)(a.z != b.z || c.z != d.z) << 16 | (uint32_t)(a.w != b.w || c.w != d.w) << 24;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_tightened(const float *__restrict__ U0,
                                                        const float *__restrict__ L0,
                                                        const float *__restrict__ U1,
                                                        const float *__restrict__ L1,
                                                        int64_t total, uint8_t *__restrict__ mask) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  if (VEC) {
    const vu4 *u0 = reinterpret_cast<const vu4 *>(U0), *u1 = reinterpret_cast<const vu4 *>(U1);
    const vu4 *l0 = reinterpret_cast<const vu4 *>(L0), *l1 = reinterpret_cast<const vu4 *>(L1);
    uint32_t *m4 = reinterpret_cast<uint32_t *>(mask);
    const int64_t n4 = total / 4;
    int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; e + stride < n4; e += 2 * stride) {
      constexpr bool N = kStreamMask;
      const vu4 a0 = get<N>(u0 + e), b0 = get<N>(u1 + e), c0 = get<N>(l0 + e), d0 = get<N>(l1 + e);
      const vu4 a1 = get<N>(u0 + e + stride), b1 = get<N>(u1 + e + stride);
      const vu4 c1 = get<N>(l0 + e + stride), d1 = get<N>(l1 + e + stride);
      put<N>(m4 + e, changed4(a0, b0, c0, d0));
      put<N>(m4 + e + stride, changed4(a1, b1, c1, d1));
    }
    if (e < n4) {
      constexpr bool N = kStreamMask;
      put<N>(m4 + e, changed4(get<N>(u0 + e), get<N>(u1 + e), get<N>(l0 + e), get<N>(l1 + e)));
    }
    return;
  }
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const bool changed = __float_as_uint(U0[e]) != __float_as_uint(U1[e]) ||
                         __float_as_uint(L0[e]) != __float_as_uint(L1[e]);
    mask[e] = changed ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_restraints(float *U, float *L, int64_t n, int64_t batch, float unknown_L,
                             float unknown_U, const int32_t *mol, const int32_t *ia,
                             const int32_t *ja, const float *lo, const float *hi, int64_t count,
                             uint32_t *status, hipStream_t s, Prof *prof) {
  const bool vec = (n % 4 == 0) && aligned16(U) && aligned16(L);
  const dim3 g((unsigned)ceil_div(n, 4 * kThreads), (unsigned)(n < kMaxGridYZ ? n : kMaxGridYZ),
               (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ));
  hipError_t e = launch(prof, kProfFill, vec ? k_fill<true> : k_fill<false>, g, dim3(kThreads), s,
                        U, L, n, batch, unknown_L, unknown_U);
  if (e != hipSuccess || count == 0) return e;
  int64_t blocks = ceil_div(count, kThreads);
  if (blocks > 65536) blocks = 65536;
  return launch(prof, kProfScatter, k_scatter, dim3((unsigned)blocks), dim3(kThreads), s, U, L, n,
                batch, mol, ia, ja, lo, hi, count, status);
}

hipError_t launch_tightened(const float *U0, const float *L0, const float *U1, const float *L1,
                            int64_t n, int64_t batch, uint8_t *mask, hipStream_t s) {
  const int64_t total = n * n * batch;
  const bool vec = total % 4 == 0 && aligned16(U0) && aligned16(L0) && aligned16(U1) &&
                   aligned16(L1) && (reinterpret_cast<uintptr_t>(mask) & 3u) == 0;
  // (two vector steps per thread)
  int64_t blocks = vec ? ceil_div(total / 4, 2 * kThreads) : ceil_div(total, kThreads);
  if (blocks > ((int64_t)1 << 20)) blocks = (int64_t)1 << 20;
  if (blocks < 1) blocks = 1;
  return launch(nullptr, 0, vec ? k_tightened<true> : k_tightened<false>, dim3((unsigned)blocks),
                dim3(kThreads), s, U0, L0, U1, L1, total, mask);
}

}  // namespace dbs
