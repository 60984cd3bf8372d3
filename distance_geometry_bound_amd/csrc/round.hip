// round.hip -- one Floyd-Warshall round k over every pair (i,j), in place.
//
// This is the round structure of GPU Gems 2, Ch. 43 notes, §3-§4: one
// launch per intermediate atom k covering the whole matrix, each cell written
// by exactly one thread.  The notes' ping-pong buffers are not needed: row k
// and column k are unchanged by round k, so the in-place result is identical.
// Each thread owns four consecutive columns of one row (the notes' RGBA
// packing of four neighbouring entries, §4) and reads the broadcast value of
// column k of its row once.
//
// Bound by HBM: per cell and round it reads U[i,j], L[i,j] and writes them
// back (16 bytes); row k (8n bytes) and column k stay in cache.
#include "dbs_internal.h"

namespace dbs {
namespace {

constexpr int kThreads = 256;

// The matrix streams through once per round (1.2 GB at n = 12288, more than
// the caches hold), so its loads and stores are nontemporal: they keep row k
// and column k, which every workgroup reads, in the caches.  The builtins
// take clang vector types.
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float4 *p) {
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void store_stream(float4 x, float4 *p) {
  const v4f v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(p));
}

// Vector path: n % 4 == 0 and both base pointers 16-byte aligned.  A thread
// owns four columns of kRows consecutive rows, and issues the loads of all
// of them before it computes (more bytes in flight per thread).
// RU: directed rounding (dbs_internal.h).
constexpr int kRows = 2;

template <bool RU>
__global__ __launch_bounds__(kThreads) void k_round_vec(float *__restrict__ U,
                                                        float *__restrict__ L, int64_t n,
                                                        int64_t batch, int64_t k) {
  rounding_prologue<RU>();
  const int64_t n4 = n >> 2;
  const int64_t j4 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j4 >= n4) return;
  const int64_t nn = n * n;
  for (int64_t b = blockIdx.z; b < batch; b += gridDim.z) {
    float *Ub = U + b * nn;
    float *Lb = L + b * nn;
    const float4 ru = reinterpret_cast<const float4 *>(Ub + k * n)[j4];
    const float4 rl = reinterpret_cast<const float4 *>(Lb + k * n)[j4];
    for (int64_t i0 = (int64_t)blockIdx.y * kRows; i0 < n; i0 += (int64_t)gridDim.y * kRows) {
      float4 u[kRows], l[kRows];
      float cu[kRows], cl[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int64_t i = i0 + r < n ? i0 + r : n - 1;  // a row past n reads the last one
        cu[r] = Ub[i * n + k];
        cl[r] = Lb[i * n + k];
        u[r] = load_stream(reinterpret_cast<const float4 *>(Ub + i * n) + j4);
        l[r] = load_stream(reinterpret_cast<const float4 *>(Lb + i * n) + j4);
      }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int64_t i = i0 + r;
        if (i >= n || i == k) continue;  // row k is unchanged by round k
        relax1<RU>(u[r].x, l[r].x, cu[r], cl[r], ru.x, rl.x);
        relax1<RU>(u[r].y, l[r].y, cu[r], cl[r], ru.y, rl.y);
        relax1<RU>(u[r].z, l[r].z, cu[r], cl[r], ru.z, rl.z);
        relax1<RU>(u[r].w, l[r].w, cu[r], cl[r], ru.w, rl.w);
        store_stream(u[r], reinterpret_cast<float4 *>(Ub + i * n) + j4);
        store_stream(make_float4(lower_out<RU>(l[r].x), lower_out<RU>(l[r].y),
                                 lower_out<RU>(l[r].z), lower_out<RU>(l[r].w)),
                     reinterpret_cast<float4 *>(Lb + i * n) + j4);
      }
    }
  }
}

// Scalar path: any n, any 4-byte alignment.
template <bool RU>
__global__ __launch_bounds__(kThreads) void k_round_scalar(float *__restrict__ U,
                                                           float *__restrict__ L, int64_t n,
                                                           int64_t batch, int64_t k) {
  rounding_prologue<RU>();
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= n) return;
  const int64_t nn = n * n;
  for (int64_t b = blockIdx.z; b < batch; b += gridDim.z) {
    float *Ub = U + b * nn;
    float *Lb = L + b * nn;
    const float ru = Ub[k * n + j];
    const float rl = Lb[k * n + j];
    for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
      if (i == k) continue;
      const float cu = Ub[i * n + k];
      const float cl = Lb[i * n + k];
      float u = Ub[i * n + j], l = Lb[i * n + j];
      relax1<RU>(u, l, cu, cl, ru, rl);
      Ub[i * n + j] = u;
      Lb[i * n + j] = lower_out<RU>(l);
    }
  }
}

}  // namespace

hipError_t launch_round(float *U, float *L, int64_t n, int64_t batch, int64_t k,
                        hipStream_t s, Prof *prof, unsigned flags) {
  const bool vec = (n % 4 == 0) && aligned16(U) && aligned16(L);
  const int64_t cols = vec ? n / 4 : n;
  const int64_t rows = vec ? ceil_div(n, kRows) : n;
  dim3 grid((unsigned)ceil_div(cols, kThreads), (unsigned)(rows < kMaxGridYZ ? rows : kMaxGridYZ),
            (unsigned)(batch < kMaxGridYZ ? batch : kMaxGridYZ));
  const bool ru = flags & kDirected;
  auto kern = vec ? (ru ? k_round_vec<true> : k_round_vec<false>)
                  : (ru ? k_round_scalar<true> : k_round_scalar<false>);
  return launch(prof, kProfRound, kern, grid, dim3(kThreads), s, U, L, n, batch, k);
}

}  // namespace dbs
