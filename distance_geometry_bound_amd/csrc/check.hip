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

}  // namespace

hipError_t launch_check(const float *U, const float *L, int64_t n, int64_t batch,
                        uint32_t *flags, hipStream_t s) {
  const int64_t total = n * n * batch;
  int64_t blocks = ceil_div(total, kThreads);
  if (blocks > 65536) blocks = 65536;
  return launch(nullptr, 0, k_check, dim3((unsigned)blocks), dim3(kThreads), s, U, L, n, batch,
                flags);
}

}  // namespace dbs
