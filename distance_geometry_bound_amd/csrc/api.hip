// api.hip -- the extern "C" entry points declared in include/dbs.h:
// argument validation, device check, algorithm choice, launch sequencing.
#include <string.h>

#include <mutex>

#include "dbs.h"
#include "dbs_internal.h"

namespace {

constexpr int kVersion = 0x000100;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
signed char g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int device_status() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DBS_EDEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DBS_EDEVICE;
    g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return g_dev_ok[dev] == 1 ? DBS_OK : DBS_EDEVICE;
}

// Host-side argument checks shared by every entry point.
int validate(const void *U, const void *L, int64_t n, int64_t batch) {
  if (!U || !L || n < 1 || batch < 1) return DBS_EINVAL;
  if (n >= ((int64_t)1 << 31)) return DBS_EINVAL;
  const int64_t nn = n * n;  // < 2^62
  if (batch > INT64_MAX / 4 / nn) return DBS_EINVAL;
  const uint64_t bytes = (uint64_t)(nn * batch) * 4u;
  const uintptr_t u = reinterpret_cast<uintptr_t>(U), l = reinterpret_cast<uintptr_t>(L);
  if (u + bytes < u || l + bytes < l) return DBS_EINVAL;  // address wrap
  if (u < l + bytes && l < u + bytes) return DBS_EINVAL;  // overlap
  if ((u | l) & 3u) return DBS_EINVAL;                     // float alignment
  return DBS_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? DBS_OK : DBS_ELAUNCH; }

int run(float *U, float *L, int64_t n, int64_t batch, void *stream, int algo,
        dbs::Prof *prof = nullptr) {
  int st = validate(U, L, n, batch);
  if (st != DBS_OK) return st;
  if (algo < DBS_ALGO_AUTO || algo > DBS_ALGO_BLOCKED) return DBS_EINVAL;
  if (algo == DBS_ALGO_AUTO) algo = dbs_auto_algo(n, batch);
  if (algo == DBS_ALGO_LDS && n > dbs::kSmallMaxN) return DBS_EUNSUPPORTED;
  st = device_status();
  if (st != DBS_OK) return st;
  if (n == 1) return DBS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (algo) {
    case DBS_ALGO_PERK: {
      hipError_t e = hipSuccess;
      for (int64_t k = 0; k < n && e == hipSuccess; ++k)
        e = dbs::launch_round(U, L, n, batch, k, s, prof);
      return status_of(e);
    }
    case DBS_ALGO_LDS:
      return status_of(dbs::launch_small(U, L, n, batch, s, prof));
    default:
      return status_of(dbs::launch_blocked(U, L, n, batch, s, prof));
  }
}

}  // namespace

extern "C" {

int dbs_smooth(float *U, float *L, int64_t n, int64_t batch, void *stream) {
  return run(U, L, n, batch, stream, DBS_ALGO_AUTO);
}

int dbs_smooth_algo(float *U, float *L, int64_t n, int64_t batch, void *stream, int algo) {
  return run(U, L, n, batch, stream, algo);
}

int dbs_smooth_profiled(float *U, float *L, int64_t n, int64_t batch, void *stream, int algo,
                        int64_t *counts, double *ms) {
  if (!counts || !ms) return DBS_EINVAL;
  for (int i = 0; i < DBS_PROF_KINDS; ++i) {
    counts[i] = 0;
    ms[i] = 0.0;
  }
  dbs::Prof prof;
  int st = run(U, L, n, batch, stream, algo, &prof);
  if (st != DBS_OK) return st;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return DBS_ELAUNCH;
  for (const auto &m : prof.marks) {
    float t = 0.0f;
    if (hipEventElapsedTime(&t, m.start, m.stop) != hipSuccess) return DBS_ELAUNCH;
    counts[m.kind] += 1;
    ms[m.kind] += t;
  }
  return DBS_OK;
}

int dbs_rounds(float *U, float *L, int64_t n, int64_t batch, int64_t k_begin, int64_t k_end,
               void *stream) {
  int st = validate(U, L, n, batch);
  if (st != DBS_OK) return st;
  if (k_begin < 0 || k_end > n || k_begin > k_end) return DBS_EINVAL;
  st = device_status();
  if (st != DBS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  for (int64_t k = k_begin; k < k_end && e == hipSuccess; ++k)
    e = dbs::launch_round(U, L, n, batch, k, s);
  return status_of(e);
}

int dbs_check(const float *U, const float *L, int64_t n, int64_t batch, uint32_t *d_flags,
              void *stream) {
  int st = validate(U, L, n, batch);
  if (st != DBS_OK) return st;
  if (!d_flags) return DBS_EINVAL;
  st = device_status();
  if (st != DBS_OK) return st;
  return status_of(dbs::launch_check(U, L, n, batch, d_flags, static_cast<hipStream_t>(stream)));
}

int dbs_lds_max_n(void) { return dbs::kSmallMaxN; }

int dbs_auto_algo(int64_t n, int64_t batch) {
  (void)batch;
  return n <= dbs::kSmallMaxN ? DBS_ALGO_LDS : DBS_ALGO_BLOCKED;
}

const char *dbs_strerror(int status) {
  switch (status) {
    case DBS_OK: return "success";
    case DBS_EINVAL: return "invalid argument";
    case DBS_EDEVICE: return "no HIP device, or the current device is not gfx950";
    case DBS_ELAUNCH: return "kernel launch failed";
    case DBS_EUNSUPPORTED: return "algorithm does not support this shape";
    default: return "unknown status";
  }
}

int dbs_version(void) { return kVersion; }

}  // extern "C"
