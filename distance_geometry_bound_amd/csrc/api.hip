// api.hip -- the extern "C" entry points declared in include/dbs.h:
// argument validation, device check, algorithm choice, launch sequencing.
#include <math.h>
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

// The largest n + 1 accepted.  No such matrix fits in device memory (2^52
// floats); the blocked kernels address a 64-row band with 32-bit offsets.
constexpr int64_t kLimitN = (int64_t)1 << 26;

// Size checks of one [batch][n][n] float buffer; 0 when fine.
int check_buffer(const void *p, int64_t n, int64_t batch, uint64_t *bytes) {
  if (!p || n < 1 || batch < 1 || n >= kLimitN) return DBS_EINVAL;
  const int64_t nn = n * n;
  if (batch > INT64_MAX / 4 / nn) return DBS_EINVAL;
  *bytes = (uint64_t)(nn * batch) * 4u;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (a + *bytes < a || (a & 3u)) return DBS_EINVAL;
  return DBS_OK;
}

bool overlap(const void *a, const void *b, uint64_t bytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bytes && y < x + bytes;
}

// Host-side argument checks shared by every entry point.
int validate(const void *U, const void *L, int64_t n, int64_t batch) {
  if (!U || !L || n < 1 || batch < 1) return DBS_EINVAL;
  if (n >= kLimitN) return DBS_EINVAL;
  const int64_t nn = n * n;  // < 2^52
  if (batch > INT64_MAX / 4 / nn) return DBS_EINVAL;
  const uint64_t bytes = (uint64_t)(nn * batch) * 4u;
  const uintptr_t u = reinterpret_cast<uintptr_t>(U), l = reinterpret_cast<uintptr_t>(L);
  if (u + bytes < u || l + bytes < l) return DBS_EINVAL;  // address wrap
  if (u < l + bytes && l < u + bytes) return DBS_EINVAL;  // overlap
  if ((u | l) & 3u) return DBS_EINVAL;                     // float alignment
  return DBS_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? DBS_OK : DBS_ELAUNCH; }

// Options of a pass with the defaults filled in; false for an invalid value.
bool read_options(const dbs_options *o, dbs_options *out) {
  dbs_options_init(out);
  if (!o) return true;
  if (o->algo < DBS_ALGO_AUTO || o->algo > DBS_ALGO_BLOCKED) return false;
  if (o->directed != 0 && o->directed != 1) return false;
  if (o->lookahead < DBS_AUTO || o->lookahead > 2) return false;
  if (o->step_blocks != DBS_AUTO && (o->step_blocks < 1 || o->step_blocks > dbs::kMaxStepBlocks))
    return false;
  if (o->lead < DBS_AUTO || o->lead > 1) return false;
  if (reinterpret_cast<uintptr_t>(o->infeasible) % alignof(uint32_t) != 0) return false;
  *out = *o;
  return true;
}

dbs::Sched sched_of(const dbs_options &o) {
  dbs::Sched sc;
  sc.lookahead = o.lookahead;
  sc.step_blocks = o.step_blocks;
  sc.lead = o.lead;
  return sc;
}

// The algorithm DBS_ALGO_AUTO takes: the single workgroup per molecule where
// the pass fits it, except for a round-to-nearest pass in the dense layout
// from n = 128 with at most kAutoBlockedBatch molecules, where the blocked
// pass is faster; else the blocked pass on k-block boundaries, else one
// launch per round.  A directed pass keeps the single workgroup where it
// fits: it applies the roundings in the plain round order (the blocked pass
// groups them differently, within the bound of the directed rounding).  (Measured
// dense pass ms, single workgroup / blocked: n120 0.076 / 0.078, n128 0.088
// / 0.080, n176 0.137 / 0.114; 16 molecules of n128 0.089 / 0.085, of n176
// 0.139 / 0.119; 64 of n128 0.088 / 0.092.  The packed single workgroup is
// faster than the packed blocked pass at every n up to 176 and batch: n128
// 0.079 / 0.089, n176 0.127 / 0.128.)
constexpr int64_t kAutoBlockedMinN = 128, kAutoBlockedBatch = 16;
int auto_algo(int64_t n, int64_t batch, bool packed, bool directed, bool aligned) {
  if (n <= dbs::kSmallMaxN && (packed || directed || n < kAutoBlockedMinN ||
                               batch > kAutoBlockedBatch || !aligned))
    return DBS_ALGO_LDS;
  return aligned ? DBS_ALGO_BLOCKED : DBS_ALGO_PERK;
}

// The kernels of a pass (arguments already checked).
int pass_dispatch(float *U, float *L, bool packed, int64_t n, int64_t batch, int64_t k_begin,
                  int64_t k_end, hipStream_t s, dbs::Prof *prof, const dbs_options &o,
                  int algo) {
  if (k_begin == k_end || n == 1) return DBS_OK;
  const int64_t B = dbs::kBlockRounds;
  const unsigned flags = (packed ? dbs::kPacked : 0u) | (o.directed ? dbs::kDirected : 0u);
  switch (algo) {
    case DBS_ALGO_PERK: {
      hipError_t e = hipSuccess;
      for (int64_t k = k_begin; k < k_end && e == hipSuccess; ++k)
        e = packed ? dbs::launch_round_packed(U, n, batch, k, s, prof, flags)
                   : dbs::launch_round(U, L, n, batch, k, s, prof, flags);
      return status_of(e);
    }
    case DBS_ALGO_LDS:
      return status_of(
          dbs::launch_small(U, L, n, batch, (int)k_begin, (int)k_end, s, prof, flags));
    default:
      return status_of(dbs::launch_blocked(U, L, n, batch, k_begin / B, dbs::ceil_div(k_end, B),
                                           s, prof, flags, sched_of(o), o.infeasible));
  }
}

// Rounds k_begin..k_end-1 of a pass on U, L (dense) or on P = U (packed,
// L ignored), with the given options (AUTO: auto_algo).
int pass_impl(float *U, float *L, bool packed, int64_t n, int64_t batch, int64_t k_begin,
              int64_t k_end, void *stream, const dbs_options *opts, dbs::Prof *prof) {
  if (packed) {
    uint64_t bytes = 0;
    if (check_buffer(U, n, batch, &bytes) != DBS_OK) return DBS_EINVAL;
    L = U;
  } else {
    const int st = validate(U, L, n, batch);
    if (st != DBS_OK) return st;
  }
  dbs_options o;
  if (!read_options(opts, &o)) return DBS_EINVAL;
  if (k_begin < 0 || k_end > n || k_begin > k_end) return DBS_EINVAL;
  const int64_t B = dbs::kBlockRounds;
  const bool aligned = k_begin % B == 0 && (k_end % B == 0 || k_end == n);
  int algo = o.algo;
  if (algo == DBS_ALGO_AUTO) algo = auto_algo(n, batch, packed, o.directed != 0, aligned);
  if (algo == DBS_ALGO_LDS && n > dbs::kSmallMaxN) return DBS_EUNSUPPORTED;
  if (algo == DBS_ALGO_BLOCKED && !aligned) return DBS_EUNSUPPORTED;
  const int st = device_status();
  if (st != DBS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ps = pass_dispatch(U, L, packed, n, batch, k_begin, k_end, s, prof, o, algo);
  if (ps != DBS_OK || !o.infeasible) return ps;
  // the infeasibility option's test of the output (DBS_INFEASIBLE_END)
  return status_of(packed ? dbs::launch_infeasible_packed(U, n, batch, o.infeasible, s)
                          : dbs::launch_infeasible(U, L, n, batch, o.infeasible, s));
}

int pass_with(float *U, float *L, bool packed, int64_t n, int64_t batch, int64_t k_begin,
              int64_t k_end, void *stream, int algo, int directed) {
  dbs_options o;
  dbs_options_init(&o);
  o.algo = algo;
  o.directed = directed;
  return pass_impl(U, L, packed, n, batch, k_begin, k_end, stream, &o, nullptr);
}

}  // namespace

extern "C" {

void dbs_options_init(dbs_options *opts) {
  if (!opts) return;
  opts->algo = DBS_ALGO_AUTO;
  opts->directed = 0;
  opts->lookahead = DBS_AUTO;
  opts->step_blocks = DBS_AUTO;
  opts->lead = DBS_AUTO;
  opts->infeasible = nullptr;
}

int dbs_smooth_opts(float *U, float *L, int64_t n, int64_t batch, int64_t k_begin,
                    int64_t k_end, void *stream, const dbs_options *opts) {
  return pass_impl(U, L, false, n, batch, k_begin, k_end, stream, opts, nullptr);
}

int dbs_smooth_packed_opts(float *P, int64_t n, int64_t batch, int64_t k_begin, int64_t k_end,
                           void *stream, const dbs_options *opts) {
  return pass_impl(P, nullptr, true, n, batch, k_begin, k_end, stream, opts, nullptr);
}

int dbs_smooth(float *U, float *L, int64_t n, int64_t batch, void *stream) {
  return pass_with(U, L, false, n, batch, 0, n, stream, DBS_ALGO_AUTO, 0);
}

int dbs_smooth_algo(float *U, float *L, int64_t n, int64_t batch, void *stream, int algo) {
  return pass_with(U, L, false, n, batch, 0, n, stream, algo, 0);
}

int dbs_smooth_profiled(float *U, float *L, int64_t n, int64_t batch, void *stream,
                        const dbs_options *opts, int64_t *counts, double *ms) {
  if (!counts || !ms) return DBS_EINVAL;
  for (int i = 0; i < DBS_PROF_KINDS; ++i) {
    counts[i] = 0;
    ms[i] = 0.0;
  }
  dbs::Prof prof;
  int st = pass_impl(U, L, false, n, batch, 0, n, stream, opts, &prof);
  if (st != DBS_OK) return st;
  // the launches may be spread over two streams: wait for every stop event
  for (const auto &m : prof.marks)
    if (hipEventSynchronize(m.stop) != hipSuccess) return DBS_ELAUNCH;
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

int dbs_round(float *U, float *L, int64_t n, int64_t batch, int64_t k, void *stream) {
  if (k < 0 || k >= n) return DBS_EINVAL;
  return dbs_rounds(U, L, n, batch, k, k + 1, stream);
}

int dbs_check(const float *U, const float *L, int64_t n, int64_t batch, void *stream,
              uint32_t *d_flags) {
  int st = validate(U, L, n, batch);
  if (st != DBS_OK) return st;
  if (!d_flags) return DBS_EINVAL;
  st = device_status();
  if (st != DBS_OK) return st;
  return status_of(dbs::launch_check(U, L, n, batch, d_flags, static_cast<hipStream_t>(stream)));
}

int dbs_smooth_range(float *U, float *L, int64_t n, int64_t batch, int64_t k_begin,
                     int64_t k_end, void *stream, int algo) {
  return pass_with(U, L, false, n, batch, k_begin, k_end, stream, algo, 0);
}

int dbs_smooth_directed_range(float *U, float *L, int64_t n, int64_t batch, int64_t k_begin,
                              int64_t k_end, void *stream, int algo) {
  return pass_with(U, L, false, n, batch, k_begin, k_end, stream, algo, 1);
}

int dbs_smooth_directed(float *U, float *L, int64_t n, int64_t batch, void *stream) {
  return pass_with(U, L, false, n, batch, 0, n, stream, DBS_ALGO_AUTO, 1);
}

int dbs_block_rounds(void) { return dbs::kBlockRounds; }

int dbs_tightened(const float *U0, const float *L0, const float *U1, const float *L1,
                  int64_t n, int64_t batch, uint8_t *mask, void *stream) {
  // the four inputs may alias one another; none may overlap the mask
  if (!U0 || !L0 || !U1 || !L1 || !mask || n < 1 || batch < 1 || n >= kLimitN)
    return DBS_EINVAL;
  if (batch > INT64_MAX / 4 / (n * n)) return DBS_EINVAL;
  const uint64_t fbytes = (uint64_t)(n * n * batch) * 4u, mbytes = fbytes / 4u;
  const uintptr_t m = reinterpret_cast<uintptr_t>(mask);
  for (const float *p : {U0, L0, U1, L1}) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if ((a & 3u) || (a < m + mbytes && m < a + fbytes)) return DBS_EINVAL;
  }
  const int st = device_status();
  if (st != DBS_OK) return st;
  return status_of(
      dbs::launch_tightened(U0, L0, U1, L1, n, batch, mask, static_cast<hipStream_t>(stream)));
}

int dbs_bounds_from_restraints(float *U, float *L, int64_t n, int64_t batch, float unknown_L,
                               float unknown_U, const int32_t *mol, const int32_t *ia,
                               const int32_t *ja, const float *lo, const float *hi,
                               int64_t count, uint32_t *d_status, void *stream) {
  int st = validate(U, L, n, batch);
  if (st != DBS_OK) return st;
  if (count < 0) return DBS_EINVAL;
  if (count > 0 && (!ia || !ja || !lo || !hi || (batch > 1 && !mol))) return DBS_EINVAL;
  if (!(unknown_L >= 0.0f && unknown_L <= unknown_U && unknown_U < 131072.0f)) return DBS_EINVAL;
  st = device_status();
  if (st != DBS_OK) return st;
  // placeholders, rounded outward on the host (exact in float: see the kernel)
  const float uL = floorf(unknown_L * 64.0f) / 64.0f, uU = ceilf(unknown_U * 64.0f) / 64.0f;
  if (uU >= 131072.0f) return DBS_EINVAL;
  return status_of(dbs::launch_restraints(U, L, n, batch, uL, uU, mol, ia, ja, lo, hi, count,
                                          d_status, static_cast<hipStream_t>(stream)));
}

int dbs_pack(const float *U, const float *L, float *P, int64_t n, int64_t batch, void *stream) {
  int st = validate(U, L, n, batch);
  if (st != DBS_OK) return st;
  uint64_t bytes = 0;
  if (check_buffer(P, n, batch, &bytes) != DBS_OK || overlap(P, U, bytes) || overlap(P, L, bytes))
    return DBS_EINVAL;
  st = device_status();
  if (st != DBS_OK) return st;
  return status_of(dbs::launch_pack(U, L, P, n, batch, static_cast<hipStream_t>(stream)));
}

int dbs_unpack(const float *P, float *U, float *L, int64_t n, int64_t batch, void *stream) {
  int st = validate(U, L, n, batch);
  if (st != DBS_OK) return st;
  uint64_t bytes = 0;
  if (check_buffer(P, n, batch, &bytes) != DBS_OK || overlap(P, U, bytes) || overlap(P, L, bytes))
    return DBS_EINVAL;
  st = device_status();
  if (st != DBS_OK) return st;
  return status_of(dbs::launch_unpack(P, U, L, n, batch, static_cast<hipStream_t>(stream)));
}

int dbs_smooth_packed_range(float *P, int64_t n, int64_t batch, int64_t k_begin, int64_t k_end,
                            void *stream) {
  return pass_with(P, nullptr, true, n, batch, k_begin, k_end, stream, DBS_ALGO_AUTO, 0);
}

int dbs_smooth_packed_directed_range(float *P, int64_t n, int64_t batch, int64_t k_begin,
                                     int64_t k_end, void *stream) {
  return pass_with(P, nullptr, true, n, batch, k_begin, k_end, stream, DBS_ALGO_AUTO, 1);
}

int dbs_check_packed(const float *P, int64_t n, int64_t batch, void *stream, uint32_t *d_flags) {
  uint64_t bytes = 0;
  if (check_buffer(P, n, batch, &bytes) != DBS_OK || !d_flags) return DBS_EINVAL;
  const int st = device_status();
  if (st != DBS_OK) return st;
  return status_of(dbs::launch_check_packed(P, n, batch, d_flags, static_cast<hipStream_t>(stream)));
}

int dbs_smooth_packed(float *P, int64_t n, int64_t batch, void *stream) {
  return dbs_smooth_packed_range(P, n, batch, 0, n, stream);
}

int dbs_lds_max_n(void) { return dbs::kSmallMaxN; }

namespace {
int schedule_query(int64_t n, int64_t batch, const dbs_options *opts, bool packed,
                   int32_t *lookahead, int32_t *step_blocks, int32_t *lead) {
  dbs_options o;
  if (n < 1 || batch < 1 || !read_options(opts, &o)) return DBS_EINVAL;
  dbs::Sched sc = sched_of(o);
  sc.packed = packed;
  if (lookahead) *lookahead = dbs::lookahead_bands(n, batch, sc);
  if (step_blocks) *step_blocks = dbs::step_blocks(n, batch, sc);
  if (lead) *lead = dbs::lead_schedule(n, batch, sc) ? 1 : 0;
  return DBS_OK;
}
}  // namespace

int dbs_schedule(int64_t n, int64_t batch, const dbs_options *opts, int32_t *lookahead,
                 int32_t *step_blocks, int32_t *lead) {
  return schedule_query(n, batch, opts, false, lookahead, step_blocks, lead);
}

int dbs_schedule_packed(int64_t n, int64_t batch, const dbs_options *opts, int32_t *lookahead,
                        int32_t *step_blocks, int32_t *lead) {
  return schedule_query(n, batch, opts, true, lookahead, step_blocks, lead);
}

int dbs_lookahead_bands(int64_t n, int64_t batch) {
  if (n < 1 || batch < 1) return DBS_EINVAL;
  return dbs::lookahead_bands(n, batch);
}

int dbs_step_blocks(int64_t n, int64_t batch) {
  if (n < 1 || batch < 1) return DBS_EINVAL;
  return dbs::step_blocks(n, batch);
}

int dbs_auto_algo(int64_t n, int64_t batch) { return auto_algo(n, batch, false, false, true); }

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
