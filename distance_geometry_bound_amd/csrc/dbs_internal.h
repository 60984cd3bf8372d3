// dbs_internal.h -- private declarations shared by the libdbs translation units.
//
// Every kernel here updates the bound matrices of GPU Gems 2, Ch. 43 "GPU
// Computing for Protein Structure Prediction" (study notes), §2:
//     U[i,j] <- min(U[i,j], U[i,k] + U[k,j])
//     L[i,j] <- max(L[i,j], L[i,k] - U[k,j], L[k,j] - U[i,k])
// for intermediate atoms k in Floyd-Warshall order (§3).
//
// Facts the kernels rely on (all under the preconditions stated in dbs.h):
//  * Row k and column k do not change in round k (U[k,k] = L[k,k] = 0 and
//    L >= 0 make every candidate for them equal to the old value), so a
//    round can run in place instead of on the notes' §4 front/back buffers,
//    cells of a round can run in any order, and the lower update may read U
//    before or after the round's upper update.
//  * Symmetry is preserved exactly (fp add and max are commutative), so
//    U[i,k] = U[k,i]: row k alone supplies both operands of a round.
//  * On the 2^-6 grid every candidate is exact, so blocked schedules and
//    merged rounds give the same bits as the plain round order.  Off the
//    grid (directed rounding below) the per-round and single-workgroup
//    kernels still give the bits of the plain round order; the blocked pass
//    groups the roundings differently and agrees within a rounding bound.
//  * Padding: an out-of-range atom p is given U = +inf and L = 0.  Then
//    every candidate through p is +inf (upper) or -inf (lower), so padded
//    rows, columns and intermediates never change a real cell.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace dbs {

constexpr float kInf = __builtin_inff();

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Directed rounding (a pass over bounds that are not on an exact grid): the
// upper-bound sums are rounded toward +inf and the lower-bound differences
// toward -inf, so that no bound is rounded past the value it stands for.
// Both come from one rounding mode, toward +inf, set for the whole kernel:
// a lower candidate L[i,k] - U[k,j] rounded down equals -(U[k,j] - L[i,k])
// rounded up, and the negation is exact (it folds into the source modifiers
// of the max instruction, so the instruction count does not change).
//
// The MODE register's FP_ROUND field holds the rounding of f32 operations in
// bits [1:0] (0 nearest even, 1 toward +inf, 2 toward -inf, 3 toward zero);
// the f64/f16 bits and the other fields are left alone.  Every wave starts
// with the mode of its kernel descriptor (nearest even), so the change ends
// with the kernel.
__device__ __forceinline__ void round_f32_toward_pos_inf() {
  constexpr int kHwRegMode = 1, kOffset = 0, kSize = 2;
  __builtin_amdgcn_s_setreg(kHwRegMode | (kOffset << 6) | ((kSize - 1) << 11), 1);
}

template <bool RU>
__device__ __forceinline__ void rounding_prologue() {
  if (RU) round_f32_toward_pos_inf();
}

// A lower bound as stored.  With directed rounding a zero candidate comes out
// as -(x - x) = -0; adding +0 (exact, and +0 for -0 when rounding up) keeps
// the stored bits those of the plain definition.
template <bool RU>
__device__ __forceinline__ float lower_out(float l) {
  return RU ? l + 0.0f : l;
}

// The smaller of two upper bounds.  Upper bounds are never negative and never
// NaN (+0, positive values and +inf, under either rounding), and on those the
// IEEE order is the unsigned order of the bit patterns, so an integer minimum
// gives the bits fminf gives.  A loop-carried fminf pays one extra VALU
// instruction to quiet a possible signalling NaN in its operand; the integer
// minimum needs none.
__device__ __forceinline__ float upper_min(float a, float b) {
  return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
}

// One intermediate atom applied to one cell:
//   (u, l) <- (min(u, cu + ru), max(l, cl - ru, rl - cu))
// where cu/cl = U/L[i,k] and ru/rl = U/L[k,j].
template <bool RU = false>
__device__ __forceinline__ void relax1(float &u, float &l, float cu, float cl, float ru,
                                       float rl) {
  u = upper_min(u, cu + ru);
  if (RU)
    l = fmaxf(fmaxf(l, -(ru - cl)), -(cu - rl));
  else
    l = fmaxf(fmaxf(l, cl - ru), rl - cu);
}

// Two intermediate atoms k0, k1 applied to one cell (folds into 3-input
// min/max instructions).  Same result as relax1(k0) then relax1(k1).
template <bool RU = false>
__device__ __forceinline__ void relax2(float &u, float &l, float cu0, float cl0, float ru0,
                                       float rl0, float cu1, float cl1, float ru1, float rl1) {
  u = fminf(fminf(u, cu0 + ru0), cu1 + ru1);
  if (RU) {
    l = fmaxf(fmaxf(l, -(ru0 - cl0)), -(cu0 - rl0));
    l = fmaxf(fmaxf(l, -(ru1 - cl1)), -(cu1 - rl1));
  } else {
    l = fmaxf(fmaxf(l, cl0 - ru0), rl0 - cu0);
    l = fmaxf(fmaxf(l, cl1 - ru1), rl1 - cu1);
  }
}

// Variants of a pass: storage layout and rounding.
enum : unsigned {
  kPacked = 1u,    // one buffer P: U above the diagonal, L below
  kDirected = 2u,  // sums rounded up, differences rounded down
};

// Largest molecule the single-workgroup path holds (4x4 cells per thread,
// upper-triangle tiles only, at most 1024 threads).
constexpr int kSmallMaxN = 176;

// Where the bounds of cell (i, j) live, as element offsets from the block's
// base (row stride ld).  Dense: U and L are two arrays with (i, j) at the
// same offset.  Packed (one array P, the notes' §6 triangle storage):
// U(i,j) = P[min(i,j)][max(i,j)], L(i,j) = P[max(i,j)][min(i,j)].
template <bool PK>
struct Cell {
  __device__ static __forceinline__ int64_t u(int64_t i, int64_t j, int64_t ld) {
    return PK ? (i < j ? i * ld + j : j * ld + i) : i * ld + j;
  }
  __device__ static __forceinline__ int64_t l(int64_t i, int64_t j, int64_t ld) {
    return PK ? (i > j ? i * ld + j : j * ld + i) : i * ld + j;
  }
};

// Optional launch timing.  When a launcher is given a Prof, every kernel it
// enqueues is bracketed by a pair of HIP events on the launch stream, tagged
// with the kernel kind (the DBS_PROF_* numbering of dbs.h).
struct Prof {
  struct Mark {
    int kind;
    hipEvent_t start, stop;
  };
  std::vector<Mark> marks;
  Prof() = default;
  Prof(const Prof &) = delete;
  Prof &operator=(const Prof &) = delete;
  ~Prof() {
    for (auto &m : marks) {
      (void)hipEventDestroy(m.start);
      (void)hipEventDestroy(m.stop);
    }
  }
};

enum ProfKind {
  kProfRound = 0,
  kProfSmall = 1,
  kProfPanel = 2,
  kProfTiles = 3,
  kProfMirror = 4,
  kProfStrip = 5,
  kProfFill = 6,
  kProfScatter = 7
};

template <typename T>
struct ident {
  using type = T;
};

// Launch `kernel` with by-value arguments (hipLaunchKernel returns the launch
// status directly), optionally timed.
template <typename... KArgs>
hipError_t launch(Prof *prof, int kind, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                  hipStream_t s, typename ident<KArgs>::type... args) {
  void *ptrs[] = {(void *)&args...};
  if (!prof) return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, s);
  Prof::Mark m{kind, nullptr, nullptr};
  hipError_t e = hipEventCreate(&m.start);
  if (e != hipSuccess) return e;
  e = hipEventCreate(&m.stop);
  if (e != hipSuccess) {
    (void)hipEventDestroy(m.start);
    return e;
  }
  prof->marks.push_back(m);
  if ((e = hipEventRecord(m.start, s)) != hipSuccess) return e;
  if ((e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, s)) !=
      hipSuccess)
    return e;
  return hipEventRecord(m.stop, s);
}

// Launchers (host side).  They enqueue on `s` and return the first launch
// error, if any.  `flags` (kPacked, kDirected) selects the variant; with
// kPacked, U == L == P in the one-buffer layout.
hipError_t launch_round(float *U, float *L, int64_t n, int64_t batch, int64_t k, hipStream_t s,
                        Prof *prof = nullptr, unsigned flags = 0);
// rounds k_lo..k_hi-1 of a whole small molecule in one workgroup
hipError_t launch_small(float *U, float *L, int64_t n, int64_t batch, int k_lo, int k_hi,
                        hipStream_t s, Prof *prof = nullptr, unsigned flags = 0);
// Schedule of a blocked pass chosen by the caller: a forced look-ahead depth
// (0..2) and k-blocks per step (1..kMaxStepBlocks), or -1 for the automatic
// choice.  Every schedule gives the same results.
struct Sched {
  int lookahead = -1;
  int step_blocks = -1;
  int lead = -1;
  bool packed = false;  // the layout (the automatic lead schedule differs)
};
// k-blocks K0..K1-1 of the blocked pass (rounds 64*K0 .. min(64*K1, n)-1)
// `infeasible` (may be null): per-molecule words for the early test of the
// infeasibility option (DBS_INFEASIBLE_EARLY, where phase 1 closes a
// diagonal tile).
hipError_t launch_blocked(float *U, float *L, int64_t n, int64_t batch, int64_t K0, int64_t K1,
                          hipStream_t s, Prof *prof = nullptr, unsigned flags = 0,
                          const Sched &sched = Sched(), uint32_t *infeasible = nullptr);
// The infeasibility option's test of a pass's output: words[b] |=
// DBS_INFEASIBLE_END where molecule b has a cell with L > U (dense U, L, or
// the packed buffer P).
hipError_t launch_infeasible(const float *U, const float *L, int64_t n, int64_t batch,
                             uint32_t *words, hipStream_t s);
hipError_t launch_infeasible_packed(const float *P, int64_t n, int64_t batch, uint32_t *words,
                                    hipStream_t s);
constexpr int kBlockRounds = 64;
// Look-ahead depth of the blocked pass: steps it updates ahead on its second
// stream (0, 1 or 2; at 2 a step is several k-blocks).
int lookahead_bands(int64_t n, int64_t batch, const Sched &sched = Sched());
// k-blocks per step of the blocked pass (1 .. kMaxStepBlocks).
constexpr int kMaxStepBlocks = 4;
int step_blocks(int64_t n, int64_t batch, const Sched &sched = Sched());
// Whether the blocked pass takes the lead schedule (one stream, one-block
// steps: phase 1 of the next k-block beside phase 3, phase 2 as a product).
bool lead_schedule(int64_t n, int64_t batch, const Sched &sched = Sched());
hipError_t launch_restraints(float *U, float *L, int64_t n, int64_t batch, float unknown_L,
                             float unknown_U, const int32_t *mol, const int32_t *ia,
                             const int32_t *ja, const float *lo, const float *hi, int64_t count,
                             uint32_t *status, hipStream_t s, Prof *prof = nullptr);
hipError_t launch_round_packed(float *P, int64_t n, int64_t batch, int64_t k, hipStream_t s,
                               Prof *prof = nullptr, unsigned flags = kPacked);
hipError_t launch_pack(const float *U, const float *L, float *P, int64_t n, int64_t batch,
                       hipStream_t s);
hipError_t launch_unpack(const float *P, float *U, float *L, int64_t n, int64_t batch,
                         hipStream_t s);
hipError_t launch_tightened(const float *U0, const float *L0, const float *U1, const float *L1,
                            int64_t n, int64_t batch, uint8_t *mask, hipStream_t s);
hipError_t launch_check(const float *U, const float *L, int64_t n, int64_t batch,
                        uint32_t *flags, hipStream_t s);
hipError_t launch_check_packed(const float *P, int64_t n, int64_t batch, uint32_t *flags,
                               hipStream_t s);

// Single-workgroup Floyd-Warshall over an m x m symmetric block (m <= kSmallMaxN)
// at element offset `off` of each molecule (row stride `ld`, molecule stride
// `mstride`); grid = molecules.  Used for whole small molecules and for the
// diagonal tile of the blocked pass.
hipError_t launch_small_block(float *U, float *L, int64_t ld, int64_t mstride, int64_t off,
                              int m, int k_lo, int k_hi, int64_t batch, hipStream_t s,
                              Prof *prof = nullptr, unsigned flags = 0);

// Tile pair p of the upper triangle, numbered column-major (p = J(J+1)/2 + I,
// I <= J): returns J.
__device__ __forceinline__ int64_t tri_col(int64_t p) {
  int64_t J = (int64_t)((sqrt(8.0 * (double)p + 1.0) - 1.0) * 0.5);
  while (J * (J + 1) / 2 > p) --J;
  while ((J + 1) * (J + 2) / 2 <= p) ++J;
  return J;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Grid dimensions above these are folded into in-kernel loops.
constexpr int64_t kMaxGridYZ = 65535;
constexpr int64_t kMaxGridX = 0x7fffffff;

}  // namespace dbs
