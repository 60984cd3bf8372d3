// valu_rates.hip -- issue rate of the VALU instructions the smoothing kernels
// use, on the current GPU.
//
// Every lane keeps 16 independent accumulators, and each loop iteration
// applies one instruction to each of them.  The instruction is written as
// inline assembly, so the compiler neither folds nor reorders it.  A launch
// puts W waves on every SIMD (256-thread workgroups, W per CU).  The rate is
// in lanes per clock per SIMD, from the wall time of the launch at the
// nominal clock.  "mix" is the per-cell instruction sequence of phase 3 for a
// pair of atoms: 2 adds, 4 subtracts, one 3-input min and two 3-input maxes,
// i.e. 12 min/max/add/sub operations.  The last rows repeat it with the
// wave-uniform row operands in SGPRs, and time an add with an SGPR operand.
//
// Build: hipcc --offload-arch=gfx950 -O3 valu_rates.hip -o valu_rates
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

constexpr int kIter = 16384;
constexpr double kClockHz = 2.4e9;

#define EACH16(S) S(0) S(1) S(2) S(3) S(4) S(5) S(6) S(7) S(8) S(9) S(10) S(11) S(12) S(13) S(14) S(15)
#define ONE(NAME, ASM, ...)                                                       \
  __global__ void NAME(float *out, float c, float d) {                            \
    float x[16];                                                                  \
    for (int i = 0; i < 16; ++i) x[i] = threadIdx.x + i;                          \
    c += threadIdx.x * 1e-7f;                                                     \
    for (int it = 0; it < kIter; ++it) {                                          \
      EACH16(ASM)                                                                 \
    }                                                                             \
    float s = 0;                                                                  \
    for (int i = 0; i < 16; ++i) s += x[i];                                       \
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;                               \
  }
#define A_ADD(i) asm volatile("v_add_f32 %0, %0, %1" : "+v"(x[i]) : "v"(c));
#define A_SUB(i) asm volatile("v_sub_f32 %0, %0, %1" : "+v"(x[i]) : "v"(c));
#define A_MIN(i) asm volatile("v_min_f32 %0, %0, %1" : "+v"(x[i]) : "v"(c));
#define A_MAX3(i) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(c), "v"(d));
#define A_MIN3(i) asm volatile("v_min3_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(c), "v"(d));
#define A_MAXI(i) asm volatile("v_max_i32 %0, %0, %1" : "+v"(x[i]) : "v"(c));
// c is written before the loop only, so the DPP source needs no wait states
#define A_DPP(i) \
  asm volatile("v_add_f32_dpp %0, %1, %0 row_newbcast:" #i " row_mask:0xf bank_mask:0xf" \
               : "+v"(x[i]) : "v"(c));
ONE(k_add, A_ADD)
ONE(k_sub, A_SUB)
ONE(k_min, A_MIN)
ONE(k_max3, A_MAX3)
ONE(k_min3, A_MIN3)
ONE(k_maxi, A_MAXI)
ONE(k_dpp, A_DPP)

// phase-3 sequence on 8 cells (u, l pairs) per iteration
__global__ void k_mix(float *out, float c, float d) {
  float u[8], l[8];
  for (int i = 0; i < 8; ++i) {
    u[i] = threadIdx.x + i;
    l[i] = threadIdx.x - i;
  }
  const float c0 = c + threadIdx.x * 1e-7f, c1 = c0 + 1.0f, d0 = d, d1 = d + 1.0f;
  const float r0 = c * 0.5f, r1 = r0 + 2.0f, q0 = d * 0.5f, q1 = q0 + 3.0f;
  for (int it = 0; it < kIter; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float t0, t1, t2, t3;
      asm volatile(
          "v_add_f32 %2, %6, %8\n\t"
          "v_add_f32 %3, %7, %9\n\t"
          "v_min3_f32 %0, %0, %2, %3\n\t"
          "v_sub_f32 %2, %10, %8\n\t"
          "v_sub_f32 %3, %12, %6\n\t"
          "v_max3_f32 %1, %1, %2, %3\n\t"
          "v_sub_f32 %4, %11, %9\n\t"
          "v_sub_f32 %5, %13, %7\n\t"
          "v_max3_f32 %1, %1, %4, %5"
          : "+v"(u[i]), "+v"(l[i]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
          : "v"(c0), "v"(c1), "v"(r0), "v"(r1), "v"(d0), "v"(d1), "v"(q0), "v"(q1));
    }
  }
  float s = 0;
  for (int i = 0; i < 8; ++i) s += u[i] + l[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same sequence with each cell's row operands (the wave-uniform values)
// in SGPRs, 4 distinct ones per cell, and a plain add with an SGPR operand.
__global__ void k_mix_sgpr(float *out, const float *__restrict__ rowops, float d) {
  float u[8], l[8];
  for (int i = 0; i < 8; ++i) {
    u[i] = threadIdx.x + i;
    l[i] = threadIdx.x - i;
  }
  const float r0 = d * 0.5f + threadIdx.x, r1 = r0 + 2.0f, q0 = d * 0.25f + threadIdx.x,
              q1 = q0 + 3.0f;
  float cs[32];
  for (int i = 0; i < 32; ++i) cs[i] = rowops[i];  // uniform loads: SGPRs
  for (int it = 0; it < kIter; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float t0, t1, t2, t3;
      asm volatile(
          "v_add_f32 %2, %6, %8\n\t"
          "v_add_f32 %3, %7, %9\n\t"
          "v_min3_f32 %0, %0, %2, %3\n\t"
          "v_sub_f32 %2, %10, %8\n\t"
          "v_subrev_f32 %3, %6, %12\n\t"
          "v_max3_f32 %1, %1, %2, %3\n\t"
          "v_sub_f32 %4, %11, %9\n\t"
          "v_subrev_f32 %5, %7, %13\n\t"
          "v_max3_f32 %1, %1, %4, %5"
          : "+v"(u[i]), "+v"(l[i]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
          : "s"(cs[4 * i]), "s"(cs[4 * i + 1]), "v"(r0), "v"(r1), "s"(cs[4 * i + 2]),
            "s"(cs[4 * i + 3]), "v"(q0), "v"(q1));
    }
  }
  float s = 0;
  for (int i = 0; i < 8; ++i) s += u[i] + l[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void k_add_sgpr(float *out, const float *__restrict__ rowops, float d) {
  float x[16], cs[16];
  for (int i = 0; i < 16; ++i) {
    x[i] = threadIdx.x + i;
    cs[i] = rowops[i];
  }
  for (int it = 0; it < kIter; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("v_add_f32 %0, %1, %0" : "+v"(x[i]) : "s"(cs[i]));
  }
  float s = 0;
  for (int i = 0; i < 16; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

int main() {
  hipDeviceProp_t p;
  CHECK(hipGetDeviceProperties(&p, 0));
  const int cus = p.multiProcessorCount;
  std::printf("device %s, %d CUs, rates at %.1f GHz\n\n", p.gcnArchName, cus, kClockHz / 1e9);
  struct K {
    const char *name;
    void (*f)(float *, float, float);
    double instr;  // instructions per lane per launch
    double ops;    // min/max/add/sub operations per lane per launch
  } ks[] = {
      {"v_add_f32", k_add, 16.0 * kIter, 16.0 * kIter},
      {"v_sub_f32", k_sub, 16.0 * kIter, 16.0 * kIter},
      {"v_min_f32", k_min, 16.0 * kIter, 16.0 * kIter},
      {"v_max3_f32", k_max3, 16.0 * kIter, 32.0 * kIter},
      {"v_min3_f32", k_min3, 16.0 * kIter, 32.0 * kIter},
      {"v_max_i32", k_maxi, 16.0 * kIter, 16.0 * kIter},
      {"v_add_f32_dpp row_newbcast", k_dpp, 16.0 * kIter, 16.0 * kIter},
      {"mix (phase 3, per atom pair)", k_mix, 8.0 * 9 * kIter, 8.0 * 12 * kIter},
  };
  const int waves[] = {4, 8};
  const int max_blocks = cus * 8;
  float *out = nullptr;
  CHECK(hipMalloc(&out, sizeof(float) * max_blocks * 256));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::printf("| instruction | waves/SIMD | ms | instr lanes/clk/SIMD | ops lanes/clk/SIMD | ops/s (chip) |\n");
  std::printf("|---|---|---|---|---|---|\n");
  for (const K &k : ks) {
    for (int w : waves) {
      const int blocks = cus * w;  // 4 waves per block, one per SIMD
      hipLaunchKernelGGL(k.f, dim3(blocks), dim3(256), 0, 0, out, 1.0f, 2.0f);  // warm-up
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(k.f, dim3(blocks), dim3(256), 0, 0, out, 1.0f, 2.0f);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      const double lanes = blocks * 256.0, simds = cus * 4.0, t = ms * 1e-3;
      std::printf("| %s | %d | %.3f | %.1f | %.1f | %.2e |\n", k.name, w, ms,
                  lanes * k.instr / simds / t / kClockHz, lanes * k.ops / simds / t / kClockHz,
                  lanes * k.ops / t);
    }
  }
  float *rowops = nullptr;
  CHECK(hipMalloc(&rowops, sizeof(float) * 32));
  CHECK(hipMemset(rowops, 0, sizeof(float) * 32));
  struct KS {
    const char *name;
    void (*f)(float *, const float *, float);
    double instr, ops;
  } kss[] = {
      {"mix, row operands in SGPRs", k_mix_sgpr, 8.0 * 9 * kIter, 8.0 * 12 * kIter},
      {"v_add_f32, SGPR operand", k_add_sgpr, 16.0 * kIter, 16.0 * kIter},
  };
  for (const KS &k : kss) {
    for (int w : waves) {
      const int blocks = cus * w;
      hipLaunchKernelGGL(k.f, dim3(blocks), dim3(256), 0, 0, out, rowops, 2.0f);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(k.f, dim3(blocks), dim3(256), 0, 0, out, rowops, 2.0f);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      const double lanes = blocks * 256.0, simds = cus * 4.0, t = ms * 1e-3;
      std::printf("| %s | %d | %.3f | %.1f | %.1f | %.2e |\n", k.name, w, ms,
                  lanes * k.instr / simds / t / kClockHz, lanes * k.ops / simds / t / kClockHz,
                  lanes * k.ops / t);
    }
  }
  CHECK(hipFree(rowops));
  std::vector<float> h(16);
  CHECK(hipMemcpy(h.data(), out, sizeof(float) * h.size(), hipMemcpyDeviceToHost));
  std::printf("\n(sink %g)\n", h[0]);
  CHECK(hipFree(out));
  return 0;
}
