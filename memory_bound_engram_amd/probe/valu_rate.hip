// valu_rate.hip -- issue cost of the vector-ALU opcodes the gate and GateConv
// kernels lean on, relative to a plain fp32 FMA, on this GPU.
//
// Measurement program, not part of libengram.  Each kernel runs 8 independent
// dependency chains per thread (enough waves and chains that the issue rate,
// not the latency, decides the time) with no memory traffic in the loop; one
// store per thread at the end keeps the chains alive.  Opcodes that need a
// companion to stay finite run paired with one full-rate operation:
//   fma        a = fma(a, c0, c1)                        1 x v_fma
//   exp2+mul   a = exp2(a) * c                           v_exp_f32 + v_mul
//   add+rcp    a = rcp(a + 1)                            v_add + v_rcp_f32
//   dot2+mul   a = dot2_bf16(x, y, a * c)                v_mul + v_dot2c_f32_bf16
// The cost of the paired opcode in FMA units is (t_pair - t_fma) / t_fma,
// taking the companion at an FMA's cost.  Median of 5 launches each.
//
//   valu_rate
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <vector>

#define CHECK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(1);                                                                            \
    }                                                                                     \
  } while (0)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

enum Op { kFma = 0, kExp2Mul = 1, kAddRcp = 2, kDot2Mul = 3 };
static const char* kOpName[] = {"fma", "exp2+mul", "add+rcp", "dot2+mul"};
constexpr int kChains = 8;
constexpr int kThreads = 256;

template <int OP>
__global__ void __launch_bounds__(kThreads) chains(float* out, int iters, float seed) {
  float a[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) a[i] = seed * (float)(threadIdx.x + 1) * (float)(i + 1) * 1e-6f;
  const uint32_t x = 0x3f803f80u, y = 0x3f003f00u;  // bf16 pairs (1, 1) and (0.5, 0.5)
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) {
      if (OP == kFma) a[i] = fmaf(a[i], 0.999f, 1e-7f);
      if (OP == kExp2Mul) a[i] = __builtin_amdgcn_exp2f(a[i]) * 1e-3f;
      if (OP == kAddRcp) a[i] = __builtin_amdgcn_rcpf(a[i] + 1.0f);
      if (OP == kDot2Mul)
        a[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y),
                                               a[i] * 0.5f, false);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += a[i];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;  // one store per thread, inside the grid's buffer
}

typedef void (*Kernel)(float*, int, float);

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int grid = 32 * prop.multiProcessorCount, iters = 4096;
  float* out;
  CHECK(hipMalloc(&out, sizeof(float) * (size_t)grid * kThreads));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const Kernel kernels[] = {chains<kFma>, chains<kExp2Mul>, chains<kAddRcp>, chains<kDot2Mul>};
  const double groups = (double)grid * (kThreads / 64) * iters;  // chain steps of 8 per wave
  printf("device %s, %d CUs; %d workgroups x %d threads, %d iterations of %d chains\n", prop.name,
         prop.multiProcessorCount, grid, kThreads, iters, kChains);
  printf("%-9s %10s %22s %18s\n", "op", "median_ms", "ps_per_wave_op_per_CU", "paired_op_in_fma");
  double t_fma = 0.0;
  for (int op = 0; op < 4; ++op) {
    std::vector<float> ms;
    for (int rep = 0; rep < 6; ++rep) {
      CHECK(hipEventRecord(e0, 0));
      hipLaunchKernelGGL(kernels[op], dim3(grid), dim3(kThreads), 0, 0, out, iters, 1.0f);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1, 0));
      CHECK(hipEventSynchronize(e1));
      float t;
      CHECK(hipEventElapsedTime(&t, e0, e1));
      if (rep > 0) ms.push_back(t);
    }
    std::sort(ms.begin(), ms.end());
    const double med = ms[ms.size() / 2];
    // time per wave-level chain step of one opcode (or pair), per CU
    const double ps = med * 1e9 / (groups * kChains / prop.multiProcessorCount);
    if (op == kFma) t_fma = med;
    const double ratio = op == kFma ? 1.0 : (med - t_fma) / t_fma;
    printf("%-9s %10.3f %22.1f %18.2f\n", kOpName[op], med, ps, ratio);
    fflush(stdout);
  }
  CHECK(hipFree(out));
  return 0;
}
