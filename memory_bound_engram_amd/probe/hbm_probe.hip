// hbm_probe.hip -- streaming ceilings of MI355X HBM for the gate's traffic.
//
// Measurement program, not part of libengram: it moves the bytes of the
// gate's tensors with no arithmetic, so that the kernels' achieved bandwidth
// can be set against what a plain stream of the same shape reaches on this
// chip.  Tensors are token-major like the gate's: X-like rows of 40,960 B
// (2,560 16-byte vectors) and KV-like rows of 51,200 B (3,200 vectors), one
// separate buffer per tensor.  A workgroup handles one token at a time: it
// loads that token's row of every input tensor (non-temporal 16-byte loads,
// all issued before any store), then stores its row of every output tensor
// (non-temporal 16-byte stores of values that depend on the loads, so no
// load can be dropped).  Shapes:
//   read   1 input  (X)                         -> 0 outputs      100:0
//   write  0 inputs                             -> 1 output (X)   0:100
//   copy   1 input  (X)                         -> 1 output (X)   50:50
//   fwd    2 inputs (X, KV)                     -> 1 output (X)   69:31, the forward's mix
//   bwd    3 inputs (X, KV, G)                  -> 2 outputs (X, KV)  59:41, the backward's mix
//   gcfwd  3 inputs of 10,240-byte rows          -> 2 outputs      60:40, GateConv's forward
//   gcbwd  5 inputs of 10,240-byte rows          -> 3 outputs      62.5:37.5, GateConv's backward
// Token dealing: "lockstep" gives workgroup w the tokens w, w + grid, ... (the
// workgroups walk the tensors together); "chunked" gives it a contiguous run
// of tokens; "bands8" cuts the tensors into 8 bands walked in lockstep side
// by side.  The next token's loads are issued before the current token's
// stores.  Every shape is measured on five layouts of its buffers (see
// place()), 512-thread workgroups, grids of 256 and 1024.  Each case runs 3
// untimed and 10 timed launches (HIP events on one stream); the line reports
// the median and the best, as TB/s of the bytes the case moves.
//
//   hbm_probe [shape ...]       (default: every shape)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <vector>

#include "stream_kernels.h"

#define CHECK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(1);                                                                            \
    }                                                                                     \
  } while (0)

__global__ void fill_kernel(u32x4* p, int64_t n, uint32_t seed) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t c = (uint32_t)i * 2246822519u + seed;
    p[i] = u32x4{c, c ^ 0x5bd1e995u, c + 7u, c * 3u};
  }
}

static const char* kDealName[] = {"lockstep", "chunked", "bands8"};

// Where the tensors live.  The same kernels stream at rates that differ by
// up to ~17% between processes, depending on the physical placement of the
// buffers; each layout below is measured in this one process.
//   0 separate  one allocation per tensor, inputs then outputs
//   1 reversed  one allocation per tensor, outputs then inputs
//   2 spaced    one allocation per tensor with a (1 GiB + k * 2 MiB) spacer allocation before tensor k
//   3 pooled    one allocation, tensors back to back
//   4 staggered one allocation, tensor k starting k * (4 MiB + 64 KiB) past the previous one's end
static const char* kLayoutName[] = {"separate", "reversed", "spaced", "pooled", "staggered"};
constexpr int kLayouts = 5;

struct Placement {
  std::vector<void*> allocs;
  std::vector<char*> tensor;  // inputs, then outputs
};

static Placement place(int layout, const std::vector<int64_t>& bytes) {
  Placement p;
  const int n = (int)bytes.size();
  p.tensor.assign(n, nullptr);
  if (layout <= 2) {
    for (int i = 0; i < n; ++i) {
      const int k = layout == 1 ? n - 1 - i : i;
      if (layout == 2) {
        void* spacer;
        CHECK(hipMalloc(&spacer, (1ll << 30) + (int64_t)(k + 1) * (2ll << 20)));
        p.allocs.push_back(spacer);
      }
      void* q;
      CHECK(hipMalloc(&q, bytes[k]));
      p.allocs.push_back(q);
      p.tensor[k] = (char*)q;
    }
    return p;
  }
  const int64_t gap = layout == 4 ? (4ll << 20) + (64ll << 10) : 0;
  int64_t total = 0;
  for (int k = 0; k < n; ++k) total += bytes[k] + k * gap + 4096;
  void* q;
  CHECK(hipMalloc(&q, total));
  p.allocs.push_back(q);
  char* c = (char*)q;
  for (int k = 0; k < n; ++k) {
    c += k * gap;
    p.tensor[k] = c;
    c += (bytes[k] + 4095) / 4096 * 4096;
  }
  return p;
}

int main(int argc, char** argv) {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  printf("device %s, %d CUs\n", prop.name, prop.multiProcessorCount);
  printf("%-6s %-9s %5s %4s %-8s %-4s %8s %12s %10s %10s %8s %8s\n", "shape", "layout", "grid", "thr", "dealing",
         "pipe", "tokens", "bytes", "median_us", "best_us", "TB/s", "best");
  const int64_t budget = 4ll << 30;  // ~4 GiB of tensors per shape: far beyond the 256 MB cache
  for (const Shape& sh : kShapes) {
    bool wanted = argc <= 1;
    for (int a = 1; a < argc; ++a) wanted |= strcmp(argv[a], sh.name) == 0;
    if (!wanted) continue;
    int64_t row_bytes = 0;
    for (int k = 0; k < sh.nin; ++k) row_bytes += 16ll * sh.in_vecs[k];
    for (int k = 0; k < sh.nout; ++k) row_bytes += 16ll * sh.out_vecs[k];
    const int64_t ntok = budget / row_bytes / 2048 * 2048;
    std::vector<int64_t> bytes;
    for (int k = 0; k < sh.nin; ++k) bytes.push_back(16ll * sh.in_vecs[k] * ntok);
    for (int k = 0; k < sh.nout; ++k) bytes.push_back(16ll * sh.out_vecs[k] * ntok);
    void* sink;
    CHECK(hipMalloc(&sink, 16 * 1024));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int layout = 0; layout < kLayouts; ++layout) {
      Placement pl = place(layout, bytes);
      Streams s = {};
      s.sink = (u32x4*)sink;
      for (int k = 0; k < sh.nin; ++k) {
        s.in[k] = (const u32x4*)pl.tensor[k];
        s.in_vecs[k] = sh.in_vecs[k];
        hipLaunchKernelGGL(fill_kernel, dim3(1024), dim3(256), 0, 0, (u32x4*)pl.tensor[k],
                           (int64_t)sh.in_vecs[k] * ntok, (uint32_t)k);
      }
      for (int k = 0; k < sh.nout; ++k) {
        s.out[k] = (u32x4*)pl.tensor[sh.nin + k];
        s.out_vecs[k] = sh.out_vecs[k];
        CHECK(hipMemset(s.out[k], 0, bytes[sh.nin + k]));
      }
      CHECK(hipDeviceSynchronize());
      const int threads = 512;
      for (int grid : {256, 1024}) {
        for (int deal = 0; deal < 3; ++deal) {
          const bool pipe = true;
          KernelFn fn = kernel_for<512>(sh, deal, pipe);
          const int64_t chunk = (ntok + grid - 1) / grid;
          std::vector<float> ms;
          for (int rep = 0; rep < 13; ++rep) {
            CHECK(hipEventRecord(e0, 0));
            hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), 0, 0, s, ntok, chunk);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1, 0));
            CHECK(hipEventSynchronize(e1));
            float t;
            CHECK(hipEventElapsedTime(&t, e0, e1));
            if (rep >= 3) ms.push_back(t);
          }
          std::sort(ms.begin(), ms.end());
          const double total = (double)row_bytes * ntok;
          const double med = ms[ms.size() / 2], best = ms[0];
          printf("%-6s %-9s %5d %4d %-8s %-4s %8lld %12.0f %10.1f %10.1f %8.3f %8.3f\n", sh.name, kLayoutName[layout],
                 grid, threads, kDealName[deal], pipe ? "yes" : "no", (long long)ntok, total, med * 1e3, best * 1e3,
                 total / (med * 1e-3) / 1e12, total / (best * 1e-3) / 1e12);
          fflush(stdout);
        }
      }
      for (void* q : pl.allocs) CHECK(hipFree(q));
    }
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    CHECK(hipFree(sink));
  }
  return 0;
}
