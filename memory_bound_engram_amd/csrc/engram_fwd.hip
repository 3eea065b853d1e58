// engram_fwd.hip -- forward of the four-stream Engram saved-state gate.
//
// Operation: "Engram saved-state gate" (cuDNN frontend docs), semantics,
// layout and saved-state paragraphs.  Per token t and stream s:
//   rstd_X = (sum x^2 / d + eps)^-1/2, rstd_key likewise,
//   dot = rstd_X * rstd_key * sum_j x_j w_j k_j   (= sum x^ w k^),
//   gate = sigmoid(sgn(dot) sqrt(max(|dot|, c))), sgn(0) = 0,
//   out = mask ? bf16(x + gate v) : x (bit copy), saved = (mask?gate:0, dot, rstd_X, rstd_key).
//
// Mapping: one wave64 per (token, stream).  A workgroup is 4 waves -- the 4
// streams of one token -- and strides over the tokens by the grid size (the
// launcher's grid holds a few workgroups per CU; one is resident at a time).  Lane l of wave s covers vectors l + 64 i
// (i = 0..9, 8 bf16 each) of stream s's rows, so every wave instruction
// moves 1 KB of contiguous memory and the three per-row sums (x.x, k.k,
// x.w.k) reduce inside the wave with DPP: no LDS and no barrier.  The weight
// slice of each lane (10 x 8 fp32) stays in VGPRs for all tokens.  The shared
// value row is read by all four waves of the workgroup with normal (L2
// resident) loads, so HBM delivers it once; X and the keys are read, and out
// written, with streaming (non-temporal) hints.
//
// Power-of-two workgroups matter on MI355X: the same traffic runs ~10% faster
// with 256-thread workgroups than with 640-thread ones (one thread per
// 16-byte column of a 5120-wide row), which this mapping avoids.
#include "engram_device.h"
#include "engram_launch.h"

#include <atomic>
#include <cstdlib>
#include <mutex>

namespace engram {

constexpr int kFwdThreads = 64 * kStreams;   // one wave per stream
constexpr int kFwdVecs = kRowVecs / 64;      // 10 vectors per lane per row

// One token of the forward: the four waves of the workgroup each handle their
// stream of token t.  kSave = false is the inference forward: saved is not
// written; out is bit-identical to the saving path (same arithmetic).
template <bool kSave>
__device__ __forceinline__ void fwd_token(const uint16_t* __restrict__ x, const uint16_t* __restrict__ kv,
                                          const uint8_t* __restrict__ mask, uint16_t* __restrict__ out,
                                          float* __restrict__ saved, const float (&w)[kFwdVecs][kVec], int64_t t,
                                          int s, int lane) {
  const bool m = mask[t] != 0;
  const uint16_t* xs = x + t * (kStreams * kHidden) + s * kHidden;
  const uint16_t* ks = kv + t * kKvCols + s * kHidden;
  const uint16_t* vs = kv + t * kKvCols + kValueCol;

  u32x4 xr[kFwdVecs], kr[kFwdVecs], vr[kFwdVecs];
#pragma unroll
  for (int i = 0; i < kFwdVecs; ++i) {
    const int col = (lane + 64 * i) * kVec;
    xr[i] = load16_stream(xs + col);
    kr[i] = load16_stream(ks + col);
  }
  if (m) {  // masked tokens never need the value
#pragma unroll
    for (int i = 0; i < kFwdVecs; ++i) vr[i] = load16(vs + (lane + 64 * i) * kVec);
  }

  float sxx = 0.f, skk = 0.f, sxwk = 0.f;
#pragma unroll
  for (int i = 0; i < kFwdVecs; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x0 = bf_lo(xr[i][q]), x1 = bf_hi(xr[i][q]);
      const float k0 = bf_lo(kr[i][q]), k1 = bf_hi(kr[i][q]);
      sxx = fmaf(x0, x0, sxx);
      sxx = fmaf(x1, x1, sxx);
      skk = fmaf(k0, k0, skk);
      skk = fmaf(k1, k1, skk);
      sxwk = fmaf(x0 * w[i][2 * q], k0, sxwk);
      sxwk = fmaf(x1 * w[i][2 * q + 1], k1, sxwk);
    }
  }
  sxx = read_lane(wave_sum_to_lane63(sxx), 63);
  skk = read_lane(wave_sum_to_lane63(skk), 63);
  sxwk = read_lane(wave_sum_to_lane63(sxwk), 63);

  const float rx = 1.0f / sqrtf(sxx / (float)kHidden + kEps);
  const float rk = 1.0f / sqrtf(skk / (float)kHidden + kEps);
  const float dot = (sxwk * rx) * rk;
  const float mag = sqrtf(fmaxf(fabsf(dot), kClamp));
  const float z = dot > 0.f ? mag : (dot < 0.f ? -mag : 0.f);
  const float gate = 1.0f / (1.0f + expf(-z));

  uint16_t* os = out + t * (kStreams * kHidden) + s * kHidden;
#pragma unroll
  for (int i = 0; i < kFwdVecs; ++i) {
    u32x4 o = xr[i];
    if (m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float o0 = fmaf(gate, bf_lo(vr[i][q]), bf_lo(xr[i][q]));
        const float o1 = fmaf(gate, bf_hi(vr[i][q]), bf_hi(xr[i][q]));
        o[q] = pack_bf16x2(o0, o1);
      }
    }
    store16_stream(os + (lane + 64 * i) * kVec, o);
  }
  if (kSave && lane == 0) {
    const f32x4 sv = {m ? gate : 0.f, dot, rx, rk};
    *reinterpret_cast<f32x4*>(saved + t * (kStreams * 4) + 4 * s) = sv;
  }
}

// Each lane's slice of the stream's weight row (10 x 8 fp32), kept in VGPRs.
__device__ __forceinline__ void load_weight_slice(const float* __restrict__ weight, float (&w)[kFwdVecs][kVec], int s,
                                                  int lane) {
#pragma unroll
  for (int i = 0; i < kFwdVecs; ++i) {
    const int col = (lane + 64 * i) * kVec;
    const f32x4 a = *reinterpret_cast<const f32x4*>(weight + s * kHidden + col);
    const f32x4 b = *reinterpret_cast<const f32x4*>(weight + s * kHidden + col + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[i][e] = a[e];
      w[i][4 + e] = b[e];
    }
  }
}

template <bool kSave>
__global__ void __launch_bounds__(kFwdThreads)
engram_fwd_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ kv,
                  const float* __restrict__ weight, const uint8_t* __restrict__ mask,
                  uint16_t* __restrict__ out, float* __restrict__ saved, int64_t n) {
  const int s = threadIdx.x >> 6;     // stream of this wave
  const int lane = threadIdx.x & 63;
  float w[kFwdVecs][kVec];
  load_weight_slice(weight, w, s, lane);
  for (int64_t t = blockIdx.x; t < n; t += gridDim.x) fwd_token<kSave>(x, kv, mask, out, saved, w, t, s, lane);
}

// ---- the paced forward, for long calls ----
//
// A long call is walked in epochs: one workgroup per CU (all resident at
// once), workgroup b taking tokens b + G i (G = grid size), and after every
// kFwdEpochSteps of them the workgroups meet at the pacing barrier
// (engram_device.h) before the next epoch.  Measured on MI355X at
// N = 1,048,512 on one set of buffers: the unpaced kernel took 23.6-24.1 ms
// (72-74% of 8 TB/s), the same tokens as 128 launches of 8192 back to back
// 22.4-22.5 ms, this kernel 22.3-22.4 ms (78%); epochs of 16 tokens were
// slower (22.8 ms: more barriers), of 64 the same as 32; 8 or 32 barrier
// groups the same as 16.  Each call takes its own slot of a file-scope
// counter array, dealt round robin per device by pace_slot().
#ifndef ENGRAM_FWD_EPOCH_STEPS
#define ENGRAM_FWD_EPOCH_STEPS 32
#endif
constexpr int kFwdEpochSteps = ENGRAM_FWD_EPOCH_STEPS;
constexpr int kPaceSlots = 16;
static __device__ __align__(256) uint32_t pace_counters[kPaceSlots * kPaceSlotWords];

template <bool kSave>
__global__ void __launch_bounds__(kFwdThreads)
engram_fwd_paced_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ kv,
                        const float* __restrict__ weight, const uint8_t* __restrict__ mask,
                        uint16_t* __restrict__ out, float* __restrict__ saved, int64_t n, uint32_t* slot,
                        int64_t epochs, uint64_t spin_ticks) {
  const int s = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  float w[kFwdVecs][kVec];
  load_weight_slice(weight, w, s, lane);
  const int64_t G = gridDim.x;
  for (int64_t e = 0; e < epochs; ++e) {
    const int64_t t0 = e * kFwdEpochSteps * G + blockIdx.x;
    for (int j = 0; j < kFwdEpochSteps; ++j) {
      const int64_t t = t0 + j * G;
      if (t < n) fwd_token<kSave>(x, kv, mask, out, saved, w, t, s, lane);
    }
    if (e + 1 < epochs) {
      __syncthreads();
      if (threadIdx.x == 0) pace_barrier(slot, (uint32_t)(e + 1), blockIdx.x, (uint32_t)G, spin_ticks);
      __syncthreads();
    }
  }
  if (epochs > 1 && threadIdx.x == 0) pace_depart(slot, (uint32_t)G);
}

hipError_t launch_fwd(const void* x, const void* kv, const float* weight, const uint8_t* mask, void* out,
                      float* saved, int64_t n, int grid, hipStream_t stream) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* kvp = static_cast<const uint16_t*>(kv);
  uint16_t* op = static_cast<uint16_t*>(out);
  void* args[] = {&xp, &kvp, &weight, &mask, &op, &saved, &n};
  const void* fn = saved ? reinterpret_cast<const void*>(&engram_fwd_kernel<true>)
                         : reinterpret_cast<const void*>(&engram_fwd_kernel<false>);
  return hipLaunchKernel(fn, dim3(grid), dim3(kFwdThreads), args, 0, stream);
}

namespace {
struct PaceDevice {
  std::atomic<uint32_t*> base{nullptr};
  std::atomic<uint64_t> ticks_per_us{0};
  std::atomic<uint32_t> next_slot{0};
};
PaceDevice g_pace[kMaxScratchDevices];
std::mutex g_pace_mu;
}  // namespace

hipError_t pace_slot(uint32_t** slot, uint64_t* ticks_per_us) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  PaceDevice& pd = g_pace[dev];
  if (!pd.base.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lock(g_pace_mu);
    if (!pd.base.load(std::memory_order_relaxed)) {
      int khz = 0;
      e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
      if (e != hipSuccess) return e;
      if (khz <= 0) return hipErrorInvalidValue;
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(pace_counters));  // this device's copy of the array
      if (e != hipSuccess) return e;
      pd.ticks_per_us.store((uint64_t)khz / 1000 > 0 ? (uint64_t)khz / 1000 : 1, std::memory_order_relaxed);
      pd.base.store(static_cast<uint32_t*>(p), std::memory_order_release);
    }
  }
  *slot = pd.base.load(std::memory_order_acquire) +
          (size_t)(pd.next_slot.fetch_add(1, std::memory_order_relaxed) % kPaceSlots) * kPaceSlotWords;
  *ticks_per_us = pd.ticks_per_us.load(std::memory_order_relaxed);
  return hipSuccess;
}

// Longest wait at a pacing barrier, in microseconds: ENGRAM_PACE_WAIT_US if
// set to a number in 0..1000000 (0: no workgroup waits, i.e. no pacing), else
// 200 (an epoch itself takes ~180 us at full speed).  Read at every call.
uint64_t pace_wait_us() {
  const char* v = std::getenv("ENGRAM_PACE_WAIT_US");
  if (v && *v) {
    char* end = nullptr;
    const long long us = std::strtoll(v, &end, 10);
    if (end && *end == '\0' && us >= 0 && us <= 1000000) return (uint64_t)us;
  }
  return 200;
}

int64_t fwd_paced_epochs(int64_t n, int grid) {
  const int64_t per_wg = (n + grid - 1) / grid;
  return (per_wg + kFwdEpochSteps - 1) / kFwdEpochSteps;
}

hipError_t launch_fwd_paced(const void* x, const void* kv, const float* weight, const uint8_t* mask, void* out,
                            float* saved, int64_t n, int grid, hipStream_t stream) {
  uint32_t* slot = nullptr;
  uint64_t ticks_per_us = 0;
  const hipError_t e = pace_slot(&slot, &ticks_per_us);
  if (e != hipSuccess) return e;
  int64_t epochs = fwd_paced_epochs(n, grid);
  uint64_t spin_ticks = pace_wait_us() * ticks_per_us;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* kvp = static_cast<const uint16_t*>(kv);
  uint16_t* op = static_cast<uint16_t*>(out);
  void* args[] = {&xp, &kvp, &weight, &mask, &op, &saved, &n, &slot, &epochs, &spin_ticks};
  const void* fn = saved ? reinterpret_cast<const void*>(&engram_fwd_paced_kernel<true>)
                         : reinterpret_cast<const void*>(&engram_fwd_paced_kernel<false>);
  return hipLaunchKernel(fn, dim3(grid), dim3(kFwdThreads), args, 0, stream);
}

}  // namespace engram
