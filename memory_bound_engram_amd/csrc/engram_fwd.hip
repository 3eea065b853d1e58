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

namespace engram {

constexpr int kFwdThreads = 64 * kStreams;   // one wave per stream
constexpr int kFwdVecs = kRowVecs / 64;      // 10 vectors per lane per row

// kSave = false is the inference forward: saved is not written; out is
// bit-identical to the saving path (same arithmetic).
template <bool kSave>
__global__ void __launch_bounds__(kFwdThreads)
engram_fwd_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ kv,
                  const float* __restrict__ weight, const uint8_t* __restrict__ mask,
                  uint16_t* __restrict__ out, float* __restrict__ saved, int64_t n) {
  const int s = threadIdx.x >> 6;     // stream of this wave
  const int lane = threadIdx.x & 63;

  float w[kFwdVecs][kVec];
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

  for (int64_t t = blockIdx.x; t < n; t += gridDim.x) {
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

}  // namespace engram
