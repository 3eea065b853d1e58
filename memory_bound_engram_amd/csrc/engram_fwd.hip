// engram_fwd.hip -- forward of the four-stream Engram saved-state gate.
//
// Operation: "Engram saved-state gate" (cuDNN frontend docs), semantics,
// layout and saved-state paragraphs.  Per token t and stream s:
//   rstd_X = (sum x^2 / d + eps)^-1/2, rstd_key likewise,
//   dot = rstd_X * rstd_key * sum_j x_j w_j k_j   (= sum x^ w k^),
//   gate = sigmoid(sgn(dot) sqrt(max(|dot|, c))), sgn(0) = 0,
//   out = mask ? bf16(x + gate v) : x (bit copy), saved = (mask?gate:0, dot, rstd_X, rstd_key).
//
// Mapping.  A workgroup of 640 threads (10 wave64s) owns one token at a
// time; thread c owns columns [8c, 8c+8) of every row, so each thread issues
// one 16-byte load per X row, per key row and for the shared value -- the
// value is read from HBM once and reused for all four streams.  The 12 sums
// per token (sum x^2, sum k^2, sum x w k for 4 streams) are reduced with DPP
// inside each wave and across the 10 waves through LDS (double-buffered, one
// barrier per token).  The grid is persistent (a few workgroups per CU, each
// striding over tokens), so the fp32 weight slice of each thread (4 x 8
// values) is loaded once into VGPRs and reused for every token.
#include "engram_device.h"
#include "engram_launch.h"

namespace engram {

constexpr int kFwdThreads = kRowVecs;        // 640
constexpr int kFwdWaves = kFwdThreads / 64;  // 10
constexpr int kFwdSums = 3 * kStreams;       // 12 per token

__global__ void __launch_bounds__(kFwdThreads)
engram_fwd_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ kv,
                  const float* __restrict__ weight, const uint8_t* __restrict__ mask,
                  uint16_t* __restrict__ out, float* __restrict__ saved, int64_t n) {
  __shared__ float red[2][kFwdWaves][16];
  const int c = threadIdx.x;
  const int wave = c >> 6, lane = c & 63;
  const int col = c * kVec;

  float w[kStreams][kVec];
#pragma unroll
  for (int s = 0; s < kStreams; ++s) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(weight + s * kHidden + col);
    const f32x4 b = *reinterpret_cast<const f32x4*>(weight + s * kHidden + col + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[s][e] = a[e];
      w[s][4 + e] = b[e];
    }
  }

  int buf = 0;
  for (int64_t t = blockIdx.x; t < n; t += gridDim.x) {
    const bool m = mask[t] != 0;
    const uint16_t* xt = x + t * (kStreams * kHidden) + col;
    const uint16_t* kt = kv + t * kKvCols + col;

    u32x4 xr[kStreams], kr[kStreams];
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
      xr[s] = load16_stream(xt + s * kHidden);
      kr[s] = load16_stream(kt + s * kHidden);
    }
    u32x4 vr = {0u, 0u, 0u, 0u};
    if (m) vr = load16_stream(kt + kValueCol);  // masked tokens never need the value

    float acc[kFwdSums];
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
      float sxx = 0.f, skk = 0.f, sxwk = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = bf_lo(xr[s][q]), x1 = bf_hi(xr[s][q]);
        const float k0 = bf_lo(kr[s][q]), k1 = bf_hi(kr[s][q]);
        sxx = fmaf(x0, x0, sxx);
        sxx = fmaf(x1, x1, sxx);
        skk = fmaf(k0, k0, skk);
        skk = fmaf(k1, k1, skk);
        sxwk = fmaf(x0 * w[s][2 * q], k0, sxwk);
        sxwk = fmaf(x1 * w[s][2 * q + 1], k1, sxwk);
      }
      acc[s] = sxx;
      acc[kStreams + s] = skk;
      acc[2 * kStreams + s] = sxwk;
    }
#pragma unroll
    for (int i = 0; i < kFwdSums; ++i) acc[i] = wave_sum_to_lane63(acc[i]);
    if (lane == 63) {
#pragma unroll
      for (int i = 0; i < kFwdSums; ++i) red[buf][wave][i] = acc[i];
    }
    __syncthreads();
    // lanes 0..11 of every wave add the 10 wave partials of sum #lane, in wave order
    float tot = 0.f;
    if (lane < kFwdSums) {
#pragma unroll
      for (int v = 0; v < kFwdWaves; ++v) tot += red[buf][v][lane];
    }
    buf ^= 1;  // the next token writes the other buffer; one barrier per token suffices

    float gate[kStreams], dot[kStreams], rx[kStreams], rk[kStreams];
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
      const float sxx = read_lane(tot, s);
      const float skk = read_lane(tot, kStreams + s);
      const float sxwk = read_lane(tot, 2 * kStreams + s);
      rx[s] = 1.0f / sqrtf(sxx / (float)kHidden + kEps);
      rk[s] = 1.0f / sqrtf(skk / (float)kHidden + kEps);
      dot[s] = (sxwk * rx[s]) * rk[s];
      const float mag = sqrtf(fmaxf(fabsf(dot[s]), kClamp));
      const float z = dot[s] > 0.f ? mag : (dot[s] < 0.f ? -mag : 0.f);
      gate[s] = 1.0f / (1.0f + expf(-z));
    }

    uint16_t* ot = out + t * (kStreams * kHidden) + col;
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
      u32x4 o = xr[s];
      if (m) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float o0 = fmaf(gate[s], bf_lo(vr[q]), bf_lo(xr[s][q]));
          const float o1 = fmaf(gate[s], bf_hi(vr[q]), bf_hi(xr[s][q]));
          o[q] = pack_bf16x2(o0, o1);
        }
      }
      store16_stream(ot + s * kHidden, o);
    }
    if (c < kStreams) {
      // thread c < 4 writes stream c's (gate, dot, rstd_X, rstd_key)
      f32x4 sv;
      sv[0] = c == 0 ? gate[0] : c == 1 ? gate[1] : c == 2 ? gate[2] : gate[3];
      sv[1] = c == 0 ? dot[0] : c == 1 ? dot[1] : c == 2 ? dot[2] : dot[3];
      sv[2] = c == 0 ? rx[0] : c == 1 ? rx[1] : c == 2 ? rx[2] : rx[3];
      sv[3] = c == 0 ? rk[0] : c == 1 ? rk[1] : c == 2 ? rk[2] : rk[3];
      if (!m) sv[0] = 0.f;
      *reinterpret_cast<f32x4*>(saved + t * (kStreams * 4) + 4 * c) = sv;
    }
  }
}

hipError_t launch_fwd(const void* x, const void* kv, const float* weight, const uint8_t* mask, void* out,
                      float* saved, int64_t n, int grid, hipStream_t stream) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* kvp = static_cast<const uint16_t*>(kv);
  uint16_t* op = static_cast<uint16_t*>(out);
  void* args[] = {&xp, &kvp, &weight, &mask, &op, &saved, &n};
  return hipLaunchKernel(reinterpret_cast<const void*>(&engram_fwd_kernel), dim3(grid), dim3(kFwdThreads), args,
                         0, stream);
}

}  // namespace engram
