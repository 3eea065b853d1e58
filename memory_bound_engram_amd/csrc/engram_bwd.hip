// engram_bwd.hip -- explicit backward of the four-stream Engram saved-state gate.
//
// Operation: "Engram saved-state gate" (cuDNN frontend docs), layout,
// saved-state and workspace paragraphs; the formulas are the gradient of the
// forward map.  From saved (gate g^, dot, rstd_X, rstd_key) and grad_out G,
// per token and stream, with x^ = rstd_X x and k^ = rstd_key k:
//   dg    = sum_j G_j v_j
//   delta = (|dot| >= c) ? dg g^ (1 - g^) / (2 sqrt|dot|) : 0
//   dx_j  = G_j + delta rstd_X (w_j k^_j - dot x^_j / d)
//         = G_j + a w_j k_j - b x_j,        a = delta rstd_X rstd_key,
//                                           b = delta rstd_X^2 dot / d
//   dk_j  = a w_j x_j - e k_j,              e = delta rstd_key^2 dot / d
//   dv_j  = sum_s g^_s G_{s,j}              (fp32, streams in order, one bf16 cast)
//   dw_{s,j} = sum_t a_{t,s} x_j k_j        (= sum_t delta x^_j k^_j)
//
// Kernel 1 (main): one workgroup per 64-token block, 640 threads; thread c
// owns columns [8c, 8c+8) of every row.  Per token it loads G, X and the keys
// for all four streams plus the shared value (13 16-byte loads per thread),
// reduces the four dg sums (DPP within a wave, LDS across waves), and writes
// grad_x and grad_kv.  The grad_weight contribution a x k of its columns is
// accumulated in VGPRs over the block's 64 tokens and written once, as row b
// of the fp32 partials [N/64][4][5120] in the workspace.
// Kernel 2 (reduce): grad_weight[s][j] = sum over b of the partials, in a
// fixed order (8 contiguous row chunks summed sequentially, then the chunk
// sums added in chunk order), so the result is bitwise reproducible.
//
// Workspace layout (size fixed by the workspace paragraph): the first 16*N
// floats are reserved for per-(token, stream) scalars and are unused by this
// implementation; the partials start at float offset 16*N (byte 64*N, which
// keeps 16-byte alignment).
#include "engram_device.h"
#include "engram_launch.h"

namespace engram {

constexpr int kBwdThreads = kRowVecs;        // 640
constexpr int kBwdWaves = kBwdThreads / 64;  // 10

__global__ void __launch_bounds__(kBwdThreads)
engram_bwd_main_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ kv,
                       const float* __restrict__ weight, const float* __restrict__ saved,
                       const uint16_t* __restrict__ gout, uint16_t* __restrict__ dx,
                       uint16_t* __restrict__ dkv, float* __restrict__ partial) {
  __shared__ float red[2][kBwdWaves][4];
  const int c = threadIdx.x;
  const int wave = c >> 6, lane = c & 63;
  const int col = c * kVec;
  const int64_t block = blockIdx.x;

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
  float acc[kStreams][kVec];
#pragma unroll
  for (int s = 0; s < kStreams; ++s)
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[s][e] = 0.f;

  int buf = 0;
  for (int i = 0; i < kTokensPerPartial; ++i) {
    const int64_t t = block * kTokensPerPartial + i;
    const uint16_t* xt = x + t * (kStreams * kHidden) + col;
    const uint16_t* kt = kv + t * kKvCols + col;
    const uint16_t* gt = gout + t * (kStreams * kHidden) + col;

    u32x4 gr[kStreams], xr[kStreams], kr[kStreams];
#pragma unroll
    for (int s = 0; s < kStreams; ++s) gr[s] = load16_stream(gt + s * kHidden);
    const u32x4 vr = load16_stream(kt + kValueCol);
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
      xr[s] = load16_stream(xt + s * kHidden);
      kr[s] = load16_stream(kt + s * kHidden);
    }

    float part[kStreams];
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
      float p = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        p = fmaf(bf_lo(gr[s][q]), bf_lo(vr[q]), p);
        p = fmaf(bf_hi(gr[s][q]), bf_hi(vr[q]), p);
      }
      part[s] = wave_sum_to_lane63(p);
    }
    if (lane == 63) {
#pragma unroll
      for (int s = 0; s < kStreams; ++s) red[buf][wave][s] = part[s];
    }
    __syncthreads();
    float tot = 0.f;
    if (lane < kStreams) {
#pragma unroll
      for (int v = 0; v < kBwdWaves; ++v) tot += red[buf][v][lane];
    }
    buf ^= 1;

    const float* sv = saved + t * (kStreams * 4);
    float gh[kStreams], ca[kStreams], cb[kStreams], ce[kStreams];
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
      const float g = sv[4 * s + 0], dot = sv[4 * s + 1];
      const float rx = sv[4 * s + 2], rk = sv[4 * s + 3];
      const float dg = read_lane(tot, s);
      const float dz = dg * g * (1.0f - g);
      const float ad = fabsf(dot);
      const float delta = ad >= kClamp ? dz / (2.0f * sqrtf(ad)) : 0.0f;
      const float dr = delta * rx;
      gh[s] = g;
      ca[s] = dr * rk;
      cb[s] = dr * rx * (dot / (float)kHidden);
      ce[s] = delta * rk * rk * (dot / (float)kHidden);
    }

    uint16_t* dxt = dx + t * (kStreams * kHidden) + col;
    uint16_t* dkt = dkv + t * kKvCols + col;
    float dv[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) dv[e] = 0.f;
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
      u32x4 ox, ok;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float gx[2] = {bf_lo(gr[s][q]), bf_hi(gr[s][q])};
        float xx[2] = {bf_lo(xr[s][q]), bf_hi(xr[s][q])};
        float kk[2] = {bf_lo(kr[s][q]), bf_hi(kr[s][q])};
        float rdx[2], rdk[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = 2 * q + h;
          const float wk = w[s][e] * kk[h];
          const float wx = w[s][e] * xx[h];
          rdx[h] = fmaf(-cb[s], xx[h], fmaf(ca[s], wk, gx[h]));
          rdk[h] = fmaf(-ce[s], kk[h], ca[s] * wx);
          acc[s][e] = fmaf(ca[s], xx[h] * kk[h], acc[s][e]);
          dv[e] = s == 0 ? gh[0] * gx[h] : fmaf(gh[s], gx[h], dv[e]);
        }
        ox[q] = pack_bf16x2(rdx[0], rdx[1]);
        ok[q] = pack_bf16x2(rdk[0], rdk[1]);
      }
      store16_stream(dxt + s * kHidden, ox);
      store16_stream(dkt + s * kHidden, ok);
    }
    u32x4 ov;
#pragma unroll
    for (int q = 0; q < 4; ++q) ov[q] = pack_bf16x2(dv[2 * q], dv[2 * q + 1]);
    store16_stream(dkt + kValueCol, ov);
  }

  float* prow = partial + block * (kStreams * kHidden) + col;
#pragma unroll
  for (int s = 0; s < kStreams; ++s) {
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = acc[s][e];
      b[e] = acc[s][4 + e];
    }
    *reinterpret_cast<f32x4*>(prow + s * kHidden) = a;
    *reinterpret_cast<f32x4*>(prow + s * kHidden + 4) = b;
  }
}

constexpr int kReduceChunks = 8;                         // row chunks per column group
constexpr int kReduceGroups = 32;                        // float4 column groups per workgroup
constexpr int kReduceThreads = kReduceChunks * kReduceGroups;  // 256
constexpr int kReduceCols4 = kStreams * kHidden / 4;     // 5120 float4 columns

__global__ void __launch_bounds__(kReduceThreads)
engram_bwd_reduce_kernel(const float* __restrict__ partial, float* __restrict__ dw, int nb) {
  __shared__ f32x4 part[kReduceChunks][kReduceGroups];
  const int g = threadIdx.x % kReduceGroups;
  const int q = threadIdx.x / kReduceGroups;
  const int col4 = blockIdx.x * kReduceGroups + g;  // grid covers exactly kReduceCols4
  const int b0 = (int)((int64_t)nb * q / kReduceChunks);
  const int b1 = (int)((int64_t)nb * (q + 1) / kReduceChunks);
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  const f32x4* p = reinterpret_cast<const f32x4*>(partial) + col4;
  for (int b = b0; b < b1; ++b) s += p[(int64_t)b * kReduceCols4];
  part[q][g] = s;
  __syncthreads();
  if (q == 0) {
    f32x4 r = part[0][g];
#pragma unroll
    for (int k = 1; k < kReduceChunks; ++k) r += part[k][g];
    reinterpret_cast<f32x4*>(dw)[col4] = r;
  }
}

hipError_t launch_bwd(const void* x, const void* kv, const float* weight, const float* saved, const void* gout,
                      void* dx, void* dkv, float* dw, void* workspace, int64_t n, hipStream_t stream) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* kvp = static_cast<const uint16_t*>(kv);
  const uint16_t* gp = static_cast<const uint16_t*>(gout);
  uint16_t* dxp = static_cast<uint16_t*>(dx);
  uint16_t* dkvp = static_cast<uint16_t*>(dkv);
  float* partial = static_cast<float*>(workspace) + 16 * n;
  const int nb = (int)(n / kTokensPerPartial);
  void* args1[] = {&xp, &kvp, &weight, &saved, &gp, &dxp, &dkvp, &partial};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&engram_bwd_main_kernel), dim3(nb),
                                 dim3(kBwdThreads), args1, 0, stream);
  if (e != hipSuccess) return e;
  const float* cpartial = partial;
  int nbv = nb;
  void* args2[] = {&cpartial, &dw, &nbv};
  return hipLaunchKernel(reinterpret_cast<const void*>(&engram_bwd_reduce_kernel),
                         dim3(kReduceCols4 / kReduceGroups), dim3(kReduceThreads), args2, 0, stream);
}

}  // namespace engram
