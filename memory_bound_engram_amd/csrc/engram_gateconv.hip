// engram_gateconv.hip -- Engram GateConv forward and backward (gfx950).
//
// Operation: "Engram Operators" (TileOPs), GateConv section: RMSNorm gating
// -> causal depthwise conv1d (4 taps) -> SiLU + residual, with saved
// (vhat, alpha, rrms_h, rrms_k, rrms_v).  The page gives no formulas; the
// readings used (same as the oracle's):
//   h^ = H rrms_h w_h, k^ = k rrms_k w_h              (one weight for H and k)
//   alpha = sigmoid(<h^, k^> / sqrt(d)),  vhat = alpha v
//   u = vhat rrms_v w_v,  c_t = sum_{i<4} conv_w[i] u_{t-3+i}  (zero history)
//   Y = SiLU(c) + vhat
// Backward (gradient of that map for L = sum dY Y; see the oracle's header):
//   dc = dY SiLU'(c),  du_t = sum_i conv_w[i] dc_{t+3-i},  dconv_w[i] += dc_t u_{t-3+i}
//   dvhat = dY + rrms_v (w_v du - vhat rrms_v^2 S1 / d),  S1 = <du w_v, vhat>
//   dalpha = <dvhat, v>,  dv = alpha dvhat,  ds = dalpha alpha (1 - alpha)
//   with g = ds rrms_h rrms_k / sqrt(d) and P = sum_j H k w_h^2:
//   dH = g (w_h^2 k - H rrms_h^2 P / d),  dk = g (w_h^2 H - k rrms_k^2 P / d)
//   dw_h += 2 g w_h H k,  dw_v += du vhat rrms_v
//
// Mapping.  A workgroup owns whole token rows: d/8 threads, thread j covers
// the 4-column quads j and j + d/8 (8-byte loads; one wave instruction moves
// 512 contiguous bytes), and walks a chunk of consecutive rows of the
// flattened [M*T] token order (a chunk may cross into the next sequence; the
// conv history restarts there).  The conv couples neighbouring tokens, so
// each chunk recomputes a 3-row halo instead of storing intermediates (a few
// percent more reads, against 20-40% more for any split into two passes).  Row sums reduce with
// DPP inside each wave and across waves through LDS in wave order.  The
// forward keeps the last four u rows of its columns in registers; the
// backward walks time with a lag of three tokens (du_t needs dc of t..t+3)
// and keeps u and dc histories.  Weights sit in LDS.  Weight gradients are
// per-workgroup fp32 partials in the workspace, summed by a second kernel in
// a fixed order.
#include "engram_device.h"
#include "engram_launch.h"

namespace engram {
namespace {

constexpr int kTaps = 4;
constexpr int kCols = 8;   // columns per thread: two quads of 4
constexpr int kMaxThreads = 640;           // d <= 5120
constexpr int kMaxWaves = kMaxThreads / 64;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack4(u32x2 w, float* f) {
  f[0] = bf_lo(w[0]);
  f[1] = bf_hi(w[0]);
  f[2] = bf_lo(w[1]);
  f[3] = bf_hi(w[1]);
}
__device__ __forceinline__ u32x2 pack4(const float* f) {
  u32x2 r;
  r[0] = pack_bf16x2(f[0], f[1]);
  r[1] = pack_bf16x2(f[2], f[3]);
  return r;
}
__device__ __forceinline__ u32x2 ld8(const uint16_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)); }
__device__ __forceinline__ u32x2 ld8_keep(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(uint16_t* p, u32x2 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p)); }

// Columns of quad q (q = 0, 1) of thread j, for a row of width d.
__device__ __forceinline__ int quad_col(int j, int q, int d) { return 4 * (j + q * (d / kCols)); }

// Sum NV values over the workgroup: DPP within waves, then the wave partials in
// wave order.  red must hold [2][kMaxWaves][4] floats; buf alternates.
template <int NV>
__device__ __forceinline__ void block_sum(float* v, float (*red)[kMaxWaves][4], int& buf, int nwaves) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_sum_to_lane63(v[i]);
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < NV; ++i) red[buf][wave][i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = 0.f;
  for (int w = 0; w < nwaves; ++w) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] += red[buf][w][i];
  }
  buf ^= 1;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// ------------------------------------------------------------------ forward

__global__ void __launch_bounds__(kMaxThreads)
gateconv_fwd_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                    const float* __restrict__ wh, const float* __restrict__ wv, const float* __restrict__ cw,
                    uint16_t* __restrict__ Y, uint16_t* __restrict__ vhat, float* __restrict__ alpha,
                    float* __restrict__ rrh, float* __restrict__ rrk, float* __restrict__ rrv, int rows, int T, int d,
                    int chunk, float eps) {
  __shared__ float red[2][kMaxWaves][4];
  const int j = threadIdx.x;
  const int nwaves = blockDim.x >> 6;
  const int r0 = blockIdx.x * chunk;
  const int r1 = min(r0 + chunk, rows);
  const int rb = max(r0 - (kTaps - 1), r0 - r0 % T);  // halo rows of the same sequence
  const float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);

  float whsq[kCols], wvv[kCols], w[kTaps][kCols];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c0 = quad_col(j, q, d);
    const f32x4 a = *reinterpret_cast<const f32x4*>(wh + c0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(wv + c0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      whsq[4 * q + e] = a[e] * a[e];
      wvv[4 * q + e] = b[e];
    }
#pragma unroll
    for (int i = 0; i < kTaps; ++i) {
      const f32x4 c = *reinterpret_cast<const f32x4*>(cw + (int64_t)i * d + c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[i][4 * q + e] = c[e];
    }
  }
  float uh[kTaps - 1][kCols];  // u of the three previous rows of the sequence (oldest first)
#pragma unroll
  for (int i = 0; i < kTaps - 1; ++i)
#pragma unroll
    for (int e = 0; e < kCols; ++e) uh[i][e] = 0.f;

  // raw bf16 of the next row, loaded one row ahead
  u32x2 nh[2], nk[2], nv[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t off = (int64_t)rb * d + quad_col(j, q, d);
    nh[q] = ld8(H + off);
    nk[q] = ld8(K + off);
    nv[q] = ld8(V + off);
  }
  int buf = 0;
  int tpos = rb % T;  // position of row r in its sequence
  for (int r = rb; r < r1; ++r) {
    const int64_t row = (int64_t)r * d;
    float h[kCols], k[kCols], v[kCols];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      unpack4(nh[q], h + 4 * q);
      unpack4(nk[q], k + 4 * q);
      unpack4(nv[q], v + 4 * q);
    }
    if (r + 1 < r1) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t off = row + d + quad_col(j, q, d);
        nh[q] = ld8(H + off);
        nk[q] = ld8(K + off);
        nv[q] = ld8(V + off);
      }
    }
    if (tpos == 0) {  // a new sequence: zero history
#pragma unroll
      for (int i = 0; i < kTaps - 1; ++i)
#pragma unroll
        for (int e = 0; e < kCols; ++e) uh[i][e] = 0.f;
    }
    float s[4] = {0.f, 0.f, 0.f, 0.f};  // sum H^2, sum k^2, sum H k w_h^2, sum v^2
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      s[0] = fmaf(h[e], h[e], s[0]);
      s[1] = fmaf(k[e], k[e], s[1]);
      s[2] = fmaf(h[e] * k[e], whsq[e], s[2]);
      s[3] = fmaf(v[e], v[e], s[3]);
    }
    block_sum<4>(s, red, buf, nwaves);
    const float rh = 1.0f / sqrtf(s[0] * inv_d + eps);
    const float rk = 1.0f / sqrtf(s[1] * inv_d + eps);
    const float a = sigmoidf_(((s[2] * rh) * rk) * inv_sqrt_d);
    const float rv = 1.0f / sqrtf((a * a) * (s[3] * inv_d) + eps);
    float vh[kCols], u[kCols];
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      vh[e] = a * v[e];
      u[e] = (vh[e] * rv) * wvv[e];
    }
    if (r >= r0) {
      float y[kCols];
#pragma unroll
      for (int e = 0; e < kCols; ++e) {
        float c = w[0][e] * uh[0][e];
        c = fmaf(w[1][e], uh[1][e], c);
        c = fmaf(w[2][e], uh[2][e], c);
        c = fmaf(w[3][e], u[e], c);
        y[e] = c * sigmoidf_(c) + vh[e];
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c0 = quad_col(j, q, d);
        st8(Y + row + c0, pack4(y + 4 * q));
        st8(vhat + row + c0, pack4(vh + 4 * q));
      }
      if (j == 0) {
        alpha[r] = a;
        rrh[r] = rh;
        rrk[r] = rk;
        rrv[r] = rv;
      }
    }
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      uh[0][e] = uh[1][e];
      uh[1][e] = uh[2][e];
      uh[2][e] = u[e];
    }
    if (++tpos == T) tpos = 0;
  }
}

// ------------------------------------------------------------------ backward

__global__ void __launch_bounds__(kMaxThreads)
gateconv_bwd_kernel(const uint16_t* __restrict__ dY, const uint16_t* __restrict__ H, const uint16_t* __restrict__ K,
                    const uint16_t* __restrict__ V, const float* __restrict__ wh, const float* __restrict__ wv,
                    const float* __restrict__ cw, const uint16_t* __restrict__ vhat, const float* __restrict__ alpha,
                    const float* __restrict__ rrh, const float* __restrict__ rrk, const float* __restrict__ rrv,
                    uint16_t* __restrict__ dH, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                    float* __restrict__ partial, int rows, int T, int d, int chunk) {
  extern __shared__ float lds[];  // w_h [d], w_v [d], conv_w [4][d]
  __shared__ float red[2][kMaxWaves][4];
  float* lwh = lds;
  float* lwv = lds + d;
  float* lcw = lds + 2 * d;
  const int j = threadIdx.x;
  const int nwaves = blockDim.x >> 6;
  const int r0 = blockIdx.x * chunk;
  const int r1 = min(r0 + chunk, rows);
  const int rb = max(r0 - (kTaps - 1), r0 - r0 % T);            // halo rows before, same sequence
  const int re = min(r1 + (kTaps - 1), ((r1 - 1) / T + 1) * T);  // rows after, same sequence
  const float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  for (int q = threadIdx.x; q < 6 * d; q += blockDim.x)
    lds[q] = q < d ? wh[q] : q < 2 * d ? wv[q - d] : cw[q - 2 * d];
  __syncthreads();

  float uh[kTaps][kCols];   // u of rows tau-3 .. tau (index 3 = newest)
  float dch[kTaps][kCols];  // dc of rows tau-3 .. tau
  float awh[kCols], awv[kCols], acw[kTaps][kCols];
#pragma unroll
  for (int e = 0; e < kCols; ++e) {
    awh[e] = awv[e] = 0.f;
#pragma unroll
    for (int i = 0; i < kTaps; ++i) uh[i][e] = dch[i][e] = acw[i][e] = 0.f;
  }

  int buf = 0;
  int tpos = rb % T;  // position of row tau in its sequence
  for (int tau = rb; tau < r1 + (kTaps - 1); ++tau) {
    // shift the histories and bring in row tau (zeros past the rows this chunk needs)
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
#pragma unroll
      for (int i = 0; i < kTaps - 1; ++i) {
        uh[i][e] = tpos == 0 ? 0.f : uh[i + 1][e];  // a sequence start has no history
        dch[i][e] = dch[i + 1][e];
      }
      uh[kTaps - 1][e] = 0.f;
      dch[kTaps - 1][e] = 0.f;
    }
    if (tau < re) {
      const int64_t row = (int64_t)tau * d;
      const float rv = rrv[tau];
      float vh[kCols];
#pragma unroll
      for (int q = 0; q < 2; ++q) unpack4(ld8_keep(vhat + row + quad_col(j, q, d)), vh + 4 * q);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) uh[kTaps - 1][4 * q + e] = (vh[4 * q + e] * rv) * lwv[quad_col(j, q, d) + e];
      if (tau >= r0) {
        float g[kCols];
#pragma unroll
        for (int q = 0; q < 2; ++q) unpack4(ld8_keep(dY + row + quad_col(j, q, d)), g + 4 * q);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int col = quad_col(j, q, d) + e, x = 4 * q + e;
            float c = lcw[col] * uh[0][x];
            c = fmaf(lcw[d + col], uh[1][x], c);
            c = fmaf(lcw[2 * d + col], uh[2][x], c);
            c = fmaf(lcw[3 * d + col], uh[3][x], c);
            const float sg = sigmoidf_(c);
            const float dc = g[x] * (sg * (1.0f + c * (1.0f - sg)));
            dch[kTaps - 1][x] = dc;
            if (tau < r1) {
#pragma unroll
              for (int i = 0; i < kTaps; ++i) acw[i][x] = fmaf(dc, uh[i][x], acw[i][x]);
            }
          }
      }
    }
    // row t = tau - 3 has dc of rows t .. t+3
    const int t = tau - (kTaps - 1);
    if (t >= r0) {  // t < r1 by the loop bound
      const int64_t row = (int64_t)t * d;
      const int ahead = T - 1 - t % T;  // rows after t in its sequence
      const float a = alpha[t], rh = rrh[t], rk = rrk[t], rv = rrv[t];
      float h[kCols], k[kCols], v[kCols], vh[kCols], gy[kCols], du[kCols];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c0 = quad_col(j, q, d);
        unpack4(ld8(H + row + c0), h + 4 * q);
        unpack4(ld8(K + row + c0), k + 4 * q);
        unpack4(ld8(V + row + c0), v + 4 * q);
        unpack4(ld8(vhat + row + c0), vh + 4 * q);  // read three rows ago: in L2
        unpack4(ld8(dY + row + c0), gy + 4 * q);
      }
      float s[2] = {0.f, 0.f};  // S1 = sum du w_v vhat, P = sum H k w_h^2
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = quad_col(j, q, d) + e, x = 4 * q + e;
          // du_t = sum_i conv_w[i] dc_{t+3-i}, dc of rows past the sequence end = 0
          float dd = lcw[3 * d + col] * dch[0][x];
          if (ahead >= 1) dd = fmaf(lcw[2 * d + col], dch[1][x], dd);
          if (ahead >= 2) dd = fmaf(lcw[d + col], dch[2][x], dd);
          if (ahead >= 3) dd = fmaf(lcw[col], dch[3][x], dd);
          du[x] = dd;
          const float wvx = lwv[col], whx = lwh[col];
          s[0] = fmaf(dd * wvx, vh[x], s[0]);
          s[1] = fmaf(h[x] * k[x], whx * whx, s[1]);
          awv[x] = fmaf(dd, vh[x] * rv, awv[x]);
        }
      block_sum<2>(s, red, buf, nwaves);
      const float c1 = (rv * rv) * (s[0] * inv_d);
      float dvh[kCols];
      float dal = 0.f;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = quad_col(j, q, d) + e, x = 4 * q + e;
          dvh[x] = fmaf(rv, fmaf(lwv[col], du[x], -vh[x] * c1), gy[x]);
          dal = fmaf(dvh[x], v[x], dal);
        }
      float sa[1] = {dal};
      block_sum<1>(sa, red, buf, nwaves);
      const float ds = (sa[0] * a) * (1.0f - a);
      const float gg = ((ds * rh) * rk) * inv_sqrt_d;
      const float ph = (rh * rh) * (s[1] * inv_d), pk = (rk * rk) * (s[1] * inv_d);
      float oh[kCols], ok[kCols], ov[kCols];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = quad_col(j, q, d) + e, x = 4 * q + e;
          const float whx = lwh[col], w2 = whx * whx;
          oh[x] = gg * fmaf(w2, k[x], -h[x] * ph);
          ok[x] = gg * fmaf(w2, h[x], -k[x] * pk);
          ov[x] = a * dvh[x];
          awh[x] = fmaf(2.0f * gg * whx, h[x] * k[x], awh[x]);
        }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c0 = quad_col(j, q, d);
        st8(dH + row + c0, pack4(oh + 4 * q));
        st8(dK + row + c0, pack4(ok + 4 * q));
        st8(dV + row + c0, pack4(ov + 4 * q));
      }
    }
    if (++tpos == T) tpos = 0;
  }
  // this workgroup's weight-gradient partials: row blockIdx of [nwg][6][d]
  float* p = partial + (int64_t)blockIdx.x * 6 * d;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c0 = quad_col(j, q, d);
    *reinterpret_cast<f32x4*>(p + c0) = f32x4{awh[4 * q], awh[4 * q + 1], awh[4 * q + 2], awh[4 * q + 3]};
    *reinterpret_cast<f32x4*>(p + d + c0) = f32x4{awv[4 * q], awv[4 * q + 1], awv[4 * q + 2], awv[4 * q + 3]};
#pragma unroll
    for (int i = 0; i < kTaps; ++i)
      *reinterpret_cast<f32x4*>(p + (2 + i) * d + c0) =
          f32x4{acw[i][4 * q], acw[i][4 * q + 1], acw[i][4 * q + 2], acw[i][4 * q + 3]};
  }
}

// out[c] = sum over nwg rows of partial[row][c], c < 6d: 8 contiguous row chunks
// summed sequentially, then the chunk sums in chunk order (fixed for given nwg).
__global__ void __launch_bounds__(256)
gateconv_reduce_kernel(const float* __restrict__ partial, float* __restrict__ dwh, float* __restrict__ dwv,
                       float* __restrict__ dcw, int nwg, int d) {
  __shared__ f32x4 part[8][32];
  const int g = threadIdx.x % 32, q = threadIdx.x / 32;
  const int c4 = blockIdx.x * 32 + g;  // float4 column of the 6d-wide rows
  const int ncol4 = 6 * d / 4;
  const int b0 = (int)((int64_t)nwg * q / 8), b1 = (int)((int64_t)nwg * (q + 1) / 8);
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (c4 < ncol4)
    for (int b = b0; b < b1; ++b) s += reinterpret_cast<const f32x4*>(partial)[(int64_t)b * ncol4 + c4];
  part[q][g] = s;
  __syncthreads();
  if (q == 0 && c4 < ncol4) {
    f32x4 r = part[0][g];
#pragma unroll
    for (int k = 1; k < 8; ++k) r += part[k][g];
    const int c = 4 * c4;
    float* dst = c < d ? dwh + c : c < 2 * d ? dwv + (c - d) : dcw + (c - 2 * d);
    *reinterpret_cast<f32x4*>(dst) = r;
  }
}

}  // namespace

int gateconv_chunk(int64_t M, int64_t T) {
  // rows per workgroup: one workgroup fits a CU (registers, LDS), so about one
  // chunk per CU of the 256, at least 32 rows (the halo costs 3 rows a chunk),
  // at most 512; a function of the sizes only, so the workspace size is too
  int64_t c = (M * T + 255) / 256;
  c = c < 32 ? 32 : c > 512 ? 512 : c;
  return (int)c;
}

int64_t gateconv_workgroups(int64_t M, int64_t T, int chunk) { return (M * T + chunk - 1) / chunk; }

hipError_t launch_gateconv_fwd(const void* H, const void* K, const void* V, const float* wh, const float* wv,
                               const float* cw, void* Y, void* vhat, float* alpha, float* rrh, float* rrk, float* rrv,
                               int64_t M, int64_t T, int64_t d, float eps, int chunk, hipStream_t stream) {
  const uint16_t *hp = static_cast<const uint16_t*>(H), *kp = static_cast<const uint16_t*>(K),
                 *vp = static_cast<const uint16_t*>(V);
  uint16_t *yp = static_cast<uint16_t*>(Y), *vhp = static_cast<uint16_t*>(vhat);
  int rows = (int)(M * T), Ti = (int)T, di = (int)d, ch = chunk;
  void* args[] = {&hp, &kp, &vp, &wh, &wv, &cw, &yp, &vhp, &alpha, &rrh, &rrk, &rrv, &rows, &Ti, &di, &ch, &eps};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gateconv_fwd_kernel),
                         dim3((unsigned)gateconv_workgroups(M, T, chunk)), dim3((unsigned)(d / kCols)), args, 0, stream);
}

hipError_t launch_gateconv_bwd(const void* dY, const void* H, const void* K, const void* V, const float* wh,
                               const float* wv, const float* cw, const void* vhat, const float* alpha, const float* rrh,
                               const float* rrk, const float* rrv, void* dH, void* dK, void* dV, float* dwh, float* dwv,
                               float* dcw, void* workspace, int64_t M, int64_t T, int64_t d, int chunk,
                               hipStream_t stream) {
  const uint16_t *gp = static_cast<const uint16_t*>(dY), *hp = static_cast<const uint16_t*>(H),
                 *kp = static_cast<const uint16_t*>(K), *vp = static_cast<const uint16_t*>(V),
                 *vhp = static_cast<const uint16_t*>(vhat);
  uint16_t *dhp = static_cast<uint16_t*>(dH), *dkp = static_cast<uint16_t*>(dK), *dvp = static_cast<uint16_t*>(dV);
  float* partial = static_cast<float*>(workspace);
  int rows = (int)(M * T), Ti = (int)T, di = (int)d, ch = chunk;
  void* args[] = {&gp, &hp, &kp, &vp, &wh, &wv, &cw, &vhp, &alpha, &rrh, &rrk, &rrv, &dhp, &dkp, &dvp, &partial,
                  &rows, &Ti, &di, &ch};
  const int64_t nwg = gateconv_workgroups(M, T, chunk);
  static const hipError_t lds_ok = hipFuncSetAttribute(reinterpret_cast<const void*>(&gateconv_bwd_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       6 * kMaxThreads * kCols * (int)sizeof(float));
  if (lds_ok != hipSuccess) return lds_ok;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&gateconv_bwd_kernel), dim3((unsigned)nwg),
                                 dim3((unsigned)(d / kCols)), args, (size_t)6 * d * sizeof(float), stream);
  if (e != hipSuccess) return e;
  const float* cp = partial;
  int nw = (int)nwg;
  void* args2[] = {&cp, &dwh, &dwv, &dcw, &nw, &di};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gateconv_reduce_kernel), dim3((unsigned)((6 * d / 4 + 31) / 32)),
                         dim3(256), args2, 0, stream);
}

}  // namespace engram
