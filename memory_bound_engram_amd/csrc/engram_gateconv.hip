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

#include <type_traits>

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

// Sum NV (<= 4) values over the NW waves of the workgroup: DPP inside each
// wave (sum in lane 63), wave partials through LDS, then lanes 0..NW-1 of
// every wave add them with a 16-lane DPP butterfly and lane 0's sum is
// broadcast.  Fixed order, so deterministic; every lane gets the same value.
// red must hold [2][kMaxWaves][4] floats; buf alternates between calls, so a
// call's reads never meet the next call's writes (one barrier apart).
template <int NV, int NW>
__device__ __forceinline__ void block_sum(float* v, float (*red)[kMaxWaves][4], int& buf) {
  static_assert(NW >= 1 && NW <= kMaxWaves && NW <= 16 && NV >= 1 && NV <= 4, "");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_sum_to_lane63(v[i]);
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < NV; ++i) red[buf][wave][i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float p = lane < NW ? red[buf][lane][i] : 0.f;
    p += dpp<0xB1, 0xF, 0xF, true>(p);
    p += dpp<0x4E, 0xF, 0xF, true>(p);
    p += dpp<0x141, 0xF, 0xF, true>(p);
    p += dpp<0x140, 0xF, 0xF, true>(p);
    v[i] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(p)));
  }
  buf ^= 1;
}

// Materialise a value at this point of the program (an empty asm that reads
// and redefines it cannot be moved across other volatile asm or barriers).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// sigmoid(x) = 1 / (1 + 2^(-x log2 e)) from the hardware exp2 and reciprocal
// (each about 1 ulp): four instructions where the correctly rounded exp and
// divide take about twenty, which this kernel pays per element.  Saturates to
// exactly 0 and 1 for large |x|.
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896340736f));
}

// ------------------------------------------------------------------ forward

// Raw bf16 of one row's H, k, v quads for one thread, loaded ahead of use.
struct FwdSlot {
  u32x2 h[2], k[2], v[2];
};

// Loads of row `row` (element offset of its first column): the row base is
// uniform, the column offset per lane.
__device__ __forceinline__ void fwd_issue(FwdSlot& s, const uint16_t* __restrict__ H, const uint16_t* __restrict__ K,
                                          const uint16_t* __restrict__ V, int64_t row, int c0, int c1) {
  const uint16_t *h = H + row, *k = K + row, *v = V + row;
  s.h[0] = ld8(h + c0);
  s.k[0] = ld8(k + c0);
  s.v[0] = ld8(v + c0);
  s.h[1] = ld8(h + c1);
  s.k[1] = ld8(k + c1);
  s.v[1] = ld8(v + c1);
}

constexpr int kFwdAhead = 3;  // rows in flight per workgroup beyond the one being processed

// NW = d / 512 waves; thread j covers columns [4j, 4j+4) and [4j+d/2, 4j+d/2+4).
template <int NW>
__global__ void __launch_bounds__(64 * NW)
gateconv_fwd_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                    const float* __restrict__ wh, const float* __restrict__ wv, const float* __restrict__ cw,
                    uint16_t* __restrict__ Y, uint16_t* __restrict__ vhat, float* __restrict__ alpha,
                    float* __restrict__ rrh, float* __restrict__ rrk, float* __restrict__ rrv, int rows, int T,
                    int chunk, float eps) {
  constexpr int d = NW * 512;
  __shared__ float red[2][kMaxWaves][4];
  const int j = threadIdx.x;
  const int c0 = 4 * j, c1 = 4 * j + d / 2;
  const int r0 = blockIdx.x * chunk;
  const int r1 = min(r0 + chunk, rows);
  const int rb = max(r0 - (kTaps - 1), r0 - r0 % T);  // halo rows of the same sequence
  constexpr float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = __builtin_amdgcn_rsqf((float)d);

  float whsq[kCols], wvv[kCols], w[kTaps][kCols];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int cq = q ? c1 : c0;
    const f32x4 a = *reinterpret_cast<const f32x4*>(wh + cq);
    const f32x4 b = *reinterpret_cast<const f32x4*>(wv + cq);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      whsq[4 * q + e] = a[e] * a[e];
      wvv[4 * q + e] = b[e];
    }
#pragma unroll
    for (int i = 0; i < kTaps; ++i) {
      const f32x4 c = *reinterpret_cast<const f32x4*>(cw + i * d + cq);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[i][4 * q + e] = c[e];
    }
  }
  // the weights arrive before any row load is issued, so no wait inside the
  // row loop is on their account
  __builtin_amdgcn_s_waitcnt(0);

  // u of the three previous rows of the sequence, as a ring: in the k-th row
  // of each group of three, slot k is the oldest and receives the new u
  float uh[kTaps - 1][kCols];
#pragma unroll
  for (int i = 0; i < kTaps - 1; ++i)
#pragma unroll
    for (int e = 0; e < kCols; ++e) uh[i][e] = 0.f;

  // three slots, each refilled with the row three ahead (clamped to the last
  // row) right after it is unpacked; the loop is unrolled by three and every
  // refill is unconditional, so a slot keeps its registers and the loads of
  // the other two slots stay in flight
  FwdSlot sa, sb, sc;
  fwd_issue(sa, H, K, V, (int64_t)rb * d, c0, c1);
  fwd_issue(sb, H, K, V, (int64_t)min(rb + 1, r1 - 1) * d, c0, c1);
  fwd_issue(sc, H, K, V, (int64_t)min(rb + 2, r1 - 1) * d, c0, c1);

  int buf = 0;
  int tpos = rb % T;  // position of the next row in its sequence

  auto step = [&](int r, FwdSlot& sl, auto kc) {
    constexpr int k0 = decltype(kc)::value;  // ring slot of the oldest u
    constexpr int k1 = (k0 + 1) % 3, k2 = (k0 + 2) % 3;
    const int64_t row = (int64_t)r * d;
    float h[kCols], k[kCols], v[kCols];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      unpack4(sl.h[q], h + 4 * q);
      unpack4(sl.k[q], k + 4 * q);
      unpack4(sl.v[q], v + 4 * q);
    }
    // the unpacked values are produced here, before the refill: were the
    // unpack moved past it, the slot's old and new contents would need
    // separate registers and a copy at the loop latch that waits for the loads
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      pin(h[e]);
      pin(k[e]);
      pin(v[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
    fwd_issue(sl, H, K, V, (int64_t)min(r + kFwdAhead, r1 - 1) * d, c0, c1);
    if (tpos == 0) {  // a new sequence: zero history
#pragma unroll
      for (int i = 0; i < kTaps - 1; ++i)
#pragma unroll
        for (int e = 0; e < kCols; ++e) uh[i][e] = 0.f;
    }
    float s[4];  // sum H^2, sum k^2, sum H k w_h^2, sum v^2
    s[0] = h[0] * h[0];
    s[1] = k[0] * k[0];
    s[2] = (h[0] * k[0]) * whsq[0];
    s[3] = v[0] * v[0];
#pragma unroll
    for (int e = 1; e < kCols; ++e) {
      s[0] = fmaf(h[e], h[e], s[0]);
      s[1] = fmaf(k[e], k[e], s[1]);
      s[2] = fmaf(h[e] * k[e], whsq[e], s[2]);
      s[3] = fmaf(v[e], v[e], s[3]);
    }
    block_sum<4, NW>(s, red, buf);
    const float rh = __builtin_amdgcn_rsqf(s[0] * inv_d + eps);
    const float rk = __builtin_amdgcn_rsqf(s[1] * inv_d + eps);
    const float a = sigmoidf_(((s[2] * rh) * rk) * inv_sqrt_d);
    const float rv = __builtin_amdgcn_rsqf((a * a) * (s[3] * inv_d) + eps);
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
        float c = w[0][e] * uh[k0][e];
        c = fmaf(w[1][e], uh[k1][e], c);
        c = fmaf(w[2][e], uh[k2][e], c);
        c = fmaf(w[3][e], u[e], c);
        y[e] = fmaf(c, sigmoidf_(c), vh[e]);
      }
      uint16_t *yr = Y + row, *vr = vhat + row;
      st8(yr + c0, pack4(y));
      st8(vr + c0, pack4(vh));
      st8(yr + c1, pack4(y + 4));
      st8(vr + c1, pack4(vh + 4));
      if (j == 0) {
        alpha[r] = a;
        rrh[r] = rh;
        rrk[r] = rk;
        rrv[r] = rv;
      }
    }
#pragma unroll
    for (int e = 0; e < kCols; ++e) uh[k0][e] = u[e];
    if (++tpos == T) tpos = 0;
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  int r = rb;
  for (; r + 2 < r1; r += 3) {
    step(r, sa, I0{});
    step(r + 1, sb, I1{});
    step(r + 2, sc, I2{});
  }
  if (r < r1) step(r, sa, I0{});
  if (r + 1 < r1) step(r + 1, sb, I1{});
}

// ------------------------------------------------------------------ backward

// The backward runs as two kernels that split the tensors between them, so
// each tensor is still read once and each kernel's per-thread state fits the
// register file of a CU that holds one row-wide workgroup:
//   conv kernel: vhat, dY, v -> dv, the per-row ds = dalpha alpha (1 - alpha),
//                and the conv_w and rms_w_v gradient partials;
//   h/k kernel:  H, k and the per-row scalars -> dH, dk and the rms_w_h partials.
//
// Conv kernel.  Row tau = newest row (its vhat and dY give u_tau and dc_tau);
// row t = tau - 3 is finished in the same step (it needs dc of t..t+3).  Loads
// run one step ahead: slot N holds vhat, dY of the next newest row, slot L
// holds v of the next finished row; the finished row's vhat and dY, read three
// steps earlier, come from L2.  The step is unrolled by four, so the u and dc
// histories are rings whose slots have fixed roles in each of the four steps.
// NW = d / 512 waves; thread j covers columns [4j, 4j+4) and [4j+d/2, 4j+d/2+4).
template <int NW>
__global__ void __launch_bounds__(64 * NW)
gateconv_bwd_conv_kernel(const uint16_t* __restrict__ dY, const uint16_t* __restrict__ V,
                         const float* __restrict__ wv, const float* __restrict__ cw,
                         const uint16_t* __restrict__ vhat, const float* __restrict__ alpha,
                         const float* __restrict__ rrv, uint16_t* __restrict__ dV, float* __restrict__ ds_out,
                         float* __restrict__ partial, int rows, int T, int chunk) {
  constexpr int d = NW * 512;
  // w_v [d], conv_w [4][d], then this thread's conv_w tap 2 and 3 gradient
  // accumulators [2][d] (each column belongs to one thread: no sharing)
  __shared__ __align__(16) float lw[7 * d];
  __shared__ float red[2][kMaxWaves][4];
  const float* lwv = lw;
  const float* lcw = lw + d;
  float* lacw = lw + 5 * d;
  const int j = threadIdx.x;
  const int c0 = 4 * j, c1 = 4 * j + d / 2;
  const int r0 = blockIdx.x * chunk;
  const int r1 = min(r0 + chunk, rows);
  const int rb = max(r0 - (kTaps - 1), r0 - r0 % T);            // halo rows before, same sequence
  const int re = min(r1 + (kTaps - 1), ((r1 - 1) / T + 1) * T);  // rows after, same sequence
  constexpr float inv_d = 1.0f / (float)d;
  for (int q = threadIdx.x; q < 5 * d / 4; q += 64 * NW) {
    const int e = 4 * q;
    const float* src = e < d ? wv + e : cw + (e - d);
    *reinterpret_cast<f32x4*>(lw + e) = *reinterpret_cast<const f32x4*>(src);
  }

  float uh[kTaps][kCols];   // ring of u rows
  float dch[kTaps][kCols];  // ring of dc rows
  float awv[kCols], acw[2][kCols];  // rms_w_v and conv_w taps 0, 1 gradients
#pragma unroll
  for (int e = 0; e < kCols; ++e) {
    awv[e] = acw[0][e] = acw[1][e] = 0.f;
#pragma unroll
    for (int i = 0; i < kTaps; ++i) uh[i][e] = dch[i][e] = 0.f;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int cq = q ? c1 : c0;
    *reinterpret_cast<f32x4*>(lacw + cq) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(lacw + d + cq) = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  u32x2 nv[2], ng[2];  // slot N: vhat, dY of the newest row
  u32x2 lv[2];         // slot L: v of the finished row
  auto issue_n = [&](int row) {
    const uint16_t *a = vhat + (int64_t)row * d, *b = dY + (int64_t)row * d;
    nv[0] = ld8_keep(a + c0);
    ng[0] = ld8_keep(b + c0);
    nv[1] = ld8_keep(a + c1);
    ng[1] = ld8_keep(b + c1);
  };
  auto issue_l = [&](int row) {
    const uint16_t* a = V + (int64_t)row * d;
    lv[0] = ld8(a + c0);
    lv[1] = ld8(a + c1);
  };
  issue_n(rb);
  issue_l(r0);
  __syncthreads();  // weights in LDS

  int buf = 0;
  int tpos = rb % T;  // position of row tau in its sequence

  auto step = [&](int tau, auto kc) {
    constexpr int k0 = decltype(kc)::value;  // ring slot receiving row tau
    constexpr int k1 = (k0 + 1) % 4, k2 = (k0 + 2) % 4, k3 = (k0 + 3) % 4;
    const int t = tau - (kTaps - 1);

    // ---- newest row tau: u_tau, dc_tau and the conv-weight gradient
    float vn[kCols], gn[kCols];
    unpack4(nv[0], vn);
    unpack4(nv[1], vn + 4);
    unpack4(ng[0], gn);
    unpack4(ng[1], gn + 4);
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      pin(vn[e]);
      pin(gn[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_n(min(tau + 1, re - 1));
    u32x2 fv[2], fg[2];  // the finished row's vhat and dY, read three steps ago: from L2
    {
      const int tr = max(t, r0);
      const uint16_t *pa = vhat + (int64_t)tr * d, *pb = dY + (int64_t)tr * d;
      fv[0] = ld8(pa + c0);
      fv[1] = ld8(pa + c1);
      fg[0] = ld8(pb + c0);
      fg[1] = ld8(pb + c1);
    }
    if (tpos == 0) {  // a sequence start: no u history
#pragma unroll
      for (int i = 0; i < kTaps; ++i)
#pragma unroll
        for (int e = 0; e < kCols; ++e) uh[i][e] = 0.f;
    }
    const float rvn = tau < re ? rrv[tau] : 0.f;  // u = 0 past the rows this chunk needs
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int cq = q ? c1 : c0;
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(lwv + cq);
#pragma unroll
      for (int e = 0; e < 4; ++e) uh[k0][4 * q + e] = (vn[4 * q + e] * rvn) * w4[e];
    }
    if (tau >= r0 && tau < re) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int cq = q ? c1 : c0;
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(lcw + cq);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(lcw + d + cq);
        const f32x4 w2 = *reinterpret_cast<const f32x4*>(lcw + 2 * d + cq);
        const f32x4 w3 = *reinterpret_cast<const f32x4*>(lcw + 3 * d + cq);
        f32x4 g2 = *reinterpret_cast<const f32x4*>(lacw + cq);  // conv_w taps 2, 3 gradients
        f32x4 g3 = *reinterpret_cast<const f32x4*>(lacw + d + cq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = 4 * q + e;
          float c = w0[e] * uh[k1][x];
          c = fmaf(w1[e], uh[k2][x], c);
          c = fmaf(w2[e], uh[k3][x], c);
          c = fmaf(w3[e], uh[k0][x], c);
          const float sg = sigmoidf_(c);
          const float dc = gn[x] * (sg * fmaf(c, 1.0f - sg, 1.0f));
          dch[k0][x] = dc;
          if (tau < r1) {
            acw[0][x] = fmaf(dc, uh[k1][x], acw[0][x]);
            acw[1][x] = fmaf(dc, uh[k2][x], acw[1][x]);
            g2[e] = fmaf(dc, uh[k3][x], g2[e]);
            g3[e] = fmaf(dc, uh[k0][x], g3[e]);
          }
        }
        *reinterpret_cast<f32x4*>(lacw + cq) = g2;
        *reinterpret_cast<f32x4*>(lacw + d + cq) = g3;
        __builtin_amdgcn_sched_barrier(0);  // one quad's weights live at a time
      }
    } else {
#pragma unroll
      for (int e = 0; e < kCols; ++e) dch[k0][e] = 0.f;
    }

    // ---- finished row t
    float v[kCols];
    unpack4(lv[0], v);
    unpack4(lv[1], v + 4);
#pragma unroll
    for (int e = 0; e < kCols; ++e) pin(v[e]);
    __builtin_amdgcn_sched_barrier(0);
    issue_l(min(max(t + 1, r0), r1 - 1));
    if (t >= r0) {  // t < r1 by the loop bound
      const int ahead = T - 1 - t % T;  // rows after t in its sequence
      const float a = alpha[t], rv = rrv[t];
      float vh[kCols], gy[kCols];
      unpack4(fv[0], vh);
      unpack4(fv[1], vh + 4);
      unpack4(fg[0], gy);
      unpack4(fg[1], gy + 4);
      // du_t = sum_i conv_w[i] dc_{t+3-i}; dc of rows past the end of t's
      // sequence count as 0 (they belong to the next sequence).  With
      // A = dY + rrms_v w_v du, dvhat = A - rrms_v c1 vhat (c1 = rrms_v^2 S1 / d):
      //   S1 = sum du w_v vhat,  dalpha = sum A v - rrms_v c1 sum vhat v
      float s[3];
      float A[kCols];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int cq = q ? c1 : c0;
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(lcw + cq);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(lcw + d + cq);
        const f32x4 w2 = *reinterpret_cast<const f32x4*>(lcw + 2 * d + cq);
        const f32x4 w3 = *reinterpret_cast<const f32x4*>(lcw + 3 * d + cq);
        const f32x4 wvq = *reinterpret_cast<const f32x4*>(lwv + cq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = 4 * q + e;
          float dd = w3[e] * dch[k1][x];
          if (ahead >= 3) {
            dd = fmaf(w2[e], dch[k2][x], dd);
            dd = fmaf(w1[e], dch[k3][x], dd);
            dd = fmaf(w0[e], dch[k0][x], dd);
          } else {
            if (ahead >= 1) dd = fmaf(w2[e], dch[k2][x], dd);
            if (ahead >= 2) dd = fmaf(w1[e], dch[k3][x], dd);
          }
          const float dw = dd * wvq[e];
          A[x] = fmaf(rv, dw, gy[x]);
          const float p0 = dw * vh[x], p1 = A[x] * v[x], p2 = vh[x] * v[x];
          s[0] = x == 0 ? p0 : s[0] + p0;
          s[1] = x == 0 ? p1 : s[1] + p1;
          s[2] = x == 0 ? p2 : s[2] + p2;
          awv[x] = fmaf(dd, vh[x] * rv, awv[x]);
        }
        __builtin_amdgcn_sched_barrier(0);  // one quad's weights live at a time
      }
      block_sum<3, NW>(s, red, buf);
      const float rc = rv * ((rv * rv) * (s[0] * inv_d));  // rrms_v c1
      const float dal = s[1] - rc * s[2];
      float ov[kCols];
#pragma unroll
      for (int x = 0; x < kCols; ++x) ov[x] = a * fmaf(-rc, vh[x], A[x]);
      const int64_t o = (int64_t)t * d;
      st8(dV + o + c0, pack4(ov));
      st8(dV + o + c1, pack4(ov + 4));
      if (j == 0) ds_out[t] = (dal * a) * (1.0f - a);
    }
    if (++tpos == T) tpos = 0;
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  const int end = r1 + (kTaps - 1);
  int tau = rb;
  for (; tau + 3 < end; tau += 4) {
    step(tau, I0{});
    step(tau + 1, I1{});
    step(tau + 2, I2{});
    step(tau + 3, I3{});
  }
  if (tau < end) step(tau, I0{});
  if (tau + 1 < end) step(tau + 1, I1{});
  if (tau + 2 < end) step(tau + 2, I2{});

  // this workgroup's partials: rows 1 (rms_w_v) and 2..5 (conv_w) of its [6][d] block
  float* p = partial + (int64_t)blockIdx.x * 6 * d;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int cq = q ? c1 : c0;
    *reinterpret_cast<f32x4*>(p + d + cq) = f32x4{awv[4 * q], awv[4 * q + 1], awv[4 * q + 2], awv[4 * q + 3]};
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<f32x4*>(p + (2 + i) * d + cq) =
          f32x4{acw[i][4 * q], acw[i][4 * q + 1], acw[i][4 * q + 2], acw[i][4 * q + 3]};
    *reinterpret_cast<f32x4*>(p + 4 * d + cq) = *reinterpret_cast<const f32x4*>(lacw + cq);
    *reinterpret_cast<f32x4*>(p + 5 * d + cq) = *reinterpret_cast<const f32x4*>(lacw + d + cq);
  }
}

// Raw bf16 of one row's H and k quads for one thread.
struct HkSlot {
  u32x2 h[2], k[2];
};

// H/k kernel: rows [r0, r1) of the chunk, no halo.  With ds from the conv
// kernel, g = ds rrms_h rrms_k / sqrt(d) and P = sum H k w_h^2:
//   dH = g (w_h^2 k - H rrms_h^2 P / d),  dk = g (w_h^2 H - k rrms_k^2 P / d),
//   drms_w_h += 2 g w_h H k.
// Loads run three rows ahead in three slots, as in the forward.
template <int NW>
__global__ void __launch_bounds__(64 * NW)
gateconv_bwd_hk_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ K, const float* __restrict__ wh,
                       const float* __restrict__ ds_in, const float* __restrict__ rrh, const float* __restrict__ rrk,
                       uint16_t* __restrict__ dH, uint16_t* __restrict__ dK, float* __restrict__ partial, int rows,
                       int chunk) {
  constexpr int d = NW * 512;
  __shared__ float red[2][kMaxWaves][4];
  const int j = threadIdx.x;
  const int c0 = 4 * j, c1 = 4 * j + d / 2;
  const int r0 = blockIdx.x * chunk;
  const int r1 = min(r0 + chunk, rows);
  constexpr float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = __builtin_amdgcn_rsqf((float)d);
  float w[kCols], awh[kCols];
  {
    const f32x4 a = *reinterpret_cast<const f32x4*>(wh + c0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(wh + c1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = a[e];
      w[4 + e] = b[e];
    }
  }
#pragma unroll
  for (int e = 0; e < kCols; ++e) awh[e] = 0.f;
  __builtin_amdgcn_s_waitcnt(0);

  auto issue = [&](HkSlot& sl, int row) {
    const int64_t o = (int64_t)row * d;
    sl.h[0] = ld8(H + o + c0);
    sl.k[0] = ld8(K + o + c0);
    sl.h[1] = ld8(H + o + c1);
    sl.k[1] = ld8(K + o + c1);
  };
  HkSlot sa, sb, sc;
  issue(sa, r0);
  issue(sb, min(r0 + 1, r1 - 1));
  issue(sc, min(r0 + 2, r1 - 1));
  int buf = 0;

  auto step = [&](int r, HkSlot& sl) {
    float h[kCols], k[kCols];
    unpack4(sl.h[0], h);
    unpack4(sl.h[1], h + 4);
    unpack4(sl.k[0], k);
    unpack4(sl.k[1], k + 4);
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      pin(h[e]);
      pin(k[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(sl, min(r + 3, r1 - 1));
    float s[1];
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      const float pe = (h[e] * k[e]) * (w[e] * w[e]);
      s[0] = e == 0 ? pe : s[0] + pe;
    }
    block_sum<1, NW>(s, red, buf);
    const float rh = rrh[r], rk = rrk[r];
    const float gg = ((ds_in[r] * rh) * rk) * inv_sqrt_d;
    const float ph = (rh * rh) * (s[0] * inv_d), pk = (rk * rk) * (s[0] * inv_d);
    float oh[kCols], ok[kCols];
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      const float w2 = w[e] * w[e];
      oh[e] = gg * fmaf(w2, k[e], -h[e] * ph);
      ok[e] = gg * fmaf(w2, h[e], -k[e] * pk);
      awh[e] = fmaf(2.0f * gg * w[e], h[e] * k[e], awh[e]);
    }
    const int64_t o = (int64_t)r * d;
    st8(dH + o + c0, pack4(oh));
    st8(dK + o + c0, pack4(ok));
    st8(dH + o + c1, pack4(oh + 4));
    st8(dK + o + c1, pack4(ok + 4));
  };
  int r = r0;
  for (; r + 2 < r1; r += 3) {
    step(r, sa);
    step(r + 1, sb);
    step(r + 2, sc);
  }
  if (r < r1) step(r, sa);
  if (r + 1 < r1) step(r + 1, sb);

  // row 0 (rms_w_h) of this workgroup's [6][d] partial block
  float* p = partial + (int64_t)blockIdx.x * 6 * d;
  *reinterpret_cast<f32x4*>(p + c0) = f32x4{awh[0], awh[1], awh[2], awh[3]};
  *reinterpret_cast<f32x4*>(p + c1) = f32x4{awh[4], awh[5], awh[6], awh[7]};
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

int gateconv_chunk(int64_t M, int64_t T, int64_t d) {
  // rows per workgroup.  A CU holds about 12 waves of these kernels (their
  // registers), i.e. 12 / (d/512) workgroups; aim at one round of workgroups
  // over the 256 CUs, with at least 32 rows (the halo costs 3 rows a chunk)
  // and at most 512.  A function of the sizes only, so is the workspace size.
  const int64_t nw = d / 512;
  const int64_t target = 256 * (nw >= 12 ? 1 : 12 / nw);
  int64_t c = (M * T + target - 1) / target;
  c = c < 32 ? 32 : c > 512 ? 512 : c;
  return (int)c;
}

int64_t gateconv_workgroups(int64_t M, int64_t T, int chunk) { return (M * T + chunk - 1) / chunk; }

template <int NW>
static const void* fwd_kernel_for() {
  return reinterpret_cast<const void*>(&gateconv_fwd_kernel<NW>);
}

hipError_t launch_gateconv_fwd(const void* H, const void* K, const void* V, const float* wh, const float* wv,
                               const float* cw, void* Y, void* vhat, float* alpha, float* rrh, float* rrk, float* rrv,
                               int64_t M, int64_t T, int64_t d, float eps, int chunk, hipStream_t stream) {
  static const void* const kernels[kMaxWaves] = {
      fwd_kernel_for<1>(), fwd_kernel_for<2>(), fwd_kernel_for<3>(), fwd_kernel_for<4>(), fwd_kernel_for<5>(),
      fwd_kernel_for<6>(), fwd_kernel_for<7>(), fwd_kernel_for<8>(), fwd_kernel_for<9>(), fwd_kernel_for<10>()};
  const int nw = (int)(d / 512);
  if (d % 512 != 0 || nw < 1 || nw > kMaxWaves) return hipErrorInvalidValue;
  const uint16_t *hp = static_cast<const uint16_t*>(H), *kp = static_cast<const uint16_t*>(K),
                 *vp = static_cast<const uint16_t*>(V);
  uint16_t *yp = static_cast<uint16_t*>(Y), *vhp = static_cast<uint16_t*>(vhat);
  int rows = (int)(M * T), Ti = (int)T, ch = chunk;
  void* args[] = {&hp, &kp, &vp, &wh, &wv, &cw, &yp, &vhp, &alpha, &rrh, &rrk, &rrv, &rows, &Ti, &ch, &eps};
  return hipLaunchKernel(kernels[nw - 1], dim3((unsigned)gateconv_workgroups(M, T, chunk)), dim3((unsigned)(64 * nw)),
                         args, 0, stream);
}

template <int NW>
static const void* bwd_conv_for() {
  return reinterpret_cast<const void*>(&gateconv_bwd_conv_kernel<NW>);
}
template <int NW>
static const void* bwd_hk_for() {
  return reinterpret_cast<const void*>(&gateconv_bwd_hk_kernel<NW>);
}

size_t gateconv_bwd_workspace(int64_t M, int64_t T, int64_t d, int chunk) {
  // [nwg][6][d] fp32 weight-gradient partials, then the per-row ds [M*T]
  return (size_t)gateconv_workgroups(M, T, chunk) * 6 * (size_t)d * sizeof(float) + (size_t)(M * T) * sizeof(float);
}

hipError_t launch_gateconv_bwd(const void* dY, const void* H, const void* K, const void* V, const float* wh,
                               const float* wv, const float* cw, const void* vhat, const float* alpha, const float* rrh,
                               const float* rrk, const float* rrv, void* dH, void* dK, void* dV, float* dwh, float* dwv,
                               float* dcw, void* workspace, int64_t M, int64_t T, int64_t d, int chunk,
                               hipStream_t stream) {
  static const void* const conv[kMaxWaves] = {bwd_conv_for<1>(), bwd_conv_for<2>(), bwd_conv_for<3>(),
                                              bwd_conv_for<4>(), bwd_conv_for<5>(), bwd_conv_for<6>(),
                                              bwd_conv_for<7>(), bwd_conv_for<8>(), bwd_conv_for<9>(),
                                              bwd_conv_for<10>()};
  static const void* const hk[kMaxWaves] = {bwd_hk_for<1>(), bwd_hk_for<2>(), bwd_hk_for<3>(), bwd_hk_for<4>(),
                                            bwd_hk_for<5>(), bwd_hk_for<6>(), bwd_hk_for<7>(), bwd_hk_for<8>(),
                                            bwd_hk_for<9>(), bwd_hk_for<10>()};
  const int nw = (int)(d / 512);
  if (d % 512 != 0 || nw < 1 || nw > kMaxWaves) return hipErrorInvalidValue;
  const uint16_t *gp = static_cast<const uint16_t*>(dY), *hp = static_cast<const uint16_t*>(H),
                 *kp = static_cast<const uint16_t*>(K), *vp = static_cast<const uint16_t*>(V),
                 *vhp = static_cast<const uint16_t*>(vhat);
  uint16_t *dhp = static_cast<uint16_t*>(dH), *dkp = static_cast<uint16_t*>(dK), *dvp = static_cast<uint16_t*>(dV);
  const int64_t nwg = gateconv_workgroups(M, T, chunk);
  float* partial = static_cast<float*>(workspace);
  float* ds = partial + nwg * 6 * d;
  int rows = (int)(M * T), Ti = (int)T, di = (int)d, ch = chunk;
  void* a1[] = {&gp, &vp, &wv, &cw, &vhp, &alpha, &rrv, &dvp, &ds, &partial, &rows, &Ti, &ch};
  hipError_t e = hipLaunchKernel(conv[nw - 1], dim3((unsigned)nwg), dim3((unsigned)(64 * nw)), a1, 0, stream);
  if (e != hipSuccess) return e;
  const float* dsc = ds;
  void* a2[] = {&hp, &kp, &wh, &dsc, &rrh, &rrk, &dhp, &dkp, &partial, &rows, &ch};
  e = hipLaunchKernel(hk[nw - 1], dim3((unsigned)nwg), dim3((unsigned)(64 * nw)), a2, 0, stream);
  if (e != hipSuccess) return e;
  const float* cp = partial;
  int nwi = (int)nwg;
  void* a3[] = {&cp, &dwh, &dwv, &dcw, &nwi, &di};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gateconv_reduce_kernel),
                         dim3((unsigned)((6 * d / 4 + 31) / 32)), dim3(256), a3, 0, stream);
}

}  // namespace engram
