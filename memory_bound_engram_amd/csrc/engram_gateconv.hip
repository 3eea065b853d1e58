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
// (dw_v is formed as sum_i conv_w[i] sum_t dc_t u_{t-3+i} / w_v: the same
// products, regrouped; see the reduce kernel).
//
// Mapping.  A workgroup owns whole token rows and walks a chunk of consecutive
// rows of the flattened [M*T] token order (a chunk may cross into the next
// sequence; the conv history restarts there).  The conv couples neighbouring
// tokens, so each chunk recomputes a 3-row halo instead of storing
// intermediates.  Each thread covers C columns of a row (the column map
// below): d = 5120 runs 512 threads x 10 columns (an octet and a pair), so
// the workgroup is a power of two and each thread has 256 VGPRs; other widths
// run d/8 threads x 8 columns (one octet), except the backward at d = 512,
// 1024 and 1536 (d/2 threads x 2 columns, one pair), at d = 2560 (256
// threads x 10 columns) and at d = 4608 (512 threads x 9 columns).  Row sums reduce with
// DPP inside each wave and across waves through LDS, in a fixed order.
// Weight gradients are per-workgroup fp32 partials in the workspace, summed
// by one last kernel (two above 512 workgroups) in a fixed order.
#include "engram_device.h"
#include "engram_launch.h"

#include <type_traits>

namespace engram {
namespace {

constexpr int kTaps = 4;
constexpr int kMaxWaves = 16;   // waves of a workgroup (the cross-wave sum adds 16 lanes)
constexpr int kMaxWidths = 10;  // widths d = 512 ... 5120
constexpr int kPartRows = 1 + kTaps;  // weight-gradient partial rows per workgroup: rms_w_h, conv_w taps

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Column map of a workgroup of THREADS threads, each covering C columns of a
// d = THREADS * C row: C/8 octets of 8 consecutive columns (octet o of thread
// j starts at 8j + 8 THREADS o: 16-byte accesses, one wave instruction moves
// 1 KB contiguous of bf16) and, when C % 8 == 2, one pair of 2 columns
// starting at 8 THREADS (C/8) + 2j (256 contiguous bytes per wave
// instruction), or, when C % 8 == 1, one single column at 8 THREADS (C/8) + j
// (128 contiguous bytes per wave instruction).  Element x < C of a thread is
// element x % 8 of octet x / 8, or element x - 8 NO of the pair or single.  Wide accesses keep the vector-memory
// instructions per row few: a workgroup can have at most 63 of them in flight
// per wave, and the row prefetch needs that headroom.
template <int THREADS_, int C_>
struct ColMap {
  static constexpr int THREADS = THREADS_, C = C_, d = THREADS_ * C_;
  static constexpr int NO = C_ / 8;
  static constexpr bool PAIR = (C_ % 8) == 2;
  static constexpr bool SINGLE = (C_ % 8) == 1;
  static constexpr int NW = THREADS_ / 64;
  static_assert(C_ % 8 == 0 || C_ % 8 == 2 || C_ % 8 == 1, "columns per thread: octets and at most one pair or single");
  static_assert(THREADS_ % 64 == 0 && NW >= 1 && NW <= kMaxWaves, "whole waves, at most sixteen");
  __device__ static constexpr int oct_col(int j, int o) { return 8 * j + 8 * THREADS_ * o; }
  __device__ static constexpr int pair_col(int j) { return 8 * THREADS_ * NO + 2 * j; }
  __device__ static constexpr int single_col(int j) { return 8 * THREADS_ * NO + j; }
};

// Raw bf16 of one thread's C columns of one row.
template <class MP>
struct Raw {
  u32x4 o[MP::NO];
  uint32_t p;  // the pair, or the single column in the low half; unused (and dead) otherwise
};

__device__ __forceinline__ uint32_t ld4(const uint16_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }
__device__ __forceinline__ uint32_t ld4_keep(const uint16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ void st4(uint16_t* p, uint32_t v) { __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p)); }

// Loads of one row (`row` points at its first element); KEEP selects normal
// loads (data read again soon, from L2) over streaming ones.
template <class MP, bool KEEP>
__device__ __forceinline__ void load_raw(Raw<MP>& r, const uint16_t* row, int j) {
#pragma unroll
  for (int o = 0; o < MP::NO; ++o) r.o[o] = KEEP ? load16(row + MP::oct_col(j, o)) : load16_stream(row + MP::oct_col(j, o));
  if constexpr (MP::PAIR) {
    // a 32-bit byte offset from the row base, so the load takes the base in
    // scalar registers (a column index alone gets a 64-bit vector address)
    const uint16_t* q = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(row) +
                                                          (uint32_t)(2 * MP::pair_col(j)));
    r.p = KEEP ? ld4_keep(q) : ld4(q);
  }
  if constexpr (MP::SINGLE) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(row) +
                                                          (uint32_t)(2 * MP::single_col(j)));
    r.p = KEEP ? (uint32_t)*q : (uint32_t)__builtin_nontemporal_load(q);
  }
}

template <class MP>
__device__ __forceinline__ void unpack_raw(const Raw<MP>& r, float* f) {
#pragma unroll
  for (int o = 0; o < MP::NO; ++o)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[8 * o + 2 * i] = bf_lo(r.o[o][i]);
      f[8 * o + 2 * i + 1] = bf_hi(r.o[o][i]);
    }
  if constexpr (MP::PAIR) {
    f[8 * MP::NO] = bf_lo(r.p);
    f[8 * MP::NO + 1] = bf_hi(r.p);
  }
  if constexpr (MP::SINGLE) f[8 * MP::NO] = bf_lo(r.p);
}

// bf16 round-to-nearest-even stores of one row.
template <class MP>
__device__ __forceinline__ void store_row(uint16_t* row, const float* f, int j) {
#pragma unroll
  for (int o = 0; o < MP::NO; ++o) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[8 * o + 2 * i], f[8 * o + 2 * i + 1]);
    store16_stream(row + MP::oct_col(j, o), w);
  }
  if constexpr (MP::PAIR) st4(row + MP::pair_col(j), pack_bf16x2(f[8 * MP::NO], f[8 * MP::NO + 1]));
  if constexpr (MP::SINGLE)
    __builtin_nontemporal_store((uint16_t)(pack_bf16x2(f[8 * MP::NO], 0.0f) & 0xffffu), row + MP::single_col(j));
}

// fp32 per-column vectors (weights, accumulators) in global memory or LDS.
template <class MP>
__device__ __forceinline__ void load_cols(const float* base, int j, float* f) {
#pragma unroll
  for (int o = 0; o < MP::NO; ++o)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(base + MP::oct_col(j, o) + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) f[8 * o + 4 * h + e] = a[e];
    }
  if constexpr (MP::PAIR) {
    const f32x2 b = *reinterpret_cast<const f32x2*>(base + MP::pair_col(j));
    f[8 * MP::NO] = b[0];
    f[8 * MP::NO + 1] = b[1];
  }
  if constexpr (MP::SINGLE) f[8 * MP::NO] = base[MP::single_col(j)];
}

template <class MP>
__device__ __forceinline__ void store_cols(float* base, int j, const float* f) {
#pragma unroll
  for (int o = 0; o < MP::NO; ++o)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<f32x4*>(base + MP::oct_col(j, o) + 4 * h) =
          f32x4{f[8 * o + 4 * h], f[8 * o + 4 * h + 1], f[8 * o + 4 * h + 2], f[8 * o + 4 * h + 3]};
  if constexpr (MP::PAIR)
    *reinterpret_cast<f32x2*>(base + MP::pair_col(j)) = f32x2{f[8 * MP::NO], f[8 * MP::NO + 1]};
  if constexpr (MP::SINGLE) base[MP::single_col(j)] = f[8 * MP::NO];
}

// Per-thread column vectors kept in LDS (weights the registers cannot hold):
// only thread j reads what thread j wrote, so the layout is free; it is
// plane-major -- plane p holds element group p of every thread, lane j at
// 16 j bytes -- so a wave's ds_read_b128 covers 1 KB contiguous without bank
// conflicts (the column-major layout, lanes 32 bytes apart, conflicts 2-way).
// Planes: octet o half h (4 floats) is plane 2o + h; the pair (or single) is last.
template <class MP>
__device__ __forceinline__ void lds_load(const float* base, int j, float* f) {
#pragma unroll
  for (int o = 0; o < MP::NO; ++o)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 a = reinterpret_cast<const f32x4*>(base + (2 * o + h) * 4 * MP::THREADS)[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) f[8 * o + 4 * h + e] = a[e];
    }
  if constexpr (MP::PAIR) {
    const f32x2 b = reinterpret_cast<const f32x2*>(base + 8 * MP::NO * MP::THREADS)[j];
    f[8 * MP::NO] = b[0];
    f[8 * MP::NO + 1] = b[1];
  }
  if constexpr (MP::SINGLE) f[8 * MP::NO] = base[8 * MP::NO * MP::THREADS + j];
}

template <class MP>
__device__ __forceinline__ void lds_store(float* base, int j, const float* f) {
#pragma unroll
  for (int o = 0; o < MP::NO; ++o)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      reinterpret_cast<f32x4*>(base + (2 * o + h) * 4 * MP::THREADS)[j] =
          f32x4{f[8 * o + 4 * h], f[8 * o + 4 * h + 1], f[8 * o + 4 * h + 2], f[8 * o + 4 * h + 3]};
  if constexpr (MP::PAIR)
    reinterpret_cast<f32x2*>(base + 8 * MP::NO * MP::THREADS)[j] = f32x2{f[8 * MP::NO], f[8 * MP::NO + 1]};
  if constexpr (MP::SINGLE) base[8 * MP::NO * MP::THREADS + j] = f[8 * MP::NO];
}

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
// divide take about twenty, which these kernels pay per element.  Saturates
// to exactly 0 and 1 for large |x|.
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896340736f));
}

// Call f(integral_constant<K>) for K = 0 .. N-1, unrolled at compile time.
template <class F, int... K>
__device__ __forceinline__ void unrolled(F&& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}

using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;
using I2 = std::integral_constant<int, 2>;
using I3 = std::integral_constant<int, 3>;

// ------------------------------------------------------------------ forward

// H, k, v of one row for one thread, loaded ahead of use.
template <class MP>
struct FwdSlot {
  Raw<MP> h, k, v;
};

// Rows of loads in flight per workgroup: with 512-thread workgroups (256
// VGPRs a thread) five, else three (168 VGPRs at ten waves).
template <class MP>
constexpr int fwd_slots() { return MP::THREADS == 512 && MP::C == 10 ? 5 : 3; }

template <class MP>
__global__ void __launch_bounds__(MP::THREADS)
gateconv_fwd_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                    const float* __restrict__ wh, const float* __restrict__ wv, const float* __restrict__ cw,
                    uint16_t* __restrict__ Y, uint16_t* __restrict__ vhat, float* __restrict__ alpha,
                    float* __restrict__ rrh, float* __restrict__ rrk, float* __restrict__ rrv, int rows, int T,
                    int chunk, float eps) {
  constexpr int d = MP::d, C = MP::C;
  __shared__ float red[2][kMaxWaves][4];
  const int j = threadIdx.x;
  const int r0 = blockIdx.x * chunk;
  const int r1 = min(r0 + chunk, rows);
  const int rb = max(r0 - (kTaps - 1), r0 - r0 % T);  // halo rows of the same sequence
  constexpr float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = __builtin_amdgcn_rsqf((float)d);

  float whsq[C], wvv[C], w[kTaps][C];
  load_cols<MP>(wh, j, whsq);
#pragma unroll
  for (int e = 0; e < C; ++e) whsq[e] *= whsq[e];
  load_cols<MP>(wv, j, wvv);
#pragma unroll
  for (int i = 0; i < kTaps; ++i) load_cols<MP>(cw + i * d, j, w[i]);
  // the weights arrive before any row load is issued, so no wait inside the
  // row loop is on their account
  __builtin_amdgcn_s_waitcnt(0);

  // S slots, each refilled with the row S ahead (clamped to the last row)
  // right after it is unpacked; the loop is unrolled by S and every refill is
  // unconditional, so a slot keeps its registers and the loads of the other
  // slots stay in flight.  The u history is a ring of S rows (three of them
  // live) whose slots have fixed roles in each of the S unrolled steps.
  constexpr int S = fwd_slots<MP>();
  float uh[S][C];
#pragma unroll
  for (int i = 0; i < S; ++i)
#pragma unroll
    for (int e = 0; e < C; ++e) uh[i][e] = 0.f;

  auto issue = [&](FwdSlot<MP>& sl, int row) __attribute__((always_inline)) {
    const int64_t o = (int64_t)row * d;
    load_raw<MP, false>(sl.h, H + o, j);
    load_raw<MP, false>(sl.k, K + o, j);
    load_raw<MP, false>(sl.v, V + o, j);
  };
  FwdSlot<MP> slot[S];
  unrolled([&](auto kc) __attribute__((always_inline)) { issue(slot[kc.value], min(rb + kc.value, r1 - 1)); }, std::make_integer_sequence<int, S>{});

  int buf = 0;
  int tpos = rb % T;  // position of the next row in its sequence

  auto step = [&](int r, auto kc) __attribute__((always_inline)) {
    constexpr int k0 = decltype(kc)::value;  // ring slot receiving this row's u (at the end)
    constexpr int k1 = (k0 + S - 1) % S, k2 = (k0 + S - 2) % S, k3 = (k0 + S - 3) % S;  // u of rows r-1, r-2, r-3
    FwdSlot<MP>& sl = slot[k0];
    float h[C], k[C], v[C];
    unpack_raw<MP>(sl.h, h);
    unpack_raw<MP>(sl.k, k);
    unpack_raw<MP>(sl.v, v);
    // the unpacked values are produced here, before the refill: were the
    // unpack moved past it, the slot's old and new contents would need
    // separate registers and a copy at the loop latch that waits for the loads
#pragma unroll
    for (int e = 0; e < C; ++e) {
      pin(h[e]);
      pin(k[e]);
      pin(v[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(sl, min(r + S, r1 - 1));
    if (tpos == 0) {  // a new sequence: zero history
#pragma unroll
      for (int i = 0; i < S; ++i)
#pragma unroll
        for (int e = 0; e < C; ++e) uh[i][e] = 0.f;
    }
    float s[4];  // sum H^2, sum k^2, sum H k w_h^2, sum v^2
    s[0] = h[0] * h[0];
    s[1] = k[0] * k[0];
    s[2] = (h[0] * k[0]) * whsq[0];
    s[3] = v[0] * v[0];
#pragma unroll
    for (int e = 1; e < C; ++e) {
      s[0] = fmaf(h[e], h[e], s[0]);
      s[1] = fmaf(k[e], k[e], s[1]);
      s[2] = fmaf(h[e] * k[e], whsq[e], s[2]);
      s[3] = fmaf(v[e], v[e], s[3]);
    }
    block_sum<4, MP::NW>(s, red, buf);
    const float rh = __builtin_amdgcn_rsqf(s[0] * inv_d + eps);
    const float rk = __builtin_amdgcn_rsqf(s[1] * inv_d + eps);
    const float a = sigmoidf_(((s[2] * rh) * rk) * inv_sqrt_d);
    const float rv = __builtin_amdgcn_rsqf((a * a) * (s[3] * inv_d) + eps);
    float vh[C], u[C];
#pragma unroll
    for (int e = 0; e < C; ++e) {
      vh[e] = a * v[e];
      u[e] = (vh[e] * rv) * wvv[e];
    }
    if (r >= r0) {
      float y[C];
#pragma unroll
      for (int e = 0; e < C; ++e) {
        float c = w[0][e] * uh[k3][e];
        c = fmaf(w[1][e], uh[k2][e], c);
        c = fmaf(w[2][e], uh[k1][e], c);
        c = fmaf(w[3][e], u[e], c);
        y[e] = fmaf(c, sigmoidf_(c), vh[e]);
      }
      const int64_t o = (int64_t)r * d;
      store_row<MP>(Y + o, y, j);
      store_row<MP>(vhat + o, vh, j);
      if (j == 0) {
        alpha[r] = a;
        rrh[r] = rh;
        rrk[r] = rk;
        rrv[r] = rv;
      }
    }
    // with S = 3 the slot of u_{r-3} is this row's: written only now
#pragma unroll
    for (int e = 0; e < C; ++e) uh[k0][e] = u[e];
    if (++tpos == T) tpos = 0;
  };

  int r = rb;
  for (; r + S - 1 < r1; r += S) unrolled([&](auto kc) __attribute__((always_inline)) { step(r + kc.value, kc); }, std::make_integer_sequence<int, S>{});
  unrolled([&](auto kc) __attribute__((always_inline)) {
    if (r + kc.value < r1) step(r + kc.value, kc);
  }, std::make_integer_sequence<int, S - 1>{});
}

// ------------------------------------------------------------------ backward
//
// The backward runs as two kernels that split the tensors between them, so
// each tensor is still read once and each kernel's per-thread state fits the
// register file of a CU that holds one row-wide workgroup:
//   conv kernel: vhat, dY, v -> dv, the per-row ds = dalpha alpha (1 - alpha),
//                and the conv_w gradient partials (against u / w_v, from which
//                the reduce also forms the rms_w_v gradient);
//   h/k kernel:  H, k and the per-row scalars -> dH, dk and the rms_w_h partials
//                (rows dealt round-robin to its workgroups).
//
// Conv kernel.  Row tau = newest row (its vhat and dY give u_tau and dc_tau);
// row t = tau - 3 is finished in the same step (it needs dc of t..t+3).  Loads
// run one step ahead: slot N holds vhat, dY of the next newest row, slot L
// holds v of the next finished row; the finished row's vhat and dY, read three
// steps earlier, come from L2.  The step is unrolled by four, so the u and dc
// histories are rings whose slots have fixed roles in each of the four steps;
// the u ring holds u / w_v = vhat rrms_v.
// LDS holds the combined tap weights W_i = conv_w[i] w_v, read once per step:
// c = sum_i W_i (u / w_v)_{t-3+i} needs no multiply by w_v, and the finished
// row needs w_v du = sum_i W_i dc_{t+3-i} rather than du itself.  With more
// than eight waves (at most 168 VGPRs a thread) the conv_w tap 2 and 3
// gradient accumulators move to LDS too.
template <class MP>
__global__ void __launch_bounds__(MP::THREADS)
gateconv_bwd_conv_kernel(const uint16_t* __restrict__ dY, const uint16_t* __restrict__ V,
                         const float* __restrict__ wv, const float* __restrict__ cw,
                         const uint16_t* __restrict__ vhat, const float* __restrict__ alpha,
                         const float* __restrict__ rrv, uint16_t* __restrict__ dV, float* __restrict__ ds_out,
                         float* __restrict__ partial, int rows, int T, int chunk) {
  constexpr int d = MP::d, C = MP::C;
  // conv_w gradient taps kRegTaps..3 accumulate in LDS when more than eight
  // waves of octet columns leave a thread at most 168 VGPRs (taps 2 and 3, the
  // split with the least spilling; no current map needs it since d = 4608
  // runs 512 x 9); all four stay in registers otherwise
  constexpr int kRegTaps = MP::NW > 8 && MP::C >= 8 ? 2 : kTaps;
  constexpr int kLdsTapPlanes = kTaps - kRegTaps;
  // the combined tap weights W_i = conv_w[i] w_v [4][d] (, taps 2-3 grads [2][d]):
  // c = sum_i W_i (u / w_v)_{t-3+i} and w_v du_t = sum_i W_i dc_{t+3-i} both use them
  __shared__ __align__(16) float lw[(kTaps + kLdsTapPlanes) * d];
  __shared__ float red[2][kMaxWaves][4];
  const float* lW = lw;
  float* lacw = lw + 4 * d;
  const int j = threadIdx.x;
  const int r0 = blockIdx.x * chunk;
  const int r1 = min(r0 + chunk, rows);
  const int rb = max(r0 - (kTaps - 1), r0 - r0 % T);            // halo rows before, same sequence
  const int re = min(r1 + (kTaps - 1), ((r1 - 1) / T + 1) * T);  // rows after, same sequence
  constexpr float inv_d = 1.0f / (float)d;
  {  // this thread's combined tap weights, plane-major (see lds_load)
    float v[C], t[C];
    load_cols<MP>(wv, j, v);
#pragma unroll
    for (int i = 0; i < kTaps; ++i) {
      load_cols<MP>(cw + i * d, j, t);
#pragma unroll
      for (int e = 0; e < C; ++e) t[e] *= v[e];
      lds_store<MP>(lw + i * d, j, t);
    }
  }

  float uh[kTaps][C];   // ring of u / w_v rows (vhat rrms_v)
  float dch[kTaps][C];  // ring of dc rows
  float acw[kTaps][C];  // conv_w gradients against u / w_v (taps from kRegTaps on unused: in LDS)
#pragma unroll
  for (int e = 0; e < C; ++e)
#pragma unroll
    for (int i = 0; i < kTaps; ++i) uh[i][e] = dch[i][e] = acw[i][e] = 0.f;
#pragma unroll
  for (int i = kRegTaps; i < kTaps; ++i) lds_store<MP>(lacw + (i - kRegTaps) * d, j, acw[i]);

  Raw<MP> nv, ng;  // slot N: vhat, dY of the newest row
  Raw<MP> lv;      // slot L: v of the finished row
  auto issue_n = [&](int row) __attribute__((always_inline)) {
    load_raw<MP, true>(nv, vhat + (int64_t)row * d, j);
    load_raw<MP, true>(ng, dY + (int64_t)row * d, j);
  };
  auto issue_l = [&](int row) __attribute__((always_inline)) { load_raw<MP, false>(lv, V + (int64_t)row * d, j); };
  issue_n(rb);
  issue_l(r0);
  __syncthreads();  // weights in LDS

  int buf = 0;
  int tpos = rb % T;  // position of row tau in its sequence

  auto step = [&](int tau, auto kc) __attribute__((always_inline)) {
    constexpr int k0 = decltype(kc)::value;  // ring slot receiving row tau
    constexpr int k1 = (k0 + 1) % 4, k2 = (k0 + 2) % 4, k3 = (k0 + 3) % 4;
    const int t = tau - (kTaps - 1);

    // ---- newest row tau: u_tau, dc_tau and the conv-weight gradient
    // The finished row's vhat and dY (read three steps ago: from L2) are
    // requested first: loads complete in order, so waiting for them later
    // does not also wait for the newest-row loads issued below.
    Raw<MP> fv, fg;
    {
      const int tr = max(t, r0);
      load_raw<MP, false>(fv, vhat + (int64_t)tr * d, j);
      load_raw<MP, false>(fg, dY + (int64_t)tr * d, j);
    }
    float vn[C], gn[C];
    unpack_raw<MP>(nv, vn);
    unpack_raw<MP>(ng, gn);
#pragma unroll
    for (int e = 0; e < C; ++e) {
      pin(vn[e]);
      pin(gn[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_n(min(tau + 1, re - 1));
    if (tpos == 0) {  // a sequence start: no u history
#pragma unroll
      for (int i = 0; i < kTaps; ++i)
#pragma unroll
        for (int e = 0; e < C; ++e) uh[i][e] = 0.f;
    }
    const float rvn = tau < re ? rrv[tau] : 0.f;  // u = 0 past the rows this chunk needs
#pragma unroll
    for (int e = 0; e < C; ++e) uh[k0][e] = vn[e] * rvn;
    // the combined tap weights, for the newest row's c and the finished row's du
    float w0[C], w1[C], w2[C], w3[C];
    lds_load<MP>(lW, j, w0);
    lds_load<MP>(lW + d, j, w1);
    lds_load<MP>(lW + 2 * d, j, w2);
    lds_load<MP>(lW + 3 * d, j, w3);
    if (tau >= r0 && tau < re) {
      float gl[kLdsTapPlanes > 0 ? kLdsTapPlanes : 1][C];  // the LDS-held taps of this step
#pragma unroll
      for (int i = 0; i < kLdsTapPlanes; ++i) lds_load<MP>(lacw + i * d, j, gl[i]);
#pragma unroll
      for (int x = 0; x < C; ++x) {
        float c = w0[x] * uh[k1][x];
        c = fmaf(w1[x], uh[k2][x], c);
        c = fmaf(w2[x], uh[k3][x], c);
        c = fmaf(w3[x], uh[k0][x], c);
        const float sg = sigmoidf_(c);
        const float dc = gn[x] * (sg * fmaf(c, 1.0f - sg, 1.0f));
        dch[k0][x] = dc;
        if (tau < r1) {  // dc of rows past the chunk enter no gradient
          // tap i pairs dc_tau with u of row tau - 3 + i: ring slots k1, k2, k3, k0
          const float up[kTaps] = {uh[k1][x], uh[k2][x], uh[k3][x], uh[k0][x]};
#pragma unroll
          for (int i = 0; i < kTaps; ++i) {
            if (i < kRegTaps)
              acw[i][x] = fmaf(dc, up[i], acw[i][x]);
            else
              gl[i - kRegTaps][x] = fmaf(dc, up[i], gl[i - kRegTaps][x]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kLdsTapPlanes; ++i) lds_store<MP>(lacw + i * d, j, gl[i]);
    } else {
#pragma unroll
      for (int e = 0; e < C; ++e) dch[k0][e] = 0.f;
    }

    // ---- finished row t
    float v[C];
    unpack_raw<MP>(lv, v);
#pragma unroll
    for (int e = 0; e < C; ++e) pin(v[e]);
    __builtin_amdgcn_sched_barrier(0);
    issue_l(min(max(t + 1, r0), r1 - 1));
    if (t >= r0) {  // t < r1 by the loop bound
      const int ahead = T - 1 - t % T;  // rows after t in its sequence
      const float a = alpha[t], rv = rrv[t];
      float vh[C], gy[C];
      unpack_raw<MP>(fv, vh);
      unpack_raw<MP>(fg, gy);
      // w_v du_t = sum_i W_i dc_{t+3-i}; dc of rows past the end of t's
      // sequence count as 0 (they belong to the next sequence).  With
      // A = dY + rrms_v w_v du, dvhat = A - rrms_v c1 vhat (c1 = rrms_v^2 S1 / d):
      //   S1 = sum du w_v vhat,  dalpha = sum A v - rrms_v c1 sum vhat v
      float s[3];
      float A[C], dwu[C];
      if (__builtin_expect(ahead >= 3, 1)) {
#pragma unroll
        for (int x = 0; x < C; ++x) {
          float dd = w3[x] * dch[k1][x];
          dd = fmaf(w2[x], dch[k2][x], dd);
          dd = fmaf(w1[x], dch[k3][x], dd);
          dwu[x] = fmaf(w0[x], dch[k0][x], dd);
        }
      } else {  // the last rows of a sequence (rare): rows past its end are skipped
#pragma unroll
        for (int x = 0; x < C; ++x) {
          float dd = w3[x] * dch[k1][x];
          if (ahead >= 1) dd = fmaf(w2[x], dch[k2][x], dd);
          if (ahead >= 2) dd = fmaf(w1[x], dch[k3][x], dd);
          dwu[x] = dd;
        }
      }
#pragma unroll
      for (int x = 0; x < C; ++x) {
        const float dw = dwu[x];  // w_v du
        A[x] = fmaf(rv, dw, gy[x]);
        const float p0 = dw * vh[x], p1 = A[x] * v[x], p2 = vh[x] * v[x];
        s[0] = x == 0 ? p0 : s[0] + p0;
        s[1] = x == 0 ? p1 : s[1] + p1;
        s[2] = x == 0 ? p2 : s[2] + p2;
      }
      block_sum<3, MP::NW>(s, red, buf);
      const float rc = rv * ((rv * rv) * (s[0] * inv_d));  // rrms_v c1
      const float dal = s[1] - rc * s[2];
      float ov[C];
#pragma unroll
      for (int x = 0; x < C; ++x) ov[x] = a * fmaf(-rc, vh[x], A[x]);
      store_row<MP>(dV + (int64_t)t * d, ov, j);
      if (j == 0) ds_out[t] = (dal * a) * (1.0f - a);
    }
    if (++tpos == T) tpos = 0;
  };

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

  // this workgroup's partials: rows 1..4 (the conv_w taps, against u / w_v) of its [5][d] block
  float* p = partial + (int64_t)blockIdx.x * kPartRows * d;
#pragma unroll
  for (int i = 0; i < kTaps; ++i) {
    if (i < kRegTaps) {
      store_cols<MP>(p + (1 + i) * d, j, acw[i]);
    } else {
      float g[C];
      lds_load<MP>(lacw + (i - kRegTaps) * d, j, g);
      store_cols<MP>(p + (1 + i) * d, j, g);
    }
  }
}

// H and k of one row for one thread.
template <class MP>
struct HkSlot {
  Raw<MP> h, k;
};

// H/k kernel.  Rows are independent here (no conv), so workgroup b takes rows
// b, b + G, b + 2G, ... (G workgroups): all workgroups step through the rows
// together and the chip reads and writes one compact band of the tensors at a
// time, which streams ~20% faster than each workgroup walking its own chunk.
// With ds from the conv kernel, g = ds rrms_h rrms_k / sqrt(d) and
// P = sum H k w_h^2:
//   dH = g (w_h^2 k - H rrms_h^2 P / d),  dk = g (w_h^2 H - k rrms_k^2 P / d),
//   drms_w_h += 2 g w_h H k  (this workgroup's rows; the reduce adds them up).
// Loads run three rows ahead in three slots, as in the forward.
template <class MP>
__global__ void __launch_bounds__(MP::THREADS)
gateconv_bwd_hk_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ K, const float* __restrict__ wh,
                       const float* __restrict__ ds_in, const float* __restrict__ rrh, const float* __restrict__ rrk,
                       uint16_t* __restrict__ dH, uint16_t* __restrict__ dK, float* __restrict__ partial, int rows) {
  constexpr int d = MP::d, C = MP::C;
  __shared__ float red[2][kMaxWaves][4];
  const int j = threadIdx.x;
  // rows blockIdx.x + i * gridDim.x, i < n: the workgroups step through the
  // rows together, so at any moment the chip reads and writes one compact band
  const int G = gridDim.x;
  const int n = (rows - (int)blockIdx.x + G - 1) / G;
  auto row_of = [&](int i) __attribute__((always_inline)) { return (int)blockIdx.x + i * G; };
  constexpr float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = __builtin_amdgcn_rsqf((float)d);
  float w[C], awh[C];
  load_cols<MP>(wh, j, w);
#pragma unroll
  for (int e = 0; e < C; ++e) awh[e] = 0.f;
  __builtin_amdgcn_s_waitcnt(0);

  auto issue = [&](HkSlot<MP>& sl, int row) __attribute__((always_inline)) {
    const int64_t o = (int64_t)row * d;
    load_raw<MP, false>(sl.h, H + o, j);
    load_raw<MP, false>(sl.k, K + o, j);
  };
  HkSlot<MP> sa, sb, sc;
  issue(sa, row_of(0));
  issue(sb, row_of(min(1, n - 1)));
  issue(sc, row_of(min(2, n - 1)));
  int buf = 0;

  auto step = [&](int i, HkSlot<MP>& sl) __attribute__((always_inline)) {
    const int r = row_of(i);
    float h[C], k[C];
    unpack_raw<MP>(sl.h, h);
    unpack_raw<MP>(sl.k, k);
#pragma unroll
    for (int e = 0; e < C; ++e) {
      pin(h[e]);
      pin(k[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(sl, row_of(min(i + 3, n - 1)));
    float s[1];
#pragma unroll
    for (int e = 0; e < C; ++e) {
      const float pe = (h[e] * k[e]) * (w[e] * w[e]);
      s[0] = e == 0 ? pe : s[0] + pe;
    }
    block_sum<1, MP::NW>(s, red, buf);
    const float rh = rrh[r], rk = rrk[r];
    const float gg = ((ds_in[r] * rh) * rk) * inv_sqrt_d;
    const float ph = (rh * rh) * (s[0] * inv_d), pk = (rk * rk) * (s[0] * inv_d);
    float oh[C], ok[C];
#pragma unroll
    for (int e = 0; e < C; ++e) {
      const float w2 = w[e] * w[e];
      oh[e] = gg * fmaf(w2, k[e], -h[e] * ph);
      ok[e] = gg * fmaf(w2, h[e], -k[e] * pk);
      awh[e] = fmaf(2.0f * gg * w[e], h[e] * k[e], awh[e]);
    }
    const int64_t o = (int64_t)r * d;
    store_row<MP>(dH + o, oh, j);
    store_row<MP>(dK + o, ok, j);
  };
  int i = 0;
  for (; i + 2 < n; i += 3) {
    step(i, sa);
    step(i + 1, sb);
    step(i + 2, sc);
  }
  if (i < n) step(i, sa);
  if (i + 1 < n) step(i + 1, sb);

  // row 0 (rms_w_h) of this workgroup's [5][d] partial block
  store_cols<MP>(partial + (int64_t)blockIdx.x * kPartRows * d, j, awh);
}

// Weight gradients from the [nwg][5][d] partials.  Per column x: s_r = sum
// over the workgroups of partial row r (64 contiguous chunks of workgroups,
// each summed sequentially, then the chunk sums in the fixed order of
// ordered_sum_rows), then
//   drms_w_h = s_0,   dconv_w[i] = w_v s_{1+i},   drms_w_v = sum_i conv_w[i] s_{1+i}.
// Above 512 workgroups the partials first go through
// gateconv_reduce_rows_kernel, and this kernel sums its ceil(nwg / 64) rows.
// The last line is the rms_w_v gradient sum_t du_t u_t / w_v regrouped: with
// du_t = sum_i conv_w[i] dc_{t+3-i}, both sides add conv_w[i] dc_tau u_t / w_v
// over the same pairs (t, tau = t + 3 - i) of rows of one sequence.
constexpr int kRedChunks = 64, kRedGroups = 8;
constexpr int kRedLanes = kPartRows * kRedGroups;  // (partial row, column group) pairs of a workgroup
constexpr int kRedRuns = 8, kRedRunLen = kRedChunks / kRedRuns;
// Above this many partial rows per thread of gateconv_reduce_kernel (above
// 512 workgroups) the sum runs in two levels.  Each kernel of it costs ~4 us
// however little it reads, so one level is as fast up to 8 rows per thread
// (d = 2048 and up at M T = 16384) and two are faster above: d = 512 and 1024
// have 1024 workgroups and d/32 = 16 or 32 reduce workgroups, which took
// 12.6 and 13.5 us for the partials alone.
constexpr int kRedTwoLevelRows = 8;

typedef f32x4 RedRows[kRedChunks][kPartRows][kRedGroups];
typedef f32x4 RedRuns[kRedRuns][kPartRows][kRedGroups];

// Sum over k of part[k][r][g] for every (r, g), in a fixed order: eight runs
// of eight consecutive k, each added in k order, then the run sums in run
// order.  Each run's rows are read into registers before they are added, so
// a thread has eight LDS reads in flight instead of the compiler's two.  Every
// thread of the workgroup calls it (it holds a barrier); thread r * 8 + g
// (< 40) gets the sum of (r, g).
__device__ __forceinline__ f32x4 ordered_sum_rows(const RedRows& part, RedRuns& runs) {
  const int tid = threadIdx.x;
  if (tid < kRedRuns * kRedLanes) {
    const int h = tid / kRedLanes, r = tid % kRedLanes / kRedGroups, g = tid % kRedGroups;
    f32x4 v[kRedRunLen];
#pragma unroll
    for (int k = 0; k < kRedRunLen; ++k) v[k] = part[h * kRedRunLen + k][r][g];
    f32x4 t = v[0];
#pragma unroll
    for (int k = 1; k < kRedRunLen; ++k) t += v[k];
    runs[h][r][g] = t;
  }
  __syncthreads();
  f32x4 t = {};
  if (tid < kRedLanes) {
    const int r = tid / kRedGroups, g = tid % kRedGroups;
    f32x4 v[kRedRuns];
#pragma unroll
    for (int h = 0; h < kRedRuns; ++h) v[h] = runs[h][r][g];
    t = v[0];
#pragma unroll
    for (int h = 1; h < kRedRuns; ++h) t += v[h];
  }
  return t;
}

__global__ void __launch_bounds__(kRedChunks * kRedGroups)
gateconv_reduce_kernel(const float* __restrict__ partial, const float* __restrict__ wv, const float* __restrict__ cw,
                       float* __restrict__ dwh, float* __restrict__ dwv, float* __restrict__ dcw, int nwg, int d) {
  __shared__ RedRows part;
  __shared__ RedRuns runs;
  __shared__ f32x4 tot[kPartRows][kRedGroups];
  const int g = threadIdx.x % kRedGroups, q = threadIdx.x / kRedGroups;
  const int c4 = blockIdx.x * kRedGroups + g;  // float4 column; the grid covers d/4 exactly
  const int ncol4 = d / 4;
  const int b0 = (int)((int64_t)nwg * q / kRedChunks), b1 = (int)((int64_t)nwg * (q + 1) / kRedChunks);
  const f32x4* p4 = reinterpret_cast<const f32x4*>(partial);
  // the weights of the final step, requested before the sums so that their
  // latency overlaps them
  f32x4 w = {}, c[kTaps] = {};
  if (q == 0) {
    w = reinterpret_cast<const f32x4*>(wv)[c4];
#pragma unroll
    for (int i = 0; i < kTaps; ++i) c[i] = reinterpret_cast<const f32x4*>(cw)[i * ncol4 + c4];
  }
  // -0 is the exact identity of IEEE addition (x + -0 = x for every x, +0
  // and -0 included), so empty chunks and the start of each sum change nothing
  f32x4 s[kPartRows];
#pragma unroll
  for (int r = 0; r < kPartRows; ++r) s[r] = f32x4{-0.f, -0.f, -0.f, -0.f};
#pragma unroll 8
  for (int b = b0; b < b1; ++b)
#pragma unroll
    for (int r = 0; r < kPartRows; ++r) s[r] += p4[((int64_t)b * kPartRows + r) * ncol4 + c4];
#pragma unroll
  for (int r = 0; r < kPartRows; ++r) part[q][r][g] = s[r];
  __syncthreads();
  const f32x4 t = ordered_sum_rows(part, runs);  // the chunk sums, in a fixed order
  if (threadIdx.x < kRedLanes) tot[threadIdx.x / kRedGroups][threadIdx.x % kRedGroups] = t;
  __syncthreads();
  if (q == 0) {
    reinterpret_cast<f32x4*>(dwh)[c4] = tot[0][g];
    f32x4 v = c[0] * tot[1][g];
#pragma unroll
    for (int i = 0; i < kTaps; ++i) {
      reinterpret_cast<f32x4*>(dcw)[i * ncol4 + c4] = w * tot[1 + i][g];
      if (i > 0) v += c[i] * tot[1 + i][g];
    }
    reinterpret_cast<f32x4*>(dwv)[c4] = v;
  }
}

// First level of the weight-gradient sum above 512 workgroups: workgroup
// (x, p) adds the [5][32 columns] blocks of partial rows 64 p ... 64 p + 63
// (fewer in the last) in the fixed order of ordered_sum_rows and writes them
// as row p of `sums`
// ([ceil(nwg / 64)][5][d]).  One thread loads one 16-byte column group of
// one partial row, so the whole [nwg][5][d] array is read at once by
// d/32 x ceil(nwg / 64) workgroups; summed by gateconv_reduce_kernel
// alone, d/32 workgroups (16 at d = 512) read it all and the sum took a
// fifth of the backward at the narrowest widths.
__global__ void __launch_bounds__(kRedChunks * kRedGroups)
gateconv_reduce_rows_kernel(const float* __restrict__ partial, float* __restrict__ sums, int nwg, int d) {
  __shared__ RedRows part;
  __shared__ RedRuns runs;
  const int g = threadIdx.x % kRedGroups, q = threadIdx.x / kRedGroups;
  const int ncol4 = d / 4;
  const int b0 = blockIdx.y * kRedChunks;
  const int nb = nwg - b0 < kRedChunks ? nwg - b0 : kRedChunks;  // rows of this block, >= 1
  const f32x4* p4 = reinterpret_cast<const f32x4*>(partial);
#pragma unroll
  for (int r = 0; r < kPartRows; ++r)  // rows past the last are -0, the exact identity of addition
    part[q][r][g] = q < nb ? p4[((int64_t)(b0 + q) * kPartRows + r) * ncol4 + blockIdx.x * kRedGroups + g]
                           : f32x4{-0.f, -0.f, -0.f, -0.f};
  __syncthreads();
  const f32x4 t = ordered_sum_rows(part, runs);
  if (threadIdx.x < kRedLanes) {  // (partial row r, column group h) of this workgroup
    const int r = threadIdx.x / kRedGroups, h = threadIdx.x % kRedGroups;
    reinterpret_cast<f32x4*>(sums)[((int64_t)blockIdx.y * kPartRows + r) * ncol4 + blockIdx.x * kRedGroups + h] = t;
  }
}

// The column map for width d = 512 nw: 512 threads x 10 columns for d = 5120,
// else 64 nw threads x 8 columns.  The backward of the three narrowest widths
// runs 256 nw threads x 2 columns instead: four times the waves for rows of
// only 1-3 KB, where one wave per 512 columns leaves the CUs with too few
// waves to hide the latency of each row step (14% faster at d = 512 and 1024;
// the forward gains nothing from it).  The backward at d = 4608 runs 512
// threads x 9 columns (an octet and a single column): nine waves of 8 columns
// would leave a thread 168 VGPRs, which the conv kernel's rings and
// accumulators do not fit without spilling.  The backward at d = 2560 runs
// 256 threads x 10 columns (the d = 5120 map at half the threads): as five
// waves of 8 columns one workgroup filled 5 of the 8 wave slots a CU has for
// the conv kernel; as four waves two workgroups fill all 8, on 32-row chunks
// (gateconv_chunk), and the backward runs 17-19% faster (cold).
template <int NW>
using MapFor = std::conditional_t<NW == 10, ColMap<512, 10>, ColMap<64 * NW, 8>>;
template <int NW>
using BwdMapFor = std::conditional_t<
    NW <= 3, ColMap<256 * NW, 2>,
    std::conditional_t<NW == 9, ColMap<512, 9>, std::conditional_t<NW == 5, ColMap<256, 10>, MapFor<NW>>>>;

struct Kernels {
  const void* fwd;
  const void* conv;
  const void* hk;
  int fwd_threads, bwd_threads;
};

template <int NW>
Kernels kernels_for() {
  using MP = MapFor<NW>;
  using MB = BwdMapFor<NW>;
  return {reinterpret_cast<const void*>(&gateconv_fwd_kernel<MP>),
          reinterpret_cast<const void*>(&gateconv_bwd_conv_kernel<MB>),
          reinterpret_cast<const void*>(&gateconv_bwd_hk_kernel<MB>), MP::THREADS, MB::THREADS};
}

const Kernels* kernels_for_width(int64_t d) {
  static const Kernels table[kMaxWidths] = {kernels_for<1>(), kernels_for<2>(), kernels_for<3>(), kernels_for<4>(),
                                           kernels_for<5>(), kernels_for<6>(), kernels_for<7>(), kernels_for<8>(),
                                           kernels_for<9>(), kernels_for<10>()};
  const int64_t nw = d / 512;
  if (d % 512 != 0 || nw < 1 || nw > kMaxWidths) return nullptr;
  return &table[nw - 1];
}

}  // namespace

int gateconv_chunk(int64_t M, int64_t T, int64_t d, bool bwd) {
  // rows per workgroup.  A CU holds 8 waves of the backward's conv kernel
  // (182-229 VGPRs: two waves per SIMD), i.e. 8 / (d/512) workgroups of d/512
  // waves (at least one); aim at one round of workgroups over the 256 CUs,
  // with at least 32 rows (the halo costs 3 rows a chunk) and at most 512.
  // (Counting 12 waves a CU put d = 2560 and 3072 into two rounds of 32-row
  // chunks, one workgroup per CU at a time: their backward ran at 3.6-4.0
  // TB/s against 4.5 for d = 3584.)  The narrowest widths (d <= 1024) take
  // chunks down to 16 rows: their rows are too short for a workgroup to hide
  // each row step's latency, so more workgroups over the same rows pay for
  // the extra halo
  // (forward 31% faster at d = 512 and 12% at 1024, backward 16% at 512;
  // down to 8 rows, or 16 at d = 2048 as well, measured slower).  A function
  // of the sizes only, so is the workspace size.
  const int64_t nw = d / 512;
  // the backward's maps at d = 1536 (768 x 2: 12 waves of ~64 VGPRs, two
  // workgroups a CU) and d = 2560 (256 x 10: 4 waves, two a CU) count as 4
  const int64_t waves = bwd && (nw == 3 || nw == 5) ? 4 : nw;
  const int64_t target = 256 * (waves >= 8 ? 1 : 8 / waves);
  int64_t c = (M * T + target - 1) / target;
  const int64_t lo = nw <= 2 ? 16 : 32;
  c = c < lo ? lo : c > 512 ? 512 : c;
  return (int)c;
}

int64_t gateconv_workgroups(int64_t M, int64_t T, int chunk) { return (M * T + chunk - 1) / chunk; }

// Rows of the first-level sums of the weight-gradient partials.
static int64_t gateconv_sum_rows(int64_t nwg) { return (nwg + kRedChunks - 1) / kRedChunks; }

size_t gateconv_bwd_workspace(int64_t M, int64_t T, int64_t d, int chunk) {
  // [nwg][5][d] fp32 weight-gradient partials, [ceil(nwg / 64)][5][d] fp32
  // first-level sums of them, then the per-row ds [M*T]
  const int64_t nwg = gateconv_workgroups(M, T, chunk);
  return (size_t)(nwg + gateconv_sum_rows(nwg)) * kPartRows * (size_t)d * sizeof(float) +
         (size_t)(M * T) * sizeof(float);
}

hipError_t launch_gateconv_fwd(const void* H, const void* K, const void* V, const float* wh, const float* wv,
                               const float* cw, void* Y, void* vhat, float* alpha, float* rrh, float* rrk, float* rrv,
                               int64_t M, int64_t T, int64_t d, float eps, int chunk, hipStream_t stream) {
  const Kernels* kn = kernels_for_width(d);
  if (!kn) return hipErrorInvalidValue;
  const uint16_t *hp = static_cast<const uint16_t*>(H), *kp = static_cast<const uint16_t*>(K),
                 *vp = static_cast<const uint16_t*>(V);
  uint16_t *yp = static_cast<uint16_t*>(Y), *vhp = static_cast<uint16_t*>(vhat);
  int rows = (int)(M * T), Ti = (int)T, ch = chunk;
  void* args[] = {&hp, &kp, &vp, &wh, &wv, &cw, &yp, &vhp, &alpha, &rrh, &rrk, &rrv, &rows, &Ti, &ch, &eps};
  return hipLaunchKernel(kn->fwd, dim3((unsigned)gateconv_workgroups(M, T, chunk)), dim3((unsigned)kn->fwd_threads), args,
                         0, stream);
}

hipError_t launch_gateconv_bwd(const void* dY, const void* H, const void* K, const void* V, const float* wh,
                               const float* wv, const float* cw, const void* vhat, const float* alpha, const float* rrh,
                               const float* rrk, const float* rrv, void* dH, void* dK, void* dV, float* dwh, float* dwv,
                               float* dcw, void* workspace, int64_t M, int64_t T, int64_t d, int chunk,
                               hipStream_t stream) {
  const Kernels* kn = kernels_for_width(d);
  if (!kn) return hipErrorInvalidValue;
  const uint16_t *gp = static_cast<const uint16_t*>(dY), *hp = static_cast<const uint16_t*>(H),
                 *kp = static_cast<const uint16_t*>(K), *vp = static_cast<const uint16_t*>(V),
                 *vhp = static_cast<const uint16_t*>(vhat);
  uint16_t *dhp = static_cast<uint16_t*>(dH), *dkp = static_cast<uint16_t*>(dK), *dvp = static_cast<uint16_t*>(dV);
  const int64_t nwg = gateconv_workgroups(M, T, chunk);
  const int64_t nsum = gateconv_sum_rows(nwg);
  float* partial = static_cast<float*>(workspace);
  float* sums = partial + nwg * kPartRows * d;
  float* ds = sums + nsum * kPartRows * d;
  int rows = (int)(M * T), Ti = (int)T, di = (int)d, ch = chunk;
  void* a1[] = {&gp, &vp, &wv, &cw, &vhp, &alpha, &rrv, &dvp, &ds, &partial, &rows, &Ti, &ch};
  hipError_t e = hipLaunchKernel(kn->conv, dim3((unsigned)nwg), dim3((unsigned)kn->bwd_threads), a1, 0, stream);
  if (e != hipSuccess) return e;
  const float* dsc = ds;
  void* a2[] = {&hp, &kp, &wh, &dsc, &rrh, &rrk, &dhp, &dkp, &partial, &rows};
  e = hipLaunchKernel(kn->hk, dim3((unsigned)nwg), dim3((unsigned)kn->bwd_threads), a2, 0, stream);
  if (e != hipSuccess) return e;
  const float* cp = partial;
  int nwi = (int)nwg;
  if (nwg > kRedChunks * kRedTwoLevelRows) {  // first level: blocks of 64 partial rows -> nsum rows
    void* a4[] = {&cp, &sums, &nwi, &di};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&gateconv_reduce_rows_kernel),
                        dim3((unsigned)(d / 4 / kRedGroups), (unsigned)nsum), dim3(kRedChunks * kRedGroups), a4, 0,
                        stream);
    if (e != hipSuccess) return e;
    cp = sums;
    nwi = (int)nsum;
  }
  void* a3[] = {&cp, &wv, &cw, &dwh, &dwv, &dcw, &nwi, &di};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gateconv_reduce_kernel), dim3((unsigned)(d / 4 / kRedGroups)),
                         dim3(kRedChunks * kRedGroups), a3, 0, stream);
}

}  // namespace engram
