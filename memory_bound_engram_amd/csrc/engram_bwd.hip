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
// Kernel 1 (main).  The grad_weight partials come in rows; each row is split
// by stream: workgroup (b, s) owns stream s of row b and writes that quarter
// of the partial row, so no two workgroups write the same bytes.  The four
// stream workgroups of a row share blockIdx % 8 (one XCD, one L2) and walk the
// same tokens in the same order, so the shared value and the grad_out slices
// they all read are fetched from HBM once (normal loads; streaming hints would
// evict them before the sibling workgroups arrive).
// A workgroup is 4 token slots x 2 half-row waves (512 threads): wave (u, h)
// handles slot u's tokens and vectors h + 2i (i = 0..4) of the 640 16-byte
// vectors of a stream row.  Rows and tokens: up to N = 4096 there are N/64
// rows of 64 tokens; above that, when 256 divides N, 64 rows of N/64 tokens,
// so that the 256 workgroups are all resident at once, one per CU (else N/64
// rows, which then run in two rounds of workgroups).  At step
// jj the workgroups of all rows together take band jj, the rows * 4
// consecutive tokens from jj * rows * 4 (slot u of row b: token
// (jj * 4 + u) * rows + b), so the chip walks the tensors front to back.
// Other orders measured on MI355X (bands visited four or eight apart, a
// random band order, a workgroup's slots on consecutive tokens, two rounds of
// 128 rows) came within 1.5% of this one, timed either cold or right after the
// forward on the same buffers.  The dg partials of the two half-row waves of a
// token meet in LDS (one barrier per step).  grad_value for vector pair i (columns
// of vectors 2i, 2i+1) is written by the stream-i workgroup for i < 4 and, for
// i = 4, by one stream workgroup chosen by (step + slot) mod 4, so every element
// is written once and the extra grad_out reads stay balanced.  The weight row
// of stream s sits in LDS.  Each wave accumulates a x k for its vectors over
// its tokens in VGPRs; the slots are added in slot order at the end.  The
// saved row of a slot's next token is fetched a step ahead through the scalar
// cache; the next token's value loads go out as soon as this token's dg sum has
// read the value, and its other loads before this token's stores.
// Where delta is 0 -- a masked token (gate 0) or the clamp path -- grad_x = G,
// grad_key = 0 and there is no grad_weight term, so X, the key and the value
// are not read; for a masked token grad_value is 0 too and the other streams'
// G are not read either.  (With mask Bernoulli(0.3) that removes ~30% of the
// bytes.)
// Kernel 2 (reduce): grad_weight[s][j] = sum over rows of the partials, in a
// fixed order (32 contiguous row chunks summed sequentially, then the chunk
// sums added in chunk order), so the result is bitwise reproducible.  When
// the source norm weights wh, we (weight = wh * we) are given, the same
// kernel also writes their product-rule gradients grad_wh = grad_weight * we
// and grad_we = grad_weight * wh ("tile-kernels 1.0.0" listing,
// test_engram_gate_bwd.py; the gate page leaves this step to the caller).
//
// Workspace layout (size fixed by the workspace paragraph): the first 16*N
// floats are reserved for per-(token, stream) scalars and are unused by this
// implementation; the partials start at float offset 16*N (byte 64*N, which
// keeps 16-byte alignment).
#include <mutex>

#include "engram_device.h"
#include "engram_launch.h"

namespace engram {

constexpr int kBwdVecs = kRowVecs / 128;              // 5 vectors per lane (half a row)

constexpr int kBwdSlots = 4;                          // token slots per workgroup

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// c + a.lo b.lo + a.hi b.hi for two packed bf16 pairs (one v_dot2 instruction;
// each bf16 product is exact in fp32)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// rows = partial rows (workgroups per stream), steps = tokens per slot:
// rows * kBwdSlots * steps = N.
__global__ void __launch_bounds__(64 * 2 * kBwdSlots)
engram_bwd_main_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ kv,
                       const float* __restrict__ weight, const float* __restrict__ saved,
                       const uint16_t* __restrict__ gout, uint16_t* __restrict__ dx,
                       uint16_t* __restrict__ dkv, float* __restrict__ partial, int rows, int steps) {
  // weight row of stream s and the token-slot combine (20 KB each), as two
  // planes: [0][vec] holds columns 8 vec .. 8 vec + 3, [1][vec] the next four,
  // so the lanes of a wave read 16-byte words 16 bytes apart (no LDS bank
  // conflicts; a 32-byte lane stride conflicts 2-way)
  __shared__ f32x4 wrow[2][kRowVecs];
  __shared__ f32x4 comb[2][kRowVecs];
  constexpr int kBwdThreads = 64 * 2 * kBwdSlots;       // 2 half-row waves per slot
  __shared__ float red[2][kBwdSlots][2];    // dg partials of the half-row waves
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int u = wave >> 1, h = wave & 1;
  // XCD-aware: blockIdx = 32 q + 8 s + r  ->  row b = 8 q + r, stream s
  const int bi = blockIdx.x;
  const int r = bi & 7, s = (bi >> 3) & 3;
  const int64_t b = (int64_t)(bi >> 5) * 8 + r;
  if (b >= rows) return;  // rows are padded to a multiple of 8

  // The stream's weight row is loaded first and written to LDS only after the
  // first token's loads have been issued (below): the wait for it then leaves
  // those in flight, and the kernel's start pays one memory latency, not two.
  constexpr int kWeightLoads = (kHidden / 4 + kBwdThreads - 1) / kBwdThreads;
  f32x4 wt[kWeightLoads];
#pragma unroll
  for (int q = 0; q < kWeightLoads; ++q) {
    const int j = threadIdx.x + q * kBwdThreads;
    if (j < kHidden / 4) wt[q] = reinterpret_cast<const f32x4*>(weight + s * kHidden)[j];
  }

  // the saved row (gate, dot, rstd_X, rstd_key of each stream; 64 bytes) of
  // this slot's next token, fetched one token ahead through the scalar cache
  // (the token index is wave-uniform), so no wait on it stalls the vector loads
  // At step jj the workgroups of all rows together take the band of
  // rows * kBwdSlots consecutive tokens from jj * rows * kBwdSlots: slot u of
  // row b the token (jj * kBwdSlots + u) * rows + b.
  auto token = [&](int jj) { return __builtin_amdgcn_readfirstlane((jj * kBwdSlots + u) * rows + (int)b); };
  const f32x4* saved4 = reinterpret_cast<const f32x4*>(saved);
  f32x4 svn[kStreams];
  {
    const int t0 = token(0);
#pragma unroll
    for (int so = 0; so < kStreams; ++so) svn[so] = saved4[t0 * kStreams + so];
  }

  // Per token, a wave loads (all before any use): its grad_out half-row G and,
  // where delta != 0, the value, X and key half-rows; where grad_value is not
  // all zero, the other streams' G at the vector pair(s) whose grad_value this
  // workgroup writes.  The loop is software-pipelined on the memory side: the
  // next token's value loads go out as soon as this token's dg sum has read
  // the value; then token jj's outputs are computed into registers, token
  // jj + 1's other loads are issued, then token jj's stores -- so the loads of
  // the next token go out ahead of the stores of this one, and the stores
  // overlap their latency.
  struct Loads {
    u32x4 g[kBwdVecs], v[kBwdVecs], x[kBwdVecs], k[kBwdVecs], go[2][kStreams];
  };
  struct Flags {
    bool live, dv_zero, dv_tail;
  };
  auto flags_of = [&](const f32x4* svr, int kk) {
    const f32x4 own = s == 0 ? svr[0] : s == 1 ? svr[1] : s == 2 ? svr[2] : svr[3];
    Flags f;
    // delta is 0 for a masked token (gate 0) and on the clamp path: then
    // grad_x = G, grad_key = 0 and no grad_weight term, so X, the key and the
    // value (needed only for dg) are not read.  A masked token's grad_value is
    // 0 as well (every stream's gate is 0): the other streams' G are not read.
    f.live = own[0] != 0.0f && fabsf(own[1]) >= kClamp;
    f.dv_zero = svr[0][0] == 0.0f && svr[1][0] == 0.0f && svr[2][0] == 0.0f && svr[3][0] == 0.0f;
    f.dv_tail = ((kk + u) & 3) == s;  // this workgroup also writes vector pair 4 (rotating over steps and slots)
    return f;
  };
  auto issue_v = [&](Loads& L, int64_t t) __attribute__((always_inline)) {
    const uint16_t* kt = kv + t * kKvCols;
#pragma unroll
    for (int v = 0; v < kBwdVecs; ++v) L.v[v] = load16(kt + kValueCol + (lane + 64 * (h + 2 * v)) * kVec);
  };
  auto issue = [&](Loads& L, int64_t t, const Flags& f, bool with_v) __attribute__((always_inline)) {
    const uint16_t* gt = gout + t * (kStreams * kHidden);
    const uint16_t* xs = x + t * (kStreams * kHidden) + s * kHidden;
    const uint16_t* kt = kv + t * kKvCols;
#pragma unroll
    for (int v = 0; v < kBwdVecs; ++v) L.g[v] = load16(gt + s * kHidden + (lane + 64 * (h + 2 * v)) * kVec);
    if (f.live) {
      if (with_v) issue_v(L, t);
#pragma unroll
      for (int v = 0; v < kBwdVecs; ++v) {
        const int col = (lane + 64 * (h + 2 * v)) * kVec;
        L.x[v] = load16_stream(xs + col);
        L.k[v] = load16_stream(kt + s * kHidden + col);
      }
    }
    if (!f.dv_zero) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m == 1 && !f.dv_tail) continue;
        const int col = (lane + 64 * (h + 2 * (m == 0 ? s : 4))) * kVec;
#pragma unroll
        for (int so = 0; so < kStreams; ++so)
          if (so != s) L.go[m][so] = load16(gt + so * kHidden + col);
      }
    }
  };

  int buf = 0;
  Loads L;
  f32x4 sv[kStreams];
#pragma unroll
  for (int so = 0; so < kStreams; ++so) sv[so] = svn[so];
  Flags fl = flags_of(sv, 0);
  issue(L, token(0), fl, true);
#pragma unroll
  for (int q = 0; q < kWeightLoads; ++q) {
    const int j = threadIdx.x + q * kBwdThreads;
    if (j < kHidden / 4) wrow[j & 1][j >> 1] = wt[q];
  }
  float acc[kBwdVecs][kVec];
#pragma unroll
  for (int v = 0; v < kBwdVecs; ++v)
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[v][e] = 0.f;
  __syncthreads();  // the weight row in LDS
  for (int jj = 0; jj < steps; ++jj) {
    const int64_t t = token(jj);
    const bool more = jj + 1 < steps;
    {  // the saved row of the next token (scalar loads)
      const int tn = token(more ? jj + 1 : jj);
#pragma unroll
      for (int so = 0; so < kStreams; ++so) svn[so] = saved4[tn * kStreams + so];
    }
    const f32x4 own = s == 0 ? sv[0] : s == 1 ? sv[1] : s == 2 ? sv[2] : sv[3];
    const float g = own[0], dot = own[1];
    const float rx = own[2], rk = own[3];

    // this lane's part of dg = sum_j G_j v_j, on the packed bf16 pairs, in two
    // independent chains
    float p0 = 0.f, p1 = 0.f;
    if (fl.live) {
#pragma unroll
      for (int v = 0; v < kBwdVecs; ++v)
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
          p0 = dot2_bf16(L.g[v][q], L.v[v][q], p0);
          p1 = dot2_bf16(L.g[v][q + 1], L.v[v][q + 1], p1);
        }
    }
    // the value is needed only for dg: its registers are free now, so the next
    // token's value loads go out here, ahead of the barrier and the outputs
    // (1-2% faster than with the rest of its loads)
    if (more && flags_of(svn, jj + 1).live) issue_v(L, token(jj + 1));
    float p = wave_sum_to_lane63(p0 + p1);
    if (lane == 63) red[buf][u][h] = p;
    __syncthreads();
    const float dg = red[buf][u][0] + red[buf][u][1];
    buf ^= 1;  // the next pair writes the other buffer: one barrier per pair suffices

    const float dz = dg * g * (1.0f - g);
    const float ad = fabsf(dot);
    const float delta = ad >= kClamp ? dz / (2.0f * sqrtf(ad)) : 0.0f;
    const float dr = delta * rx;
    const float ca = dr * rk;
    const float cb = dr * rx * (dot / (float)kHidden);
    const float ce = delta * rk * rk * (dot / (float)kHidden);

    // this token's outputs, packed: grad_x, grad_key, and grad_value at up to two vector pairs
    u32x4 ox[kBwdVecs], ok[kBwdVecs], ov[2];
    if (!fl.live) {
#pragma unroll
      for (int v = 0; v < kBwdVecs; ++v) {
        ox[v] = L.g[v];
        ok[v] = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int v = 0; v < kBwdVecs; ++v) {
        const int vec = lane + 64 * (h + 2 * v);
        const f32x4 w0 = wrow[0][vec], w1 = wrow[1][vec];
        const float wv[kVec] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float rdx[2], rdk[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int e = 2 * q + hh;
            const float gx = hh ? bf_hi(L.g[v][q]) : bf_lo(L.g[v][q]);
            const float xx = hh ? bf_hi(L.x[v][q]) : bf_lo(L.x[v][q]);
            const float kk = hh ? bf_hi(L.k[v][q]) : bf_lo(L.k[v][q]);
            const float cw = ca * wv[e];  // a w_j, shared by grad_x and grad_key
            rdx[hh] = fmaf(-cb, xx, fmaf(cw, kk, gx));
            rdk[hh] = fmaf(-ce, kk, cw * xx);
            acc[v][e] = fmaf(ca, xx * kk, acc[v][e]);
          }
          ox[v][q] = pack_bf16x2(rdx[0], rdx[1]);
          ok[v][q] = pack_bf16x2(rdk[0], rdk[1]);
        }
      }
    }
    // grad_value = sum over streams (order 0..3) of gate_s G_s, one bf16 cast
    float gh[kStreams];
#pragma unroll
    for (int so = 0; so < kStreams; ++so) gh[so] = sv[so][0];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      ov[m] = u32x4{0u, 0u, 0u, 0u};
      if (fl.dv_zero || (m == 1 && !fl.dv_tail)) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // this wave's own stream: vector slot s (m == 0) or 4 (m == 1), selected without
        // dynamic register indexing
        const uint32_t ownw =
            m == 1 ? L.g[4][q] : s == 0 ? L.g[0][q] : s == 1 ? L.g[1][q] : s == 2 ? L.g[2][q] : L.g[3][q];
        float d2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float a = 0.f;
#pragma unroll
          for (int so = 0; so < kStreams; ++so) {
            const uint32_t wd = so == s ? ownw : L.go[m][so][q];
            const float gv = hh ? bf_hi(wd) : bf_lo(wd);
            a = so == 0 ? gh[0] * gv : fmaf(gh[so], gv, a);
          }
          d2[hh] = a;
        }
        ov[m][q] = pack_bf16x2(d2[0], d2[1]);
      }
    }
    const Flags fo = fl;  // this token's flags, for its stores

    // the next token's loads go out before this token's stores
    if (more) {
#pragma unroll
      for (int so = 0; so < kStreams; ++so) sv[so] = svn[so];
      fl = flags_of(sv, jj + 1);
      issue(L, token(jj + 1), fl, false);
    }
    __builtin_amdgcn_sched_barrier(0);

    uint16_t* dxs = dx + t * (kStreams * kHidden) + s * kHidden;
    uint16_t* dkt = dkv + t * kKvCols;
#pragma unroll
    for (int v = 0; v < kBwdVecs; ++v) {
      const int vec = lane + 64 * (h + 2 * v);
      store16_stream(dxs + vec * kVec, ox[v]);
      store16_stream(dkt + s * kHidden + vec * kVec, ok[v]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m == 1 && !fo.dv_tail) continue;
      const int vec = lane + 64 * (h + 2 * (m == 0 ? s : 4));
      store16_stream(dkt + kValueCol + vec * kVec, ov[m]);
    }
  }

  // add the token slots in slot order, then write stream s of partial row b
  for (int uu = 0; uu < kBwdSlots; ++uu) {
    if (u == uu) {
#pragma unroll
      for (int v = 0; v < kBwdVecs; ++v) {
        const int vec = lane + 64 * (h + 2 * v);
        f32x4 a0 = {acc[v][0], acc[v][1], acc[v][2], acc[v][3]};
        f32x4 a1 = {acc[v][4], acc[v][5], acc[v][6], acc[v][7]};
        if (uu > 0) {
          a0 += comb[0][vec];
          a1 += comb[1][vec];
        }
        comb[0][vec] = a0;
        comb[1][vec] = a1;
      }
    }
    __syncthreads();
  }
  f32x4* prow = reinterpret_cast<f32x4*>(partial + b * (kStreams * kHidden) + s * kHidden);
  for (int j = threadIdx.x; j < kHidden / 4; j += kBwdThreads) prow[j] = comb[j & 1][j >> 1];
}

constexpr int kReduceChunks = 32;                        // row chunks per column group
constexpr int kReduceGroups = 8;                         // float4 column groups per workgroup
constexpr int kReduceThreads = kReduceChunks * kReduceGroups;  // 256
constexpr int kReduceCols4 = kStreams * kHidden / 4;     // 5120 float4 columns

__global__ void __launch_bounds__(kReduceThreads)
engram_bwd_reduce_kernel(const float* __restrict__ partial, float* __restrict__ dw, int nb,
                         const uint16_t* __restrict__ wh, const uint16_t* __restrict__ we,
                         float* __restrict__ gwh, float* __restrict__ gwe) {
  __shared__ f32x4 part[kReduceChunks][kReduceGroups];
  // 640 workgroups of 8 column groups x 32 row chunks (enough waves to keep
  // the partial rows streaming); a wave reads 8 rows of 128 contiguous bytes
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
    if (gwh) {
      // product rule for weight = wh * we (both bf16): one fp32 multiply each
      const uint2 h = reinterpret_cast<const uint2*>(wh)[col4];
      const uint2 e = reinterpret_cast<const uint2*>(we)[col4];
      const f32x4 hf = {bf_lo(h.x), bf_hi(h.x), bf_lo(h.y), bf_hi(h.y)};
      const f32x4 ef = {bf_lo(e.x), bf_hi(e.x), bf_lo(e.y), bf_hi(e.y)};
      reinterpret_cast<f32x4*>(gwh)[col4] = r * ef;
      reinterpret_cast<f32x4*>(gwe)[col4] = r * hf;
    }
  }
}

// weight = float(wh) * float(we): the product of two bf16 values (8-bit
// significands) is exact in fp32, so this is bit-exact by construction.
__global__ void __launch_bounds__(256)
engram_fused_weight_kernel(const uint16_t* __restrict__ wh, const uint16_t* __restrict__ we,
                           float* __restrict__ weight) {
  const int v = blockIdx.x * 256 + threadIdx.x;  // one 8-element vector; grid covers 2560 exactly
  const u32x4 h = load16(wh + v * kVec);
  const u32x4 e = load16(we + v * kVec);
  f32x4 lo, hi;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    lo[2 * q] = bf_lo(h[q]) * bf_lo(e[q]);
    lo[2 * q + 1] = bf_hi(h[q]) * bf_hi(e[q]);
    hi[2 * q] = bf_lo(h[q + 2]) * bf_lo(e[q + 2]);
    hi[2 * q + 1] = bf_hi(h[q + 2]) * bf_hi(e[q + 2]);
  }
  reinterpret_cast<f32x4*>(weight)[2 * v] = lo;
  reinterpret_cast<f32x4*>(weight)[2 * v + 1] = hi;
}

hipError_t launch_fused_weight(const void* wh, const void* we, float* weight, hipStream_t stream) {
  const uint16_t* hp = static_cast<const uint16_t*>(wh);
  const uint16_t* ep = static_cast<const uint16_t*>(we);
  void* args[] = {&hp, &ep, &weight};
  return hipLaunchKernel(reinterpret_cast<const void*>(&engram_fused_weight_kernel),
                         dim3(kStreams * kRowVecs / 256), dim3(256), args, 0, stream);
}

hipError_t launch_bwd(const void* x, const void* kv, const float* weight, const float* saved, const void* gout,
                      void* dx, void* dkv, float* dw, const void* wh, const void* we, float* gwh, float* gwe,
                      float* partial, int64_t n, hipStream_t stream) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* kvp = static_cast<const uint16_t*>(kv);
  const uint16_t* gp = static_cast<const uint16_t*>(gout);
  uint16_t* dxp = static_cast<uint16_t*>(dx);
  uint16_t* dkvp = static_cast<uint16_t*>(dkv);
  // Partial rows: N/64 of 64 tokens up to N = 4096; above that, when 256
  // tokens divide N, 64 rows of N/64 tokens each, so that all 256
  // workgroups of 512 threads are resident at once (one per CU) and every
  // step is one contiguous band; otherwise N/64 rows in two rounds.
  const int nb = (int)(n / kTokensPerPartial);
  int rows = nb, steps = kTokensPerPartial / kBwdSlots;
  if (nb > 64 && n % 256 == 0) {
    rows = 64;
    steps = (int)(n / (64 * kBwdSlots));
  }
  void* args1[] = {&xp, &kvp, &weight, &saved, &gp, &dxp, &dkvp, &partial, &rows, &steps};
  const int grid1 = (rows + 7) / 8 * 8 * kStreams;  // (row, stream) pairs, rows padded to 8
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&engram_bwd_main_kernel), dim3(grid1),
                                 dim3(64 * 2 * kBwdSlots), args1, 0, stream);
  if (e != hipSuccess) return e;
  const float* cpartial = partial;
  const uint16_t* whp = static_cast<const uint16_t*>(wh);
  const uint16_t* wep = static_cast<const uint16_t*>(we);
  void* args2[] = {&cpartial, &dw, &rows, &whp, &wep, &gwh, &gwe};
  return hipLaunchKernel(reinterpret_cast<const void*>(&engram_bwd_reduce_kernel),
                         dim3(kReduceCols4 / kReduceGroups), dim3(kReduceThreads), args2, 0, stream);
}

// ---- the allocation-free backward: partial rows in a file-scope device array ----
//
// For callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid allocation), the grad_weight partial rows can live in
// a fixed array of this library instead of the caller's workspace: room for
// N/64 rows at the backward's largest N (128 rows of [4][5120] fp32, 10 MiB;
// no accepted N uses more, and N = 8192 itself uses 64),
// held by every GPU the library runs on until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address is taken once per device with hipGetSymbolAddress (that device
// current) and only that address is handed to the kernels.  Every call on a
// GPU shares that GPU's array; the main kernel writes each partial row it
// needs before the reduce reads it, so nothing carries over between calls,
// but two calls that overlap in time on one GPU (different streams) race.
constexpr int64_t kScratchFloats = (kMaxBwdTokens / kTokensPerPartial) * kStreams * kHidden;
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxScratchDevices] = {};
}  // namespace

hipError_t scratch_partials(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

}  // namespace engram
