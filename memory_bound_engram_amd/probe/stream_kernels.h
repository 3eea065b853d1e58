// stream_kernels.h -- the plain streaming kernels of the HBM probe.
//
// Measurement code, not part of libengram: token-major tensors shaped like
// the gate's (X-like rows of 2,560 16-byte vectors, KV-like rows of 3,200) or
// GateConv's (rows of 640 at d = 5120), a workgroup of THREADS threads per
// token, non-temporal 16-byte loads of every input row then non-temporal
// 16-byte stores of every output row (values that depend on the loads, so no
// load can be dropped).  Used by the probe program (hbm_probe.hip) and by the
// probe library (stream_lib.hip) that bench.py runs over the gate's and
// GateConv's own buffers.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kXVecs = 2560;   // 40,960-byte rows
constexpr int kKvVecs = 3200;  // 51,200-byte rows
constexpr int kGcVecs = 640;   // 10,240-byte rows (GateConv, d = 5120)

struct Streams {
  const u32x4* in[5];
  u32x4* out[3];
  int in_vecs[5];
  int out_vecs[3];
  u32x4* sink;  // written only if an impossible value shows up (keeps read-only loads alive)
};

template <int NIN, int MAXV>
struct Rows {
  u32x4 v[NIN > 0 ? NIN : 1][MAXV];
};

// A workgroup streams part `q` of SPLIT equal parts of every row (the whole
// row when SPLIT = 1): vectors [q rv / SPLIT, (q + 1) rv / SPLIT).
template <int SPLIT>
__device__ __forceinline__ int part_lo(int rv, int q) { return (int)((int64_t)rv * q / SPLIT); }

template <int NIN, int THREADS, int MAXV, int SPLIT>
__device__ __forceinline__ void load_rows(const Streams& s, int64_t t, int q, Rows<NIN, MAXV>& r) {
#pragma unroll
  for (int k = 0; k < NIN; ++k) {
    const int lo = part_lo<SPLIT>(s.in_vecs[k], q), hi = part_lo<SPLIT>(s.in_vecs[k], q + 1);
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      const int idx = lo + threadIdx.x + v * THREADS;
      if (idx < hi)
        r.v[k][v] = __builtin_nontemporal_load(s.in[k] + t * s.in_vecs[k] + idx);
      else
        r.v[k][v] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int NIN, int NOUT, int THREADS, int MAXV, int SPLIT>
__device__ __forceinline__ void store_rows(const Streams& s, int64_t t, int q, const Rows<NIN, MAXV>& r,
                                           u32x4& acc) {
  if (NOUT == 0) {
#pragma unroll
    for (int k = 0; k < NIN; ++k)
#pragma unroll
      for (int v = 0; v < MAXV; ++v) acc ^= r.v[k][v];
    return;
  }
#pragma unroll
  for (int k = 0; k < NOUT; ++k) {
    const int lo = part_lo<SPLIT>(s.out_vecs[k], q), hi = part_lo<SPLIT>(s.out_vecs[k], q + 1);
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      const int idx = lo + threadIdx.x + v * THREADS;
      if (idx < hi) {
        u32x4 o;
        if (NIN == 0) {
          const uint32_t c = (uint32_t)t * 2654435761u + (uint32_t)idx;
          o = u32x4{c, c + 1u, c + 2u, c + 3u};
        } else {
          o = r.v[k % (NIN > 0 ? NIN : 1)][v];
#pragma unroll
          for (int q = 1; q < NIN; ++q) o ^= r.v[(k + q) % NIN][v];
        }
        __builtin_nontemporal_store(o, s.out[k] + t * s.out_vecs[k] + idx);
      }
    }
  }
}

enum Dealing { kLockstep = 0, kChunked = 1, kBands = 2 };
constexpr int kBandCount = 8;

// SPLIT > 1: workgroup w streams part w % SPLIT of its tokens' rows (as the
// gate's backward splits rows by stream); the tokens follow the dealing over
// gridDim / SPLIT workgroup groups (lockstep only).
template <int NIN, int NOUT, int THREADS, int MAXV, int DEAL, bool PIPE, int SPLIT = 1>
__global__ void __launch_bounds__(THREADS) token_stream(Streams s, int64_t ntok, int64_t chunk) {
  const int q = SPLIT > 1 ? (int)(blockIdx.x % SPLIT) : 0;
  // token i of this workgroup, or -1 past its last one
  auto token = [&](int64_t i) -> int64_t {
    if (SPLIT > 1) {
      const int64_t t = (int64_t)(blockIdx.x / SPLIT) + i * (gridDim.x / SPLIT);
      return t < ntok ? t : -1;
    }
    if (DEAL == kLockstep) {
      const int64_t t = (int64_t)blockIdx.x + i * gridDim.x;
      return t < ntok ? t : -1;
    }
    if (DEAL == kChunked) {
      const int64_t t = (int64_t)blockIdx.x * chunk + i;
      return (i < chunk && t < ntok) ? t : -1;
    }
    // kBands: the tensors are cut into kBandCount equal bands; workgroup b
    // walks band b % kBandCount in lockstep with the other workgroups of that
    // band, so the chip touches kBandCount separate regions at a time
    const int64_t band_len = (ntok + kBandCount - 1) / kBandCount;
    const int64_t per = gridDim.x / kBandCount;
    const int64_t local = (int64_t)(blockIdx.x / kBandCount) + i * per;
    const int64_t t = (int64_t)(blockIdx.x % kBandCount) * band_len + local;
    return (local < band_len && t < ntok) ? t : -1;
  };
  u32x4 acc = {0u, 0u, 0u, 0u};
  Rows<NIN, MAXV> cur;
  int64_t t = token(0);
  if (PIPE && t >= 0) load_rows<NIN, THREADS, MAXV, SPLIT>(s, t, q, cur);
  for (int64_t i = 0; t >= 0; ++i) {
    const int64_t tn = token(i + 1);
    if (PIPE) {
      Rows<NIN, MAXV> nxt;
      if (tn >= 0) load_rows<NIN, THREADS, MAXV, SPLIT>(s, tn, q, nxt);
      store_rows<NIN, NOUT, THREADS, MAXV, SPLIT>(s, t, q, cur, acc);
      cur = nxt;
    } else {
      load_rows<NIN, THREADS, MAXV, SPLIT>(s, t, q, cur);
      store_rows<NIN, NOUT, THREADS, MAXV, SPLIT>(s, t, q, cur, acc);
    }
    t = tn;
  }
  if (NOUT == 0 && acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) s.sink[threadIdx.x] = acc;
}

struct Shape {
  const char* name;
  int nin, nout;
  int in_vecs[5], out_vecs[3];
};

static const Shape kShapes[] = {
    {"read", 1, 0, {kXVecs}, {}},
    {"write", 0, 1, {}, {kXVecs}},
    {"copy", 1, 1, {kXVecs}, {kXVecs}},
    {"fwd", 2, 1, {kXVecs, kKvVecs}, {kXVecs}},
    {"bwd", 3, 2, {kXVecs, kKvVecs, kXVecs}, {kXVecs, kKvVecs}},
    // GateConv at d = 5120 (10,240-byte rows): the forward's H, k, v -> Y, vhat
    // and the backward's dY, H, k, v, vhat -> dH, dk, dv
    {"gcfwd", 3, 2, {kGcVecs, kGcVecs, kGcVecs}, {kGcVecs, kGcVecs}},
    {"gcbwd", 5, 3, {kGcVecs, kGcVecs, kGcVecs, kGcVecs, kGcVecs}, {kGcVecs, kGcVecs, kGcVecs}},
};

typedef void (*KernelFn)(Streams, int64_t, int64_t);

template <int NIN, int NOUT, int THREADS, int MAXV = (kKvVecs + THREADS - 1) / THREADS>
static KernelFn pick(int deal, bool pipe) {
  if (deal == kLockstep) return pipe ? token_stream<NIN, NOUT, THREADS, MAXV, kLockstep, true>
                                     : token_stream<NIN, NOUT, THREADS, MAXV, kLockstep, false>;
  if (deal == kChunked) return pipe ? token_stream<NIN, NOUT, THREADS, MAXV, kChunked, true>
                                    : token_stream<NIN, NOUT, THREADS, MAXV, kChunked, false>;
  return pipe ? token_stream<NIN, NOUT, THREADS, MAXV, kBands, true>
              : token_stream<NIN, NOUT, THREADS, MAXV, kBands, false>;
}

template <int THREADS>
static KernelFn kernel_for(const Shape& sh, int deal, bool pipe) {
  constexpr int GCV = (kGcVecs + THREADS - 1) / THREADS;  // GateConv rows: fewer vectors per thread
  if (sh.in_vecs[0] == kGcVecs)
    return sh.nin == 3 ? pick<3, 2, THREADS, GCV>(deal, pipe) : pick<5, 3, THREADS, GCV>(deal, pipe);
  if (sh.nin == 1 && sh.nout == 0) return pick<1, 0, THREADS>(deal, pipe);
  if (sh.nin == 0 && sh.nout == 1) return pick<0, 1, THREADS>(deal, pipe);
  if (sh.nin == 1 && sh.nout == 1) return pick<1, 1, THREADS>(deal, pipe);
  if (sh.nin == 2 && sh.nout == 1) return pick<2, 1, THREADS>(deal, pipe);
  return pick<3, 2, THREADS>(deal, pipe);
}

