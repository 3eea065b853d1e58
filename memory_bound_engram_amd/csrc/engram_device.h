// engram_device.h -- device helpers shared by the libengram kernels (gfx950).
//
// Storage: bf16 values travel as 16-byte vectors of eight (u32x4); a bf16 is
// the upper half of a binary32, so widening is exact and takes one shift or
// mask per value.  Narrowing uses gfx950's v_cvt_pk_bf16_f32 (round to
// nearest even), which the compiler emits for a float2 -> bf16x2 vector
// conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace engram {

constexpr int kStreams = 4;
constexpr int kHidden = 5120;                 // per-stream hidden size d
constexpr int kKvCols = 5 * kHidden;          // four keys, then the shared value
constexpr int kValueCol = 4 * kHidden;        // first column of the shared value
constexpr int kVec = 8;                       // bf16 per 16-byte vector
constexpr int kRowVecs = kHidden / kVec;      // 640 vectors per row
constexpr int kTokensPerPartial = 64;         // grad_weight partial granularity
constexpr float kEps = 1e-20f;                // normalisation epsilon
constexpr float kClamp = 1e-6f;               // signed-sqrt clamp

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2 (lo in bits 15:0), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

template <int kCtrl, int kRowMask, int kBankMask, bool kBoundCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, kBankMask, kBoundCtrl));
}

// v += the value of lane 15 of the previous row, in rows 1 and 3 only
// (row_bcast:15, row mask 0xa); lanes of rows 0 and 2 are not written.  One
// DPP add: the builtin form needs a zero moved in and a separate add.  The
// s_nop gives the two wait states a DPP read of a VGPR written by the
// previous VALU instruction needs.
__device__ __forceinline__ float add_row_bcast15(float v) {
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf" : "+v"(v));
  return v;
}

// v += the value of lane 31, in rows 2 and 3 only (row_bcast:31, row mask 0xc).
__device__ __forceinline__ float add_row_bcast31(float v) {
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf" : "+v"(v));
  return v;
}

// Sum over the 64 lanes of a wave; the full sum lands in lane 63 (other
// lanes hold partial sums).  Fixed order, so the result is deterministic.
//   quad_perm[1,0,3,2], quad_perm[2,3,0,1]  -> sums of 4
//   row_half_mirror, row_mirror             -> sums of 16 in every lane of a row
//   row_bcast:15 (rows 1,3), row_bcast:31 (rows 2,3) -> lane 63 holds all 64
// (lane 63 adds, in order: its row's sum, row 2's, then lane 31's sum of rows
// 0 and 1 -- lane 31 is in row 1, which the first broadcast does update)
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp<0xB1, 0xF, 0xF, true>(v);
  v += dpp<0x4E, 0xF, 0xF, true>(v);
  v += dpp<0x141, 0xF, 0xF, true>(v);
  v += dpp<0x140, 0xF, 0xF, true>(v);
  v = add_row_bcast15(v);
  v = add_row_bcast31(v);
  return v;
}

__device__ __forceinline__ float read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---- pacing barrier: keeps the workgroups of a long kernel in step ----
//
// Workgroups that run a long loop drift apart, so that at any moment some of
// them read while others write; kept in step, the chip reads a band of tokens,
// then writes it, and HBM delivers more.  The barrier only paces -- no kernel
// exchanges data through it -- so every wait is bounded (`spin_ticks` of the
// device's constant-rate clock) and results never depend on it.  Two levels,
// since 256 atomic increments of one word queue behind each other (a one-level
// barrier cost ~15 us): the G workgroups count in kPaceGroups group counters
// (workgroup b in group b mod kPaceGroups), the last arrival of a group counts
// in the top counter and waits there, then raises its group's release word,
// which the group's other workgroups wait on.  Counts accumulate over a call's
// barriers; `depart` counts workgroups past their last barrier, and the last to
// depart sets the slot back to zero for its next call.  A slot is a run of
// 256-byte lines, one word used in each.  Called by one thread per workgroup.
constexpr int kPaceGroups = 16;
constexpr int kPaceLineWords = 64;                   // 256 bytes
constexpr int kPaceSlotLines = 3 + 2 * kPaceGroups;  // top, depart, abandon, group arrive words, group release words
constexpr int kPaceSlotWords = kPaceSlotLines * kPaceLineWords;

// Wait until *p >= target.  A wait that runs out of time marks the call's
// slot abandoned, and every later wait of the call sees that and returns at
// once: a call whose workgroups cannot all be resident (other kernels hold
// CUs) pays the bound once, then runs unpaced.
__device__ __forceinline__ void pace_wait(uint32_t* slot, const uint32_t* p, uint32_t target, uint64_t spin_ticks) {
  uint32_t* abandon = slot + 2 * kPaceLineWords;
  const uint64_t start = wall_clock64();
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (__hip_atomic_load(abandon, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
    if (wall_clock64() - start >= spin_ticks) {
      __hip_atomic_store(abandon, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The `done`-th barrier of the call (done = 1, 2, ...) for workgroup wg of G.
__device__ __forceinline__ void pace_barrier(uint32_t* slot, uint32_t done, uint32_t wg, uint32_t G,
                                             uint64_t spin_ticks) {
  const uint32_t groups = G < (uint32_t)kPaceGroups ? G : (uint32_t)kPaceGroups;
  const uint32_t g = wg % groups;
  const uint32_t group_size = (G - g + groups - 1) / groups;
  uint32_t* top = slot;
  uint32_t* arrive = slot + (3 + g) * kPaceLineWords;
  uint32_t* release = slot + (3 + kPaceGroups + g) * kPaceLineWords;
  const uint32_t before = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (before + 1 == done * group_size) {  // the group's last arrival
    __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pace_wait(slot, top, done * groups, spin_ticks);
    __hip_atomic_fetch_max(release, done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    pace_wait(slot, release, done, spin_ticks);
  }
}

// After a workgroup's last barrier of the call.
__device__ __forceinline__ void pace_depart(uint32_t* slot, uint32_t G) {
  uint32_t* depart = slot + kPaceLineWords;
  const uint32_t before = __hip_atomic_fetch_add(depart, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  if (before + 1 == G) {  // every workgroup is past its last barrier
    for (int l = 0; l < kPaceSlotLines; ++l)
      __hip_atomic_store(slot + l * kPaceLineWords, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace engram
