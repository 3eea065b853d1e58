// engram_launch.h -- host-side launchers of the libengram kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace engram {

// Enqueue the forward kernel with `grid` workgroups striding over the tokens (no saved
// state is written when saved == nullptr).
hipError_t launch_fwd(const void* x, const void* kv, const float* weight, const uint8_t* mask, void* out,
                      float* saved, int64_t n, int grid, hipStream_t stream);

// Enqueue the paced forward for long calls: `grid` workgroups, one per CU,
// walking the tokens in epochs with a bounded-wait barrier between them; the
// same per-token arithmetic as launch_fwd, so the same out and saved.
hipError_t launch_fwd_paced(const void* x, const void* kv, const float* weight, const uint8_t* mask, void* out,
                            float* saved, int64_t n, int grid, hipStream_t stream);
int64_t fwd_paced_epochs(int64_t n, int grid);

// A slot of the pacing counters (zero between calls) for the next call on the
// current device, dealt round robin, and the device clock's ticks per us.
hipError_t pace_slot(uint32_t** slot, uint64_t* ticks_per_us);

// Enqueue the backward main kernel (4 workgroups per partial row: N/64 rows,
// or 64 above N = 4096 when 256 divides N) and the grad_weight reduction;
// `partial` has room for N/64 rows of [4][5120] fp32 (written, then read
// back).  With wh/we/gwh/gwe non-null the reduction also writes the
// product-rule gradients of weight = wh * we.
hipError_t launch_bwd(const void* x, const void* kv, const float* weight, const float* saved, const void* gout,
                      void* dx, void* dkv, float* dw, const void* wh, const void* we, float* gwh, float* gwe,
                      float* partial, int64_t n, hipStream_t stream);

// The backward's largest N, and the devices the library keeps a scratch
// address for.
constexpr int64_t kMaxBwdTokens = 8192;
constexpr int kMaxScratchDevices = 64;

// Calls longer than this many tokens take the paced forward.
constexpr int64_t kFwdPacedMinTokens = 16384;

// Device address, on the current device, of the library's own partial-row
// array (room for kMaxBwdTokens tokens); taken once per device.
hipError_t scratch_partials(float** out);

// Enqueue weight = float(wh) * float(we) for [4][5120] bf16 inputs.
hipError_t launch_fused_weight(const void* wh, const void* we, float* weight, hipStream_t stream);

// GateConv: rows per workgroup chunk (a function of M*T and d only), the number of
// workgroups, and the launchers (forward; backward main + weight-gradient
// reduce, in two levels above 512 workgroups).
int gateconv_chunk(int64_t M, int64_t T, int64_t d, bool bwd);
int64_t gateconv_workgroups(int64_t M, int64_t T, int chunk);
size_t gateconv_bwd_workspace(int64_t M, int64_t T, int64_t d, int chunk);
hipError_t launch_gateconv_fwd(const void* H, const void* K, const void* V, const float* wh, const float* wv,
                               const float* cw, void* Y, void* vhat, float* alpha, float* rrh, float* rrk, float* rrv,
                               int64_t M, int64_t T, int64_t d, float eps, int chunk, hipStream_t stream);
hipError_t launch_gateconv_bwd(const void* dY, const void* H, const void* K, const void* V, const float* wh,
                               const float* wv, const float* cw, const void* vhat, const float* alpha, const float* rrh,
                               const float* rrk, const float* rrv, void* dH, void* dK, void* dV, float* dwh, float* dwv,
                               float* dcw, void* workspace, int64_t M, int64_t T, int64_t d, int chunk,
                               hipStream_t stream);

}  // namespace engram
