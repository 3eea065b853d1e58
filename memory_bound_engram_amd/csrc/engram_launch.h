// engram_launch.h -- host-side launchers of the libengram kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace engram {

// Enqueue the forward kernel with `grid` persistent workgroups (no saved
// state is written when saved == nullptr).
hipError_t launch_fwd(const void* x, const void* kv, const float* weight, const uint8_t* mask, void* out,
                      float* saved, int64_t n, int grid, hipStream_t stream);

// Enqueue the backward main kernel (4 x N/64 workgroups) and the grad_weight
// reduction; with wh/we/gwh/gwe non-null the reduction also writes the
// product-rule gradients of weight = wh * we.
hipError_t launch_bwd(const void* x, const void* kv, const float* weight, const float* saved, const void* gout,
                      void* dx, void* dkv, float* dw, const void* wh, const void* we, float* gwh, float* gwe,
                      void* workspace, int64_t n, hipStream_t stream);

// Enqueue weight = float(wh) * float(we) for [4][5120] bf16 inputs.
hipError_t launch_fused_weight(const void* wh, const void* we, float* weight, hipStream_t stream);

}  // namespace engram
