// engram_launch.h -- host-side launchers of the libengram kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace engram {

// Enqueue the forward kernel with `grid` persistent workgroups.
hipError_t launch_fwd(const void* x, const void* kv, const float* weight, const uint8_t* mask, void* out,
                      float* saved, int64_t n, int grid, hipStream_t stream);

// Enqueue the backward main kernel (N/64 workgroups) and the grad_weight reduction.
hipError_t launch_bwd(const void* x, const void* kv, const float* weight, const float* saved, const void* gout,
                      void* dx, void* dkv, float* dw, void* workspace, int64_t n, hipStream_t stream);

}  // namespace engram
