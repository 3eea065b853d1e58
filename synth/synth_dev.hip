// synth_dev.hip -- device twin of synth_host.c: the same counter-based recipe
// (SplitMix64 words, 12-field Irwin-Hall normals, 24-bit Bernoulli masks),
// producing bit-identical bytes on the GPU for inputs too large to build on
// the host.  Input generation only; none of the gate's arithmetic is here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint32_t id) {
  return mix64(seed + kGamma * ((uint64_t)id + 1));
}

__device__ inline uint64_t word(uint64_t key, uint64_t c) { return mix64(key + kGamma * (c + 1)); }

__device__ inline uint16_t normal_bf16(uint64_t key, uint64_t e) {
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    uint64_t w = word(key, 3 * e + (uint64_t)i);
#pragma unroll
    for (int l = 0; l < 4; ++l) s += (int32_t)((w >> (16 * l)) & 0xFFFFu);
  }
  // (s - 393210) * 2^-16 is exact in fp32; then round to bf16, ties to even.
  float f = __fmul_rn((float)(s - 393210), 0x1p-16f);
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Each thread writes 8 consecutive elements (one 16-byte store when whole).
__global__ void fill_normal_bf16(uint16_t* __restrict__ dst, int64_t count, uint64_t key, int64_t offset) {
  const int64_t nvec = (count + 7) / 8;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i0 = v * 8;
    if (i0 + 8 <= count) {
      uint32_t p[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t lo = normal_bf16(key, (uint64_t)(offset + i0 + 2 * q));
        uint32_t hi = normal_bf16(key, (uint64_t)(offset + i0 + 2 * q + 1));
        p[q] = lo | (hi << 16);
      }
      uint4 val = make_uint4(p[0], p[1], p[2], p[3]);
      *reinterpret_cast<uint4*>(dst + i0) = val;
    } else {
      for (int64_t i = i0; i < count; ++i) dst[i] = normal_bf16(key, (uint64_t)(offset + i));
    }
  }
}

__global__ void fill_mask(uint8_t* __restrict__ dst, int64_t count, uint64_t key, int64_t offset, uint32_t thr) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = (uint8_t)((word(key, (uint64_t)(offset + i)) >> 40) < thr);
}

int grid_for(int64_t work) {
  int64_t g = (work + 255) / 256;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

// dst (device) must be 16-byte aligned; returns a hipError_t value (0 = ok).
extern "C" int synth_dev_normal_bf16(void* dst, int64_t count, uint64_t seed, uint32_t id, int64_t offset,
                                     void* stream) {
  if (count <= 0) return 0;
  if (!dst || (reinterpret_cast<uintptr_t>(dst) & 15)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_normal_bf16, dim3(grid_for((count + 7) / 8)), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)dst, count, stream_key(seed, id), offset);
  return (int)hipGetLastError();
}

extern "C" int synth_dev_mask(void* dst, int64_t count, uint64_t seed, uint32_t id, int64_t offset, uint32_t thr,
                              void* stream) {
  if (count <= 0) return 0;
  if (!dst) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_mask, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)stream, (uint8_t*)dst, count,
                     stream_key(seed, id), offset, thr);
  return (int)hipGetLastError();
}
