// stream_lib.hip -- the probe's plain streaming kernels as a small C-ABI
// library (libengram_probe.so), so that a stream with exactly the gate's
// traffic can be timed over the gate's own buffers in the same process
// (bench.py --same-buffers).  Measurement code, not part of libengram.
#include <string.h>

#include "stream_kernels.h"

extern "C" {

// Stream `ntok` tokens of one shape over caller-owned device tensors:
//   shape "fwd": in = {X [ntok][40960 B], KV [ntok][51200 B]}, out = {[ntok][40960 B]}
//   shape "bwd": in = {X, KV, G [ntok][40960 B]},             out = {[ntok][40960 B], [ntok][51200 B]}
//   shapes "gcfwd" / "gcbwd": 3 / 5 inputs and 2 / 3 outputs of [ntok][10240 B]
// (also "write" and "copy" on X-sized rows; the read-only shape, which has
// no output to write, is not offered here).  512-thread workgroups,
// `grid` of them, dealing 0 lockstep / 1 chunked / 2 eight bands (grid a
// multiple of 8), next token's loads before the current token's stores;
// dealing 3 is the gate backward's split: 256-thread workgroups, each
// streaming one quarter of every row of its tokens, lockstep over grid / 4
// workgroup groups (grid a multiple of 8).  All
// pointers 16-byte aligned device memory; the outputs receive values derived
// from the inputs.  Returns 0 once the kernel is enqueued on `stream`, -1 for
// an unknown shape or bad arguments, or the HIP error code of the launch.
int probe_stream(const char* shape, const void* const* in, void* const* out, int64_t ntok, int grid, int dealing,
                 void* stream) {
  const Shape* sh = nullptr;
  for (const Shape& s : kShapes)
    if (strcmp(s.name, shape) == 0) sh = &s;
  if (!sh || sh->nout == 0 || ntok < 1 || grid < 8 || grid % 8 != 0 || dealing < 0 || dealing > 3) return -1;
  Streams s = {};
  for (int k = 0; k < sh->nin; ++k) {
    if (!in || !in[k]) return -1;
    s.in[k] = static_cast<const u32x4*>(in[k]);
    s.in_vecs[k] = sh->in_vecs[k];
  }
  for (int k = 0; k < sh->nout; ++k) {
    if (!out || !out[k]) return -1;
    s.out[k] = static_cast<u32x4*>(out[k]);
    s.out_vecs[k] = sh->out_vecs[k];
  }
  s.sink = s.out[0];  // used by the read-only shape only
  const int64_t chunk = (ntok + grid - 1) / grid;
  if (dealing == 3) {
    if (strcmp(sh->name, "bwd") != 0) return -1;
    // a quarter of a 3,200-vector row is 800 vectors: 4 per thread of 256
    hipLaunchKernelGGL((token_stream<3, 2, 256, 4, kLockstep, true, 4>), dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), s, ntok, chunk);
    return (int)hipGetLastError();
  }
  KernelFn fn = kernel_for<512>(*sh, dealing, true);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(512), 0, static_cast<hipStream_t>(stream), s, ntok, chunk);
  return (int)hipGetLastError();
}

}  // extern "C"
