// engram_api.cpp -- the C ABI of libengram: argument validation on the host,
// then kernel launches on the caller's stream.  Nothing here allocates,
// copies or synchronises.  Limits and rules: "Engram saved-state gate"
// (cuDNN frontend docs), layout, saved-state and workspace paragraphs.
#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

#include "engram.h"
#include "engram_launch.h"

namespace {

constexpr int64_t kXRowBytes = (int64_t)ENGRAM_STREAMS * ENGRAM_HIDDEN * 2;  // 40960
constexpr int64_t kKvRowBytes = (int64_t)ENGRAM_KV_COLS * 2;                 // 51200
constexpr int64_t kWeightBytes = (int64_t)ENGRAM_STREAMS * ENGRAM_HIDDEN * 4;  // 81920
constexpr int64_t kSavedRowBytes = (int64_t)ENGRAM_STREAMS * 4 * 4;          // 64
// forward workgroups per CU, one resident, the rest queued: of 1, 2, 4 and 8,
// timed cold, the fastest at N = 8192 and within 1% of the fastest at
// N = 1,048,512; back to back in the forward + backward step 8 was 0.3%
// faster, less than the step moves with where the buffers land, and 16 or
// 32 were 2-4% slower
constexpr int kFwdWorkgroupsPerCu = 4;
constexpr int kMaxDevices = 64;

thread_local int g_last_hip_error = 0;
std::atomic<int> g_cu_count[kMaxDevices];

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)bytes};
}

bool overlaps(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Outputs (and scratch) may overlap neither an input nor each other.
bool any_overlap(const Range* in, int nin, const Range* out, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(out[i], in[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(out[i], out[j])) return true;
  }
  return false;
}

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    g_cu_count[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

engram_status launched(hipError_t e) {
  g_last_hip_error = (int)e;
  return e == hipSuccess ? ENGRAM_OK : ENGRAM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t engram_gate_bwd_workspace_bytes(int64_t N) {
  if (N <= 0) return 0;
  return (size_t)4 * ((size_t)16 * (size_t)N + (size_t)4 * ENGRAM_HIDDEN * (size_t)(N / 64));
}

engram_status engram_gate_fwd(const void* x, const void* kv, const float* weight, const uint8_t* mask, void* out,
                              float* saved, int64_t N, void* stream) {
  // saved == NULL selects the inference forward (no saved state written)
  if (!x || !kv || !weight || !mask || !out) return ENGRAM_ERR_NULL;
  if (N < 1 || N > ENGRAM_N_MAX) return ENGRAM_ERR_N_RANGE;
  if (!aligned16(x) || !aligned16(kv) || !aligned16(weight) || !aligned16(out) || (saved && !aligned16(saved)))
    return ENGRAM_ERR_ALIGN;
  const Range in[] = {range_of(x, N * kXRowBytes), range_of(kv, N * kKvRowBytes), range_of(weight, kWeightBytes),
                      range_of(mask, N)};
  const Range outs[] = {range_of(out, N * kXRowBytes), range_of(saved, saved ? N * kSavedRowBytes : 0)};
  if (any_overlap(in, 4, outs, 2)) return ENGRAM_ERR_OVERLAP;
  if (N > engram::kFwdPacedMinTokens)  // one workgroup per CU, epochs with a bounded-wait barrier between them
    return launched(engram::launch_fwd_paced(x, kv, weight, mask, out, saved, N, cu_count(), (hipStream_t)stream));
  int64_t grid = (int64_t)kFwdWorkgroupsPerCu * cu_count();
  if (grid > N) grid = N;
  return launched(engram::launch_fwd(x, kv, weight, mask, out, saved, N, (int)grid, (hipStream_t)stream));
}

static engram_status bwd_common(const void* x, const void* kv, const float* weight, const float* saved,
                                const void* grad_out, void* grad_x, void* grad_kv, float* grad_weight,
                                const void* wh, const void* we, float* grad_wh, float* grad_we, void* workspace,
                                int64_t N, void* stream) {
  const bool rule = wh != nullptr;  // product-rule variant: all four extra pointers present
  if (!x || !kv || !weight || !saved || !grad_out || !grad_x || !grad_kv || !grad_weight || !workspace)
    return ENGRAM_ERR_NULL;
  if (rule && (!we || !grad_wh || !grad_we)) return ENGRAM_ERR_NULL;
  if (N < 1 || N > ENGRAM_BWD_N_MAX) return ENGRAM_ERR_N_RANGE;
  if (N % ENGRAM_BWD_N_MULTIPLE != 0) return ENGRAM_ERR_N_MULT64;
  if (!aligned16(x) || !aligned16(kv) || !aligned16(weight) || !aligned16(saved) || !aligned16(grad_out) ||
      !aligned16(grad_x) || !aligned16(grad_kv) || !aligned16(grad_weight) || !aligned16(workspace))
    return ENGRAM_ERR_ALIGN;
  if (rule && (!aligned16(wh) || !aligned16(we) || !aligned16(grad_wh) || !aligned16(grad_we)))
    return ENGRAM_ERR_ALIGN;
  const int64_t nw = rule ? kWeightBytes / 2 : 0;  // bf16 norm weights
  const int64_t gw = rule ? kWeightBytes : 0;
  const Range in[] = {range_of(x, N * kXRowBytes),      range_of(kv, N * kKvRowBytes),
                      range_of(weight, kWeightBytes),   range_of(saved, N * kSavedRowBytes),
                      range_of(grad_out, N * kXRowBytes), range_of(wh, nw), range_of(we, nw)};
  const Range outs[] = {range_of(grad_x, N * kXRowBytes), range_of(grad_kv, N * kKvRowBytes),
                        range_of(grad_weight, kWeightBytes),
                        range_of(workspace, (int64_t)engram_gate_bwd_workspace_bytes(N)),
                        range_of(grad_wh, gw), range_of(grad_we, gw)};
  if (any_overlap(in, 7, outs, 6)) return ENGRAM_ERR_OVERLAP;
  // the first 16 N floats of the workspace are reserved; the partial rows follow
  float* partial = static_cast<float*>(workspace) + 16 * N;
  return launched(engram::launch_bwd(x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, wh, we, grad_wh,
                                     grad_we, partial, N, (hipStream_t)stream));
}

engram_status engram_gate_bwd(const void* x, const void* kv, const float* weight, const float* saved,
                              const void* grad_out, void* grad_x, void* grad_kv, float* grad_weight, void* workspace,
                              int64_t N, void* stream) {
  return bwd_common(x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, nullptr, nullptr, nullptr, nullptr,
                    workspace, N, stream);
}

engram_status engram_gate_bwd_with_norm_weights(const void* x, const void* kv, const float* weight, const float* saved,
                                                const void* grad_out, void* grad_x, void* grad_kv, float* grad_weight,
                                                const void* wh, const void* we, float* grad_wh, float* grad_we,
                                                void* workspace, int64_t N, void* stream) {
  if (!wh) return ENGRAM_ERR_NULL;
  return bwd_common(x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, wh, we, grad_wh, grad_we, workspace,
                    N, stream);
}

engram_status engram_gate_bwd_noalloc(const void* x, const void* kv, const float* weight, const float* saved,
                                      const void* grad_out, void* grad_x, void* grad_kv, float* grad_weight, int64_t N,
                                      void* stream) {
  if (!x || !kv || !weight || !saved || !grad_out || !grad_x || !grad_kv || !grad_weight) return ENGRAM_ERR_NULL;
  if (N < 1 || N > ENGRAM_NOALLOC_N_MAX || N > ENGRAM_BWD_N_MAX) return ENGRAM_ERR_N_RANGE;
  if (N % ENGRAM_BWD_N_MULTIPLE != 0) return ENGRAM_ERR_N_MULT64;
  if (!aligned16(x) || !aligned16(kv) || !aligned16(weight) || !aligned16(saved) || !aligned16(grad_out) ||
      !aligned16(grad_x) || !aligned16(grad_kv) || !aligned16(grad_weight))
    return ENGRAM_ERR_ALIGN;
  const Range in[] = {range_of(x, N * kXRowBytes), range_of(kv, N * kKvRowBytes), range_of(weight, kWeightBytes),
                      range_of(saved, N * kSavedRowBytes), range_of(grad_out, N * kXRowBytes)};
  const Range outs[] = {range_of(grad_x, N * kXRowBytes), range_of(grad_kv, N * kKvRowBytes),
                        range_of(grad_weight, kWeightBytes)};
  if (any_overlap(in, 5, outs, 3)) return ENGRAM_ERR_OVERLAP;
  float* partial = nullptr;
  const hipError_t e = engram::scratch_partials(&partial);
  if (e != hipSuccess) return launched(e);
  return launched(engram::launch_bwd(x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, nullptr, nullptr,
                                     nullptr, nullptr, partial, N, (hipStream_t)stream));
}

engram_status engram_fused_weight(const void* wh, const void* we, float* weight, void* stream) {
  if (!wh || !we || !weight) return ENGRAM_ERR_NULL;
  if (!aligned16(wh) || !aligned16(we) || !aligned16(weight)) return ENGRAM_ERR_ALIGN;
  const Range in[] = {range_of(wh, kWeightBytes / 2), range_of(we, kWeightBytes / 2)};
  const Range outs[] = {range_of(weight, kWeightBytes)};
  if (any_overlap(in, 2, outs, 1)) return ENGRAM_ERR_OVERLAP;
  return launched(engram::launch_fused_weight(wh, we, weight, (hipStream_t)stream));
}

// ---- GateConv ("Engram Operators", TileOPs, GateConv section) ----

static bool gateconv_dims_ok(int64_t M, int64_t T, int64_t d) {
  return M >= 1 && T >= 1 && M <= ENGRAM_GATECONV_ROWS_MAX && T <= ENGRAM_GATECONV_ROWS_MAX &&
         M * T <= ENGRAM_GATECONV_ROWS_MAX && d >= 512 && d <= ENGRAM_GATECONV_D_MAX && d % 512 == 0;
}

size_t engram_gateconv_bwd_workspace_bytes(int64_t M, int64_t T, int64_t d) {
  if (!gateconv_dims_ok(M, T, d)) return 0;
  return engram::gateconv_bwd_workspace(M, T, d, engram::gateconv_chunk(M, T, d, true));
}

engram_status engram_gateconv_fwd(const void* H, const void* k, const void* v, const float* rms_w_h,
                                  const float* rms_w_v, const float* conv_w, void* Y, void* vhat, float* alpha,
                                  float* rrms_h, float* rrms_k, float* rrms_v, int64_t M, int64_t T, int64_t d,
                                  float eps, void* stream) {
  if (!H || !k || !v || !rms_w_h || !rms_w_v || !conv_w || !Y || !vhat || !alpha || !rrms_h || !rrms_k || !rrms_v)
    return ENGRAM_ERR_NULL;
  if (!gateconv_dims_ok(M, T, d) || !(eps >= 0.0f) || eps > 1.0f) return ENGRAM_ERR_N_RANGE;
  const void* f16[] = {H, k, v, rms_w_h, rms_w_v, conv_w, Y, vhat, alpha, rrms_h, rrms_k, rrms_v};
  for (const void* p : f16)
    if (!aligned16(p)) return ENGRAM_ERR_ALIGN;
  const int64_t rows = M * T, tb = rows * d * 2, sb = rows * 4;
  const Range in[] = {range_of(H, tb), range_of(k, tb), range_of(v, tb), range_of(rms_w_h, d * 4),
                      range_of(rms_w_v, d * 4), range_of(conv_w, 4 * d * 4)};
  const Range outs[] = {range_of(Y, tb),      range_of(vhat, tb),   range_of(alpha, sb),
                        range_of(rrms_h, sb), range_of(rrms_k, sb), range_of(rrms_v, sb)};
  if (any_overlap(in, 6, outs, 6)) return ENGRAM_ERR_OVERLAP;
  return launched(engram::launch_gateconv_fwd(H, k, v, rms_w_h, rms_w_v, conv_w, Y, vhat, alpha, rrms_h, rrms_k,
                                              rrms_v, M, T, d, eps, engram::gateconv_chunk(M, T, d, false),
                                              (hipStream_t)stream));
}

engram_status engram_gateconv_bwd(const void* dY, const void* H, const void* k, const void* v, const float* rms_w_h,
                                  const float* rms_w_v, const float* conv_w, const void* vhat, const float* alpha,
                                  const float* rrms_h, const float* rrms_k, const float* rrms_v, void* dH, void* dk,
                                  void* dv, float* drms_w_h, float* drms_w_v, float* dconv_w, void* workspace,
                                  int64_t M, int64_t T, int64_t d, void* stream) {
  if (!dY || !H || !k || !v || !rms_w_h || !rms_w_v || !conv_w || !vhat || !alpha || !rrms_h || !rrms_k ||
      !rrms_v || !dH || !dk || !dv || !drms_w_h || !drms_w_v || !dconv_w || !workspace)
    return ENGRAM_ERR_NULL;
  if (!gateconv_dims_ok(M, T, d)) return ENGRAM_ERR_N_RANGE;
  const void* f16[] = {dY, H, k, v, rms_w_h, rms_w_v, conv_w, vhat, alpha, rrms_h, rrms_k, rrms_v,
                       dH, dk, dv, drms_w_h, drms_w_v, dconv_w, workspace};
  for (const void* p : f16)
    if (!aligned16(p)) return ENGRAM_ERR_ALIGN;
  const int64_t rows = M * T, tb = rows * d * 2, sb = rows * 4;
  const Range in[] = {range_of(dY, tb),          range_of(H, tb),           range_of(k, tb),
                      range_of(v, tb),           range_of(rms_w_h, d * 4),  range_of(rms_w_v, d * 4),
                      range_of(conv_w, 16 * d),  range_of(vhat, tb),        range_of(alpha, sb),
                      range_of(rrms_h, sb),      range_of(rrms_k, sb),      range_of(rrms_v, sb)};
  const Range outs[] = {range_of(dH, tb),          range_of(dk, tb),          range_of(dv, tb),
                        range_of(drms_w_h, d * 4), range_of(drms_w_v, d * 4), range_of(dconv_w, 16 * d),
                        range_of(workspace, (int64_t)engram_gateconv_bwd_workspace_bytes(M, T, d))};
  if (any_overlap(in, 12, outs, 7)) return ENGRAM_ERR_OVERLAP;
  return launched(engram::launch_gateconv_bwd(dY, H, k, v, rms_w_h, rms_w_v, conv_w, vhat, alpha, rrms_h, rrms_k,
                                              rrms_v, dH, dk, dv, drms_w_h, drms_w_v, dconv_w, workspace, M, T, d,
                                              engram::gateconv_chunk(M, T, d, true), (hipStream_t)stream));
}

const char* engram_status_string(int status) {
  switch (status) {
    case ENGRAM_OK: return "ok";
    case ENGRAM_ERR_NULL: return "a required pointer is NULL";
    case ENGRAM_ERR_N_RANGE: return "size out of range (gate: forward N 1..4194240, backward N <= 8192; GateConv: M, T >= 1, M*T <= 4194304, d a multiple of 512 up to 5120, 0 <= eps <= 1)";
    case ENGRAM_ERR_N_MULT64: return "backward N must be a multiple of 64";
    case ENGRAM_ERR_ALIGN: return "floating tensors and workspace must be 16-byte aligned";
    case ENGRAM_ERR_OVERLAP: return "outputs/workspace overlap an input or each other";
    case ENGRAM_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int engram_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
