/*
 * engram.h -- C ABI of libengram: the four-stream Engram saved-state gate,
 * forward and explicit backward, for AMD Instinct MI355X (gfx950).
 *
 * Operation ("Engram saved-state gate", cuDNN frontend documentation,
 * semantics paragraph).  For token t and stream s (4 streams, d = 5120):
 *   x = X[t,s,:], k = KV[t, s*d : (s+1)*d], v = KV[t, 4d : 5d], w = weight[s,:]
 *   rstd_X   = (mean_j x_j^2 + 1e-20)^(-1/2),  rstd_key likewise for k
 *   dot      = sum_j (x_j rstd_X) w_j (k_j rstd_key)          (fp32)
 *   gate     = sigmoid( sgn(dot) * sqrt(max(|dot|, 1e-6)) ),   sgn(0) = 0
 *   out[t,s,j] = mask[t] ? bf16_rne(x_j + gate * v_j) : X[t,s,j]
 *   saved[t,s,:] = (mask[t] ? gate : 0, dot, rstd_X, rstd_key)
 * The backward is the gradient of that map for an upstream grad_out G:
 *   grad_x, grad_kv (keys, then the shared value whose four stream
 *   contributions are summed in fp32 before one bf16 cast) and grad_weight
 *   (summed over all tokens).
 *
 * Shapes and layout (layout and saved-state paragraphs).  Everything is
 * dense, row-major and contiguous:
 *   x, out, grad_out, grad_x : [N][4][5120]  bf16
 *   kv, grad_kv              : [N][25600]    bf16 (4 keys, then the value)
 *   weight, grad_weight      : [4][5120]     fp32
 *   mask                     : [N]           bytes, nonzero = true
 *   saved                    : [N][4][4]     fp32 (gate, dot, rstd_X, rstd_key)
 *   workspace                : engram_gate_bwd_workspace_bytes(N) bytes
 *
 * Common contract of the compute calls.
 *   - Every pointer except `stream` is a device pointer on the current HIP
 *     device; `stream` is a hipStream_t of that device, passed as void*
 *     (NULL = the null stream).
 *   - Arguments are validated on the host before any HIP call; a rejected
 *     call returns a nonzero status and touches neither the device nor the
 *     stream.  Validation reads no device memory.
 *   - Accepted calls only enqueue kernels on `stream` and return: no
 *     allocation, copy, conversion, compilation or synchronisation.  Launch
 *     errors come back as ENGRAM_ERR_LAUNCH.  Results are ready when the
 *     stream reaches that point.
 *   - The caller owns every buffer.  Outputs and the workspace are treated
 *     as uninitialised on entry and are written in full.  Inputs may alias
 *     each other; outputs and workspace must not overlap any input or each
 *     other (saved-state paragraph).
 *   - The library holds no state between calls beyond per-device caches of
 *     fixed facts (the CU count, the addresses of its own device arrays) and
 *     the round-robin position of the forward's pacing slots, and is
 *     thread-safe; calls on different streams are independent, except
 *     engram_gate_bwd_noalloc calls on one GPU, which share that GPU's
 *     scratch array.  Results are bitwise reproducible for identical inputs
 *     (fixed reduction orders; the only atomics are the forward's pacing
 *     counters, which no result depends on).
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every compute entry point returns one of these. */
typedef enum {
  ENGRAM_OK = 0,
  ENGRAM_ERR_NULL = 1,     /* a required pointer is NULL */
  ENGRAM_ERR_N_RANGE = 2,  /* a size out of range: N outside 1..4194240 (forward) or 1..8192
                              (backward); GateConv M, T, d, eps outside their limits */
  ENGRAM_ERR_N_MULT64 = 3, /* backward N not a multiple of 64 */
  ENGRAM_ERR_ALIGN = 4,    /* a floating tensor or the workspace is not 16-byte aligned */
  ENGRAM_ERR_OVERLAP = 5,  /* an output or the workspace overlaps an input or another output */
  ENGRAM_ERR_LAUNCH = 6    /* the HIP runtime refused the launch (see engram_last_hip_error) */
} engram_status;

/* Size limits (layout paragraph). */
#define ENGRAM_STREAMS 4
#define ENGRAM_HIDDEN 5120
#define ENGRAM_KV_COLS 25600
#define ENGRAM_N_MAX 4194240
#define ENGRAM_BWD_N_MAX 8192
#define ENGRAM_BWD_N_MULTIPLE 64

/*
 * Forward ("Engram saved-state gate": semantics, layout and saved-state
 * paragraphs; argument order of the plan's execute call).
 *   x      [N][4][5120] bf16, in       16-byte aligned
 *   kv     [N][25600]   bf16, in       16-byte aligned
 *   weight [4][5120]    fp32, in       16-byte aligned
 *   mask   [N]          u8,   in       any alignment
 *   out    [N][4][5120] bf16, out      16-byte aligned
 *   saved  [N][4][4]    fp32, out      16-byte aligned, or NULL for the
 *                                      inference forward (nothing saved; out is
 *                                      bit-identical to the saving call, as the
 *                                      "tile-kernels 1.0.0" forward test requires
 *                                      of save_for_backward=False)
 *   N      1 <= N <= 4194240
 * No workspace.  A false mask byte makes out[t] a bit copy of x[t] and saves
 * gate 0 for every stream of t; dot and both rstd are still saved.
 * Calls with N > 16384 keep their workgroups in step with counters in a small
 * device array of the library (16 slots per GPU, one taken per call round
 * robin, each set back to zero by the call that used it).  They only pace the
 * kernel: results never depend on them, and every wait on them is bounded, so
 * more than 16 such calls in flight at once on one GPU (sharing a slot) can
 * run slower but not differently or forever; a call whose wait runs out
 * (its workgroups not all resident, e.g. beside another kernel) stops pacing
 * for the rest of that call.  The environment variable
 * ENGRAM_PACE_WAIT_US (read at every call; 0..1000000, default 200) bounds
 * one wait in microseconds; 0 turns the pacing off.
 */
engram_status engram_gate_fwd(const void *x, const void *kv, const float *weight, const uint8_t *mask,
                              void *out, float *saved, int64_t N, void *stream);

/*
 * Backward ("Engram saved-state gate": layout, saved-state and workspace
 * paragraphs).
 *   x, kv, weight  as in the forward, in
 *   saved  [N][4][4]    fp32, in       the forward's saved for these x/kv/weight
 *                                      (not verified: the page leaves identity
 *                                      to the caller)
 *   grad_out [N][4][5120] bf16, in
 *   grad_x   [N][4][5120] bf16, out
 *   grad_kv  [N][25600]   bf16, out    keys' gradients, then the shared value's
 *   grad_weight [4][5120] fp32, out    overwritten (not accumulated)
 *   workspace  engram_gate_bwd_workspace_bytes(N) bytes, scratch, 16-byte
 *              aligned, contents ignored on entry and undefined on exit
 *   N      64 <= N <= 8192, N % 64 == 0
 * The mask reaches the backward through saved (gate 0 for a masked token).
 */
engram_status engram_gate_bwd(const void *x, const void *kv, const float *weight, const float *saved,
                              const void *grad_out, void *grad_x, void *grad_kv, float *grad_weight,
                              void *workspace, int64_t N, void *stream);

/*
 * Backward plus the product rule of the fused weight.  Same arguments and
 * contract as engram_gate_bwd, and in addition
 *   wh, we   [4][5120] bf16, in   the source q/k normalisation weights with
 *                                 weight == float(wh) * float(we)
 *   grad_wh  [4][5120] fp32, out  grad_weight * float(we)  (one fp32 multiply)
 *   grad_we  [4][5120] fp32, out  grad_weight * float(wh)
 * grad_weight is still written.  The gate page leaves these gradients to the
 * caller ("Engram saved-state gate", semantics paragraph); the
 * "tile-kernels 1.0.0" backward test forms them this way.  They are produced
 * by the grad_weight reduction kernel, so they cost no extra launch.
 * All four extra pointers are required (ENGRAM_ERR_NULL otherwise), 16-byte
 * aligned, and the outputs must not overlap anything.
 */
engram_status engram_gate_bwd_with_norm_weights(const void *x, const void *kv, const float *weight,
                                                const float *saved, const void *grad_out, void *grad_x,
                                                void *grad_kv, float *grad_weight, const void *wh,
                                                const void *we, float *grad_wh, float *grad_we,
                                                void *workspace, int64_t N, void *stream);

/*
 * Backward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, results and
 * contract as engram_gate_bwd without `workspace`: the grad_weight partial
 * rows go to a fixed array inside the library, sized for
 * ENGRAM_NOALLOC_N_MAX tokens (ENGRAM_NOALLOC_SCRATCH_BYTES = 10 MiB), which
 * every GPU the library runs on holds from its first such call until the
 * process ends.  Results are bit-identical to engram_gate_bwd's.
 *   N   64 <= N <= ENGRAM_NOALLOC_N_MAX (= the backward's own limit), N % 64 == 0;
 *       larger N returns ENGRAM_ERR_N_RANGE before anything is enqueued.
 * The first call on a device looks up the array's address on that device
 * (the current device; a failure returns ENGRAM_ERR_LAUNCH).  No call
 * allocates, frees or synchronises.  Every call on one GPU shares its array:
 * nothing carries over from one call to the next, but calls that overlap in
 * time on one GPU (on different streams) race and must be serialised by the
 * caller.
 */
#define ENGRAM_NOALLOC_N_MAX 8192
#define ENGRAM_NOALLOC_SCRATCH_BYTES 10485760 /* (8192/64) * 4 * 5120 * 4 */
engram_status engram_gate_bwd_noalloc(const void *x, const void *kv, const float *weight, const float *saved,
                                      const void *grad_out, void *grad_x, void *grad_kv, float *grad_weight,
                                      int64_t N, void *stream);

/*
 * Fused weight: weight = float(wh) * float(we), [4][5120] bf16 inputs, fp32
 * output ("Engram saved-state gate", semantics paragraph: the weight argument
 * is the FP32 product of the source q/k normalisation weights; the
 * "tile-kernels 1.0.0" fused-weight test requires it bit-exact).  The product
 * of two bf16 values is exact in fp32.  All pointers device, 16-byte aligned;
 * weight must not overlap wh or we.
 */
engram_status engram_fused_weight(const void *wh, const void *we, float *weight, void *stream);

/*
 * Workspace size of the backward in bytes ("Engram saved-state gate",
 * workspace paragraph): 4 * (16*N + 4*5120*(N/64)), integer division.
 * Pure host arithmetic; returns 0 for N <= 0.
 */
size_t engram_gate_bwd_workspace_bytes(int64_t N);

/* ==========================================================================
 * Engram GateConv ("Engram Operators", TileOPs, GateConv section): the
 * post-projection part of an Engram layer -- RMSNorm gating, a causal
 * depthwise conv1d with 4 taps, SiLU and the gated value as residual -- with
 * the saved tensors of the page's backward (vhat, alpha, rrms_h, rrms_k,
 * rrms_v).  The page gives no formulas; the readings implemented are:
 *   h^ = H rrms_h w_h, k^ = k rrms_k w_h, rrms = (mean square + eps)^(-1/2)
 *   alpha = sigmoid(<h^, k^> / sqrt(d)),  vhat = alpha v
 *   u = vhat rrms_v w_v,  c_t = sum_{i<4} conv_w[i] u_{t-3+i} (zero history)
 *   Y = SiLU(c) + vhat
 * Shapes: H, k, v, Y, vhat, dY, dH, dk, dv [M][T][d] bf16; rms_w_h, rms_w_v
 * [d] fp32; conv_w [4][d] fp32; alpha, rrms_* [M][T] fp32; the weight
 * gradients are fp32 and overwritten.  d is a multiple of 512, at most 5120;
 * M, T >= 1 and M * T <= ENGRAM_GATECONV_ROWS_MAX.  All pointers device,
 * 16-byte aligned, outputs overlapping nothing; asynchronous on `stream`, no
 * allocation or synchronisation.  Errors as for the gate: ENGRAM_ERR_NULL,
 * ENGRAM_ERR_N_RANGE (sizes, or eps outside [0, 1] or NaN), ENGRAM_ERR_ALIGN,
 * ENGRAM_ERR_OVERLAP, all before any work is enqueued.
 * ========================================================================== */
#define ENGRAM_GATECONV_D_MAX 5120
#define ENGRAM_GATECONV_ROWS_MAX 4194304 /* M * T */

/* Forward; argument order of the page's forward(H, k, v, rms_w_h, rms_w_v,
 * conv_w), then its returned list [Y, vhat, alpha, rrms_h, rrms_k, rrms_v],
 * then the norms' eps (the page's default is 1e-6). */
engram_status engram_gateconv_fwd(const void *H, const void *k, const void *v, const float *rms_w_h,
                                  const float *rms_w_v, const float *conv_w, void *Y, void *vhat, float *alpha,
                                  float *rrms_h, float *rrms_k, float *rrms_v, int64_t M, int64_t T, int64_t d,
                                  float eps, void *stream);

/* Backward; argument order of the page's backward operator, forward(dY, H, k,
 * v, rms_w_h, rms_w_v, conv_w, vhat, alpha, rrms_h, rrms_k, rrms_v), then its
 * returned list [dH, dk, dv, drms_w_h, drms_w_v, dconv_w], then scratch of
 * engram_gateconv_bwd_workspace_bytes(M, T, d) bytes (contents ignored). */
engram_status engram_gateconv_bwd(const void *dY, const void *H, const void *k, const void *v,
                                  const float *rms_w_h, const float *rms_w_v, const float *conv_w,
                                  const void *vhat, const float *alpha, const float *rrms_h, const float *rrms_k,
                                  const float *rrms_v, void *dH, void *dk, void *dv, float *drms_w_h,
                                  float *drms_w_v, float *dconv_w, void *workspace, int64_t M, int64_t T,
                                  int64_t d, void *stream);

/* Scratch bytes of engram_gateconv_bwd (fp32 weight-gradient partials of each
 * token chunk, fp32 sums of those partials in blocks of 64 chunks, then one
 * fp32 per row); 0 for sizes the call would reject. */
size_t engram_gateconv_bwd_workspace_bytes(int64_t M, int64_t T, int64_t d);

/* Human-readable name of a status code (static storage). */
const char *engram_status_string(int status);

/* The hipError_t value behind the last ENGRAM_ERR_LAUNCH on this thread (0 if none). */
int engram_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
