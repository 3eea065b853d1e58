/*
 * engram_oracle.c -- plain, slow, fp64 CPU oracle for the four-stream Engram
 * saved-state gate (forward and explicit backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Sources (web pages; cited by title and paragraph):
 *   [GATE]  "Engram saved-state gate", cuDNN frontend documentation.
 *           - semantics paragraph: per token and stream, X and its key are
 *             RMS-normalised separately (eps 1e-20), x^ * weight * k^ is
 *             reduced in FP32, passed through a signed square root whose
 *             magnitude is clamped below at 1e-6, then a sigmoid; the output
 *             is X + gate * shared value, rounded once to BF16; a false token
 *             mask leaves X unchanged; weight is the FP32 product of the
 *             source q/k norm weights.
 *           - layout paragraph: packed KV holds four keys in its first
 *             4*5120 columns and the shared value in the last 5120; backward
 *             writes the same packed layout and sums the four shared-value
 *             contributions before the single BF16 cast.
 *           - saved-state paragraph: saved holds (gate, dot, rstd_X,
 *             rstd_key) per stream.
 *   [TK]    "tile-kernels 1.0.0" sdist listing, tests/engram/
 *           test_engram_gate_bwd.py: the backward is checked by running it
 *           on the reference forward's saved intermediates, with grad_weight
 *           summed over tokens.
 *
 * Readings where the pages leave a step open (numbered as in the design
 * notes):
 *   R1  sgn(0) = 0, so dot == 0 gives z = 0 and gate = 1/2.
 *   R2  The clamp passes the derivative when |dot| >= c and blocks it
 *       (derivative 0) when |dot| < c.
 *   R3  eps and c are the FP32 constants 1e-20f and 1e-6f, widened exactly
 *       to double.
 *   R4  No 1/sqrt(d) scale on the dot.
 *   R5  rstd = (mean_j v_j^2 + eps)^(-1/2); the weight is outside the norm.
 *   R6  The dot is over the normalised vectors: sum_j x^_j w_j k^_j.
 *   R7  A masked token saves gate = 0 (the effective gate); dot and both
 *       rstd are still the true values.  The backward has no mask argument,
 *       so every gate-derived gradient of a masked token vanishes through
 *       that zero.
 *   R8  saved[t][s][f], f = 0 gate, 1 dot, 2 rstd_X, 3 rstd_key.
 *   R9  key of stream s = KV columns [s*d, (s+1)*d); value = [4d, 5d).
 *   R10 Rounding: fp64 result -> fp32 (RNE) -> bf16 (RNE).  A masked
 *       token's output is a bit copy of X.
 *   R11 grad of the value = sum over the four streams of gate_s * G_s,
 *       accumulated before one cast.
 *   R12 grad_weight is the sum over all tokens, overwritten.
 *
 * The backward below is the analytic gradient of the forward definition for
 * the loss L = sum G * out, with x^ = rstd_X * x and k^ = rstd_key * k:
 *   dg    = sum_j G_j v_j
 *   dz    = dg * gate * (1 - gate)
 *   delta = (|dot| >= c) ? dz / (2 sqrt|dot|) : 0
 *   dx_j  = G_j + delta * rstd_X * (w_j k^_j - dot x^_j / d)
 *   dk_j  =       delta * rstd_key * (w_j x^_j - dot k^_j / d)
 *   dv_j  = sum_s gate_s G_{s,j}
 *   dw_{s,j} = sum_t delta_{t,s} x^_j k^_j
 * It is checked against fp64 central differences of the forward in the
 * CPU tests.
 *
 * d (the per-stream hidden size) is a parameter so that tiny cases can be
 * brute-forced; the library itself is fixed at d = 5120.  Streams are 4.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define NS 4 /* streams per token */

/* R3: the FP32 constants, widened exactly. */
static double eps_value(void) { return (double)1e-20f; }
static double clamp_value(void) { return (double)1e-6f; }

/* ---- storage-type conversions (bit definitions of IEEE binary32 / bf16) ---- */

static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16; /* bf16 is the upper half of a binary32 */
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN: keep sign, force quiet */
    return (uint16_t)((u >> 16) | 0x0040u);
  /* round to nearest, ties to even, on the 16 dropped bits */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* R10: fp64 -> fp32 (RNE, C's default rounding) -> bf16 (RNE). */
static uint16_t double_to_bf16(double v) { return float_to_bf16_rne((float)v); }

/* ---- scalar gate map (semantics paragraph; R1, R2, R3) ---- */

/* z = sgn(dot) * sqrt(max(|dot|, c)), sgn(0) = 0. */
static double signed_sqrt_clamped(double dot) {
  const double c = clamp_value();
  double a = fabs(dot);
  if (dot > 0.0) return sqrt(a > c ? a : c);
  if (dot < 0.0) return -sqrt(a > c ? a : c);
  return 0.0;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* d(gate)/d(dot), used only as a tolerance scale by the tests. */
static double gate_slope(double dot, double g) {
  const double c = clamp_value();
  if (fabs(dot) >= c) return g * (1.0 - g) / (2.0 * sqrt(fabs(dot)));
  return 0.0;
}

/* ---- one token, fp64 in / fp64 out ---- */

/*
 * Forward for one token.
 *   x[s*d + j], k[s*d + j], v[j], w[s*d + j]; m = token mask.
 *   out[s*d + j]; sv[4*s + f] per R8.
 *   aux (may be NULL): aux[2*s] = sum_j |x^_j w_j k^_j| (conditioning of the
 *   dot), aux[2*s+1] = d(gate)/d(dot) (0 for a masked token).
 */
static void fwd_token(int64_t d, const double *x, const double *k, const double *v, const double *w,
                      int m, double *out, double *sv, double *aux) {
  const double eps = eps_value();
  for (int s = 0; s < NS; ++s) {
    const double *xs = x + (int64_t)s * d, *ks = k + (int64_t)s * d, *ws = w + (int64_t)s * d;
    double sxx = 0.0, skk = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      sxx += xs[j] * xs[j];
      skk += ks[j] * ks[j];
    }
    const double rx = 1.0 / sqrt(sxx / (double)d + eps); /* R5 */
    const double rk = 1.0 / sqrt(skk / (double)d + eps);
    double dot = 0.0, absdot = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      double term = (xs[j] * rx) * ws[j] * (ks[j] * rk); /* R6 */
      dot += term;
      absdot += fabs(term);
    }
    const double g = sigmoid(signed_sqrt_clamped(dot));
    double *os = out + (int64_t)s * d;
    for (int64_t j = 0; j < d; ++j) os[j] = m ? xs[j] + g * v[j] : xs[j];
    sv[4 * s + 0] = m ? g : 0.0; /* R7 */
    sv[4 * s + 1] = dot;
    sv[4 * s + 2] = rx;
    sv[4 * s + 3] = rk;
    if (aux) {
      aux[2 * s + 0] = absdot;
      aux[2 * s + 1] = m ? gate_slope(dot, g) : 0.0;
    }
  }
}

/*
 * Backward for one token, from saved state sv (R8) and upstream gradient G.
 *   dx[s*d + j], dk[s*d + j], dv[j] are written; dw[s*d + j] is accumulated.
 *   mdx, mdk, mdv (may be NULL) receive a magnitude scale of each output
 *   element: the sum of |terms|, where |delta| is replaced by its bound
 *   through sum_j |G_j v_j| (dg is a cancelling fp32 sum on the device);
 *   mdw (may be NULL) accumulates that bound times |x^_j k^_j| over tokens.
 */
static void bwd_token(int64_t d, const double *x, const double *k, const double *v, const double *w,
                      const double *sv, const double *G, double *dx, double *dk, double *dv,
                      double *dw, double *mdx, double *mdk, double *mdv, double *mdw) {
  const double c = clamp_value();
  for (int64_t j = 0; j < d; ++j) {
    dv[j] = 0.0;
    if (mdv) mdv[j] = 0.0;
  }
  for (int s = 0; s < NS; ++s) {
    const double gate = sv[4 * s + 0], dot = sv[4 * s + 1];
    const double rx = sv[4 * s + 2], rk = sv[4 * s + 3];
    const double *xs = x + (int64_t)s * d, *ks = k + (int64_t)s * d, *ws = w + (int64_t)s * d;
    const double *Gs = G + (int64_t)s * d;
    double dg = 0.0, dgabs = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      dg += Gs[j] * v[j];
      dgabs += fabs(Gs[j] * v[j]);
    }
    const double dz = dg * gate * (1.0 - gate);
    const double delta = (fabs(dot) >= c) ? dz / (2.0 * sqrt(fabs(dot))) : 0.0; /* R2 */
    /* Magnitude scale of delta for the tolerance outputs: dg is a cancelling
       sum, so an evaluation of delta is bounded through sum_j |G_j v_j|. */
    const double dmag = (fabs(dot) >= c) ? dgabs * gate * (1.0 - gate) / (2.0 * sqrt(fabs(dot))) : 0.0;
    double *dxs = dx + (int64_t)s * d, *dks = dk + (int64_t)s * d, *dws = dw + (int64_t)s * d;
    for (int64_t j = 0; j < d; ++j) {
      const double xh = rx * xs[j], kh = rk * ks[j];
      const double tx1 = delta * rx * ws[j] * kh, tx2 = delta * rx * dot * xh / (double)d;
      const double tk1 = delta * rk * ws[j] * xh, tk2 = delta * rk * dot * kh / (double)d;
      dxs[j] = Gs[j] + tx1 - tx2;
      dks[j] = tk1 - tk2;
      dws[j] += delta * xh * kh;
      dv[j] += gate * Gs[j]; /* R11: streams summed in order 0..3 */
      if (mdx) mdx[(int64_t)s * d + j] = fabs(Gs[j]) + dmag * rx * (fabs(ws[j] * kh) + fabs(dot * xh) / (double)d);
      if (mdk) mdk[(int64_t)s * d + j] = dmag * rk * (fabs(ws[j] * xh) + fabs(dot * kh) / (double)d);
      if (mdv) mdv[j] += fabs(gate * Gs[j]);
      if (mdw) mdw[(int64_t)s * d + j] += dmag * fabs(xh * kh);
    }
  }
}

/* ---- a minimal parallel-for over contiguous token ranges ---- */

typedef struct job job;
typedef void (*range_fn)(job *, int64_t t0, int64_t t1, int tid);

struct job {
  range_fn fn;
  int64_t n;
  int nthreads;
  int64_t d;
  /* fp64 entry points */
  const double *x64, *kv64, *w64, *sv64, *g64;
  double *out64, *dx64, *dkv64, *aux;
  /* storage-type entry points */
  const uint16_t *x16, *kv16, *g16;
  const float *w32, *sv32;
  uint16_t *out16, *dx16, *dkv16;
  float *saved32;
  const uint8_t *mask;
  double *saved64;
  double *mdx, *mdkv;
  /* per-thread accumulators for grad_weight and its magnitude: [nthreads][4d] */
  double *dw_acc, *mdw_acc;
  int failed;
};

typedef struct {
  job *j;
  int tid;
} thread_arg;

static void *thread_main(void *p) {
  thread_arg *a = (thread_arg *)p;
  job *j = a->j;
  int64_t per = (j->n + j->nthreads - 1) / j->nthreads;
  int64_t t0 = per * a->tid, t1 = t0 + per;
  if (t1 > j->n) t1 = j->n;
  if (t0 < t1) j->fn(j, t0, t1, a->tid);
  return NULL;
}

static int run_job(job *j) {
  if (j->nthreads < 1) j->nthreads = 1;
  if (j->nthreads > 256) j->nthreads = 256;
  if ((int64_t)j->nthreads > j->n) j->nthreads = (int)(j->n > 0 ? j->n : 1);
  pthread_t th[256];
  thread_arg args[256];
  int started = 0;
  for (int i = 0; i < j->nthreads; ++i) {
    args[i].j = j;
    args[i].tid = i;
    if (i == 0) continue;
    if (pthread_create(&th[i], NULL, thread_main, &args[i]) != 0) break;
    started = i;
  }
  thread_main(&args[0]);
  for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
  /* threads that failed to start: run their ranges here, in order */
  for (int i = started + 1; i < j->nthreads; ++i) thread_main(&args[i]);
  return j->failed;
}

/* per-thread scratch: x, k (4d each), v (d), w (4d), G (4d), out/dx (4d), dk (4d), dv (d),
   mags (4d + 4d + d) */
static double *alloc_scratch(int64_t d) { return (double *)calloc((size_t)(40 * d + 64), sizeof(double)); }

/* ---- fp64 entry points (for finite differences and invariants) ---- */

static void fwd64_range(job *j, int64_t t0, int64_t t1, int tid) {
  (void)tid;
  const int64_t d = j->d;
  for (int64_t t = t0; t < t1; ++t) {
    const double *xt = j->x64 + t * NS * d, *kvt = j->kv64 + t * 5 * d;
    fwd_token(d, xt, kvt, kvt + NS * d, j->w64, j->mask[t] != 0, j->out64 + t * NS * d,
              j->saved64 + t * 16, j->aux ? j->aux + t * 8 : NULL);
  }
}

/*
 * Forward in fp64 with no rounding of inputs or outputs.
 *   x [n][4][d], kv [n][5d], w [4][d], mask [n] (nonzero = true)
 *   out [n][4][d], saved [n][4][4], aux [n][4][2] (may be NULL)
 * Returns 0, or -1 for bad arguments.
 */
int engram_oracle_fwd_f64(int64_t d, int64_t n, const double *x, const double *kv, const double *w,
                          const uint8_t *mask, double *out, double *saved, double *aux, int nthreads) {
  if (d < 1 || n < 0 || (n > 0 && (!x || !kv || !w || !mask || !out || !saved))) return -1;
  job j;
  memset(&j, 0, sizeof j);
  j.fn = fwd64_range;
  j.n = n;
  j.nthreads = nthreads;
  j.d = d;
  j.x64 = x;
  j.kv64 = kv;
  j.w64 = w;
  j.mask = mask;
  j.out64 = out;
  j.saved64 = saved;
  j.aux = aux;
  if (n == 0) return 0;
  return run_job(&j);
}

static void bwd64_range(job *j, int64_t t0, int64_t t1, int tid) {
  const int64_t d = j->d;
  double *scr = alloc_scratch(d);
  if (!scr) {
    j->failed = -2;
    return;
  }
  double *dv = scr, *mdv = scr + d;
  double *dwacc = j->dw_acc + (int64_t)tid * NS * d;
  double *mdwacc = j->mdw_acc ? j->mdw_acc + (int64_t)tid * NS * d : NULL;
  for (int64_t t = t0; t < t1; ++t) {
    const double *xt = j->x64 + t * NS * d, *kvt = j->kv64 + t * 5 * d;
    double *dkvt = j->dkv64 + t * 5 * d;
    bwd_token(d, xt, kvt, kvt + NS * d, j->w64, j->sv64 + t * 16, j->g64 + t * NS * d,
              j->dx64 + t * NS * d, dkvt, dv, dwacc, j->mdx ? j->mdx + t * NS * d : NULL,
              j->mdkv ? j->mdkv + t * 5 * d : NULL, j->mdkv ? mdv : NULL, mdwacc);
    for (int64_t q = 0; q < d; ++q) {
      dkvt[NS * d + q] = dv[q];
      if (j->mdkv) j->mdkv[t * 5 * d + NS * d + q] = mdv[q];
    }
  }
  free(scr);
}

static void reduce_dw(const job *j, int64_t d, double *dw, double *mdw) {
  for (int64_t q = 0; q < NS * d; ++q) {
    double s = 0.0, m = 0.0;
    for (int i = 0; i < j->nthreads; ++i) { /* fixed thread order */
      s += j->dw_acc[(int64_t)i * NS * d + q];
      if (j->mdw_acc) m += j->mdw_acc[(int64_t)i * NS * d + q];
    }
    dw[q] = s;
    if (mdw) mdw[q] = m;
  }
}

/*
 * Backward in fp64 from a given fp64 saved state (no rounding anywhere).
 *   saved [n][4][4] (R8), g = grad_out [n][4][d]
 *   dx [n][4][d], dkv [n][5d] (packed like KV), dw [4][d]
 *   mag_dx, mag_dkv, mag_dw (may be NULL): sum of |terms| per element.
 */
int engram_oracle_bwd_f64(int64_t d, int64_t n, const double *x, const double *kv, const double *w,
                          const double *saved, const double *g, double *dx, double *dkv, double *dw,
                          double *mag_dx, double *mag_dkv, double *mag_dw, int nthreads) {
  if (d < 1 || n < 0 || !w || !dw) return -1;
  if (n > 0 && (!x || !kv || !saved || !g || !dx || !dkv)) return -1;
  job j;
  memset(&j, 0, sizeof j);
  j.fn = bwd64_range;
  j.n = n;
  j.nthreads = nthreads;
  j.d = d;
  j.x64 = x;
  j.kv64 = kv;
  j.w64 = w;
  j.sv64 = saved;
  j.g64 = g;
  j.dx64 = dx;
  j.dkv64 = dkv;
  j.mdx = mag_dx;
  j.mdkv = mag_dkv;
  if (n == 0) {
    for (int64_t q = 0; q < NS * d; ++q) {
      dw[q] = 0.0;
      if (mag_dw) mag_dw[q] = 0.0;
    }
    return 0;
  }
  /* clamp the thread count the same way run_job will, then size accumulators */
  if (j.nthreads < 1) j.nthreads = 1;
  if (j.nthreads > 256) j.nthreads = 256;
  if ((int64_t)j.nthreads > n) j.nthreads = (int)n;
  j.dw_acc = (double *)calloc((size_t)j.nthreads * NS * d, sizeof(double));
  j.mdw_acc = mag_dw ? (double *)calloc((size_t)j.nthreads * NS * d, sizeof(double)) : NULL;
  if (!j.dw_acc || (mag_dw && !j.mdw_acc)) {
    free(j.dw_acc);
    free(j.mdw_acc);
    return -2;
  }
  int rc = run_job(&j);
  if (rc == 0) reduce_dw(&j, d, dw, mag_dw);
  free(j.dw_acc);
  free(j.mdw_acc);
  return rc;
}

/* ---- storage-type entry points (bf16 / fp32 in, rounded outputs) ---- */

static void fwd16_range(job *j, int64_t t0, int64_t t1, int tid) {
  (void)tid;
  const int64_t d = j->d;
  double *scr = alloc_scratch(d);
  if (!scr) {
    j->failed = -2;
    return;
  }
  double *x = scr, *kv = scr + 4 * d, *w = scr + 9 * d, *out = scr + 13 * d;
  double sv[16], aux[8];
  for (int64_t q = 0; q < NS * d; ++q) w[q] = (double)j->w32[q];
  for (int64_t t = t0; t < t1; ++t) {
    const uint16_t *xt = j->x16 + t * NS * d, *kvt = j->kv16 + t * 5 * d;
    for (int64_t q = 0; q < NS * d; ++q) x[q] = bf16_bits_to_double(xt[q]);
    for (int64_t q = 0; q < 5 * d; ++q) kv[q] = bf16_bits_to_double(kvt[q]);
    const int m = j->mask[t] != 0;
    fwd_token(d, x, kv, kv + NS * d, w, m, out, sv, aux);
    uint16_t *ot = j->out16 + t * NS * d;
    for (int64_t q = 0; q < NS * d; ++q) ot[q] = m ? double_to_bf16(out[q]) : xt[q]; /* R10 */
    if (j->out64)
      for (int64_t q = 0; q < NS * d; ++q) j->out64[t * NS * d + q] = out[q];
    for (int q = 0; q < 16; ++q) {
      j->saved32[t * 16 + q] = (float)sv[q];
      if (j->saved64) j->saved64[t * 16 + q] = sv[q];
    }
    if (j->aux)
      for (int q = 0; q < 8; ++q) j->aux[t * 8 + q] = aux[q];
  }
  free(scr);
}

/*
 * Forward on storage types.
 *   x [n][4][d] bf16 bits, kv [n][5d] bf16 bits, w [4][d] fp32, mask [n]
 *   out [n][4][d] bf16 bits, saved [n][4][4] fp32 (rounded from fp64)
 *   out64 [n][4][d], saved64 [n][4][4], aux [n][4][2]: optional fp64 views
 *   before rounding (NULL to skip).
 */
int engram_oracle_fwd_bf16(int64_t d, int64_t n, const uint16_t *x, const uint16_t *kv, const float *w,
                           const uint8_t *mask, uint16_t *out, float *saved, double *out64,
                           double *saved64, double *aux, int nthreads) {
  if (d < 1 || n < 0 || (n > 0 && (!x || !kv || !w || !mask || !out || !saved))) return -1;
  job j;
  memset(&j, 0, sizeof j);
  j.fn = fwd16_range;
  j.n = n;
  j.nthreads = nthreads;
  j.d = d;
  j.x16 = x;
  j.kv16 = kv;
  j.w32 = w;
  j.mask = mask;
  j.out16 = out;
  j.saved32 = saved;
  j.out64 = out64;
  j.saved64 = saved64;
  j.aux = aux;
  if (n == 0) return 0;
  return run_job(&j);
}

static void bwd16_range(job *j, int64_t t0, int64_t t1, int tid) {
  const int64_t d = j->d;
  double *scr = alloc_scratch(d);
  if (!scr) {
    j->failed = -2;
    return;
  }
  double *x = scr, *kv = scr + 4 * d, *w = scr + 9 * d, *G = scr + 13 * d;
  double *dx = scr + 17 * d, *dk = scr + 21 * d, *dv = scr + 25 * d;
  double *mdx = scr + 26 * d, *mdk = scr + 30 * d, *mdv = scr + 34 * d;
  double sv[16];
  double *dwacc = j->dw_acc + (int64_t)tid * NS * d;
  double *mdwacc = j->mdw_acc ? j->mdw_acc + (int64_t)tid * NS * d : NULL;
  for (int64_t q = 0; q < NS * d; ++q) w[q] = (double)j->w32[q];
  for (int64_t t = t0; t < t1; ++t) {
    const uint16_t *xt = j->x16 + t * NS * d, *kvt = j->kv16 + t * 5 * d, *gt = j->g16 + t * NS * d;
    for (int64_t q = 0; q < NS * d; ++q) {
      x[q] = bf16_bits_to_double(xt[q]);
      G[q] = bf16_bits_to_double(gt[q]);
    }
    for (int64_t q = 0; q < 5 * d; ++q) kv[q] = bf16_bits_to_double(kvt[q]);
    for (int q = 0; q < 16; ++q) sv[q] = (double)j->sv32[t * 16 + q];
    bwd_token(d, x, kv, kv + NS * d, w, sv, G, dx, dk, dv, dwacc, mdx, mdk, mdv, mdwacc);
    uint16_t *dxt = j->dx16 + t * NS * d, *dkvt = j->dkv16 + t * 5 * d;
    for (int64_t q = 0; q < NS * d; ++q) {
      dxt[q] = double_to_bf16(dx[q]);
      dkvt[q] = double_to_bf16(dk[q]);
    }
    for (int64_t q = 0; q < d; ++q) dkvt[NS * d + q] = double_to_bf16(dv[q]);
    if (j->dx64)
      for (int64_t q = 0; q < NS * d; ++q) j->dx64[t * NS * d + q] = dx[q];
    if (j->dkv64) {
      for (int64_t q = 0; q < NS * d; ++q) j->dkv64[t * 5 * d + q] = dk[q];
      for (int64_t q = 0; q < d; ++q) j->dkv64[t * 5 * d + NS * d + q] = dv[q];
    }
    if (j->mdx)
      for (int64_t q = 0; q < NS * d; ++q) j->mdx[t * NS * d + q] = mdx[q];
    if (j->mdkv) {
      for (int64_t q = 0; q < NS * d; ++q) j->mdkv[t * 5 * d + q] = mdk[q];
      for (int64_t q = 0; q < d; ++q) j->mdkv[t * 5 * d + NS * d + q] = mdv[q];
    }
  }
  free(scr);
}

/*
 * Backward on storage types, from a given fp32 saved state (as the
 * tile-kernels backward test feeds the reference forward's intermediates).
 *   x, kv, g: bf16 bits; w: fp32 [4][d]; saved: fp32 [n][4][4]
 *   dx [n][4][d], dkv [n][5d]: bf16 bits; dw [4][d]: fp32
 *   dx64, dkv64, dw64, mag_dx, mag_dkv, mag_dw: optional fp64 views.
 */
int engram_oracle_bwd_bf16(int64_t d, int64_t n, const uint16_t *x, const uint16_t *kv, const float *w,
                           const float *saved, const uint16_t *g, uint16_t *dx, uint16_t *dkv, float *dw,
                           double *dx64, double *dkv64, double *dw64, double *mag_dx, double *mag_dkv,
                           double *mag_dw, int nthreads) {
  if (d < 1 || n < 0 || !w || !dw) return -1;
  if (n > 0 && (!x || !kv || !saved || !g || !dx || !dkv)) return -1;
  job j;
  memset(&j, 0, sizeof j);
  j.fn = bwd16_range;
  j.n = n;
  j.d = d;
  j.nthreads = nthreads;
  j.x16 = x;
  j.kv16 = kv;
  j.w32 = w;
  j.sv32 = saved;
  j.g16 = g;
  j.dx16 = dx;
  j.dkv16 = dkv;
  j.dx64 = dx64;
  j.dkv64 = dkv64;
  j.mdx = mag_dx;
  j.mdkv = mag_dkv;
  if (j.nthreads < 1) j.nthreads = 1;
  if (j.nthreads > 256) j.nthreads = 256;
  if (n > 0 && (int64_t)j.nthreads > n) j.nthreads = (int)n;
  j.dw_acc = (double *)calloc((size_t)j.nthreads * NS * d, sizeof(double));
  j.mdw_acc = mag_dw ? (double *)calloc((size_t)j.nthreads * NS * d, sizeof(double)) : NULL;
  if (!j.dw_acc || (mag_dw && !j.mdw_acc)) {
    free(j.dw_acc);
    free(j.mdw_acc);
    return -2;
  }
  int rc = 0;
  if (n > 0) rc = run_job(&j);
  if (rc == 0) {
    double *tmp = (double *)malloc((size_t)NS * d * sizeof(double));
    if (!tmp) {
      rc = -2;
    } else {
      reduce_dw(&j, d, tmp, mag_dw);
      for (int64_t q = 0; q < NS * d; ++q) {
        dw[q] = (float)tmp[q];
        if (dw64) dw64[q] = tmp[q];
      }
      free(tmp);
    }
  }
  free(j.dw_acc);
  free(j.mdw_acc);
  return rc;
}

/* Exposed so the tests can pin the conversion itself against its definition. */
uint16_t engram_oracle_f32_to_bf16(float f) { return float_to_bf16_rne(f); }

/* ---- fused weight and its product rule ---- */

/*
 * weight = fp32(wh) * fp32(we) for bf16 inputs ("Engram saved-state gate",
 * semantics paragraph: the weight argument is the FP32 product of the source
 * q/k normalisation weights).  Formed in fp64 and rounded to fp32; for
 * normal-range inputs the product has at most 16 significant bits, so both
 * steps are exact.
 */
int engram_oracle_fused_weight(int64_t count, const uint16_t *wh, const uint16_t *we, float *weight) {
  if (count < 0 || (count > 0 && (!wh || !we || !weight))) return -1;
  for (int64_t q = 0; q < count; ++q) weight[q] = (float)(bf16_bits_to_double(wh[q]) * bf16_bits_to_double(we[q]));
  return 0;
}

/*
 * Product rule of weight = wh * we: with G_w = dL/dweight,
 *   dL/dwh = G_w * we,  dL/dwe = G_w * wh      (fp64, no rounding)
 * The gate page leaves this to the caller; the "tile-kernels 1.0.0" backward
 * test forms it this way from the summed grad_weight.
 */
int engram_oracle_weight_grads(int64_t count, const double *dw, const uint16_t *wh, const uint16_t *we,
                               double *grad_wh, double *grad_we) {
  if (count < 0 || (count > 0 && (!dw || !wh || !we || !grad_wh || !grad_we))) return -1;
  for (int64_t q = 0; q < count; ++q) {
    grad_wh[q] = dw[q] * bf16_bits_to_double(we[q]);
    grad_we[q] = dw[q] * bf16_bits_to_double(wh[q]);
  }
  return 0;
}
