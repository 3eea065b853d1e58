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
 *           - semantics paragraph: the map evaluated here, per token t and
 *             stream s, with m the token's mask bit:
 *               r_x = (mean_j x_j^2 + eps)^(-1/2),  r_k the same for the key
 *               dot = sum_j (r_x x_j) w_j (r_k k_j)          (eps = 1e-20)
 *               gate = sigmoid(sgn(dot) * sqrt(max(|dot|, 1e-6)))
 *               out = m ? bf16(x + gate v) : x
 *             where w is a weight the caller forms as a product of two
 *             normalisation weights (fused_weight below).
 *           - layout paragraph: a KV row is [key 0 | key 1 | key 2 | key 3 |
 *             value], 5120 columns each; grad_kv uses the same packing, and
 *             its value part is one bf16 rounding of the fp32 sum over the
 *             four streams.
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

/* ======================================================================
 * Engram GateConv ("Engram Operators", TileOPs; GateConv section).
 *
 * The page gives the stages (RMSNorm gating -> causal depthwise conv1d ->
 * SiLU + residual), the shapes and the saved tensors, but no formulas.
 * Readings (the plainest the page supports):
 *   G1  h^ = H rrms_h w_h, k^ = k rrms_k w_h: one RMSNorm weight for H and k,
 *       rrms = (mean of squares + eps)^(-1/2), eps default 1e-6.
 *   G2  alpha = sigmoid(<h^, k^> / sqrt(d)), one scalar per (m, t).
 *   G3  vhat = alpha v (the gated value; saved).
 *   G4  u = vhat rrms_v w_v, rrms_v the reciprocal RMS of vhat (saved).
 *   G5  c[t] = sum_{i<4} conv_w[i] u[t-3+i], causal within each sequence m,
 *       zero history before t = 0, dilation 1 (the op has no dilation).
 *   G6  Y = SiLU(c) + vhat, SiLU(c) = c sigmoid(c).
 * Parity unpinned on two points: the page fixes neither the 1/sqrt(d) in G2
 * (it names a scalar gate from the normalised H and k, nothing about a scale;
 * the scaled dot product is the usual form of such a gate, and without it the
 * logit grows sqrt(d) times and alpha saturates at 0 or 1 on most rows) nor
 * which tensor the "+ residual" of G6 adds (it lists SiLU + residual among the
 * op's stages, and separately says the caller adds Y to H; vhat is the one
 * op-internal tensor of matching shape -- the alternative Y = SiLU(c) drops
 * the vhat term from Y and from the gradient of vhat).  The tests pin the
 * oracle to these readings, not to the page.
 * Layout: H, k, v, Y, vhat, dY, dH, dk, dv [M][T][d]; alpha, rrms_* [M][T];
 * w_h, w_v [d]; conv_w [4][d].
 *
 * Magnitude outputs (for tolerances only): a first-order bound m(q) of the
 * terms that build each output, so that an fp32 evaluation errs by a modest
 * multiple of 2^-24 m(q): m(a+b) = m(a)+m(b), m(ab) = m(a)m(b), and a scalar
 * map f adds |f'(x)| m(x) to |f(x)|.
 * ====================================================================== */

#define GC_TAPS 4

static double silu(double c) { return c * sigmoid(c); }
static double silu_grad(double c) {
  const double s = sigmoid(c);
  return s * (1.0 + c * (1.0 - s));
}

/*
 * Forward for one sequence of T tokens (fp64).  u_scr and um_scr are
 * scratch of T*d doubles, da_scr of T doubles.  magY may be NULL.
 */
static void gateconv_fwd_seq(int64_t T, int64_t d, double eps, const double *H, const double *k, const double *v,
                             const double *wh, const double *wv, const double *cw, double *Y, double *vhat,
                             double *alpha, double *rrh, double *rrk, double *rrv, double *magY, double *u_scr,
                             double *um_scr, double *da_scr) {
  const double sd = sqrt((double)d);
  for (int64_t t = 0; t < T; ++t) {
    const double *Ht = H + t * d, *kt = k + t * d, *vt = v + t * d;
    double shh = 0.0, skk = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      shh += Ht[j] * Ht[j];
      skk += kt[j] * kt[j];
    }
    const double rh = 1.0 / sqrt(shh / (double)d + eps), rk = 1.0 / sqrt(skk / (double)d + eps); /* G1 */
    double s = 0.0, smag = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      const double term = (Ht[j] * rh * wh[j]) * (kt[j] * rk * wh[j]);
      s += term;
      smag += fabs(term);
    }
    s /= sd; /* G2 */
    smag /= sd;
    const double a = sigmoid(s);
    da_scr[t] = a * (1.0 - a) * smag; /* magnitude of alpha's error term */
    double svv = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      vhat[t * d + j] = a * vt[j]; /* G3 */
      svv += vhat[t * d + j] * vhat[t * d + j];
    }
    const double rv = 1.0 / sqrt(svv / (double)d + eps); /* G4 */
    for (int64_t j = 0; j < d; ++j) {
      u_scr[t * d + j] = vhat[t * d + j] * rv * wv[j];
      /* alpha enters u directly and through rrms_v (at most as strongly again) */
      um_scr[t * d + j] = fabs(u_scr[t * d + j]) * (1.0 + (a > 0.0 ? 2.0 * da_scr[t] / a : 0.0));
    }
    alpha[t] = a;
    rrh[t] = rh;
    rrk[t] = rk;
    rrv[t] = rv;
  }
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = 0; j < d; ++j) {
      double c = 0.0, cm = 0.0;
      for (int i = 0; i < GC_TAPS; ++i) { /* G5 */
        const int64_t tau = t - (GC_TAPS - 1) + i;
        if (tau < 0) continue;
        c += cw[(int64_t)i * d + j] * u_scr[tau * d + j];
        cm += fabs(cw[(int64_t)i * d + j]) * um_scr[tau * d + j];
      }
      Y[t * d + j] = silu(c) + vhat[t * d + j]; /* G6 */
      if (magY)
        magY[t * d + j] = fabs(silu(c)) + fabs(silu_grad(c)) * cm + fabs(vhat[t * d + j]) +
                          fabs(v[t * d + j]) * da_scr[t];
    }
  }
}

/* ---- sequences in parallel: thread i takes the contiguous range i of [0, M) ---- */

typedef struct {
  void (*fn)(void *ctx, int64_t m0, int64_t m1, int tid);
  void *ctx;
  int64_t n;
  int nthreads, tid;
} seq_arg;

static void *seq_main(void *p) {
  seq_arg *a = (seq_arg *)p;
  const int64_t per = (a->n + a->nthreads - 1) / a->nthreads;
  int64_t m0 = per * a->tid, m1 = m0 + per;
  if (m1 > a->n) m1 = a->n;
  if (m0 < m1) a->fn(a->ctx, m0, m1, a->tid);
  return NULL;
}

static int seq_threads(int64_t M, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  if ((int64_t)threads > M) threads = (int)(M > 0 ? M : 1);
  return threads;
}

static void run_sequences(int64_t M, int nthreads, void (*fn)(void *, int64_t, int64_t, int), void *ctx) {
  pthread_t th[64];
  seq_arg args[64];
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    args[i] = (seq_arg){fn, ctx, M, nthreads, i};
    if (i == 0) continue;
    if (pthread_create(&th[i], NULL, seq_main, &args[i]) != 0) break;
    started = i;
  }
  seq_main(&args[0]);
  for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
  for (int i = started + 1; i < nthreads; ++i) seq_main(&args[i]); /* threads that did not start */
}

typedef struct {
  int64_t T, d;
  double eps;
  const double *H, *k, *v, *wh, *wv, *cw;
  double *Y, *vhat, *alpha, *rrh, *rrk, *rrv, *magY;
  int failed;
} gc_fwd_ctx;

static void gc_fwd_range(void *p, int64_t m0, int64_t m1, int tid) {
  gc_fwd_ctx *c = (gc_fwd_ctx *)p;
  (void)tid;
  const int64_t T = c->T, d = c->d;
  double *scr = (double *)malloc(((size_t)2 * T * d + (size_t)T + 1) * sizeof(double));
  if (!scr) {
    c->failed = -2;
    return;
  }
  for (int64_t m = m0; m < m1; ++m) {
    const int64_t o = m * T * d, os = m * T;
    gateconv_fwd_seq(T, d, c->eps, c->H + o, c->k + o, c->v + o, c->wh, c->wv, c->cw, c->Y + o, c->vhat + o,
                     c->alpha + os, c->rrh + os, c->rrk + os, c->rrv + os, c->magY ? c->magY + o : NULL, scr,
                     scr + T * d, scr + 2 * T * d);
  }
  free(scr);
}

/*
 * Forward, fp64 in and out, sequences spread over `threads` threads (each
 * sequence is computed by one thread exactly as alone).  Returns 0, or -1 for
 * bad arguments, -2 when out of memory.  magY may be NULL.
 */
int engram_oracle_gateconv_fwd_f64(int64_t M, int64_t T, int64_t d, double eps, const double *H, const double *k,
                                   const double *v, const double *wh, const double *wv, const double *cw, double *Y,
                                   double *vhat, double *alpha, double *rrh, double *rrk, double *rrv,
                                   double *magY, int threads) {
  if (M < 0 || T < 0 || d < 1) return -1;
  if (M * T > 0 && (!H || !k || !v || !wh || !wv || !cw || !Y || !vhat || !alpha || !rrh || !rrk || !rrv))
    return -1;
  if (M * T == 0) return 0;
  gc_fwd_ctx c = {T, d, eps, H, k, v, wh, wv, cw, Y, vhat, alpha, rrh, rrk, rrv, magY, 0};
  run_sequences(M, seq_threads(M, threads), gc_fwd_range, &c);
  return c.failed;
}

/*
 * Backward for one sequence, from the saved tensors (vhat, alpha, rrms_h,
 * rrms_k, rrms_v), as the page's backward op takes them.  Gradient of
 * L = sum dY * Y through G1..G6:
 *   u_t   = vhat_t rrms_v w_v;  c_t = sum_i cw_i u_{t-3+i}
 *   dc_t  = dY_t SiLU'(c_t);    dcw_i += dc_t u_{t-3+i}
 *   du_t  = sum_i cw_i dc_{t+3-i}
 *   dwv  += du_t vhat_t rrms_v
 *   dvhat = dY_t + rrms_v (w_v du_t - vhat_t rrms_v^2 <du_t w_v, vhat_t> / d)
 *   dalpha = <dvhat, v_t>;  dv = alpha dvhat;  ds = dalpha alpha (1 - alpha)
 *   dh^ = ds k^ / sqrt(d);  dk^ = ds h^ / sqrt(d)
 *   dH  = rrms_h (w_h dh^ - H rrms_h^2 <dh^ w_h, H> / d)     (likewise dk)
 *   dwh += dh^ H rrms_h + dk^ k rrms_k
 * Scratch: 3*T*d + 2*T doubles.  Accumulates dwh, dwv, dcw (and their
 * magnitudes when mag* are given).
 */
static void gateconv_bwd_seq(int64_t T, int64_t d, const double *dY, const double *H, const double *k,
                             const double *v, const double *wh, const double *wv, const double *cw,
                             const double *vhat, const double *alpha, const double *rrh, const double *rrk,
                             const double *rrv, double *dH, double *dk, double *dv, double *dwh, double *dwv,
                             double *dcw, double *magH, double *magk, double *magv, double *mdwh, double *mdwv,
                             double *mdcw, double *scr) {
  const double sd = sqrt((double)d);
  double *u = scr, *dc = scr + T * d, *dcm = scr + 2 * T * d;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < d; ++j) u[t * d + j] = vhat[t * d + j] * rrv[t] * wv[j];
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < d; ++j) {
      double c = 0.0, cm = 0.0;
      for (int i = 0; i < GC_TAPS; ++i) {
        const int64_t tau = t - (GC_TAPS - 1) + i;
        if (tau < 0) continue;
        c += cw[(int64_t)i * d + j] * u[tau * d + j];
        cm += fabs(cw[(int64_t)i * d + j] * u[tau * d + j]);
      }
      const double g = silu_grad(c);
      /* SiLU'' is bounded by 0.5: error of c moves dc by at most |dY| 0.5 m(c) */
      dc[t * d + j] = dY[t * d + j] * g;
      dcm[t * d + j] = fabs(dY[t * d + j]) * (fabs(g) + 0.5 * cm);
      for (int i = 0; i < GC_TAPS; ++i) {
        const int64_t tau = t - (GC_TAPS - 1) + i;
        if (tau < 0) continue;
        dcw[(int64_t)i * d + j] += dc[t * d + j] * u[tau * d + j];
        if (mdcw) mdcw[(int64_t)i * d + j] += dcm[t * d + j] * fabs(u[tau * d + j]);
      }
    }
  for (int64_t t = 0; t < T; ++t) {
    const double *Ht = H + t * d, *kt = k + t * d, *vt = v + t * d, *vh = vhat + t * d;
    const double a = alpha[t], rh = rrh[t], rk = rrk[t], rv = rrv[t];
    /* du_t and the first row sum */
    double s1 = 0.0, s1m = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      double du = 0.0, dum = 0.0;
      for (int i = 0; i < GC_TAPS; ++i) {
        const int64_t tau = t + (GC_TAPS - 1) - i;
        if (tau >= T) continue;
        du += cw[(int64_t)i * d + j] * dc[tau * d + j];
        dum += fabs(cw[(int64_t)i * d + j]) * dcm[tau * d + j];
      }
      dv[t * d + j] = du; /* temporarily hold du */
      if (magv) magv[t * d + j] = dum;
      s1 += du * wv[j] * vh[j];
      s1m += dum * fabs(wv[j] * vh[j]);
      dwv[j] += du * vh[j] * rv;
      if (mdwv) mdwv[j] += dum * fabs(vh[j] * rv);
    }
    /* dvhat and dalpha */
    double dal = 0.0, dalm = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      const double du = dv[t * d + j];
      const double dvh = dY[t * d + j] + rv * (wv[j] * du - vh[j] * rv * rv * s1 / (double)d);
      const double dvhm = fabs(dY[t * d + j]) +
                          rv * (fabs(wv[j]) * (magv ? magv[t * d + j] : fabs(du)) + fabs(vh[j]) * rv * rv * s1m / (double)d);
      dv[t * d + j] = dvh; /* hold dvhat */
      if (magv) magv[t * d + j] = dvhm;
      dal += dvh * vt[j];
      dalm += dvhm * fabs(vt[j]);
    }
    const double ds = dal * a * (1.0 - a), dsm = dalm * a * (1.0 - a);
    double p = 0.0, pm = 0.0; /* sum_j H k w_h^2 */
    for (int64_t j = 0; j < d; ++j) {
      p += Ht[j] * kt[j] * wh[j] * wh[j];
      pm += fabs(Ht[j] * kt[j]) * wh[j] * wh[j];
    }
    const double s2 = ds / sd * rk * p, s3 = ds / sd * rh * p; /* <dh^ w_h, H>, <dk^ w_h, k> */
    const double s2m = dsm / sd * rk * pm, s3m = dsm / sd * rh * pm;
    for (int64_t j = 0; j < d; ++j) {
      const double hh = Ht[j] * rh * wh[j], kh = kt[j] * rk * wh[j];
      const double dhh = ds * kh / sd, dkh = ds * hh / sd;
      dH[t * d + j] = rh * (wh[j] * dhh - Ht[j] * rh * rh * s2 / (double)d);
      dk[t * d + j] = rk * (wh[j] * dkh - kt[j] * rk * rk * s3 / (double)d);
      dwh[j] += dhh * Ht[j] * rh + dkh * kt[j] * rk;
      if (magH) magH[t * d + j] = rh * (fabs(wh[j]) * dsm * fabs(kh) / sd + fabs(Ht[j]) * rh * rh * s2m / (double)d);
      if (magk) magk[t * d + j] = rk * (fabs(wh[j]) * dsm * fabs(hh) / sd + fabs(kt[j]) * rk * rk * s3m / (double)d);
      if (mdwh) mdwh[j] += dsm * (fabs(kh * Ht[j] * rh) + fabs(hh * kt[j] * rk)) / sd;
    }
    for (int64_t j = 0; j < d; ++j) {
      if (magv) magv[t * d + j] *= a; /* alpha is given (saved), so it adds no error */
      dv[t * d + j] *= a;
    }
  }
}

typedef struct {
  int64_t T, d;
  const double *dY, *H, *k, *v, *wh, *wv, *cw, *vhat, *alpha, *rrh, *rrk, *rrv;
  double *dH, *dk, *dv, *magH, *magk, *magv;
  double *acc; /* per thread [12][d]: dwh, dwv, dcw (4d), then their magnitudes */
  int mags, failed;
} gc_bwd_ctx;

static void gc_bwd_range(void *p, int64_t m0, int64_t m1, int tid) {
  gc_bwd_ctx *c = (gc_bwd_ctx *)p;
  const int64_t T = c->T, d = c->d;
  double *scr = (double *)malloc(((size_t)3 * T * d + 1) * sizeof(double));
  if (!scr) {
    c->failed = -2;
    return;
  }
  double *a = c->acc + (int64_t)tid * 12 * d;
  for (int64_t m = m0; m < m1; ++m) {
    const int64_t o = m * T * d, os = m * T;
    gateconv_bwd_seq(T, d, c->dY + o, c->H + o, c->k + o, c->v + o, c->wh, c->wv, c->cw, c->vhat + o,
                     c->alpha + os, c->rrh + os, c->rrk + os, c->rrv + os, c->dH + o, c->dk + o, c->dv + o, a, a + d,
                     a + 2 * d, c->magH ? c->magH + o : NULL, c->magk ? c->magk + o : NULL,
                     c->magv ? c->magv + o : NULL, c->mags ? a + 6 * d : NULL, c->mags ? a + 7 * d : NULL,
                     c->mags ? a + 8 * d : NULL, scr);
  }
  free(scr);
}

/*
 * Backward, fp64 in and out, from fp64 saved tensors, sequences spread over
 * `threads` threads.  dwh, dwv [d] and dcw [4][d] are overwritten with the
 * sums over all M*T tokens: each thread sums its sequences in order, then the
 * thread sums are added in thread order.  The mag* outputs may be NULL (the
 * three weight magnitudes together).
 */
int engram_oracle_gateconv_bwd_f64(int64_t M, int64_t T, int64_t d, const double *dY, const double *H,
                                   const double *k, const double *v, const double *wh, const double *wv,
                                   const double *cw, const double *vhat, const double *alpha, const double *rrh,
                                   const double *rrk, const double *rrv, double *dH, double *dk, double *dv,
                                   double *dwh, double *dwv, double *dcw, double *magH, double *magk, double *magv,
                                   double *mdwh, double *mdwv, double *mdcw, int threads) {
  if (M < 0 || T < 0 || d < 1 || !wh || !wv || !cw || !dwh || !dwv || !dcw) return -1;
  if (M * T > 0 && (!dY || !H || !k || !v || !vhat || !alpha || !rrh || !rrk || !rrv || !dH || !dk || !dv))
    return -1;
  const int mags = mdwh && mdwv && mdcw;
  const int nt = seq_threads(M, threads);
  double *acc = (double *)calloc((size_t)nt * 12 * d, sizeof(double));
  if (!acc) return -2;
  gc_bwd_ctx c = {T, d, dY, H, k, v, wh, wv, cw, vhat, alpha, rrh, rrk, rrv, dH, dk, dv, magH, magk, magv, acc,
                  mags, 0};
  if (M * T > 0) run_sequences(M, nt, gc_bwd_range, &c);
  for (int64_t j = 0; j < 6 * d; ++j) {
    double s = 0.0, sm = 0.0;
    for (int i = 0; i < nt; ++i) {
      s += acc[(int64_t)i * 12 * d + j];
      sm += acc[(int64_t)i * 12 * d + 6 * d + j];
    }
    double *dst = j < d ? dwh + j : j < 2 * d ? dwv + (j - d) : dcw + (j - 2 * d);
    *dst = s;
    if (mags) {
      double *mdst = j < d ? mdwh + j : j < 2 * d ? mdwv + (j - d) : mdcw + (j - 2 * d);
      *mdst = sm;
    }
  }
  free(acc);
  return c.failed;
}

/* fp64 -> fp32 (RNE) -> bf16 (RNE), elementwise (R10's rounding chain). */
int engram_oracle_round_bf16(int64_t count, const double *in, uint16_t *out) {
  if (count < 0 || (count > 0 && (!in || !out))) return -1;
  for (int64_t q = 0; q < count; ++q) out[q] = double_to_bf16(in[q]);
  return 0;
}
