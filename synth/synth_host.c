/*
 * synth_host.c -- seeded, counter-based synthetic inputs (host side).
 *
 * This module holds input generation only, none of the gate's arithmetic.
 * The device twin (synth_dev.hip) implements the same recipe; both sides
 * produce bit-identical bytes, which a GPU test checks.
 *
 * Recipe
 *   SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014; finaliser constants as in Vigna's public
 *   splitmix64.c): gamma = 0x9E3779B97F4A7C15,
 *     mix(z) = z ^= z>>30, z *= 0xBF58476D1CE4E5B9, z ^= z>>27,
 *              z *= 0x94D049BB133111EB, z ^= z>>31.
 *   Stream key of (seed, tensor id):  key = mix(seed + gamma * (id + 1)).
 *   Counter word c of a stream:       word(c) = mix(key + gamma * (c + 1)).
 *
 *   Normal element e ("N(0,1)"): the twelve 16-bit fields of words 3e,
 *   3e+1, 3e+2 are summed to an integer S (Irwin-Hall with 12 terms), and
 *   z = (S - 393210) * 2^-16, which is exact in fp32 (|S - 393210| < 2^19);
 *   mean 0, variance 1 - 2^-32, support [-6, 6].  bf16 tensors store
 *   bf16_rne(z); fp32 tensors with mean mu and sd sigma store
 *   fl(mu + fl(sigma * z)) (two separately rounded fp32 operations).
 *
 *   Mask element t (Bernoulli(p)): (word(t) >> 40) < thr, thr = round(p*2^24).
 *
 *   Edge rows (a row r = 4t + s is stream s of token t; stream key id 6):
 *   with u = word(r) >> 40, rows with u < thr_eps get either their X row
 *   (word bit 0 clear) or their key row (bit 0 set) multiplied by 1e-12f in
 *   fp32, then rounded to bf16; rows with thr_eps <= u < thr_eps + thr_clamp
 *   get their key row multiplied by 2^-64 (exact).  Then, with stream key
 *   id 7, rows word(i) mod 4N for i = 0..7 get an all-zero key row and rows
 *   word(i) mod 4N for i = 8..15 an all-zero X row.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint32_t id) { return mix64(seed + GAMMA * ((uint64_t)id + 1)); }

uint64_t synth_word(uint64_t key, uint64_t c) { return mix64(key + GAMMA * (c + 1)); }

static float normal_f32(uint64_t key, uint64_t e) {
  int32_t s = 0;
  for (int i = 0; i < 3; ++i) {
    uint64_t w = synth_word(key, 3 * e + (uint64_t)i);
    for (int l = 0; l < 4; ++l) s += (int32_t)((w >> (16 * l)) & 0xFFFFu);
  }
  return (float)(s - 393210) * 0x1p-16f; /* both steps exact */
}

static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* ---- threaded fill over [0, count) ---- */

typedef struct {
  int kind; /* 0 normal bf16, 1 normal f32, 2 mask */
  void *dst;
  int64_t count, offset;
  uint64_t key;
  float mu, sigma;
  uint32_t thr;
  int64_t i0, i1;
} fill_job;

static void *fill_main(void *p) {
  fill_job *j = (fill_job *)p;
  for (int64_t i = j->i0; i < j->i1; ++i) {
    uint64_t e = (uint64_t)(j->offset + i);
    if (j->kind == 0) {
      ((uint16_t *)j->dst)[i] = bf16_rne(normal_f32(j->key, e));
    } else if (j->kind == 1) {
      volatile float t = j->sigma * normal_f32(j->key, e); /* keep the two roundings separate */
      ((float *)j->dst)[i] = j->mu + t;
    } else {
      ((uint8_t *)j->dst)[i] = (uint8_t)((synth_word(j->key, e) >> 40) < j->thr);
    }
  }
  return NULL;
}

static void fill(fill_job base, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (base.count < 65536) nthreads = 1;
  pthread_t th[64];
  fill_job jobs[64];
  int64_t per = (base.count + nthreads - 1) / nthreads;
  int started[64] = {0};
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].i0 = per * i;
    jobs[i].i1 = per * (i + 1) < base.count ? per * (i + 1) : base.count;
    if (i > 0 && pthread_create(&th[i], NULL, fill_main, &jobs[i]) == 0) started[i] = 1;
  }
  fill_main(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) {
    if (started[i])
      pthread_join(th[i], NULL);
    else
      fill_main(&jobs[i]);
  }
}

/* dst[i] = bf16 normal element (offset + i) of stream (seed, id). */
void synth_normal_bf16(uint16_t *dst, int64_t count, uint64_t seed, uint32_t id, int64_t offset,
                       int nthreads) {
  fill_job j;
  memset(&j, 0, sizeof j);
  j.kind = 0;
  j.dst = dst;
  j.count = count;
  j.offset = offset;
  j.key = synth_stream_key(seed, id);
  fill(j, nthreads);
}

/* dst[i] = fl(mu + fl(sigma * z)), z the normal element (offset + i). */
void synth_normal_f32(float *dst, int64_t count, uint64_t seed, uint32_t id, int64_t offset, float mu,
                      float sigma, int nthreads) {
  fill_job j;
  memset(&j, 0, sizeof j);
  j.kind = 1;
  j.dst = dst;
  j.count = count;
  j.offset = offset;
  j.key = synth_stream_key(seed, id);
  j.mu = mu;
  j.sigma = sigma;
  fill(j, nthreads);
}

/* dst[i] = 1 if (word(offset + i) >> 40) < thr else 0. */
void synth_mask(uint8_t *dst, int64_t count, uint64_t seed, uint32_t id, int64_t offset, uint32_t thr,
                int nthreads) {
  fill_job j;
  memset(&j, 0, sizeof j);
  j.kind = 2;
  j.dst = dst;
  j.count = count;
  j.offset = offset;
  j.key = synth_stream_key(seed, id);
  j.thr = thr;
  fill(j, nthreads);
}

/*
 * Apply the edge-row recipe to tokens [t0, t0 + nt) of an N-token batch
 * (x points at token t0's X rows, kv at token t0's KV row; d per stream).
 * Returns the number of rows modified, per kind, in counts[0..3]
 * (eps-X, eps-key, clamp-key, zero rows touched).
 */
void synth_edge_rows(uint16_t *x, uint16_t *kv, int64_t d, int64_t n_total, int64_t t0, int64_t nt,
                     uint64_t seed, uint32_t thr_eps, uint32_t thr_clamp, int64_t *counts) {
  const uint64_t key6 = synth_stream_key(seed, 6), key7 = synth_stream_key(seed, 7);
  const int64_t rows = 4 * n_total;
  int64_t cnt[4] = {0, 0, 0, 0};
  for (int64_t t = t0; t < t0 + nt; ++t) {
    for (int s = 0; s < 4; ++s) {
      int64_t r = 4 * t + s;
      uint64_t w = synth_word(key6, (uint64_t)r);
      uint32_t u = (uint32_t)(w >> 40);
      uint16_t *xrow = x + ((t - t0) * 4 + s) * d;
      uint16_t *krow = kv + (t - t0) * 5 * d + (int64_t)s * d;
      if (u < thr_eps) {
        uint16_t *row = (w & 1u) ? krow : xrow;
        for (int64_t j = 0; j < d; ++j) {
          volatile float p = bf16_to_f32(row[j]) * 1e-12f;
          row[j] = bf16_rne(p);
        }
        cnt[(w & 1u) ? 1 : 0]++;
      } else if (u < thr_eps + thr_clamp) {
        for (int64_t j = 0; j < d; ++j) {
          float p = ldexpf(bf16_to_f32(krow[j]), -64); /* exact for these magnitudes */
          krow[j] = bf16_rne(p);
        }
        cnt[2]++;
      }
    }
  }
  for (uint64_t i = 0; i < 16; ++i) {
    int64_t r = (int64_t)(synth_word(key7, i) % (uint64_t)rows);
    int64_t t = r / 4, s = r % 4;
    if (t < t0 || t >= t0 + nt) continue;
    uint16_t *row = (i < 8) ? kv + (t - t0) * 5 * d + s * d : x + ((t - t0) * 4 + s) * d;
    for (int64_t j = 0; j < d; ++j) row[j] = 0;
    cnt[3]++;
  }
  if (counts)
    for (int q = 0; q < 4; ++q) counts[q] = cnt[q];
}

/* Row indices chosen for zero rows (for tests): rows[i], i < 16. */
void synth_zero_rows(int64_t n_total, uint64_t seed, int64_t *rows) {
  const uint64_t key7 = synth_stream_key(seed, 7);
  for (uint64_t i = 0; i < 16; ++i) rows[i] = (int64_t)(synth_word(key7, i) % (uint64_t)(4 * n_total));
}
