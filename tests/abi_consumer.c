/*
 * A C11 consumer of include/engram.h: built with gcc (and as C++ with g++)
 * against libengram.so by tests/test_c_consumer_cpu.py, to show that the
 * boundary is a plain C ABI usable without Python or HIP headers.
 *
 * It calls every declared function, but only with arguments the library
 * rejects on the host before touching any memory (NULL pointers, sizes out of
 * range, misalignment, overlap), plus the pure size and status helpers, so it
 * needs no GPU and never dereferences the fake addresses it passes.  Each
 * expected status follows the header's rules; exit status 0 means all held.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "engram.h"

static int failures = 0;

static void expect(const char *what, long long got, long long want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

/* 16-byte-aligned fake addresses, far apart (never dereferenced) */
static void *fake(uintptr_t slot) { return (void *)(uintptr_t)(((uintptr_t)1 << 40) + slot * ((uintptr_t)1 << 34)); }

int main(void) {
  void *x = fake(1), *kv = fake(2), *g = fake(3), *out = fake(4), *dx = fake(5), *dkv = fake(6), *ws = fake(7);
  float *w = (float *)fake(8), *sv = (float *)fake(9), *dw = (float *)fake(10);
  const uint8_t *mask = (const uint8_t *)fake(11);
  void *wh = fake(12), *we = fake(13);
  float *gwh = (float *)fake(14), *gwe = (float *)fake(15);

  /* size helpers: the workspace paragraph's formula, 0 for N <= 0 */
  expect("gate workspace N=8192", (long long)engram_gate_bwd_workspace_bytes(8192),
         4LL * (16LL * 8192 + 4LL * 5120 * (8192 / 64)));
  expect("gate workspace N=64", (long long)engram_gate_bwd_workspace_bytes(64), 4LL * (16LL * 64 + 4LL * 5120));
  expect("gate workspace N=0", (long long)engram_gate_bwd_workspace_bytes(0), 0);
  expect("gateconv workspace d=640 (rejected)", (long long)engram_gateconv_bwd_workspace_bytes(4, 4096, 640), 0);
  expect("gateconv workspace M=0 (rejected)", (long long)engram_gateconv_bwd_workspace_bytes(0, 4096, 5120), 0);
  if (engram_gateconv_bwd_workspace_bytes(4, 4096, 5120) <= 4u * 4 * 4096) {
    fprintf(stderr, "FAIL gateconv workspace 4x4096x5120 holds no partials\n");
    ++failures;
  }

  /* the gate forward */
  expect("fwd NULL x", engram_gate_fwd(NULL, kv, w, mask, out, sv, 8, NULL), ENGRAM_ERR_NULL);
  expect("fwd N=0", engram_gate_fwd(x, kv, w, mask, out, sv, 0, NULL), ENGRAM_ERR_N_RANGE);
  expect("fwd N too large", engram_gate_fwd(x, kv, w, mask, out, sv, ENGRAM_N_MAX + 1, NULL), ENGRAM_ERR_N_RANGE);
  expect("fwd misaligned out", engram_gate_fwd(x, kv, w, mask, (char *)out + 8, sv, 8, NULL), ENGRAM_ERR_ALIGN);
  expect("fwd out over x", engram_gate_fwd(x, kv, w, mask, x, sv, 8, NULL), ENGRAM_ERR_OVERLAP);

  /* the gate backward and its variants */
  expect("bwd NULL workspace", engram_gate_bwd(x, kv, w, sv, g, dx, dkv, dw, NULL, 64, NULL), ENGRAM_ERR_NULL);
  expect("bwd N=100", engram_gate_bwd(x, kv, w, sv, g, dx, dkv, dw, ws, 100, NULL), ENGRAM_ERR_N_MULT64);
  expect("bwd N=8256", engram_gate_bwd(x, kv, w, sv, g, dx, dkv, dw, ws, 8256, NULL), ENGRAM_ERR_N_RANGE);
  expect("bwd grad_x over grad_out", engram_gate_bwd(x, kv, w, sv, g, g, dkv, dw, ws, 64, NULL), ENGRAM_ERR_OVERLAP);
  expect("bwd+norm NULL grad_we",
         engram_gate_bwd_with_norm_weights(x, kv, w, sv, g, dx, dkv, dw, wh, we, gwh, NULL, ws, 64, NULL),
         ENGRAM_ERR_NULL);
  expect("bwd+norm grad_wh over grad_we",
         engram_gate_bwd_with_norm_weights(x, kv, w, sv, g, dx, dkv, dw, wh, we, gwe, gwe, ws, 64, NULL),
         ENGRAM_ERR_OVERLAP);
  expect("noalloc N beyond its array",
         engram_gate_bwd_noalloc(x, kv, w, sv, g, dx, dkv, dw, ENGRAM_NOALLOC_N_MAX + 64, NULL), ENGRAM_ERR_N_RANGE);
  expect("noalloc misaligned grad_weight",
         engram_gate_bwd_noalloc(x, kv, w, sv, g, dx, dkv, (float *)((char *)dw + 4), 64, NULL), ENGRAM_ERR_ALIGN);
  expect("fused weight NULL we", engram_fused_weight(wh, NULL, w, NULL), ENGRAM_ERR_NULL);

  /* GateConv */
  {
    void *H = fake(16), *k = fake(17), *v = fake(18), *Y = fake(19), *vh = fake(20), *dY = fake(21);
    void *dH = fake(22), *dk = fake(23), *dv = fake(24);
    float *rwh = (float *)fake(25), *rwv = (float *)fake(26), *cw = (float *)fake(27), *al = (float *)fake(28);
    float *rh = (float *)fake(29), *rk = (float *)fake(30), *rv = (float *)fake(31), *dwh = (float *)fake(32);
    float *dwv = (float *)fake(33), *dcw = (float *)fake(34);
    expect("gateconv fwd d=640", engram_gateconv_fwd(H, k, v, rwh, rwv, cw, Y, vh, al, rh, rk, rv, 1, 8, 640, 1e-6f, NULL),
           ENGRAM_ERR_N_RANGE);
    expect("gateconv fwd eps=2", engram_gateconv_fwd(H, k, v, rwh, rwv, cw, Y, vh, al, rh, rk, rv, 1, 8, 512, 2.0f, NULL),
           ENGRAM_ERR_N_RANGE);
    expect("gateconv fwd NULL Y", engram_gateconv_fwd(H, k, v, rwh, rwv, cw, NULL, vh, al, rh, rk, rv, 1, 8, 512, 1e-6f, NULL),
           ENGRAM_ERR_NULL);
    expect("gateconv bwd NULL workspace",
           engram_gateconv_bwd(dY, H, k, v, rwh, rwv, cw, vh, al, rh, rk, rv, dH, dk, dv, dwh, dwv, dcw, NULL, 1, 8, 512,
                               NULL),
           ENGRAM_ERR_NULL);
    expect("gateconv bwd dH over H",
           engram_gateconv_bwd(dY, H, k, v, rwh, rwv, cw, vh, al, rh, rk, rv, H, dk, dv, dwh, dwv, dcw, ws, 1, 8, 512,
                               NULL),
           ENGRAM_ERR_OVERLAP);
  }

  /* status helpers */
  {
    int s;
    for (s = ENGRAM_OK; s <= ENGRAM_ERR_LAUNCH; ++s) {
      const char *name = engram_status_string(s);
      if (!name || !*name) {
        fprintf(stderr, "FAIL status string %d\n", s);
        ++failures;
      }
    }
    if (strcmp(engram_status_string(ENGRAM_OK), engram_status_string(ENGRAM_ERR_NULL)) == 0) {
      fprintf(stderr, "FAIL status strings not distinct\n");
      ++failures;
    }
  }
  expect("no launch error recorded", engram_last_hip_error(), 0);

  if (failures) return 1;
  printf("abi consumer ok\n");
  return 0;
}
