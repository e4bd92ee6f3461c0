/* Drives the host side of libdgdenoise's C ABI -- configuration checks,
 * size queries and the argument validation of every entry point -- for a
 * build whose host code carries AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Written in C, as
 * a C caller would call the library: enum-typed fields may hold any int.
 * No GPU is needed: every call here must be rejected (or answered) before
 * any device work, and the device pointers are placeholders that must never
 * be dereferenced on the host.  Prints "ok" and exits 0. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "dgdenoise.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);    \
      return 1;                                                         \
    }                                                                   \
  } while (0)

static dg_config cfg3(void) {
  dg_config c;
  memset(&c, 0, sizeof c);
  c.canvas_len = 256;
  c.vocab = 262144;
  c.d_model = 2816;
  c.n_q_heads = 16;
  c.n_kv_heads = 8;
  c.head_dim = 128;
  c.ffn_hidden = 2816;
  c.dtype = DG_BF16;
  c.rms_eps = 1e-6f;
  c.conf_eps = 0.005f;
  return c;
}

/* configuration k with one field broken; returns the status it must get */
static dg_status broken(int k, dg_config *x) {
  *x = cfg3();
  switch (k) {
    case 0: x->dtype = (dg_dtype)7; return DG_ERR_INVALID_ARG;
    case 1: x->accept_rule = (dg_accept_rule)-1; return DG_ERR_INVALID_ARG;
    case 2: x->candidate_rule = (dg_candidate_rule)2; return DG_ERR_INVALID_ARG;
    case 3: x->sampler = (dg_sampler)9; return DG_ERR_INVALID_ARG;
    case 4: x->table_format = (dg_table_format)3; return DG_ERR_INVALID_ARG;
    case 5: x->stable_rule = (dg_stable_rule)5; return DG_ERR_INVALID_ARG;
    case 6: x->table_format = DG_TABLE_FP8; x->table_exp = 99; return DG_ERR_INVALID_ARG;
    case 7: x->canvas_len = 0; return DG_ERR_INVALID_ARG;
    case 8: x->canvas_len = 257; return DG_ERR_UNSUPPORTED;
    case 9: x->canvas_len = -5; return DG_ERR_INVALID_ARG;
    case 10: x->vocab = 1000; return DG_ERR_UNSUPPORTED;
    case 11: x->vocab = 1 << 30; return DG_ERR_UNSUPPORTED;
    case 12: x->vocab = -2147483647 - 1; return DG_ERR_INVALID_ARG;
    case 13: x->d_model = 1000; return DG_ERR_UNSUPPORTED;
    case 14: x->d_model = 8192; return DG_ERR_UNSUPPORTED;
    case 15: x->head_dim = 64; return DG_ERR_UNSUPPORTED;
    case 16: x->n_q_heads = 12; return DG_ERR_UNSUPPORTED;
    case 17: x->n_kv_heads = 0; return DG_ERR_INVALID_ARG;
    case 18: x->rms_eps = nanf(""); return DG_ERR_INVALID_ARG;
    case 19: x->rms_eps = -1.f; return DG_ERR_INVALID_ARG;
    case 20: x->conf_eps = INFINITY; return DG_ERR_INVALID_ARG;
  }
  return DG_OK;
}

int main(void) {
  char *const dev = (char *)0x1000; /* placeholder device address */
  CHECK(dg_abi_version() == DG_ABI_VERSION);
  for (int s = -1; s <= 7; ++s) CHECK(dg_status_string((dg_status)s) != NULL);

  /* configurations: valid ones of both dtypes, then one field broken at a time */
  dg_config c = cfg3();
  CHECK(dg_validate_config(&c) == DG_OK);
  CHECK(dg_validate_config(NULL) == DG_ERR_INVALID_ARG);
  dg_config f = c;
  f.dtype = DG_F32;
  f.canvas_len = 16;
  f.vocab = 512;
  f.d_model = 64;
  f.n_q_heads = f.n_kv_heads = 4;
  f.head_dim = 16;
  f.ffn_hidden = 128;
  CHECK(dg_validate_config(&f) == DG_OK);
  for (int k = 0; k <= 20; ++k) {
    dg_config x;
    const dg_status want = broken(k, &x);
    CHECK(dg_validate_config(&x) == want);
    CHECK(dg_workspace_bytes(&x, 0) == 0 && dg_stats_bytes(&x) == 0 && dg_probs_bytes(&x) == 0);
    CHECK(dg_embedding_pack_bytes(&x) == 0 && dg_workspace_bytes_batch(&x, 2) == 0);
  }
  /* sizes */
  const size_t ws = dg_workspace_bytes(&c, 0);
  CHECK(ws > 0 && dg_workspace_bytes(&c, 1024) >= ws && dg_workspace_bytes(&c, -1) == 0);
  CHECK(dg_workspace_bytes_batch(&c, 0) == 0 && dg_workspace_bytes_batch(&c, DG_MAX_BATCH + 1) == 0);
  CHECK(dg_workspace_bytes_batch(&c, DG_MAX_BATCH) >= ws);
  CHECK(dg_stats_bytes(&c) > 0 && dg_probs_bytes(&c) > 0 && dg_embedding_pack_bytes(&c) > 0);
  CHECK(dg_embedding_pack_bytes(&f) == 0 && dg_test_logits_ws_bytes(&c) >= ws);

  /* entry points: argument errors are found before any device work */
  dg_weights w = {dev, dev, dev, dev, dev, dev, dev, dev, dev, dev, NULL};
  dg_kv_cache kv = {dev, dev, 2048, 2304};
  dg_canvas cv;
  memset(&cv, 0, sizeof cv);
  cv.tokens = (int32_t *)dev;
  cv.probs = dev;
  cv.stats = dev;
  cv.entropy = (float *)dev;
  cv.argmax = (int32_t *)dev;
  cv.accept = (uint8_t *)dev;
  cv.status = (int32_t *)dev;
  const int32_t *tok = (const int32_t *)dev;
  CHECK(dg_pack_embedding(&c, NULL, dev, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_canvas_init(&c, NULL, 1, 0, NULL) == DG_ERR_INVALID_ARG);
  dg_canvas nocv = cv;
  nocv.status = NULL;
  CHECK(dg_canvas_init(&c, &nocv, 1, 0, NULL) == DG_ERR_INVALID_ARG);
  /* prefill */
  CHECK(dg_prefill_append(&c, NULL, &kv, tok, 4, NULL, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_prefill_append(&c, &w, &kv, tok, -1, NULL, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_prefill_append(&c, &w, &kv, tok, 257, NULL, dev, ws, NULL) == DG_ERR_CAPACITY);
  CHECK(dg_prefill_append(&c, &w, &kv, NULL, 4, NULL, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_prefill_append(&c, &w, &kv, tok, 4, NULL, dev, 16, NULL) == DG_ERR_WORKSPACE);
  CHECK(dg_prefill_append(&c, &w, &kv, tok, 0, NULL, dev, 0, NULL) == DG_OK); /* nothing to do */
  CHECK(kv.length == 2048);
  dg_kv_cache badkv = kv;
  badkv.length = 5000;
  CHECK(dg_prefill_append(&c, &w, &badkv, tok, 1, NULL, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  /* one step */
  const float nan = nanf("");
  CHECK(dg_denoise_step(&c, &w, &kv, &cv, nan, 16.f, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_denoise_step(&c, &w, &kv, &cv, 0.f, 16.f, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_denoise_step(&c, &w, &kv, &cv, 1.f, -1.f, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_denoise_step(&c, &w, &kv, &cv, 1.f, nan, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_denoise_step(&c, &w, &kv, &cv, 1.f, 16.f, dev, ws - 1, NULL) == DG_ERR_WORKSPACE);
  CHECK(dg_denoise_step(&c, &w, &kv, &cv, 1.f, 16.f, NULL, ws, NULL) == DG_ERR_WORKSPACE);
  CHECK(dg_denoise_step(&c, &w, &badkv, &cv, 1.f, 16.f, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_denoise_step(&c, &w, &kv, &nocv, 1.f, 16.f, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  dg_weights now = w;
  now.E_pack = NULL;
  CHECK(dg_denoise_step(&c, &now, &kv, &cv, 1.f, 16.f, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  dg_config masked = c;
  masked.sampler = DG_SAMPLER_MASKED; /* needs a 16-byte aligned [MASK] row */
  CHECK(dg_denoise_step(&masked, &w, &kv, &cv, 1.f, 16.f, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  dg_weights mw = w;
  mw.mask_emb = dev + 4;
  CHECK(dg_denoise_step(&masked, &mw, &kv, &cv, 1.f, 16.f, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(cv.step == 0 && cv.has_prev == 0);
  /* a batch */
  dg_kv_cache kvs[3] = {kv, kv, kv};
  dg_canvas cvs[3] = {cv, cv, cv};
  const size_t wsb = dg_workspace_bytes_batch(&c, 3);
  CHECK(dg_denoise_step_batch(&c, &w, kvs, cvs, 0, 1.f, 16.f, dev, wsb, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_denoise_step_batch(&c, &w, kvs, cvs, DG_MAX_BATCH + 1, 1.f, 16.f, dev, wsb, NULL) ==
        DG_ERR_INVALID_ARG);
  CHECK(dg_denoise_step_batch(&c, &w, kvs, cvs, 3, 1.f, 16.f, dev, wsb, NULL) ==
        DG_ERR_INVALID_ARG); /* the three canvases share buffers */
  for (int b = 0; b < 3; ++b) {
    char *base = dev + 0x100000 * (b + 1);
    cvs[b].tokens = (int32_t *)base;
    cvs[b].probs = base + 0x1000;
    cvs[b].stats = base + 0x2000;
    cvs[b].entropy = (float *)(base + 0x3000);
    cvs[b].argmax = (int32_t *)(base + 0x4000);
    cvs[b].accept = (uint8_t *)(base + 0x5000);
    cvs[b].status = (int32_t *)(base + 0x6000);
  }
  cvs[1].has_prev = 1;
  CHECK(dg_denoise_step_batch(&c, &w, kvs, cvs, 3, 1.f, 16.f, dev, wsb, NULL) ==
        DG_ERR_INVALID_ARG); /* mixed has_prev */
  cvs[1].has_prev = 0;
  CHECK(dg_denoise_step_batch(&c, &w, kvs, cvs, 3, 1.f, 16.f, dev, wsb - 1, NULL) == DG_ERR_WORKSPACE);
  kvs[2].length = -1;
  CHECK(dg_denoise_step_batch(&c, &w, kvs, cvs, 3, 1.f, 16.f, dev, wsb, NULL) == DG_ERR_INVALID_ARG);
  /* the stop test and the loop */
  int32_t stop = 0, steps = 0, stopped = 0;
  CHECK(dg_should_stop(&c, &cv, 3, NULL, NULL, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_should_stop(&c, NULL, 3, &stop, NULL, NULL) == DG_ERR_INVALID_ARG);
  const float temps[3] = {1.5f, nan, 0.3f};
  CHECK(dg_run_canvas(&c, &w, &kv, &cv, 1, 0, temps, 3, 16.f, 1, 3, dev, ws, NULL, &steps, &stopped) ==
        DG_ERR_INVALID_ARG);
  CHECK(dg_run_canvas(&c, &w, &kv, &cv, 1, 0, temps, -1, 16.f, 1, 3, dev, ws, NULL, &steps, &stopped) ==
        DG_ERR_INVALID_ARG);
  CHECK(dg_run_canvas(&c, &w, &kv, &cv, 1, 0, NULL, 2, 16.f, 1, 3, dev, ws, NULL, &steps, &stopped) ==
        DG_ERR_INVALID_ARG);
  CHECK(dg_run_canvas(&c, &w, &kv, &cv, 1, 0, temps, 1, 16.f, 1, 3, dev, 8, NULL, &steps, &stopped) ==
        DG_ERR_WORKSPACE);
  CHECK(dg_run_canvas(&c, &w, &kv, &cv, 1, 0, temps, 1, 16.f, 1, 3, dev, ws, NULL, NULL, &stopped) ==
        DG_ERR_INVALID_ARG);
  /* test exports */
  dg_ws_offsets off;
  CHECK(dg_test_ws_offsets(&c, &off) == DG_OK && off.h0 < ws && off.selfcond < ws);
  CHECK(dg_test_ws_offsets(&c, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_test_selfcond(&c, &w, NULL, dev, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_test_selfcond(&c, &w, dev, dev, dev, ws, NULL) == DG_ERR_WORKSPACE); /* needs the dump size */
  CHECK(dg_test_selfcond_canvas(&c, &w, &nocv, dev, dev, ws, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_test_select(&c, &cv, nan, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_test_philox(NULL, 0, 0, NULL, 4, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_test_philox(NULL, 0, 0, NULL, -1, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_test_gumbel((const uint32_t *)dev, 4, 3, (float *)dev, NULL) == DG_ERR_INVALID_ARG);
  CHECK(dg_test_copy(dev, dev, 15, NULL) == DG_ERR_INVALID_ARG);
  float ms = 0.f;
  int32_t n = 0;
  CHECK(dg_profile_read(&ms, &n, &ms, &n) == DG_OK && n == 0); /* nothing recorded */
  printf("ok\n");
  return 0;
}
