/* Drives every function of the CPU oracle on small inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).
 * Prints "ok" and exits 0 when every call returns what it should; any
 * out-of-bounds access, leak or undefined operation aborts the run. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dg_oracle.h"

static uint64_t lcg = 88172645463325252ull;
static double unif(void) { /* xorshift64, in [0, 1) */
  lcg ^= lcg << 13;
  lcg ^= lcg >> 7;
  lcg ^= lcg << 17;
  return (double)(lcg >> 11) * (1.0 / 9007199254740992.0);
}
static float *rnd(size_t n, double scale) {
  float *p = (float *)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = (float)((unif() * 2.0 - 1.0) * scale);
  return p;
}
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                   \
    }                                                             \
  } while (0)

int main(void) {
  enum { N = 8, V = 64, d = 32, Hq = 4, Hkv = 2, hd = 8, F = 16, L = 5, CAP = 40 };
  const int qw = Hq * hd;
  /* Philox, tokens, canvas */
  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
  orc_philox4x32_10(ctr, key, out);
  CHECK(orc_uniform_token(7, 1, 2, 3, 1, V) < V);
  int32_t tok[N];
  orc_canvas_init(11, 0, N, V, tok);
  for (int i = 0; i < N; ++i) CHECK(tok[i] >= 0 && tok[i] < V);

  /* building blocks */
  CHECK(fabs(orc_gelu(0.0)) == 0.0);
  double x[d], y[d];
  for (int k = 0; k < d; ++k) x[k] = unif() - 0.5;
  float g[d];
  for (int k = 0; k < d; ++k) g[k] = 1.0f;
  orc_rmsnorm(x, g, d, 1e-6, y);
  float *b = rnd((size_t)3 * d, 1.0);
  double ym[2 * 3];
  double a2[2 * d];
  memcpy(a2, x, sizeof x);
  memcpy(a2 + d, y, sizeof y);
  orc_matmul_nt(a2, b, 2, 3, d, ym);
  double z[V], p[V], H;
  for (int v = 0; v < V; ++v) z[v] = unif() * 4.0;
  orc_softmax_entropy(z, V, p, &H);
  CHECK(H >= 0.0 && H <= log((double)V) + 1e-12);
  CHECK(orc_argmax(z, V) >= 0);
  float zf[V];
  for (int v = 0; v < V; ++v) zf[v] = (float)z[v];
  CHECK(orc_argmax_f32(zf, V) >= 0);
  CHECK(orc_ln_f32(1.0f) == 0.0f);
  CHECK(isfinite(orc_gumbel_f32(0u)) && isfinite(orc_gumbel_f32(0xFFFFFFFFu)));

  /* multinomial candidates: 2 tiles per row, with a NaN and a zero weight */
  {
    enum { NT = 2 };
    float zmax[N * NT], lsum[N * NT], num[N * NT * 64];
    int32_t fb[N], cand[N];
    for (int i = 0; i < N * NT; ++i) {
      zmax[i] = (float)unif();
      lsum[i] = (float)(1.0 + unif());
    }
    for (int i = 0; i < N * NT * 64; ++i) num[i] = (float)unif();
    num[3] = NAN;
    num[4] = 0.0f;
    lsum[1] = NAN;
    for (int i = 0; i < N; ++i) fb[i] = i;
    orc_multinomial_candidates(zmax, lsum, N, NT, num, 1.25f, 9, 2, 1, fb, cand);
    for (int i = 0; i < N; ++i) CHECK(cand[i] >= 0 && cand[i] < NT * 64);
  }

  /* attention, both modes */
  {
    const int nk = 6;
    double *q = (double *)calloc((size_t)3 * qw, sizeof(double));
    double *k = (double *)calloc((size_t)Hkv * nk * hd, sizeof(double));
    double *v = (double *)calloc((size_t)Hkv * nk * hd, sizeof(double));
    double *o = (double *)calloc((size_t)3 * qw, sizeof(double));
    for (int i = 0; i < 3 * qw; ++i) q[i] = unif();
    for (int i = 0; i < Hkv * nk * hd; ++i) {
      k[i] = unif();
      v[i] = unif();
    }
    orc_attention(q, k, v, 3, nk, Hq, Hkv, hd, 0, 0, o);
    orc_attention(q, k, v, 3, nk, Hq, Hkv, hd, 1, 3, o);
    free(q);
    free(k);
    free(v);
    free(o);
  }

  /* selection: both accept rules, both stability rules, the masked sampler, NaN */
  {
    float Hs[N];
    int32_t am[N], pred[N], prev[N], tout[N];
    uint8_t acc[N];
    orc_flags fl;
    for (int i = 0; i < N; ++i) {
      Hs[i] = (float)(unif() * 3.0);
      am[i] = (int32_t)(unif() * V);
      pred[i] = am[i];
      prev[i] = am[i];
    }
    Hs[2] = NAN;
    Hs[5] = -0.0f;
    for (int rule = 0; rule < 2; ++rule)
      for (int srule = 0; srule < 2; ++srule) {
        orc_select(N, V, Hs, am, tok, 4.0, rule, 3, 1, 2, 0, 0.005, -1, pred, prev, srule, acc, tout, &fl);
        orc_select(N, V, Hs, am, tok, 1e30, rule, 3, 1, 0, 7, 0.005, -1, pred, NULL, srule, acc, tout, &fl);
        int32_t mtok[N];
        for (int i = 0; i < N; ++i) mtok[i] = (i % 3) ? V : tok[i];
        orc_select(N, V, Hs, am, mtok, 2.0, rule, 3, 1, 2, 0, 0.005, V, pred, prev, srule, acc, tout, &fl);
        CHECK(fl.masked >= 0);
      }
    CHECK(orc_should_stop(&fl, 3) == 0 || orc_should_stop(&fl, 3) == 1);
  }

  /* the model: forward without and with self-conditioning, row selection, prefill */
  {
    float *E = rnd((size_t)V * d, 0.2), *w1 = rnd((size_t)F * d, 0.2), *w2 = rnd((size_t)d * F, 0.2);
    float *wq = rnd((size_t)qw * d, 0.2), *wk = rnd((size_t)Hkv * hd * d, 0.2);
    float *wv = rnd((size_t)Hkv * hd * d, 0.2), *wo = rnd((size_t)d * qw, 0.2);
    float *mask = rnd(d, 0.2);
    orc_model m = {N, V, d, Hq, Hkv, hd, F, 1e-6, E, w1, w2, wq, wk, wv, wo, g, g, mask};
    double *kc = (double *)calloc((size_t)Hkv * CAP * hd, sizeof(double));
    double *vc = (double *)calloc((size_t)Hkv * CAP * hd, sizeof(double));
    for (int i = 0; i < Hkv * CAP * hd; ++i) {
      kc[i] = unif();
      vc[i] = unif();
    }
    orc_step_out so;
    so.h0 = (double *)calloc((size_t)N * d, sizeof(double));
    so.q = (double *)calloc((size_t)N * qw, sizeof(double));
    so.k_canvas = (double *)calloc((size_t)Hkv * N * hd, sizeof(double));
    so.v_canvas = (double *)calloc((size_t)Hkv * N * hd, sizeof(double));
    so.attn = (double *)calloc((size_t)N * qw, sizeof(double));
    so.h1 = (double *)calloc((size_t)N * d, sizeof(double));
    so.logits = (double *)calloc((size_t)N * V, sizeof(double));
    so.probs = (double *)calloc((size_t)N * V, sizeof(double));
    so.entropy = (double *)calloc(N, sizeof(double));
    so.argmax = (int32_t *)calloc(N, sizeof(int32_t));
    CHECK(orc_denoise_forward(&m, tok, NULL, kc, vc, L, CAP, 1.0, NULL, &so) == 0);
    double *pp = (double *)malloc(sizeof(double) * (size_t)N * V);
    memcpy(pp, so.probs, sizeof(double) * (size_t)N * V);
    uint8_t rs[N] = {1, 0, 0, 1, 0, 0, 0, 1};
    int32_t mtok[N];
    memcpy(mtok, tok, sizeof mtok);
    mtok[4] = V; /* a [MASK] row */
    CHECK(orc_denoise_forward(&m, mtok, pp, kc, vc, L, CAP, 0.7, rs, &so) == 0);
    int32_t bad[N];
    memcpy(bad, tok, sizeof bad);
    bad[0] = V + 1;
    CHECK(orc_denoise_forward(&m, bad, NULL, kc, vc, L, CAP, 1.0, NULL, &so) == -2);
    CHECK(orc_denoise_forward(&m, tok, NULL, kc, vc, CAP + 1, CAP, 1.0, NULL, &so) == -1);
    double a[d];
    orc_selfcond_row(&m, pp, a);
    double *ao = (double *)calloc((size_t)N * qw, sizeof(double));
    CHECK(orc_prefill_append(&m, tok, N, kc, vc, L, CAP, ao) == 0);
    CHECK(orc_prefill_append(&m, tok, N, kc, vc, CAP - 2, CAP, NULL) == -1);
    CHECK(orc_prefill_append(&m, tok, 0, kc, vc, L, CAP, NULL) == 0);
    free(ao);
    free(pp);
    free(so.h0);
    free(so.q);
    free(so.k_canvas);
    free(so.v_canvas);
    free(so.attn);
    free(so.h1);
    free(so.logits);
    free(so.probs);
    free(so.entropy);
    free(so.argmax);
    free(kc);
    free(vc);
    free(E);
    free(w1);
    free(w2);
    free(wq);
    free(wk);
    free(wv);
    free(wo);
    free(mask);
  }
  for (int kind = 0; kind < 3; ++kind) CHECK(isfinite(orc_temperature(kind, 1.5, 0.3, 3, 16)));
  CHECK(orc_temperature(2, 1.5, 0.3, 0, 1) == 1.5);
  free(b);
  CHECK(orc_num_threads() >= 1);
  printf("ok\n");
  return 0;
}
