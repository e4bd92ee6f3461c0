/*
 * dg_oracle.c -- CPU oracle (test infrastructure only; see dg_oracle.h).
 *
 * Double precision, plain loops, one function per step of the method in the
 * order the pages describe it.  No blocking, no fusion, no reordering of any
 * sum beyond "index ascending".  OpenMP only distributes independent outputs.
 */
#include "dg_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int32_t orc_num_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11, section 4): ten rounds of a Feistel-  */
/* like S-box built from two 32x32->64 multiplications; the two key words are */
/* bumped by the Weyl constants (golden ratio and sqrt(3)-1) between rounds.  */
/* ------------------------------------------------------------------------ */
static void philox_round(uint32_t x[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)x[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)x[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  const uint32_t y0 = hi1 ^ x[1] ^ k[0];
  const uint32_t y2 = hi0 ^ x[3] ^ k[1];
  x[0] = y0;
  x[1] = lo1;
  x[2] = y2;
  x[3] = lo0;
}

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox_round(x, k);
  }
  out[0] = x[0];
  out[1] = x[1];
  out[2] = x[2];
  out[3] = x[3];
}

static int32_t ilog2_exact(int32_t V) {
  int32_t b = 0;
  while ((1 << b) < V) ++b;
  return b;
}

int32_t orc_uniform_token(uint64_t seed, uint32_t pos, uint32_t step,
                          uint32_t canvas_id, uint32_t stream, int32_t V) {
  const uint32_t ctr[4] = {pos, step, canvas_id, stream};
  const uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  const int32_t bits = ilog2_exact(V);
  /* V is a power of two: the top log2(V) bits are uniform over [0, V). */
  return (int32_t)(out[0] >> (32 - bits));
}

void orc_canvas_init(uint64_t seed, uint32_t canvas_id, int32_t N, int32_t V,
                     int32_t *tokens) {
  for (int32_t i = 0; i < N; ++i)
    tokens[i] = orc_uniform_token(seed, (uint32_t)i, 0u, canvas_id, 0u, V);
}

/* ------------------------------------------------------------------------ */
/* Building blocks                                                           */
/* ------------------------------------------------------------------------ */
/* Embedding row of token t: E[t] for a vocabulary token, the [MASK] row for */
/* t = V when the model has one ([P1] §1, [P3] §3.1); NULL otherwise.        */
static const float *embed_row(const orc_model *m, int32_t t) {
  if (t >= 0 && t < m->V) return m->E + (int64_t)t * m->d;
  if (t == m->V && m->mask_emb) return m->mask_emb;
  return NULL;
}

double orc_gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

void orc_rmsnorm(const double *x, const float *g, int32_t d, double eps, double *out) {
  double ss = 0.0;
  for (int32_t k = 0; k < d; ++k) ss += x[k] * x[k];
  const double inv = 1.0 / sqrt(ss / (double)d + eps);
  for (int32_t k = 0; k < d; ++k) out[k] = x[k] * inv * (double)g[k];
}

void orc_matmul_nt(const double *a, const float *b, int32_t rows, int32_t cols,
                   int32_t k, double *y) {
  const int64_t total = (int64_t)rows * cols;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < total; ++t) {
    const int64_t r = t / cols, c = t % cols;
    const double *ar = a + r * (int64_t)k;
    const float *bc = b + c * (int64_t)k;
    double s = 0.0;
    for (int32_t j = 0; j < k; ++j) s += ar[j] * (double)bc[j];
    y[t] = s;
  }
}

void orc_softmax_entropy(const double *y, int32_t V, double *p, double *H) {
  double m = -INFINITY;
  for (int32_t v = 0; v < V; ++v)
    if (y[v] > m) m = y[v];
  double l = 0.0;
  for (int32_t v = 0; v < V; ++v) l += exp(y[v] - m);
  double h = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    const double pv = exp(y[v] - m) / l;
    if (p) p[v] = pv;
    if (pv > 0.0) h -= pv * log(pv);
  }
  *H = h;
}

int32_t orc_argmax(const double *z, int32_t V) {
  int32_t best = 0;
  for (int32_t v = 1; v < V; ++v)
    if (z[v] > z[best]) best = v;
  return best;
}

int32_t orc_argmax_f32(const float *z, int32_t V) {
  int32_t best = 0;
  for (int32_t v = 1; v < V; ++v)
    if (z[v] > z[best]) best = v;
  return best;
}

/* ------------------------------------------------------------------------ */
/* Multinomial candidate ([P3] §5.3, logits scheduler: the token is drawn     */
/* from the tempered softmax rather than always taken as the most likely).    */
/* Drawn by the Gumbel-max method: argmax_v (y_v + G_v) with G_v independent  */
/* standard Gumbel variables is distributed as softmax(y).  Every quantity    */
/* is single precision and every operation a separately rounded IEEE one      */
/* (the file is built with -ffp-contract=off), so the draw is a function of   */
/* the float logits alone and can be replayed exactly.                        */
/* ------------------------------------------------------------------------ */

/* Natural log of a positive normal float.  x = m 2^e with m folded into     */
/* (sqrt(1/2), sqrt(2)]; ln m = 2 atanh(s), s = (m - 1) / (m + 1), from the   */
/* odd series 2 (s + s^3/3 + s^5/5 + s^7/7 + s^9/9) (|s| <= 0.1716, so the    */
/* first omitted term is below 2^-27 of the result); ln 2 in two parts so     */
/* that e ln2_hi is exact.                                                    */
float orc_ln_f32(float x) {
  uint32_t b;
  memcpy(&b, &x, 4);
  int32_t e = (int32_t)((b >> 23) & 0xFFu) - 127;
  const uint32_t mb = (b & 0x7FFFFFu) | 0x3F800000u;
  float m;
  memcpy(&m, &mb, 4);
  if (m > 1.41421353816986083984375f) { /* the float nearest sqrt(2) */
    m = m * 0.5f;
    e = e + 1;
  }
  const float f = m - 1.0f;
  const float s = f / (2.0f + f);
  const float z = s * s;
  const float c3 = 2.0f / 3.0f, c5 = 2.0f / 5.0f, c7 = 2.0f / 7.0f, c9 = 2.0f / 9.0f;
  const float P = z * (c3 + z * (c5 + z * (c7 + z * c9)));
  const float lnm = (s + s) + s * P;
  const float ef = (float)e;
  const float ln2_hi = 0.693145751953125f;      /* 16 significant bits */
  const float ln2_lo = 1.42860676533018704e-6f; /* ln 2 - ln2_hi */
  return ef * ln2_hi + (ef * ln2_lo + lnm);
}

/* Standard Gumbel variable from a 32-bit word: u = (2 floor(w / 512) + 1)   */
/* 2^-24 lies in (0, 1) and is exact in float; G = -ln(-ln u).                */
float orc_gumbel_f32(uint32_t w) {
  const float u = (float)(2u * (w >> 9) + 1u) * 5.9604644775390625e-8f; /* 2^-24 */
  return -orc_ln_f32(-orc_ln_f32(u));
}

/* Key of a positive weight x in the log domain plus an offset and a Gumbel  */
/* variable: fl(fl(ln x + add) + G(word)); weights that are not positive     */
/* finite normal floats (zero, subnormal, inf, NaN) get -inf.                 */
static float gumbel_log_key(float x, float add, uint32_t word) {
  if (!(x >= 1.17549435e-38f && x <= 3.40282347e38f)) return -INFINITY;
  const float lx = orc_ln_f32(x) + add;
  return lx + orc_gumbel_f32(word);
}

/* Multinomial candidates ([P3] §5.3) drawn in two levels from the          */
/* distribution the step keeps, per row i (tiles of 64 columns):            */
/*   tile masses w_t = l_t e^{m_t}: l_t the tile's sum of e^{y - m_t},      */
/*   m_t = zmax_t inv_T; inside tile t the stored numerators num_v, which   */
/*   are e^{y_v - m_t} times a factor common to the tile.                   */
/* Level 1, the tile: the lowest t with the largest fl(fl(ln l_t + m_t) +   */
/*   G), G from word t%4 of Philox(seed; i, step, canvas_id, 2 + 4 floor(t/4)). */
/* Level 2, the column c of that tile: the lowest c with the largest        */
/*   fl(ln num_{64t+c} + G'), G' from word c%4 of Philox(seed; i, step,      */
/*   canvas_id, 3 + 4 floor(c/4)).                                          */
/* Gumbel-max at each level draws exactly from its categorical law, so the  */
/* token is drawn with probability (w_t / sum w) (num_v / sum_tile num),    */
/* i.e. softmax(y)_v.  NaN keys never win; a row with no key above -inf at  */
/* either level takes fallback[i].                                          */
void orc_multinomial_candidates(const float *tile_zmax, const float *tile_l, int32_t N,
                                int32_t ntiles, const float *num, float inv_T, uint64_t seed,
                                uint32_t step, uint32_t canvas_id, const int32_t *fallback,
                                int32_t *out) {
  const uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
  for (int32_t i = 0; i < N; ++i) {
    float best = -INFINITY;
    int32_t tile = -1;
    for (int32_t t = 0; t < ntiles; ++t) {
      const uint32_t ctr[4] = {(uint32_t)i, step, canvas_id, 2u + 4u * ((uint32_t)t >> 2)};
      uint32_t w[4];
      orc_philox4x32_10(ctr, key, w);
      const float m = tile_zmax[(int64_t)i * ntiles + t] * inv_T;
      const float k = gumbel_log_key(tile_l[(int64_t)i * ntiles + t], m, w[t & 3]);
      if (k > best) {
        best = k;
        tile = t;
      }
    }
    int32_t col = -1;
    if (tile >= 0) {
      best = -INFINITY;
      for (int32_t c = 0; c < 64; ++c) {
        const uint32_t ctr[4] = {(uint32_t)i, step, canvas_id, 3u + 4u * ((uint32_t)c >> 2)};
        uint32_t w[4];
        orc_philox4x32_10(ctr, key, w);
        const float k = gumbel_log_key(num[(int64_t)i * ntiles * 64 + (int64_t)tile * 64 + c], 0.0f,
                                       w[c & 3]);
        if (k > best) {
          best = k;
          col = c;
        }
      }
    }
    out[i] = col >= 0 ? tile * 64 + col : fallback[i];
  }
}

void orc_attention(const double *q, const double *k, const double *v,
                   int32_t nq, int32_t nk, int32_t Hq, int32_t Hkv, int32_t hd,
                   int32_t causal, int32_t q_pos0, double *out) {
  const int32_t group = Hq / Hkv;
  const double scale = 1.0 / sqrt((double)hd);
  const int64_t total = (int64_t)nq * Hq;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < total; ++t) {
    const int32_t i = (int32_t)(t / Hq), h = (int32_t)(t % Hq);
    const int32_t g = h / group;
    const double *qi = q + (int64_t)i * Hq * hd + (int64_t)h * hd;
    const double *kg = k + (int64_t)g * nk * hd;
    const double *vg = v + (int64_t)g * nk * hd;
    const int32_t nvis = causal ? (q_pos0 + i + 1 < nk ? q_pos0 + i + 1 : nk) : nk;
    double *s = (double *)malloc(sizeof(double) * (size_t)(nvis > 0 ? nvis : 1));
    double m = -INFINITY;
    for (int32_t j = 0; j < nvis; ++j) {
      double dot = 0.0;
      for (int32_t e = 0; e < hd; ++e) dot += qi[e] * kg[(int64_t)j * hd + e];
      s[j] = dot * scale;
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int32_t j = 0; j < nvis; ++j) {
      s[j] = exp(s[j] - m);
      l += s[j];
    }
    double *o = out + (int64_t)i * Hq * hd + (int64_t)h * hd;
    for (int32_t e = 0; e < hd; ++e) {
      double acc = 0.0;
      for (int32_t j = 0; j < nvis; ++j) acc += s[j] * vg[(int64_t)j * hd + e];
      o[e] = acc / l;
    }
    free(s);
  }
}

/* ------------------------------------------------------------------------ */
/* Entropy-bounded selection.                                                */
/* [P3] §5.4 token acceptance: order the positions from lowest to highest    */
/* entropy; walking that order, a position is kept while the running sum of  */
/* entropies seen so far, less the largest of them, stays within the limit;  */
/* the first failure ends the walk.  [P5] states the same walk with the plain */
/* cumulative sum (ORC_ACCEPT_CUMSUM).  [P3] §5.4 re-noise: every rejected   */
/* position receives a fresh uniform token.  [P3] §5.3 / [P5] adaptive stop: */
/* confidence (entropies below a threshold) and stability (predictions, or  */
/* the canvas, unchanged from the previous step).                            */
/*                                                                           */
/* Readings where the pages leave a step open:                               */
/*  - the running sums are taken in 2^-32-nat fixed point, q = floor(H*2^32), */
/*    so the decision does not depend on summation order;                     */
/*  - entropies are ordered by (H, position) with H clamped at +0; NaN and   */
/*    absurd values (>= 2^20 nats) end the walk and are never accepted;       */
/*  - an accepted position takes the argmax token.                           */
/* ------------------------------------------------------------------------ */
static int cmp_u64(const void *a, const void *b) {
  const uint64_t x = *(const uint64_t *)a, y = *(const uint64_t *)b;
  return (x > y) - (x < y);
}

static float clamp_entropy(float h) { return (h <= 0.0f) ? 0.0f : h; }

static uint64_t fixed_point_nats(double x) {
  /* x >= 0 and finite; 2^32 scaling is exact in double. */
  const double s = x * 4294967296.0;
  if (s >= 18446744073709551615.0) return UINT64_MAX;
  return (uint64_t)s;
}

void orc_select(int32_t N, int32_t V, const float *H, const int32_t *argmax,
                const int32_t *tokens_in, double gamma, int32_t rule,
                uint64_t seed, uint32_t canvas_id, uint32_t step,
                int32_t stable_in, double conf_eps, int32_t mask_id,
                const int32_t *pred, const int32_t *pred_prev, int32_t stable_rule,
                uint8_t *accept, int32_t *tokens_out, orc_flags *flags) {
  /* the positions that take part: all of them, or (masked sampler) those */
  /* still holding [MASK]                                                  */
  uint64_t *keys = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)(N > 0 ? N : 1));
  int32_t n = 0;
  for (int32_t i = 0; i < N; ++i) {
    accept[i] = 0;
    if (mask_id >= 0 && tokens_in[i] != mask_id) continue;
    const float h = clamp_entropy(H[i]);
    uint32_t bits;
    memcpy(&bits, &h, 4);
    keys[n++] = ((uint64_t)bits << 32) | (uint32_t)i;
  }
  qsort(keys, (size_t)n, sizeof(uint64_t), cmp_u64);

  const uint64_t limit = (gamma > 0.0) ? fixed_point_nats(gamma) : 0u;
  uint64_t sum_before = 0; /* sum of q over the positions already accepted */
  int32_t accepted = 0;
  for (int32_t r = 0; r < n; ++r) {
    const int32_t i = (int32_t)(keys[r] & 0xFFFFFFFFu);
    const float h = clamp_entropy(H[i]);
    if (!(h < 1048576.0f)) break; /* NaN, inf or absurd: never accepted */
    const uint64_t q = fixed_point_nats((double)h);
    /* ascending order: the largest entropy of the walked prefix is q itself,
     * so "sum minus max" is the sum of the positions before this one. */
    const uint64_t test = (rule == ORC_ACCEPT_CUMSUM) ? sum_before + q : sum_before;
    if (test > limit) break;
    accept[i] = 1;
    ++accepted;
    sum_before += q;
  }
  free(keys);

  /* the entropies are floats, so the confidence test is a float comparison */
  const float eps = (float)conf_eps;
  int32_t allconf = 1, changed = 0, masked = 0;
  for (int32_t i = 0; i < N; ++i) {
    int32_t t;
    if (accept[i])
      t = argmax[i];
    else if (mask_id >= 0)
      t = tokens_in[i]; /* a locked token, or [MASK] staying [MASK] */
    else
      t = orc_uniform_token(seed, (uint32_t)i, step, canvas_id, 1u, V);
    tokens_out[i] = t;
    if (t != tokens_in[i]) changed = 1;
    if (mask_id >= 0 && t == mask_id) ++masked;
    const float h = clamp_entropy(H[i]);
    if (!(h < eps)) allconf = 0;
  }
  /* [P3] §5.3 / [P5]: are the predictions those of the previous step?  Not  */
  /* at a canvas's first step, and not when any entropy is NaN (a position  */
  /* without a distribution has no prediction to compare).                   */
  int32_t pred_changed = 1;
  if (pred != NULL && pred_prev != NULL) {
    pred_changed = 0;
    for (int32_t i = 0; i < N; ++i)
      if (pred[i] != pred_prev[i] || H[i] != H[i]) pred_changed = 1;
  }
  flags->allconf = allconf;
  flags->changed = changed;
  flags->pred_changed = pred_changed;
  if (stable_rule == ORC_STABLE_PREDICTIONS)
    flags->stable = pred_changed ? 0 : stable_in + 1;
  else
    flags->stable = changed ? 0 : stable_in + 1;
  flags->accepted = accepted;
  flags->masked = mask_id >= 0 ? masked : -1;
}

/* ------------------------------------------------------------------------ */
/* One denoising step                                                         */
/* ------------------------------------------------------------------------ */

/* [P3] §5.1 self-conditioning: the previous step's softmax probabilities   */
/* weight the rows of the token-embedding table.                              */
void orc_selfcond_row(const orc_model *m, const double *p_row, double *a) {
  for (int32_t k = 0; k < m->d; ++k) a[k] = 0.0;
  for (int32_t v = 0; v < m->V; ++v) {
    const double pv = p_row[v];
    const float *ev = m->E + (int64_t)v * m->d;
    for (int32_t k = 0; k < m->d; ++k) a[k] += pv * (double)ev[k];
  }
}

static int row_on(const uint8_t *row_sel, int32_t i) { return row_sel == NULL || row_sel[i]; }

int orc_denoise_forward(const orc_model *m, const int32_t *tokens,
                        const double *p_prev, const double *k_cache,
                        const double *v_cache, int32_t L, int32_t cap,
                        double T, const uint8_t *row_sel, orc_step_out *out) {
  const int32_t N = m->N, V = m->V, d = m->d, F = m->F;
  const int32_t Hq = m->Hq, Hkv = m->Hkv, hd = m->hd;
  const int32_t qw = Hq * hd, kw = Hkv * hd;
  if (Hq % Hkv != 0 || L < 0 || L > cap || !(T > 0.0)) return -1;
  for (int32_t i = 0; i < N; ++i)
    if (!embed_row(m, tokens[i])) return -2;

  /* 1. token embeddings ([P3] §5.1: the self-conditioning vector is added to */
  /*    the next step's token embeddings).                                     */
  double *h0 = out->h0;
  for (int32_t i = 0; i < N; ++i)
    for (int32_t k = 0; k < d; ++k) h0[(int64_t)i * d + k] = (double)embed_row(m, tokens[i])[k];

  /* 2. self-conditioning: p_prev @ E, then a small feed-forward network     */
  /*    (two layers, exact GELU, no biases), added to the embeddings.         */
  if (p_prev) {
    double *a = (double *)malloc(sizeof(double) * (size_t)N * d);
    double *u = (double *)malloc(sizeof(double) * (size_t)N * F);
    double *w = (double *)malloc(sizeof(double) * (size_t)N * d);
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < N; ++i) orc_selfcond_row(m, p_prev + (int64_t)i * V, a + (int64_t)i * d);
    orc_matmul_nt(a, m->w1, N, F, d, u);
    for (int64_t t = 0; t < (int64_t)N * F; ++t) u[t] = orc_gelu(u[t]);
    orc_matmul_nt(u, m->w2, N, d, F, w);
    for (int64_t t = 0; t < (int64_t)N * d; ++t) h0[t] += w[t];
    free(a);
    free(u);
    free(w);
  }

  /* 3-4. pre-attention RMSNorm and the Q/K/V projections of every row. */
  double *nrm = (double *)malloc(sizeof(double) * (size_t)N * d);
  for (int32_t i = 0; i < N; ++i) orc_rmsnorm(h0 + (int64_t)i * d, m->g_attn, d, m->rms_eps, nrm + (int64_t)i * d);
  double *q = (double *)malloc(sizeof(double) * (size_t)N * qw);
  double *kc = (double *)malloc(sizeof(double) * (size_t)N * kw);
  double *vc = (double *)malloc(sizeof(double) * (size_t)N * kw);
  orc_matmul_nt(nrm, m->wq, N, qw, d, q);
  orc_matmul_nt(nrm, m->wk, N, kw, d, kc);
  orc_matmul_nt(nrm, m->wv, N, kw, d, vc);
  if (out->q) memcpy(out->q, q, sizeof(double) * (size_t)N * qw);

  /* 5. bidirectional attention of every canvas query over                  */
  /*    [prefix cache || canvas] with no mask ([P1]/[P4] denoise mode; [P3]   */
  /*    §4.1).  The cache is only read ([P3] §4.2).                           */
  const int32_t nk = L + N;
  double *K = (double *)malloc(sizeof(double) * (size_t)Hkv * nk * hd);
  double *Vv = (double *)malloc(sizeof(double) * (size_t)Hkv * nk * hd);
  for (int32_t g = 0; g < Hkv; ++g) {
    for (int32_t j = 0; j < L; ++j)
      for (int32_t e = 0; e < hd; ++e) {
        K[((int64_t)g * nk + j) * hd + e] = k_cache[((int64_t)g * cap + j) * hd + e];
        Vv[((int64_t)g * nk + j) * hd + e] = v_cache[((int64_t)g * cap + j) * hd + e];
      }
    for (int32_t i = 0; i < N; ++i)
      for (int32_t e = 0; e < hd; ++e) {
        K[((int64_t)g * nk + L + i) * hd + e] = kc[(int64_t)i * kw + (int64_t)g * hd + e];
        Vv[((int64_t)g * nk + L + i) * hd + e] = vc[(int64_t)i * kw + (int64_t)g * hd + e];
      }
  }
  if (out->k_canvas)
    for (int32_t g = 0; g < Hkv; ++g)
      for (int32_t i = 0; i < N; ++i)
        for (int32_t e = 0; e < hd; ++e) {
          out->k_canvas[((int64_t)g * N + i) * hd + e] = kc[(int64_t)i * kw + (int64_t)g * hd + e];
          out->v_canvas[((int64_t)g * N + i) * hd + e] = vc[(int64_t)i * kw + (int64_t)g * hd + e];
        }

  /* selected rows only from here on */
  int32_t nsel = 0;
  for (int32_t i = 0; i < N; ++i) nsel += row_on(row_sel, i);
  int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nsel > 0 ? nsel : 1));
  for (int32_t i = 0, c = 0; i < N; ++i)
    if (row_on(row_sel, i)) sel[c++] = i;

  double *o1 = (double *)malloc(sizeof(double) * (size_t)qw);
  double *t1 = (double *)malloc(sizeof(double) * (size_t)d);
  double *n2 = (double *)malloc(sizeof(double) * (size_t)d);
  double *z = (double *)malloc(sizeof(double) * (size_t)V);
  double *y = (double *)malloc(sizeof(double) * (size_t)V);
  for (int32_t c = 0; c < nsel; ++c) {
    const int32_t i = sel[c];
    orc_attention(q + (int64_t)i * qw, K, Vv, 1, nk, Hq, Hkv, hd, 0, 0, o1);
    if (out->attn) memcpy(out->attn + (int64_t)i * qw, o1, sizeof(double) * (size_t)qw);

    /* 6. output projection + residual */
    orc_matmul_nt(o1, m->wo, 1, d, qw, t1);
    double *h1 = out->h1 + (int64_t)i * d;
    for (int32_t k = 0; k < d; ++k) h1[k] = h0[(int64_t)i * d + k] + t1[k];

    /* 7. final RMSNorm, tied LM head: z = n2 . E^T */
    orc_rmsnorm(h1, m->g_final, d, m->rms_eps, n2);
    orc_matmul_nt(n2, m->E, 1, V, d, z);
    if (out->logits) memcpy(out->logits + (int64_t)i * V, z, sizeof(double) * (size_t)V);

    /* 8. logits temperature ([P3] §5.3: logits divided by the temperature), */
    /*    softmax and per-position entropy in nats ([P3] §5.4). */
    for (int32_t v = 0; v < V; ++v) y[v] = z[v] / T;
    double H;
    orc_softmax_entropy(y, V, out->probs ? out->probs + (int64_t)i * V : NULL, &H);
    out->entropy[i] = H;
    out->argmax[i] = orc_argmax(z, V);
  }
  free(o1);
  free(t1);
  free(n2);
  free(z);
  free(y);
  free(sel);
  free(K);
  free(Vv);
  free(q);
  free(kc);
  free(vc);
  free(nrm);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Causal incremental prefill: the encoder mode writes keys/values of new   */
/* tokens into the cache; each token attends causally; no LM head.           */
/* ([P1]/[P4] architecture section; [P3] §4.2 and §5.2.)                    */
/* ------------------------------------------------------------------------ */
int orc_prefill_append(const orc_model *m, const int32_t *tokens, int32_t n,
                       double *k_cache, double *v_cache, int32_t L, int32_t cap,
                       double *attn_out) {
  const int32_t d = m->d, Hq = m->Hq, Hkv = m->Hkv, hd = m->hd;
  const int32_t qw = Hq * hd, kw = Hkv * hd;
  if (n < 0 || L < 0 || L + n > cap || Hq % Hkv != 0) return -1;
  for (int32_t i = 0; i < n; ++i)
    if (!embed_row(m, tokens[i])) return -2;
  if (n == 0) return 0;
  double *x = (double *)malloc(sizeof(double) * (size_t)n * d);
  double *nrm = (double *)malloc(sizeof(double) * (size_t)n * d);
  double *kk = (double *)malloc(sizeof(double) * (size_t)n * kw);
  double *vv = (double *)malloc(sizeof(double) * (size_t)n * kw);
  for (int32_t i = 0; i < n; ++i) {
    for (int32_t k = 0; k < d; ++k) x[(int64_t)i * d + k] = (double)embed_row(m, tokens[i])[k];
    orc_rmsnorm(x + (int64_t)i * d, m->g_attn, d, m->rms_eps, nrm + (int64_t)i * d);
  }
  orc_matmul_nt(nrm, m->wk, n, kw, d, kk);
  orc_matmul_nt(nrm, m->wv, n, kw, d, vv);
  for (int32_t i = 0; i < n; ++i)
    for (int32_t g = 0; g < Hkv; ++g)
      for (int32_t e = 0; e < hd; ++e) {
        k_cache[((int64_t)g * cap + L + i) * hd + e] = kk[(int64_t)i * kw + (int64_t)g * hd + e];
        v_cache[((int64_t)g * cap + L + i) * hd + e] = vv[(int64_t)i * kw + (int64_t)g * hd + e];
      }
  if (attn_out) {
    double *q = (double *)malloc(sizeof(double) * (size_t)n * qw);
    orc_matmul_nt(nrm, m->wq, n, qw, d, q);
    /* keys of the cache as a contiguous [Hkv][L+n][hd] view */
    const int32_t nk = L + n;
    double *K = (double *)malloc(sizeof(double) * (size_t)Hkv * nk * hd);
    double *Vv = (double *)malloc(sizeof(double) * (size_t)Hkv * nk * hd);
    for (int32_t g = 0; g < Hkv; ++g)
      for (int32_t j = 0; j < nk; ++j)
        for (int32_t e = 0; e < hd; ++e) {
          K[((int64_t)g * nk + j) * hd + e] = k_cache[((int64_t)g * cap + j) * hd + e];
          Vv[((int64_t)g * nk + j) * hd + e] = v_cache[((int64_t)g * cap + j) * hd + e];
        }
    orc_attention(q, K, Vv, n, nk, Hq, Hkv, hd, 1, L, attn_out);
    free(q);
    free(K);
    free(Vv);
  }
  free(x);
  free(nrm);
  free(kk);
  free(vv);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Scheduler                                                                 */
/* [P3] §5.3: the logits temperature falls as the steps count down, so early */
/* steps explore and late steps exploit; [P5] names a cosine schedule.  With */
/* t = s/(S-1): linear T0 + (T1-T0) t; cosine T1 + (T0-T1)(1 + cos(pi t))/2. */
/* Adaptive stop ([P5] scheduler, either condition suffices): every entropy */
/* below the confidence threshold, or stable for the given number of steps. */
/* ------------------------------------------------------------------------ */
double orc_temperature(int32_t kind, double T0, double T1, int32_t s, int32_t S) {
  const double t = (S > 1) ? (double)s / (double)(S - 1) : 0.0;
  if (kind == ORC_SCHED_LINEAR) return T0 + (T1 - T0) * t;
  if (kind == ORC_SCHED_COSINE) return T1 + (T0 - T1) * 0.5 * (1.0 + cos(M_PI * t));
  return T0;
}

int32_t orc_should_stop(const orc_flags *f, int32_t stable_steps) {
  if (f->allconf) return 1;
  if (f->masked == 0) return 1; /* masked sampler: no [MASK] left */
  if (stable_steps > 0 && f->stable >= stable_steps) return 1;
  return 0;
}
