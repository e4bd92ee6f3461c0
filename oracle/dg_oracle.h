/*
 * dg_oracle.h -- CPU oracle for the uniform-state text-diffusion denoising
 * step.  TEST INFRASTRUCTURE ONLY: this library is the independent,
 * slow, obviously-correct reference that the HIP path is checked against.
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load it; the product path never does.
 *
 * Arithmetic is IEEE double throughout, except the multinomial draw, which
 * is defined in single precision so that it replays exactly on the GPU's
 * float statistics.  Inputs arrive as float arrays whose
 * values are exactly what the GPU path receives (for bf16 configurations the
 * harness rounds them to bf16 first, so they upcast exactly), which leaves
 * the arithmetic as the only difference between the two sides.
 *
 * It shares no code, header, table or constant generator with the GPU
 * library.  Loops are plain; OpenMP splits only independent outputs, so every
 * result is bitwise independent of the thread count.
 *
 * Sources (web pages on DiffusionGemma):
 *   [P1] "文字生成中的擴散模型解析" (DiffusionGemma explained, zh-TW mirror)
 *   [P2] "DiffusionGemma——把文字生成從自迴歸換成擴散去噪" (deep-dive blog)
 *   [P3] "DiffusionGemma 图解" (A Visual Guide to DiffusionGemma, zh-CN)
 *   [P4] DiffusionGemma explained (ai.google.dev, Japanese)
 *   [P5] DiffusionGemma local-deployment workshop (yomxxx.com)
 * Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 *   easy as 1, 2, 3", SC'11.
 *
 * Parity pins: every function here is pinned by a CPU test (closed forms,
 * library routines on small cases, invariants, published Philox known-answer
 * vectors).  The whole-model convergence behaviour of the pages' trained
 * 26B model is "parity unpinned": no trained weights or worked numeric
 * example exist to pin it against.
 */
#ifndef DG_ORACLE_H
#define DG_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* ---- counter-based random numbers (Philox4x32-10, SC'11) ---------------- */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* Uniform vocabulary token for canvas position `pos`: the top log2(V) bits of
 * word 0 of Philox4x32-10 with key = (seed low 32, seed high 32) and counter
 * (pos, step, canvas_id, stream).  stream 0 = canvas initialisation, stream 1
 * = re-noise.  V must be a power of two >= 2. */
int32_t orc_uniform_token(uint64_t seed, uint32_t pos, uint32_t step,
                          uint32_t canvas_id, uint32_t stream, int32_t V);

/* [P3] §5.4 canvas initialisation; [P5] reverse process, first step:
 * every canvas position starts as a uniformly drawn vocabulary token. */
void orc_canvas_init(uint64_t seed, uint32_t canvas_id, int32_t N, int32_t V,
                     int32_t *tokens);

/* ---- model description --------------------------------------------------- */
typedef struct {
  int32_t N, V, d, Hq, Hkv, hd, F;
  double rms_eps;
  const float *E;       /* [V][d] token-embedding table, tied LM head        */
  const float *w1;      /* [F][d] self-conditioning FFN, first layer         */
  const float *w2;      /* [d][F] self-conditioning FFN, second layer        */
  const float *wq;      /* [Hq*hd][d]                                        */
  const float *wk;      /* [Hkv*hd][d]                                       */
  const float *wv;      /* [Hkv*hd][d]                                       */
  const float *wo;      /* [d][Hq*hd]                                        */
  const float *g_attn;  /* [d] RMSNorm gain before attention                 */
  const float *g_final; /* [d] RMSNorm gain before the LM head               */
  const float *mask_emb; /* [d] embedding of the [MASK] token, id V (masked    */
                         /* sampler); NULL: the model has no [MASK] token      */
} orc_model;

/* ---- building blocks (exported so the tests can pin each one) ----------- */
double orc_gelu(double x);                                     /* exact erf GELU */
void orc_rmsnorm(const double *x, const float *g, int32_t d, double eps, double *out);
/* y[r][c] = sum_k a[r][k] * b[c][k]  (b given row-major [cols][k], float) */
void orc_matmul_nt(const double *a, const float *b, int32_t rows, int32_t cols,
                   int32_t k, double *y);
/* Softmax of y[0..V) and its entropy in nats; p may be NULL. */
void orc_softmax_entropy(const double *y, int32_t V, double *p, double *H);
int32_t orc_argmax(const double *z, int32_t V);          /* lowest index on ties */
int32_t orc_argmax_f32(const float *z, int32_t V);       /* same, float input    */
/* Multinomial candidate ([P3] §5.3) by Gumbel-max, single precision with
 * separately rounded operations so the draw replays exactly:
 *   orc_ln_f32: natural log of a positive normal float (fixed evaluation);
 *   orc_gumbel_f32: -ln(-ln u), u = (2 floor(w/512) + 1) 2^-24;
 *   orc_multinomial_candidates: two levels over 64-column tiles -- the tile
 *     by the largest fl(fl(ln l_t + zmax_t inv_T) + G) (Philox counter
 *     (i, step, canvas_id, 2 + 4 floor(t/4)), word t%4), then the column c
 *     by the largest fl(ln num + G') (counter (i, step, canvas_id,
 *     3 + 4 floor(c/4)), word c%4); lowest index on ties, NaN never wins,
 *     fallback[i] when no key exceeds -inf.  tile_zmax, tile_l: [N][ntiles];
 *     num: the numerators [N][64 ntiles] (row-major floats). */
float orc_ln_f32(float x);
float orc_gumbel_f32(uint32_t w);
void orc_multinomial_candidates(const float *tile_zmax, const float *tile_l, int32_t N,
                                int32_t ntiles, const float *num, float inv_T, uint64_t seed,
                                uint32_t step, uint32_t canvas_id, const int32_t *fallback,
                                int32_t *out);
/* Multi-head attention, query head h reads KV head h / (Hq/Hkv).
 * q: [nq][Hq*hd]; keys/values: [Hkv][nk][hd] (key-major inside a head);
 * causal: query i may read keys 0 .. q_pos0 + i (absolute key positions).
 * out: [nq][Hq*hd]. */
void orc_attention(const double *q, const double *k, const double *v,
                   int32_t nq, int32_t nk, int32_t Hq, int32_t Hkv, int32_t hd,
                   int32_t causal, int32_t q_pos0, double *out);

/* ---- entropy-bounded selection ([P3] §5.4, [P5] entropy-constrained sampler) */
enum { ORC_ACCEPT_SUM_MINUS_MAX = 0, ORC_ACCEPT_CUMSUM = 1 };
/* What "stable" counts ([P3] §5.3 adaptive stop: the highest-probability    */
/* predictions unchanged over the last N steps; [P5] scheduler: the         */
/* predictions identical for N consecutive steps).                           */
/*   PREDICTIONS: steps in a row whose predictions (each position's most     */
/*     likely token) equal the previous step's at every position; a step    */
/*     with no previous step, or with a NaN entropy anywhere, resets it.     */
/*   CANVAS: steps in a row that left the canvas unchanged (equal to         */
/*     PREDICTIONS whenever every position is accepted with its argmax).     */
enum { ORC_STABLE_PREDICTIONS = 0, ORC_STABLE_CANVAS = 1 };
typedef struct {
  int32_t allconf;   /* every entropy < conf_eps (NaN counts as not confident) */
  int32_t changed;   /* canvas after != canvas before                          */
  int32_t stable;    /* consecutive stable steps, by the stability rule        */
  int32_t accepted;  /* number of accepted positions                           */
  int32_t masked;    /* [MASK] positions after the step; -1 under re-noise      */
  int32_t pred_changed; /* predictions differ from the previous step's, or    */
                        /* there is none, or an entropy is NaN                */
} orc_flags;

/* Decisions of one step from the per-position entropies H (float, as the
 * kernel produces them) and candidate tokens.  Writes accept[N] (0/1),
 * tokens_out[N] and flags.  pred[N]: the step's predictions (the most
 * likely token of each position); pred_prev[N]: the previous step's, NULL at
 * a canvas's first step; pred_changed is reported under either rule, the
 * stable count follows stable_rule.
 * conf_eps is compared in single precision, as the entropies are.
 * mask_id < 0: uniform-state sampler -- every position takes part, rejected
 *   ones are re-noised with a uniform token.
 * mask_id >= 0: masked sampler ([P1] §1, [P3] §3.1) -- only positions holding
 *   mask_id take part in the walk; accepted ones take their candidate and
 *   lock, rejected ones stay mask_id, the others keep their token. */
void orc_select(int32_t N, int32_t V, const float *H, const int32_t *argmax,
                const int32_t *tokens_in, double gamma, int32_t rule,
                uint64_t seed, uint32_t canvas_id, uint32_t step,
                int32_t stable_in, double conf_eps, int32_t mask_id,
                const int32_t *pred, const int32_t *pred_prev, int32_t stable_rule,
                uint8_t *accept, int32_t *tokens_out, orc_flags *flags);

/* ---- one denoising step ---------------------------------------------------- */
typedef struct {
  double *h0;        /* [N][d]      embeddings + self-conditioning            */
  double *q;         /* [N][Hq*hd]  (nullable)                                */
  double *k_canvas;  /* [Hkv][N][hd] (nullable)                               */
  double *v_canvas;  /* [Hkv][N][hd] (nullable)                               */
  double *attn;      /* [N][Hq*hd]  attention output (selected rows)          */
  double *h1;        /* [N][d]      after the output projection (selected)    */
  double *logits;    /* [N][V]      z, before temperature (selected rows)     */
  double *probs;     /* [N][V]      softmax(z/T) (selected rows)              */
  double *entropy;   /* [N]         nats (selected rows)                      */
  int32_t *argmax;   /* [N]         (selected rows)                           */
} orc_step_out;

/* Everything up to per-position entropy/argmax.  p_prev is the previous
 * step's tempered softmax [N][V] (NULL on the first step of a canvas).
 * Cache K/V: [Hkv][cap][hd], positions [0, L) are valid; the step only reads
 * them.  row_sel[N] (nullable) restricts attention, output projection and the
 * LM head to the selected rows; the canvas keys/values always use all rows. */
int orc_denoise_forward(const orc_model *m, const int32_t *tokens,
                        const double *p_prev, const double *k_cache,
                        const double *v_cache, int32_t L, int32_t cap,
                        double T, const uint8_t *row_sel, orc_step_out *out);

/* Self-conditioning vector of one canvas row: a = sum_v p[v] * E[v][:]. */
void orc_selfcond_row(const orc_model *m, const double *p_row, double *a);

/* ---- causal (incremental) prefill ([P1]/[P4] architecture; [P3] §5.2) ----- */
/* Appends the keys/values of tokens[0..n) at cache positions [L, L+n).
 * If attn_out is non-NULL also writes the causal attention output
 * [n][Hq*hd] of the new tokens over keys [0, L+i]. */
int orc_prefill_append(const orc_model *m, const int32_t *tokens, int32_t n,
                       double *k_cache, double *v_cache, int32_t L, int32_t cap,
                       double *attn_out);

/* ---- scheduler ([P3] §5.3, [P5] scheduler knobs) --------------------------- */
enum { ORC_SCHED_CONST = 0, ORC_SCHED_LINEAR = 1, ORC_SCHED_COSINE = 2 };
double orc_temperature(int32_t kind, double T0, double T1, int32_t s, int32_t S);
int32_t orc_should_stop(const orc_flags *f, int32_t stable_steps);

int32_t orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
