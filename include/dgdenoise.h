/*
 * dgdenoise.h -- C ABI of libdgdenoise: the uniform-state text-diffusion
 * denoising step on AMD Instinct MI355X (gfx950).
 *
 * The operations follow the DiffusionGemma pages:
 *   [P1] "文字生成中的擴散模型解析" (DiffusionGemma explained, zh-TW mirror)
 *   [P2] "DiffusionGemma——把文字生成從自迴歸換成擴散去噪" (deep-dive blog)
 *   [P3] "DiffusionGemma 图解" (A Visual Guide to DiffusionGemma, zh-CN)
 *   [P4] DiffusionGemma explained (ai.google.dev, Japanese)
 *   [P5] DiffusionGemma local-deployment workshop (yomxxx.com)
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are device (HBM) addresses owned by the caller;
 *    the library never frees or retains them.  Pointers marked "host" are
 *    read or written before the call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Entry points are asynchronous on that stream unless stated otherwise.
 *  - Every argument is validated on the host before the first launch.  A call
 *    that returns anything other than DG_OK has launched nothing and changed
 *    no buffer (cache, canvas or workspace).  DG_ERR_HIP means a launch was
 *    rejected by the runtime after validation; device faults surface at the
 *    caller's next synchronisation.
 *  - Dense matrices are row-major.  bf16 values are IEEE binary32 truncated
 *    to the upper 16 bits after round-to-nearest-even.
 *  - The library allocates no device memory on the compute path: scratch
 *    lives in a caller-provided workspace of dg_workspace_bytes() bytes.
 *  - Calls that share a workspace or a canvas must be ordered (same stream or
 *    explicit events); concurrent calls on them race.
 */
#ifndef DGDENOISE_H
#define DGDENOISE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_ABI_VERSION 9

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad enum, NaN/negative threshold */
  DG_ERR_UNSUPPORTED = 2,   /* shape outside what the kernels implement */
  DG_ERR_CAPACITY = 3,      /* KV cache would overflow */
  DG_ERR_WORKSPACE = 4,     /* workspace smaller than dg_workspace_bytes() */
  DG_ERR_HIP = 5            /* the HIP runtime rejected a launch or copy */
} dg_status;

typedef enum { DG_F32 = 0, DG_BF16 = 1 } dg_dtype;

/* Acceptance rule of the entropy-bounded sampler.
 * SUM_MINUS_MAX: [P3] §5.4 -- walking positions from lowest entropy upward, a
 *   position is accepted while (sum of entropies walked so far) minus (their
 *   maximum) stays <= the threshold.  Always accepts at least one position.
 * CUMSUM: [P5] entropy-constrained sampler -- the plain running sum must stay
 *   <= the threshold. */
typedef enum { DG_ACCEPT_SUM_MINUS_MAX = 0, DG_ACCEPT_CUMSUM = 1 } dg_accept_rule;

/* Token placed at an accepted position.
 * ARGMAX: the most likely token (highest logit, lowest index on ties); the
 *   pages' figures speak of the most likely token.
 * MULTINOMIAL: [P3] §5.3 logits scheduler -- a draw from the tempered
 *   softmax p = softmax(z / T), made from the distribution the step keeps
 *   (tile statistics and stored numerators, 64-column tiles) in two
 *   Gumbel-max levels, each of which draws exactly from its categorical law:
 *     tile t: the largest fl(fl(ln l_t + zmax_t * inv_T) + G), l_t the
 *       tile's sum of e^(y - m_t), G from word t % 4 of Philox4x32-10(key =
 *       seed, counter = (i, step, canvas_id, 2 + 4 floor(t / 4)));
 *     column c of that tile: the largest fl(ln num_c + G'), num_c the stored
 *       numerator, G' from word c % 4 of counter (i, step, canvas_id,
 *       3 + 4 floor(c / 4));
 *   lowest index on equal keys, NaN keys (and weights that are not positive
 *   normal floats) never drawn, the argmax when nothing is drawable.
 *   G = -ln(-ln u), u = (2 floor(w / 512) + 1) 2^-24, inv_T = (float)(1 / T)
 *   as the step computes it, and ln a fixed single-precision evaluation
 *   (x = m 2^e, m in (sqrt(1/2), sqrt(2)]; 2 atanh((m-1)/(m+1)) to the s^9
 *   term; e ln 2 with ln 2 = 0.693145751953125 + 1.42860676533018704e-6),
 *   every operation rounded on its own, so the draw replays exactly from the
 *   step's float statistics. */
typedef enum { DG_CANDIDATE_ARGMAX = 0, DG_CANDIDATE_MULTINOMIAL = 1 } dg_candidate_rule;

/* Noise of the reverse process.
 * UNIFORM: uniform-state diffusion ([P1] §2, [P3] §3.2, §5.4) -- the canvas
 *   starts as uniform vocabulary tokens and every rejected position is
 *   re-noised with a fresh one; no position is ever locked.
 * MASKED: masked diffusion, the variant the pages contrast it with ([P1] §1,
 *   [P3] §3.1) -- the [MASK] token, id V (one past the vocabulary, embedded
 *   by dg_weights.mask_emb and never predicted by the tied head), stands for
 *   the noise: the canvas starts all [MASK]; a step walks only the positions
 *   still holding [MASK] (same order, rule and threshold), accepted ones take
 *   their candidate and are locked from then on, rejected ones stay [MASK];
 *   the loop also stops when no [MASK] is left. */
typedef enum { DG_SAMPLER_UNIFORM = 0, DG_SAMPLER_MASKED = 1 } dg_sampler;

/* Storage of the packed table (DG_BF16 only; DG_F32 ignores it).  The
 * library keeps E once: the LM head streams it as it is, the
 * self-conditioning contraction streams the same bytes and transposes them
 * in LDS, and the row gathers (embeddings, the exact top-token terms) read
 * single rows of it.  [P2] (local-deployment numbers) runs the model
 * quantised (NVFP4) to fit a consumer GPU; the MI355X counterparts kept here
 * are OCP fp8 e4m3 and block-scaled fp4 e2m1.
 * BF16: E_pack holds E in bf16, tiled (2 V d bytes).
 * FP8:  E_pack holds q = E * 2^table_exp as fp8 e4m3, one byte per value in
 *       the tiled order with 8-byte chunks (V d bytes; dg_pack_embedding
 *       rounds to nearest even and saturates at +-448).  The kernels turn
 *       each value back into bf16 as q * 2^-table_exp, exactly, so the
 *       arithmetic is that of the bf16 path on a table whose entries are
 *       those values: the model's table is E rounded to that grid
 *       (fp8(E * 2^table_exp) * 2^-table_exp).
 * FP4:  E_pack holds E as e2m1 codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 *       their negatives) with one power-of-two scale byte u per 32 x 32 block
 *       of E (value = code * 2^(u - 127), an E8M0 exponent as in the OCP
 *       microscaling formats, over a square block so that the 8 values a
 *       lane widens share one scale whether E is read along its rows or
 *       along its columns).  dg_pack_embedding sets u = floor(log2 of the
 *       block's largest magnitude) - 2 + 127, clamped to [2, 252] (127 for
 *       an all-zero block), and rounds each value divided by the scale to the
 *       nearest code (ties to the even code, saturated at 6; a value rounded
 *       to zero is +0).  table_exp must be 0.  As with FP8 the kernels widen
 *       each value to bf16 exactly: the model's table is E on that grid.
 *       E_pack is V d / 2 + V d / 1024 bytes (codes, then the scale bytes). */
typedef enum { DG_TABLE_BF16 = 0, DG_TABLE_FP8 = 1, DG_TABLE_FP4 = 2 } dg_table_format;

/* What the adaptive stop's stability counter counts ([P3] §5.3 adaptive
 * stop: the most likely token predictions unchanged over the last N steps;
 * [P5] scheduler: the predictions identical for N consecutive steps).
 * PREDICTIONS: consecutive steps whose predictions -- each position's most
 *   likely token (highest logit, lowest index on ties), whatever token the
 *   candidate rule places -- equal the previous step's at every position.
 *   A canvas's first step (step 0) and a step with any NaN entropy count as
 *   changed.
 * CANVAS: consecutive steps that left the canvas unchanged.  The two agree
 *   whenever every position is accepted with its argmax; under re-noise the
 *   canvas changes even when the predictions do not. */
typedef enum { DG_STABLE_PREDICTIONS = 0, DG_STABLE_CANVAS = 1 } dg_stable_rule;

/* Model and canvas shape.
 * Supported: 1 <= canvas_len <= 256; vocab a power of two in [256, 2^24];
 * n_q_heads a multiple of n_kv_heads.  DG_BF16 additionally needs head_dim ==
 * 128, d_model <= 4096 and d_model, ffn_hidden multiples of 64; DG_F32 needs
 * head_dim <= 128 and a multiple of 16 (its contractions and attention run on
 * the 16x16x4 fp32 matrix-core instruction). */
typedef struct {
  int32_t canvas_len;   /* N: tokens per canvas ([P1]: 256; [P5] table: 128) */
  int32_t vocab;        /* V */
  int32_t d_model;      /* d */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* Hkv (grouped-query attention when < Hq) */
  int32_t head_dim;     /* hd */
  int32_t ffn_hidden;   /* F: hidden width of the self-conditioning FFN */
  dg_dtype dtype;       /* storage/operand type of weights, cache, activations */
  float rms_eps;        /* RMSNorm epsilon (1e-6 in the shipped configurations) */
  float conf_eps;       /* adaptive-stop confidence threshold on entropy, nats
                           ([P3] §5.3: 0.005) */
  dg_accept_rule accept_rule;
  dg_candidate_rule candidate_rule;
  dg_sampler sampler;
  dg_table_format table_format;
  int32_t table_exp;    /* DG_TABLE_FP8: q = E * 2^table_exp, in [-32, 32]; 0 for DG_TABLE_FP4 */
  dg_stable_rule stable_rule;
} dg_config;

/* Weights (device, dtype of the config, caller-owned, read-only).
 * E [V][d] is the token-embedding table, tied to the LM head ([P3] §4.1):
 * DG_F32 reads it row-major (fp32) in every step; DG_BF16 reads only E_pack,
 * the one packed copy dg_pack_embedding() writes from it (tiled layout
 * below, in the form of table_format), so E may be null in the weights a
 * DG_BF16 step is given and its row-major copy freed once packed.
 * w_sc1 [F][d], w_sc2 [d][F]: self-conditioning FFN ([P3] §5.1).
 * wq [Hq*hd][d], wk/wv [Hkv*hd][d], wo [d][Hq*hd]: attention projections.
 * g_attn, g_final [d]: RMSNorm gains (pre-attention, pre-LM-head).
 * mask_emb [d]: the [MASK] token's embedding (id V), required (16-byte
 * aligned) by DG_SAMPLER_MASKED and ignored otherwise. */
typedef struct {
  const void *E, *E_pack, *w_sc1, *w_sc2, *wq, *wk, *wv, *wo, *g_attn, *g_final, *mask_emb;
} dg_weights;

/* Prefix KV cache ([P1]/[P4]: written causally by prefill, read by denoise).
 * k, v: device buffers of Hkv * capacity * hd * 4 bytes each.  DG_F32:
 * float32 [Hkv][capacity][hd].  DG_BF16: split pairs, bf16
 * [2][Hkv][capacity][hd]: the hi terms, then the lo terms, value =
 * hi + lo with hi = bf16(x) and lo = bf16(x - hi) (16 significant bits),
 * the form the attention kernel copies to the matrix cores unconverted;
 * a caller filling a cache itself writes that form.  Positions
 * [0, length) are valid.  dg_denoise_step never writes the cache
 * ([P3] §4.2); dg_prefill_append writes [length, length+n) and then
 * advances `length` (host field) by n. */
typedef struct {
  void *k, *v;
  int32_t length;
  int32_t capacity;
} dg_kv_cache;

/* Per-canvas state.  Device buffers are caller-owned:
 *   tokens  int32 [N]            current canvas
 *   probs   bytes dg_probs_bytes(): softmax probabilities of the last step,
 *                                the self-conditioning input of the next.
 *                                DG_F32: float [N][V].  DG_BF16: bf16
 *                                numerators in the tiled layout, each
 *                                relative to a power-of-two reference of
 *                                its (row, 64-column tile); the probability
 *                                is the stored value times the tile's
 *                                factor kept in stats (the dominant token's
 *                                exact probability is kept there too)
 *   stats   bytes dg_stats_bytes(): per-(row, tile) softmax statistics,
 *                                factors and exponents, per-row factors,
 *                                each row's dominant token with its exact
 *                                probability and the previous step's
 *                                predictions; opaque
 *   entropy float [N]            nats, clamped >= +0 (NaN propagates)
 *   argmax  int32 [N]            the candidate token of the last step: the
 *                                highest logit (lowest index on ties), or the
 *                                multinomial draw (candidate_rule)
 *   accept  uint8 [N]            1 = accepted in the last step
 *   status  int32 [DG_STATUS_WORDS]  see DG_ST_* below
 * Host fields: step (index of the next step), has_prev (the next step uses
 * self-conditioning), seed and canvas_id (Philox key and counter word). */
#define DG_STATUS_WORDS 16
enum {
  DG_ST_ALLCONF = 0,   /* every entropy < conf_eps */
  DG_ST_CHANGED = 1,   /* last step changed the canvas */
  DG_ST_STABLE = 2,    /* consecutive stable steps (stable_rule) */
  DG_ST_ACCEPTED = 3,  /* positions accepted in the last step */
  DG_ST_NAN = 4,       /* positions whose entropy was NaN */
  DG_ST_STEP = 5,      /* index of the last completed step */
  DG_ST_HMIN = 6,      /* float bits: min entropy */
  DG_ST_HMAX = 7,      /* float bits: max entropy */
  DG_ST_HMEAN = 8,     /* float bits: mean entropy */
  DG_ST_MASKED = 9,    /* [MASK] positions left (DG_SAMPLER_MASKED), else -1 */
  DG_ST_PRED_CHANGED = 10  /* 1: the predictions differ from the previous
                              step's (or step 0, or a NaN entropy), 0: same */
};
typedef struct {
  int32_t *tokens;
  void *probs;
  void *stats;
  float *entropy;
  int32_t *argmax;
  uint8_t *accept;
  int32_t *status;
  int32_t step;
  int32_t has_prev;
  uint64_t seed;
  uint32_t canvas_id;
} dg_canvas;

typedef struct {
  int32_t accepted;
  int32_t stable;
  int32_t allconf;
  int32_t changed;
  float h_min, h_mean, h_max;
  int32_t masked;      /* [MASK] positions left; -1 under DG_SAMPLER_UNIFORM */
} dg_step_stats;

/* ---- sizes and checks (host only, no device work) ---------------------- */
int32_t dg_abi_version(void);
const char *dg_status_string(dg_status s);
/* DG_OK if the configuration is supported; otherwise why not. */
dg_status dg_validate_config(const dg_config *cfg);
/* Workspace bytes for dg_denoise_step and for dg_prefill_append of up to
 * max_prefill_tokens tokens (0 if unsupported configuration). */
size_t dg_workspace_bytes(const dg_config *cfg, int32_t max_prefill_tokens);
/* Bytes of the canvas `stats` buffer (0 if unsupported configuration). */
size_t dg_stats_bytes(const dg_config *cfg);

/* ---- one-time preparation ----------------------------------------------- */
/* Tiled layout of a bf16 matrix X [R][K] (K a multiple of 32): blocks of 256
 * rows x 32 columns, 16 KB each, block (b, s) at index b * (K / 32) + s;
 * inside a block, 16-byte chunk p = 0..1023 holds the eight values
 * X[256 b + r][32 s + 8 c .. 32 s + 8 c + 7] with r = p / 4 and
 * c = (p % 4) ^ ((r / 4) % 4).  Rows past R up to a multiple of 256 are
 * padding.  This is the order in which the two table-streaming kernels stage
 * a 32-wide slice in LDS, so each of their copy instructions reads 1 KB of
 * consecutive memory. */

/* Bytes of dg_weights.E_pack (0 for DG_F32 or an unsupported config). */
size_t dg_embedding_pack_bytes(const dg_config *cfg);

/* Bytes of dg_canvas.probs (0 if unsupported). */
size_t dg_probs_bytes(const dg_config *cfg);

/* Writes E_pack (device, caller-allocated dg_embedding_pack_bytes(cfg)
 * bytes) from E (row-major bf16 [V][d]): E in the tiled layout.
 * DG_TABLE_BF16: a layout copy only, the same values as E; DG_TABLE_FP8 /
 * DG_TABLE_FP4: the rounded codes (and scale bytes) described at
 * dg_table_format.  Does nothing for DG_F32. */
dg_status dg_pack_embedding(const dg_config *cfg, const void *E, void *E_pack, void *stream);

/* [P3] §5.4 canvas initialisation: tokens[i] = the top log2(V) bits of word 0
 * of Philox4x32-10(key = seed, counter = (i, 0, canvas_id, 0)) -- uniform
 * vocabulary tokens; DG_SAMPLER_MASKED: tokens[i] = V ([MASK]) everywhere.
 * Resets status (stable = 0) and the host fields step = 0, has_prev = 0,
 * seed, canvas_id. */
dg_status dg_canvas_init(const dg_config *cfg, dg_canvas *canvas, uint64_t seed,
                         uint32_t canvas_id, void *stream);

/* ---- the hot path --------------------------------------------------------- */
/* Causal (incremental) prefill, [P1]/[P4] architecture and [P3] §5.2: for the
 * n_tokens device tokens at absolute positions length..length+n-1,
 *   x = E[t]; h = RMSNorm(x) * g_attn; K = h Wk^T, V = h Wv^T  -> cache
 * and, if attn_out (device, float32 [n][Hq*hd]) is non-NULL, the causal
 * attention output of the new tokens over keys [0, length+i].  No LM head.
 * Then cache->length += n_tokens (host field).
 * Errors: DG_ERR_CAPACITY if length + n_tokens > capacity; DG_ERR_WORKSPACE
 * if ws_bytes < dg_workspace_bytes(cfg, n_tokens); tokens must be in [0, V),
 * or [0, V] under DG_SAMPLER_MASKED where V is [MASK] (not checked on the
 * device: out-of-range ids are clamped into that range). */
dg_status dg_prefill_append(const dg_config *cfg, const dg_weights *w, dg_kv_cache *cache,
                            const int32_t *tokens, int32_t n_tokens, void *attn_out,
                            void *ws, size_t ws_bytes, void *stream);

/* One denoising step over the canvas ([P2] update loop; [P3] §4.1, §5.1-§5.4):
 *  1. h0 = E[c] (+ W2 GELU(W1 (p_prev E)) when has_prev: self-conditioning)
 *  2. bidirectional attention (no mask) of every canvas query over
 *     [cache 0..length) || canvas keys; h1 = h0 + O Wo^T
 *  3. z = RMSNorm(h1) E^T (tied head); y = z / temperature; p = softmax(y);
 *     entropy (nats) and the candidate token per position (`candidate_rule`:
 *     argmax, or the multinomial draw with Philox counter words 3 of
 *     2 + 4k and 3 + 4k); probs/stats keep p for the next step
 *  4. accept by `accept_rule` under `accept_threshold_nats`; accepted
 *     positions take the candidate token, every rejected one a fresh uniform
 *     token (Philox counter (i, step, canvas_id, 1)) -- or, under
 *     DG_SAMPLER_MASKED, only [MASK] positions are walked, rejected ones
 *     stay [MASK] and decided ones are kept; status flags updated, the
 *     stability counter by cfg->stable_rule (the predictions are kept in
 *     stats for the next step's comparison)
 * Then canvas->step += 1 and canvas->has_prev = 1 (host fields).
 * Errors: temperature must be finite and > 0; the threshold >= 0 and not NaN;
 * DG_ERR_WORKSPACE if ws_bytes < dg_workspace_bytes(cfg, 0). */
dg_status dg_denoise_step(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *cache,
                          dg_canvas *canvas, float temperature, float accept_threshold_nats,
                          void *ws, size_t ws_bytes, void *stream);

/* dg_denoise_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, semantics and kernels as dg_denoise_step,
 * minus the workspace: the step's scratch is a device array inside the
 * library, DG_STATIC_SCRATCH_BYTES (160 MiB) on every device the library
 * is loaded on, held until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or event creation; the profiling switch and the
 * logits dump do not apply to it).  The device current on the calling
 * thread must be the device of `stream`; its array's address is looked up
 * once per device, on the device's first call.
 * Every call on one device shares that device's array, whose contents are
 * whatever the last call left (the step needs none of it cleared): calls
 * that overlap on one device -- other streams, other host threads -- race
 * and must be ordered by the caller.
 * Errors: as dg_denoise_step; DG_ERR_WORKSPACE when the configuration's
 * dg_workspace_bytes(cfg, 0) exceeds DG_STATIC_SCRATCH_BYTES (checked
 * before anything else runs); DG_ERR_HIP if the array's address cannot be
 * obtained. */
#define DG_STATIC_SCRATCH_BYTES ((size_t)160 << 20)
dg_status dg_denoise_step_static(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *cache,
                                 dg_canvas *canvas, float temperature, float accept_threshold_nats,
                                 void *stream);

/* Batched canvases.  [P5] (current limitations) notes that several users
 * cannot share one denoising pass the way autoregressive decoding shares a
 * batch: each user's canvas runs its own loop.  This call steps n_canvases
 * such canvases (each with its own cache, tokens, probabilities, seed and
 * step counter) at once: their rows are stacked for the projections and the
 * two table-streaming contractions, so the embedding table is read from HBM
 * about once per step for the whole batch instead of once per canvas
 * (DG_BF16; canvases of at most 128 rows share 256-row blocks two by two).
 * Attention runs per canvas over that canvas's own cache; the row
 * statistics and the selection are per canvas, each computed by one launch
 * for the batch.  Every canvas ends in exactly the state dg_denoise_step
 * would give it (bit for bit), so a batch may mix canvases at different
 * steps of their own schedules, with one temperature and threshold for the
 * call.  DG_F32 runs the single-canvas step for each canvas in turn.
 *   caches:   host array of n_canvases cache descriptors (device K/V as for
 *             dg_denoise_step; several may name the same cache: it is only
 *             read);
 *   canvases: host array of n_canvases canvases, all with the same has_prev
 *             (all past their first step, or none); no two may share any
 *             device buffer (tokens, probs, stats, entropy, argmax, accept,
 *             status);
 *   ws:       device workspace of at least dg_workspace_bytes_batch(cfg,
 *             n_canvases) bytes (0 for an unsupported config or count);
 *   1 <= n_canvases <= DG_MAX_BATCH.
 * Each canvas's step += 1 and has_prev = 1 (host fields of the array).
 * Errors as dg_denoise_step, checked for every canvas before the first
 * launch; DG_ERR_INVALID_ARG also for a count out of range, mixed has_prev
 * or shared canvas buffers.  The test switch dg_test_set_logits_dump does
 * not apply to this call. */
#define DG_MAX_BATCH 16
size_t dg_workspace_bytes_batch(const dg_config *cfg, int32_t n_canvases);
dg_status dg_denoise_step_batch(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *caches,
                                dg_canvas *canvases, int32_t n_canvases, float temperature,
                                float accept_threshold_nats, void *ws, size_t ws_bytes, void *stream);

/* Adaptive stop, [P3] §5.3 and [P5] scheduler: stop when every entropy is
 * below conf_eps, or when the stability counter (the predictions, or the
 * canvas, unchanged: cfg->stable_rule) has reached stable_steps
 * (stable_steps <= 0 disables the stability test), or, under
 * DG_SAMPLER_MASKED, when no [MASK] is left ([P3] §3.1).
 * Synchronises `stream`, then writes *stop_host (0/1) and, if non-NULL,
 * *stats_host.  This is the only device-to-host transfer of a step. */
dg_status dg_should_stop(const dg_config *cfg, const dg_canvas *canvas, int32_t stable_steps,
                         int32_t *stop_host, dg_step_stats *stats_host, void *stream);

/* The denoising loop of one canvas ([P3] §5.4, the [P5] scheduler): the
 * canvas is initialised as by dg_canvas_init(seed, canvas_id), then steps
 * s = 0, 1, ... run as dg_denoise_step at temperature temps[s] (host array
 * of max_steps values, the caller's schedule) and accept threshold
 * accept_threshold_nats.  With adaptive_stop != 0 each step is followed by
 * the dg_should_stop test (stable_steps as there) and the loop ends at the
 * first step where it holds.  The step's selection kernel writes its status
 * words straight into coherent pinned host memory the library keeps per host
 * thread (the step word last, after a system-scope fence), and the host polls
 * that word: no copy, no event.  The poll checks the stream every few
 * thousand reads, so a stream that ends or fails without writing the word
 * returns DG_ERR_HIP instead of waiting forever.
 * Writes *steps_run and *stopped (1 if the adaptive stop ended the loop).
 * Errors as dg_denoise_step, checked before the first launch; max_steps >= 0.
 * Returns with the stream synchronised when adaptive_stop != 0, otherwise
 * with the steps enqueued.  With adaptive_stop (DG_BF16) the next step's
 * self-conditioning contraction is enqueued before the host reads a step's
 * status, guarded on the device by those status words; it writes only the
 * workspace, and does nothing when the step stopped the canvas. */
dg_status dg_run_canvas(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *cache,
                        dg_canvas *canvas, uint64_t seed, uint32_t canvas_id, const float *temps,
                        int32_t max_steps, float accept_threshold_nats, int32_t adaptive_stop,
                        int32_t stable_steps, void *ws, size_t ws_bytes, void *stream,
                        int32_t *steps_run, int32_t *stopped);

/* ---- test and measurement exports -------------------------------------------
 * Not part of the generation path; they expose single kernels for parity
 * tests and timing.  Same validation rules as above. */

/* Byte offsets inside the workspace of the step's intermediates, all f32:
 * h0 [N][d], attn [N][Hq*hd], h1 [N][d], selfcond [N][d] (p_prev E),
 * logits [N][V] (the LM head's fp32 accumulators; bf16 configurations
 * write them only when dg_test_set_logits_dump(1)). */
typedef struct {
  size_t h0, attn, h1, selfcond, logits;
} dg_ws_offsets;
dg_status dg_test_ws_offsets(const dg_config *cfg, dg_ws_offsets *out);
/* 1: dg_denoise_step also writes the fp32 logits z into the workspace (the
 * workspace must then be dg_test_logits_ws_bytes() large).  Global switch. */
void dg_test_set_logits_dump(int32_t on);
size_t dg_test_logits_ws_bytes(const dg_config *cfg);

/* Self-conditioning contraction alone ([P3] §5.1): S (f32 [N][d]) = P E,
 * with P given as plain probabilities in the layout of dg_canvas.probs
 * (DG_BF16: tiled bf16 [N][V]; DG_F32: float [N][V]), run by the kernels
 * dg_denoise_step runs, with every tile exponent 0, row factor 1 and no
 * dominant-token correction.  ws: at least dg_test_logits_ws_bytes() bytes
 * (the zero exponents are written there). */
dg_status dg_test_selfcond(const dg_config *cfg, const dg_weights *w, const void *P, void *S,
                           void *ws, size_t ws_bytes, void *stream);
/* The self-conditioning vector S (f32 [N][d], device) = p E of the canvas's
 * kept state (its last step's probabilities: numerators, tile exponents,
 * row factors and the dominant token's exact probability), computed exactly
 * as the canvas's next dg_denoise_step computes it ([P3] §5.1).
 * ws: at least dg_workspace_bytes(cfg, 0) bytes. */
dg_status dg_test_selfcond_canvas(const dg_config *cfg, const dg_weights *w, const dg_canvas *canvas, void *S,
                                  void *ws, size_t ws_bytes, void *stream);
/* Selection kernel alone on given entropies/argmax/tokens (device):
 * writes tokens (in place), accept and status exactly as dg_denoise_step. */
dg_status dg_test_select(const dg_config *cfg, dg_canvas *canvas, float accept_threshold_nats,
                         void *stream);
/* Philox4x32-10 on the device: out[4*i .. 4*i+3] for counters ctr[4*i..]
 * and key (k0, k1); n counters; all device pointers. */
dg_status dg_test_philox(const uint32_t *ctr, uint32_t k0, uint32_t k1, uint32_t *out, int32_t n,
                         void *stream);
/* The multinomial draw's single-precision pieces on the device, for n
 * device words w: mode 0 writes out[i] = ln of the float whose bits are
 * w[i] (positive normal floats), mode 1 the Gumbel variable of word w[i]
 * (see DG_CANDIDATE_MULTINOMIAL); out is device float [n]. */
dg_status dg_test_gumbel(const uint32_t *w, int32_t n, int32_t mode, float *out, void *stream);
/* Plain device copy of `bytes` bytes (multiple of 16) used to calibrate
 * memory-traffic counters. */
dg_status dg_test_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Timing of the kernels inside dg_denoise_step: HIP events are recorded on
 * the step's stream around the LM-head kernel (mask bit 0) and the
 * self-conditioning contraction (mask bit 1); 0 stops recording.  Each pair
 * of records adds a marker to the stream, so a timed run records only the
 * kernels it needs.  dg_profile_read synchronises on the last recorded
 * events and returns the summed milliseconds and launch counts. */
void dg_profile_enable(int32_t mask);
dg_status dg_profile_read(float *lm_head_ms, int32_t *lm_head_count, float *selfcond_ms,
                          int32_t *selfcond_count);

#ifdef __cplusplus
}
#endif
#endif /* DGDENOISE_H */
