// dg_kernels.h -- host-side launchers of the libdgdenoise kernels.  Every
// launcher enqueues on `s` and returns the launch status; shapes have been
// validated by the caller (dg_api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "dgdenoise.h"
#include "dg_tiled.h"

namespace dg {

typedef uint16_t bf16;  // raw bfloat16 bits

// One-time per-device set-up of a launcher (raising a kernel's dynamic LDS
// limit): `done` keeps one bit per device; set_up() is idempotent, so two
// host threads that race on the first launch both run it, harmlessly.
template <typename F>
hipError_t once_per_device(std::atomic<uint64_t> &done, F &&set_up) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = uint64_t(1) << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  const hipError_t err = set_up();
  if (err == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return err;
}

// Epilogue of the dense GEMMs: how an output element (row, col) is stored.
//   index(row, col) = row * rstride + (col / cdiv) * chi + (col % cdiv)
// which covers plain row-major outputs (cdiv >= N) and the head-split
// layouts of Q/K/V ([head][row][hd]: cdiv = hd, chi = head stride).
// A bf16 output with lo_off != 0 is a split pair: hi = bf16(v) at the index,
// lo = bf16(v - hi) at index + lo_off (the operand format of SplitGemm).
// EPI_ADD_ROW: out = acc + E[tok[row]][col] (rows of the packed table gtab,
// token ids clamped to [0, gV)): a residual gathered on the fly; with gmask
// (the [MASK] row of the masked sampler, bf16) ids >= gV read gmask.
enum EpiKind { EPI_STORE = 0, EPI_GELU = 1, EPI_ADD = 2, EPI_ADD_ROW = 3 };
struct Epi {
  int kind;
  void *out;
  int out_f32;           // 1: float output, 0: bf16 output
  int64_t rstride;
  int cdiv;
  int64_t chi;
  const float *resid;    // EPI_ADD: out = resid + acc (f32, same index)
  int64_t lo_off;        // bf16 output: offset of the lo term (0: plain bf16)
  PackedTable gtab;  // EPI_ADD_ROW
  const int32_t *gtok;
  int gV;
  const uint16_t *gmask;  // EPI_ADD_ROW: row of token ids >= gV (nullable)
};

// fp32 activation x bf16 weight GEMM on the bf16 MFMA.  The activation
// comes as a split pair (two bf16 terms a = hi + lo, hi = bf16(a),
// lo = bf16(a - hi), written by the kernel that produced it): hi at
// A[m * lda + k], lo at A[lo_off + m * lda + k].  C_seg[M][N_seg] =
// A[M][K] B_seg[N_seg][K]^T for up to three weight matrices sharing A;
// K % 32 == 0.  With ksplit > 1 the K range is split over workgroups whose
// fp32 partials ([seg][ksplit][M][N_seg] in `part`) are summed by a second
// kernel that applies the epilogue.
struct SplitGemm {
  const uint16_t *A;
  int64_t lda, lo_off;
  int M, K;
  const void *B[3];
  int N[3];
  Epi e[3];
  int count;
  float *part;
  int ksplit;
};
// K-split the planner picks for a weight shape (K, N[0..count)) and rows_ref,
// the configuration's canvas length: the same for every launch of one
// configuration (single or batched step, prefill of any length), never a
// launch's own row count.
int gemm_split_plan(int rows_ref, int K, const int *N, int count);
// Bytes of partials gemm_split needs for that plan at M rows (0 when ksplit == 1).
size_t gemm_split_part_bytes(int M, int rows_ref, int K, const int *N, int count);
hipError_t gemm_split(const SplitGemm &g, hipStream_t s);
// RMSNorm of a projection's output rows, fused into its split-K merge:
// y = epilogue(sum of partials) (EPI_STORE, EPI_ADD or EPI_ADD_ROW, fp32,
// row-major),
// then out = y / sqrt(mean(y^2) + eps) * gain (fp32 [M][N], nullable) and
// out_tiled (bf16 tiled block(s), rows past M zero; nullable) and out_split
// (split pair [M][N], lo term at + M * N; nullable).  One segment; with
// ksplit == 1 it runs the GEMM and a separate RMSNorm.
struct RowNorm {
  const uint16_t *gain;  // bf16 [N]
  float eps;
  float *out;
  uint16_t *out_tiled;
  uint16_t *out_split;
};
hipError_t gemm_split_norm(const SplitGemm &g, const RowNorm &rn, hipStream_t s);
// Canvas rows per workgroup of the two table-streaming kernels (128 or 256).
int estream_bm(int M);
// The self-conditioning contraction (selfcond_bf16_batch below): A = probs
// (tiled bf16), B = the packed table E read transposed, K = V split in
// ksplit ranges.  shift (uint8 [K/64][256]): A's value at (row, k) is the
// stored bf16 times 2^-shift[k / 64][row], applied exactly on the exponent
// field.
// The f32 partials are stored in register order, one 256 x 256 block per
// (operand block b, K range kc, column tile nt) at float offset
// ((b * ksplit + kc) * ceil(N / 256) + nt) * 65536; inside it the float4
// at slot s = (((w * 2 + i) * 4 + j) * 4 + q) * 64 + l holds block row
// 64 (w / 2) + 32 i + l % 32 and columns 256 nt + 128 (w % 2) + 32 j +
// 8 q + 4 (l / 32) .. + 3 (so one store instruction writes 1 KB).  Operand
// block b is canvas b, or (selfcond_paired) canvases 2b (rows 0..127) and
// 2b + 1 (rows 128..255).  Slots of rows or columns past the canvas are not
// written.
inline bool selfcond_paired(int B, int M) { return B > 1 && 2 * M <= 256; }
inline int selfcond_blocks(int B, int M) { return selfcond_paired(B, M) ? (B + 1) / 2 : B; }
inline size_t selfcond_part_bytes(int B, int M, int N, int ksplit) {
  return (size_t)selfcond_blocks(B, M) * ksplit * ((N + 255) / 256) * 65536 * 4;
}
// guard: a launch made before the host knows whether the canvas loop stops
// after the previous step; every workgroup returns at once when the status
// words (written by that step's selection) say stop.
struct SelfcondGuard {
  const int32_t *status;  // null: unconditional
  int stable_steps;
  __device__ bool stopped() const {
    if (!status) return false;
    return status[DG_ST_ALLCONF] != 0 || (stable_steps > 0 && status[DG_ST_STABLE] >= stable_steps) ||
           status[DG_ST_MASKED] == 0;
  }
};
// fp32 GEMM on the fp32 MFMA: C[m][n] = sum_k A[m*sam + k*sak] * B[n*sbn + k*sbk].
struct GemmShapeF32 {
  const float *A;
  int64_t sam, sak;
  const float *B;
  int64_t sbn, sbk;
  int M, N, K;
  const float *a_scale;
  int64_t a_scale_ld;
};
hipError_t gemm_f32(const GemmShapeF32 &g, const Epi &e, hipStream_t s);

// Tied LM head + temperature softmax statistics (bf16 operands): for each
// row and 64-column tile t of z = A E^T: zmax_t, argmax_t, and with
// y = z * inv_T, m_t = zmax_t * inv_T: l_t = sum exp(y - m_t),
// s_t = sum exp(y - m_t) (y - m_t); probs = bf16(exp(y - m_t) f_t) with
// f_t = 2^(m_t log2e - r_t), r_t = ceil(m_t log2e): numerators relative to
// a power-of-two reference 2^r_t.
// tile_stats: float4 [M][V/64] = (zmax, l, s, argmax as int bits).
// A batch of B canvases of N rows each (B * N rows stacked in A_tiled, row r
// = row r % N of canvas r / N; the normalised rows, tiled): canvas c's
// numerators (tiled [N][V]) and statistics go to cv.probs[c] and
// cv.tile_stats[c].  Each row's results are those of the single-canvas
// launch bit for bit.  tab: the packed table E [V][K] (tab.d == K).
constexpr int ES_MAX_BATCH = DG_MAX_BATCH;
struct EsCanvases {
  uint16_t *probs[ES_MAX_BATCH];
  float4 *tile_stats[ES_MAX_BATCH];
};
hipError_t lm_head_bf16_batch(const uint16_t *A_tiled, int B, int N, int K, const PackedTable &tab, int V,
                              float inv_T, const EsCanvases &cv, float *logits_dump, hipStream_t s);
// The self-conditioning contraction S = P E of B canvases at once, K = V:
// canvas c's operand cin.probs[c] (its exponents cin.shift[c] when scaled),
// partials at partials + c * ksplit * M * N (the single-canvas layout per
// canvas).  tab: the same packed table E [K][N] the LM head reads
// (tab.d == N), transposed in LDS.  Canvases of M <= 128 rows are paired in
// one 256-row block (the second canvas's rows read from its own buffers).
// Each row's partials are those of the single-canvas launch bit for bit
// (same K ranges, same MFMA order).
struct EsCanvasesIn {
  const uint16_t *probs[ES_MAX_BATCH];
  const uint8_t *shift[ES_MAX_BATCH];
};
hipError_t selfcond_bf16_batch(const EsCanvasesIn &cin, int B, const PackedTable &tab, int M, int N, int K,
                               bool scaled, float *partials, int ksplit, hipStream_t s,
                               SelfcondGuard guard = SelfcondGuard{nullptr, 0});
// Same statistics from fp32 logits already in memory (fp32 path).
hipError_t tile_stats_f32(const float *logits, int M, int V, float inv_T, float *probs,
                          float4 *tile_stats, hipStream_t s);
// Multinomial draw of one step: the canvas's Philox key and counter words,
// and the stored weights the second level reads (one of the two pointers).
struct DrawArgs {
  uint64_t seed;
  uint32_t step, canvas;
  const uint16_t *num_tiled;  // bf16 path: numerators in the tiled layout [256][V]
  const float *num_f32;       // fp32 path: the normalised probabilities, row-major [M][V]
};
// Row combine: entropy (nats), argmax, and the factors that turn the stored
// numerators into probabilities.  shift == nullptr (numerators exp(y - m_t)):
// tile_scale[row][t] = exp(m_t - M_row) / L_row.  shift given (numerators
// relative to 2^r_t, M <= 256): p = stored * 2^-shift[t][row] * row_scale[row]
// and tile_scale (nullable) = 2^-shift * row_scale.  With n2 (fp32 [M][d],
// d <= 4096, the packed table E [V][d]) given, the argmax token's logit is
// recomputed exactly and top[row] = (argmax as int bits, its exact
// probability).  cand receives the argmax (the candidate token unless a
// multinomial draw follows).
hipError_t row_combine(const float4 *tile_stats, int M, int ntiles, float inv_T, float *entropy,
                       int32_t *cand, float *tile_scale, float *row_scale, uint8_t *shift, const float *n2,
                       const PackedTable &E, float2 *top, hipStream_t s);
// The row combine of B canvases (bf16 path, N <= 256 rows each) in one
// launch: canvas c's statistics, entropy, candidates, row factors, exponents
// and top tokens at the c-th pointers; n2 the stacked normalised rows
// ([B * N][d]).  The single-canvas step launches it with B = 1, so a row's
// results do not depend on the batch it is in.
struct RowCombineBatch {
  const float4 *stats[ES_MAX_BATCH];
  float *entropy[ES_MAX_BATCH];
  int32_t *cand[ES_MAX_BATCH];
  float *row_scale[ES_MAX_BATCH];
  uint8_t *shift[ES_MAX_BATCH];
  float2 *top[ES_MAX_BATCH];
};
hipError_t row_combine_batch(const RowCombineBatch &bt, int B, int N, int ntiles, float inv_T, const float *n2,
                             const PackedTable &E, hipStream_t s);
// Multinomial draw of the candidate tokens (two Gumbel-max levels over the
// tile statistics and the stored weights, dg_device.h), run once the step's
// probabilities are final; cand holds the argmax and keeps it for a row with
// nothing drawable.  Exactly one of draw.num_tiled / draw.num_f32 is set.
hipError_t multinomial_draw(const float4 *tile_stats, int M, int ntiles, float inv_T, const DrawArgs &draw,
                            int32_t *cand, hipStream_t s);
// Test export: out[i] = ln_fixed(bits of w[i]) (mode 0) or gumbel_word(w[i])
// (mode 1), the multinomial draw's single-precision pieces.
hipError_t gumbel_test(const uint32_t *w, int n, int mode, float *out, hipStream_t s);

// Attention over two key segments [A: nA keys][B: nB keys] per KV head, all
// fp32 in memory.  q: [Hq][nq][hd] (heads q_hstride apart); k/v segment X: base + (g * capX + j) * hd.
// out: fp32 [nq][Hq*hd].  causal: query i may read keys <= q_pos0 + i.
struct AttnArgs {
  const void *q;
  int nq, Hq, Hkv, hd;
  const void *kA, *vA;
  int nA, capA;
  const void *kB, *vB;
  int nB, capB;
  int causal, q_pos0;
  void *out;
  uint16_t *out_split;  // nullable: also the split pair of out (lo term at + nq * Hq * hd)
  int64_t q_hstride;   // elements between q's heads (0: nq * hd)
  int64_t out_lo_off;  // offset of out_split's lo terms (0: nq * Hq * hd)
  float *part_o;   // workspace [splits][Hq][nq][hd]
  float *part_ml;  // workspace [splits][Hq][nq][2]
  int splits, keys_per_split;
};
// head_dim 128 on the MFMA (split-bf16 products), split-KV + merge
hipError_t attention_mfma(const AttnArgs &a, hipStream_t s);
// Several canvases' attention in one split launch and one merge launch:
// canvas c (same nq, Hq, Hkv for all) with its own buffers, partials and
// split plan, its splits at grid z-slices zbase[c] .. zbase[c + 1] - 1.  A
// single canvas is a batch of one, so each canvas's results are those of
// its own launch bit for bit.
struct AttnBatch {
  AttnArgs c[DG_MAX_BATCH];
  int zbase[DG_MAX_BATCH + 1];
  int B;
};
hipError_t attention_mfma_batch(const AttnBatch &bt, hipStream_t s);
// fp32 path (head_dim <= 128, a multiple of 16) on the fp32 MFMA
hipError_t attention_f32(const AttnArgs &a, hipStream_t s);
void attention_plan(int nq, int Hq, int nk, int *splits, int *keys_per_split);

// Small ops.
// out[i] = E[tokens[i]] (fp32 [n][d]); ids clamped to [0, V), except that with
// mask_row (the [MASK] embedding, id V, masked sampler) ids >= V read mask_row.
// The fp32 path's row-major table, and the packed table of the bf16 path
// (mask_row bf16, 8-byte aligned; d % 4 == 0).
hipError_t gather_rows(const float *E, const int32_t *tokens, int n, int d, int V, const float *mask_row,
                       float *out, hipStream_t s);
hipError_t gather_rows(const PackedTable &E, const int32_t *tokens, int n, int V, const uint16_t *mask_row,
                       float *out, hipStream_t s);
// out (fp32 [n][d], nullable), out_tiled (bf16, tiled block(s) of the
// rows, the rows past n up to the block end written as zeros; nullable)
// and/or out_split (split pair [n][d], lo term at + n * d; nullable).
template <typename T>
hipError_t rmsnorm_rows(const float *x, const T *g, int n, int d, float eps, float *out, bf16 *out_tiled,
                        bf16 *out_split, hipStream_t s);
// S (fp32 [N][d]) = row_scale[row] (1 when null) * the sum of the ksplit
// partials (the contraction's register-order blocks) + exact correction of each row's dominant token (top = (token
// bits, exact p); nullable): the contraction used the value of probs
// (tiled) at (row, a), scaled by 2^-shift of a's tile when shift is given,
// times row_scale.  out_split (nullable): S also as a split pair [N][d], lo
// term at + lo_off (0: + N * d).
hipError_t selfcond_reduce(const float *part, int ksplit, int N, int d, const float2 *top,
                           const uint16_t *probs_tiled, int V, const float *row_scale, const uint8_t *shift,
                           const PackedTable &E, float *out, uint16_t *out_split, hipStream_t s,
                           int64_t lo_off = 0);
// The same for B canvases in one launch (the partials of the batched
// contraction): canvas c's rows of out / out_split at c * N * d (lo terms
// at + lo_off, 0: + B * N * d), its state at the c-th pointers.
struct ReduceBatch {
  const float2 *top[DG_MAX_BATCH];
  const uint16_t *probs[DG_MAX_BATCH];
  const float *row_scale[DG_MAX_BATCH];
  const uint8_t *shift[DG_MAX_BATCH];
};
hipError_t selfcond_reduce_batch(const float *part, int ksplit, int B, int N, int d, const ReduceBatch &rb, int V,
                                 const PackedTable &E, float *out, uint16_t *out_split, hipStream_t s,
                                 int64_t lo_off = 0);
// The token ids of B canvases (src.p[c], N each) copied into one array
// out[B * N], canvas after canvas.
struct TokenPtrs {
  const int32_t *p[ES_MAX_BATCH];
};
hipError_t stack_tokens(const TokenPtrs &src, int B, int N, int32_t *out, hipStream_t s);
// In place (fp32 path): p(row, v) *= tile_scale[row][v / 64], numerators ->
// probabilities; row-major [N][V].
hipError_t normalize_probs_f32(float *probs, const float *tile_scale, int N, int V, hipStream_t s);
// out[c * ld_out + r] = in[r * cols + c]
template <typename T>
hipError_t transpose(const T *in, int rows, int cols, T *out, int64_t ld_out, hipStream_t s);
// Tiled copy of a row-major bf16 matrix X [R][K] (leading dimension ldx):
// out = the tiled layout of dg_tiled.h, rows past R zero-filled.
hipError_t tile_rows(const uint16_t *X, int R, int K, int64_t ldx, uint16_t *out, hipStream_t s);
hipError_t copy_bytes(const void *src, void *dst, size_t bytes, hipStream_t s);
// fp8 e4m3 copy in the 8-byte-chunk tiled layout (dg_tiled.h) of Y = X
// (X [R][K]) or Y = X^T (trans: X [K][R]), leading dimension ldx: each value
// times scale, clamped to +-448, rounded to nearest even; rows past R zero.
hipError_t tile_fp8(const uint16_t *X, int R, int K, int64_t ldx, bool trans, float scale, uint8_t *out,
                    hipStream_t s);
// fp4 e2m1 copy in the 4-byte-chunk tiled layout (dg_tiled.h) of Y = X or
// Y = X^T as for tile_fp8, with the scale bytes of its 32 x 32 blocks: per
// block u = clamp(floor(log2 amax) - 2 + 127, 2, 252) (127 for an all-zero
// block), codes = y * 2^(127 - u) rounded to the nearest e2m1 value (ties
// to the even code, saturated at +-6; a code rounded to zero is +0); rows
// past R are zero codes with scale byte 127.
hipError_t tile_fp4(const uint16_t *X, int R, int K, int64_t ldx, bool trans, uint8_t *codes, uint8_t *scales,
                    hipStream_t s);

// Selection and canvas.  mask_id >= 0: the masked sampler (the canvas starts
// as mask_id; only positions holding it are walked; rejected ones keep it,
// decided ones are locked); mask_id < 0: uniform-state re-noise.
hipError_t canvas_init(int32_t *tokens, int32_t *status, int N, int log2v, uint64_t seed,
                       uint32_t canvas_id, int mask_id, hipStream_t s);
// The selection of B canvases (N <= 256 each) in one launch, one workgroup
// per canvas, each with its own buffers, seed, canvas id and step; a single
// canvas is a batch of one.
struct SelectBatch {
  const float *entropy[ES_MAX_BATCH];
  const int32_t *argmax[ES_MAX_BATCH];
  int32_t *tokens[ES_MAX_BATCH];
  uint8_t *accept[ES_MAX_BATCH];
  int32_t *status[ES_MAX_BATCH];
  uint64_t seed[ES_MAX_BATCH];
  uint32_t canvas_id[ES_MAX_BATCH];
  uint32_t step[ES_MAX_BATCH];
  // nullable: a copy of the status words in host-visible memory, the step
  // word written last (after a system-scope fence)
  int32_t *host_status[ES_MAX_BATCH];
  // the step's predictions (the row combine's top tokens, as int bits of
  // .x) and the previous step's, which the kernel replaces (int32 [N])
  const float2 *pred[ES_MAX_BATCH];
  int32_t *pred_prev[ES_MAX_BATCH];
};
// stable_rule: dg_stable_rule (what DG_ST_STABLE counts).
hipError_t select_step_batch(const SelectBatch &bt, int B, int N, int log2v, double gamma, int rule,
                             float conf_eps, int mask_id, int stable_rule, hipStream_t s);
hipError_t philox_test(const uint32_t *ctr, uint32_t k0, uint32_t k1, uint32_t *out, int n,
                       hipStream_t s);

}  // namespace dg
