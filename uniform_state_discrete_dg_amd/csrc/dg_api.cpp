// dg_api.cpp -- the C ABI of libdgdenoise (declared in include/dgdenoise.h):
// host-side validation, workspace carving and the launch sequence of one
// denoising step / one prefill append.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "dg_kernels.h"
#include "dg_tiled.h"
#include "dgdenoise.h"

using dg::bf16;

namespace {

constexpr int kTile = 64;  // vocabulary columns per softmax-statistics tile

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int64_t v) {
  int b = 0;
  while ((int64_t(1) << b) < v) ++b;
  return b;
}
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
size_t dsize(const dg_config *c) { return c->dtype == DG_BF16 ? 2 : 4; }

// The integer a caller stored in an enum-typed field of the ABI.  A C caller
// may store any int there; reading it through the enum type would be
// undefined for values outside the enum's range, so the bytes are copied.
template <typename E>
int32_t enum_value(const E &e) {
  static_assert(sizeof(E) == sizeof(int32_t), "ABI enums are 32-bit");
  int32_t v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}
bool in_range(int32_t v, int32_t lo, int32_t hi) { return v >= lo && v <= hi; }

dg_status check_config(const dg_config *c) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (!in_range(enum_value(c->dtype), DG_F32, DG_BF16) ||
      !in_range(enum_value(c->accept_rule), DG_ACCEPT_SUM_MINUS_MAX, DG_ACCEPT_CUMSUM) ||
      !in_range(enum_value(c->candidate_rule), DG_CANDIDATE_ARGMAX, DG_CANDIDATE_MULTINOMIAL) ||
      !in_range(enum_value(c->sampler), DG_SAMPLER_UNIFORM, DG_SAMPLER_MASKED) ||
      !in_range(enum_value(c->table_format), DG_TABLE_BF16, DG_TABLE_FP4) ||
      !in_range(enum_value(c->stable_rule), DG_STABLE_PREDICTIONS, DG_STABLE_CANVAS))
    return DG_ERR_INVALID_ARG;
  if (c->table_format == DG_TABLE_FP8 && (c->table_exp < -32 || c->table_exp > 32)) return DG_ERR_INVALID_ARG;
  if (c->table_format == DG_TABLE_FP4 && c->table_exp != 0) return DG_ERR_INVALID_ARG;  // scales are per block
  if (c->canvas_len < 1 || c->vocab < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 1 || c->ffn_hidden < 1)
    return DG_ERR_INVALID_ARG;
  if (!(std::isfinite(c->rms_eps) && c->rms_eps >= 0.f) || !std::isfinite(c->conf_eps))
    return DG_ERR_INVALID_ARG;
  if (c->canvas_len > 256) return DG_ERR_UNSUPPORTED;
  if (!is_pow2(c->vocab) || c->vocab < 256 || c->vocab > (1 << 24)) return DG_ERR_UNSUPPORTED;
  if (c->n_q_heads % c->n_kv_heads != 0) return DG_ERR_UNSUPPORTED;
  if (c->dtype == DG_BF16) {
    if (c->head_dim != 128 || c->d_model % 64 != 0 || c->ffn_hidden % 64 != 0 || c->d_model > 4096)
      return DG_ERR_UNSUPPORTED;
  } else {
    if (c->head_dim > 128 || c->head_dim % 16) return DG_ERR_UNSUPPORTED;  // fp32 MFMA tiles of 16
  }
  return DG_OK;
}

// Self-conditioning split of K = V over workgroups (bf16 path): about one
// work item per CU.
// The packed table (DG_BF16): E [V][d] once, tiled, in the configured
// form; both contractions and every row gather read it.
size_t pack_elems(const dg_config *c) { return dg::tl_elems(c->vocab, c->d_model); }
bool table_fp8(const dg_config *c) { return c->dtype == DG_BF16 && c->table_format == DG_TABLE_FP8; }
bool table_fp4(const dg_config *c) { return c->dtype == DG_BF16 && c->table_format == DG_TABLE_FP4; }
// fp4: the codes (half a byte per element), then the blocks' scale bytes
// (one per 1024 elements)
size_t pack4_codes(const dg_config *c) { return pack_elems(c) / 2; }
size_t pack4_scales(const dg_config *c) { return pack_elems(c) / 1024; }

dg::PackedTable packed_table(const dg_config *c, const dg_weights *w) {
  const uint8_t *p8 = static_cast<const uint8_t *>(w->E_pack);
  if (table_fp8(c)) return {dg::TF_FP8, p8, nullptr, std::ldexp(1.f, -c->table_exp), c->d_model};
  if (table_fp4(c)) return {dg::TF_FP4, p8, p8 + pack4_codes(c), 1.f, c->d_model};
  return {dg::TF_BF16, p8, nullptr, 1.f, c->d_model};
}

int selfcond_ksplit(const dg_config *c) {
  const int bm = dg::estream_bm(c->canvas_len);
  const int ntile = (c->d_model + 255) / 256 * ((c->canvas_len + bm - 1) / bm);
  int ks = 256 / ntile;
  if (ks < 1) ks = 1;
  const int slices = c->vocab / 64;
  if (ks > slices) ks = slices;
  return ks;
}

// The canvas `stats` buffer: float4 tile statistics [N][V/64], float
// tile_scale [N][V/64], float2 top [N], float row_scale [N], int32 pred [N]
// (the last step's predictions, for the stability test), then (256-byte
// aligned) the uint8 tile exponents [V/64][256].
struct StatsLayout {
  size_t tstats, tscale, top, rscale, pred, shift, total;
};
StatsLayout stats_layout(const dg_config *c) {
  StatsLayout S{};
  const size_t N = c->canvas_len, nt = (size_t)c->vocab / kTile;
  S.tstats = 0;
  S.tscale = N * nt * sizeof(float4);
  S.top = S.tscale + N * nt * sizeof(float);
  S.rscale = S.top + N * sizeof(float2);
  S.pred = S.rscale + N * sizeof(float);
  S.shift = align256(S.pred + N * sizeof(int32_t));
  S.total = S.shift + nt * 256;
  return S;
}

struct Layout {
  size_t h0, h1, nrm, nrm16, nrm_s, sc, sc_s, g, q, kc, vc, o, o_s, ap_o, ap_ml, sc_part, gpart, logits, tok, total;
  size_t ap_stride_o, ap_stride_ml;  // floats between canvases' attention partials (a batch)
  // prefill view (same region)
  size_t p_x, p_nrm, p_q, p_ap_o, p_ap_ml, p_gpart, p_total;
};

// Activations are fp32 in the workspace for both dtypes; the bf16 path also
// keeps each projection operand as a split pair (hi and lo bf16 terms, the
// lo array after the hi array, 4 bytes per value: nrm_s, sc_s, o_s, and g,
// which holds only that form there) and the canvas keys and values kc / vc
// only as split pairs ([Hkv][N][hd] hi terms, then the lo terms); nrm16 is
// the bf16 copy of the final normalised state used by the LM head.  nb > 1:
// a batch of nb canvases, whose rows are stacked (N = nb * canvas_len rows)
// in every activation; the attention partials serve one canvas at a time;
// tok holds the stacked ids.
Layout layout(const dg_config *c, int32_t nprefill, bool with_logits, int nb = 1) {
  Layout L{};
  const size_t N = (size_t)nb * c->canvas_len, V = c->vocab, d = c->d_model, F = c->ffn_hidden;
  const int Nc = c->canvas_len;
  const size_t Hq = c->n_q_heads, Hkv = c->n_kv_heads, hd = c->head_dim;
  const bool bf = c->dtype == DG_BF16;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.h0 = take(N * d * 4);
  L.h1 = take(N * d * 4);
  L.nrm = take(N * d * 4);
  L.nrm16 = take(bf ? dg::tl_elems((int)N, (int)d) * 2 : 0);
  L.nrm_s = take(bf ? N * d * 4 : 0);
  L.sc = take(N * d * 4);
  L.sc_s = take(bf ? N * d * 4 : 0);
  L.g = take(N * F * 4);
  L.q = take(Hq * N * hd * 4);
  L.kc = take(Hkv * N * hd * 4);
  L.vc = take(Hkv * N * hd * 4);
  L.o = take(N * Hq * hd * 4);
  L.o_s = take(bf ? N * Hq * hd * 4 : 0);
  int splits = 1, kps = 0;
  // the plan for any key count never uses more splits than for 2^20 keys
  dg::attention_plan(Nc, (int)Hq, 1 << 20, &splits, &kps);
  L.ap_stride_o = (size_t)splits * Hq * Nc * hd;
  L.ap_stride_ml = (size_t)splits * Hq * Nc * 2;
  L.ap_o = take(nb * L.ap_stride_o * 4);
  L.ap_ml = take(nb * L.ap_stride_ml * 4);
  L.sc_part = take(bf ? dg::selfcond_part_bytes(nb, Nc, (int)d, selfcond_ksplit(c)) : 0);
  if (bf) {  // K-split partials of the projections, the largest of the step's four
    const int nqkv[3] = {(int)(Hq * hd), (int)(Hkv * hd), (int)(Hkv * hd)};
    const int nd[1] = {(int)d}, nf[1] = {(int)F};
    size_t m = dg::gemm_split_part_bytes((int)N, Nc, (int)d, nqkv, 3);
    m = std::max(m, dg::gemm_split_part_bytes((int)N, Nc, (int)(Hq * hd), nd, 1));
    m = std::max(m, dg::gemm_split_part_bytes((int)N, Nc, (int)d, nf, 1));
    m = std::max(m, dg::gemm_split_part_bytes((int)N, Nc, (int)F, nd, 1));
    L.gpart = take(m);
  }
  L.logits = take(nb == 1 && (!bf || with_logits) ? N * V * 4 : 0);
  L.tok = take(N * 4);
  L.total = off;
  // prefill
  off = 0;
  const size_t n = nprefill > 0 ? (size_t)nprefill : 0;
  L.p_x = take(n * d * 4);
  L.p_nrm = take(n * d * 4);  // fp32, or the split pair of the bf16 path
  L.p_q = take(Hq * n * hd * 4);
  dg::attention_plan((int)(n ? n : 1), (int)Hq, 1 << 20, &splits, &kps);
  L.p_ap_o = take((size_t)splits * Hq * n * hd * 4);
  L.p_ap_ml = take((size_t)splits * Hq * n * 2 * 4);
  if (bf && n) {
    const int nkvq[3] = {(int)(Hkv * hd), (int)(Hkv * hd), (int)(Hq * hd)};
    L.p_gpart = take(std::max(dg::gemm_split_part_bytes((int)n, Nc, (int)d, nkvq, 2),
                              dg::gemm_split_part_bytes((int)n, Nc, (int)d, nkvq + 2, 1)));
  }
  L.p_total = off;
  return L;
}

std::atomic<bool> g_logits_dump{false};

// profiling (events around the two E-streaming contractions)
std::mutex g_prof_mu;
std::atomic<int> g_prof_mask{0};  // bit 0: LM head, bit 1: self-conditioning contraction
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_prof_lm, g_prof_sc;
// Events created ahead (when profiling is switched on), so that a profiled
// launch costs two event records and no event creation on the host.
std::vector<hipEvent_t> g_prof_pool;
constexpr size_t kProfPool = 1024;

bool prof_take(hipEvent_t *e) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_pool.empty()) {
    *e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return true;
  }
  return hipEventCreate(e) == hipSuccess;
}

struct ProfScope {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> *vec = nullptr;
  hipEvent_t e0{}, e1{};
  hipStream_t s;
  // enabled = false: records nothing (the entry point that allocates nothing)
  ProfScope(std::vector<std::pair<hipEvent_t, hipEvent_t>> &v, hipStream_t st, bool enabled = true) : s(st) {
    if (!enabled || !(g_prof_mask.load(std::memory_order_relaxed) & (&v == &g_prof_lm ? 1 : 2))) return;
    if (!prof_take(&e0)) return;
    if (!prof_take(&e1)) {
      (void)hipEventDestroy(e0);
      return;
    }
    vec = &v;
    (void)hipEventRecord(e0, s);
  }
  ~ProfScope() {
    if (!vec) return;
    (void)hipEventRecord(e1, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    vec->emplace_back(e0, e1);
  }
};

#define DG_TRY(x)                                  \
  do {                                             \
    if ((x) != hipSuccess) return DG_ERR_HIP;      \
  } while (0)

dg::Epi epi_store(void *out, bool f32, int64_t rstride, int cdiv, int64_t chi) {
  dg::Epi e{};
  e.kind = dg::EPI_STORE;
  e.out = out;
  e.out_f32 = f32 ? 1 : 0;
  e.rstride = rstride;
  e.cdiv = cdiv;
  e.chi = chi;
  return e;
}

// Keys or values written by their projection ([head][row][hd], head stride
// head_stride): fp32 for DG_F32; for DG_BF16 a split pair, hi = bf16(v)
// and lo = bf16(v - hi) `plane` elements further on, the form the attention
// kernel copies into LDS unconverted.
dg::Epi epi_kv(const dg_config *c, void *out, int64_t head_stride, int64_t plane) {
  const bool bf = c->dtype == DG_BF16;
  dg::Epi e = epi_store(out, !bf, c->head_dim, c->head_dim, head_stride);
  if (bf) e.lo_off = plane;
  return e;
}

bool weights_ok(const dg_config *c, const dg_weights *w) {
  if (!w || !w->w_sc1 || !w->w_sc2 || !w->wq || !w->wk || !w->wv || !w->wo || !w->g_attn || !w->g_final)
    return false;
  if (c->dtype == DG_BF16 ? !w->E_pack : !w->E) return false;  // DG_BF16 reads only the packed copy
  if (c->sampler == DG_SAMPLER_MASKED && (!w->mask_emb || reinterpret_cast<uintptr_t>(w->mask_emb) % 16))
    return false;
  return true;
}

// The [MASK] token id of the masked sampler (one past the vocabulary), -1 for
// uniform-state re-noise; and the embedding row that id reads.
int mask_id(const dg_config *c) { return c->sampler == DG_SAMPLER_MASKED ? c->vocab : -1; }
template <typename T>
const T *mask_row(const dg_config *c, const dg_weights *w) {
  return c->sampler == DG_SAMPLER_MASKED ? static_cast<const T *>(w->mask_emb) : nullptr;
}

// The adaptive stop on a step's status words: every entropy below conf_eps,
// the canvas stable for stable_steps steps, or (masked sampler) no [MASK] left.
bool status_stops(const int32_t *w, int32_t stable_steps) {
  return w[DG_ST_ALLCONF] != 0 || (stable_steps > 0 && w[DG_ST_STABLE] >= stable_steps) || w[DG_ST_MASKED] == 0;
}

bool canvas_ok(const dg_canvas *cv) {
  return cv && cv->tokens && cv->probs && cv->stats && cv->entropy && cv->argmax && cv->accept && cv->status;
}

// Dense projections C_i[M][N_i] = A[M][K] W_i[N_i][K]^T (up to three weight
// matrices sharing the activation A) with epilogues e_i.  A is dense
// [M][K]: fp32 for DG_F32; for DG_BF16 the split pair (bf16 hi terms
// [M][K], then the lo terms [M][K]).  `part` holds the K-split partials
// (gemm_split_part_bytes; bf16 only).
dg::SplitGemm split_gemm(const void *A, int M, int K) {
  dg::SplitGemm g{};
  g.A = static_cast<const uint16_t *>(A);
  g.lda = K;
  g.lo_off = (int64_t)M * K;
  g.M = M;
  g.K = K;
  return g;
}

hipError_t proj(const dg_config *c, const void *A, int M, int K, int count, const void *const *W, const int *Nout,
                const dg::Epi *e, float *part, hipStream_t s) {
  if (c->dtype == DG_BF16) {
    dg::SplitGemm g = split_gemm(A, M, K);
    g.count = count;
    for (int i = 0; i < count; ++i) {
      g.B[i] = W[i];
      g.N[i] = Nout[i];
      g.e[i] = e[i];
    }
    g.part = part;
    g.ksplit = dg::gemm_split_plan(c->canvas_len, K, Nout, count);
    return dg::gemm_split(g, s);
  }
  for (int i = 0; i < count; ++i) {
    dg::GemmShapeF32 g{static_cast<const float *>(A), K, 1, static_cast<const float *>(W[i]), K, 1, M, Nout[i], K,
                       nullptr, 0};
    const hipError_t err = dg::gemm_f32(g, e[i], s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t proj1(const dg_config *c, const void *A, int M, int K, const void *W, int Nout, const dg::Epi &e,
                 float *part, hipStream_t s) {
  return proj(c, A, M, K, 1, &W, &Nout, &e, part, s);
}

// proj1 whose output rows (fp32 [M][Nout], row-major) then go through
// RMSNorm(gain) into norm_out (fp32), norm_tiled (bf16 tiled) and/or
// norm_split (split pair): for the bf16 path with a K split the norm is
// fused into the split-K merge.
hipError_t proj1_norm(const dg_config *c, const void *A, int M, int K, const void *W, int Nout, const dg::Epi &e,
                      float *part, const void *gain, float *norm_out, bf16 *norm_tiled, bf16 *norm_split,
                      hipStream_t s) {
  if (c->dtype == DG_BF16 && dg::gemm_split_plan(c->canvas_len, K, &Nout, 1) > 1) {
    dg::SplitGemm g = split_gemm(A, M, K);
    g.count = 1;
    g.B[0] = W;
    g.N[0] = Nout;
    g.e[0] = e;
    g.part = part;
    g.ksplit = dg::gemm_split_plan(c->canvas_len, K, &Nout, 1);
    const dg::RowNorm rn{static_cast<const uint16_t *>(gain), c->rms_eps, norm_out, norm_tiled, norm_split};
    return dg::gemm_split_norm(g, rn, s);
  }
  hipError_t err = proj1(c, A, M, K, W, Nout, e, part, s);
  if (err != hipSuccess) return err;
  const float *y = static_cast<const float *>(e.out);
  if (c->dtype == DG_BF16)
    return dg::rmsnorm_rows<bf16>(y, static_cast<const bf16 *>(gain), M, Nout, c->rms_eps, norm_out, norm_tiled,
                                  norm_split, s);
  return dg::rmsnorm_rows<float>(y, static_cast<const float *>(gain), M, Nout, c->rms_eps, norm_out, norm_tiled,
                                 norm_split, s);
}

}  // namespace

extern "C" {

int32_t dg_abi_version(void) { return DG_ABI_VERSION; }

const char *dg_status_string(dg_status status) {
  switch (enum_value(status)) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARG: return "invalid argument";
    case DG_ERR_UNSUPPORTED: return "unsupported shape or configuration";
    case DG_ERR_CAPACITY: return "KV cache capacity exceeded";
    case DG_ERR_WORKSPACE: return "workspace too small";
    case DG_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

dg_status dg_validate_config(const dg_config *cfg) { return check_config(cfg); }

size_t dg_workspace_bytes(const dg_config *cfg, int32_t max_prefill_tokens) {
  if (check_config(cfg) != DG_OK || max_prefill_tokens < 0) return 0;
  const Layout L = layout(cfg, max_prefill_tokens, false);
  return L.total > L.p_total ? L.total : L.p_total;
}

size_t dg_stats_bytes(const dg_config *cfg) {
  if (check_config(cfg) != DG_OK) return 0;
  return stats_layout(cfg).total;
}

size_t dg_embedding_pack_bytes(const dg_config *cfg) {
  if (check_config(cfg) != DG_OK || cfg->dtype != DG_BF16) return 0;
  if (table_fp4(cfg)) return pack4_codes(cfg) + pack4_scales(cfg);
  return pack_elems(cfg) * (table_fp8(cfg) ? 1 : 2);  // fp8: a byte per element, bf16: two
}

size_t dg_probs_bytes(const dg_config *cfg) {
  if (check_config(cfg) != DG_OK) return 0;
  if (cfg->dtype == DG_BF16) return dg::tl_elems(cfg->canvas_len, cfg->vocab) * 2;
  return (size_t)cfg->canvas_len * cfg->vocab * 4;
}

dg_status dg_pack_embedding(const dg_config *cfg, const void *E, void *E_pack, void *stream) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (cfg->dtype != DG_BF16) return DG_OK;  // the fp32 path reads E directly
  if (!E || !E_pack) return DG_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int V = cfg->vocab, d = cfg->d_model;
  const uint16_t *Eb = static_cast<const uint16_t *>(E);
  uint8_t *q = static_cast<uint8_t *>(E_pack);
  if (table_fp8(cfg)) {  // q = E * 2^table_exp as fp8
    DG_TRY(dg::tile_fp8(Eb, V, d, d, false, std::ldexp(1.f, cfg->table_exp), q, s));
  } else if (table_fp4(cfg)) {  // e2m1 codes, then the 32 x 32 blocks' scale bytes
    DG_TRY(dg::tile_fp4(Eb, V, d, d, false, q, q + pack4_codes(cfg), s));
  } else {
    DG_TRY(dg::tile_rows(Eb, V, d, d, static_cast<uint16_t *>(E_pack), s));
  }
  return DG_OK;
}

dg_status dg_canvas_init(const dg_config *cfg, dg_canvas *cv, uint64_t seed, uint32_t canvas_id, void *stream) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!canvas_ok(cv)) return DG_ERR_INVALID_ARG;
  DG_TRY(dg::canvas_init(cv->tokens, cv->status, cfg->canvas_len, ilog2(cfg->vocab), seed, canvas_id,
                         mask_id(cfg), static_cast<hipStream_t>(stream)));
  cv->step = 0;
  cv->has_prev = 0;
  cv->seed = seed;
  cv->canvas_id = canvas_id;
  return DG_OK;
}

dg_status dg_prefill_append(const dg_config *cfg, const dg_weights *w, dg_kv_cache *cache, const int32_t *tokens,
                            int32_t n_tokens, void *attn_out, void *ws, size_t ws_bytes, void *stream) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!weights_ok(cfg, w) || !cache || !cache->k || !cache->v || n_tokens < 0) return DG_ERR_INVALID_ARG;
  if (cache->length < 0 || cache->capacity < 0 || cache->length > cache->capacity) return DG_ERR_INVALID_ARG;
  if (n_tokens > 0 && !tokens) return DG_ERR_INVALID_ARG;
  if ((int64_t)cache->length + n_tokens > cache->capacity) return DG_ERR_CAPACITY;
  if (n_tokens == 0) return DG_OK;
  const Layout L = layout(cfg, n_tokens, false);
  if (!ws || ws_bytes < L.p_total) return DG_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n = n_tokens, d = cfg->d_model, Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads, hd = cfg->head_dim;
  const int V = cfg->vocab, cap = cache->capacity, Lp = cache->length;
  const bool bf = cfg->dtype == DG_BF16;
  char *base = static_cast<char *>(ws);
  float *x = reinterpret_cast<float *>(base + L.p_x);
  float *nrm = reinterpret_cast<float *>(base + L.p_nrm);

  if (bf) {  // nrm holds the split pair
    DG_TRY(dg::gather_rows(packed_table(cfg, w), tokens, n, V, mask_row<uint16_t>(cfg, w), x, s));
    DG_TRY(dg::rmsnorm_rows<bf16>(x, static_cast<const bf16 *>(w->g_attn), n, d, cfg->rms_eps, nullptr, nullptr,
                                  reinterpret_cast<bf16 *>(nrm), s));
  } else {
    DG_TRY(dg::gather_rows(static_cast<const float *>(w->E), tokens, n, d, V, mask_row<float>(cfg, w), x, s));
    DG_TRY(dg::rmsnorm_rows<float>(x, static_cast<const float *>(w->g_attn), n, d, cfg->rms_eps, nrm, nullptr,
                                   nullptr, s));
  }
  // keys/values of the new tokens straight into the cache at [length, length+n)
  // (fp32, or the split pair of a bf16 model)
  const size_t row0 = (size_t)Lp * hd;
  void *kbase = bf ? static_cast<void *>(static_cast<bf16 *>(cache->k) + row0)
                   : static_cast<void *>(static_cast<float *>(cache->k) + row0);
  void *vbase = bf ? static_cast<void *>(static_cast<bf16 *>(cache->v) + row0)
                   : static_cast<void *>(static_cast<float *>(cache->v) + row0);
  float *q = reinterpret_cast<float *>(base + L.p_q);
  const void *W[3] = {w->wk, w->wv, w->wq};
  const int No[3] = {Hkv * hd, Hkv * hd, Hq * hd};
  const int64_t plane = (int64_t)Hkv * cap * hd;
  const dg::Epi E3[3] = {epi_kv(cfg, kbase, (int64_t)cap * hd, plane), epi_kv(cfg, vbase, (int64_t)cap * hd, plane),
                         epi_store(q, true, hd, hd, (int64_t)n * hd)};
  // K and V in one launch whether or not the prompt's attention output is
  // wanted (the split of K follows the launch's shape, so the cache's bits do
  // not depend on that choice); Q in a launch of its own
  float *gp = reinterpret_cast<float *>(base + L.p_gpart);
  DG_TRY(proj(cfg, nrm, n, d, 2, W, No, E3, gp, s));
  if (attn_out) DG_TRY(proj(cfg, nrm, n, d, 1, W + 2, No + 2, E3 + 2, gp, s));
  if (attn_out) {
    dg::AttnArgs a{};
    a.q = q;
    a.nq = n;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.hd = hd;
    a.kA = cache->k;
    a.vA = cache->v;
    a.nA = Lp + n;
    a.capA = cap;
    a.kB = nullptr;
    a.vB = nullptr;
    a.nB = 0;
    a.capB = 0;
    a.causal = 1;
    a.q_pos0 = Lp;
    a.out = attn_out;
    a.part_o = reinterpret_cast<float *>(base + L.p_ap_o);
    a.part_ml = reinterpret_cast<float *>(base + L.p_ap_ml);
    dg::attention_plan(n, Hq, Lp + n, &a.splits, &a.keys_per_split);
    DG_TRY(bf ? dg::attention_mfma(a, s) : dg::attention_f32(a, s));
  }
  cache->length = Lp + n;
  return DG_OK;
}

// How a step treats its self-conditioning contraction (bf16 path):
//   SC_INLINE  launch it in order (the whole step);
//   SC_AHEAD   launch only it, guarded by the status words of the step
//              before (see dg_run_canvas), and return;
//   SC_DONE    it was launched ahead: launch the rest of the step.
enum ScMode { SC_INLINE = 0, SC_AHEAD = 1, SC_DONE = 2 };

// The arguments of one step, short of the workspace.
static dg_status check_step_args(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *cache,
                                 const dg_canvas *cv, float temperature, float gamma) {
  const dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!weights_ok(cfg, w) || !cache || !cache->k || !cache->v || !canvas_ok(cv)) return DG_ERR_INVALID_ARG;
  if (cache->length < 0 || cache->length > cache->capacity) return DG_ERR_INVALID_ARG;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return DG_ERR_INVALID_ARG;
  if (std::isnan(gamma) || gamma < 0.f) return DG_ERR_INVALID_ARG;
  if (cv->step < 0) return DG_ERR_INVALID_ARG;
  return DG_OK;
}

static dg_status denoise_impl(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *cache, dg_canvas *cv,
                              float temperature, float gamma, void *ws, size_t ws_bytes, void *stream,
                              bool logits_dump, ScMode sc_mode = SC_INLINE, int32_t stable_steps = 0,
                              int32_t *host_status = nullptr, bool profile = true) {
  const dg_status st = check_step_args(cfg, w, cache, cv, temperature, gamma);
  if (st != DG_OK) return st;
  const bool bf = cfg->dtype == DG_BF16;
  const bool dump = logits_dump && bf;
  const Layout L = layout(cfg, 0, dump);
  if (!ws || ws_bytes < L.total) return DG_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int N = cfg->canvas_len, V = cfg->vocab, d = cfg->d_model, F = cfg->ffn_hidden;
  const int Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads, hd = cfg->head_dim;
  const int ntiles = V / kTile;
  const float inv_T = 1.0f / temperature;
  char *base = static_cast<char *>(ws);
  float *h0 = reinterpret_cast<float *>(base + L.h0);
  float *h1 = reinterpret_cast<float *>(base + L.h1);
  float *nrm = reinterpret_cast<float *>(base + L.nrm);
  bf16 *nrm16 = reinterpret_cast<bf16 *>(base + L.nrm16);
  float *sc = reinterpret_cast<float *>(base + L.sc), *G = reinterpret_cast<float *>(base + L.g);
  float *q = reinterpret_cast<float *>(base + L.q), *kc = reinterpret_cast<float *>(base + L.kc);
  float *vc = reinterpret_cast<float *>(base + L.vc), *o = reinterpret_cast<float *>(base + L.o);
  char *stats = static_cast<char *>(cv->stats);
  const StatsLayout SL = stats_layout(cfg);
  float4 *tstats = reinterpret_cast<float4 *>(stats + SL.tstats);
  float *tscale = reinterpret_cast<float *>(stats + SL.tscale);
  float2 *top = reinterpret_cast<float2 *>(stats + SL.top);
  float *rscale = reinterpret_cast<float *>(stats + SL.rscale);
  uint8_t *shift = reinterpret_cast<uint8_t *>(stats + SL.shift);
  float *gpart = reinterpret_cast<float *>(base + L.gpart);
  bf16 *nrm_s = reinterpret_cast<bf16 *>(base + L.nrm_s);  // split pairs (bf16 path)
  bf16 *sc_s = reinterpret_cast<bf16 *>(base + L.sc_s);
  bf16 *o_s = reinterpret_cast<bf16 *>(base + L.o_s);

  // 1. embeddings (+ self-conditioning from the previous step's probabilities);
  // with self-conditioning on the bf16 path the embedding rows are gathered
  // by the FFN's output merge (its residual), so h0 is written once
  const bool fused_embed = bf && cv->has_prev;
  if (bf && !fused_embed)
    DG_TRY(dg::gather_rows(packed_table(cfg, w), cv->tokens, N, V, mask_row<uint16_t>(cfg, w), h0, s));
  else if (!bf)
    DG_TRY(dg::gather_rows(static_cast<const float *>(w->E), cv->tokens, N, d, V, mask_row<float>(cfg, w), h0, s));
  if (cv->has_prev) {
    if (bf) {
      const int ks = selfcond_ksplit(cfg);
      float *part = reinterpret_cast<float *>(base + L.sc_part);
      if (sc_mode != SC_DONE) {
        ProfScope ps(g_prof_sc, s, profile);
        const dg::SelfcondGuard guard{sc_mode == SC_AHEAD ? cv->status : nullptr, stable_steps};
        dg::EsCanvasesIn cin{};
        cin.probs[0] = static_cast<const uint16_t *>(cv->probs);
        cin.shift[0] = shift;
        DG_TRY(dg::selfcond_bf16_batch(cin, 1, packed_table(cfg, w), N, d, V, true, part, ks, s, guard));
      }
      if (sc_mode == SC_AHEAD) return DG_OK;
      DG_TRY(dg::selfcond_reduce(part, ks, N, d, top, static_cast<const uint16_t *>(cv->probs), V, rscale, shift,
                                 packed_table(cfg, w), sc, sc_s, s));
    } else {
      dg::GemmShapeF32 g{static_cast<const float *>(cv->probs), V, 1, static_cast<const float *>(w->E), 1, d,
                         N, d, V, nullptr, 0};
      DG_TRY(dg::gemm_f32(g, epi_store(sc, true, d, d, 0), s));
    }
    // G = GELU(W1 S): fp32, or the split pair of the bf16 path
    dg::Epi eg = epi_store(G, !bf, F, F, 0);
    eg.kind = dg::EPI_GELU;
    if (bf) eg.lo_off = (int64_t)N * F;
    DG_TRY(proj1(cfg, bf ? static_cast<const void *>(sc_s) : sc, N, d, w->w_sc1, F, eg, gpart, s));
    dg::Epi ea = epi_store(h0, true, d, d, 0);
    if (fused_embed) {  // h0 = E[tokens] + W2 G
      ea.kind = dg::EPI_ADD_ROW;
      ea.gtab = packed_table(cfg, w);
      ea.gtok = cv->tokens;
      ea.gV = V;
      ea.gmask = mask_row<uint16_t>(cfg, w);
    } else {
      ea.kind = dg::EPI_ADD;
      ea.resid = h0;
    }
    // h0 += W2 G, then 2. the pre-attention RMSNorm of h0 (fused when the GEMM splits K)
    DG_TRY(proj1_norm(cfg, G, N, F, w->w_sc2, d, ea, gpart, w->g_attn, bf ? nullptr : nrm, nullptr,
                      bf ? nrm_s : nullptr, s));
  } else {
    // 2. RMSNorm of the embeddings (no self-conditioning at a canvas's first step)
    if (bf)
      DG_TRY(dg::rmsnorm_rows<bf16>(h0, static_cast<const bf16 *>(w->g_attn), N, d, cfg->rms_eps, nullptr, nullptr,
                                    nrm_s, s));
    else
      DG_TRY(dg::rmsnorm_rows<float>(h0, static_cast<const float *>(w->g_attn), N, d, cfg->rms_eps, nrm, nullptr,
                                     nullptr, s));
  }
  // Q/K/V of the canvas (the canvas keys stay in the workspace)
  {
    const void *W[3] = {w->wq, w->wk, w->wv};
    const int No[3] = {Hq * hd, Hkv * hd, Hkv * hd};
    const int64_t plane = (int64_t)Hkv * N * hd;
    const dg::Epi E3[3] = {epi_store(q, true, hd, hd, (int64_t)N * hd), epi_kv(cfg, kc, (int64_t)N * hd, plane),
                           epi_kv(cfg, vc, (int64_t)N * hd, plane)};
    DG_TRY(proj(cfg, bf ? static_cast<const void *>(nrm_s) : nrm, N, d, 3, W, No, E3, gpart, s));
  }
  // 3. bidirectional attention over [cache || canvas], output projection
  dg::AttnArgs a{};
  a.q = q;
  a.nq = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.hd = hd;
  a.kA = cache->k;
  a.vA = cache->v;
  a.nA = cache->length;
  a.capA = cache->capacity;
  a.kB = kc;
  a.vB = vc;
  a.nB = N;
  a.capB = N;
  a.causal = 0;
  a.q_pos0 = 0;
  a.out = o;
  a.out_split = bf ? o_s : nullptr;
  a.part_o = reinterpret_cast<float *>(base + L.ap_o);
  a.part_ml = reinterpret_cast<float *>(base + L.ap_ml);
  dg::attention_plan(N, Hq, cache->length + N, &a.splits, &a.keys_per_split);
  DG_TRY(bf ? dg::attention_mfma(a, s) : dg::attention_f32(a, s));
  {
    dg::Epi ea = epi_store(h1, true, d, d, 0);
    ea.kind = dg::EPI_ADD;
    ea.resid = h0;
    // h1 = h0 + O Wo^T, then 4. the final RMSNorm (fp32 for the exact top logit,
    // tiled bf16 for the LM head; fused when the GEMM splits K)
    DG_TRY(proj1_norm(cfg, bf ? static_cast<const void *>(o_s) : o, N, Hq * hd, w->wo, d, ea, gpart, w->g_final, nrm,
                      bf ? nrm16 : nullptr, nullptr, s));
  }
  // tied LM head with the softmax/entropy statistics
  float *logits = reinterpret_cast<float *>(base + L.logits);
  if (bf) {
    {
      ProfScope ps(g_prof_lm, s, profile);
      dg::EsCanvases ec{};
      ec.probs[0] = static_cast<uint16_t *>(cv->probs);
      ec.tile_stats[0] = tstats;
      DG_TRY(dg::lm_head_bf16_batch(nrm16, 1, N, d, packed_table(cfg, w), V, inv_T, ec, dump ? logits : nullptr, s));
    }
    // the numerators stay as stored: the next step's contraction applies the
    // power-of-two tile exponents and the row factor (the batch launch with
    // one canvas: a batched step runs this same code for each of its rows)
    dg::RowCombineBatch rc{};
    rc.stats[0] = tstats;
    rc.entropy[0] = cv->entropy;
    rc.cand[0] = cv->argmax;
    rc.row_scale[0] = rscale;
    rc.shift[0] = shift;
    rc.top[0] = top;
    DG_TRY(dg::row_combine_batch(rc, 1, N, ntiles, inv_T, nrm, packed_table(cfg, w), s));
  } else {
    dg::GemmShapeF32 g{nrm, d, 1, static_cast<const float *>(w->E), d, 1, N, V, d, nullptr, 0};
    DG_TRY(dg::gemm_f32(g, epi_store(logits, true, V, V, 0), s));
    DG_TRY(dg::tile_stats_f32(logits, N, V, inv_T, static_cast<float *>(cv->probs), tstats, s));
    DG_TRY(dg::row_combine(tstats, N, ntiles, inv_T, cv->entropy, cv->argmax, tscale, nullptr, nullptr, nullptr,
                           dg::PackedTable{}, top, s));
    DG_TRY(dg::normalize_probs_f32(static_cast<float *>(cv->probs), tscale, N, V, s));
  }
  // [P3] §5.3 multinomial candidates, drawn from the probabilities as kept
  if (cfg->candidate_rule == DG_CANDIDATE_MULTINOMIAL) {
    dg::DrawArgs draw{cv->seed, (uint32_t)cv->step, cv->canvas_id, nullptr, nullptr};
    if (bf)
      draw.num_tiled = static_cast<const uint16_t *>(cv->probs);
    else
      draw.num_f32 = static_cast<const float *>(cv->probs);
    DG_TRY(dg::multinomial_draw(tstats, N, ntiles, inv_T, draw, cv->argmax, s));
  }
  // 5. accept / re-noise / stop flags (the batch launch with one canvas)
  {
    dg::SelectBatch sel{};
    sel.entropy[0] = cv->entropy;
    sel.argmax[0] = cv->argmax;
    sel.tokens[0] = cv->tokens;
    sel.accept[0] = cv->accept;
    sel.status[0] = cv->status;
    sel.seed[0] = cv->seed;
    sel.canvas_id[0] = cv->canvas_id;
    sel.step[0] = (uint32_t)cv->step;
    sel.host_status[0] = host_status;
    sel.pred[0] = top;
    sel.pred_prev[0] = reinterpret_cast<int32_t *>(stats + SL.pred);
    DG_TRY(dg::select_step_batch(sel, 1, N, ilog2(V), (double)gamma, (int)cfg->accept_rule, cfg->conf_eps,
                                 mask_id(cfg), (int)cfg->stable_rule, s));
  }
  cv->step += 1;
  cv->has_prev = 1;
  return DG_OK;
}

// A batch of canvases on the bf16 path ([P5] current limitations: several
// users' canvases in one pass over the table).  Rows are stacked canvas after
// canvas in every activation; the projections and both table-streaming
// contractions run once for the batch (their per-row results do not depend
// on the other rows: the projections' K ranges are a function of K, the
// contractions accumulate each row on its own); attention once per canvas;
// the row statistics and the selection per canvas, one launch each for the
// batch (the kernels the single-canvas step runs).  Validated by the caller.
static dg_status denoise_batch_bf16(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *caches,
                                    dg_canvas *cvs, int B, float temperature, float gamma, void *ws,
                                    hipStream_t s) {
  const Layout L = layout(cfg, 0, false, B);
  const int N = cfg->canvas_len, V = cfg->vocab, d = cfg->d_model, F = cfg->ffn_hidden;
  const int Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads, hd = cfg->head_dim;
  const int BN = B * N, ntiles = V / kTile;
  const float inv_T = 1.0f / temperature;
  char *base = static_cast<char *>(ws);
  float *h0 = reinterpret_cast<float *>(base + L.h0);
  float *h1 = reinterpret_cast<float *>(base + L.h1);
  float *nrm = reinterpret_cast<float *>(base + L.nrm);
  bf16 *nrm16 = reinterpret_cast<bf16 *>(base + L.nrm16);
  float *sc = reinterpret_cast<float *>(base + L.sc), *G = reinterpret_cast<float *>(base + L.g);
  float *q = reinterpret_cast<float *>(base + L.q), *kc = reinterpret_cast<float *>(base + L.kc);
  float *vc = reinterpret_cast<float *>(base + L.vc), *o = reinterpret_cast<float *>(base + L.o);
  float *gpart = reinterpret_cast<float *>(base + L.gpart);
  bf16 *nrm_s = reinterpret_cast<bf16 *>(base + L.nrm_s);
  bf16 *sc_s = reinterpret_cast<bf16 *>(base + L.sc_s);
  bf16 *o_s = reinterpret_cast<bf16 *>(base + L.o_s);
  int32_t *tok = reinterpret_cast<int32_t *>(base + L.tok);
  const StatsLayout SL = stats_layout(cfg);
  auto st_of = [&](int b, size_t off) { return static_cast<char *>(cvs[b].stats) + off; };
  const dg::PackedTable tab = packed_table(cfg, w);

  dg::TokenPtrs tp{};
  for (int b = 0; b < B; ++b) tp.p[b] = cvs[b].tokens;
  DG_TRY(dg::stack_tokens(tp, B, N, tok, s));
  if (cvs[0].has_prev) {
    // S = p_prev E for every canvas in one pass over the table, then the merges
    const int ks = selfcond_ksplit(cfg);
    float *part = reinterpret_cast<float *>(base + L.sc_part);
    dg::EsCanvasesIn cin{};
    for (int b = 0; b < B; ++b) {
      cin.probs[b] = static_cast<const uint16_t *>(cvs[b].probs);
      cin.shift[b] = reinterpret_cast<const uint8_t *>(st_of(b, SL.shift));
    }
    {
      ProfScope ps(g_prof_sc, s);
      DG_TRY(dg::selfcond_bf16_batch(cin, B, tab, N, d, V, true, part, ks, s));
    }
    dg::ReduceBatch rb{};
    for (int b = 0; b < B; ++b) {
      rb.top[b] = reinterpret_cast<const float2 *>(st_of(b, SL.top));
      rb.probs[b] = cin.probs[b];
      rb.row_scale[b] = reinterpret_cast<const float *>(st_of(b, SL.rscale));
      rb.shift[b] = cin.shift[b];
    }
    DG_TRY(dg::selfcond_reduce_batch(part, ks, B, N, d, rb, V, tab, sc, sc_s, s, (int64_t)BN * d));
    dg::Epi eg = epi_store(G, false, F, F, 0);
    eg.kind = dg::EPI_GELU;
    eg.lo_off = (int64_t)BN * F;
    DG_TRY(proj1(cfg, sc_s, BN, d, w->w_sc1, F, eg, gpart, s));
    dg::Epi ea = epi_store(h0, true, d, d, 0);  // h0 = E[tokens] + W2 G
    ea.kind = dg::EPI_ADD_ROW;
    ea.gtab = tab;
    ea.gtok = tok;
    ea.gV = V;
    ea.gmask = mask_row<uint16_t>(cfg, w);
    DG_TRY(proj1_norm(cfg, G, BN, F, w->w_sc2, d, ea, gpart, w->g_attn, nullptr, nullptr, nrm_s, s));
  } else {
    DG_TRY(dg::gather_rows(tab, tok, BN, V, mask_row<uint16_t>(cfg, w), h0, s));
    DG_TRY(dg::rmsnorm_rows<bf16>(h0, static_cast<const bf16 *>(w->g_attn), BN, d, cfg->rms_eps, nullptr, nullptr,
                                  nrm_s, s));
  }
  {
    const void *W[3] = {w->wq, w->wk, w->wv};
    const int No[3] = {Hq * hd, Hkv * hd, Hkv * hd};
    const dg::Epi E3[3] = {epi_store(q, true, hd, hd, (int64_t)BN * hd),
                           epi_kv(cfg, kc, (int64_t)BN * hd, (int64_t)Hkv * BN * hd),
                           epi_kv(cfg, vc, (int64_t)BN * hd, (int64_t)Hkv * BN * hd)};
    DG_TRY(proj(cfg, nrm_s, BN, d, 3, W, No, E3, gpart, s));
  }
  dg::AttnBatch ab{};  // every canvas's attention in one split launch and one merge launch
  ab.B = B;
  for (int b = 0; b < B; ++b) {  // canvas b: its queries over [its cache || its own keys]
    dg::AttnArgs &a = ab.c[b];
    a.q = q + (size_t)b * N * hd;
    a.q_hstride = (int64_t)BN * hd;
    a.nq = N;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.hd = hd;
    a.kA = caches[b].k;
    a.vA = caches[b].v;
    a.nA = caches[b].length;
    a.capA = caches[b].capacity;
    a.kB = reinterpret_cast<bf16 *>(kc) + (size_t)b * N * hd;  // split pairs (the batch is bf16)
    a.vB = reinterpret_cast<bf16 *>(vc) + (size_t)b * N * hd;
    a.nB = N;
    a.capB = BN;
    a.causal = 0;
    a.q_pos0 = 0;
    a.out = o + (size_t)b * N * Hq * hd;
    a.out_split = o_s + (size_t)b * N * Hq * hd;
    a.out_lo_off = (int64_t)BN * Hq * hd;
    a.part_o = reinterpret_cast<float *>(base + L.ap_o) + (size_t)b * L.ap_stride_o;
    a.part_ml = reinterpret_cast<float *>(base + L.ap_ml) + (size_t)b * L.ap_stride_ml;
    dg::attention_plan(N, Hq, caches[b].length + N, &a.splits, &a.keys_per_split);
    ab.zbase[b + 1] = ab.zbase[b] + a.splits;
  }
  DG_TRY(dg::attention_mfma_batch(ab, s));
  {
    dg::Epi ea = epi_store(h1, true, d, d, 0);
    ea.kind = dg::EPI_ADD;
    ea.resid = h0;
    DG_TRY(proj1_norm(cfg, o_s, BN, Hq * hd, w->wo, d, ea, gpart, w->g_final, nrm, nrm16, nullptr, s));
  }
  {
    dg::EsCanvases ec{};
    for (int b = 0; b < B; ++b) {
      ec.probs[b] = static_cast<uint16_t *>(cvs[b].probs);
      ec.tile_stats[b] = reinterpret_cast<float4 *>(st_of(b, SL.tstats));
    }
    ProfScope ps(g_prof_lm, s);
    DG_TRY(dg::lm_head_bf16_batch(nrm16, B, N, d, tab, V, inv_T, ec, nullptr, s));
  }
  {  // row statistics of every canvas in one launch, then its candidates, then one selection launch
    dg::RowCombineBatch rc{};
    dg::SelectBatch sel{};
    for (int b = 0; b < B; ++b) {
      dg_canvas *cv = &cvs[b];
      rc.stats[b] = reinterpret_cast<const float4 *>(st_of(b, SL.tstats));
      rc.entropy[b] = cv->entropy;
      rc.cand[b] = cv->argmax;
      rc.row_scale[b] = reinterpret_cast<float *>(st_of(b, SL.rscale));
      rc.shift[b] = reinterpret_cast<uint8_t *>(st_of(b, SL.shift));
      rc.top[b] = reinterpret_cast<float2 *>(st_of(b, SL.top));
      sel.entropy[b] = cv->entropy;
      sel.argmax[b] = cv->argmax;
      sel.tokens[b] = cv->tokens;
      sel.accept[b] = cv->accept;
      sel.status[b] = cv->status;
      sel.seed[b] = cv->seed;
      sel.canvas_id[b] = cv->canvas_id;
      sel.step[b] = (uint32_t)cv->step;
      sel.pred[b] = reinterpret_cast<const float2 *>(st_of(b, SL.top));
      sel.pred_prev[b] = reinterpret_cast<int32_t *>(st_of(b, SL.pred));
    }
    DG_TRY(dg::row_combine_batch(rc, B, N, ntiles, inv_T, nrm, tab, s));
    if (cfg->candidate_rule == DG_CANDIDATE_MULTINOMIAL)
      for (int b = 0; b < B; ++b) {
        dg_canvas *cv = &cvs[b];
        dg::DrawArgs draw{cv->seed, (uint32_t)cv->step, cv->canvas_id, static_cast<const uint16_t *>(cv->probs),
                          nullptr};
        DG_TRY(dg::multinomial_draw(rc.stats[b], N, ntiles, inv_T, draw, cv->argmax, s));
      }
    DG_TRY(dg::select_step_batch(sel, B, N, ilog2(V), (double)gamma, (int)cfg->accept_rule, cfg->conf_eps,
                                 mask_id(cfg), (int)cfg->stable_rule, s));
  }
  for (int b = 0; b < B; ++b) {
    cvs[b].step += 1;
    cvs[b].has_prev = 1;
  }
  return DG_OK;
}

dg_status dg_denoise_step(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *cache, dg_canvas *cv,
                          float temperature, float accept_threshold_nats, void *ws, size_t ws_bytes, void *stream) {
  return denoise_impl(cfg, w, cache, cv, temperature, accept_threshold_nats, ws, ws_bytes, stream,
                      g_logits_dump.load());
}

// ---- the step without a caller workspace ---------------------------------------
// For callers that cannot allocate (graph capture, tight serving loops,
// harnesses that forbid hipMalloc): the step's scratch lives in this
// file-scope device array, one copy per device the library is loaded on,
// held until the process ends.  Host code never names the array itself (its
// host-side symbol is a stand-in, not a device address): each device's
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and is what the kernels receive.
static __device__ __align__(256) char scratch[DG_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up on the device's first call).
dg_status scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DG_ERR_HIP;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // idempotent: two threads racing here both get the same address
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DG_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return DG_OK;
}
}  // namespace

dg_status dg_denoise_step_static(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *cache, dg_canvas *cv,
                                 float temperature, float accept_threshold_nats, void *stream) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (layout(cfg, 0, false).total > DG_STATIC_SCRATCH_BYTES) return DG_ERR_WORKSPACE;
  st = check_step_args(cfg, w, cache, cv, temperature, accept_threshold_nats);
  if (st != DG_OK) return st;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != DG_OK) return st;
  return denoise_impl(cfg, w, cache, cv, temperature, accept_threshold_nats, ws, DG_STATIC_SCRATCH_BYTES, stream,
                      /*logits_dump=*/false, SC_INLINE, 0, nullptr, /*profile=*/false);
}

// The batch's stacked layout; at least the single step's (the fp32 path steps
// the canvases one by one).
static size_t batch_ws_bytes(const dg_config *cfg, int32_t n) {
  return std::max(layout(cfg, 0, false, n).total, layout(cfg, 0, false).total);
}

size_t dg_workspace_bytes_batch(const dg_config *cfg, int32_t n_canvases) {
  if (check_config(cfg) != DG_OK || n_canvases < 1 || n_canvases > DG_MAX_BATCH) return 0;
  return batch_ws_bytes(cfg, n_canvases);
}

dg_status dg_denoise_step_batch(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *caches,
                                dg_canvas *canvases, int32_t n_canvases, float temperature,
                                float accept_threshold_nats, void *ws, size_t ws_bytes, void *stream) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (n_canvases < 1 || n_canvases > DG_MAX_BATCH || !caches || !canvases || !weights_ok(cfg, w))
    return DG_ERR_INVALID_ARG;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return DG_ERR_INVALID_ARG;
  if (std::isnan(accept_threshold_nats) || accept_threshold_nats < 0.f) return DG_ERR_INVALID_ARG;
  for (int32_t b = 0; b < n_canvases; ++b) {
    const dg_kv_cache &c = caches[b];
    if (!c.k || !c.v || c.length < 0 || c.length > c.capacity) return DG_ERR_INVALID_ARG;
    if (!canvas_ok(&canvases[b]) || canvases[b].step < 0 || canvases[b].has_prev != canvases[0].has_prev)
      return DG_ERR_INVALID_ARG;
    for (int32_t a = 0; a < b; ++a) {  // the canvases' buffers are written: no two may share one
      const dg_canvas &x = canvases[a], &y = canvases[b];
      if (x.tokens == y.tokens || x.probs == y.probs || x.stats == y.stats || x.entropy == y.entropy ||
          x.argmax == y.argmax || x.accept == y.accept || x.status == y.status)
        return DG_ERR_INVALID_ARG;
    }
  }
  if (!ws || ws_bytes < batch_ws_bytes(cfg, n_canvases)) return DG_ERR_WORKSPACE;
  if (cfg->dtype != DG_BF16) {  // the fp32 path: the single-canvas step, canvas after canvas
    for (int32_t b = 0; b < n_canvases; ++b) {
      st = denoise_impl(cfg, w, &caches[b], &canvases[b], temperature, accept_threshold_nats, ws, ws_bytes, stream,
                        false);
      if (st != DG_OK) return st;
    }
    return DG_OK;
  }
  return denoise_batch_bf16(cfg, w, caches, canvases, n_canvases, temperature, accept_threshold_nats, ws,
                            static_cast<hipStream_t>(stream));
}

dg_status dg_should_stop(const dg_config *cfg, const dg_canvas *cv, int32_t stable_steps, int32_t *stop_host,
                         dg_step_stats *stats_host, void *stream) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!canvas_ok(cv) || !stop_host) return DG_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t w[DG_STATUS_WORDS];
  DG_TRY(hipMemcpyAsync(w, cv->status, sizeof(w), hipMemcpyDeviceToHost, s));
  DG_TRY(hipStreamSynchronize(s));
  *stop_host = status_stops(w, stable_steps) ? 1 : 0;
  if (stats_host) {
    stats_host->accepted = w[DG_ST_ACCEPTED];
    stats_host->stable = w[DG_ST_STABLE];
    stats_host->allconf = w[DG_ST_ALLCONF];
    stats_host->changed = w[DG_ST_CHANGED];
    float f;
    std::memcpy(&f, &w[DG_ST_HMIN], 4);
    stats_host->h_min = f;
    std::memcpy(&f, &w[DG_ST_HMEAN], 4);
    stats_host->h_mean = f;
    std::memcpy(&f, &w[DG_ST_HMAX], 4);
    stats_host->h_max = f;
    stats_host->masked = w[DG_ST_MASKED];
  }
  return DG_OK;
}

dg_status dg_run_canvas(const dg_config *cfg, const dg_weights *w, const dg_kv_cache *cache, dg_canvas *cv,
                        uint64_t seed, uint32_t canvas_id, const float *temps, int32_t max_steps,
                        float accept_threshold_nats, int32_t adaptive_stop, int32_t stable_steps, void *ws,
                        size_t ws_bytes, void *stream, int32_t *steps_run, int32_t *stopped) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!weights_ok(cfg, w) || !cache || !cache->k || !cache->v || !canvas_ok(cv) || !steps_run || !stopped)
    return DG_ERR_INVALID_ARG;
  if (cache->length < 0 || cache->length > cache->capacity) return DG_ERR_INVALID_ARG;
  if (max_steps < 0 || (max_steps > 0 && !temps)) return DG_ERR_INVALID_ARG;
  for (int32_t i = 0; i < max_steps; ++i)
    if (!(std::isfinite(temps[i]) && temps[i] > 0.f)) return DG_ERR_INVALID_ARG;
  if (std::isnan(accept_threshold_nats) || accept_threshold_nats < 0.f) return DG_ERR_INVALID_ARG;
  const bool dump = g_logits_dump.load();
  if (!ws || ws_bytes < layout(cfg, 0, dump && cfg->dtype == DG_BF16).total) return DG_ERR_WORKSPACE;
  // Host-visible copy of the status words, one per host thread (kept for the
  // process): coherent pinned memory that the selection kernel writes
  // directly, the step word last, so the host learns a step's outcome without
  // a copy or an event; it polls that word.
  thread_local int32_t *host_words = nullptr;
  thread_local int32_t *host_words_dev = nullptr;
  if (adaptive_stop && !host_words) {
    if (hipHostMalloc(reinterpret_cast<void **>(&host_words), DG_STATUS_WORDS * sizeof(int32_t),
                      hipHostMallocCoherent | hipHostMallocMapped) != hipSuccess) {
      host_words = nullptr;
      return DG_ERR_HIP;
    }
    if (hipHostGetDevicePointer(reinterpret_cast<void **>(&host_words_dev), host_words, 0) != hipSuccess) {
      (void)hipHostFree(host_words);
      host_words = nullptr;
      return DG_ERR_HIP;
    }
  }
  *steps_run = 0;
  *stopped = 0;
  st = dg_canvas_init(cfg, cv, seed, canvas_id, stream);
  if (st != DG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // With the adaptive stop, step i+1's self-conditioning contraction (its
  // first kernel, which writes only the workspace) is launched before the
  // host reads step i's status, guarded by those status words on the
  // device: the host's wait and the next launches hide behind a kernel that
  // is running anyway, and if step i did stop the canvas, every workgroup
  // of the guarded launch returns at once.
  const bool ahead_ok = adaptive_stop && cfg->dtype == DG_BF16;
  bool ahead = false;  // step i's contraction is already in the stream
  for (int32_t i = 0; i < max_steps; ++i) {
    const int32_t step_index = cv->step;
    if (adaptive_stop) reinterpret_cast<volatile int32_t *>(host_words)[DG_ST_STEP] = -1;
    st = denoise_impl(cfg, w, cache, cv, temps[i], accept_threshold_nats, ws, ws_bytes, stream, dump,
                      ahead ? SC_DONE : SC_INLINE, 0, adaptive_stop ? host_words_dev : nullptr);
    if (st != DG_OK) return st;
    *steps_run = i + 1;
    if (adaptive_stop) {
      ahead = ahead_ok && i + 1 < max_steps;
      if (ahead) {
        st = denoise_impl(cfg, w, cache, cv, temps[i + 1], accept_threshold_nats, ws, ws_bytes, stream, dump,
                          SC_AHEAD, stable_steps);
        if (st != DG_OK) return st;
      }
      // wait for the step word; every 4096 polls make sure the stream is
      // still running (a stream that finished or failed without writing it
      // is an error, never an endless wait)
      volatile int32_t *hw = host_words;
      for (uint32_t polls = 1; hw[DG_ST_STEP] != step_index; ++polls) {
        if ((polls & 4095) == 0) {
          const hipError_t q = hipStreamQuery(s);
          if (q == hipSuccess) {
            if (hw[DG_ST_STEP] == step_index) break;
            return DG_ERR_HIP;
          }
          if (q != hipErrorNotReady) return DG_ERR_HIP;
        }
      }
      std::atomic_thread_fence(std::memory_order_acquire);
      int32_t words[DG_STATUS_WORDS];
      for (int k = 0; k < DG_STATUS_WORDS; ++k) words[k] = hw[k];
      if (status_stops(words, stable_steps)) {
        *stopped = 1;
        if (ahead) DG_TRY(hipStreamSynchronize(s));  // the guarded launch returns at once
        break;
      }
    }
  }
  return DG_OK;
}

// ---- test and measurement exports --------------------------------------------
dg_status dg_test_ws_offsets(const dg_config *cfg, dg_ws_offsets *out) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!out) return DG_ERR_INVALID_ARG;
  const Layout L = layout(cfg, 0, true);
  out->h0 = L.h0;
  out->attn = L.o;
  out->h1 = L.h1;
  out->selfcond = L.sc;
  out->logits = L.logits;
  return DG_OK;
}

void dg_test_set_logits_dump(int32_t on) { g_logits_dump.store(on != 0); }

size_t dg_test_logits_ws_bytes(const dg_config *cfg) {
  if (check_config(cfg) != DG_OK) return 0;
  return layout(cfg, 0, true).total;
}

// The step's self-conditioning vector S = p E as dg_denoise_step computes
// it (bf16: the production contraction with per-tile exponents, then the
// merge with the row factor and the dominant-token correction; f32: the
// fp32 GEMM).  probs, shift, rscale, top as in the canvas state; S fp32.
static hipError_t selfcond_vector(const dg_config *cfg, const dg_weights *w, const void *probs, const uint8_t *shift,
                                  const float *rscale, const float2 *top, float *S, float *part, hipStream_t s) {
  const int N = cfg->canvas_len, V = cfg->vocab, d = cfg->d_model;
  if (cfg->dtype == DG_BF16) {
    const int ks = selfcond_ksplit(cfg);
    const dg::PackedTable tab = packed_table(cfg, w);
    dg::EsCanvasesIn cin{};
    cin.probs[0] = static_cast<const uint16_t *>(probs);
    cin.shift[0] = shift;
    hipError_t e = dg::selfcond_bf16_batch(cin, 1, tab, N, d, V, true, part, ks, s);
    if (e != hipSuccess) return e;
    return dg::selfcond_reduce(part, ks, N, d, top, static_cast<const uint16_t *>(probs), V, rscale, shift, tab, S,
                               nullptr, s);
  }
  dg::GemmShapeF32 g{static_cast<const float *>(probs), V, 1, static_cast<const float *>(w->E), 1, d, N, d, V,
                     nullptr, 0};
  return dg::gemm_f32(g, epi_store(S, true, d, d, 0), s);
}

dg_status dg_test_selfcond(const dg_config *cfg, const dg_weights *w, const void *P, void *S, void *ws,
                           size_t ws_bytes, void *stream) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!weights_ok(cfg, w) || !P || !S) return DG_ERR_INVALID_ARG;
  const Layout L = layout(cfg, 0, true);  // the dump layout: room for zero exponents
  if (!ws || ws_bytes < L.total) return DG_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *base = static_cast<char *>(ws);
  uint8_t *zero_shift = nullptr;
  if (cfg->dtype == DG_BF16) {  // exponents 0 (plain probabilities) in the logits region
    zero_shift = reinterpret_cast<uint8_t *>(base + L.logits);
    DG_TRY(hipMemsetAsync(zero_shift, 0, (size_t)(cfg->vocab / kTile) * 256, s));
  }
  DG_TRY(selfcond_vector(cfg, w, P, zero_shift, nullptr, nullptr, static_cast<float *>(S),
                         reinterpret_cast<float *>(base + L.sc_part), s));
  return DG_OK;
}

dg_status dg_test_selfcond_canvas(const dg_config *cfg, const dg_weights *w, const dg_canvas *cv, void *S, void *ws,
                                  size_t ws_bytes, void *stream) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!weights_ok(cfg, w) || !canvas_ok(cv) || !S) return DG_ERR_INVALID_ARG;
  const Layout L = layout(cfg, 0, false);
  if (!ws || ws_bytes < L.total) return DG_ERR_WORKSPACE;
  const StatsLayout SL = stats_layout(cfg);
  const char *stats = static_cast<const char *>(cv->stats);
  const bool bf = cfg->dtype == DG_BF16;
  DG_TRY(selfcond_vector(cfg, w, cv->probs, bf ? reinterpret_cast<const uint8_t *>(stats + SL.shift) : nullptr,
                         bf ? reinterpret_cast<const float *>(stats + SL.rscale) : nullptr,
                         bf ? reinterpret_cast<const float2 *>(stats + SL.top) : nullptr, static_cast<float *>(S),
                         reinterpret_cast<float *>(static_cast<char *>(ws) + L.sc_part),
                         static_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_test_select(const dg_config *cfg, dg_canvas *cv, float gamma, void *stream) {
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!canvas_ok(cv) || std::isnan(gamma) || gamma < 0.f || cv->step < 0) return DG_ERR_INVALID_ARG;
  dg::SelectBatch sel{};  // the kernel the step launches
  sel.entropy[0] = cv->entropy;
  sel.argmax[0] = cv->argmax;
  sel.tokens[0] = cv->tokens;
  sel.accept[0] = cv->accept;
  sel.status[0] = cv->status;
  sel.seed[0] = cv->seed;
  sel.canvas_id[0] = cv->canvas_id;
  sel.step[0] = (uint32_t)cv->step;
  const StatsLayout SL = stats_layout(cfg);
  sel.pred[0] = reinterpret_cast<const float2 *>(static_cast<char *>(cv->stats) + SL.top);
  sel.pred_prev[0] = reinterpret_cast<int32_t *>(static_cast<char *>(cv->stats) + SL.pred);
  DG_TRY(dg::select_step_batch(sel, 1, cfg->canvas_len, ilog2(cfg->vocab), (double)gamma, (int)cfg->accept_rule,
                               cfg->conf_eps, mask_id(cfg), (int)cfg->stable_rule,
                               static_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_test_philox(const uint32_t *ctr, uint32_t k0, uint32_t k1, uint32_t *out, int32_t n, void *stream) {
  if (n < 0 || (n > 0 && (!ctr || !out))) return DG_ERR_INVALID_ARG;
  DG_TRY(dg::philox_test(ctr, k0, k1, out, n, static_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_test_gumbel(const uint32_t *w, int32_t n, int32_t mode, float *out, void *stream) {
  if (n < 0 || (mode != 0 && mode != 1) || (n > 0 && (!w || !out))) return DG_ERR_INVALID_ARG;
  DG_TRY(dg::gumbel_test(w, n, mode, out, static_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_test_copy(const void *src, void *dst, size_t bytes, void *stream) {
  if (!src || !dst || bytes % 16 != 0) return DG_ERR_INVALID_ARG;
  DG_TRY(dg::copy_bytes(src, dst, bytes, static_cast<hipStream_t>(stream)));
  return DG_OK;
}

void dg_profile_enable(int32_t mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  while (mask && g_prof_pool.size() < kProfPool) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) break;
    g_prof_pool.push_back(e);
  }
  g_prof_mask = mask & 3;
}

dg_status dg_profile_read(float *lm_ms, int32_t *lm_n, float *sc_ms, int32_t *sc_n) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  auto drain = [](std::vector<std::pair<hipEvent_t, hipEvent_t>> &v, float *ms, int32_t *n) -> bool {
    float tot = 0.f;
    bool ok = true;
    for (auto &pr : v) {
      if (hipEventSynchronize(pr.second) != hipSuccess) ok = false;
      float t = 0.f;
      if (hipEventElapsedTime(&t, pr.first, pr.second) != hipSuccess) ok = false;
      tot += t;
      for (hipEvent_t e : {pr.first, pr.second}) {
        if (g_prof_pool.size() < kProfPool)
          g_prof_pool.push_back(e);
        else
          (void)hipEventDestroy(e);
      }
    }
    if (ms) *ms = tot;
    if (n) *n = (int32_t)v.size();
    v.clear();
    return ok;
  };
  const bool a = drain(g_prof_lm, lm_ms, lm_n);
  const bool b = drain(g_prof_sc, sc_ms, sc_n);
  return (a && b) ? DG_OK : DG_ERR_HIP;
}

}  // extern "C"
