// attention.hip -- attention of canvas (or prompt) queries over the prefix KV
// cache and the canvas, head_dim 128, on CDNA4 matrix cores.
//
// Denoise mode reads every key (bidirectional, no mask); prefill mode masks
// keys beyond each query's absolute position (causal).  Keys come from two
// segments, the committed cache [0, nA) and the step's own canvas keys
// [0, nB), so the cache is never written by a denoising step.
//
// Queries are fp32 in memory and split into two bf16 terms (hi + lo) as
// they are loaded; keys and values are stored as such split pairs already
// (the projection that produces them writes both terms: the KV cache of a
// bf16 model and the step's own canvas keys), so a tile of them reaches LDS
// by the DMA form of the vector load, unconverted.  Every product of two
// split operands is formed from three bf16 MFMAs (hi*hi + hi*lo + lo*hi),
// which keeps the scores and the output within ~1e-5 of fp32.
//
// Flash-style: a workgroup owns 128 queries of G query heads that share one
// KV head (G = 2 when the group size is even, else 1; 4 waves of 32
// queries per head) and a contiguous range of keys (split-KV, partial
// results merged by a second kernel), so each 64-key tile of K and V is
// staged through LDS once for G heads, in a two-tile ring (the next tile
// is in flight while the current one is used).  The wave computes
// S^T = K Q^T so that each lane ends up holding one query's scores, keeps
// the running max / sum per lane, and computes O^T = V^T P^T with the
// probabilities taken straight from registers; the V^T fragments come out
// of the row-major V tile through the gfx950 transposing LDS read.
// Grouped-query attention maps query head h to KV head h / (Hq / Hkv).
#include "dg_device.h"
#include "dg_kernels.h"

namespace dg {

namespace {
constexpr int HD = 128;
constexpr int BQ = 128;   // queries per workgroup
constexpr int KT = 64;    // keys per tile
constexpr int NTH = 256;  // 4 waves
constexpr float LOG2E = 1.4426950408889634f;
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
}  // namespace

// K tile in LDS: [64 keys][16 chunks of 8], chunk c of key r at c ^ (r & 15),
// so the 32 keys one fragment read touches at one chunk fall on distinct banks.
__device__ __forceinline__ int kswz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }
// V tile in LDS: [64 keys][16 chunks of 8 hd], chunk c of key r at
// c ^ 4 (r & 3): a transposing read covers 4 consecutive keys x 16 hd
// (two chunks per key) for each of two 16-hd halves, 16 distinct chunks.
__device__ __forceinline__ int vswz(int row, int chunk) { return row * 16 + (chunk ^ (4 * (row & 3))); }
constexpr int ATT_TERM = KT * HD * 2;     // bytes of one term (hi or lo) of a K or V tile
constexpr int ATT_STAGE = 4 * ATT_TERM;   // K hi, K lo, V hi, V lo
constexpr int ATT_LDS = 2 * ATT_STAGE;    // two stages

// The canvas of grid z-slice `z` of a batch launch (canvas c owns z-slices
// zbase[c] .. zbase[c + 1] - 1: its own split plan) and that slice's split.
__device__ __forceinline__ int attn_canvas(const AttnBatch &bt, int &z) {
  int c = 0;
  while (c + 1 < bt.B && z >= bt.zbase[c + 1]) ++c;
  z -= bt.zbase[c];
  return c;
}

template <int n>
__device__ __forceinline__ void att_wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// DMA of the 64-key tile at kt0 into a stage: four 16 KB terms (K hi, K lo,
// V hi, V lo) in 1 KB parts (4 keys x 16 chunks), PERW per wave, all of a
// wave's parts in one term.  Each lane copies one 16-byte chunk, the
// swizzle applied to its source, from the cache or the canvas segment by
// its own key; a key past the range copies the range's last key (its
// scores are masked and its probabilities are 0).
template <int G>
__device__ __forceinline__ void att_issue(const bf16 *__restrict__ kA, const bf16 *__restrict__ vA,
                                          const bf16 *__restrict__ kB, const bf16 *__restrict__ vB, int64_t loA,
                                          int64_t loB, int nA, int kt0, int kend, char *__restrict__ st) {
  constexpr int PERW = 64 / (4 * G);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int term = (wave * PERW) >> 4, part0 = (wave * PERW) & 15;
  const bool isV = term >= 2, isLo = term & 1;
  char *dst = st + term * ATT_TERM + part0 * 1024;
  const int sl = lane & 15;
  if (kt0 + KT <= kend && (kt0 + KT <= nA || kt0 >= nA)) {  // the tile lies in one segment: one base
    const bool inA = kt0 < nA;
    const bf16 *base = (isV ? (inA ? vA : vB) : (inA ? kA : kB)) + (int64_t)(inA ? kt0 : kt0 - nA) * HD +
                       (isLo ? (inA ? loA : loB) : 0);
#pragma unroll
    for (int u = 0; u < PERW; ++u) {
      const int key = (part0 + u) * 4 + (lane >> 4);
      const int ch = isV ? (sl ^ (4 * (key & 3))) : (sl ^ (key & 15));
      __builtin_amdgcn_global_load_lds(base + key * HD + ch * 8, dst + u * 1024, 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int u = 0; u < PERW; ++u) {
      const int key = (part0 + u) * 4 + (lane >> 4);
      const int ch = isV ? (sl ^ (4 * (key & 3))) : (sl ^ (key & 15));
      const int kc = min(kt0 + key, kend - 1);
      const bool inA = kc < nA;
      const bf16 *base = isV ? (inA ? vA : vB) : (inA ? kA : kB);
      const int64_t off = (int64_t)(inA ? kc : kc - nA) * HD + ch * 8 + (isLo ? (inA ? loA : loB) : 0);
      __builtin_amdgcn_global_load_lds(base + off, dst + u * 1024, 16, 0, 0);
    }
  }
}

// The key range [kbeg, kend) of one KV group against the wave's 32 queries
// (fragments qh / ql): running max m_run, sum l_run and O^T accumulators.
// The operands come in as restrict-qualified parameters, which tells the
// compiler the LDS reads do not depend on the DMA copies in flight (the
// wait / barrier pair before each tile orders them).
template <int G>
__device__ __forceinline__ void att_tiles(const bf16 *__restrict__ kA, const bf16 *__restrict__ vA,
                                          const bf16 *__restrict__ kB, const bf16 *__restrict__ vB, int64_t loA,
                                          int64_t loB, int nA, int kbeg, int kend, int qlimit, bool causal,
                                          const bf16x8_t (&qh)[HD / 16], const bf16x8_t (&ql)[HD / 16],
                                          char *__restrict__ lds, f32x16_t (&oacc)[HD / 32], float &m_run,
                                          float &l_run) {
  constexpr int PERW = 64 / (4 * G);
  const int lane = threadIdx.x & 63, g4 = lane >> 5;
  const float sc = rsqrtf((float)HD) * LOG2E;
  const int ntile = (kend - kbeg + KT - 1) / KT;
  if (ntile <= 0) return;
  att_issue<G>(kA, vA, kB, vB, loA, loB, nA, kbeg, kend, lds);
  if (ntile > 1) att_issue<G>(kA, vA, kB, vB, loA, loB, nA, kbeg + KT, kend, lds + ATT_STAGE);
  for (int t = 0; t < ntile; ++t) {
    const int kt0 = kbeg + t * KT;
    if (t + 1 < ntile)
      att_wait_vmcnt<PERW>();  // this wave's copies of tile t landed (tile t + 1's may be in flight)
    else
      att_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // ... and every wave's
    const char *st = lds + (t & 1) * ATT_STAGE;
    const uint4 *Kh = reinterpret_cast<const uint4 *>(st), *Kl = reinterpret_cast<const uint4 *>(st + ATT_TERM);
    const char *Vh = st + 2 * ATT_TERM, *Vl = st + 3 * ATT_TERM;

    // S^T for two 32-key blocks: K_hi Q_hi + K_lo Q_hi + K_hi Q_lo.
    f32x16_t sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[b][r] = 0.f;
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) {
        const int li = kswz(b * 32 + (lane & 31), 2 * s + g4);
        const bf16x8_t kh = __builtin_bit_cast(bf16x8_t, Kh[li]);
        const bf16x8_t kl = __builtin_bit_cast(bf16x8_t, Kl[li]);
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qh[s], sacc[b], 0, 0, 0);
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, ql[s], sacc[b], 0, 0, 0);
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qh[s], sacc[b], 0, 0, 0);
      }
    }
    // mask (only a partial tile or causal mode needs it), scale, running max
    float tmax = -INFINITY;
    if (kt0 + KT > kend || causal) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kabs = kt0 + b * 32 + (r & 3) + 4 * g4 + 8 * (r >> 2);
          float v = sacc[b][r] * sc;
          if (kabs >= kend || kabs > qlimit) v = -INFINITY;
          sacc[b][r] = v;
          tmax = fmaxf(tmax, v);
        }
    } else {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[b][r] *= sc;
          tmax = fmaxf(tmax, sacc[b][r]);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    // with m_new = -inf every score is -inf and exp2(-inf - 0) = 0
    const float msub = (m_new == -INFINITY) ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sacc[b][r] - msub);
        sacc[b][r] = p;
        psum += p;
      }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {  // the running max moved for some query of the wave
#pragma unroll
      for (int nb = 0; nb < HD / 32; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[nb][r] *= alpha;
    }

    // O^T += V^T P^T over the four 16-key steps of the tile (3 products
    // each).  A lane's probabilities of step (b, hh) are those of keys
    // K0 + {0..3} and K0 + 8 + {0..3}, K0 = 32 b + 16 hh + 4 g4; its V^T
    // fragment (hd row nb * 32 + lane % 32, the same keys) comes from two
    // transposing reads: within each 16-lane group lane i receives element
    // i + 16 e of the group's 16 8-byte loads, so lane L of the group loads
    // key K0 + 8 u + L / 4 at hd c0 + 4 (L % 4) .. + 3 and lane i gets hd
    // c0 + i of keys K0 + 8 u + {0..3}.
    const int Lg = lane & 15;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint4 ph4, pl4;
        split8(make_float4(sacc[b][8 * hh + 0], sacc[b][8 * hh + 1], sacc[b][8 * hh + 2], sacc[b][8 * hh + 3]),
               make_float4(sacc[b][8 * hh + 4], sacc[b][8 * hh + 5], sacc[b][8 * hh + 6], sacc[b][8 * hh + 7]),
               ph4, pl4);
        const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, ph4);
        const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, pl4);
        const int K0 = b * 32 + 16 * hh + 4 * g4;
#pragma unroll
        for (int nb = 0; nb < HD / 32; ++nb) {
          const int c0 = nb * 32 + 16 * ((lane >> 4) & 1);
          uint2 rh[2], rl[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int key = K0 + 8 * u + (Lg >> 2), hd = c0 + 4 * (Lg & 3);
            const int addr = vswz(key, hd >> 3) * 16 + ((hd >> 2) & 1) * 8;
            rh[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t *)(Vh + addr)));
            rl[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t *)(Vl + addr)));
          }
          const bf16x8_t vh = __builtin_bit_cast(bf16x8_t, make_uint4(rh[0].x, rh[0].y, rh[1].x, rh[1].y));
          const bf16x8_t vl = __builtin_bit_cast(bf16x8_t, make_uint4(rl[0].x, rl[0].y, rl[1].x, rl[1].y));
          oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl, ph, oacc[nb], 0, 0, 0);
          oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, pl, oacc[nb], 0, 0, 0);
          oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, ph, oacc[nb], 0, 0, 0);
        }
      }
    if (t + 2 < ntile) {
      __builtin_amdgcn_s_barrier();  // every wave is done with this stage
      att_issue<G>(kA, vA, kB, vB, loA, loB, nA, kt0 + 2 * KT, kend, lds + (t & 1) * ATT_STAGE);
    }
  }
}

template <int G>
__global__ void __launch_bounds__(NTH * G) attn_split_kernel(AttnBatch bt) {
  extern __shared__ __align__(16) char lds[];  // ATT_LDS: two stages of K and V
  int z = blockIdx.z;
  const AttnArgs &a = bt.c[attn_canvas(bt, z)];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), g4 = lane >> 5;
  const int h = blockIdx.y * G + (wave >> 2);
  const int g = h / (a.Hq / a.Hkv);
  const int q = blockIdx.x * BQ + (wave & 3) * 32 + (lane & 31);
  const int nk = a.nA + a.nB;
  const int kbeg = z * a.keys_per_split;
  const int kend = min(nk, kbeg + a.keys_per_split);
  const float *Q = static_cast<const float *>(a.q);
  const int64_t qhs = a.q_hstride ? a.q_hstride : (int64_t)a.nq * HD;

  // This lane's query fragments (B operand of S^T = K Q^T), hi and lo.
  bf16x8_t qh[HD / 16], ql[HD / 16];
#pragma unroll
  for (int s = 0; s < HD / 16; ++s) {
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (q < a.nq) {
      const float4 *src = reinterpret_cast<const float4 *>(Q + (int64_t)h * qhs + (int64_t)q * HD + s * 16 + g4 * 8);
      x0 = src[0];
      x1 = src[1];
    }
    uint4 hi, lo;
    split8(x0, x1, hi, lo);
    qh[s] = __builtin_bit_cast(bf16x8_t, hi);
    ql[s] = __builtin_bit_cast(bf16x8_t, lo);
  }
  // the split fragments exist before the first DMA copy is issued, so the
  // wait for the query loads cannot land after the copies (a wait there
  // would also wait for the copies of both prologue tiles)
#pragma unroll
  for (int s = 0; s < HD / 16; ++s) asm volatile("" ::"v"(qh[s]), "v"(ql[s]));

  const int qlimit = a.causal ? a.q_pos0 + q : INT32_MAX;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[HD / 32];
#pragma unroll
  for (int nb = 0; nb < HD / 32; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[nb][r] = 0.f;
  const bf16 *kA = static_cast<const bf16 *>(a.kA), *vA = static_cast<const bf16 *>(a.vA);
  const bf16 *kB = static_cast<const bf16 *>(a.kB), *vB = static_cast<const bf16 *>(a.vB);
  const int64_t gA = (int64_t)g * a.capA * HD, gB = (int64_t)g * a.capB * HD;
  att_tiles<G>(kA + gA, vA + gA, kB ? kB + gB : kB, vB ? vB + gB : vB, (int64_t)a.Hkv * a.capA * HD,
               (int64_t)a.Hkv * a.capB * HD, a.nA, kbeg, kend, qlimit, a.causal != 0, qh, ql, lds, oacc, m_run,
               l_run);

  if (q < a.nq) {
    float *po = a.part_o + (((int64_t)z * a.Hq + h) * a.nq + q) * HD;
#pragma unroll
    for (int nb = 0; nb < HD / 32; ++nb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int hd = nb * 32 + 4 * g4 + 8 * rr;
        *reinterpret_cast<float4 *>(po + hd) =
            make_float4(oacc[nb][4 * rr], oacc[nb][4 * rr + 1], oacc[nb][4 * rr + 2], oacc[nb][4 * rr + 3]);
      }
    if (g4 == 0) {
      float *pml = a.part_ml + (((int64_t)z * a.Hq + h) * a.nq + q) * 2;
      pml[0] = m_run;
      pml[1] = l_run;
    }
  }
}

// Merge of the split-KV partial results (both dtypes); canvas blockIdx.y of
// a batch.
template <typename T>
__device__ __forceinline__ void attn_combine_body(const float *__restrict__ part_o, const float *__restrict__ part_ml,
                                                  int splits, int nq, int Hq, int hd, T *__restrict__ out,
                                                  bf16 *__restrict__ out_split, int64_t lo_off) {
  const int qh = blockIdx.x;
  const int q = qh / Hq, h = qh % Hq;
  const int e = threadIdx.x;
  // the ranges' (m, l) pairs and output columns, CH ranges' loads issued
  // together; the sums run over the ranges in order, as one at a time
  constexpr int CH = 8;
  const int64_t zs = (int64_t)Hq * nq;
  const float2 *ml = reinterpret_cast<const float2 *>(part_ml) + (int64_t)h * nq + q;
  const float *po = part_o + ((int64_t)h * nq + q) * hd + (e < hd ? e : 0);
  float M = -INFINITY;
  for (int z0 = 0; z0 < splits; z0 += CH) {
    float mv[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) mv[j] = z0 + j < splits ? ml[(z0 + j) * zs].x : -INFINITY;
#pragma unroll
    for (int j = 0; j < CH; ++j) M = fmaxf(M, mv[j]);
  }
  float num = 0.f, den = 0.f;
  for (int z0 = 0; z0 < splits; z0 += CH) {
    float2 mlv[CH];
    float ov[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const bool in = z0 + j < splits;
      mlv[j] = in ? ml[(z0 + j) * zs] : make_float2(-INFINITY, 0.f);
      ov[j] = in ? po[(z0 + j) * zs * hd] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (z0 + j >= splits) break;
      const float w = (mlv[j].x == -INFINITY) ? 0.f : exp2f(mlv[j].x - M);
      den += w * mlv[j].y;
      num += w * ov[j];
    }
  }
  if (e < hd) {
    const int64_t i = (int64_t)q * Hq * hd + (int64_t)h * hd + e;
    const float v = num / den;
    Elem<T>::store(out, i, v);
    if (out_split) {  // the output projection's operand: hi + lo terms
      const bf16 hi = f32_to_bf16(v);
      out_split[i] = hi;
      out_split[lo_off + i] = f32_to_bf16(v - bf16_to_f32(hi));
    }
  }
}

template <typename T>
__global__ void attn_combine_kernel(AttnBatch bt) {
  const AttnArgs &a = bt.c[blockIdx.y];
  attn_combine_body<T>(a.part_o, a.part_ml, a.splits, a.nq, a.Hq, HD, static_cast<T *>(a.out), a.out_split,
                       a.out_lo_off ? a.out_lo_off : (int64_t)a.nq * a.Hq * HD);
}

void attention_plan(int nq, int Hq, int nk, int *splits, int *keys_per_split) {
  const int qb = (nq + BQ - 1) / BQ;
  int want = (512 + qb * Hq - 1) / (qb * Hq);  // aim for ~2 workgroups per CU
  const int max_splits = (nk + KT - 1) / KT;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  int kps = (nk + want - 1) / want;
  kps = (kps + KT - 1) / KT * KT;
  if (kps < KT) kps = KT;
  *keys_per_split = kps;
  *splits = (nk + kps - 1) / kps;
  if (*splits < 1) *splits = 1;
}

hipError_t attention_mfma_batch(const AttnBatch &bt, hipStream_t s) {
  if (bt.B < 1 || bt.B > ES_MAX_BATCH || bt.zbase[0] != 0) return hipErrorInvalidValue;
  const AttnArgs &a0 = bt.c[0];
  for (int c = 0; c < bt.B; ++c) {  // one grid: the same queries and heads for every canvas
    const AttnArgs &a = bt.c[c];
    if (a.nq != a0.nq || a.Hq != a0.Hq || a.Hkv != a0.Hkv || a.hd != HD || a.splits < 1 ||
        bt.zbase[c + 1] - bt.zbase[c] != a.splits)
      return hipErrorInvalidValue;
  }
  static std::atomic<uint64_t> attr{0};
  if (once_per_device(attr, [] {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(attn_split_kernel<2>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, ATT_LDS);
        if (e != hipSuccess) return e;
        return hipFuncSetAttribute(reinterpret_cast<const void *>(attn_split_kernel<1>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, ATT_LDS);
      }) != hipSuccess)
    return hipErrorInvalidValue;
  const int zt = bt.zbase[bt.B];
  if ((a0.Hq / a0.Hkv) % 2 == 0)  // pairs of query heads share their KV head's tiles
    hipLaunchKernelGGL(attn_split_kernel<2>, dim3((a0.nq + BQ - 1) / BQ, a0.Hq / 2, zt), dim3(NTH * 2), ATT_LDS, s,
                       bt);
  else
    hipLaunchKernelGGL(attn_split_kernel<1>, dim3((a0.nq + BQ - 1) / BQ, a0.Hq, zt), dim3(NTH), ATT_LDS, s, bt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(attn_combine_kernel<float>, dim3(a0.nq * a0.Hq, bt.B), dim3(HD), 0, s, bt);
  return hipGetLastError();
}

hipError_t attention_mfma(const AttnArgs &a, hipStream_t s) {
  AttnBatch bt{};  // a batch of one: the same kernels, so a canvas's results do not depend on its batch
  bt.c[0] = a;
  bt.B = 1;
  bt.zbase[0] = 0;
  bt.zbase[1] = a.splits;
  return attention_mfma_batch(bt, s);
}

// ---------------------------------------------------------------------------
// fp32 path (the fp32 configuration) on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: products exact in fp32, fp32 accumulation).  One
// wave owns 16 queries of one query head and walks the keys 16 at a time:
// S = Q K^T (hd / 4 MFMAs), a running max and sum per query row, P = exp(S
// - max), then O += P V (4 MFMAs per 16 output dims).  Lane l holds rows
// 4 (l / 16) + r, r = 0..3, of a 16 x 16 result at column l % 16, so a
// query row's scores sit in the 16 lanes of one lane group and its running
// statistics are reduced there; P goes through LDS to become the A operand.
// ---------------------------------------------------------------------------
constexpr int F32_HDMAX = 128;

__global__ void __launch_bounds__(64) attn_f32_kernel(AttnArgs a) {
  __shared__ float Ps[16][17];
  const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y, g = h / (a.Hq / a.Hkv), hd = a.hd;
  const int q0 = blockIdx.x * 16;
  const int nk = a.nA + a.nB;
  const float *Q = static_cast<const float *>(a.q) + (int64_t)h * a.nq * hd;
  const float scale = rsqrtf((float)hd);
  // A operand of S = Q K^T: lane supplies Q[q0 + col][4 s + grp]
  float qa[F32_HDMAX / 4];
#pragma unroll
  for (int s4 = 0; s4 < F32_HDMAX / 4; ++s4) {
    const int k = 4 * s4 + grp;
    qa[s4] = (s4 < hd / 4 && q0 + col < a.nq) ? Q[(int64_t)(q0 + col) * hd + k] : 0.f;
  }
  auto key_row = [&](int j, const float *&kp, const float *&vp) {
    if (j < a.nA) {
      kp = static_cast<const float *>(a.kA) + ((int64_t)g * a.capA + j) * hd;
      vp = static_cast<const float *>(a.vA) + ((int64_t)g * a.capA + j) * hd;
    } else {
      kp = static_cast<const float *>(a.kB) + ((int64_t)g * a.capB + (j - a.nA)) * hd;
      vp = static_cast<const float *>(a.vB) + ((int64_t)g * a.capB + (j - a.nA)) * hd;
    }
  };
  f32x4_t o[F32_HDMAX / 16];
#pragma unroll
  for (int t = 0; t < F32_HDMAX / 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
  for (int k0 = 0; k0 < nk; k0 += 16) {
    // S block: key k0 + col for this lane's B operand
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
    {
      const int j = k0 + col;
      const float *kp = nullptr, *vp = nullptr;
      if (j < nk) key_row(j, kp, vp);
#pragma unroll
      for (int s4 = 0; s4 < F32_HDMAX / 4; ++s4) {
        if (s4 >= hd / 4) break;
        const float kb = j < nk ? kp[4 * s4 + grp] : 0.f;
        sc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[s4], kb, sc, 0, 0, 0);
      }
    }
    // scale, mask, running max/sum per query row 4 grp + r (over the 16 lanes of the group)
    float p[4], alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = q0 + 4 * grp + r, j = k0 + col;
      float v = sc[r] * scale;
      if (j >= nk || (a.causal && j > a.q_pos0 + qi)) v = -INFINITY;
      float mx = v;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m_run[r], mx);
      const float msub = m_new == -INFINITY ? 0.f : m_new;  // a row with no visible key yet
      alpha[r] = m_new == -INFINITY ? 1.f : expf(m_run[r] - m_new);
      p[r] = expf(v - msub);
      float ps = p[r];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ps += __shfl_xor(ps, off);
      l_run[r] = l_run[r] * alpha[r] + ps;
      m_run[r] = m_new;
      Ps[4 * grp + r][col] = p[r];
    }
#pragma unroll
    for (int t = 0; t < F32_HDMAX / 16; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[t][r] *= alpha[r];
    __syncthreads();
    // O += P V: A operand P[col][4 s + grp] (query col, key 4 s + grp), B operand V[key][dim 16 t + col]
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const float pa = Ps[col][4 * s4 + grp];
      const int j = k0 + 4 * s4 + grp;
      const float *kp = nullptr, *vp = nullptr;
      if (j < nk) key_row(j, kp, vp);
#pragma unroll
      for (int t = 0; t < F32_HDMAX / 16; ++t) {
        if (t >= hd / 16) break;
        const float vb = j < nk ? vp[16 * t + col] : 0.f;
        o[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, vb, o[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  float *out = static_cast<float *>(a.out);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qi = q0 + 4 * grp + r;
    if (qi >= a.nq) continue;
#pragma unroll
    for (int t = 0; t < F32_HDMAX / 16; ++t) {
      if (t >= hd / 16) break;
      out[(int64_t)qi * a.Hq * hd + (int64_t)h * hd + 16 * t + col] = o[t][r] / l_run[r];
    }
  }
}

hipError_t attention_f32(const AttnArgs &a, hipStream_t s) {
  if (a.hd > F32_HDMAX || a.hd % 16) return hipErrorInvalidValue;
  if (a.nq <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_f32_kernel, dim3((a.nq + 15) / 16, a.Hq), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace dg
