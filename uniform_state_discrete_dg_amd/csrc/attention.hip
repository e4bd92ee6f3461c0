// attention.hip -- attention of canvas (or prompt) queries over the prefix KV
// cache and the canvas, head_dim 128, on CDNA4 matrix cores.
//
// Denoise mode reads every key (bidirectional, no mask); prefill mode masks
// keys beyond each query's absolute position (causal).  Keys come from two
// segments, the committed cache [0, nA) and the step's own canvas keys
// [0, nB), so the cache is never written by a denoising step.
//
// Queries, keys and values are fp32 in memory.  While they are staged, each
// value is split into two bf16 terms (hi + lo), and every product of two
// split operands is formed from three bf16 MFMAs (hi*hi + hi*lo + lo*hi),
// which keeps the scores and the output within ~1e-5 of fp32.
//
// Flash-style: a workgroup owns 128 queries of G query heads that share one
// KV head (G = 2 when the group size is even, else 1; 4 waves of 32
// queries per head) and a contiguous range of keys (split-KV, partial
// results merged by a second kernel), so each 64-key tile of K and V is
// staged through LDS once for G heads.  The wave
// computes S^T = K Q^T so that each lane ends up holding one query's scores,
// keeps the running max / sum per lane, and computes O^T = V^T P^T with the
// probabilities taken straight from registers; V is transposed while it is
// staged into LDS.  Grouped-query attention maps query head h to KV head
// h / (Hq / Hkv).
#include "dg_device.h"
#include "dg_kernels.h"

namespace dg {

namespace {
constexpr int HD = 128;
constexpr int BQ = 128;   // queries per workgroup
constexpr int KT = 64;    // keys per tile
constexpr int NTH = 256;  // 4 waves
constexpr float LOG2E = 1.4426950408889634f;
}  // namespace

__device__ __forceinline__ int kswz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }
// V^T in LDS: [128 hd][8 groups of 8 keys], group u of row hd at u ^ ((hd >> 1) & 7),
// so the 16 rows a fragment read touches at one group fall on distinct banks.
__device__ __forceinline__ int vswz(int hd, int u) { return hd * 8 + (u ^ ((hd >> 1) & 7)); }

// The canvas of grid z-slice `z` of a batch launch (canvas c owns z-slices
// zbase[c] .. zbase[c + 1] - 1: its own split plan) and that slice's split.
__device__ __forceinline__ int attn_canvas(const AttnBatch &bt, int &z) {
  int c = 0;
  while (c + 1 < bt.B && z >= bt.zbase[c + 1]) ++c;
  z -= bt.zbase[c];
  return c;
}

template <int G>
__global__ void __launch_bounds__(NTH * G) attn_split_kernel(AttnBatch bt) {
  __shared__ uint4 Ks[2][KT * HD / 8];     // hi, lo: [64 keys][16 chunks of 8]
  __shared__ uint4 Vt[2][HD * KT / 8];     // hi, lo: [128 hd][8 chunks of 8 keys]

  int z = blockIdx.z;
  const AttnArgs &a = bt.c[attn_canvas(bt, z)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 5;
  const int h = blockIdx.y * G + (wave >> 2);
  const int g = h / (a.Hq / a.Hkv);
  const int q = blockIdx.x * BQ + (wave & 3) * 32 + (lane & 31);
  const int nk = a.nA + a.nB;
  const int kbeg = z * a.keys_per_split;
  const int kend = min(nk, kbeg + a.keys_per_split);
  const float *Q = static_cast<const float *>(a.q);
  const int64_t qhs = a.q_hstride ? a.q_hstride : (int64_t)a.nq * HD;
  const float *kA = static_cast<const float *>(a.kA), *vA = static_cast<const float *>(a.vA);
  const float *kB = static_cast<const float *>(a.kB), *vB = static_cast<const float *>(a.vB);

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

  const float sc = rsqrtf((float)HD) * LOG2E;
  const int qlimit = a.causal ? a.q_pos0 + q : INT32_MAX;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[HD / 32];
#pragma unroll
  for (int nb = 0; nb < HD / 32; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[nb][r] = 0.f;

  // A tile is 64 keys x 128.  K: 1024 chunks of 8 floats, 4 / G per thread
  // (thread -> key idx / 16, chunk idx % 16).  V: thread -> DV = 4 / G dims
  // (DV (tid % (32 G)) ..) x the 8 keys of group u = tid / (32 G), which it
  // writes as 8-key vectors of V^T.  Group u holds, in MFMA k order, the keys
  // that a lane's probabilities cover in the P^T fragment: with c = u / 2 and
  // g = u % 2, keys 16 c + 4 g + {0..3} then 16 c + 8 + 4 g + {0..3}.
  constexpr int KPT = 4 / G, DV = 4 / G;
  typedef float fv_t __attribute__((ext_vector_type(DV)));
  float4 rk[KPT][2];
  fv_t rv[8];
  auto kv_src = [&](int kabs, int col, const float *&kp, const float *&vp, int64_t &off) {
    if (kabs < a.nA) {
      off = ((int64_t)g * a.capA + kabs) * HD + col;
      kp = kA;
      vp = vA;
    } else {
      off = ((int64_t)g * a.capB + (kabs - a.nA)) * HD + col;
      kp = kB;
      vp = vB;
    }
  };
  auto load = [&](int kt0) {
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
      const int idx = tid + t * NTH * G;
      const int key = idx >> 4, ch = idx & 15;
      const int kabs = kt0 + key;
      float4 k0 = make_float4(0.f, 0.f, 0.f, 0.f), k1 = k0;
      if (kabs < kend) {
        int64_t off;
        const float *kp, *vp;
        kv_src(kabs, ch * 8, kp, vp, off);
        k0 = *reinterpret_cast<const float4 *>(kp + off);
        k1 = *reinterpret_cast<const float4 *>(kp + off + 4);
      }
      rk[t][0] = k0;
      rk[t][1] = k1;
    }
    const int dv = tid & (32 * G - 1), kg = tid / (32 * G);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kabs = kt0 + 16 * (kg >> 1) + 4 * (kg & 1) + (j & 3) + 8 * (j >> 2);
      fv_t v = {};
      if (kabs < kend) {
        int64_t off;
        const float *kp, *vp;
        kv_src(kabs, dv * DV, kp, vp, off);
        v = *reinterpret_cast<const fv_t *>(vp + off);
      }
      rv[j] = v;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
      const int idx = tid + t * NTH * G;
      const int key = idx >> 4, ch = idx & 15;
      uint4 hi, lo;
      split8(rk[t][0], rk[t][1], hi, lo);
      Ks[0][kswz(key, ch)] = hi;
      Ks[1][kswz(key, ch)] = lo;
    }
    const int dv = tid & (32 * G - 1), kg = tid / (32 * G);
#pragma unroll
    for (int e = 0; e < DV; ++e) {
      const float x[8] = {rv[0][e], rv[1][e], rv[2][e], rv[3][e], rv[4][e], rv[5][e], rv[6][e], rv[7][e]};
      uint4 hi, lo;
      split8(make_float4(x[0], x[1], x[2], x[3]), make_float4(x[4], x[5], x[6], x[7]), hi, lo);
      Vt[0][vswz(dv * DV + e, kg)] = hi;
      Vt[1][vswz(dv * DV + e, kg)] = lo;
    }
  };

  if (kbeg < kend) {
    load(kbeg);
    store();
    __syncthreads();
  }
  for (int kt0 = kbeg; kt0 < kend; kt0 += KT) {
    const bool more = kt0 + KT < kend;
    if (more) load(kt0 + KT);

    // S^T for two 32-key blocks: K_hi Q_hi + K_lo Q_hi + K_hi Q_lo.
    f32x16_t sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[b][r] = 0.f;
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) {
        const int li = kswz(b * 32 + (lane & 31), 2 * s + g4);
        const bf16x8_t kh = __builtin_bit_cast(bf16x8_t, Ks[0][li]);
        const bf16x8_t kl = __builtin_bit_cast(bf16x8_t, Ks[1][li]);
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qh[s], sacc[b], 0, 0, 0);
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, ql[s], sacc[b], 0, 0, 0);
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qh[s], sacc[b], 0, 0, 0);
      }
    }
    // mask (only a partial tile or causal mode needs it), scale, running max
    float tmax = -INFINITY;
    if (kt0 + KT > kend || a.causal) {
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

    // O^T += V^T P^T over the four 16-key steps of the tile (3 products each).
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
        const int u = 4 * b + 2 * hh + g4;  // the lane's 8 keys of this 16-key step
#pragma unroll
        for (int nb = 0; nb < HD / 32; ++nb) {
          const int hd = nb * 32 + (lane & 31);
          const bf16x8_t vh = __builtin_bit_cast(bf16x8_t, Vt[0][vswz(hd, u)]);
          const bf16x8_t vl = __builtin_bit_cast(bf16x8_t, Vt[1][vswz(hd, u)]);
          oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl, ph, oacc[nb], 0, 0, 0);
          oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, pl, oacc[nb], 0, 0, 0);
          oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, ph, oacc[nb], 0, 0, 0);
        }
      }
    __syncthreads();
    if (more) {
      store();
      __syncthreads();
    }
  }

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
  float M = -INFINITY;
  for (int z = 0; z < splits; ++z) M = fmaxf(M, part_ml[(((int64_t)z * Hq + h) * nq + q) * 2]);
  float num = 0.f, den = 0.f;
  for (int z = 0; z < splits; ++z) {
    const float m = part_ml[(((int64_t)z * Hq + h) * nq + q) * 2];
    const float l = part_ml[(((int64_t)z * Hq + h) * nq + q) * 2 + 1];
    const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
    den += w * l;
    if (e < hd) num += w * part_o[(((int64_t)z * Hq + h) * nq + q) * hd + e];
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
  const int zt = bt.zbase[bt.B];
  if ((a0.Hq / a0.Hkv) % 2 == 0)  // pairs of query heads share their KV head's tiles
    hipLaunchKernelGGL(attn_split_kernel<2>, dim3((a0.nq + BQ - 1) / BQ, a0.Hq / 2, zt), dim3(NTH * 2), 0, s, bt);
  else
    hipLaunchKernelGGL(attn_split_kernel<1>, dim3((a0.nq + BQ - 1) / BQ, a0.Hq, zt), dim3(NTH), 0, s, bt);
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
