// gemm.hip -- dense contractions of the denoising step on CDNA4 matrix cores.
//
// One block-tile engine (bf16 operands, fp32 accumulation, the gfx950
// 32x32x16 MFMA) serves every contraction of the step:
//   * the tied LM head z = RMSNorm(h1) E^T with a fused softmax/entropy
//     epilogue (per 256-column tile: max, argmax, sum of exp, sum of
//     exp * shifted logit; the probability numerators are written once in
//     bf16 and the logits never reach memory),
//   * the self-conditioning contraction S = p_prev E (K = V, split over V),
//   * the small projections (QKV, output, self-conditioning FFN).
// All operands are K-contiguous ("NT"): A[M][K] and B[N][K].  K is staged
// through LDS in 64-wide slices (two buffers, global loads for slice k+1 in
// flight while slice k feeds the MFMAs); 16-byte chunks of each LDS row are
// XOR-swizzled by the row index so the 32 rows a fragment read touches fall
// in distinct banks.
#include "dg_device.h"
#include "dg_kernels.h"

namespace dg {

template <int BM_, int BN_, int WGM_, int WGN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int BK = 64;
  static constexpr int NT = WGM * WGN * 64;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_VEC = BM * BK / 8;  // 16-byte vectors per slice
  static constexpr int B_VEC = BN * BK / 8;
  static constexpr int A_PT = A_VEC / NT, B_PT = B_VEC / NT;
  static constexpr int LDS_VEC = 2 * (A_VEC + B_VEC);
  static_assert(A_VEC % NT == 0 && B_VEC % NT == 0, "tile/thread mismatch");
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float s) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16) * s;
    const float hi = __uint_as_float(w[i] & 0xffff0000u) * s;
    w[i] = pack_bf16x2(lo, hi);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Accumulates the (m0, n0) block tile over K slices [kb, ke) (multiples of 64).
template <class C, bool SCALE_A>
__device__ __forceinline__ void mfma_tile(const bf16 *__restrict__ A, int64_t lda, int M, int m0,
                                          const bf16 *__restrict__ B, int64_t ldb, int N, int n0,
                                          int kb, int ke, const float *__restrict__ a_scale,
                                          int64_t a_scale_ld, uint4 *lds,
                                          f32x16_t (&acc)[C::FM][C::FN]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  uint4 *ldsA = lds;                   // [2][A_VEC]
  uint4 *ldsB = lds + 2 * C::A_VEC;    // [2][B_VEC]

#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[C::A_PT], rb[C::B_PT];
  auto load = [&](int k0) {
#pragma unroll
    for (int t = 0; t < C::A_PT; ++t) {
      const int idx = tid + t * C::NT;
      const int row = idx >> 3, ch = idx & 7;
      const int gr = m0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gr < M) {
        v = *reinterpret_cast<const uint4 *>(A + (int64_t)gr * lda + k0 + ch * 8);
        if (SCALE_A) v = scale_bf16x8(v, a_scale[(int64_t)gr * a_scale_ld + (k0 >> 8)]);
      }
      ra[t] = v;
    }
#pragma unroll
    for (int t = 0; t < C::B_PT; ++t) {
      const int idx = tid + t * C::NT;
      const int row = idx >> 3, ch = idx & 7;
      const int gn = n0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gn < N) v = *reinterpret_cast<const uint4 *>(B + (int64_t)gn * ldb + k0 + ch * 8);
      rb[t] = v;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int t = 0; t < C::A_PT; ++t) {
      const int idx = tid + t * C::NT;
      ldsA[buf * C::A_VEC + swz(idx >> 3, idx & 7)] = ra[t];
    }
#pragma unroll
    for (int t = 0; t < C::B_PT; ++t) {
      const int idx = tid + t * C::NT;
      ldsB[buf * C::B_VEC + swz(idx >> 3, idx & 7)] = rb[t];
    }
  };

  const int nk = (ke - kb) / C::BK;
  if (nk <= 0) return;
  load(kb);
  store(0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) load(kb + (it + 1) * C::BK);
#pragma unroll
    for (int kk = 0; kk < C::BK / 16; ++kk) {
      bf16x8_t fa[C::FM], fb[C::FN];
      const int ch = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::WM + i * 32 + (lane & 31);
        fa[i] = __builtin_bit_cast(bf16x8_t, ldsA[buf * C::A_VEC + swz(row, ch)]);
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WN + j * 32 + (lane & 31);
        fb[j] = __builtin_bit_cast(bf16x8_t, ldsB[buf * C::B_VEC + swz(row, ch)]);
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (it + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
}

// Row/column of accumulator element r of lane `lane` in fragment (i, j),
// relative to the wave tile origin (32x32 MFMA output layout).
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
}
__device__ __forceinline__ int acc_col(int j, int lane) { return j * 32 + (lane & 31); }

__device__ __forceinline__ void epi_store(const Epi &e, int row, int col, float v) {
  const int64_t idx = (int64_t)row * e.rstride + (int64_t)(col / e.cdiv) * e.chi + (col % e.cdiv);
  switch (e.kind) {
    case EPI_GELU: v = gelu_erf(v); break;
    case EPI_ADD: v += e.resid[idx]; break;
    default: break;
  }
  if (e.kind == EPI_PARTIAL) {
    static_cast<float *>(e.out)[(int64_t)blockIdx.z * e.split_stride + idx] = v;
  } else if (e.out_f32) {
    static_cast<float *>(e.out)[idx] = v;
  } else {
    static_cast<bf16 *>(e.out)[idx] = f32_to_bf16(v);
  }
}

// ---------------------------------------------------------------------------
// Projections and the self-conditioning FFN: fp32 activations against bf16
// weights.  Each activation is split into two bf16 terms, a = hi + lo with
// hi = bf16(a) and lo = bf16(a - hi) (16 significant bits), so one fp32
// product costs two MFMAs and keeps ~1e-5 relative accuracy; the weights
// are exact in bf16.  64x64 tiles, 4 waves; up to three weight matrices
// (Q, K, V) share the activation operand in one launch (blockIdx.z).
// ---------------------------------------------------------------------------
using SmallTile = TileCfg<64, 64, 2, 2>;

template <class C>
__global__ void __launch_bounds__(C::NT) gemm_split_kernel(SplitGemm g) {
  __shared__ uint4 lds[2 * (2 * C::A_VEC + C::B_VEC)];
  const int seg = blockIdx.z;
  const bf16 *__restrict__ B = static_cast<const bf16 *>(g.B[seg]);
  const int N = g.N[seg];
  const int m0 = blockIdx.y * C::BM, n0 = blockIdx.x * C::BN;
  if (n0 >= N) return;  // uniform per block
  const int M = g.M, K = g.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  constexpr int STAGE = 2 * C::A_VEC + C::B_VEC;

  f32x16_t acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  float4 ra[C::A_PT][2];
  uint4 rb[C::B_PT];
  auto load = [&](int k0) {
#pragma unroll
    for (int t = 0; t < C::A_PT; ++t) {
      const int idx = tid + t * C::NT;
      const int row = idx >> 3, ch = idx & 7;
      const int gr = m0 + row;
      float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
      if (gr < M) {
        const float4 *src = reinterpret_cast<const float4 *>(g.A + (int64_t)gr * g.lda + k0 + ch * 8);
        a0 = src[0];
        a1 = src[1];
      }
      ra[t][0] = a0;
      ra[t][1] = a1;
    }
#pragma unroll
    for (int t = 0; t < C::B_PT; ++t) {
      const int idx = tid + t * C::NT;
      const int row = idx >> 3, ch = idx & 7;
      const int gn = n0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gn < N) v = *reinterpret_cast<const uint4 *>(B + (int64_t)gn * K + k0 + ch * 8);
      rb[t] = v;
    }
  };
  auto store = [&](int buf) {
    uint4 *st = lds + buf * STAGE;
#pragma unroll
    for (int t = 0; t < C::A_PT; ++t) {
      const int idx = tid + t * C::NT;
      uint4 hi, lo;
      split8(ra[t][0], ra[t][1], hi, lo);
      st[swz(idx >> 3, idx & 7)] = hi;
      st[C::A_VEC + swz(idx >> 3, idx & 7)] = lo;
    }
#pragma unroll
    for (int t = 0; t < C::B_PT; ++t) {
      const int idx = tid + t * C::NT;
      st[2 * C::A_VEC + swz(idx >> 3, idx & 7)] = rb[t];
    }
  };

  const int nk = K / C::BK;
  load(0);
  store(0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) load((it + 1) * C::BK);
    const uint4 *st = lds + buf * STAGE;
#pragma unroll
    for (int kk = 0; kk < C::BK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8_t fh[C::FM], fl[C::FM], fb[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::WM + i * 32 + (lane & 31);
        fh[i] = __builtin_bit_cast(bf16x8_t, st[swz(row, ch)]);
        fl[i] = __builtin_bit_cast(bf16x8_t, st[C::A_VEC + swz(row, ch)]);
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WN + j * 32 + (lane & 31);
        fb[j] = __builtin_bit_cast(bf16x8_t, st[2 * C::A_VEC + swz(row, ch)]);
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl[i], fb[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }
    if (it + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  const Epi e = g.e[seg];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * C::WM + acc_row(i, r, lane);
        const int col = n0 + wn * C::WN + acc_col(j, lane);
        if (row < M && col < N) epi_store(e, row, col, acc[i][j][r]);
      }
}

hipError_t gemm_split(const SplitGemm &g, hipStream_t s) {
  using C = SmallTile;
  int maxN = 0;
  for (int i = 0; i < g.count; ++i) maxN = g.N[i] > maxN ? g.N[i] : maxN;
  dim3 grid((maxN + C::BN - 1) / C::BN, (g.M + C::BM - 1) / C::BM, g.count);
  hipLaunchKernelGGL(gemm_split_kernel<C>, grid, dim3(C::NT), 0, s, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Self-conditioning contraction: 256 (or 128) canvas rows x 256 columns of d
// per workgroup, K = V split over blockIdx.z.  Each probability numerator
// is multiplied by its (row, tile) normaliser while staged into LDS.
// ---------------------------------------------------------------------------
using BigTile256 = TileCfg<256, 256, 4, 2>;
using BigTile128 = TileCfg<128, 256, 2, 4>;

template <class C>
__global__ void __launch_bounds__(C::NT) selfcond_kernel(GemmShape g, float *part, int ksplit) {
  __shared__ uint4 lds[C::LDS_VEC];
  const int m0 = blockIdx.y * C::BM, n0 = blockIdx.x * C::BN;
  const int nslices = g.K / 64;
  const int z = blockIdx.z;
  const int kb = (int)((int64_t)nslices * z / ksplit) * 64;
  const int ke = (int)((int64_t)nslices * (z + 1) / ksplit) * 64;
  f32x16_t acc[C::FM][C::FN];
  if (g.a_scale)
    mfma_tile<C, true>(static_cast<const bf16 *>(g.A), g.lda, g.M, m0,
                       static_cast<const bf16 *>(g.B), g.ldb, g.N, n0, kb, ke, g.a_scale,
                       g.a_scale_ld, lds, acc);
  else
    mfma_tile<C, false>(static_cast<const bf16 *>(g.A), g.lda, g.M, m0,
                        static_cast<const bf16 *>(g.B), g.ldb, g.N, n0, kb, ke, nullptr, 0, lds,
                        acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  float *out = part + (int64_t)z * g.M * g.N;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * C::WM + acc_row(i, r, lane);
        const int col = n0 + wn * C::WN + acc_col(j, lane);
        if (row < g.M && col < g.N) out[(int64_t)row * g.N + col] = acc[i][j][r];
      }
}

hipError_t selfcond_bf16(const GemmShape &g, float *partials, int ksplit, hipStream_t s) {
  if (g.M <= 128) {
    using C = BigTile128;
    dim3 grid((g.N + C::BN - 1) / C::BN, (g.M + C::BM - 1) / C::BM, ksplit);
    hipLaunchKernelGGL(selfcond_kernel<C>, grid, dim3(C::NT), 0, s, g, partials, ksplit);
  } else {
    using C = BigTile256;
    dim3 grid((g.N + C::BN - 1) / C::BN, (g.M + C::BM - 1) / C::BM, ksplit);
    hipLaunchKernelGGL(selfcond_kernel<C>, grid, dim3(C::NT), 0, s, g, partials, ksplit);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LM head with the softmax/entropy epilogue.
// ---------------------------------------------------------------------------
template <class C>
__global__ void __launch_bounds__(C::NT) lm_head_kernel(const bf16 *__restrict__ A, int M, int K,
                                                         const bf16 *__restrict__ E, int V,
                                                         float inv_T, bf16 *__restrict__ probs,
                                                         float4 *__restrict__ tile_stats,
                                                         float *__restrict__ logits) {
  __shared__ uint4 lds[C::LDS_VEC];
  __shared__ float red_v[C::WGN][C::BM];
  __shared__ int red_i[C::WGN][C::BM];
  __shared__ float red_l[C::WGN][C::BM];
  __shared__ float red_s[C::WGN][C::BM];
  __shared__ float row_m[C::BM];  // tile max of y for each row

  const int m0 = blockIdx.y * C::BM;
  const int tile = blockIdx.x;
  const int n0 = tile * C::BN;
  f32x16_t acc[C::FM][C::FN];
  mfma_tile<C, false>(A, K, M, m0, E, K, V, n0, 0, K, nullptr, 0, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int ntiles = V / C::BN;

  // 1. per-row max of z and its lowest column index within the wave.
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float best = acc[i][0][r];
      int bcol = acc_col(0, lane);
#pragma unroll
      for (int j = 1; j < C::FN; ++j) {
        const float v = acc[i][j][r];
        if (v > best) {
          best = v;
          bcol = acc_col(j, lane);
        }
      }
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o);
        const int oc = __shfl_xor(bcol, o);
        if (ov > best || (ov == best && oc < bcol)) {
          best = ov;
          bcol = oc;
        }
      }
      if ((lane & 31) == 0) {
        const int row = wm * C::WM + acc_row(i, r, lane);
        red_v[wn][row] = best;
        red_i[wn][row] = wn * C::WN + bcol;
      }
    }
  __syncthreads();
  if (threadIdx.x < C::BM) {
    const int row = threadIdx.x;
    float best = red_v[0][row];
    int bcol = red_i[0][row];
#pragma unroll
    for (int w = 1; w < C::WGN; ++w) {
      const float v = red_v[w][row];
      const int c = red_i[w][row];
      if (v > best || (v == best && c < bcol)) {
        best = v;
        bcol = c;
      }
    }
    red_v[0][row] = best;
    red_i[0][row] = bcol;
    row_m[row] = best * inv_T;
  }
  __syncthreads();

  // 2. exp(y - m), the numerators (bf16), and the two sums per row.
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lrow = wm * C::WM + acc_row(i, r, lane);
      const int grow = m0 + lrow;
      const float m = row_m[lrow];
      float l = 0.f, sacc = 0.f;
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const float z = acc[i][j][r];
        const float t = z * inv_T - m;
        const float ev = exp2f(t * 1.4426950408889634f);
        l += ev;
        sacc += ev * t;
        const int gcol = n0 + wn * C::WN + acc_col(j, lane);
        if (grow < M) {
          probs[(int64_t)grow * V + gcol] = f32_to_bf16(ev);
          if (logits) logits[(int64_t)grow * V + gcol] = z;
        }
      }
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) {
        l += __shfl_xor(l, o);
        sacc += __shfl_xor(sacc, o);
      }
      if ((lane & 31) == 0) {
        red_l[wn][lrow] = l;
        red_s[wn][lrow] = sacc;
      }
    }
  __syncthreads();
  if (threadIdx.x < C::BM) {
    const int row = threadIdx.x;
    const int grow = m0 + row;
    float l = red_l[0][row], sacc = red_s[0][row];
#pragma unroll
    for (int w = 1; w < C::WGN; ++w) {
      l += red_l[w][row];
      sacc += red_s[w][row];
    }
    if (grow < M)
      tile_stats[(int64_t)grow * ntiles + tile] =
          make_float4(red_v[0][row], l, sacc, __int_as_float(n0 + red_i[0][row]));
  }
}

hipError_t lm_head_bf16(const uint16_t *A, int M, int K, const uint16_t *E, int V, float inv_T,
                        uint16_t *probs, float4 *tile_stats, float *logits_dump, hipStream_t s) {
  if (M <= 128) {
    using C = BigTile128;
    dim3 grid(V / C::BN, (M + C::BM - 1) / C::BM);
    hipLaunchKernelGGL(lm_head_kernel<C>, grid, dim3(C::NT), 0, s, A, M, K, E, V, inv_T, probs,
                       tile_stats, logits_dump);
  } else {
    using C = BigTile256;
    dim3 grid(V / C::BN, (M + C::BM - 1) / C::BM);
    hipLaunchKernelGGL(lm_head_kernel<C>, grid, dim3(C::NT), 0, s, A, M, K, E, V, inv_T, probs,
                       tile_stats, logits_dump);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 SIMT GEMM (the fp32 configuration): 16x16 outputs per workgroup,
// K staged through LDS in slices of 16, generic strides on both operands.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmShapeF32 g, Epi e) {
  __shared__ float sa[16][17];
  __shared__ float sb[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m = blockIdx.y * 16 + ty, n = blockIdx.x * 16 + tx;
  float acc = 0.f;
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    {
      const int am = blockIdx.y * 16 + ty, ak = k0 + tx;
      float v = 0.f;
      if (am < g.M && ak < g.K) {
        v = g.A[(int64_t)am * g.sam + (int64_t)ak * g.sak];
        if (g.a_scale) v *= g.a_scale[(int64_t)am * g.a_scale_ld + (ak >> 8)];
      }
      sa[ty][tx] = v;
      const int bn = blockIdx.x * 16 + ty, bk = k0 + tx;
      sb[ty][tx] = (bn < g.N && bk < g.K) ? g.B[(int64_t)bn * g.sbn + (int64_t)bk * g.sbk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(sa[ty][kk], sb[tx][kk], acc);
    __syncthreads();
  }
  if (m < g.M && n < g.N) epi_store(e, m, n, acc);
}

hipError_t gemm_f32(const GemmShapeF32 &g, const Epi &e, hipStream_t s) {
  dim3 grid((g.N + 15) / 16, (g.M + 15) / 16, 1);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, g, e);
  return hipGetLastError();
}

}  // namespace dg
