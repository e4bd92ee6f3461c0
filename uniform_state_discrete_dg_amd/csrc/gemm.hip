// gemm.hip -- dense contractions of the denoising step on CDNA4 matrix cores.
//
// The small contractions of the step (QKV, output projection, the
// self-conditioning FFN) on the gfx950 32x32x16 bf16 MFMA with fp32
// accumulation, plus the fp32 SIMT GEMM of the fp32 configuration.  (The
// two table-streaming contractions live in estream.hip.)
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
        if (g.a_scale) v *= g.a_scale[(int64_t)am * g.a_scale_ld + (ak >> 6)];
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
