// gemm.hip -- dense contractions of the denoising step on CDNA4 matrix cores.
//
// The small contractions of the step (QKV, output projection, the
// self-conditioning FFN) on the gfx950 32x32x16 bf16 MFMA with fp32
// accumulation, plus the fp32 GEMM of the fp32 configuration on the
// 16x16x4 fp32 MFMA.  (The
// two table-streaming contractions live in estream.hip.)
// All operands are K-contiguous ("NT"): A[M][K] and B[N][K].
#include "dg_device.h"
#include "dg_kernels.h"
#include "dg_tiled.h"

namespace dg {

// EPI_ADD_ROW: columns col .. col + 3 (col % 4 == 0) of the row's table entry
__device__ __forceinline__ float4 epi_row4(const Epi &e, int row, int col) {
  int t = e.gtok[row];
  if (t >= e.gV && e.gmask) {  // [MASK] (masked sampler)
    const uint2 r = *reinterpret_cast<const uint2 *>(e.gmask + col);
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                       __uint_as_float(r.y & 0xffff0000u));
  }
  t = t < 0 ? 0 : (t >= e.gV ? e.gV - 1 : t);
  return table_get4(e.gtab, t, col);
}

__device__ __forceinline__ void epi_store(const Epi &e, int row, int col, float v) {
  const int64_t idx = (int64_t)row * e.rstride + (int64_t)(col / e.cdiv) * e.chi + (col % e.cdiv);
  switch (e.kind) {
    case EPI_GELU: v = gelu_erf(v); break;
    case EPI_ADD: v += e.resid[idx]; break;
    case EPI_ADD_ROW: {
      const float4 r = epi_row4(e, row, col & ~3);
      const int k = col & 3;
      v += k == 0 ? r.x : k == 1 ? r.y : k == 2 ? r.z : r.w;
      break;
    }
    default: break;
  }
  if (e.out_f32) {
    static_cast<float *>(e.out)[idx] = v;
  } else {
    const bf16 hi = f32_to_bf16(v);
    static_cast<bf16 *>(e.out)[idx] = hi;
    if (e.lo_off) static_cast<bf16 *>(e.out)[idx + e.lo_off] = f32_to_bf16(v - bf16_to_f32(hi));
  }
}

// ---------------------------------------------------------------------------
// Projections and the self-conditioning FFN: fp32 activations against bf16
// weights.  Each activation is carried as two bf16 terms, a = hi + lo with
// hi = bf16(a) and lo = bf16(a - hi) (16 significant bits), written in that
// form by the kernel that produces it, so one fp32 product costs two MFMAs
// and keeps ~1e-5 relative accuracy; the weights are exact in bf16.
//
// At a 256-row canvas these contractions are small (M = 256, N and K a few
// thousand), so the work is cut into 64 x 128 output tiles and, along K,
// into ranges of about 1408 (a 256 x 2816 x 2816 product: 88 tiles x 2
// ranges = 176 workgroups).  Each workgroup (8 waves, 2 x 4, wave tile 32 x
// 32: two waves per SIMD, so one's MFMAs run while the other waits on LDS
// or the barrier) streams its A rows (both bf16 terms) and B rows (bf16)
// through a 4-stage LDS ring fed by the DMA form of the vector load, 32 k
// per slice, three slices ahead of the MFMAs.  The MFMA takes the weight
// fragment first, so a lane's accumulators are one output row and runs of
// four consecutive output columns.
// ---------------------------------------------------------------------------
namespace {
constexpr int PG_BK = 32;
// default tile: rows x columns per workgroup, LDS stages; waves as a
// PG_WM x PG_WN grid over the tile
constexpr int PG_BM = 64, PG_BN = 128, PG_STAGES = 4;
constexpr int PG_WM = 2, PG_WN = 4, PG_NT = 64 * PG_WM * PG_WN;

template <int n>
__device__ __forceinline__ void pg_wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// B slice: rows x 4 chunks of 8 bf16; chunk c of row r at c ^ ((r >> 2) & 3).
// The A slice is two such arrays of BM rows, the hi terms then the lo terms.
__device__ __forceinline__ int b_slot(int row, int c) { return row * 4 + (c ^ ((row >> 2) & 3)); }

template <int BM, int BN, int STAGES>
struct PgCfg {
  static constexpr int ASLICE = BM * PG_BK * 4;  // A slice: hi and lo bf16 terms
  static constexpr int BSLICE = BN * PG_BK * 2;  // bf16 B slice
  static constexpr int STAGE = ASLICE + BSLICE;
  static constexpr int LDS = STAGES * STAGE;
  static constexpr int NW = PG_WM * PG_WN;
  static constexpr int UA = BM / 8 / NW, UB = BN / 16 / NW;  // DMA instructions per wave per slice
  static constexpr int PER = UA + UB;
  static constexpr int TM = BM / PG_WM, TN = BN / PG_WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;         // 32-wide fragments per wave
  static_assert(UA >= 1 && UB >= 1 && UA * NW * 8 == BM && UB * NW * 16 == BN && STAGES >= 3, "tile");
  static_assert(FM >= 1 && FN >= 1 && FM * 32 == TM && FN * 32 == TN, "wave tile");
  static_assert((STAGES - 2) * PER < 64, "vmcnt range");
};
}  // namespace

// Accumulates acc[i][j] (wave tile rows wm*TM + 32 i + [0, 32), columns
// wn*TN + 32 j + [0, 32)) over the slices [sb, sb + nk) of K.  The
// operands come in as restrict-qualified parameters: that tells the
// compiler the LDS reads do not depend on the DMA copies in flight (the
// s_waitcnt / s_barrier pair before each slice orders them), so it adds no
// wait of its own.
template <int BM, int BN, int STAGES>
__device__ __forceinline__ void pg_tile(const bf16 *__restrict__ A, int64_t lda, int64_t lo_off, int M, int m0,
                                        const bf16 *__restrict__ B, int K, int N, int n0, int sb, int nk, char *lds,
                                        f32x16_t (&acc)[PgCfg<BM, BN, STAGES>::FM][PgCfg<BM, BN, STAGES>::FN]) {
  using C = PgCfg<BM, BN, STAGES>;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / PG_WN, wn = wave % PG_WN, r32 = lane & 31, gq = lane >> 5;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  if (nk <= 0) return;

  // DMA sources: per slice each wave copies its share of the A slice and of
  // the B slice in instructions of 64 lanes x 16 bytes; rows past M / N read
  // a clamped valid row and only feed discarded accumulators.
  const bf16 *asrc[C::UA];
  const bf16 *bsrc[C::UB];
#pragma unroll
  for (int u = 0; u < C::UA; ++u) {
    const int p = (wave * C::UA + u) * 64 + lane;  // one instruction stays inside one term's array
    const int t = p / (BM * 4), q = p % (BM * 4);
    const int row = q >> 2, c = (q & 3) ^ ((row >> 2) & 3);
    const int gr = m0 + row < M ? m0 + row : M - 1;
    asrc[u] = A + t * lo_off + (int64_t)gr * lda + c * 8;
  }
#pragma unroll
  for (int u = 0; u < C::UB; ++u) {
    const int p = (wave * C::UB + u) * 64 + lane;
    const int row = p >> 2, c = (p & 3) ^ ((row >> 2) & 3);
    const int gn = n0 + row < N ? n0 + row : N - 1;
    bsrc[u] = B + (int64_t)gn * K + c * 8;
  }
  auto issue = [&](int slice, int stage) {
    const int k0 = (sb + min(slice, nk - 1)) * PG_BK;
    char *st = lds + stage * C::STAGE;
#pragma unroll
    for (int u = 0; u < C::UA; ++u)
      __builtin_amdgcn_global_load_lds(asrc[u] + k0, st + (wave * C::UA + u) * 1024, 16, 0, 0);
#pragma unroll
    for (int u = 0; u < C::UB; ++u)
      __builtin_amdgcn_global_load_lds(bsrc[u] + k0, st + C::ASLICE + (wave * C::UB + u) * 1024, 16, 0, 0);
  };
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t) issue(t, t);
  int stage = 0, nstage = STAGES - 1;  // stage of slice it, stage slice it + STAGES - 1 goes to
  for (int it = 0; it < nk; ++it) {
    pg_wait_vmcnt<(STAGES - 2) * C::PER>();  // this wave's copies of slice `it` landed
    __builtin_amdgcn_s_barrier();             // ... and every wave's; slice it-1 is consumed
    issue(it + STAGES - 1, nstage);
    const uint4 *sa = reinterpret_cast<const uint4 *>(lds + stage * C::STAGE);
    const uint4 *sbq = reinterpret_cast<const uint4 *>(lds + stage * C::STAGE + C::ASLICE);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // k of this lane: 16 kk + 8 gq + [0, 8) for both operands
      bf16x8_t fh[C::FM], fl[C::FM];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int arow = wm * C::TM + 32 * i + r32;
        fh[i] = __builtin_bit_cast(bf16x8_t, sa[b_slot(arow, 2 * kk + gq)]);
        fl[i] = __builtin_bit_cast(bf16x8_t, sa[BM * 4 + b_slot(arow, 2 * kk + gq)]);
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const bf16x8_t fb =
            __builtin_bit_cast(bf16x8_t, sbq[b_slot(wn * C::TN + 32 * j + r32, 2 * kk + gq)]);
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fl[i], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fh[i], acc[i][j], 0, 0, 0);
        }
      }
    }
    stage = stage + 1 == STAGES ? 0 : stage + 1;
    nstage = nstage + 1 == STAGES ? 0 : nstage + 1;
  }
  pg_wait_vmcnt<0>();  // retire the trailing (unused) prefetches
}

// Work items are (column tile p, row tile, K range), the column tiles of all
// segments numbered one after the other.  The hardware hands consecutive
// workgroups to the 8 XCDs in turn; workgroup b serves column tiles
// p = b % 8 (mod 8), so each weight tile is fetched into one XCD's L2 and
// shared there by the row tiles and K ranges that use it.
template <int BM, int BN, int STAGES>
__global__ void __launch_bounds__(PG_NT) gemm_split_kernel(SplitGemm g) {
  using C = PgCfg<BM, BN, STAGES>;
  extern __shared__ __align__(16) char lds[];
  const int M = g.M, K = g.K;
  const int mt = (M + BM - 1) / BM;
  int P = 0;
  for (int t = 0; t < g.count; ++t) P += (g.N[t] + BN - 1) / BN;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int per = mt * g.ksplit;
  if (xcd >= P || local >= ((P - xcd + 7) >> 3) * per) return;  // uniform per block
  int p = xcd + 8 * (local / per);
  const int kc = (local % per) / mt, m0 = (local % per % mt) * BM;
  int seg = 0;
  while (p >= (g.N[seg] + BN - 1) / BN) {
    p -= (g.N[seg] + BN - 1) / BN;
    ++seg;
  }
  const int N = g.N[seg], n0 = p * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / PG_WN, wn = wave % PG_WN, r32 = lane & 31, gq = lane >> 5;
  const int nsl = K / PG_BK;
  const int sb = (int)((int64_t)nsl * kc / g.ksplit), se = (int)((int64_t)nsl * (kc + 1) / g.ksplit);
  f32x16_t acc[C::FM][C::FN];
  pg_tile<BM, BN, STAGES>(g.A, g.lda, g.lo_off, M, m0, static_cast<const bf16 *>(g.B[seg]), K, N, n0, sb, se - sb, lds,
                          acc);

  // lane: output rows m0 + wm*TM + 32 i + r32; register r of fragment j is
  // column n0 + wn*TN + 32 j + 8 (r >> 2) + 4 gq + (r & 3)
  size_t base = 0;
  if (g.ksplit > 1)
    for (int t = 0; t < seg; ++t) base += (size_t)g.ksplit * M * g.N[t];
  const Epi e = g.e[seg];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int row = m0 + wm * C::TM + 32 * i + r32;
    if (row >= M) continue;
    if (g.ksplit > 1) {
      float *out = g.part + base + ((size_t)kc * M + row) * N;
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * C::TN + 32 * j + 8 * q + 4 * gq;
          if (col < N)
            *reinterpret_cast<float4 *>(out + col) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
    } else {
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int col = n0 + wn * C::TN + 32 * j + 8 * (r >> 2) + 4 * gq + (r & 3);
          if (col < N) epi_store(e, row, col, acc[i][j][r]);
        }
    }
  }
}

// Sum of the K-split partials + epilogue: one thread per 4 consecutive
// columns of one output row (N % 4 == 0).
__global__ void __launch_bounds__(256) gemm_splitk_epilogue_kernel(SplitGemm g) {
  const int seg = blockIdx.y;
  const int M = g.M, N = g.N[seg];
  const int64_t quads = (int64_t)M * N / 4;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= quads) return;
  size_t base = 0;
  for (int s = 0; s < seg; ++s) base += (size_t)g.ksplit * M * g.N[s];
  const float4 *p = reinterpret_cast<const float4 *>(g.part + base) + t;
  const int64_t stride = (int64_t)M * N / 4;
  float4 v = p[0];
  for (int z = 1; z < g.ksplit; ++z) {
    const float4 w = p[z * stride];
    v.x += w.x;
    v.y += w.y;
    v.z += w.z;
    v.w += w.w;
  }
  const int row = (int)(t * 4 / N), col = (int)(t * 4 - (int64_t)row * N);
  const Epi e = g.e[seg];
  const int64_t idx = (int64_t)row * e.rstride + (int64_t)(col / e.cdiv) * e.chi + (col % e.cdiv);
  if (e.cdiv % 4 || ((idx | e.lo_off) & 3)) {  // the four outputs are not one aligned run
    epi_store(e, row, col, v.x);
    epi_store(e, row, col + 1, v.y);
    epi_store(e, row, col + 2, v.z);
    epi_store(e, row, col + 3, v.w);
    return;
  }
  if (e.kind == EPI_GELU) {
    v = make_float4(gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w));
  } else if (e.kind == EPI_ADD) {
    const float4 r = *reinterpret_cast<const float4 *>(e.resid + idx);
    v = make_float4(v.x + r.x, v.y + r.y, v.z + r.z, v.w + r.w);
  } else if (e.kind == EPI_ADD_ROW) {
    const float4 r = epi_row4(e, row, col);
    v = make_float4(v.x + r.x, v.y + r.y, v.z + r.z, v.w + r.w);
  }
  if (e.out_f32) {
    *reinterpret_cast<float4 *>(static_cast<float *>(e.out) + idx) = v;
  } else if (e.lo_off) {
    uint2 hi, lo;
    split4(v, hi, lo);
    *reinterpret_cast<uint2 *>(static_cast<bf16 *>(e.out) + idx) = hi;
    *reinterpret_cast<uint2 *>(static_cast<bf16 *>(e.out) + idx + e.lo_off) = lo;
  } else {
    *reinterpret_cast<uint2 *>(static_cast<bf16 *>(e.out) + idx) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
}

// Split-K merge + epilogue + RMSNorm, one workgroup per output row: the row
// (N <= 4096 columns, 4 per thread per pass) stays in registers between the
// sum of squares and the normalised store.
constexpr int RN_MAXQ = 4;  // float4 per thread: N <= 256 * 4 * RN_MAXQ
__global__ void __launch_bounds__(256) gemm_splitk_norm_kernel(SplitGemm g, RowNorm rn) {
  __shared__ float sh[4];
  const int row = blockIdx.x, M = g.M, N = g.N[0];
  if (row >= M) {  // padding rows of the tiled output block
    for (int c = threadIdx.x; c < N; c += 256) rn.out_tiled[tl_index(row, c, N)] = 0;
    return;
  }
  const Epi e = g.e[0];
  const int64_t stride = (int64_t)M * N;
  const float *p0 = g.part + (int64_t)row * N;
  float4 y[RN_MAXQ];
  uint2 gw[RN_MAXQ];  // the gain's four bf16 values per float4, loaded with the partials
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < RN_MAXQ; ++k) {
    const int c = (threadIdx.x + 256 * k) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    gw[k] = make_uint2(0u, 0u);
    if (c < N) {
      gw[k] = *reinterpret_cast<const uint2 *>(rn.gain + c);
      v = *reinterpret_cast<const float4 *>(p0 + c);
      for (int z = 1; z < g.ksplit; ++z) {
        const float4 w = *reinterpret_cast<const float4 *>(p0 + z * stride + c);
        v.x += w.x;
        v.y += w.y;
        v.z += w.z;
        v.w += w.w;
      }
      float *o = static_cast<float *>(e.out) + (int64_t)row * e.rstride + c;
      if (e.kind == EPI_ADD) {
        const float4 r = *reinterpret_cast<const float4 *>(e.resid + (int64_t)row * e.rstride + c);
        v.x += r.x;
        v.y += r.y;
        v.z += r.z;
        v.w += r.w;
      } else if (e.kind == EPI_ADD_ROW) {
        const float4 r = epi_row4(e, row, c);
        v.x += r.x;
        v.y += r.y;
        v.z += r.z;
        v.w += r.w;
      }
      *reinterpret_cast<float4 *>(o) = v;
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    y[k] = v;
  }
  ss = warp_sum(ss);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  const float inv = rsqrtf(ss / (float)N + rn.eps);
#pragma unroll
  for (int k = 0; k < RN_MAXQ; ++k) {
    const int c = (threadIdx.x + 256 * k) * 4;
    if (c >= N) continue;
    const float q[4] = {y[k].x * inv * __uint_as_float(gw[k].x << 16),
                        y[k].y * inv * __uint_as_float(gw[k].x & 0xffff0000u),
                        y[k].z * inv * __uint_as_float(gw[k].y << 16),
                        y[k].w * inv * __uint_as_float(gw[k].y & 0xffff0000u)};
    if (rn.out) *reinterpret_cast<float4 *>(rn.out + (int64_t)row * N + c) = make_float4(q[0], q[1], q[2], q[3]);
    if (rn.out_split) {
      uint2 hi, lo;
      split4(make_float4(q[0], q[1], q[2], q[3]), hi, lo);
      *reinterpret_cast<uint2 *>(rn.out_split + (int64_t)row * N + c) = hi;
      *reinterpret_cast<uint2 *>(rn.out_split + (int64_t)M * N + (int64_t)row * N + c) = lo;
    }
    if (rn.out_tiled) {
      // four consecutive columns of one 8-column chunk: one 8-byte store
      *reinterpret_cast<uint2 *>(rn.out_tiled + tl_index(row, c, N)) =
          make_uint2(pack_bf16x2(q[0], q[1]), pack_bf16x2(q[2], q[3]));
    }
  }
}

// The K ranges depend on the weights' shape (K and the launch's column tiles
// P) and on the configuration's canvas length (its R = ceil(rows_ref / 64)
// row tiles), never on a launch's own row count M: a row's result then does
// not depend on how many rows are computed with it, which keeps an
// incremental prefill bitwise equal to a one-shot one and a batched step
// equal to its single steps.  At least one range per 44 slices (1408 k), and
// at least 160 / (R P) ranges, so that a launch of few tiles still spreads
// its chains over the chip; no range shorter than 4 slices.  Measured (split
// count against time, merge included): at 256 rows, 2816 x 2816 and
// 2816 -> 4096 best at 2; 1024 -> 3072 at 2 (19.2 -> 15.2 us against 1),
// 1024 -> 2048 at 2-3, 2048 -> 1024 at 4-6 (16.5 -> 13.4 us against 2),
// 1024 -> 1024 at 4-5 (18.4 -> 11.5 us); at 128 rows, 2816 x 2816 at 4-5
// (21.0 -> 16.4 us against 2), 2816 -> 4096 at 3-4 (21.7 -> 18.4 / 16.9 us),
// 2048 -> 2816 at 4 (17.0 -> 14.3 us).
int gemm_split_plan(int rows_ref, int K, const int *N, int count) {
  const int nsl = K / PG_BK;
  const int R = rows_ref > 0 ? (rows_ref + PG_BM - 1) / PG_BM : 1;
  int P = 0;
  for (int i = 0; i < count; ++i) P += (N[i] + PG_BN - 1) / PG_BN;
  int ks = (nsl + 43) / 44;
  const int want = R * (P > 0 ? P : 1);
  const int spread = (160 + want - 1) / want;
  if (spread > ks) ks = spread;
  if (ks > nsl / 4) ks = nsl / 4;
  return ks > 1 ? ks : 1;
}

size_t gemm_split_part_bytes(int M, int rows_ref, int K, const int *N, int count) {
  const int ks = gemm_split_plan(rows_ref, K, N, count);
  if (ks <= 1) return 0;
  size_t n = 0;
  for (int i = 0; i < count; ++i) n += (size_t)ks * M * N[i];
  return n * 4;
}

template <int BM, int BN, int STAGES>
hipError_t gemm_split_launch(const SplitGemm &g, hipStream_t s, bool partials_only = false) {
  using C = PgCfg<BM, BN, STAGES>;
  if (g.ksplit < 1 || (g.ksplit > 1 && !g.part) || g.K % PG_BK) return hipErrorInvalidValue;
  for (int i = 0; i < g.count; ++i)
    if (g.N[i] % 4) return hipErrorInvalidValue;
  static std::atomic<uint64_t> attr{0};
  if (once_per_device(attr, [] {
        return hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_split_kernel<BM, BN, STAGES>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
      }) != hipSuccess)
    return hipErrorInvalidValue;
  int maxN = 0, P = 0;
  for (int i = 0; i < g.count; ++i) {
    maxN = g.N[i] > maxN ? g.N[i] : maxN;
    P += (g.N[i] + BN - 1) / BN;
  }
  const int per = (g.M + BM - 1) / BM * g.ksplit;
  const int grid = 8 * ((P + 7) / 8) * per;  // XCD 0 serves the most column tiles
  hipLaunchKernelGGL((gemm_split_kernel<BM, BN, STAGES>), dim3(grid), dim3(PG_NT), C::LDS, s, g);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || g.ksplit == 1 || partials_only) return err;
  const int64_t quads = (int64_t)g.M * maxN / 4;
  hipLaunchKernelGGL(gemm_splitk_epilogue_kernel, dim3((unsigned)((quads + 255) / 256), g.count), dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t gemm_split(const SplitGemm &g, hipStream_t s) { return gemm_split_launch<PG_BM, PG_BN, PG_STAGES>(g, s); }

static hipError_t gemm_split_kernel_launch(const SplitGemm &g, hipStream_t s) {
  return gemm_split_launch<PG_BM, PG_BN, PG_STAGES>(g, s, true);
}

hipError_t gemm_split_norm(const SplitGemm &g, const RowNorm &rn, hipStream_t s) {
  const Epi &e = g.e[0];
  if (g.count != 1 || g.ksplit < 2 || !g.part || !e.out_f32 || e.cdiv < g.N[0] || g.N[0] % 4 ||
      g.N[0] > 256 * 4 * RN_MAXQ || (e.kind != EPI_STORE && e.kind != EPI_ADD && e.kind != EPI_ADD_ROW) ||
      e.rstride % 4 || (e.kind == EPI_ADD_ROW && (e.gtab.d != g.N[0] || !e.gtab.p)) ||
      (rn.out_tiled && g.N[0] % TL_K))
    return hipErrorInvalidValue;
  hipError_t err = gemm_split_kernel_launch(g, s);  // partials only; the merge applies the epilogue
  if (err != hipSuccess) return err;
  const int rows = rn.out_tiled ? (g.M + TL_ROWS - 1) / TL_ROWS * TL_ROWS : g.M;
  hipLaunchKernelGGL(gemm_splitk_norm_kernel, dim3(rows), dim3(256), 0, s, g, rn);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 GEMM (the fp32 configuration) on the fp32 matrix cores: every product
// exact in fp32, accumulated in fp32 by v_mfma_f32_16x16x4_f32.  A
// workgroup of 4 waves owns a 32 x 32 output tile (a 16 x 16 tile per wave);
// K is staged through LDS 32 at a time.  Generic strides on both operands
// (the self-conditioning contraction reads E as its transpose).
// MFMA lane layout (16x16x4): lane l supplies A[l % 16][l / 16] and
// B^T[l % 16][l / 16] and holds D[4 (l / 16) + r][l % 16], r = 0..3.
// ---------------------------------------------------------------------------
namespace {
constexpr int F32_BM = 32, F32_BN = 32, F32_BK = 32;
}

__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmShapeF32 g, Epi e) {
  __shared__ float sa[F32_BM][F32_BK + 1];
  __shared__ float sb[F32_BN][F32_BK + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * F32_BM, n0 = blockIdx.x * F32_BN;
  const int wm = (wave >> 1) * 16, wn = (wave & 1) * 16;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < g.K; k0 += F32_BK) {
    for (int t = tid; t < F32_BM * F32_BK; t += 256) {
      const int r = t / F32_BK, k = t % F32_BK, gk = k0 + k;
      float va = 0.f, vb = 0.f;
      if (m0 + r < g.M && gk < g.K) {
        va = g.A[(int64_t)(m0 + r) * g.sam + (int64_t)gk * g.sak];
        if (g.a_scale) va *= g.a_scale[(int64_t)(m0 + r) * g.a_scale_ld + (gk >> 6)];
      }
      if (n0 + r < g.N && gk < g.K) vb = g.B[(int64_t)(n0 + r) * g.sbn + (int64_t)gk * g.sbk];
      sa[r][k] = va;
      sb[r][k] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F32_BK; kk += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[wm + (lane & 15)][kk + (lane >> 4)],
                                                 sb[wn + (lane & 15)][kk + (lane >> 4)], acc, 0, 0, 0);
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + wm + 4 * (lane >> 4) + r, n = n0 + wn + (lane & 15);
    if (m < g.M && n < g.N) epi_store(e, m, n, acc[r]);
  }
}

hipError_t gemm_f32(const GemmShapeF32 &g, const Epi &e, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  dim3 grid((g.N + F32_BN - 1) / F32_BN, (g.M + F32_BM - 1) / F32_BM, 1);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, g, e);
  return hipGetLastError();
}

}  // namespace dg
