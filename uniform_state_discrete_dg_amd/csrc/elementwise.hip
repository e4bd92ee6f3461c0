// elementwise.hip -- the small kernels around the contractions: embedding
// gather, RMSNorm, split-K merge, the one-time E transpose, per-tile softmax
// statistics for the fp32 path, and the per-row entropy/argmax combine.
// Every reduction is a fixed tree, so results do not depend on timing.
#include "dg_device.h"
#include "dg_kernels.h"
#include "dg_tiled.h"

namespace dg {

namespace {
constexpr float LOG2E = 1.4426950408889634f;
constexpr int TILE = 64;  // vocabulary columns per softmax-statistics tile
}  // namespace

// Block-wide (256 threads) sum with a fixed reduction tree.
__device__ __forceinline__ float block_sum256(float v, float *sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
#pragma unroll
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  const float r = sh[0];
  __syncthreads();
  return r;
}

// [P3] §5.1: the token embeddings of the canvas (rows of the tied table);
// under the masked sampler ([P3] §3.1) ids >= V are [MASK] and read mask_row.
template <typename T>
__device__ __forceinline__ const T *embed_row(const T *E, int t, int d, int V, const T *mask_row) {
  if (t >= V && mask_row) return mask_row;
  t = t < 0 ? 0 : (t >= V ? V - 1 : t);
  return E + (int64_t)t * d;
}

template <typename T>
__global__ void gather_kernel(const T *__restrict__ E, const int32_t *__restrict__ tokens, int d, int V,
                              const T *__restrict__ mask_row, float *__restrict__ out) {
  const int i = blockIdx.x;
  const T *row = embed_row(E, tokens[i], d, V, mask_row);
  for (int k = threadIdx.x; k < d; k += blockDim.x) out[(int64_t)i * d + k] = Elem<T>::load(row, k);
}

hipError_t gather_rows(const float *E, const int32_t *tokens, int n, int d, int V, const float *mask_row,
                       float *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel<float>, dim3(n), dim3(256), 0, s, E, tokens, d, V, mask_row, out);
  return hipGetLastError();
}

// Rows of the packed table (any form), four values per thread.
__global__ void gather_table_kernel(PackedTable E, const int32_t *__restrict__ tokens, int V,
                                    const bf16 *__restrict__ mask_row, float *__restrict__ out) {
  const int i = blockIdx.x, d = E.d;
  int t = tokens[i];
  const bool masked = t >= V && mask_row;
  t = t < 0 ? 0 : (t >= V ? V - 1 : t);
  float4 *dst = reinterpret_cast<float4 *>(out + (int64_t)i * d);
  for (int k = threadIdx.x; k < d / 4; k += blockDim.x) {
    float4 v;
    if (masked) {
      const uint2 r = reinterpret_cast<const uint2 *>(mask_row)[k];
      v = make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                      __uint_as_float(r.y & 0xffff0000u));
    } else {
      v = table_get4(E, t, 4 * k);
    }
    dst[k] = v;
  }
}

hipError_t gather_rows(const PackedTable &E, const int32_t *tokens, int n, int V, const uint16_t *mask_row,
                       float *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (E.d % 4 || (reinterpret_cast<uintptr_t>(mask_row) & 7)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_table_kernel, dim3(n), dim3(256), 0, s, E, tokens, V, mask_row, out);
  return hipGetLastError();
}

// RMSNorm: out = x / sqrt(mean(x^2) + eps) * g, written in fp32 and/or, when
// requested, rounded to bf16 (the operand of the tied LM head) and as a
// split pair hi + lo (the operand of the projections).
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float *__restrict__ x, const T *__restrict__ g, int n,
                                                      int d, float eps, float *__restrict__ out,
                                                      bf16 *__restrict__ out_tiled, bf16 *__restrict__ out_split) {
  __shared__ float sh[256];
  const int i = blockIdx.x;
  if (i >= n) {  // padding rows of the tiled block
    for (int k = threadIdx.x; k < d; k += 256) out_tiled[tl_index(i, k, d)] = 0;
    return;
  }
  const float *xi = x + (int64_t)i * d;
  float ss = 0.f;
  for (int k = threadIdx.x; k < d; k += 256) ss += xi[k] * xi[k];
  ss = block_sum256(ss, sh);
  const float inv = rsqrtf(ss / (float)d + eps);
  for (int k = threadIdx.x; k < d; k += 256) {
    const float v = xi[k] * inv * Elem<T>::load(g, k);
    if (out) out[(int64_t)i * d + k] = v;
    if (out_tiled) out_tiled[tl_index(i, k, d)] = f32_to_bf16(v);
    if (out_split) {
      const bf16 hi = f32_to_bf16(v);
      out_split[(int64_t)i * d + k] = hi;
      out_split[(int64_t)n * d + (int64_t)i * d + k] = f32_to_bf16(v - bf16_to_f32(hi));
    }
  }
}

template <typename T>
hipError_t rmsnorm_rows(const float *x, const T *g, int n, int d, float eps, float *out, bf16 *out_tiled,
                        bf16 *out_split, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (out_tiled && d % TL_K) return hipErrorInvalidValue;
  const int rows = out_tiled ? (n + TL_ROWS - 1) / TL_ROWS * TL_ROWS : n;
  hipLaunchKernelGGL(rmsnorm_kernel<T>, dim3(rows), dim3(256), 0, s, x, g, n, d, eps, out, out_tiled, out_split);
  return hipGetLastError();
}
template hipError_t rmsnorm_rows<float>(const float *, const float *, int, int, float, float *, bf16 *, bf16 *,
                                        hipStream_t);
template hipError_t rmsnorm_rows<bf16>(const float *, const bf16 *, int, int, float, float *, bf16 *, bf16 *,
                                       hipStream_t);

// Merge of the self-conditioning split-K partials into S (fp32), times the
// row factor g (row_scale; 1 when null), plus the exact correction of each
// row's dominant token: the contraction used p~ = g * (the tiled value at
// (row, a) scaled by 2^-shift of a's tile, as the contraction scaled it),
// the previous step's exact probability of a is p_a, so S += (p_a - p~) E[a].
// One thread per float4 slot of the contraction's register-order blocks
// (selfcond_part_bytes): slot blockIdx.x * 256 + thread of column tile
// blockIdx.y of operand block blockIdx.z, so the ksplit partial reads are
// contiguous across a wave; the slot's canvas row and 4 columns follow from
// its index.  Canvas c of a batch (a single canvas is a batch of one) has
// its output rows at c * N * d.
__global__ void __launch_bounds__(256) selfcond_reduce_kernel(const float *__restrict__ part, int ksplit, int B, int N,
                                                            int d, int paired, ReduceBatch rb, int V, PackedTable E,
                                                            float *__restrict__ out, bf16 *__restrict__ out_split,
                                                            int64_t lo_off) {
  const int sl = blockIdx.x * 256 + threadIdx.x, nt = blockIdx.y, blk = blockIdx.z, ntn = gridDim.y;
  const int l = sl & 63, q = (sl >> 6) & 3, j = (sl >> 8) & 3, ii = (sl >> 10) & 1, w = sl >> 11;
  const int brow = (w >> 1) * 64 + 32 * ii + (l & 31);
  const int k = nt * 256 + (w & 1) * 128 + 32 * j + 8 * q + 4 * (l >> 5);
  const int c = paired ? 2 * blk + (brow >> 7) : blk, row = paired ? brow & 127 : brow;
  if (c >= B || row >= N || k >= d) return;  // slots the contraction did not write
  const int64_t count = (int64_t)N * d;
  const int64_t i = (int64_t)row * d + k, io = c * count + i;
  const float *pc = part + (((int64_t)blk * ksplit * ntn + nt) << 16) + (sl << 2);
  const int64_t zstride = (int64_t)ntn << 16;
  const float2 *top = rb.top[c];
  const float *row_scale = rb.row_scale[c];
  const uint8_t *shift = rb.shift[c];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int z = 0; z < ksplit; ++z) {
    const float4 v = *reinterpret_cast<const float4 *>(pc + z * zstride);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  const float g = row_scale ? row_scale[row] : 1.f;
  acc = make_float4(acc.x * g, acc.y * g, acc.z * g, acc.w * g);
  if (top) {
    const float2 tp = top[row];
    const int a = __float_as_int(tp.x);
    int bits = rb.probs[c][tl_index(row, a, V)];
    if (shift) bits = max(bits - ((int)shift[(int64_t)(a >> 6) * 256 + row] << 7), 0);
    const float cf = tp.y - g * bf16_to_f32((bf16)bits);
    const float4 e = table_get4(E, a, k);
    acc.x += cf * e.x;
    acc.y += cf * e.y;
    acc.z += cf * e.z;
    acc.w += cf * e.w;
  }
  *reinterpret_cast<float4 *>(out + io) = acc;
  if (out_split) {
    uint2 hi, lo;
    split4(acc, hi, lo);
    *reinterpret_cast<uint2 *>(out_split + io) = hi;
    *reinterpret_cast<uint2 *>(out_split + lo_off + io) = lo;
  }
}

// out[c * N + i] = canvas c's token i: the token ids of a batch of canvases
// as the stacked rows of the batched step.
__global__ void stack_tokens_kernel(TokenPtrs src, int N, int total, int32_t *__restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int c = i / N;
  out[i] = src.p[c][i - c * N];
}

hipError_t stack_tokens(const TokenPtrs &src, int B, int N, int32_t *out, hipStream_t s) {
  if (B < 1 || B > ES_MAX_BATCH || N < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stack_tokens_kernel, dim3((B * N + 255) / 256), dim3(256), 0, s, src, N, B * N, out);
  return hipGetLastError();
}

// fp8 copy of a bf16 matrix in the 8-byte-chunk tiled layout (dg_tiled.h):
// Y = X (X [R][K], leading dimension ldx) or, with trans, Y = X^T (X [K][R]);
// each value y * scale rounded to fp8 e4m3 (nearest even), clamped to
// +-448 first; rows past R are zero.  One workgroup per 256 x 32 block,
// staged through LDS so that both forms read X along its rows.
__global__ void __launch_bounds__(256) tile_fp8_kernel(const bf16 *__restrict__ X, int R, int K, int64_t ldx,
                                                       int trans, float scale, uint8_t *__restrict__ out) {
  __shared__ float tile[256][33];
  const int nks = K / TL_K;
  const int b = blockIdx.x / nks, s = blockIdx.x % nks;
  const int t = threadIdx.x;
  for (int i = 0; i < 32; ++i) {
    const int idx = t + 256 * i;
    int r, k;
    float v = 0.f;
    if (trans) {
      k = idx >> 8;
      r = idx & 255;
      if (256 * b + r < R) v = bf16_to_f32(X[(int64_t)(32 * s + k) * ldx + 256 * b + r]);
    } else {
      r = idx >> 5;
      k = idx & 31;
      if (256 * b + r < R) v = bf16_to_f32(X[(int64_t)(256 * b + r) * ldx + 32 * s + k]);
    }
    tile[r][k] = v;
  }
  __syncthreads();
  for (int j = 0; j < 4; ++j) {
    const int p = t + 256 * j, r = p >> 2, c = (p & 3) ^ (tl8_pos(r, 0) & 3);  // slot p holds chunk c
    uint32_t w[2] = {0u, 0u};
    for (int h = 0; h < 2; ++h) {
      float q[4];
      for (int e = 0; e < 4; ++e) q[e] = fminf(fmaxf(tile[r][8 * c + 4 * h + e] * scale, -448.f), 448.f);
      int packed = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], packed, true);
      w[h] = (uint32_t)packed;
    }
    *reinterpret_cast<uint2 *>(out + (int64_t)blockIdx.x * TL8_BYTES + (int64_t)p * 8) = make_uint2(w[0], w[1]);
  }
}

hipError_t tile_fp8(const uint16_t *X, int R, int K, int64_t ldx, bool trans, float scale, uint8_t *out,
                    hipStream_t s) {
  if (R < 1 || K % TL_K) return hipErrorInvalidValue;
  const int blocks = (R + TL_ROWS - 1) / TL_ROWS * (K / TL_K);
  hipLaunchKernelGGL(tile_fp8_kernel, dim3(blocks), dim3(256), 0, s, X, R, K, ldx, trans ? 1 : 0, scale, out);
  return hipGetLastError();
}

// fp4 e2m1 copy of a bf16 matrix in the 4-byte-chunk tiled layout
// (dg_tiled.h), Y = X or Y = X^T as in tile_fp8_kernel, with a scale byte per
// 32 x 32 block.  One workgroup per 256 x 32 block; thread t finds the
// largest magnitude of row t, threads 0..7 that of a 32-row group.
__device__ inline uint32_t fp4_code(float y) {  // nearest e2m1 code, ties to even, saturated; zero is +0
  const float a = fabsf(y);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.f ? 6u : 7u;
  return (c != 0u && signbit(y)) ? c | 8u : c;
}
__global__ void __launch_bounds__(256) tile_fp4_kernel(const bf16 *__restrict__ X, int R, int K, int64_t ldx,
                                                       int trans, uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales) {
  __shared__ float tile[256][33];
  __shared__ float rowmax[256];
  __shared__ float gmul[8];
  const int nks = K / TL_K;
  const int b = blockIdx.x / nks, s = blockIdx.x % nks;
  const int t = threadIdx.x;
  for (int i = 0; i < 32; ++i) {
    const int idx = t + 256 * i;
    int r, k;
    float v = 0.f;
    if (trans) {
      k = idx >> 8;
      r = idx & 255;
      if (256 * b + r < R) v = bf16_to_f32(X[(int64_t)(32 * s + k) * ldx + 256 * b + r]);
    } else {
      r = idx >> 5;
      k = idx & 31;
      if (256 * b + r < R) v = bf16_to_f32(X[(int64_t)(256 * b + r) * ldx + 32 * s + k]);
    }
    tile[r][k] = v;
  }
  __syncthreads();
  float m = 0.f;
  for (int k = 0; k < 32; ++k) m = fmaxf(m, fabsf(tile[t][k]));  // NaN entries are passed over
  rowmax[t] = m;
  __syncthreads();
  if (t < 8) {
    float a = 0.f;
    for (int r = 0; r < 32; ++r) a = fmaxf(a, rowmax[32 * t + r]);
    const int ef = (int)((__float_as_uint(a) >> 23) & 0xFF);  // floor(log2 a) + 127 for normal a
    const int u = a == 0.f ? 127 : min(max(ef - 2, 2), 252);
    scales[(int64_t)blockIdx.x * TL4_SCALES + t] = (uint8_t)u;
    gmul[t] = __uint_as_float((uint32_t)(254 - u) << 23);  // 2^(127 - u), exact
  }
  __syncthreads();
  for (int j = 0; j < 4; ++j) {
    // slot p: stored row p / 4 = block row r, columns 8c .. 8c + 7
    const int p = t + 256 * j, r = tl4_row(p >> 2), c = tl4_chunk_at(p >> 2, p & 3);
    const float mul = gmul[r >> 5];
    uint32_t w = 0u;
    for (int e = 0; e < 8; ++e) w |= fp4_code(tile[r][8 * c + e] * mul) << (4 * e);
    *reinterpret_cast<uint32_t *>(codes + (int64_t)blockIdx.x * TL4_BYTES + (int64_t)p * 4) = w;
  }
}

hipError_t tile_fp4(const uint16_t *X, int R, int K, int64_t ldx, bool trans, uint8_t *codes, uint8_t *scales,
                    hipStream_t s) {
  if (R < 1 || K % TL_K) return hipErrorInvalidValue;
  const int blocks = (R + TL_ROWS - 1) / TL_ROWS * (K / TL_K);
  hipLaunchKernelGGL(tile_fp4_kernel, dim3(blocks), dim3(256), 0, s, X, R, K, ldx, trans ? 1 : 0, codes, scales);
  return hipGetLastError();
}

hipError_t selfcond_reduce_batch(const float *part, int ksplit, int B, int N, int d, const ReduceBatch &rb, int V,
                                 const PackedTable &E, float *out, uint16_t *out_split, hipStream_t s,
                                 int64_t lo_off) {
  if (B < 1 || B > ES_MAX_BATCH || d % 4) return hipErrorInvalidValue;
  for (int c = 0; c < B; ++c)
    if (rb.top[c] && (!E.p || E.d != d || !rb.probs[c])) return hipErrorInvalidValue;
  if (N > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(selfcond_reduce_kernel, dim3(64, (d + 255) / 256, selfcond_blocks(B, N)), dim3(256), 0, s, part,
                     ksplit, B, N, d, selfcond_paired(B, N) ? 1 : 0, rb, V, E, out, out_split,
                     lo_off ? lo_off : (int64_t)B * N * d);
  return hipGetLastError();
}

hipError_t selfcond_reduce(const float *part, int ksplit, int N, int d, const float2 *top, const uint16_t *probs,
                           int V, const float *row_scale, const uint8_t *shift, const PackedTable &E, float *out,
                           uint16_t *out_split, hipStream_t s, int64_t lo_off) {
  ReduceBatch rb{};  // a batch of one: the same kernel, so a canvas's S does not depend on its batch
  rb.top[0] = top;
  rb.probs[0] = probs;
  rb.row_scale[0] = row_scale;
  rb.shift[0] = shift;
  return selfcond_reduce_batch(part, ksplit, 1, N, d, rb, V, E, out, out_split, s, lo_off ? lo_off : (int64_t)N * d);
}

// Numerators -> probabilities, in place (fp32 path, row-major [N][V]).
__global__ void normalize_f32_kernel(float *__restrict__ probs, const float *__restrict__ tile_scale, int64_t chunks,
                                     int V) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i * 4;
    const int64_t row = e / V;
    const int col = (int)(e - row * V);
    const float c = tile_scale[row * (V / TILE) + col / TILE];
    float4 v = reinterpret_cast<const float4 *>(probs)[i];
    v.x *= c;
    v.y *= c;
    v.z *= c;
    v.w *= c;
    reinterpret_cast<float4 *>(probs)[i] = v;
  }
}

hipError_t normalize_probs_f32(float *probs, const float *tile_scale, int N, int V, hipStream_t s) {
  const int64_t chunks = (int64_t)N * V / 4;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(normalize_f32_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s,
                     probs, tile_scale, chunks, V);
  return hipGetLastError();
}

// Tiled copy: one thread per 16-byte chunk of the output.
__global__ void tile_rows_kernel(const bf16 *__restrict__ X, int R, int K, int64_t ldx, bf16 *__restrict__ out,
                                 int64_t chunks) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(i & (TL_CHUNKS - 1));
    const int64_t bs = i >> 10;
    const int ks = K / TL_K;
    const int b = (int)(bs / ks), slice = (int)(bs % ks);
    const int r = p >> 2, c = (p & 3) ^ ((r >> 2) & 3);
    const int row = b * TL_ROWS + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < R) {
      const bf16 *src = X + (int64_t)row * ldx + slice * TL_K + c * 8;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = (uint32_t)src[2 * k] | ((uint32_t)src[2 * k + 1] << 16);
      v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    reinterpret_cast<uint4 *>(out)[i] = v;
  }
}

hipError_t tile_rows(const uint16_t *X, int R, int K, int64_t ldx, uint16_t *out, hipStream_t s) {
  if (K % TL_K) return hipErrorInvalidValue;
  const int64_t chunks = (int64_t)tl_elems(R, K) / 8;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(tile_rows_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s, X, R, K,
                     ldx, out, chunks);
  return hipGetLastError();
}

template <typename T>
__global__ void transpose_kernel(const T *__restrict__ in, int rows, int cols, T *__restrict__ out, int64_t ld_out) {
  __shared__ T tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int k = ty; k < 32; k += 8) {
    const int r = r0 + k, c = c0 + tx;
    if (r < rows && c < cols) tile[k][tx] = in[(int64_t)r * cols + c];
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int c = c0 + k, r = r0 + tx;
    if (r < rows && c < cols) out[(int64_t)c * ld_out + r] = tile[tx][k];
  }
}

template <typename T>
hipError_t transpose(const T *in, int rows, int cols, T *out, int64_t ld_out, hipStream_t s) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  hipLaunchKernelGGL(transpose_kernel<T>, grid, dim3(256), 0, s, in, rows, cols, out, ld_out);
  return hipGetLastError();
}
template hipError_t transpose<float>(const float *, int, int, float *, int64_t, hipStream_t);
template hipError_t transpose<bf16>(const bf16 *, int, int, bf16 *, int64_t, hipStream_t);

__global__ void copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t copy_bytes(const void *src, void *dst, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(copy_kernel, dim3(2048), dim3(256), 0, s, static_cast<const uint4 *>(src),
                     static_cast<uint4 *>(dst), n);
  return hipGetLastError();
}

// Per-(row, 64-column tile) softmax statistics from fp32 logits (the fp32
// configuration); the same quantities the bf16 LM-head epilogue produces.
// One wave per tile.
__global__ void __launch_bounds__(64) tile_stats_f32_kernel(const float *__restrict__ logits, int V, float inv_T,
                                                            float *__restrict__ probs, float4 *__restrict__ stats) {
  const int row = blockIdx.y, tile = blockIdx.x;
  const int col = tile * TILE + threadIdx.x;
  const float z = logits[(int64_t)row * V + col];
  float best = z;
  int bcol = col;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o);
    const int oc = __shfl_xor(bcol, o);
    if (ov > best || (ov == best && oc < bcol)) {
      best = ov;
      bcol = oc;
    }
  }
  const float m = best * inv_T;
  const float t = z * inv_T - m;
  const float e = exp2f(t * LOG2E);
  probs[(int64_t)row * V + col] = e;
  const float l = warp_sum(e);
  const float sacc = warp_sum(e * t);
  if (threadIdx.x == 0) stats[(int64_t)row * (V / TILE) + tile] = make_float4(best, l, sacc, __int_as_float(bcol));
}

hipError_t tile_stats_f32(const float *logits, int M, int V, float inv_T, float *probs, float4 *stats,
                          hipStream_t s) {
  hipLaunchKernelGGL(tile_stats_f32_kernel, dim3(V / TILE, M), dim3(64), 0, s, logits, V, inv_T, probs, stats);
  return hipGetLastError();
}

__global__ void gumbel_test_kernel(const uint32_t *__restrict__ w, int n, int mode, float *__restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = mode == 0 ? ln_fixed(__uint_as_float(w[i])) : gumbel_word(w[i]);
}

hipError_t gumbel_test(const uint32_t *w, int n, int mode, float *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gumbel_test_kernel, dim3((n + 255) / 256), dim3(256), 0, s, w, n, mode, out);
  return hipGetLastError();
}

// Reductions over the NW waves of a row's workgroup: within each wave by lane
// exchanges, then across the waves through LDS (two barriers).
template <int NW>
__device__ __forceinline__ float rc_sum(float v, float *sh) {
  v = warp_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += sh[w];
  __syncthreads();
  return r;
}
template <int NW>
__device__ __forceinline__ float2 rc_sum2(float a, float b, float *sh) {
  a = warp_sum(a);
  b = warp_sum(b);
  if ((threadIdx.x & 63) == 0) {
    sh[threadIdx.x >> 6] = a;
    sh[NW + (threadIdx.x >> 6)] = b;
  }
  __syncthreads();
  float2 r = make_float2(sh[0], sh[NW]);
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    r.x += sh[w];
    r.y += sh[NW + w];
  }
  __syncthreads();
  return r;
}
template <int NW>
__device__ __forceinline__ float3 rc_sum3(float a, float b, float c, float *sh) {
  a = warp_sum(a);
  b = warp_sum(b);
  c = warp_sum(c);
  if ((threadIdx.x & 63) == 0) {
    sh[threadIdx.x >> 6] = a;
    sh[NW + (threadIdx.x >> 6)] = b;
    sh[2 * NW + (threadIdx.x >> 6)] = c;
  }
  __syncthreads();
  float3 r = make_float3(sh[0], sh[NW], sh[2 * NW]);
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    r.x += sh[w];
    r.y += sh[NW + w];
    r.z += sh[2 * NW + w];
  }
  __syncthreads();
  return r;
}
// max of (value, lowest index on ties)
template <int NW>
__device__ __forceinline__ void rc_argmax(float &v, int &i, float *shv, int *shi) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o);
    const int i2 = __shfl_xor(i, o);
    if (v2 > v || (v2 == v && i2 < i)) {
      v = v2;
      i = i2;
    }
  }
  if ((threadIdx.x & 63) == 0) {
    shv[threadIdx.x >> 6] = v;
    shi[threadIdx.x >> 6] = i;
  }
  __syncthreads();
  v = shv[0];
  i = shi[0];
#pragma unroll
  for (int w = 1; w < NW; ++w)
    if (shv[w] > v || (shv[w] == v && shi[w] < i)) {
      v = shv[w];
      i = shi[w];
    }
  __syncthreads();
}

// Entropy of softmax(y) from the tile statistics ([P3] §5.4 measures
// confidence by the entropy of each position's distribution):
//   M = max_t m_t, L = sum_t l_t e^{m_t - M},
//   S = sum_t e^{m_t - M} (s_t + (m_t - M) l_t),  H = ln L - S / L  (nats),
// clamped at +0 (NaN propagates).  Also the argmax (lowest index on ties)
// and the normaliser c_t = e^{m_t - M} / L of each tile, which turns the
// stored numerators into probabilities for the next self-conditioning.
//
// With n2 given (bf16 path) the logit of the row's argmax token a is first
// recomputed exactly from the fp32 normalised hidden state (the LM head used
// its bf16 rounding), and a's term in its tile's sums is replaced: the
// dominant token carries most of the entropy's sensitivity to logit error.
// The exact probability of a is kept in top[row] = (a, p_a) for the next
// step's self-conditioning.  The argmax itself stays the LM head's.
//
// With shift given (bf16 path) the stored numerators are relative to the
// power-of-two reference 2^r_t, r_t = ceil(m_t log2e) (the LM head's
// choice), so p = stored * 2^-(R - r_t) * g with R = ceil(M log2e) and
// g = 2^(R - M log2e) / L: the row factor g goes to row_scale, the
// per-tile exponent R - r_t (capped at 255) to shift ([tile][256 rows],
// uint8); tile_scale (nullable then) holds 2^-(R - r_t) g.  Without shift,
// tile_scale is e^{m_t - M} / L for numerators relative to m_t itself.
// RC_NT threads per row; RC_CACHE tiles per thread are held in registers
// (one read of the row's statistics) when ntiles <= RC_NT * RC_CACHE;
// otherwise the passes re-read.
constexpr int RC_NT = 512;
constexpr int RC_NW = RC_NT / 64;
constexpr int RC_CACHE = 4096 / RC_NT;
constexpr int RC_D = 4096 / RC_NT;  // normalised-row values per thread: d <= 4096

// One row: row indexes the canvas's own buffers, n2 points at that row's
// normalised state.
template <bool CACHED>
__device__ __forceinline__ void row_combine_row(const int row, const float4 *__restrict__ stats, int ntiles,
                                                float inv_T, float *__restrict__ entropy,
                                                int32_t *__restrict__ cand, float *__restrict__ tile_scale,
                                                float *__restrict__ row_scale, uint8_t *__restrict__ shift,
                                                const float *__restrict__ n2, const PackedTable &E,
                                                float2 *__restrict__ top, float *shv, int *shi) {
  const int d = E.d;
  // the normalised row for the exact top logit, loaded before the argmax is known
  float nv[RC_D];
  const bool fix = n2 != nullptr;
  if (fix) {
#pragma unroll
    for (int i = 0; i < RC_D; ++i) {
      const int k = threadIdx.x + RC_NT * i;
      nv[i] = k < d ? n2[k] : 0.f;
    }
  }
  const float4 *st = stats + (int64_t)row * ntiles;
  float4 c[CACHED ? RC_CACHE : 1];
  auto tile = [&](int i, int t) -> float4 { return CACHED ? c[i] : st[t]; };
  if (CACHED) {
#pragma unroll
    for (int i = 0; i < RC_CACHE; ++i) {
      const int t = threadIdx.x + RC_NT * i;
      c[i] = t < ntiles ? st[t] : make_float4(-INFINITY, 0.f, 0.f, __int_as_float(INT32_MAX));
    }
  }
  const int nper = CACHED ? RC_CACHE : (ntiles + RC_NT - 1) / RC_NT;
  float best = -INFINITY;
  int bidx = INT32_MAX;
#pragma unroll
  for (int i = 0; i < nper; ++i) {
    const int t = threadIdx.x + RC_NT * i;
    if (t >= ntiles) break;
    const float4 v = tile(i, t);
    const int idx = __float_as_int(v.w);
    if (v.x > best || (v.x == best && idx < bidx)) {
      best = v.x;
      bidx = idx;
    }
  }
  rc_argmax<RC_NW>(best, bidx, shv, shi);
  const float Mz = best;
  // every tile maximum NaN (a NaN hidden state): no argmax; token 0 stands in
  // and nothing is recomputed (the entropy comes out NaN)
  const bool found = bidx < ntiles * TILE;
  const int amax = found ? bidx : 0;
  const float My = Mz * inv_T;
  // the argmax token's table row, in flight while the tile sums are formed
  float ev[RC_D];
  if (fix && found) {
#pragma unroll
    for (int i = 0; i < RC_D; ++i) {
      const int k = threadIdx.x + RC_NT * i;
      ev[i] = k < d ? table_get(E, amax, k) : 0.f;
    }
  }
  float L = 0.f, S = 0.f;
#pragma unroll
  for (int i = 0; i < nper; ++i) {
    const int t = threadIdx.x + RC_NT * i;
    if (t >= ntiles) break;
    const float4 v = tile(i, t);
    const float dd = v.x * inv_T - My;
    const float w = exp2f(dd * LOG2E);
    L += v.y * w;
    S += w * (v.z + dd * v.y);
  }
  float part = 0.f;
  if (fix && found) {
#pragma unroll
    for (int i = 0; i < RC_D; ++i) part += nv[i] * ev[i];
  }
  {
    const float3 r = rc_sum3<RC_NW>(part, L, S, shv);
    L = r.y;
    S = r.z;
    part = r.x;
  }
  // the argmax token's term replaced by its exact one: its tile holds the
  // row maximum, so that tile's weight is exactly 1 (dd = 0) and the
  // correction adds e - 1 to L and e d_top to S (reference m_ta = My)
  float d_top = 0.f;
  if (fix && found) {
    d_top = part * inv_T - My;
    const float e = exp2f(d_top * LOG2E);
    L += e - 1.f;
    S += e * d_top;
  }
  const float invL = 1.f / L;
  const float R = ceilf(My * LOG2E);
  const float g = exp2f(R - My * LOG2E) * invL;
#pragma unroll
  for (int i = 0; i < nper; ++i) {
    const int t = threadIdx.x + RC_NT * i;
    if (t >= ntiles) break;
    const float mt = tile(i, t).x * inv_T;
    if (shift) {
      const float sh = fminf(fmaxf(R - ceilf(mt * LOG2E), 0.f), 255.f);  // NaN -> 0
      shift[(int64_t)t * 256 + row] = (uint8_t)sh;
      if (tile_scale) tile_scale[(int64_t)row * ntiles + t] = exp2f(-sh) * g;
    } else {
      tile_scale[(int64_t)row * ntiles + t] = exp2f((mt - My) * LOG2E) * invL;
    }
  }
  if (threadIdx.x == 0) {
    float H = logf(L) - S * invL;
    if (H <= 0.f) H = 0.f;
    entropy[row] = H;
    cand[row] = amax;
    if (top) top[row] = make_float2(__int_as_float(amax), exp2f(d_top * LOG2E) * invL);
    if (row_scale) row_scale[row] = g;
  }
}

template <bool CACHED>
__global__ void __launch_bounds__(RC_NT) row_combine_kernel(const float4 *__restrict__ stats, int ntiles,
                                                          float inv_T, float *__restrict__ entropy,
                                                          int32_t *__restrict__ cand,
                                                          float *__restrict__ tile_scale,
                                                          float *__restrict__ row_scale, uint8_t *__restrict__ shift,
                                                          const float *__restrict__ n2, PackedTable E,
                                                          float2 *__restrict__ top) {
  __shared__ float shv[3 * RC_NW];
  __shared__ int shi[RC_NW];
  const int row = blockIdx.x;
  row_combine_row<CACHED>(row, stats, ntiles, inv_T, entropy, cand, tile_scale, row_scale, shift,
                          n2 ? n2 + (int64_t)row * E.d : nullptr, E, top, shv, shi);
}

// A batch: workgroup r is row r % N of canvas r / N (the bf16 path's
// buffers, exponents and top tokens per canvas); n2 holds the stacked rows.
template <bool CACHED>
__global__ void __launch_bounds__(RC_NT) row_combine_batch_kernel(RowCombineBatch bt, int N, int ntiles,
                                                                float inv_T, const float *__restrict__ n2,
                                                                PackedTable E) {
  __shared__ float shv[3 * RC_NW];
  __shared__ int shi[RC_NW];
  const int c = blockIdx.x / N, row = blockIdx.x - c * N;
  row_combine_row<CACHED>(row, bt.stats[c], ntiles, inv_T, bt.entropy[c], bt.cand[c], nullptr, bt.row_scale[c],
                          bt.shift[c], n2 + (int64_t)blockIdx.x * E.d, E, bt.top[c], shv, shi);
}

hipError_t row_combine_batch(const RowCombineBatch &bt, int B, int N, int ntiles, float inv_T, const float *n2,
                             const PackedTable &E, hipStream_t s) {
  if (B < 1 || B > ES_MAX_BATCH || N < 1 || N > 256 || !n2 || !E.p || E.d % 4 || E.d > RC_NT * RC_D)
    return hipErrorInvalidValue;
  if (ntiles <= RC_NT * RC_CACHE)
    hipLaunchKernelGGL(row_combine_batch_kernel<true>, dim3(B * N), dim3(RC_NT), 0, s, bt, N, ntiles, inv_T, n2, E);
  else
    hipLaunchKernelGGL(row_combine_batch_kernel<false>, dim3(B * N), dim3(RC_NT), 0, s, bt, N, ntiles, inv_T, n2, E);
  return hipGetLastError();
}

hipError_t row_combine(const float4 *tile_stats, int M, int ntiles, float inv_T, float *entropy,
                       int32_t *cand, float *tile_scale, float *row_scale, uint8_t *shift, const float *n2,
                       const PackedTable &E, float2 *top, hipStream_t s) {
  if ((shift && M > 256) || (n2 && (!E.p || E.d % 4 || E.d > RC_NT * RC_D))) return hipErrorInvalidValue;
  if (ntiles <= RC_NT * RC_CACHE)
    hipLaunchKernelGGL(row_combine_kernel<true>, dim3(M), dim3(RC_NT), 0, s, tile_stats, ntiles, inv_T, entropy,
                       cand, tile_scale, row_scale, shift, n2, E, top);
  else
    hipLaunchKernelGGL(row_combine_kernel<false>, dim3(M), dim3(RC_NT), 0, s, tile_stats, ntiles, inv_T, entropy,
                       cand, tile_scale, row_scale, shift, n2, E, top);
  return hipGetLastError();
}

// Multinomial candidate ([P3] §5.3: the token is drawn from the tempered
// softmax), drawn from the distribution the step keeps in two Gumbel-max
// levels (dg_device.h), one workgroup per canvas row:
//   the tile t, by the largest fl(fl(ln l_t + zmax_t inv_T) + G), G from word
//   t%4 of Philox(seed; row, step, canvas, 2 + 4 floor(t/4)): l_t e^{m_t} is
//   the tile's mass up to a factor common to the row;
//   then the column c of that tile, by the largest fl(ln w_c + G'), G' from
//   word c%4 of Philox(seed; row, step, canvas, 3 + 4 floor(c/4)), w_c the
//   stored weight (bf16 numerator, or the fp32 path's probability), which is
//   e^{y_c} up to a factor common to the tile.
// Lowest index on equal keys; a NaN key never wins.  cand holds the argmax on
// entry and keeps it when nothing is drawable.
// 1024 threads per row; thread k owns tiles 4k .. 4k+3 (and every 4096th
// after), whose noise is the four words of one Philox block.
constexpr int DRAW_NT = 1024;
__global__ void __launch_bounds__(DRAW_NT) draw_kernel(const float4 *__restrict__ stats, int ntiles, float inv_T,
                                                       DrawArgs draw, int32_t *__restrict__ cand) {
  __shared__ float shv[DRAW_NT / 64];
  __shared__ int shi[DRAW_NT / 64];
  const int row = blockIdx.x;
  const uint32_t k0 = (uint32_t)draw.seed, k1 = (uint32_t)(draw.seed >> 32);
  const float4 *st = stats + (int64_t)row * ntiles;
  float kb = -INFINITY;
  int kt = INT32_MAX;
  for (int t0 = 4 * threadIdx.x; t0 < ntiles; t0 += 4 * DRAW_NT) {  // ascending tiles per thread
    const Philox4 w = philox4x32_10((uint32_t)row, draw.step, draw.canvas, 2u + (uint32_t)t0, k0, k1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = st[t0 + j];
      const float k = gumbel_key_tile(v.y, v.x, inv_T, w.v[j]);
      if (k > kb) {
        kb = k;
        kt = t0 + j;
      }
    }
  }
  // largest key, lowest tile on ties: within each wave, then across the 16 waves
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(kb, o);
    const int i2 = __shfl_xor(kt, o);
    if (v2 > kb || (v2 == kb && i2 < kt)) {
      kb = v2;
      kt = i2;
    }
  }
  if ((threadIdx.x & 63) == 0) {
    shv[threadIdx.x >> 6] = kb;
    shi[threadIdx.x >> 6] = kt;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  kb = shv[0];
  kt = shi[0];
#pragma unroll
  for (int w = 1; w < DRAW_NT / 64; ++w)
    if (shv[w] > kb || (shv[w] == kb && shi[w] < kt)) {
      kb = shv[w];
      kt = shi[w];
    }
  if (kt == INT32_MAX) return;

  // one wave: lane c = column c of tile kt
  const int c = threadIdx.x;
  float wgt;
  if (draw.num_tiled)  // slice 2 kt + c / 32, chunk (c % 32) / 8 of the row, element c % 8
    wgt = bf16_to_f32(draw.num_tiled[(int64_t)(2 * kt + (c >> 5)) * TL_ELEMS + tl_pos(row, (c & 31) >> 3) * 8 +
                                     (c & 7)]);
  else
    wgt = draw.num_f32[(int64_t)row * ntiles * TILE + (int64_t)kt * TILE + c];
  const Philox4 w = philox4x32_10((uint32_t)row, draw.step, draw.canvas, 3u + 4u * ((uint32_t)c >> 2), k0, k1);
  float kc = gumbel_key_col(wgt, w.v[c & 3]);
  int cc = kc > -INFINITY ? c : INT32_MAX;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(kc, o);
    const int oc = __shfl_xor(cc, o);
    if (ov > kc || (ov == kc && oc < cc)) {
      kc = ov;
      cc = oc;
    }
  }
  if (c == 0 && cc != INT32_MAX) cand[row] = kt * TILE + cc;
}

hipError_t multinomial_draw(const float4 *tile_stats, int M, int ntiles, float inv_T, const DrawArgs &draw,
                            int32_t *cand, hipStream_t s) {
  if ((draw.num_tiled == nullptr) == (draw.num_f32 == nullptr) || (draw.num_tiled && M > 256) || ntiles % 4)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(draw_kernel, dim3(M), dim3(DRAW_NT), 0, s, tile_stats, ntiles, inv_T, draw, cand);
  return hipGetLastError();
}

}  // namespace dg
