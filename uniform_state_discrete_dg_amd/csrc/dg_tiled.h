// dg_tiled.h -- the tiled bf16 layout of the two table-streaming
// contractions' operands (host and device).
//
// A bf16 matrix X [R][K] (K a multiple of 32) is stored as blocks of 256 rows
// x 32 columns, 16 KB each, block (b, s) at index b * (K / 32) + s.  Inside a
// block, 16-byte chunk p (p = 0..1023) holds the 8 values
// X[256 b + r][32 s + 8 c .. 32 s + 8 c + 7] with r = p / 4 and
// c = (p % 4) ^ ((r / 4) % 4): exactly the order of an LDS slice of the
// streaming kernels, so each 64-lane DMA instruction copies 1 KB of
// consecutive memory.  Rows past R (up to the next multiple of 256) are
// padding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace dg {

constexpr int TL_ROWS = 256;    // rows per block
constexpr int TL_K = 32;        // columns per block
constexpr int TL_CHUNKS = 1024; // 16-byte chunks per block
constexpr int TL_ELEMS = 8192;  // bf16 values per block

// position of logical chunk c (columns 8c..8c+7 of the block) of block row r
__host__ __device__ inline int tl_pos(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// element index of X[row][col] in the tiled layout of a matrix with K columns
__host__ __device__ inline int64_t tl_index(int row, int col, int K) {
  const int b = row >> 8, r = row & 255, s = col >> 5, k = col & 31;
  return (((int64_t)b * (K >> 5) + s) * TL_CHUNKS + tl_pos(r, k >> 3)) * 8 + (k & 7);
}

inline size_t tl_elems(int R, int K) { return (size_t)((R + TL_ROWS - 1) / TL_ROWS) * TL_ROWS * (size_t)K; }

// The fp8 form (one byte per value): the same blocks of 256 rows x 32
// columns, 8 KB each, with 8-byte chunks: chunk p holds the 8 values
// X[256 b + r][32 s + 8 c .. + 7], r = p / 4, c = (p % 4) ^ w(r) with
// w(r) = (bit 2 of r xor bit 4 of r) + 2 (bit 3 of r).  A table fragment is
// one 8-byte LDS read per lane; with this w the reads of a fragment's 32
// rows measured no bank conflict (the r / 4 and r / 8 swizzles measured 3 and
// 17 M conflict cycles per LM-head launch).
constexpr int TL8_BYTES = 8192;  // bytes per block
__host__ __device__ inline int tl8_pos(int r, int c) {
  return r * 4 + (c ^ ((((r >> 2) ^ (r >> 4)) & 1) | (((r >> 3) & 1) << 1)));
}
__host__ __device__ inline int64_t tl8_index(int row, int col, int K) {
  const int b = row >> 8, r = row & 255, s = col >> 5, k = col & 31;
  return (((int64_t)b * (K >> 5) + s) * TL_CHUNKS + tl8_pos(r, k >> 3)) * 8 + (k & 7);
}

// The fp4 form (e2m1, two values per byte): the same blocks of 256 rows x 32
// columns, 4 KB each.  A row is 16 bytes: two 8-byte words, word w holding
// the 8 values of columns 8 w .. 8 w + 7 (4 bytes) and then those of columns
// 16 + 8 w .. 16 + 8 w + 7, value 2 i in the low nibble of byte i.  Block
// row r is stored as row rho(r) = r with bits 3 and 4 swapped, its word w at
// position w ^ ((bit 3 xor bit 4) of rho(r)).  One 8-byte read gives a
// row-fragment lane both 16-wide k halves of its columns (the LM head), and
// is the unit of the transposing LDS read (the self-conditioning
// contraction), whose 32-lane halves read rows 0-7 with 16-23 and 8-15 with
// 24-31: rho makes each such set 16 consecutive stored rows, and the word
// swizzle keeps the rows of a row-fragment read off each other's banks.
// Each 32 x 32 sub-block (rows 32 g .. 32 g + 31 of the block) has one scale
// byte u (value = code * 2^(u - 127)), stored apart from the codes: byte g of
// 8 per block, blocks in the same order.
constexpr int TL4_BYTES = 4096;  // bytes of codes per block
constexpr int TL4_SCALES = 8;    // scale bytes per block
// rho (an involution: stored row <-> block row) and the word swizzle of a stored row
__host__ __device__ inline int tl4_row(int r) { return (r & ~0x18) | ((r >> 1) & 0x8) | ((r << 1) & 0x10); }
__host__ __device__ inline int tl4_swz(int sr) { return ((sr >> 3) ^ (sr >> 4)) & 1; }
// position (in 4-byte units from the block's start) of the 8 values of
// columns 8 c .. 8 c + 7 of block row r, and the inverse: which columns unit
// u of stored row sr holds
__host__ __device__ inline int tl4_pos(int r, int c) {
  const int sr = tl4_row(r);
  return sr * 4 + 2 * ((c & 1) ^ tl4_swz(sr)) + (c >> 1);
}
__host__ __device__ inline int tl4_chunk_at(int sr, int u) { return ((u >> 1) ^ tl4_swz(sr)) + 2 * (u & 1); }
// byte holding X[row][col] (low nibble for even col) and that value's scale byte
__host__ __device__ inline int64_t tl4_index(int row, int col, int K) {
  const int b = row >> 8, r = row & 255, s = col >> 5, k = col & 31;
  return (((int64_t)b * (K >> 5) + s) * TL_CHUNKS + tl4_pos(r, k >> 3)) * 4 + ((k & 7) >> 1);
}
__host__ __device__ inline int64_t tl4_scale_index(int row, int col, int K) {
  return ((int64_t)(row >> 8) * (K >> 5) + (col >> 5)) * TL4_SCALES + ((row & 255) >> 5);
}

// The tied table E [V][d] as the library keeps it: one copy, in one of the
// three tiled forms.  The LM head streams it as it is; the self-conditioning
// contraction streams the same bytes and transposes them in LDS; the row
// gathers (embeddings, the exact top-token terms) read single rows.
enum TableForm { TF_BF16 = 0, TF_FP8 = 1, TF_FP4 = 2 };
struct PackedTable {
  int tf;             // TableForm
  const void *p;      // bf16 values, fp8 codes or fp4 codes (tiled)
  const uint8_t *s4;  // TF_FP4: the blocks' scale bytes
  float scale;        // TF_FP8: value = code * scale
  int d;              // columns
};

#if defined(__HIPCC__)
// 4 consecutive values of one row (col % 4 == 0) as floats, exactly.
__device__ inline float4 table_get4(const PackedTable &t, int row, int col) {
  uint32_t w0, w1;  // two packed bf16 pairs
  if (t.tf == TF_BF16) {
    const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(t.p) + tl_index(row, col, t.d));
    w0 = v.x;
    w1 = v.y;
  } else if (t.tf == TF_FP8) {
    const uint32_t q = *reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(t.p) + tl8_index(row, col, t.d));
    w0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, t.scale, false));
    w1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, t.scale, true));
  } else {
    const uint32_t q = *reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(t.p) + tl4_index(row, col, t.d));
    const float sc = __uint_as_float((uint32_t)t.s4[tl4_scale_index(row, col, t.d)] << 23);
    w0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 0));
    w1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 1));
  }
  return make_float4(__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xffff0000u), __uint_as_float(w1 << 16),
                     __uint_as_float(w1 & 0xffff0000u));
}
// One value.
__device__ inline float table_get(const PackedTable &t, int row, int col) {
  const float4 v = table_get4(t, row, col & ~3);
  const int k = col & 3;
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}
#endif

}  // namespace dg
