// estream.hip -- the two contractions that stream the token-embedding table
// (V x d, 1.5 GB at V = 262144, d = 2816) once per step each:
//   * the tied LM head z = RMSNorm(h1) E^T, with the softmax/entropy
//     statistics fused into its epilogue (the logits never reach memory; the
//     probability numerators are written once in bf16), and
//   * the self-conditioning contraction S = p_prev E, streaming the same
//     copy of E (transposed on its way out of LDS) split over V, with the
//     probability numerators' power-of-two tile exponents applied as they
//     are read.
// At a 256-row canvas both sit at the chip's ridge point (256 flop per byte
// of the table: HBM and matrix cores would finish together), and with both
// busy the chip runs at its power limit (the engine clock drops to about
// 2 GHz in the step, lower back to back), so the design keeps bytes in
// flight and spends as few instructions and LDS bytes per MFMA as it can.
// A workgroup owns all canvas rows x 256 table rows.  k advances in 32-wide
// slices; each slice of both operands (16 KB + 16 KB) is copied global ->
// LDS by the DMA form of the vector load (global_load_lds_dwordx4, no
// registers involved) into one of four LDS stages, three slices ahead of
// the MFMAs.  The waits are explicit (s_waitcnt vmcnt + s_barrier, one
// barrier per slice): a plain __syncthreads would carry a release fence
// that drains every DMA in flight.  8 waves (2 per SIMD), each 64 canvas
// rows x 128 table rows; a single canvas of at most 128 rows runs 4 waves
// over its 128 rows instead (the same wave tile), the LM head then in a
// compact 3-stage ring so that two workgroups share a CU.
//
// Both operands are in the tiled layout of dg_tiled.h: a slice of a 256-row
// block is 16 KB of consecutive memory already in LDS order (chunk c of row
// r at position c ^ ((r >> 2) & 3), which keeps the 32 rows a fragment read
// touches, 16 lanes at a time, on distinct banks), so every DMA instruction
// copies 1 KB of consecutive bytes (the self-conditioning contraction's
// table slice: 8 runs of 2 KB, see TR below).
//
// The MFMA takes the table fragment as its first operand, so a lane's
// accumulators hold one canvas row and 16 of the 32 table rows of a
// fragment (its partner lane, lane ^ 32, holds the other 16): the softmax
// statistics over a 64-column tile are reduced in registers, with a single
// exchange between the two partner lanes.
#include "dg_device.h"
#include "dg_kernels.h"
#include "dg_tiled.h"

namespace dg {

namespace {
constexpr int ES_NT = 512;        // 8 waves
constexpr int ES_BM = 256;        // canvas rows per workgroup
constexpr int ES_BN = 256;        // table rows per workgroup
constexpr int ES_BK = 32;         // k per slice
constexpr int ES_CUS = 256;       // compute units of the part (a launch-shape choice only)
constexpr int ES_SLICE = ES_BM * ES_BK * 2;  // bytes of one operand slice (16 KB)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// LDS of a workgroup of NW waves (32 NW canvas rows) and STG stages: each
// stage holds the canvas operand's slice (NW * 2 KB) then the table's
// (16 KB), then come the exponents ([stage][256]) and fp4 scales
// ([stage][32]).  Four stages keep three slices in flight; so do three, by
// refilling the stage of the slice just read (its LDS reads are waited for
// before the barrier), in less LDS: the 4-wave LM head uses three, so that
// two of its workgroups share a CU.  The LM head stages its numerators
// (8 slices of NW * 2 KB) and statistics (32 NW rows x 64 bytes) in the
// same memory afterwards.
// A 16-byte store written through the L2 (system scope, sc0 sc1): the line
// is not left dirty in this XCD's L2 for the write-back at the kernel's end,
// which the next kernel would wait for.  The s_nop keeps the store's data
// registers from being rewritten in the cycle after it issues.
typedef int es_v4i_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_through(void *p, es_v4i_t v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1\n\ts_nop 1" ::"v"(p), "v"(v));
}

constexpr int es_abytes(int NW) { return NW * 2048; }
constexpr int es_stage_bytes(int NW) { return es_abytes(NW) + ES_SLICE; }
constexpr int es_lds(int NW, int STG) { return STG * (es_stage_bytes(NW) + 256 + 32); }
constexpr int es_lm_stages(int NW) { return NW == 8 ? 4 : 3; }
constexpr int es_lds_lm(int NW) {
  return es_lds(NW, es_lm_stages(NW)) > 9 * es_abytes(NW) ? es_lds(NW, es_lm_stages(NW)) : 9 * es_abytes(NW);
}
static_assert(ES_BM == TL_ROWS && ES_BN == TL_ROWS && ES_BK == TL_K, "slices are tiled-layout blocks");

// s_waitcnt immediate (gfx9 encoding): vmcnt <= n, no wait on exp, and on
// lgkm only with lgkm0 (then every LDS read issued has returned).
template <int n, bool lgkm0 = false>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | ((lgkm0 ? 0 : 0xF) << 8));
}

}  // namespace

// Accumulates acc[i][j] (wave tile: canvas rows wm*64 + 32i, table rows
// wn*128 + 32j) over the slices [sb, se) of two tiled blocks: At is the
// canvas block, Bt the table block (each 256 rows, slice s at + s * 8192).
// Layout of acc[i][j]: lane holds canvas row 32i + (lane & 31) and, in
// register r, table row 8 (r >> 2) + 4 (lane >> 5) + (r & 3) of the fragment.
// The operands are restrict-qualified parameters: the compiler then adds no
// wait of its own between the DMA copies and the LDS reads (the s_waitcnt /
// s_barrier pairs order them).
//
// SCALED: the canvas operand holds numerators whose scale is a power of two
// per (row, 64-column tile): value = stored * 2^-shift[t][row] with shift
// (uint8, tile-major [K/64][256]) copied into LDS beside each slice s by
// wave s % 8.  The scaling is exact integer arithmetic on the bf16 exponent
// field: a saturating subtraction of shift << 7 from each 16-bit value
// (positive values; anything scaled below the normal range becomes zero or
// a denormal).
//
// TF (the table's storage) = TF_FP8: the table operand is fp8 e4m3
// (q = E * 2^e) in the 8-byte-chunk tiled layout (8 KB per slice, one DMA
// instruction per wave); each table fragment is read as 8 bytes and turned
// into bf16 q * b8_scale (b8_scale = 2^-e: exact) before the MFMAs, so the
// accumulation is that of the bf16 table holding the same values.
// TF = TF_FP4: fp4 e2m1 with a power-of-two scale per 32 x 32 block
// (dg_tiled.h), 4 KB per slice copied by the low 32 lanes of every wave; a
// fragment is 8 codes widened to bf16 exactly by four
// v_cvt_scalef32_pk_bf16_fp4.  The 8 scale bytes of slice s (one per
// 32-row group of the table operand) are copied beside it by wave s % 8.
//
// TR: the table operand is read from E [K][...] itself, whose tiled blocks
// run along the table operand's k (the self-conditioning contraction,
// K = V): Bt is the table's base, the workgroup's 256 operand rows are the
// E columns of blocks tr_d0 .. tr_d0 + 7 (tr_ksd blocks per 256 E rows,
// indices past the last clamped: those columns are never stored), and
// slice s is rows 32 s .. 32 s + 31 of those 8 blocks, 8 runs of
// consecutive bytes (wave w copies block tr_d0 + w).  The fragments are
// transposed on the way out of LDS by the gfx950 transposing reads
// (ds_read_b64_tr_b16 / _b8 / _b4): within each 16-lane group, lane i gets
// element i + 16 e (e = 0, 1, ...) of the group's 16 consecutive 8-byte
// loads, so each lane addresses a short run of one E row and receives one
// E column.  Without TR, Bt is the workgroup's block row of the table (slice
// s at s blocks on) and Bs4 its scale bytes (slice s at Bs4 + 8 s); with TR
// Bs4 is the table's whole scale array.
template <bool SCALED, bool PAIR = false, int TF = TF_BF16, bool TR = false, int NW = 8, int STG = 4>
__device__ __forceinline__ void estream_tile(const bf16 *__restrict__ At, const uint8_t *__restrict__ Bt,
                                             const uint8_t *__restrict__ shift, int sb, int se, char *lds,
                                             f32x16_t (&acc)[2][4], const bf16 *__restrict__ At2 = nullptr,
                                             const uint8_t *__restrict__ shift2 = nullptr, float b8_scale = 1.f,
                                             const uint8_t *__restrict__ Bs4 = nullptr, int tr_ksd = 0,
                                             int tr_d0 = 0) {
  constexpr bool B8 = TF == TF_FP8, B4 = TF == TF_FP4, BQ = B8 || B4;
  static_assert(NW == 8 || (NW == 4 && !PAIR), "8 waves (256 canvas rows) or 4 (128 rows, one canvas)");
  static_assert(STG == 3 || STG == 4, "three or four LDS stages");
  // bytes of one 256 x 32 block of the table, and of one of its rows
  constexpr int BLK = B8 ? TL8_BYTES : B4 ? TL4_BYTES : TL_ELEMS * 2, ROWB = BLK / 256;
  // the table slice is copied in 8 parts of BLK / 8 bytes, part p by wave p % NW
  constexpr int NPART = 8 / NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, g = lane >> 5;

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = se - sb;
  if (nk <= 0) return;
  // DMA: this wave copies 2 KB of the canvas operand's slice (2 instructions
  // of 64 lanes x 16 bytes), chunks p = (2 wave + u) * 64 + lane: rows
  // 0 .. 32 NW - 1.
  // PAIR: rows 128..255 of the canvas operand (chunks 512..1023, copied by
  // waves 4..7) are rows 0..127 of a second block At2, and their exponents
  // (bytes 128..255 of a tile's row, lanes 32..63) rows 0..127 of shift2.
  const bf16 *asrc = (PAIR && wave >= 4) ? At2 + (int64_t)sb * TL_ELEMS + ((wave - 4) * 2 * 64 + lane) * 8
                                         : At + (int64_t)sb * TL_ELEMS + (wave * 2 * 64 + lane) * 8;
  const uint8_t *ssrc = !SCALED ? nullptr : (PAIR && lane >= 32) ? shift2 + (lane - 32) * 4 : shift + lane * 4;
  // this lane's 16 bytes of each DMA instruction of a table part: bf16
  // 2 instructions of 64 lanes per part, fp8 1, fp4 1 of 32 lanes
  const int blane = (B4 ? (lane & 31) : lane) * 16;
  const uint8_t *bsrc[NPART];
#pragma unroll
  for (int v = 0; v < NPART; ++v) {
    const int pt = wave + NW * v;
    bsrc[v] = TR ? Bt + (int64_t)min(tr_d0 + pt, tr_ksd - 1) * BLK + blane
                 : Bt + (int64_t)sb * BLK + pt * (BLK / 8) + blane;
  }
  constexpr int AB = es_abytes(NW), SB = es_stage_bytes(NW);
  char *lds_shift = lds + STG * SB;          // SCALED: [stage][256] bytes
  char *lds_s4 = lds_shift + STG * 256;      // B4: [stage][32] bytes, the slice's 8 scales
  auto issue = [&](int slice, int stage) {
    const int64_t off = (int64_t)min(slice, nk - 1) * TL_ELEMS;  // past the end: a repeat, never read
    char *st = lds + stage * SB;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      __builtin_amdgcn_global_load_lds(asrc + off + u * 512, st + (wave * 2 + u) * 1024, 16, 0, 0);
    }
    // the table slice: BLK / 8 bytes per part (rows 32 sg .. + 31 of column
    // block tr_d0 + p with TR, rows 32 p .. + 31 of the block otherwise)
    const int sg = sb + min(slice, nk - 1);
#pragma unroll
    for (int v = 0; v < NPART; ++v) {
      const uint8_t *bs = TR ? bsrc[v] + (int64_t)(sg >> 3) * tr_ksd * BLK + (sg & 7) * 32 * ROWB
                             : bsrc[v] + (int64_t)min(slice, nk - 1) * BLK;
      char *bd = st + AB + (wave + NW * v) * (BLK / 8);
      if (!BQ) {
#pragma unroll
        for (int u = 0; u < 2; ++u) __builtin_amdgcn_global_load_lds(bs + u * 1024, bd + u * 1024, 16, 0, 0);
      } else if (B8 || lane < 32) {
        __builtin_amdgcn_global_load_lds(bs, bd, 16, 0, 0);
      }
    }
    if (SCALED && wave == (slice & (NW - 1)))  // the slice tile's 256 row exponents, 4 bytes per lane
      __builtin_amdgcn_global_load_lds(ssrc + (int64_t)((sb + min(slice, nk - 1)) >> 1) * 256,
                                       lds_shift + stage * 256, 4, 0, 0);
    if (B4 && !TR && wave == (slice & (NW - 1)) && lane < 2)  // the slice's 8 block scales, 4 bytes per lane
      __builtin_amdgcn_global_load_lds(Bs4 + (int64_t)sg * 8 + lane * 4, lds_s4 + stage * 32, 4, 0, 0);
    if (B4 && TR && wave == (slice & (NW - 1)) && lane < 8)  // lane l: the 4 bytes holding block tr_d0 + l's scale
      __builtin_amdgcn_global_load_lds(
          Bs4 + (((int64_t)(sg >> 3) * tr_ksd + min(tr_d0 + lane, tr_ksd - 1)) * TL4_SCALES + ((sg & 7) & ~3)),
          lds_s4 + stage * 32, 4, 0, 0);
  };
  // DMA instructions per slice per wave: 2 for the canvas operand plus 2
  // (bf16) or 1 (fp8, fp4) per table part, plus XTRA more for wave s % NW
  // on slice s (exponents when SCALED, fp4 block scales)
  constexpr int PER = 2 + NPART * (BQ ? 1 : 2);
  constexpr int XTRA = (SCALED ? 1 : 0) + (B4 ? 1 : 0);

  // Fragment f of one 16-wide k step as stored: f < 2 a canvas fragment
  // (rows wm*64 + 32f), else table fragment f - 2 (rows wn*128 + 32(f-2)).
  // TR: table fragment j's E rows (slice rows v) and block (wn * 4 + j) in
  // LDS; the lane's place in its 16-lane group
  typedef short v4s_t __attribute__((ext_vector_type(4)));
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
  typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
  const int g16 = lane >> 4, i16 = lane & 15;
  auto tblk = [&](int stage, int j) -> const char * {
    return lds + stage * SB + AB + (wn * 4 + j) * (BLK / 8);
  };
  auto frag = [&](int stage, int kk, int f) -> uint4 {
    if (TR && f >= 2) {  // two 4-row reads: lane i16 gets column 16 (g16 & 1) + i16, rows 8 (g16 >> 1) + 0..7
      const char *b = tblk(stage, f - 2);
      const int c = 2 * (g16 & 1) + ((i16 >> 1) & 1), hf = i16 & 1;  // 4 columns 4 (i16 & 3) of the 16
      uint2 r[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int v = kk * 16 + 8 * (g16 >> 1) + 4 * u + (i16 >> 2);
        const v4s_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s_t *)(b + v * ROWB + (c ^ ((v >> 2) & 3)) * 16 + hf * 8));
        r[u] = __builtin_bit_cast(uint2, t);
      }
      return make_uint4(r[0].x, r[0].y, r[1].x, r[1].y);
    }
    const uint4 *sl = reinterpret_cast<const uint4 *>(lds + stage * SB + (f < 2 ? 0 : AB));
    const int row = f < 2 ? wm * 64 + f * 32 + r32 : wn * 128 + (f - 2) * 32 + r32;
    return sl[tl_pos(row, kk * 2 + g)];
  };
  // B8: the 8 fp8 bytes of table fragment j (rows wn*128 + 32j), and their bf16 form
  auto frag8 = [&](int stage, int kk, int j) -> uint2 {
    if (TR) {  // one read: lane i16 gets column 16 (g16 & 1) + i16, rows 8 (g16 >> 1) + 0..7
      const int v = kk * 16 + 8 * (g16 >> 1) + (i16 >> 1), c = 2 * (g16 & 1) + (i16 & 1);
      const v2i_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_v2i_t *)(tblk(stage, j) + (v * 4 + (c ^ (tl8_pos(v, 0) & 3))) * 8));
      return __builtin_bit_cast(uint2, t);
    }
    const uint2 *sl = reinterpret_cast<const uint2 *>(lds + stage * SB + AB);
    return sl[tl8_pos(wn * 128 + j * 32 + r32, kk * 2 + g)];
  };
  // B4: the 8 bytes holding table fragment j's 8 fp4 values for both k
  // halves of the slice (x: k half 0, y: k half 1).  Row fragment: row
  // wn*128 + 32j + r32, word g.  TR: one transposing read; lane i16 gets
  // rows kk * 16 + 8 (g16 >> 1) + 0..7 in word kk of E column
  // 8 w + i16 (i16 < 8) or 16 + 8 w + i16 - 8 (w = g16 & 1): the fragment's
  // 8-column groups 1 and 2 trade places (undone where the results are
  // stored).  Rows are stored at tl4_row (dg_tiled.h).
  auto frag4w = [&](int stage, int j) -> uint2 {
    if (TR) {
      const int h = g16 >> 1, v = tl4_row(i16 < 8 ? 8 * h + i16 : 16 + 8 * h + (i16 - 8)), w = g16 & 1;
      const v2i_t t = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
          (lds_v2i_t *)(tblk(stage, j) + v * 16 + 8 * (w ^ tl4_swz(v))));
      return __builtin_bit_cast(uint2, t);
    }
    const int row = tl4_row(wn * 128 + j * 32 + r32);
    return *reinterpret_cast<const uint2 *>(lds + stage * SB + AB + row * 16 +
                                            8 * (g ^ tl4_swz(row)));
  };
  // the scale bytes of this wave's four table fragments (byte j for the
  // fragment of rows wn*128 + 32j), broadcast reads of the stage holding
  // slice `slice`; fragment j's scale 2^(byte - 127).  TR: dword 4 wn + j
  // holds the fragment's byte at position (sg & 3).
  auto scales4 = [&](int stage, int slice) -> uint32_t {
    if (TR) {
      const uint4 w = *reinterpret_cast<const uint4 *>(lds_s4 + stage * 32 + wn * 16);
      const int sh = 8 * ((sb + min(slice, nk - 1)) & 3);
      return ((w.x >> sh) & 0xFFu) | (((w.y >> sh) & 0xFFu) << 8) | (((w.z >> sh) & 0xFFu) << 16) |
             (((w.w >> sh) & 0xFFu) << 24);
    }
    return *reinterpret_cast<const uint32_t *>(lds_s4 + stage * 32 + wn * 4);
  };
  auto scale4 = [](uint32_t w, int j) -> float { return __uint_as_float(((w >> (8 * j)) & 0xFFu) << 23); };
  auto widen4 = [&](uint32_t q, float sc) -> uint4 {
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 0)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 2)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 3)));
  };
  auto widen = [&](uint2 q) -> uint4 {
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, b8_scale, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, b8_scale, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, b8_scale, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, b8_scale, true)));
  };
  // SCALED: the exponent of canvas fragment i's row, and its packed form
  // (shift << 7 in both 16-bit halves)
  auto expo = [&](int stage, int i) -> uint32_t { return (uint8_t)lds_shift[stage * 256 + wm * 64 + i * 32 + r32]; };
  auto packed = [](uint32_t sh) -> u16x2_t { return __builtin_bit_cast(u16x2_t, (sh << 7) | (sh << 23)); };
  auto scale = [&](uint4 &v, u16x2_t e) {
    v.x = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, v.x), e));
    v.y = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, v.y), e));
    v.z = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, v.z), e));
    v.w = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, v.w), e));
    asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));  // computed here, not sunk past the barrier
  };
  // The 8 MFMAs of one k half with the 6 fragment reads of the next k half
  // interleaved (two after each of the first three MFMAs), each step pinned
  // in place, so a fragment is read a full k half before its first use.
  // With ex, the next half's exponents are read too (a new slice).
  uint32_t q4hi[4];  // B4: the second k half's codes of the current slice
  // nsl: the slice the next k half belongs to
  auto half = [&](const uint4 (&cur)[6], uint4 (&nxt)[6], int nstage, int nkk, bool ex, u16x2_t (&e)[2], int nsl) {
    uint32_t sh[2];
    uint2 q8[4];
    uint32_t q4[4], s4 = 0;  // B4: this half's codes (the second half's kept in q4hi)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int i = m >> 2, j = m & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cur[2 + j]),
                                                          __builtin_bit_cast(bf16x8_t, cur[i]), acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (m < 3) {
        if (!BQ || m == 0) {
          nxt[2 * m] = frag(nstage, nkk, 2 * m);
          nxt[2 * m + 1] = frag(nstage, nkk, 2 * m + 1);
        } else if (B8) {
          q8[2 * m - 2] = frag8(nstage, nkk, 2 * m - 2);
          q8[2 * m - 1] = frag8(nstage, nkk, 2 * m - 1);
        } else {
#pragma unroll
          for (int jj = 2 * m - 2; jj < 2 * m; ++jj) {
            if (nkk == 0) {  // a new slice: both halves' codes in one read
              const uint2 t = frag4w(nstage, jj);
              q4[jj] = t.x;
              q4hi[jj] = t.y;
            } else {
              q4[jj] = q4hi[jj];
            }
          }
          if (m == 1) s4 = scales4(nstage, nsl);
        }
        if (SCALED && ex && m == 0) {
          sh[0] = expo(nstage, 0);
          sh[1] = expo(nstage, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (B8) {  // while the last MFMAs run
#pragma unroll
      for (int j = 0; j < 4; ++j) nxt[2 + j] = widen(q8[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (B4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) nxt[2 + j] = widen4(q4[j], scale4(s4, j));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (SCALED) {  // while the last MFMAs run
      if (ex) {
        e[0] = packed(sh[0]);
        e[1] = packed(sh[1]);
      }
      scale(nxt[0], e[0]);
      scale(nxt[1], e[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Software pipeline: the barrier sits between the two k halves of a slice.
  // The second-half fragments of slice it are read during the first-half
  // MFMAs, the first-half fragments of slice it+1 (after the barrier) during
  // the second-half MFMAs.  At the barrier of iteration it every wave has
  // consumed slice it-1 (its second half ran before), so the DMA of slice
  // it+3 may refill that stage.
  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  uint4 F0[6], F1[6];
  u16x2_t ex[2];
  if (XTRA && (wave == 1 || wave == 2))
    wait_vmcnt<2 * PER + XTRA>();
  else
    wait_vmcnt<2 * PER>();
  __builtin_amdgcn_s_barrier();
  const uint32_t s40 = B4 ? scales4(0, 0) : 0u;
#pragma unroll
  for (int f = 0; f < 6; ++f) {
    if (B4 && f >= 2) {
      const uint2 t = frag4w(0, f - 2);
      q4hi[f - 2] = t.y;
      F0[f] = widen4(t.x, scale4(s40, f - 2));
    } else {
      F0[f] = (B8 && f >= 2) ? widen(frag8(0, 0, f - 2)) : frag(0, 0, f);
    }
  }
  if (SCALED) {
    ex[0] = packed(expo(0, 0));
    ex[1] = packed(expo(0, 1));
    scale(F0[0], ex[0]);
    scale(F0[1], ex[1]);
  }
  for (int it = 0; it < nk; ++it) {
    half(F0, F1, it % STG, 1, false, ex, it);  // second half of slice it, same exponents
    // this wave's copies of slice it+1 landed (with 3 stages also its LDS
    // reads of slice it returned) ...
    if (XTRA && wave == ((it + 2) & (NW - 1)))
      wait_vmcnt<PER + XTRA, STG == 3>();
    else
      wait_vmcnt<PER, STG == 3>();
    __builtin_amdgcn_s_barrier();  // ... every wave's; every wave is done with slice it-1 (3 stages: it)
    issue(it + 3, (it + 3) % STG);
    __builtin_amdgcn_sched_barrier(0);
    half(F1, F0, (it + 1) % STG, 0, true, ex, it + 1);  // past the last slice: a repeat, unused
  }
  wait_vmcnt<0>();  // retire the trailing (unused) prefetches before LDS is reused
  __builtin_amdgcn_s_barrier();
}

// ---------------------------------------------------------------------------
// LM head: workgroup = one 256-row block of the (stacked) canvas rows x 256
// vocabulary columns; a wave holds 64 rows x 128 columns = two 64-column
// tiles of the softmax statistics.  Per canvas row and tile a lane holds 32
// of the 64 logits (its partner lane the other 32): the max of z and its
// lowest column, exp(y - m) written once as bf16 (tiled layout), l = sum
// exp(y - m) and s = sum exp(y - m)(y - m), with y = z / T and m = zmax / T,
// are reduced in registers plus one exchange with the partner.
// Several canvases (a batch) stack their rows: stacked row r is row r % N of
// canvas r / N, whose numerators and statistics go to that canvas's buffers.
// With more than one row block, the blocks that read the same 256 table rows
// run back to back on one XCD, so the table tile comes from HBM once and from
// that XCD's L2 for the other blocks.
// ---------------------------------------------------------------------------
template <bool BATCH, int TF, int NW = 8>
__global__ void __launch_bounds__(NW * 64, NW == 8 ? 1 : 2)
    lm_head_es_kernel(const bf16 *__restrict__ At, int M, int N, int K, PackedTable tab, int V, float inv_T,
                      EsCanvases cv, int nblk, int items, float *__restrict__ logits) {
  extern __shared__ __align__(16) char lds[];
  // 4 waves: the canvas's rows in nh = ceil(M / 128) halves, item = (table
  // tile, half), the halves of a tile back to back on one XCD
  const int nh = NW == 8 ? 1 : (M + 127) / 128;
  int item = blockIdx.x;
  if (BATCH || nh > 1) item = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;  // grid: a multiple of 8
  if ((BATCH || nh > 1) && item >= items) return;
  const int jt = BATCH ? item / nblk : item / nh, bb = BATCH ? item % nblk : 0;
  const int r0 = NW == 8 ? 0 : (item % nh) * 128;  // the workgroup's first canvas row
  const int n0 = jt * ES_BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 5;
  const int ksl = K / ES_BK;
  f32x16_t acc[2][4];
  constexpr int BLK = TF == TF_FP8 ? TL8_BYTES : TF == TF_FP4 ? TL4_BYTES : TL_ELEMS * 2;
  estream_tile<false, false, TF, false, NW, es_lm_stages(NW)>(At + (int64_t)bb * ksl * TL_ELEMS + r0 * ES_BK,
                                 static_cast<const uint8_t *>(tab.p) + (int64_t)jt * ksl * BLK, nullptr, 0, ksl, lds,
                                 acc, nullptr, nullptr, tab.scale,
                                 TF == TF_FP4 ? tab.s4 + (int64_t)jt * ksl * TL4_SCALES : nullptr);
  const int ntiles = V / 64;
  // The numerators and statistics are staged in LDS (free once the ring has
  // drained) and leave as contiguous runs: each canvas row's 64 bytes of a
  // 32-column slice, and its 4 tiles' statistics, are consecutive in the
  // canvas's buffers, so a wave stores 1 KB runs instead of 8-byte pieces
  // of 64-byte lines.  Staging: slice ls (0..7) at ls * 16 KB, row r's
  // chunks at r * 64 in stored order (tl_pos of the canvas's own row);
  // statistics at 8 * (NW * 2 KB) + r * 64 + 16 * (local tile xor r / 4 mod 4).
  constexpr int AB = es_abytes(NW);
  char *stage_num = lds, *stage_st = lds + 8 * AB;

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wm * 64 + i * 32 + (lane & 31);
    const int grow = bb * ES_BM + r0 + row;  // stacked row
    const int c = BATCH ? min(grow, M - 1) / N : 0, lrow = grow - c * N;  // c < M / N even past the last row
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tile = (n0 + wn * 128 + h * 64) / 64;
      // lane's columns: tile*64 + 32jj + 8q + 4g + t for jj < 2, q < 4, t < 4
      // (register r = 4q + t of fragment 2h + jj), increasing in (jj, r)
      const int cbase = tile * 64 + 4 * g;
      float best = acc[i][2 * h][0];
      int bcol = cbase;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float z = acc[i][2 * h + jj][r];
          if (z > best) {
            best = z;
            bcol = cbase + 32 * jj + 8 * (r >> 2) + (r & 3);
          }
        }
      {
        const float ov = __shfl_xor(best, 32);
        const int oc = __shfl_xor(bcol, 32);
        if (ov > best || (ov == best && oc < bcol)) {
          best = ov;
          bcol = oc;
        }
      }
      const float m = best * inv_T;
      // stored numerators are 2^(y log2e - r) = exp(y - m) * f with
      // r = ceil(m log2e) and f = 2^-(r - m log2e): the tile's reference is
      // a power of two (see row_combine).  Each is one fma and one exp2,
      // x = z (log2e / T) - r; l = sum exp(y - m) and s = sum exp(y - m)(y - m)
      // follow from the sums of n = 2^x and n x, since y - m = (x + dl) / log2e
      // with dl = r - m log2e.  The hardware exp2 returns no denormals: a
      // term below 2^-126 of the tile's largest counts as zero.
      const float r = ceilf(m * LOG2E), dl = r - m * LOG2E, c1 = inv_T * LOG2E;
      float ln = 0.f, sn = 0.f;
      uint32_t pk[2][8];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float x0 = fmaf(acc[i][2 * h + jj][v], c1, -r), x1 = fmaf(acc[i][2 * h + jj][v + 1], c1, -r);
          const float n0 = __builtin_amdgcn_exp2f(x0), n1 = __builtin_amdgcn_exp2f(x1);
          ln += n0 + n1;
          sn = fmaf(n0, x0, fmaf(n1, x1, sn));
          pk[jj][v >> 1] = pack_bf16x2(n0, n1);
        }
      ln += __shfl_xor(ln, 32);
      sn += __shfl_xor(sn, 32);
      const float inv_f = __builtin_amdgcn_exp2f(dl), l = ln * inv_f, sacc = fmaf(dl, ln, sn) * (inv_f * LN2);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        // local slice wn * 4 + 2h + jj; the lane's four values of chunk q are elements 4g..4g+3
        char *sl = stage_num + (wn * 4 + 2 * h + jj) * AB + row * 64 + g * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *reinterpret_cast<uint2 *>(sl + (q ^ ((lrow >> 2) & 3)) * 16) = make_uint2(pk[jj][2 * q], pk[jj][2 * q + 1]);
          if (logits && grow < M) {
            const f32x16_t &z = acc[i][2 * h + jj];
            *reinterpret_cast<float4 *>(logits + (int64_t)grow * V + cbase + 32 * jj + 8 * q) =
                make_float4(z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]);
          }
        }
      }
      if (g == 0)  // local tile wn * 2 + h at slot (tile ^ (row / 4 mod 4)): 32 rows on distinct banks
        *reinterpret_cast<float4 *>(stage_st + row * 64 + ((wn * 2 + h) ^ ((row >> 2) & 3)) * 16) =
            make_float4(best, l, sacc, __int_as_float(bcol));
    }
  }
  __syncthreads();
  // copy out: thread t moves the 16-byte chunk t % 4 of rows t / 4 and
  // t / 4 + 128, in each of the 8 slices and of the statistics
  const int u4 = threadIdx.x & 3;
#pragma unroll
  for (int rh = 0; rh < 2; ++rh) {
    const int row = (threadIdx.x >> 2) + rh * NW * 16;  // rows 0 .. 32 NW - 1
    const int grow = bb * ES_BM + r0 + row;
    if (grow >= M) continue;
    const int c = BATCH ? grow / N : 0, lrow = grow - c * N;
    char *dst = reinterpret_cast<char *>(cv.probs[c]) + (int64_t)(n0 / 32) * ES_SLICE + lrow * 64 + u4 * 16;
    const char *src = stage_num + row * 64 + u4 * 16;
    es_v4i_t v[8];
#pragma unroll
    for (int ls = 0; ls < 8; ++ls) v[ls] = *reinterpret_cast<const es_v4i_t *>(src + ls * AB);
#pragma unroll
    for (int ls = 0; ls < 8; ++ls) store_through(dst + ls * ES_SLICE, v[ls]);
    reinterpret_cast<uint4 *>(cv.tile_stats[c] + (int64_t)lrow * ntiles + n0 / 64)[u4] =
        *reinterpret_cast<const uint4 *>(stage_st + row * 64 + (u4 ^ ((row >> 2) & 3)) * 16);
  }
}


int estream_bm(int) { return ES_BM; }

// the self-conditioning contraction: four stages (one workgroup per CU)
static size_t es_lds_bytes(int NW = 8) { return (size_t)(NW == 8 ? es_lds(8, 4) : es_lds(4, 4)); }
// the LM head also stages its numerators and statistics
static size_t es_lds_bytes_lm(int NW = 8) { return (size_t)(NW == 8 ? es_lds_lm(8) : es_lds_lm(4)); }

static bool table_ok(const PackedTable &t, int d) {
  return t.p && t.d == d && (t.tf == TF_BF16 || t.tf == TF_FP8 || (t.tf == TF_FP4 && t.s4));
}

hipError_t lm_head_bf16_batch(const uint16_t *A_tiled, int B, int N, int K, const PackedTable &tab, int V,
                              float inv_T, const EsCanvases &cv, float *logits_dump, hipStream_t s) {
  if (B < 1 || B > ES_MAX_BATCH || N < 1 || N > ES_BM || K % ES_BK || V % ES_BN) return hipErrorInvalidValue;
  if (!table_ok(tab, K)) return hipErrorInvalidValue;
  static std::atomic<uint64_t> attr{0};
  if (once_per_device(attr, [] {
        const void *fns[9] = {reinterpret_cast<const void *>(lm_head_es_kernel<false, TF_BF16>),
                              reinterpret_cast<const void *>(lm_head_es_kernel<true, TF_BF16>),
                              reinterpret_cast<const void *>(lm_head_es_kernel<false, TF_FP8>),
                              reinterpret_cast<const void *>(lm_head_es_kernel<true, TF_FP8>),
                              reinterpret_cast<const void *>(lm_head_es_kernel<false, TF_FP4>),
                              reinterpret_cast<const void *>(lm_head_es_kernel<true, TF_FP4>),
                              reinterpret_cast<const void *>(lm_head_es_kernel<false, TF_BF16, 4>),
                              reinterpret_cast<const void *>(lm_head_es_kernel<false, TF_FP8, 4>),
                              reinterpret_cast<const void *>(lm_head_es_kernel<false, TF_FP4, 4>)};
        for (const void *f : fns) {
          const hipError_t e =
              hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)es_lds_bytes_lm());
          if (e != hipSuccess) return e;
        }
        return hipSuccess;
      }) != hipSuccess)
    return hipErrorInvalidValue;
  const int M = B * N, nblk = (M + ES_BM - 1) / ES_BM;
  // one canvas runs 4-wave workgroups over 128-row halves when it has at
  // most 128 rows, or when its table has fewer 256-row tiles than the chip
  // has CUs (so 8-wave workgroups would leave CUs idle; with the CUs full,
  // copying each table slice into LDS twice costs more than it returns)
  const bool narrow = B == 1 && (2 * N <= ES_BM || V / ES_BN < ES_CUS);
  const int items = (V / ES_BN) * (narrow ? (N + 127) / 128 : nblk);
  const dim3 grid(B == 1 && 2 * N <= ES_BM ? items : (items + 7) / 8 * 8);
  // one canvas of at most 128 rows: 4 waves over its 128 rows, not 8 over
  // 256 with half of them padding
#define DG_LM_LAUNCH(BT, TF, NW)                                                                      \
  hipLaunchKernelGGL((lm_head_es_kernel<BT, TF, NW>), grid, dim3(NW * 64), es_lds_bytes_lm(NW), s, A_tiled, M, N, K, \
                     tab, V, inv_T, cv, nblk, items, logits_dump)
#define DG_LM_FORMS(BT, NW)                                   \
  do {                                                        \
    if (tab.tf == TF_FP8) DG_LM_LAUNCH(BT, TF_FP8, NW);       \
    else if (tab.tf == TF_FP4) DG_LM_LAUNCH(BT, TF_FP4, NW);  \
    else DG_LM_LAUNCH(BT, TF_BF16, NW);                       \
  } while (0)
  if (narrow) DG_LM_FORMS(false, 4);
  else if (B == 1) DG_LM_FORMS(false, 8);
  else DG_LM_FORMS(true, 8);
#undef DG_LM_FORMS
#undef DG_LM_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Self-conditioning contraction, split over K = V: work item (kc, nt, c) =
// K-chunk kc of canvas c x 256 columns of d.  The hardware hands consecutive
// workgroups to the 8 XCDs in turn; the mapping below gives consecutive work
// items to workgroups of one XCD, so the items of one K-chunk (which share
// each canvas's chunk of probabilities, and across canvases each chunk of
// the table) run on one XCD where they can and fetch the shared data into
// its L2 once.
// ---------------------------------------------------------------------------
// MODE: 0 one canvas; 1 a batch, one canvas per 256-row block; 2 a batch of
// canvases of at most 128 rows, two per block (canvas 2p in rows 0..127,
// canvas 2p + 1 in rows 128..255, read from its own buffers); 3 one canvas
// of at most 128 rows, 4 waves over its 128 rows.
template <bool SCALED, int MODE, int TF>
__global__ void __launch_bounds__(MODE == 3 ? ES_NT / 2 : ES_NT, 1)
    selfcond_es_kernel(EsCanvasesIn cin, PackedTable tab, int M, int N, int K, float *__restrict__ part, int ksplit,
                       int ntn, int nb, int items, SelfcondGuard guard) {
  extern __shared__ __align__(16) char lds[];
  const int b = blockIdx.x, ng = gridDim.x;
  const int per_xcd = ng / 8;  // grid is a multiple of 8
  const int item = (b % 8) * per_xcd + b / 8;
  if (item >= items || guard.stopped()) return;
  const int nblk = MODE == 2 ? (nb + 1) / 2 : nb;  // canvas operand blocks
  constexpr bool ONE = MODE == 0 || MODE == 3;
  const int blk = ONE ? 0 : item % nblk, kn = ONE ? item : item / nblk;
  const int kc = kn / ntn, nt = kn % ntn;
  const int ksl = K / ES_BK;
  const int sb = (int)((int64_t)ksl * kc / ksplit), se = (int)((int64_t)ksl * (kc + 1) / ksplit);
  const int n0 = nt * ES_BN;
  f32x16_t acc[2][4];
  // the table E [K][N] read transposed: columns n0 .. n0 + 255 are its blocks 8 nt .. 8 nt + 7
  const uint8_t *Bt = static_cast<const uint8_t *>(tab.p);
  const int ksd = N / ES_BK;
  if (MODE == 2) {
    const int c0 = 2 * blk, c1 = c0 + 1;
    // an odd batch's last block: its upper half is the canvas's own padding rows
    const bf16 *A2 = c1 < nb ? cin.probs[c1] : cin.probs[c0] + 512 * 8;
    const uint8_t *s2 = c1 < nb ? cin.shift[c1] : cin.shift[c0] + 128;
    estream_tile<SCALED, true, TF, true>(cin.probs[c0], Bt, cin.shift[c0], sb, se, lds, acc, A2, s2, tab.scale,
                                         tab.s4, ksd, 8 * nt);
  } else {
    estream_tile<SCALED, false, TF, true, MODE == 3 ? 4 : 8>(cin.probs[blk], Bt, cin.shift[blk], sb, se, lds, acc,
                                                            nullptr, nullptr, tab.scale, tab.s4, ksd, 8 * nt);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // the block of partials in register order (selfcond_part_bytes): each
  // store instruction writes 64 lanes x 16 consecutive bytes
  float *out = part + ((((int64_t)blk * ksplit + kc) * ntn + nt) << 16);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wm * 64 + i * 32 + (lane & 31);
    const int c = MODE == 2 ? 2 * blk + (row >> 7) : blk, lrow = MODE == 2 ? row & 127 : row;
    if (lrow >= M || c >= nb) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // registers 4q..4q+3 are four consecutive columns, 8-column group qc
        // of the fragment (the fp4 table's transposing read swaps groups 1
        // and 2); the slot is that of group qc
        const int qc = TF == TF_FP4 ? ((q & 1) << 1) | (q >> 1) : q;
        const int col = n0 + wn * 128 + j * 32 + 8 * qc + 4 * (lane >> 5);
        if (col < N)
          store_through(out + (((((wave * 2 + i) * 4 + j) * 4 + qc) * 64 + lane) << 2),
                        es_v4i_t{__float_as_int(acc[i][j][4 * q]), __float_as_int(acc[i][j][4 * q + 1]),
                                 __float_as_int(acc[i][j][4 * q + 2]), __float_as_int(acc[i][j][4 * q + 3])});
      }
  }
}

hipError_t selfcond_bf16_batch(const EsCanvasesIn &cin, int B, const PackedTable &tab, int M, int N, int K,
                               bool scaled, float *partials, int ksplit, hipStream_t s, SelfcondGuard guard) {
  if (B < 1 || B > ES_MAX_BATCH || M > ES_BM || K % 256 || N % ES_BK || ksplit < 1 || ksplit > K / ES_BK)
    return hipErrorInvalidValue;
  if (!table_ok(tab, N)) return hipErrorInvalidValue;
  static std::atomic<uint64_t> attr{0};
  if (once_per_device(attr, [] {
#define DG_SC_FN(SC, MD, TF) reinterpret_cast<const void *>(selfcond_es_kernel<SC, MD, TF>)
#define DG_SC_FN8(TF) \
  DG_SC_FN(false, 0, TF), DG_SC_FN(true, 0, TF), DG_SC_FN(false, 1, TF), DG_SC_FN(true, 1, TF), \
      DG_SC_FN(false, 2, TF), DG_SC_FN(true, 2, TF), DG_SC_FN(false, 3, TF), DG_SC_FN(true, 3, TF)
        const void *fns[24] = {DG_SC_FN8(TF_BF16), DG_SC_FN8(TF_FP8), DG_SC_FN8(TF_FP4)};
#undef DG_SC_FN8
#undef DG_SC_FN
        for (const void *f : fns) {
          const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)es_lds_bytes());
          if (e != hipSuccess) return e;
        }
        return hipSuccess;
      }) != hipSuccess)
    return hipErrorInvalidValue;
  const int mode = B == 1 ? (2 * M <= ES_BM ? 3 : 0) : (selfcond_paired(B, M) ? 2 : 1);
  const int ntn = (N + ES_BN - 1) / ES_BN;
  const int items = ntn * ksplit * (mode == 2 ? (B + 1) / 2 : B);
  const dim3 grid((items + 7) / 8 * 8);
#define DG_SC_LAUNCH(SC, MD, TF)                                                                                 \
  hipLaunchKernelGGL((selfcond_es_kernel<SC, MD, TF>), grid, dim3(MD == 3 ? ES_NT / 2 : ES_NT),                   \
                     es_lds_bytes(MD == 3 ? 4 : 8), s, \
                     cin, tab, M, N, K, partials, ksplit, ntn, B, items, guard)
#define DG_SC_MODES(SC, TF)                      \
  do {                                           \
    if (mode == 0) DG_SC_LAUNCH(SC, 0, TF);      \
    else if (mode == 1) DG_SC_LAUNCH(SC, 1, TF); \
    else if (mode == 2) DG_SC_LAUNCH(SC, 2, TF); \
    else DG_SC_LAUNCH(SC, 3, TF);                \
  } while (0)
#define DG_SC_FORMS(SC)                                \
  do {                                                 \
    if (tab.tf == TF_FP8) DG_SC_MODES(SC, TF_FP8);      \
    else if (tab.tf == TF_FP4) DG_SC_MODES(SC, TF_FP4); \
    else DG_SC_MODES(SC, TF_BF16);                     \
  } while (0)
  if (scaled) DG_SC_FORMS(true);
  else DG_SC_FORMS(false);
#undef DG_SC_FORMS
#undef DG_SC_MODES
#undef DG_SC_LAUNCH
  return hipGetLastError();
}

}  // namespace dg
