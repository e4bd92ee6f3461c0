// dg_device.h -- device-side helpers shared by the libdgdenoise kernels
// (gfx950 / CDNA4).  bf16 is carried as raw 16-bit words; conversions are
// written out so that every kernel rounds the same way (round to nearest
// even, NaN kept quiet).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef uint16_t bf16;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(bf16 h) { return __uint_as_float(((uint32_t)h) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed pair of bf16 (low word = a), round to nearest even,
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ bf16 f32_to_bf16(float f) { return (bf16)(pack_bf16x2(f, 0.f) & 0xffffu); }

// Split of a float into two bf16 terms, x = hi + lo with hi = bf16(x) and
// lo = bf16(x - hi): 16 significant bits, so a product against an exact
// bf16 operand costs two MFMAs and stays within ~1e-5 of fp32.  The pair
// form below packs two consecutive values per 32-bit word.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
__device__ __forceinline__ void split4(const float4 v, uint2 &hi, uint2 &lo) {
  split2(v.x, v.y, hi.x, lo.x);
  split2(v.z, v.w, hi.y, lo.y);
}
__device__ __forceinline__ void split8(const float4 a, const float4 b, uint4 &hi, uint4 &lo) {
  split2(a.x, a.y, hi.x, lo.x);
  split2(a.z, a.w, hi.y, lo.y);
  split2(b.x, b.y, hi.z, lo.z);
  split2(b.z, b.w, hi.w, lo.w);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16> {
  static __device__ __forceinline__ float load(const bf16 *p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(bf16 *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds, each two
// 32x32 -> 64-bit products (multipliers 0xD2511F53, 0xCD9E8D57) mixed with
// the key, which is bumped by the Weyl increments 0x9E3779B9 / 0xBB67AE85
// between rounds.
struct Philox4 {
  uint32_t v[4];
};
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  Philox4 o;
  o.v[0] = c0;
  o.v[1] = c1;
  o.v[2] = c2;
  o.v[3] = c3;
  return o;
}

// Uniform token in [0, 2^log2v): top bits of Philox word 0, key = seed,
// counter = (pos, step, canvas, stream).
__device__ __forceinline__ int32_t uniform_token(uint64_t seed, uint32_t pos, uint32_t step,
                                                 uint32_t canvas, uint32_t stream, int log2v) {
  const Philox4 o = philox4x32_10(pos, step, canvas, stream, (uint32_t)seed, (uint32_t)(seed >> 32));
  return (int32_t)(o.v[0] >> (32 - log2v));
}

// Multinomial candidate ([P3] §5.3: the token is drawn from the tempered
// softmax) by Gumbel-max: argmax_v (ln w_v + G_v) with independent standard
// Gumbel G_v draws v with probability w_v / sum w.  Everything below is
// single precision with every operation rounded on its own (no fused
// multiply-add: contraction is off in these bodies; the division is the
// correctly rounded one), so the draw is a fixed function of its float
// inputs and reproduces bit for bit.
//
// Natural log of a positive normal float: x = m 2^e with m folded into
// (sqrt(1/2), sqrt(2)], ln m = 2 atanh(s), s = (m - 1) / (m + 1), by the odd
// series to the s^9 term (|s| <= 0.1716), and e ln 2 with ln 2 split so that
// e times the high part is exact.
__device__ __forceinline__ float ln_fixed(float x) {
#pragma clang fp contract(off)
  const uint32_t b = __float_as_uint(x);
  int e = (int)((b >> 23) & 0xFFu) - 127;
  float m = __uint_as_float((b & 0x7FFFFFu) | 0x3F800000u);
  if (m > 1.41421353816986083984375f) {  // the float nearest sqrt(2)
    m = m * 0.5f;
    e = e + 1;
  }
  const float f = m - 1.0f;
  const float s = f / (2.0f + f);
  const float z = s * s;
  const float P = z * (0.666666686534881591796875f +                  // float(2/3)
                       z * (0.4000000059604644775390625f +            // float(2/5)
                            z * (0.2857142984867095947265625f +       // float(2/7)
                                 z * 0.2222222238779067993164062f)));  // float(2/9)
  const float lnm = (s + s) + s * P;
  const float ef = (float)e;
  return ef * 0.693145751953125f + (ef * 1.42860676533018704e-6f + lnm);  // ln 2 = hi + lo
}

// Standard Gumbel variable of a 32-bit random word: u = (2 floor(w/512) + 1)
// 2^-24, exact in float and inside (0, 1); G = -ln(-ln u).
__device__ __forceinline__ float gumbel_word(uint32_t w) {
#pragma clang fp contract(off)
  const float u = (float)(2u * (w >> 9) + 1u) * 5.9604644775390625e-8f;
  return -ln_fixed(-ln_fixed(u));
}

// Gumbel-max keys of weights given in the linear domain; a weight that is
// not a positive finite normal float (zero, subnormal, inf, NaN) gets -inf
// and is never drawn.
//   tile level: fl(fl(ln l + fl(zmax inv_T)) + G(word))  (mass l e^{zmax inv_T})
//   column level: fl(ln w + G(word))
__device__ __forceinline__ float gumbel_key_tile(float l, float zmax, float inv_T, uint32_t word) {
#pragma clang fp contract(off)
  if (!(l >= 1.17549435e-38f && l <= 3.40282347e38f)) return -INFINITY;
  const float m = zmax * inv_T;
  const float lx = ln_fixed(l) + m;
  return lx + gumbel_word(word);
}
__device__ __forceinline__ float gumbel_key_col(float w, uint32_t word) {
#pragma clang fp contract(off)
  if (!(w >= 1.17549435e-38f && w <= 3.40282347e38f)) return -INFINITY;
  return ln_fixed(w) + gumbel_word(word);
}

// 64-bit lane exchanges of a wavefront, as two 32-bit shuffles
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o), hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int o) {
  const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)v, o), hi = (uint32_t)__shfl_up((int)(uint32_t)(v >> 32), o);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace dg
