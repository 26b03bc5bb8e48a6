// Device-side group quantizer shared by the append and calibration kernels.
//
// One thread quantizes one group of 32 values (keys: 32 channels of a token; values: 32
// tokens of a channel — grouping along the inner dimension, InnerQ "Core claim").
// Every step is an IEEE operation in the order written; this file must be compiled with
// -ffp-contract=off so that no multiply-add is fused:
//   asymmetric: s = f16(fl32(max - min) / fl32(2^b - 1)), z = f16(min + 0),
//               c = clamp(rint(fl32(fl32(x - z) * fl32(1/s))), 0, 2^b - 1)  (s == 0: c = 0)
//   symmetric:  s = f16(fl32(max|x|) / fl32(2^(b-1) - 1)), z = -2^(b-1) s,
//               c = clamp(rint(fl32(x * fl32(1/s))), -(2^(b-1)-1), 2^(b-1)-1) + 2^(b-1)
//   both dequantize as x_hat = c s + z; hybrid (InnerQ technique (i)) keeps the variant
//   whose float64 squared error (summed over elements 0..31 in order) is strictly lower,
//   ties to asymmetric.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

__device__ __forceinline__ float widen16(uint16_t raw, int dtype) {
  if (dtype == KVQ_BF16) return __uint_as_float((uint32_t)raw << 16);
  return __half2float(__ushort_as_half(raw));
}

__device__ __forceinline__ uint16_t f16_bits(float x) {  // round to nearest even
  return __half_as_ushort(__float2half_rn(x));
}
__device__ __forceinline__ float f16_value(uint16_t h) { return __half2float(__ushort_as_half(h)); }

struct GroupQ {
  float s, z, r;        // stored s, z as float; r = fl32(1 / s)
  uint16_t s_bits, z_bits;
  float lo, hi;         // clamp range of rint(t)
  int add;              // code = clamped value + add
  bool sym, zero;       // zero: s == 0 (every code is the zero level)
};

__device__ __forceinline__ GroupQ asym_params(const float (&x)[32], int b) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  GroupQ q;
  const float L = (float)((1 << b) - 1);
  q.s_bits = f16_bits((mx - mn) / L);
  q.z_bits = f16_bits(mn + 0.0f);  // + 0 stores a zero minimum as +0 whatever its sign
  q.s = f16_value(q.s_bits);
  q.z = f16_value(q.z_bits);
  q.zero = (q.s == 0.0f);
  q.r = 1.0f / q.s;
  q.lo = 0.0f;
  q.hi = L;
  q.add = 0;
  q.sym = false;
  return q;
}

__device__ __forceinline__ GroupQ sym_params(const float (&x)[32], int b) {
  float m = fabsf(x[0]);
#pragma unroll
  for (int i = 1; i < 32; ++i) m = fmaxf(m, fabsf(x[i]));
  GroupQ q;
  const int half = 1 << (b - 1);
  const float Q = (float)(half - 1);
  q.s_bits = f16_bits(m / Q);
  q.s = f16_value(q.s_bits);
  q.z_bits = f16_bits(-(float)half * q.s);  // exact: power-of-two multiple of an fp16 value
  q.z = f16_value(q.z_bits);
  q.zero = (q.s == 0.0f);
  q.r = 1.0f / q.s;
  q.lo = -Q;
  q.hi = Q;
  q.add = half;
  q.sym = true;
  return q;
}

__device__ __forceinline__ int code_of(float x, const GroupQ& q) {
  if (q.zero) return q.sym ? q.add : 0;
  const float t = q.sym ? x * q.r : (x - q.z) * q.r;
  const float c = fminf(fmaxf(rintf(t), q.lo), q.hi);
  return (int)c + q.add;
}

// sum_i (x_i - (c_i s + z))^2 in float64, elements in order, no fused multiply-add
__device__ __forceinline__ double group_sse(const float (&x)[32], const GroupQ& q) {
  const double s = (double)q.s, z = (double)q.z;
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double xh = (double)code_of(x[i], q) * s + z;
    const double d = (double)x[i] - xh;
    const double sq = d * d;
    acc = acc + sq;
  }
  return acc;
}

// Quantizer for one group: asymmetric, or the hybrid choice.
__device__ __forceinline__ GroupQ choose_quant(const float (&x)[32], int b, bool hybrid) {
  GroupQ a = asym_params(x, b);
  if (!hybrid) return a;
  GroupQ s = sym_params(x, b);
  const double ea = group_sse(x, a);
  const double es = group_sse(x, s);
  return es < ea ? s : a;
}

__device__ __forceinline__ bool out_of_range(const float (&x)[32]) {
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) bad |= !(fabsf(x[i]) <= 16384.0f);  // also catches NaN
  return bad;
}

// Codes of one variant for the 32 elements, packed at stream bits [i*B, i*B+B) of w, and
// (when SSE) the float64 squared error of group_sse, computed with the same operations in
// the same order.
template <int B, bool SSE>
__device__ __forceinline__ double codes_sse(const float (&x)[32], const GroupQ& q, uint32_t (&w)[B]) {
#pragma unroll
  for (int k = 0; k < B; ++k) w[k] = 0u;
  const double s = (double)q.s, z = (double)q.z;
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int c = code_of(x[i], q);
    const int pos = i * B, wi = pos >> 5, off = pos & 31;
    w[wi] |= (uint32_t)c << off;
    if (off + B > 32) w[wi + 1] |= (uint32_t)c >> (32 - off);
    if constexpr (SSE) {
      const double xh = (double)c * s + z;
      const double d = (double)x[i] - xh;
      const double sq = d * d;
      acc = acc + sq;
    }
  }
  return acc;
}

// choose_quant with the codes of the chosen variant packed into w (one code pass per variant).
template <int B>
__device__ __forceinline__ GroupQ quantize_pack(const float (&x)[32], bool hybrid, uint32_t (&w)[B]) {
  const GroupQ a = asym_params(x, B);
  if (!hybrid) {
    (void)codes_sse<B, false>(x, a, w);
    return a;
  }
  const double ea = codes_sse<B, true>(x, a, w);
  const GroupQ s = sym_params(x, B);
  uint32_t ws[B];
  const double es = codes_sse<B, true>(x, s, ws);
  if (es < ea) {
#pragma unroll
    for (int k = 0; k < B; ++k) w[k] = ws[k];
    return s;
  }
  return a;
}

// Pack the 32 codes of a group into b little-endian words (code i at stream bits
// [i*b, i*b+b)) and hand each finished word to store(word_index, word).
template <class Store>
__device__ __forceinline__ void pack_group(const float (&x)[32], const GroupQ& q, int b, Store store) {
  uint64_t acc = 0;
  int nbits = 0, w = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    acc |= (uint64_t)(uint32_t)code_of(x[i], q) << nbits;
    nbits += b;
    if (nbits >= 32) {
      store(w, (uint32_t)acc);
      ++w;
      acc >>= 32;
      nbits -= 32;
    }
  }
}

// ---------------------------------------------------------------------------------------
// The append kernel's forms of the same quantizer: identical codes, scales, zeros and
// choices, in fewer instructions.
//
// Rounding by addition. With t = fl32(fl32(x - z) * r) (asymmetric) or fl32(x * r)
// (symmetric), and M = 2^23 + a (a = 0, or 2^(b-1) for the symmetric offset), fl32(t + M) is
// M + rint(t) whenever M + t lies in [2^23, 2^24): the spacing there is 1 and IEEE addition
// rounds to the nearest integer with ties to the even one, which is rint's tie rule because M
// is even. Its fp32 bit pattern is 0x4B000000 + a + rint(t), so the code plus 0x4B000000 comes
// out of one addition, and the clamp of rint(t) to its range is an unsigned clamp of the
// pattern (positive floats order like their patterns, so a sum that falls below 2^23 clamps
// to the lowest code). |t| stays far below 2^22 for inputs within the range limit.
constexpr uint32_t kTwo23Bits = 0x4B000000u;  // fp32 bit pattern of 2^23

struct FastForm {
  float r;          // 1 / s, or 0 when s == 0 (every t is 0: the zero level)
  float z;          // the zero subtracted before the product (asymmetric only)
  float m;          // 2^23 + a
  uint32_t lo, hi;  // pattern range of the codes
};

template <bool SYM>
__device__ __forceinline__ FastForm fast_form(const GroupQ& q) {
  FastForm f;
  f.r = q.zero ? 0.0f : q.r;
  f.z = q.z;
  f.m = 8388608.0f + (float)q.add;
  f.lo = kTwo23Bits + (uint32_t)((int)q.lo + q.add);
  f.hi = kTwo23Bits + (uint32_t)((int)q.hi + q.add);
  return f;
}

// code + 0x4B000000 of element x (code_of's value)
template <bool SYM>
__device__ __forceinline__ uint32_t code_pattern(float x, const FastForm& f) {
  const float t = SYM ? x * f.r : (x - f.z) * f.r;
  const uint32_t u = __float_as_uint(t + f.m);
  return min(max(u, f.lo), f.hi);
}

// The squared errors of group_sse from code patterns take c s + z as one fused operation:
// c s is exact in float64 (an 8-bit integer times an fp16 value), so the fused sum rounds
// once, as the separate product and sum do.

// What the patterns' constant 0x4B000000 adds to word k when element i's pattern is added in
// at stream bit i * B (mod 2^32; a code that crosses into the next word adds its top there).
__host__ __device__ constexpr uint32_t magic_in_word(int B, int i, int k) {
  const int pos = i * B, wi = pos >> 5, off = pos & 31;
  uint32_t c = 0u;
  if (wi == k) c += kTwo23Bits << off;
  if (off + B > 32 && wi + 1 == k) c += kTwo23Bits >> (32 - off);
  return c;
}

template <int B>
struct MagicTotals {  // v[k]: the constant part of word k once all 32 patterns are added in
  uint32_t v[B];
  constexpr MagicTotals() : v() {
    for (int k = 0; k < B; ++k)
      for (int i = 0; i < 32; ++i) v[k] += magic_in_word(B, i, k);
  }
};

// Adds pattern u at stream bit `bit` of w (bit fields do not overlap, so adding is or-ing up
// to the constant parts, which the caller takes out once).
template <int N, int B>
__device__ __forceinline__ void add_at(uint32_t (&w)[N], int bit, uint32_t u) {
  const int wi = bit >> 5, off = bit & 31;
  w[wi] += u << off;
  if (off + B > 32) w[wi + 1] += u >> (32 - off);
}

// The 32 codes packed at stream bits [i B, i B + B) of w (pack_group's words).
template <int B>
__device__ __forceinline__ void pack_patterns(const uint32_t (&cb)[32], uint32_t (&w)[B]) {
  constexpr MagicTotals<B> mt{};
#pragma unroll
  for (int k = 0; k < B; ++k) w[k] = 0u - mt.v[k];
#pragma unroll
  for (int i = 0; i < 32; ++i) add_at<B, B>(w, i * B, cb[i]);
}

}  // namespace kvq
