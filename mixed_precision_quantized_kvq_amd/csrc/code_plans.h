// Code placement plans for the MFMA operands, shared by the decode kernel (unpacking) and the
// append kernel (value streams are written in the order the value plan reads them). Host and
// device code: the host build checks the plans against the packing rules.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------
// Slot plans: MFMA step s (0..7) of a 32-element group takes 4 codes; slot k of step s
// holds group element chan(s, k) as the fp16 subnormal c * 2^(exp(s, k) - 24). The 2^exp of
// each slot is divided out of the other operand, so a code may sit anywhere in the 10-bit
// mantissa. Both MFMA shapes sum such subnormals to within 5e-5 relative at exp 0 and 2e-7 at
// exp 8 (measured on gfx950): the error halves per bit that a code sits higher. Over 128k
// tokens that floor reaches a quarter of the decode tolerance, so the plans keep codes high
// where that costs at most one more shift per code word.
// Each register (slots 2h, 2h + 1) is one AND of a "window" of the group's code stream (the
// stream shifted right by sh bits): the low code in bits 0-9, the high code in bits 16-25.
// One window serves several registers, so a group costs 16 ANDs plus one shift per window
// that is not a raw word:
//   b = 2: per word, codes (i, i + 8) from the word << 4 (i < 3, at bits 2 i + 4), the word
//          (i = 3, 4, at bits 2 i) or the word >> 6 (i > 4, at bits 2 i - 6): every code at
//          bit 4, 6 or 8; 4 shifts per group
//   b = 3: the 16 pairs of pair3() from 9 windows (raw words at 0, 32, 64; shifted at -4, 5,
//          26, 35, 58, 70): every code at bit 2 or above; 6 shifts per group
//   b = 4: per word, codes (i, i + 4) from the word << 2 (i < 2) or the word >> 6 (i >= 2),
//          at bits 4 (i % 2) + 2: 8 shifts per group
//   b = 5, 6, 7: the 16 pairs of wide_pair<B>() (one table serves keys and values), every code
//          at most 4 bits below the top of the mantissa: 13, 13 and 15 shifts per group
//   b = 8: codes k, k+2 of a word at bits 2-9 (exp 2)
// ---------------------------------------------------------------------------------------
struct CodePair {
  int lo, hi, sh, el, eh;  // low code, high code, window shift, their bit positions in the halves
};
__host__ __device__ constexpr CodePair pair3(int j) {
  constexpr CodePair t[16] = {{0, 5, -4, 4, 3},   {1, 6, -4, 7, 6},   {2, 7, 0, 6, 5},    {3, 8, 5, 4, 3},
                           {4, 9, 5, 7, 6},    {10, 15, 26, 4, 3}, {11, 16, 26, 7, 6}, {12, 17, 32, 4, 3},
                           {13, 18, 32, 7, 6}, {14, 19, 35, 7, 6}, {20, 26, 58, 2, 4}, {21, 27, 58, 5, 7},
                           {22, 28, 64, 2, 4}, {23, 29, 64, 5, 7}, {24, 30, 70, 2, 4}, {25, 31, 70, 5, 7}};
  return t[j];
}

// b = 5, 6, 7: registers j and j + 8 hold pairs of the same bit positions (the value-plan rule
// below), from 16 windows each:
//   b = 5: shifted at -5, 5, 25, 39, 52, 70, 75, 95, 100, 105, 125, 130, 135 (raw 0, 32, 64)
//   b = 6: shifted at 4, 10, 40, 52, 76, 88, 98, 118, 124, 130, 154, 160, 168 (raw 0, 32, 64)
//   b = 7: shifted at -3, 4, 25, 53, 60, 81, 88, 109, 116, 137, 144, 165, 172, 193, 200 (raw 32)
template <int B>
__host__ __device__ constexpr CodePair wide_pair(int j) {
  static_assert(B >= 5 && B <= 7, "table-driven wide widths");
  if constexpr (B == 5) {
    constexpr CodePair t[16] = {{0, 3, -5, 5, 4},   {2, 5, 5, 5, 4},     {7, 10, 32, 3, 2},   {8, 12, 39, 1, 5},
                                {15, 18, 70, 5, 4}, {20, 23, 95, 5, 4},  {22, 25, 105, 5, 4}, {27, 30, 130, 5, 4},
                                {1, 4, 0, 5, 4},    {6, 9, 25, 5, 4},    {11, 14, 52, 3, 2},  {13, 17, 64, 1, 5},
                                {16, 19, 75, 5, 4}, {21, 24, 100, 5, 4}, {26, 29, 125, 5, 4}, {28, 31, 135, 5, 4}};
    return t[j];
  } else if constexpr (B == 6) {
    constexpr CodePair t[16] = {{0, 3, 0, 0, 2},     {1, 4, 4, 2, 4},     {6, 8, 32, 4, 0},    {7, 10, 40, 2, 4},
                                {11, 14, 64, 2, 4},  {15, 18, 88, 2, 4},  {21, 24, 124, 2, 4}, {26, 29, 154, 2, 4},
                                {28, 31, 168, 0, 2}, {2, 5, 10, 2, 4},    {17, 19, 98, 4, 0},  {9, 12, 52, 2, 4},
                                {13, 16, 76, 2, 4},  {20, 23, 118, 2, 4}, {22, 25, 130, 2, 4}, {27, 30, 160, 2, 4}};
    return t[j];
  } else {
    constexpr CodePair t[16] = {{0, 2, -3, 3, 1},    {4, 6, 25, 3, 1},    {8, 10, 53, 3, 1},   {12, 14, 81, 3, 1},
                                {16, 18, 109, 3, 1}, {20, 22, 137, 3, 1}, {24, 26, 165, 3, 1}, {28, 30, 193, 3, 1},
                                {1, 3, 4, 3, 1},     {5, 7, 32, 3, 1},    {9, 11, 60, 3, 1},   {13, 15, 88, 3, 1},
                                {17, 19, 116, 3, 1}, {21, 23, 144, 3, 1}, {25, 27, 172, 3, 1}, {29, 31, 200, 3, 1}};
    return t[j];
  }
}

template <int B>
struct Slots {
  __host__ __device__ static constexpr int chan(int s, int k) {
    const int j = 2 * s + (k >> 1);  // register (pair) index in the group
    if constexpr (B == 2) {
      return 16 * (j >> 3) + (j & 7) + 8 * (k & 1);
    } else if constexpr (B == 3) {
      return (k & 1) ? pair3(j).hi : pair3(j).lo;
    } else if constexpr (B == 4) {
      return 8 * (j >> 2) + (j & 3) + 4 * (k & 1);
    } else if constexpr (B == 8) {
      return 4 * s + (k >> 1) + 2 * (k & 1);
    } else {
      return (k & 1) ? wide_pair<B>(j).hi : wide_pair<B>(j).lo;
    }
  }
  __host__ __device__ static constexpr int exp(int s, int k) {
    const int j = 2 * s + (k >> 1);
    if constexpr (B == 2) {
      const int i = j & 7;
      return i < 3 ? 2 * i + 4 : i < 5 ? 2 * i : 2 * i - 6;
    } else if constexpr (B == 3) {
      return (k & 1) ? pair3(j).eh : pair3(j).el;
    } else if constexpr (B == 4) {
      return 4 * (j & 1) + 2;
    } else if constexpr (B == 8) {
      return 2;
    } else {
      return (k & 1) ? wide_pair<B>(j).eh : wide_pair<B>(j).el;
    }
  }
};

// Low 32 bits of (hi:lo) >> n, 0 <= n < 32 (v_alignbit_b32 on the device; written as a funnel
// shift of two registers so the code words stay in registers).
__host__ __device__ __forceinline__ uint32_t funnel(uint32_t hi, uint32_t lo, int n) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_alignbit(hi, lo, n);
#else
  return (uint32_t)((((uint64_t)hi << 32) | lo) >> n);
#endif
}

// 32 bits of the group's stream starting at stream bit `sh` (sh may be negative: shifted
// in zeros), read from the group's B words.
template <int B, int N>
__host__ __device__ __forceinline__ uint32_t window(const uint32_t (&w)[N], int base, int sh) {
  if (sh < 0) return w[base] << (-sh);
  const int wi = sh >> 5, off = sh & 31;
  if (wi + 1 >= B || off == 0) return w[base + wi] >> off;
  return funnel(w[base + wi + 1], w[base + wi], off);
}

// B operand (two fp16 pairs) of step s for the group whose words start at w[base].
template <int B, int N>
__host__ __device__ __forceinline__ u32x2 unpack_step(const uint32_t (&w)[N], int base, int s) {
  if constexpr (B == 2) {
    const uint32_t x = w[base + (s >> 2)];
    uint32_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = (2 * s + h) & 7;  // pair (i, i + 8) of this word
      const uint32_t y = i < 3 ? x << 4 : i < 5 ? x : x >> 6;
      const int e = i < 3 ? 2 * i + 4 : i < 5 ? 2 * i : 2 * i - 6;
      r[h] = y & ((3u << e) | (3u << (16 + e)));
    }
    return u32x2{r[0], r[1]};
  } else if constexpr (B == 3) {
    uint32_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const CodePair q = pair3(2 * s + h);
      r[h] = window<3>(w, base, q.sh) & ((7u << q.el) | (7u << (16 + q.eh)));
    }
    return u32x2{r[0], r[1]};
  } else if constexpr (B == 4) {
    const uint32_t x = w[base + (s >> 1)];
    uint32_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = (2 * s + h) & 3;  // pair (i, i + 4) of this word
      const uint32_t y = i < 2 ? x << 2 : x >> 6;
      const int e = 4 * (i & 1) + 2;
      r[h] = y & ((15u << e) | (15u << (16 + e)));
    }
    return u32x2{r[0], r[1]};
  } else if constexpr (B == 8) {
    const uint32_t x = w[base + s];
    return u32x2{(x << 2) & 0x03FC03FCu, (x >> 6) & 0x03FC03FCu};
  } else {
    constexpr uint32_t m = (1u << B) - 1u;
    uint32_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const CodePair q = wide_pair<B>(2 * s + h);
      r[h] = window<B>(w, base, q.sh) & ((m << q.el) | (m << (16 + q.eh)));
    }
    return u32x2{r[0], r[1]};
  }
}

// ---------------------------------------------------------------------------------------
// Value slot plans. The value product runs on the 16x16x32 MFMA: a lane's B operand is 8
// consecutive tokens u = 0..7 of one channel ("chunk"), two steps s of a 32-code stream:
// u = 4 (s % 2) + k. Chunks 2 c' + kk of a stream (steps 4 c' + 2 kk, +1) take the weight
// operand of K-step kk, shared with every other chunk of that K-step, so the exponent of a
// slot may depend on (s % 4, k) only. The key plans for b = 2 and 4 have that property; for
// b = 3 the values use vpair3(): 8 pair types (bit positions), each used by registers j and
// j + 8, cut from 10 windows (raw words at 0, 32, 64; shifted at -4, 5, 26, 36, 58, 67, 70),
// every code at bit 2 or above: 7 shifts per stream.
// ---------------------------------------------------------------------------------------
__host__ __device__ constexpr CodePair vpair3(int j) {
  // register j = 2 s + h; steps s and s + 4 hold pairs of the same type
  constexpr CodePair t[16] = {{0, 5, -4, 4, 3},   {1, 6, -4, 7, 6},   {2, 7, 0, 6, 5},    {10, 15, 26, 4, 3},
                           {11, 16, 26, 7, 6}, {20, 26, 58, 2, 4}, {21, 27, 58, 5, 7}, {24, 30, 67, 5, 7},
                           {3, 8, 5, 4, 3},    {4, 9, 5, 7, 6},    {14, 19, 36, 6, 5}, {12, 17, 32, 4, 3},
                           {13, 18, 32, 7, 6}, {22, 28, 64, 2, 4}, {23, 29, 64, 5, 7}, {25, 31, 70, 5, 7}};
  return t[j];
}

template <int B>
struct VSlots {
  __host__ __device__ static constexpr int chan(int s, int k) {
    if constexpr (B == 3) {
      const CodePair q = vpair3(2 * s + (k >> 1));
      return (k & 1) ? q.hi : q.lo;
    } else {
      return Slots<B>::chan(s, k);
    }
  }
  __host__ __device__ static constexpr int exp(int s, int k) {
    if constexpr (B == 3) {
      const CodePair q = vpair3(2 * s + (k >> 1));
      return (k & 1) ? q.eh : q.el;
    } else {
      return Slots<B>::exp(s, k);
    }
  }
};

template <int B, int N>
__host__ __device__ __forceinline__ u32x2 unpack_step_v(const uint32_t (&w)[N], int base, int s) {
  if constexpr (B == 3) {
    uint32_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const CodePair q = vpair3(2 * s + h);
      r[h] = window<3>(w, base, q.sh) & ((7u << q.el) | (7u << (16 + q.eh)));
    }
    return u32x2{r[0], r[1]};
  } else {
    return unpack_step<B>(w, base, s);
  }
}

}  // namespace kvq
