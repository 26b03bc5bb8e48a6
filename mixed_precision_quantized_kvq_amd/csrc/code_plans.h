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
// holds group element chan(s, k) as the fp16 subnormal c * 2^(exp(s, k) - 24).
// Codes sit at the TOP of the 10-bit subnormal mantissa (exp = 10 - b or close to it): the
// 4x4x4 f16 MFMA keeps fp32 accuracy in its sums only when the subnormal operands are not
// deeply denormalized (codes at the bottom bits lose up to ~2^-16 of relative accuracy).
// Each pair of codes is cut out of the packed words with one shift/funnel shift and one AND:
//   b = 2: codes k, k+8 of a word; k even at bits 8-9, k odd at bits 6-7 (exp 8 / 6)
//   b = 3: pairs (a, a+5) or (a, a+6): code a at bits 5-7, code b at high-half bits 4-6 / 7-9
//   b = 4: codes k, k+4 of a word at bits 6-9 (exp 6)
//   b = 8: codes k, k+2 of a word at bits 2-9 (exp 2)
//   b = 5, 6, 7: codes 4s .. 4s+3 in order, each field extracted and placed at exp 10 - b
// ---------------------------------------------------------------------------------------
__host__ __device__ constexpr int pair3_a(int j) { return j < 5 ? j : (j < 10 ? j + 5 : j + 10); }
__host__ __device__ constexpr int pair3_b(int j) { return j < 10 ? pair3_a(j) + 5 : pair3_a(j) + 6; }

template <int B>
struct Slots {
  __host__ __device__ static constexpr int chan(int s, int k) {
    if constexpr (B == 2) {
      return 16 * (s >> 2) + 2 * (s & 3) + (k >> 1) + 8 * (k & 1);
    } else if constexpr (B == 3) {
      const int j = 2 * s + (k >> 1);
      return (k & 1) ? pair3_b(j) : pair3_a(j);
    } else if constexpr (B == 4) {
      return 8 * (s >> 1) + 2 * (s & 1) + (k >> 1) + 4 * (k & 1);
    } else if constexpr (B == 8) {
      return 4 * s + (k >> 1) + 2 * (k & 1);
    } else {
      return 4 * s + k;
    }
  }
  __host__ __device__ static constexpr int exp(int s, int k) {
    if constexpr (B == 2) {
      return ((2 * (s & 3) + (k >> 1)) & 1) ? 6 : 8;
    } else if constexpr (B == 3) {
      const int j = 2 * s + (k >> 1);
      return (k & 1) ? (j < 10 ? 4 : 7) : 5;
    } else if constexpr (B == 4) {
      return 6;
    } else if constexpr (B == 8) {
      return 2;
    } else {
      return 10 - B;
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

// Bits [pos, pos + B) of a group's little-endian code stream starting at word `base`.
template <int B, int N>
__host__ __device__ __forceinline__ uint32_t field(const uint32_t (&w)[N], int base, int pos) {
  const int wi = base + (pos >> 5), off = pos & 31;
  if (off + B <= 32) return (w[wi] >> off) & ((1u << B) - 1u);
  return funnel(w[wi + 1], w[wi], off) & ((1u << B) - 1u);
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
      const int k = 2 * (s & 3) + h;            // pair (k, k + 8) of this word
      const int sh = (k & 1) ? 2 * k - 6 : 2 * k - 8;
      const uint32_t y = sh >= 0 ? (x >> sh) : (x << -sh);
      r[h] = y & ((k & 1) ? 0x00C000C0u : 0x03000300u);
    }
    return u32x2{r[0], r[1]};
  } else if constexpr (B == 3) {
    uint32_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = 2 * s + h;
      const int a = pair3_a(j);
      const uint32_t y = window<3>(w, base, 3 * a - 5);
      r[h] = y & ((7u << 5) | (7u << (16 + (j < 10 ? 4 : 7))));
    }
    return u32x2{r[0], r[1]};
  } else if constexpr (B == 4) {
    const uint32_t x = w[base + (s >> 1)];
    uint32_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 2 * (s & 1) + h;            // pair (k, k + 4) of this word
      const int sh = 4 * k - 6;
      const uint32_t y = sh >= 0 ? (x >> sh) : (x << -sh);
      r[h] = y & 0x03C003C0u;
    }
    return u32x2{r[0], r[1]};
  } else if constexpr (B == 8) {
    const uint32_t x = w[base + s];
    return u32x2{(x << 2) & 0x03FC03FCu, (x >> 6) & 0x03FC03FCu};
  } else {
    constexpr int e = 10 - B;
    const uint32_t c0 = field<B>(w, base, (4 * s + 0) * B), c1 = field<B>(w, base, (4 * s + 1) * B);
    const uint32_t c2 = field<B>(w, base, (4 * s + 2) * B), c3 = field<B>(w, base, (4 * s + 3) * B);
    return u32x2{(c0 << e) | (c1 << (16 + e)), (c2 << e) | (c3 << (16 + e))};
  }
}

// fp16 2^(exp(s, k) - 14) in every slot of step s: the weight sum sum_t p_t comes out of the
// value MFMA with this operand (normal numbers, so its sums are exact to fp32).

// ---------------------------------------------------------------------------------------
// Value slot plans. The value product runs on the 16x16x32 MFMA: a lane's B operand is 8
// consecutive tokens u = 0..7 of one channel ("chunk"), two steps s of a 32-code stream:
// u = 4 (s % 2) + k. The weight operand is shared by every chunk of the tile, so the
// exponent of a slot may depend on (s % 2, k) only. The key plans have that property for
// b != 3; for b = 3 the values pair codes (a, a + 5) on even steps (high code at bits 4-6)
// and (a, a + 6) on odd steps (bits 7-9), low code at bits 5-7.
// ---------------------------------------------------------------------------------------
__host__ __device__ constexpr int vpair3_a(int s, int h) {
  // low codes of the 8 even-step pairs (distance 5), then of the 8 odd-step pairs (distance 6)
  constexpr int even_a[8] = {0, 1, 2, 3, 11, 12, 13, 14};
  constexpr int odd_a[8] = {4, 9, 20, 21, 22, 23, 24, 25};
  return (s & 1) ? odd_a[2 * (s >> 1) + h] : even_a[2 * (s >> 1) + h];
}

template <int B>
struct VSlots {
  __host__ __device__ static constexpr int chan(int s, int k) {
    if constexpr (B == 3) {
      const int a = vpair3_a(s, k >> 1);
      return (k & 1) ? a + ((s & 1) ? 6 : 5) : a;
    } else {
      return Slots<B>::chan(s, k);
    }
  }
  __host__ __device__ static constexpr int exp(int s, int k) {
    if constexpr (B == 3)
      return (k & 1) ? ((s & 1) ? 7 : 4) : 5;
    else
      return Slots<B>::exp(s, k);
  }
};

template <int B, int N>
__host__ __device__ __forceinline__ u32x2 unpack_step_v(const uint32_t (&w)[N], int base, int s) {
  if constexpr (B == 3) {
    uint32_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int a = vpair3_a(s, h);
      const uint32_t y = window<3>(w, base, 3 * a - 5);
      r[h] = y & ((7u << 5) | (7u << (16 + ((s & 1) ? 7 : 4))));
    }
    return u32x2{r[0], r[1]};
  } else {
    return unpack_step<B>(w, base, s);
  }
}

// fp16 2^(exp - 14) for token u = 0..7 of a chunk, as 4 registers (u = 2r low, 2r + 1 high)

}  // namespace kvq
