// Split-K decode attention over the packed cache, dequantization fused into q.K^T and P.V
// (InnerQ: grouping along the inner dimension of each vector-matrix product; the decode
// structure of its "Algorithm 1 ... decode phase"), with the log-sum-exp merge of the split
// partials done by the last workgroup of each (row, KV head).
//
// Grid (n_splits + 1, KV heads, rows), 4 wavefronts per workgroup. Workgroup `split` <
// n_splits owns a contiguous range of 64-token body tiles (wavefronts take tiles round-robin);
// workgroup n_splits takes the 16-bit sink and recent-window tokens.
//
// Both products run on the 4x4x4 (16-block) f16/bf16 MFMA. Lane l belongs to block l/4 and
// to row/column l%4, so with the G <= 4 query heads of a KV head as the 4-wide dimension:
//   q.K^T  lane = token. B operand = 4 codes of the lane's token, A = the 4 matching q values
//          of query l%4; output element i is query i's partial dot for that token.
//   P.V    lane = channel. B operand = 4 tokens' codes of the lane's channel, A = the 4
//          matching softmax weights of query l%4; output element i is query i's partial.
// Codes enter the MFMA as fp16 subnormals: one shift and one AND of a packed word leave two
// codes in the top mantissa bits of two fp16 halves, i.e. the values c * 2^(e - 24) (slot
// plans below). The 2^e of each slot is divided out of the matching A value (q or p), so
// every product is exact and each sum carries one known power of two.
// Each group's scale and zero are applied once to its partial sums:
//   q . k_hat = s (q . c) + z sum(q)                     key group: 32 channels of a token
//   sum_t p_t v_hat_t = s sum_t p_t c_t + z sum_t p_t    value group: 32 tokens of a channel
// Softmax weights travel as an fp16 (bf16 for bf16 windows) pair hi + lo; sum_t p_t comes
// from the same MFMA with a constant operand in every slot, so numerator and denominator use
// identical weights.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxG = 4;
constexpr int kEp = 11;  // softmax weights enter the value MFMA as p * 2^(kEp - e)
// Lazy rescaling: the running max m moves only when a score exceeds it by more than kTau
// (log2 units), so weights stay below 2^kTau and p * 2^kEp * 2^kTau fits fp16.
constexpr float kTau = 4.0f;
constexpr int kMaxParts = 257;  // n_splits <= 256 body partials + the window partial

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4_t mfma_f16(u32x2 a, u32x2 b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma_bf16(u32x2 a, u32x2 b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(short4_t, a), __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
}
template <bool BF16>
__device__ __forceinline__ float4_t mfma16(u32x2 a, u32x2 b, float4_t c) {
  if constexpr (BF16) return mfma_bf16(a, b, c);
  else return mfma_f16(a, b, c);
}

__device__ __forceinline__ float h2f(uint32_t bits16) { return __half2float(__ushort_as_half((uint16_t)bits16)); }
__device__ __forceinline__ uint32_t f2h(float x) { return (uint32_t)__half_as_ushort(__float2half_rn(x)); }
__device__ __forceinline__ uint32_t f2bf(float x) {  // round to nearest even (finite x)
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float widen(uint32_t raw, int dtype) {
  return dtype == KVQ_BF16 ? bf2f(raw & 0xFFFFu) : h2f(raw & 0xFFFFu);
}

// Maximum over the 64 lanes of a wavefront: DPP reductions within rows of 16, then row
// broadcasts; the total lands in lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_step_max(float v) {
  const int t = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
  return fmaxf(v, __int_as_float(t));
}
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_step_max<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_step_max<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_step_max<0x124, 0xF>(v);  // row_ror:4
  v = dpp_step_max<0x128, 0xF>(v);  // row_ror:8
  v = dpp_step_max<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_step_max<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// LDS traffic of one wavefront is executed in issue order, so a wavefront reading back what
// it wrote only needs the compiler not to reorder the accesses.
__device__ __forceinline__ void wave_lds_sync() { __asm__ __volatile__("" ::: "memory"); }

// Keeps global loads issued above this point from being sunk below it (software prefetch).
__device__ __forceinline__ void issue_barrier() { __asm__ __volatile__("" ::: "memory"); }

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
template <int B>
__device__ __forceinline__ u32x2 ones_step(int s) {
  auto one = [&](int k) { return (uint32_t)(Slots<B>::exp(s, k) + 1) << 10; };
  return u32x2{one(0) | (one(1) << 16), one(2) | (one(3) << 16)};
}

template <int D>
struct Smem {
  // rows of the 4 query slots are padded by 4 words so that the 4 distinct addresses of an
  // operand read fall in different LDS banks
  uint32_t qA[kMaxG][D / 2 + 4];         // key-MFMA A operand: fp16 q * 2^(Eq - e), slot order
  uint32_t qW[kMaxG][D / 2 + 4];         // 16-bit-row A operand: q in the cache dtype
  float qsum[kMaxG][D / 32];             // sum of q over each key group, times the softmax scale
  uint32_t pw[kWaves][2][kMaxG][36];     // per wave: hi/lo, query, 2 blocks x 16 words (+4 pad)
  float red_o[kWaves][kMaxG][D];
  float red_m[kWaves][kMaxG];
  float red_l[kWaves][kMaxG];
  float qmax[kWaves];
};

struct WaveState {
  float m[kMaxG];  // running max of the scores (log2 units), uniform over the wave
  float l[kMaxG];  // running sum of the weights, uniform over the wave
};

// Softmax for one tile (lane = token): weights written to LDS as a hi/lo pair at the value
// slot `ppos` of the lane's token, scaled by pscl; accumulators rescaled when the max moves.
template <int D>
__device__ __forceinline__ void softmax_tile(Smem<D>& sm, int wave, int lane, bool valid, const float (&sc)[kMaxG],
                                             WaveState& st, float (&o)[kMaxG][D / 64], int ppos, float pscl,
                                             bool bf16_weights) {
  const int jj = lane >> 5;
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    const float x = valid ? sc[i] : -INFINITY;
    if (__ballot(x > st.m[i] + kTau)) {  // rare after the first tile: move the running max
      const float mn = fmaxf(st.m[i], wave_max(x));
      const float alpha = __builtin_amdgcn_exp2f(st.m[i] - mn);
      st.m[i] = mn;
      st.l[i] *= alpha;
#pragma unroll
      for (int h = 0; h < D / 64; ++h) o[i][h] *= alpha;
    }
    const float mn = st.m[i];
    const float p = __builtin_amdgcn_exp2f(x - mn) * pscl;
    uint32_t hi, lo;
    if (bf16_weights) {
      hi = f2bf(p);
      lo = f2bf(p - bf2f(hi));
    } else {
      hi = f2h(p);
      lo = f2h(p - h2f(hi));
    }
    reinterpret_cast<uint16_t*>(&sm.pw[wave][0][i][16 * jj])[ppos] = (uint16_t)hi;
    reinterpret_cast<uint16_t*>(&sm.pw[wave][1][i][16 * jj])[ppos] = (uint16_t)lo;
  }
  wave_lds_sync();
}

// ---------------------------------------------------------------------------------------
// Quantized body tiles
// ---------------------------------------------------------------------------------------
template <int D, int KB>
struct KTile {
  static constexpr int W = (D / 32) * KB;
  uint32_t w[W];
  uint32_t m[D / 32];
};
template <int D, int VB>
struct VTile {
  uint32_t w[D / 64][2 * VB];
  uint32_t m[D / 64][2];
};

template <int D, int KB>
__device__ __forceinline__ void load_k(KTile<D, KB>& t, const uint32_t* kc, const uint32_t* km, int tile, int lane) {
  constexpr int W = KTile<D, KB>::W;
  const uint32_t* base = kc + (size_t)tile * kTile * W;
#pragma unroll
  for (int q = 0; q < (W + 3) / 4; ++q) {
    const int nq = (W - 4 * q) < 4 ? (W - 4 * q) : 4;  // 4, or 2 for the last chunk
    const uint32_t* src = base + 256 * q + lane * nq;
    if (nq == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      t.w[4 * q] = v.x; t.w[4 * q + 1] = v.y; t.w[4 * q + 2] = v.z; t.w[4 * q + 3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      t.w[4 * q] = v.x; t.w[4 * q + 1] = v.y;
    }
  }
  const uint32_t* mp = km + ((size_t)tile * kTile + lane) * (D / 32);
  if constexpr (D == 128) {
    const uint4 v = *reinterpret_cast<const uint4*>(mp);
    t.m[0] = v.x; t.m[1] = v.y; t.m[2] = v.z; t.m[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(mp);
    t.m[0] = v.x; t.m[1] = v.y;
  }
}

template <int D, int VB>
__device__ __forceinline__ void load_v(VTile<D, VB>& t, const uint32_t* vc, const uint32_t* vm, int tile, int lane) {
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    const int c = lane + 64 * h;
    const uint32_t* src = vc + (size_t)tile * 2 * D * VB + (size_t)c * 2 * VB;
    if constexpr (VB % 2 == 0) {
#pragma unroll
      for (int x = 0; x < 2 * VB; x += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + x);
        t.w[h][x] = v.x; t.w[h][x + 1] = v.y; t.w[h][x + 2] = v.z; t.w[h][x + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int x = 0; x < 2 * VB; x += 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(src + x);
        t.w[h][x] = v.x; t.w[h][x + 1] = v.y;
      }
    }
    const uint2 mv = *reinterpret_cast<const uint2*>(vm + (size_t)tile * 2 * D + c * 2);
    t.m[h][0] = mv.x;
    t.m[h][1] = mv.y;
  }
}

// Scores (log2 units) of the lane's token for the 4 query slots.
template <int D, int KB>
__device__ __forceinline__ void key_phase(const Smem<D>& sm, const KTile<D, KB>& t, int lane, float kscale,
                                          float (&sc)[kMaxG]) {
  const int qi = lane & 3;
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) sc[i] = 0.0f;
#pragma unroll
  for (int g = 0; g < D / 32; ++g) {
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x2 a = *reinterpret_cast<const u32x2*>(&sm.qA[qi][(g * 8 + s) * 2]);
      acc = mfma_f16(a, unpack_step<KB>(t.w, g * KB, s), acc);
    }
    const float sg = h2f(t.m[g] & 0xFFFFu) * kscale;
    const float zg = h2f(t.m[g] >> 16);
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) sc[i] += sg * acc[i] + zg * sm.qsum[i][g];
  }
}

template <int D, int VB>
__device__ __forceinline__ void value_phase(const Smem<D>& sm, int wave, const VTile<D, VB>& t, int lane, int nblk,
                                            float (&o)[kMaxG][D / 64], WaveState& st) {
  const int qi = lane & 3;
  constexpr float kV = (float)(1 << (24 - kEp));   // code products carry 2^(kEp - 24)
  constexpr float kV1 = (float)(1 << (14 - kEp));  // weight sums carry 2^(kEp - 14)
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    if (jj < nblk) {
      float4_t acc[D / 64], acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int h = 0; h < D / 64; ++h) acc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x2 ahi = *reinterpret_cast<const u32x2*>(&sm.pw[wave][0][qi][16 * jj + 2 * s]);
        const u32x2 alo = *reinterpret_cast<const u32x2*>(&sm.pw[wave][1][qi][16 * jj + 2 * s]);
#pragma unroll
        for (int h = 0; h < D / 64; ++h) {
          const u32x2 b = unpack_step<VB>(t.w[h], jj * VB, s);
          acc[h] = mfma_f16(ahi, b, acc[h]);
          acc[h] = mfma_f16(alo, b, acc[h]);
        }
        const u32x2 one = ones_step<VB>(s);
        acc1 = mfma_f16(ahi, one, acc1);
        acc1 = mfma_f16(alo, one, acc1);
      }
#pragma unroll
      for (int h = 0; h < D / 64; ++h) {
        const float sv = h2f(t.m[h][jj] & 0xFFFFu) * kV, zv = h2f(t.m[h][jj] >> 16) * kV1;
#pragma unroll
        for (int i = 0; i < kMaxG; ++i) o[i][h] += sv * acc[h][i] + zv * acc1[i];
      }
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) st.l[i] += acc1[i] * kV1;
    }
  }
}

// value slot (and its exponent) that holds token tb (0..31) of a block
template <int VB>
__device__ __forceinline__ void value_slot(int tb, int& ppos, int& pe) {
  ppos = 0;
  pe = 0;
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (Slots<VB>::chan(s, k) == tb) {
        ppos = 4 * s + k;
        pe = Slots<VB>::exp(s, k);
      }
}

// ---------------------------------------------------------------------------------------
// 16-bit rows (sink and recent windows; heads kept unquantized)
// ---------------------------------------------------------------------------------------
template <int D, bool BF16>
__device__ __forceinline__ void key_phase_16(const Smem<D>& sm, const uint16_t* row, int lane,
                                             float scale_log2, float (&sc)[kMaxG]) {
  const int qi = lane & 3;
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint4* r4 = reinterpret_cast<const uint4*>(row);
#pragma unroll 1
  for (int part = 0; part < D / 64; ++part) {
    uint4 x[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) x[v] = r4[part * 8 + v];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int vv = part * 8 + v;
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(&sm.qW[qi][4 * vv]);
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(&sm.qW[qi][4 * vv + 2]);
      acc = mfma16<BF16>(a0, u32x2{x[v].x, x[v].y}, acc);
      acc = mfma16<BF16>(a1, u32x2{x[v].z, x[v].w}, acc);
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) sc[i] = acc[i] * scale_log2;
}

// lane = channel; row_of(k) is the row of token k of the tile (k < n_valid)
template <int D, bool BF16, class RowOf>
__device__ __forceinline__ void value_phase_16(const Smem<D>& sm, int wave, int lane, int n_valid,
                                               RowOf row_of, float (&o)[kMaxG][D / 64], WaveState& st) {
  const int qi = lane & 3;
  const uint32_t one1 = BF16 ? 0x3F80u : 0x3C00u;
  const u32x2 one = u32x2{one1 | (one1 << 16), one1 | (one1 << 16)};
  float4_t acc[D / 64], acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int h = 0; h < D / 64; ++h) acc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int jj = 0; jj * 32 < n_valid; ++jj) {
    uint32_t pk[8][D / 64][2];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint16_t* r0 = row_of(min(jj * 32 + 4 * s + 0, n_valid - 1));
      const uint16_t* r1 = row_of(min(jj * 32 + 4 * s + 1, n_valid - 1));
      const uint16_t* r2 = row_of(min(jj * 32 + 4 * s + 2, n_valid - 1));
      const uint16_t* r3 = row_of(min(jj * 32 + 4 * s + 3, n_valid - 1));
#pragma unroll
      for (int h = 0; h < D / 64; ++h) {
        const int c = lane + 64 * h;
        pk[s][h][0] = (uint32_t)r0[c] | ((uint32_t)r1[c] << 16);
        pk[s][h][1] = (uint32_t)r2[c] | ((uint32_t)r3[c] << 16);
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x2 ahi = *reinterpret_cast<const u32x2*>(&sm.pw[wave][0][qi][16 * jj + 2 * s]);
      const u32x2 alo = *reinterpret_cast<const u32x2*>(&sm.pw[wave][1][qi][16 * jj + 2 * s]);
#pragma unroll
      for (int h = 0; h < D / 64; ++h) {
        const u32x2 b = u32x2{pk[s][h][0], pk[s][h][1]};
        acc[h] = mfma16<BF16>(ahi, b, acc[h]);
        acc[h] = mfma16<BF16>(alo, b, acc[h]);
      }
      acc1 = mfma16<BF16>(ahi, one, acc1);
      acc1 = mfma16<BF16>(alo, one, acc1);
    }
  }
#pragma unroll
  for (int h = 0; h < D / 64; ++h)
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) o[i][h] += acc[h][i];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) st.l[i] += acc1[i];
}

// ---------------------------------------------------------------------------------------
// Tile loops
// ---------------------------------------------------------------------------------------

// Quantized keys and values, both widths fixed: loads of the next tile are issued before the
// current tile is computed.
template <int D, int KB, int VB>
__device__ __forceinline__ void body_loop(Smem<D>& sm, const DecodePlan& p, const uint64_t* off, int t0, int t1,
                                          int lane, int wave, float kscale, WaveState& st,
                                          float (&o)[kMaxG][D / 64]) {
  const uint32_t* kc = reinterpret_cast<const uint32_t*>(p.blob + off[KC]);
  const uint32_t* km = reinterpret_cast<const uint32_t*>(p.blob + off[KM]);
  const uint32_t* vc = reinterpret_cast<const uint32_t*>(p.blob + off[VC]);
  const uint32_t* vm = reinterpret_cast<const uint32_t*>(p.blob + off[VM]);
  int ppos, pe;
  value_slot<VB>(lane & 31, ppos, pe);
  const float pscl = __builtin_ldexpf(1.0f, kEp - pe);
  int tile = t0 + wave;
  if (tile >= t1) return;
  KTile<D, KB> kt[2];
  VTile<D, VB> vt[2];
  load_k<D, KB>(kt[0], kc, km, tile, lane);
  load_v<D, VB>(vt[0], vc, vm, tile, lane);
  auto run = [&](const KTile<D, KB>& kcur, const VTile<D, VB>& vcur, KTile<D, KB>& knext, VTile<D, VB>& vnext) {
    // the next tile (or, past the end, this one again) is always fetched, so both buffers
    // keep fixed registers and the loads stay in flight while this tile is computed
    const int next = tile + kWaves;
    const int fetch = next < t1 ? next : tile;
    load_k<D, KB>(knext, kc, km, fetch, lane);
    load_v<D, VB>(vnext, vc, vm, fetch, lane);
    issue_barrier();
    float sc[kMaxG];
    key_phase<D, KB>(sm, kcur, lane, kscale, sc);
    softmax_tile<D>(sm, wave, lane, tile * kTile + lane < p.body, sc, st, o, ppos, pscl, false);
    value_phase<D, VB>(sm, wave, vcur, lane, min(2, (p.body - tile * kTile) / 32), o, st);
    wave_lds_sync();
    tile = next;
  };
  while (true) {
    run(kt[0], vt[0], kt[1], vt[1]);
    if (tile >= t1) break;
    run(kt[1], vt[1], kt[0], vt[0]);
    if (tile >= t1) break;
  }
}

template <int D, int KB>
__device__ __forceinline__ void key_tile_q(const Smem<D>& sm, const uint32_t* kc, const uint32_t* km, int tile, int lane,
                                           float kscale, float (&sc)[kMaxG]) {
  KTile<D, KB> t;
  load_k<D, KB>(t, kc, km, tile, lane);
  key_phase<D, KB>(sm, t, lane, kscale, sc);
}

template <int D, int VB>
__device__ __forceinline__ void value_tile_q(Smem<D>& sm, int wave, const uint32_t* vc, const uint32_t* vm, int tile,
                                             int lane, bool valid, const float (&sc)[kMaxG], int nblk, WaveState& st,
                                             float (&o)[kMaxG][D / 64]) {
  int ppos, pe;
  value_slot<VB>(lane & 31, ppos, pe);
  softmax_tile<D>(sm, wave, lane, valid, sc, st, o, ppos, __builtin_ldexpf(1.0f, kEp - pe), false);
  VTile<D, VB> t;
  load_v<D, VB>(t, vc, vm, tile, lane);
  value_phase<D, VB>(sm, wave, t, lane, nblk, o, st);
}

// Body tiles of heads with a 16-bit key or value side (one phase 16-bit, the other packed
// or 16-bit); no prefetch.
template <int D>
__device__ __forceinline__ void mixed_body_loop(Smem<D>& sm, const DecodePlan& p, const uint64_t* off, int t0, int t1, int lane,
                                int wave, float kscale, WaveState& st, float (&o)[kMaxG][D / 64]) {
  const int kb = p.k_bits[blockIdx.y], vb = p.v_bits[blockIdx.y];
  const bool bf16 = p.dtype == KVQ_BF16;
  const uint16_t* kr = reinterpret_cast<const uint16_t*>(p.blob + off[KC]);
  const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.blob + off[VC]);
  const uint32_t* kc = reinterpret_cast<const uint32_t*>(p.blob + off[KC]);
  const uint32_t* km = reinterpret_cast<const uint32_t*>(p.blob + off[KM]);
  const uint32_t* vc = reinterpret_cast<const uint32_t*>(p.blob + off[VC]);
  const uint32_t* vm = reinterpret_cast<const uint32_t*>(p.blob + off[VM]);
  for (int tile = t0 + wave; tile < t1; tile += kWaves) {
    const int tok = tile * kTile + lane;
    const bool valid = tok < p.body;
    const int n_valid = min(kTile, p.body - tile * kTile);
    float sc[kMaxG];
    switch (kb) {
      case 2: key_tile_q<D, 2>(sm, kc, km, tile, lane, kscale, sc); break;
      case 3: key_tile_q<D, 3>(sm, kc, km, tile, lane, kscale, sc); break;
      case 4: key_tile_q<D, 4>(sm, kc, km, tile, lane, kscale, sc); break;
      case 5: key_tile_q<D, 5>(sm, kc, km, tile, lane, kscale, sc); break;
      case 6: key_tile_q<D, 6>(sm, kc, km, tile, lane, kscale, sc); break;
      case 7: key_tile_q<D, 7>(sm, kc, km, tile, lane, kscale, sc); break;
      case 8: key_tile_q<D, 8>(sm, kc, km, tile, lane, kscale, sc); break;
      default:
        if (bf16)
          key_phase_16<D, true>(sm, kr + (size_t)(valid ? tok : tile * kTile) * D, lane, p.scale_log2, sc);
        else
          key_phase_16<D, false>(sm, kr + (size_t)(valid ? tok : tile * kTile) * D, lane, p.scale_log2, sc);
        break;
    }
    const int nblk = n_valid / 32;
    switch (vb) {
      case 2: value_tile_q<D, 2>(sm, wave, vc, vm, tile, lane, valid, sc, nblk, st, o); break;
      case 3: value_tile_q<D, 3>(sm, wave, vc, vm, tile, lane, valid, sc, nblk, st, o); break;
      case 4: value_tile_q<D, 4>(sm, wave, vc, vm, tile, lane, valid, sc, nblk, st, o); break;
      case 5: value_tile_q<D, 5>(sm, wave, vc, vm, tile, lane, valid, sc, nblk, st, o); break;
      case 6: value_tile_q<D, 6>(sm, wave, vc, vm, tile, lane, valid, sc, nblk, st, o); break;
      case 7: value_tile_q<D, 7>(sm, wave, vc, vm, tile, lane, valid, sc, nblk, st, o); break;
      case 8: value_tile_q<D, 8>(sm, wave, vc, vm, tile, lane, valid, sc, nblk, st, o); break;
      default:
        softmax_tile<D>(sm, wave, lane, valid, sc, st, o, lane & 31, 1.0f, bf16);
        if (bf16)
          value_phase_16<D, true>(sm, wave, lane, n_valid, [&](int k) { return vr + (size_t)(tile * kTile + k) * D; }, o, st);
        else
          value_phase_16<D, false>(sm, wave, lane, n_valid, [&](int k) { return vr + (size_t)(tile * kTile + k) * D; }, o, st);
        break;
    }
    wave_lds_sync();
  }
}

// 16-bit rows for tokens [first, n_tok) in 64-token tiles.
template <int D, bool BF16, class KRowOf, class VRowOf>
__device__ __forceinline__ void rows16_loop_t(Smem<D>& sm, const DecodePlan& p, int first, int n_tok, int lane,
                                              int wave, WaveState& st, float (&o)[kMaxG][D / 64], KRowOf krow,
                                              VRowOf vrow) {
  for (int base = first + wave * kTile; base < n_tok; base += kWaves * kTile) {
    const int u = base + lane;
    const bool valid = u < n_tok;
    float sc[kMaxG];
    key_phase_16<D, BF16>(sm, krow(valid ? u : base), lane, p.scale_log2, sc);
    softmax_tile<D>(sm, wave, lane, valid, sc, st, o, lane & 31, 1.0f, BF16);
    value_phase_16<D, BF16>(sm, wave, lane, min(kTile, n_tok - base), [&](int k) { return vrow(base + k); }, o, st);
    wave_lds_sync();
  }
}
template <int D, class KRowOf, class VRowOf>
__device__ __forceinline__ void rows16_loop(Smem<D>& sm, const DecodePlan& p, int first, int n_tok, int lane, int wave,
                                            WaveState& st, float (&o)[kMaxG][D / 64], KRowOf krow, VRowOf vrow) {
  if (p.dtype == KVQ_BF16)
    rows16_loop_t<D, true>(sm, p, first, n_tok, lane, wave, st, o, krow, vrow);
  else
    rows16_loop_t<D, false>(sm, p, first, n_tok, lane, wave, st, o, krow, vrow);
}

// ---------------------------------------------------------------------------------------
// Kernel
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodePlan p) {
  __shared__ Smem<D> sm;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int kb = p.k_bits[h], vb = p.v_bits[h];
  const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)b * p.Hq + (size_t)h * G) * D;

  // ---- q operands in LDS: raw 16-bit copy, and the fp16 key operand in slot order with
  // q scaled by 2^Eq so that max|q| * 2^Eq lies in [2^14, 2^15)
  float qmax = 0.0f;
  for (int idx = tid; idx < kMaxG * D; idx += kThreads) {
    const int i = idx / D, c = idx % D;
    const uint32_t raw = i < G ? q[(size_t)i * D + c] : 0u;
    reinterpret_cast<uint16_t*>(sm.qW[i])[c] = (uint16_t)raw;
    qmax = fmaxf(qmax, fabsf(widen(raw, p.dtype)));
  }
  qmax = wave_max(qmax);
  if (lane == 0) sm.qmax[wave] = qmax;
  __syncthreads();
  qmax = fmaxf(fmaxf(sm.qmax[0], sm.qmax[1]), fmaxf(sm.qmax[2], sm.qmax[3]));
  int qe = 0;
  if (qmax > 0.0f) (void)frexpf(qmax, &qe);
  const int Eq = 15 - qe;
  const float kscale = __builtin_ldexpf(p.scale_log2, 24 - Eq);
  for (int idx = tid; idx < kMaxG * D; idx += kThreads) {
    const int i = idx / D, slot = idx % D;  // slot = (g * 8 + s) * 4 + k
    const int g = slot / 32, s = (slot / 4) % 8, k = slot % 4;
    int ch = 0, e = 0;
    switch (kb) {
#define KVQ_SLOT(B_) \
  case B_: ch = Slots<B_>::chan(s, k); e = Slots<B_>::exp(s, k); break;
      KVQ_SLOT(2) KVQ_SLOT(3) KVQ_SLOT(4) KVQ_SLOT(5) KVQ_SLOT(6) KVQ_SLOT(7) KVQ_SLOT(8)
#undef KVQ_SLOT
      default: break;
    }
    const float qv = widen(reinterpret_cast<const uint16_t*>(sm.qW[i])[g * 32 + ch], p.dtype);
    reinterpret_cast<uint16_t*>(sm.qA[i])[slot] = (uint16_t)f2h(__builtin_ldexpf(qv, Eq - e));
  }
  if (tid < kMaxG * (D / 32)) {
    const int i = tid / (D / 32), g = tid % (D / 32);
    float s = 0.0f;
    for (int k = 0; k < 32; ++k) s += widen(reinterpret_cast<const uint16_t*>(sm.qW[i])[g * 32 + k], p.dtype);
    sm.qsum[i][g] = s * p.scale_log2;
  }
  __syncthreads();

  WaveState st;
  float o[kMaxG][D / 64];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    st.m[i] = -INFINITY;
    st.l[i] = 0.0f;
#pragma unroll
    for (int hh = 0; hh < D / 64; ++hh) o[i][hh] = 0.0f;
  }
  const uint64_t* off = p.off + ((size_t)b * p.H + h) * kRegions;

  if (split < p.n_splits) {
    const int t0 = split * p.tiles_per_split;
    const int t1 = min(p.n_tiles, t0 + p.tiles_per_split);
    if (kb == 16 && vb == 16) {
      const uint16_t* kr = reinterpret_cast<const uint16_t*>(p.blob + off[KC]);
      const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.blob + off[VC]);
      rows16_loop<D>(sm, p, t0 * kTile, min(p.body, t1 * kTile), lane, wave, st, o,
                     [&](int u) { return kr + (size_t)u * D; }, [&](int u) { return vr + (size_t)u * D; });
    } else if (kb <= 4 && vb <= 4) {
      // the widths the allocator hands out in {2,3,4}: prefetching loop per combination
#define KVQ_BODY(KB_, VB_) \
  case KB_ * 16 + VB_: body_loop<D, KB_, VB_>(sm, p, off, t0, t1, lane, wave, kscale, st, o); break;
      switch (kb * 16 + vb) {
        KVQ_BODY(2, 2) KVQ_BODY(2, 3) KVQ_BODY(2, 4) KVQ_BODY(3, 2) KVQ_BODY(3, 3) KVQ_BODY(3, 4)
        KVQ_BODY(4, 2) KVQ_BODY(4, 3) KVQ_BODY(4, 4)
        default: break;
      }
#undef KVQ_BODY
    } else {
      // wider codes or a 16-bit side: one phase at a time
      mixed_body_loop<D>(sm, p, off, t0, t1, lane, wave, kscale, st, o);
    }
  } else {
    // 16-bit windows: token u < n_sink_live is sink row u, else the ring slot of absolute
    // token n_sink + body + (u - n_sink_live)
    const uint16_t* sk = reinterpret_cast<const uint16_t*>(p.blob + off[SK]);
    const uint16_t* sv = reinterpret_cast<const uint16_t*>(p.blob + off[SV]);
    const uint16_t* rk = reinterpret_cast<const uint16_t*>(p.blob + off[RK]);
    const uint16_t* rv = reinterpret_cast<const uint16_t*>(p.blob + off[RV]);
    const int nsl = p.n_sink_live, body = p.body, ring = p.ring;
    auto krow = [&](int u) { return u < nsl ? sk + (size_t)u * D : rk + (size_t)((body + u - nsl) % ring) * D; };
    auto vrow = [&](int u) { return u < nsl ? sv + (size_t)u * D : rv + (size_t)((body + u - nsl) % ring) * D; };
    rows16_loop<D>(sm, p, 0, p.n_sink_live + p.n_win, lane, wave, st, o, krow, vrow);
  }

  // ---- combine the wavefronts of this workgroup into one partial (m, l, o)
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    if (lane == 0) {
      sm.red_m[wave][i] = st.m[i];
      sm.red_l[wave][i] = st.l[i];
    }
#pragma unroll
    for (int hh = 0; hh < D / 64; ++hh) sm.red_o[wave][i][lane + 64 * hh] = o[i][hh];
  }
  __syncthreads();
  const size_t rows = (size_t)p.B * p.Hq;
  const size_t row0 = (size_t)b * p.Hq + (size_t)h * G;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int i = idx / D, c = idx % D;
    float ms = -INFINITY;
    for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, sm.red_m[w][i]);
    float oo = 0.0f, ll = 0.0f;
    if (ms != -INFINITY) {
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(sm.red_m[w][i] - ms);
        oo += f * sm.red_o[w][i][c];
        ll += f * sm.red_l[w][i];
      }
    }
    p.ws_o[((size_t)split * rows + row0 + i) * D + c] = oo;
    if (c == 0) {
      p.ws_ml[((size_t)split * rows + row0 + i) * 2] = ms;
      p.ws_ml[((size_t)split * rows + row0 + i) * 2 + 1] = ll;
    }
  }

}

// ---------------------------------------------------------------------------------------
// Log-sum-exp merge of the n_splits + 1 partials of one (row, KV head):
//   out = sum_j 2^(m_j - m*) o_j / sum_j 2^(m_j - m*) l_j,  m* = max_j m_j.
// A separate launch: the kernel boundary makes every partial visible, so no workgroup has
// to write back or invalidate the L2 caches.
// ---------------------------------------------------------------------------------------
struct MergeSmem {
  float part_m[kMaxParts][kMaxG];  // (m, l) of every partial, then its weight
  float part_l[kMaxParts][kMaxG];
  float linv[kMaxG];
};

template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(const DecodePlan p) {
  __shared__ MergeSmem sm;
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, parts = p.n_splits + 1;
  const size_t rows = (size_t)p.B * p.Hq;
  const size_t row0 = (size_t)b * p.Hq + (size_t)h * G;
  for (int idx = tid; idx < parts * G; idx += kThreads) {
    const int j = idx / G, i = idx % G;
    const float* ml = p.ws_ml + ((size_t)j * rows + row0 + i) * 2;
    sm.part_m[j][i] = ml[0];
    sm.part_l[j][i] = ml[1];
  }
  __syncthreads();
  // wavefront i reduces query i: m* = max_j m_j, l* = sum_j 2^(m_j - m*) l_j
  if (wave < G) {
    float mx = -INFINITY;
    for (int j = lane; j < parts; j += 64) mx = fmaxf(mx, sm.part_m[j][wave]);
    mx = wave_max(mx);
    float ls = 0.0f;
    for (int j = lane; j < parts; j += 64) {
      const float mj = sm.part_m[j][wave];
      const float f = mj == -INFINITY ? 0.0f : exp2f(mj - mx);
      sm.part_m[j][wave] = f;  // the partial's weight from here on
      ls += f * sm.part_l[j][wave];
    }
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) ls += __shfl_xor(ls, o2, 64);
    if (lane == 0) sm.linv[wave] = 1.0f / ls;
  }
  __syncthreads();
  // eight partials per batch of independent loads
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int i = idx / D, c = idx % D;
    const float* op = p.ws_o + (row0 + i) * D + c;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    int j = 0;
    for (; j + 8 <= parts; j += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = op[(size_t)(j + u) * rows * D];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += sm.part_m[j + u][i] * v[u];
    }
    for (; j < parts; ++j) acc[0] += sm.part_m[j][i] * op[(size_t)j * rows * D];
    const float oo = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    p.out[(row0 + i) * D + c] = oo * sm.linv[i];
  }
}

}  // namespace

int launch_decode_splitk(const DecodePlan& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  dim3 grid(p.n_splits + 1, p.H, p.B);
  if (p.D == 128)
    hipLaunchKernelGGL(decode_kernel<128>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(decode_kernel<64>, grid, dim3(kThreads), 0, s, p);
  return (int)hipGetLastError();
}

int launch_decode_merge(const DecodePlan& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (p.D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(p.H, p.B), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3(p.H, p.B), dim3(kThreads), 0, s, p);
  return (int)hipGetLastError();
}

}  // namespace kvq
