// Multi-token decode with up to 16 query rows per KV head: G query heads x Q query tokens (the
// InnerQ page's "Algorithm 1 ... decode phase" once per query token, GQA heads grouped on
// their shared KV head). One launch reads every packed tile once for all rows, so a step
// that decodes Q tokens (speculative or multi-token decoding) costs one pass over the cache.
//
// Grid (n_splits, KV heads, rows), 4 wavefronts per workgroup; workgroup `split` owns a
// contiguous range of 64-token body tiles, taken round-robin by its wavefronts, and the
// 64-token chunks of the 16-bit sink + recent window are dealt out to the last splits.
// Query row r of KV head h is query token r / G of query head h G + r % G, the (T - Q + r /
// G)-th token; the causal mask only touches window tokens (the host checks that the newest
// Q - 1 tokens are still in the window).
//
// q.K^T: lane = token, the 4x4x4 (16-block) f16 MFMA with B = 4 codes of the lane's token as
// fp16 subnormals (the decode kernel's key slot plans) and A = 4 query rows; the 16 rows take
// four MFMAs per step that share the unpacked B. Each key group's scale and zero are applied
// to its partial sums: q . k_hat = s (q . c) + z sum(q).
// P.V: the 16x16x32 f16 MFMA with rows = the 16 query rows, K = the 32 tokens of one value
// block, columns = 16 channels. A lane's value record holds 8 tokens of one channel of either
// block; one 32-lane swap (v_permlane32_swap) per register pair regroups the unpacked codes
// so that each MFMA sees one block, whose scale and zero are then applied per (block,
// channel): sum_t p_t v_hat_t = s sum_t p_t c_t + z sum_t p_t. Weights travel as fp16 hi + lo.
// 16-bit rows (windows, unquantized heads): keys on the 4x4x4 MFMA with the raw 16-bit q,
// values on the 16x16x32 MFMA (f16 or bf16) with the rows gathered 8 tokens per lane.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include "code_plans.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kDW = 4;                // wavefronts per workgroup
constexpr int kDThreads = 64 * kDW;
constexpr int kR = kMaxDenseRows;     // query rows per KV head (16)
constexpr float kMasked = -1e30f;     // causally masked window score (log2 units)
constexpr int kEpD = 11;              // packed-value weights enter the MFMA as p * 2^(kEpD - e)
constexpr float kTauD = 4.0f;         // lazy rescale threshold (log2 units)
constexpr float kVD = (float)(1 << (24 - kEpD));   // units of the value sums
constexpr float kV1D = (float)(1 << (14 - kEpD));  // units of the weight sums

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <bool BF16>
__device__ __forceinline__ float4_t mfma4(u32x2 a, u32x2 b, float4_t c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(short4_t, a), __builtin_bit_cast(short4_t, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b), c, 0,
                                              0, 0);
}
// 16x16x32: lane l holds A[l % 16][8 (l / 16) + 0..7], B[8 (l / 16) + 0..7][l % 16] and
// D[4 (l / 16) + j][l % 16], j = 0..3
template <bool BF16>
__device__ __forceinline__ float4_t mfma32(u32x4 a, u32x4 b, float4_t c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ int bits_of(const uint8_t* table, int h) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(table)[h >> 2];
  return (int)((w >> (8 * (h & 3))) & 0xFFu);
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
__device__ __forceinline__ void lds_order() { __asm__ __volatile__("" ::: "memory"); }

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max(float v) {
  const int t = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
  return fmaxf(v, __int_as_float(t));
}
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x124, 0xF>(v);  // row_ror:4
  v = dpp_max<0x128, 0xF>(v);  // row_ror:8
  v = dpp_max<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_max<0x143, 0xC>(v);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <int D>
struct DSmem {
  alignas(16) uint32_t qA[kR][D / 2 + 4];  // packed-key A operand: fp16 q * 2^(Eq - e), slot order
  alignas(16) uint32_t qW[kR][D / 2 + 4];  // 16-bit-row A operand: q in the cache dtype
  alignas(16) float qsum[kR][D / 32];      // sum of q over each key group, times the softmax scale
  alignas(8) uint16_t qsh[2][kR][4];      // the same as fp16 hi + lo (groups past D/32 zero)
  // softmax weights per wavefront: [hi/lo][row][token of the 64-token tile] (+8 pad)
  alignas(16) uint16_t pv[kDW][2][kR][72];
  union {
    alignas(16) float qn[kR][D];    // prologue: packed-key query (q, or q * n with key norms)
    float red_o[kDW][kR][D];        // epilogue: the wavefronts' partial outputs
  };
  float red_m[kDW][kR];
  float red_l[kDW][kR];
  float qmax[kDW];
};

// Running softmax state of a wavefront. m: per row, uniform. o[nb][j] and l[j]: row 4 (lane /
// 16) + j, channel 16 nb + lane % 16 (the 16x16x32 output layout), in units of 2^(kEpD - 24)
// and 2^(kEpD - 14).
template <int D>
struct DState {
  float m[kR];
  float4_t o[D / 16];
  float l[4];
};

// Softmax of one 64-token tile (lane = token) for the rows in use: moves the running max
// where a score exceeds it by more than kTauD (rescaling that row's sums), and writes the
// weights p * pscl as hi/lo pairs to the wavefront's LDS rows.
template <int D, int NRG>
__device__ __forceinline__ void softmax_dense(DSmem<D>& sm, int wave, int lane, bool valid, const float (&sc)[kR],
                                              DState<D>& st, float pscl, bool bf16w) {
  const int grp = lane >> 4;
  // every row's score relative to its running max first, then one test for all rows: the
  // common path has a single branch, and the rows' exponentials interleave (the per-row test
  // sits in the rare path)
  float y[4 * NRG];
  float ymax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4 * NRG; ++r) {
    y[r] = (valid ? sc[r] : -INFINITY) - st.m[r];
    ymax = fmaxf(ymax, y[r]);
  }
  if (__ballot(ymax > kTauD)) {
#pragma unroll
    for (int r = 0; r < 4 * NRG; ++r) {
      if (!__ballot(y[r] > kTauD)) continue;
      const float x = valid ? sc[r] : -INFINITY;
      const float mn = fmaxf(st.m[r], wave_max(x));
      const float alpha = __builtin_amdgcn_exp2f(st.m[r] - mn);
      st.m[r] = mn;
      const float a = grp == (r >> 2) ? alpha : 1.0f;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) st.o[nb][r & 3] *= a;
      st.l[r & 3] *= a;
      y[r] = x - mn;
    }
  }
#pragma unroll
  for (int r = 0; r < 4 * NRG; ++r) {
    const float p = __builtin_amdgcn_exp2f(y[r]) * pscl;
    uint32_t hi, lo;
    if (bf16w) {
      hi = f2bf(p);
      lo = f2bf(p - bf2f(hi));
    } else {
      hi = f2h(p);
      lo = f2h(p - h2f(hi));
    }
    sm.pv[wave][0][r][lane] = (uint16_t)hi;
    sm.pv[wave][1][r][lane] = (uint16_t)lo;
  }
  lds_order();
}

// Factor of the weight of body token tb (0..31 of its block) for packed values: 2^(kEpD - e)
// with e the exponent of the token's value slot
template <int VB>
__device__ __forceinline__ float vscale(int tb) {
  float f = 1.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if ((tb & 7) == u)
      f = (tb & 16) ? (float)(1 << kEpD) / (float)(1 << VSlots<VB>::exp(2 + (u >> 2), u & 3))
                    : (float)(1 << kEpD) / (float)(1 << VSlots<VB>::exp(u >> 2, u & 3));
  return f;
}
__device__ __forceinline__ float vscale_rt(int vb, int tb) {
  switch (vb) {
    case 2: return vscale<2>(tb);
    case 3: return vscale<3>(tb);
    case 4: return vscale<4>(tb);
    case 5: return vscale<5>(tb);
    case 6: return vscale<6>(tb);
    case 7: return vscale<7>(tb);
    case 8: return vscale<8>(tb);
    default: return 1.0f;
  }
}
// Constant B operand of the weight sums for K-step kk: slot (u) holds 2^(e - 14), e the
// exponent of token u's value slot, so sum_k A[m][k] ones[k] = sum of p * 2^(kEpD - 14)
template <int B>
__device__ __forceinline__ u32x4 ones_for(int kk) {
  auto one = [&](int u) { return (uint32_t)(VSlots<B>::exp(2 * kk + (u >> 2), u & 3) + 1) << 10; };
  return u32x4{one(0) | (one(1) << 16), one(2) | (one(3) << 16), one(4) | (one(5) << 16),
               one(6) | (one(7) << 16)};
}

// ---- packed tiles: loads through buffer descriptors (an offset past the region reads zeros)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const char* blob, const uint64_t* off, int r) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(blob + off[r]), (short)0,
                                           (int)(uint32_t)(off[r + 1] - off[r]), 0x00020000);
}
__device__ __forceinline__ void ld4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* d) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
}
__device__ __forceinline__ void ld2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* d) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
  d[0] = v[0]; d[1] = v[1];
}

// Scores (log2 units) of the lane's token for every row in use, from packed keys (tile slot pg).
template <int D, int KB, int NRG>
__device__ __forceinline__ void key_packed(const DSmem<D>& sm, __amdgpu_buffer_rsrc_t kc, __amdgpu_buffer_rsrc_t km,
                                           int pg, int lane, float kscale, float (&sc)[kR]) {
  constexpr int NG = D / 32, W = NG * KB;
  uint32_t w[W], m[NG];
  const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)pg * (kTile * W * 4));
#pragma unroll
  for (int q = 0; q < (W + 3) / 4; ++q) {
    const int nq = (W - 4 * q) < 4 ? (W - 4 * q) : 4;
    const uint32_t voff = (uint32_t)(256 * q + lane * nq) * 4;
    if (nq == 4) ld4(kc, voff, soff, &w[4 * q]);
    else ld2(kc, voff, soff, &w[4 * q]);
  }
  const uint32_t msoff = __builtin_amdgcn_readfirstlane((uint32_t)pg * (kTile * NG * 4));
  if constexpr (NG == 4) ld4(km, (uint32_t)lane * NG * 4, msoff, m);
  else ld2(km, (uint32_t)lane * NG * 4, msoff, m);
  const int qi = lane & 3;
  // group by group: the group's 4 row-group chains share each unpacked B operand, and its
  // scale is applied as soon as they end (t1 holds sum_g s_g (q . c_g) per row)
  float t1[4 * NRG];
#pragma unroll
  for (int r = 0; r < 4 * NRG; ++r) t1[r] = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float4_t acc[NRG];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) acc[rg] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x2 bop = unpack_step<KB>(w, g * KB, s);
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(&sm.qA[4 * rg + qi][(g * 8 + s) * 2]);
        acc[rg] = mfma4<false>(a, bop, acc[rg]);
      }
    }
    const float sg = h2f(m[g] & 0xFFFFu);
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int i = 0; i < 4; ++i) t1[4 * rg + i] = __builtin_fmaf(sg, acc[rg][i], t1[4 * rg + i]);
  }
  // sum_g z_g sum(q)_g on the same MFMA: A = the rows' group sums (hi + lo fp16 halves),
  // B = the token's 4 group zeros (fp16, exact)
  const u32x2 zb = u32x2{__builtin_amdgcn_perm(m[1], m[0], 0x07060302u), NG == 4 ? __builtin_amdgcn_perm(m[3], m[2], 0x07060302u) : 0u};
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const u32x2 ah = *reinterpret_cast<const u32x2*>(&sm.qsh[0][4 * rg + qi][0]);
    const u32x2 al = *reinterpret_cast<const u32x2*>(&sm.qsh[1][4 * rg + qi][0]);
    float4_t t2 = mfma4<false>(ah, zb, float4_t{0.0f, 0.0f, 0.0f, 0.0f});
    t2 = mfma4<false>(al, zb, t2);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[4 * rg + i] = __builtin_fmaf(kscale, t1[4 * rg + i], t2[i]);
  }
}

// Scores of the lane's token from its 16-bit key row (x: D/8 16-byte pieces).
template <int D, bool BF16, int NRG>
__device__ __forceinline__ void key_rows16(const DSmem<D>& sm, const uint4 (&x)[D / 8], int lane, float scale_log2,
                                           float (&sc)[kR]) {
  const int qi = lane & 3;
  float4_t acc[NRG];
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) acc[rg] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int v = 0; v < D / 8; ++v)
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(&sm.qW[4 * rg + qi][4 * v]);
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(&sm.qW[4 * rg + qi][4 * v + 2]);
      acc[rg] = mfma4<BF16>(a0, u32x2{x[v].x, x[v].y}, acc[rg]);
      acc[rg] = mfma4<BF16>(a1, u32x2{x[v].z, x[v].w}, acc[rg]);
    }
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[4 * rg + i] = acc[rg][i] * scale_log2;
}

// P.V of one packed value tile (slot pg). Lane (g4, n) = (lane / 16, lane % 16) holds the
// codes of channels 16 nb + n, block g4 / 2, tokens 16 kk + 8 (g4 % 2) + u; after the swap,
// x (y) holds block 0 (1) with K index = token of the block. nblk: blocks with body tokens.
template <int D, int VB>
__device__ __forceinline__ void value_packed(const DSmem<D>& sm, int wave, __amdgpu_buffer_rsrc_t vc,
                                             __amdgpu_buffer_rsrc_t vm, int pg, int lane, int nblk, DState<D>& st) {
  constexpr int NB = D / 16, NW = (NB / 2) * VB;
  uint32_t w[NW], mw[2][NB];
  const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)pg * (2 * D * VB * 4));
  const uint32_t voff = (uint32_t)lane * NW * 4;
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int x = 0; x < NW; x += 4) ld4(vc, voff + 4 * x, soff, &w[x]);
  } else {
#pragma unroll
    for (int x = 0; x < NW; x += 2) ld2(vc, voff + 4 * x, soff, &w[x]);
  }
  const int n = lane & 15;
  const uint32_t msoff = __builtin_amdgcn_readfirstlane((uint32_t)pg * (2 * D * 4));
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int x = 0; x < NB; x += 4) ld4(vm, (uint32_t)(blk * D + n * NB + x) * 4, msoff, &mw[blk][x]);
  // weights: A of block blk, hi/lo hl = row lane % 16, tokens 32 blk + 8 (lane / 16) + 0..7
  u32x4 a[2][2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) a[blk][hl] = *reinterpret_cast<const u32x4*>(&sm.pv[wave][hl][n][32 * blk + 8 * (lane >> 4)]);
  const u32x4 ones = lane < 32 ? ones_for<VB>(0) : ones_for<VB>(1);
  float4_t d1[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    d1[blk] = mfma32<false>(a[blk][0], ones, float4_t{0.0f, 0.0f, 0.0f, 0.0f});
    d1[blk] = mfma32<false>(a[blk][1], ones, d1[blk]);
  }
  // two column blocks at a time: their four MFMA chains hide each other's latency, and
  // their scale and zero are applied as soon as they end
#pragma unroll
  for (int nb0 = 0; nb0 < NB; nb0 += 2) {
    float4_t d[2][2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int nb = nb0 + h2;
      const int base = (nb >> 1) * VB, c0 = 2 * (nb & 1), c1 = c0 + 1;  // chunks of kk = 0, 1
      const u32x2 p0 = unpack_step_v<VB>(w, base, 2 * c0), p1 = unpack_step_v<VB>(w, base, 2 * c0 + 1);
      const u32x2 p2 = unpack_step_v<VB>(w, base, 2 * c1), p3 = unpack_step_v<VB>(w, base, 2 * c1 + 1);
      const uint32_t k0[4] = {p0.x, p0.y, p1.x, p1.y}, k1[4] = {p2.x, p2.y, p3.x, p3.y};
      u32x4 x, y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto sw = __builtin_amdgcn_permlane32_swap(k0[i], k1[i], false, false);
        x[i] = sw[0];
        y[i] = sw[1];
      }
      d[h2][0] = mfma32<false>(a[0][0], x, float4_t{0.0f, 0.0f, 0.0f, 0.0f});
      d[h2][1] = mfma32<false>(a[1][0], y, float4_t{0.0f, 0.0f, 0.0f, 0.0f});
      d[h2][0] = mfma32<false>(a[0][1], x, d[h2][0]);
      d[h2][1] = mfma32<false>(a[1][1], y, d[h2][1]);
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const uint32_t sz = blk < nblk ? mw[blk][nb0 + h2] : 0u;  // an empty block's meta was never written
        const float sv = h2f(sz & 0xFFFFu), zv = h2f(sz >> 16) * (kV1D / kVD);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st.o[nb0 + h2][j] = __builtin_fmaf(sv, d[h2][blk][j], __builtin_fmaf(zv, d1[blk][j], st.o[nb0 + h2][j]));
      }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) st.l[j] += d1[0][j] + d1[1][j];
}

// P.V of 64 tokens of 16-bit value rows: K-step kk = tokens 32 kk + 8 (lane / 16) + 0..7 of
// channel 16 nb + lane % 16, gathered per lane (row u0 + t, clamped to the last valid row,
// whose weight is 0).
template <int D, bool BF16, class VRowOf>
__device__ __forceinline__ void value_rows16(const DSmem<D>& sm, int wave, int lane, int n_valid, VRowOf vrow,
                                             DState<D>& st) {
  constexpr int NB = D / 16;
  const int n = lane & 15;
  const uint32_t one1 = BF16 ? 0x3F80u : 0x3C00u;
  const u32x4 ones = u32x4{one1 * 0x10001u, one1 * 0x10001u, one1 * 0x10001u, one1 * 0x10001u};
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    if (32 * kk >= n_valid) continue;
    const u32x4 ahi = *reinterpret_cast<const u32x4*>(&sm.pv[wave][0][n][32 * kk + 8 * (lane >> 4)]);
    const u32x4 alo = *reinterpret_cast<const u32x4*>(&sm.pv[wave][1][n][32 * kk + 8 * (lane >> 4)]);
    float4_t d1 = mfma32<BF16>(ahi, ones, float4_t{0.0f, 0.0f, 0.0f, 0.0f});
    d1 = mfma32<BF16>(alo, ones, d1);
    const uint16_t* rows[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rows[j] = vrow(min(32 * kk + 8 * (lane >> 4) + j, n_valid - 1));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint32_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = rows[j][16 * nb + n];
      const u32x4 bop = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
      float4_t d = mfma32<BF16>(ahi, bop, float4_t{0.0f, 0.0f, 0.0f, 0.0f});
      d = mfma32<BF16>(alo, bop, d);
#pragma unroll
      for (int j = 0; j < 4; ++j) st.o[nb][j] = __builtin_fmaf(d[j], 1.0f / kVD, st.o[nb][j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) st.l[j] = __builtin_fmaf(d1[j], 1.0f / kV1D, st.l[j]);
  }
}

// NRG: row groups of 4 in use (rows past G Q hold a zero query and are not written out)
template <int D, int NRG>
// two wavefronts per SIMD (two workgroups per CU): the register budget is 256
__global__ __launch_bounds__(kDThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_dense_kernel(const DecodePlan p) {
  __shared__ DSmem<D> sm;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G, R = G * p.Q;
  const int kb = bits_of(p.k_bits, h), vb = bits_of(p.v_bits, h);
  auto grow = [&](int r) { return ((size_t)b * p.Q + r / G) * p.Hq + (size_t)h * G + r % G; };
  const uint64_t* tab = p.off + ((size_t)b * p.H + h) * kRegions;
  uint64_t off[kRegions];
#pragma unroll
  for (int r = 0; r < kRegions; ++r) off[r] = tab[r];

  // ---- query rows (all wavefronts together): raw 16-bit copy, packed-key query (q * n with
  // key norms), per-group sums, then the fp16 key operand for this head's width with q
  // scaled by 2^Eq so that max |q| 2^Eq lies in [2^14, 2^15)
  constexpr int E = kR * D / kDThreads;  // 8 (D = 128) or 4 (D = 64) consecutive elements per thread
  {
    const int i0 = tid * E / D, c0 = tid * E % D;
    const bool live = i0 < R;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(p.q) + grow(live ? i0 : R - 1) * D + c0;
    uint32_t qw[E / 2];
    if constexpr (E == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      qw[0] = v.x; qw[1] = v.y; qw[2] = v.z; qw[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      qw[0] = v.x; qw[1] = v.y;
    }
    const float* kn = p.key_norm && kb != 16 ? reinterpret_cast<const float*>(p.blob + off[KN]) + c0 : nullptr;
    float qmax = 0.0f, qs = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t qh = live ? (qw[e / 2] >> (16 * (e & 1))) & 0xFFFFu : 0u;
      reinterpret_cast<uint16_t*>(sm.qW[i0])[c0 + e] = (uint16_t)qh;
      const float v = widen(qh, p.dtype) * (kn ? kn[e] : 1.0f);
      sm.qn[i0][c0 + e] = v;
      qmax = fmaxf(qmax, fabsf(v));
      qs += v;
    }
#pragma unroll
    for (int o2 = 16 / E; o2 >= 1; o2 >>= 1) qs += __shfl_xor(qs, o2, 64);
    if (c0 % 32 == 0) sm.qsum[i0][c0 / 32] = qs * p.scale_log2;
    qmax = wave_max(qmax);
    if (lane == 0) sm.qmax[wave] = qmax;
    // this wavefront's weight rows start at zero (rows past R are read by the value MFMAs)
    uint32_t* pz = reinterpret_cast<uint32_t*>(&sm.pv[wave][0][0][0]);
    for (int i = lane; i < 2 * kR * 72 / 2; i += 64) pz[i] = 0u;
  }
  __syncthreads();
  if (tid < kR * 4) {
    const int r = tid / 4, g = tid % 4;
    const float v = g < D / 32 ? sm.qsum[r][g] : 0.0f;
    const uint32_t hi = f2h(v);
    sm.qsh[0][r][g] = (uint16_t)hi;
    sm.qsh[1][r][g] = (uint16_t)f2h(v - h2f(hi));
  }
  int Eq = 0;
  {
    const float qm = fmaxf(fmaxf(sm.qmax[0], sm.qmax[1]), fmaxf(sm.qmax[2], sm.qmax[3]));
    int qe = 0;
    if (qm > 0.0f) (void)frexpf(qm, &qe);
    Eq = 15 - qe;
  }
  if (kb != 16) {
    // slot (g * 8 + s) * 4 + k of row i holds q_i of channel 32 g + chan(s, k) times 2^(Eq -
    // exp(s, k)); a thread's slot index, tid % D, is the same for every row it writes
    auto build = [&](auto bc) {
      constexpr int B = decltype(bc)::value;
      const int slot = tid % D, s = (slot >> 2) & 7, k = slot & 3, g = slot / 32;
      int ch = 0, ex = 0;
#pragma unroll
      for (int ss = 0; ss < 8; ++ss)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          if (s == ss && k == kk) {
            ch = Slots<B>::chan(ss, kk);
            ex = Slots<B>::exp(ss, kk);
          }
      for (int i = tid / D; i < kR; i += kDThreads / D)
        reinterpret_cast<uint16_t*>(sm.qA[i])[slot] = (uint16_t)f2h(__builtin_ldexpf(sm.qn[i][g * 32 + ch], Eq - ex));
    };
    switch (kb) {
      case 2: build(std::integral_constant<int, 2>{}); break;
      case 3: build(std::integral_constant<int, 3>{}); break;
      case 4: build(std::integral_constant<int, 4>{}); break;
      case 5: build(std::integral_constant<int, 5>{}); break;
      case 6: build(std::integral_constant<int, 6>{}); break;
      case 7: build(std::integral_constant<int, 7>{}); break;
      default: build(std::integral_constant<int, 8>{}); break;
    }
  }
  __syncthreads();  // qA complete; qn is dead from here on (red_o shares its memory)
  const float kscale = __builtin_ldexpf(p.scale_log2, 24 - Eq);

  DState<D> st;
#pragma unroll
  for (int r = 0; r < kR; ++r) st.m[r] = -INFINITY;
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) st.o[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) st.l[j] = 0.0f;

  const int body = p.body;
  const int t0 = split * p.tiles_per_split, t1 = min(p.n_tiles, t0 + p.tiles_per_split);
  const int32_t* pages = p.pages ? p.pages + (size_t)b * p.page_stride : nullptr;
  auto page_of = [&](int t) {
    if (!pages) return t;
    const int pg = pages[t];  // an unmapped entry is clamped into the pools (its values are meaningless)
    return pg < 0 ? 0 : (pg >= p.n_pages ? p.n_pages - 1 : pg);
  };
  const bool bf = p.dtype == KVQ_BF16;
  float sc[kR];

  // ---- body tiles [t0, t1), round-robin over the wavefronts
  const auto kc = rsrc(p.blob, off, KC), km = rsrc(p.blob, off, KM);
  const auto vcr = rsrc(p.blob, off, VC), vmr = rsrc(p.blob, off, VM);
  const uint16_t* kr16 = reinterpret_cast<const uint16_t*>(p.blob + off[KC]);
  const uint16_t* vr16 = reinterpret_cast<const uint16_t*>(p.blob + off[VC]);
  for (int t = t0 + wave; t < t1; t += kDW) {
    // the lane index, opaque to the compiler for this iteration: the per-lane offsets of every
    // width's loads derive from it, and hoisting those of all widths out of the loop would hold
    // dozens of registers across it
    int lane = threadIdx.x & 63;
    __asm__ __volatile__("" : "+v"(lane));
    const int pg = page_of(t);
    const int n_valid = min(kTile, body - t * kTile);
    const bool valid = lane < n_valid;
    if (kb == 16) {
      uint4 x[D / 8];
      const uint4* r4 = reinterpret_cast<const uint4*>(kr16 + ((size_t)pg * kTile + (valid ? lane : 0)) * D);
#pragma unroll
      for (int v = 0; v < D / 8; ++v) x[v] = r4[v];
      if (bf) key_rows16<D, true, NRG>(sm, x, lane, p.scale_log2, sc);
      else key_rows16<D, false, NRG>(sm, x, lane, p.scale_log2, sc);
    } else {
      switch (kb) {
        case 2: key_packed<D, 2, NRG>(sm, kc, km, pg, lane, kscale, sc); break;
        case 3: key_packed<D, 3, NRG>(sm, kc, km, pg, lane, kscale, sc); break;
        case 4: key_packed<D, 4, NRG>(sm, kc, km, pg, lane, kscale, sc); break;
        case 5: key_packed<D, 5, NRG>(sm, kc, km, pg, lane, kscale, sc); break;
        case 6: key_packed<D, 6, NRG>(sm, kc, km, pg, lane, kscale, sc); break;
        case 7: key_packed<D, 7, NRG>(sm, kc, km, pg, lane, kscale, sc); break;
        default: key_packed<D, 8, NRG>(sm, kc, km, pg, lane, kscale, sc); break;
      }
    }
    if (vb == 16) {
      softmax_dense<D, NRG>(sm, wave, lane, valid, sc, st, 1.0f, bf);
      auto vrow = [&](int u) { return vr16 + ((size_t)pg * kTile + u) * D; };
      if (bf) value_rows16<D, true>(sm, wave, lane, n_valid, vrow, st);
      else value_rows16<D, false>(sm, wave, lane, n_valid, vrow, st);
    } else {
      softmax_dense<D, NRG>(sm, wave, lane, valid, sc, st, vscale_rt(vb, lane & 31), false);
      const int nblk = min(2, n_valid / kGroup);
      switch (vb) {
        case 2: value_packed<D, 2>(sm, wave, vcr, vmr, pg, lane, nblk, st); break;
        case 3: value_packed<D, 3>(sm, wave, vcr, vmr, pg, lane, nblk, st); break;
        case 4: value_packed<D, 4>(sm, wave, vcr, vmr, pg, lane, nblk, st); break;
        case 5: value_packed<D, 5>(sm, wave, vcr, vmr, pg, lane, nblk, st); break;
        case 6: value_packed<D, 6>(sm, wave, vcr, vmr, pg, lane, nblk, st); break;
        case 7: value_packed<D, 7>(sm, wave, vcr, vmr, pg, lane, nblk, st); break;
        default: value_packed<D, 8>(sm, wave, vcr, vmr, pg, lane, nblk, st); break;
      }
    }
    lds_order();
  }

  // ---- the 16-bit sink + window tokens, 64 at a time: chunk w goes to split n_splits - 1 -
  // w % n_splits (the last splits have the fewest body tiles), wavefront (w / n_splits) % 4.
  // Window token u < n_sink_live is sink row u, else ring slot (ring0 + u - n_sink_live) mod
  // ring; its position in the sequence is u (sink) or u + body (ring).
  {
    const int nsl = p.n_sink_live, n_wtok = nsl + p.n_win;
    const uint16_t* sk = reinterpret_cast<const uint16_t*>(p.blob + off[SK]);
    const uint16_t* sv = reinterpret_cast<const uint16_t*>(p.blob + off[SV]);
    const uint16_t* rk = reinterpret_cast<const uint16_t*>(p.blob + off[RK]);
    const uint16_t* rv = reinterpret_cast<const uint16_t*>(p.blob + off[RV]);
    auto slot = [&](int u) {
      const int r = p.ring0 + (u - nsl);
      return r >= p.ring ? r - p.ring : r;
    };
    const int n_chunks = (n_wtok + kTile - 1) / kTile;
    for (int w = 0; w < n_chunks; ++w) {
      if (p.n_splits - 1 - w % p.n_splits != split || (w / p.n_splits) % kDW != wave) continue;
      int lane = threadIdx.x & 63;  // opaque per chunk, as in the body loop
      __asm__ __volatile__("" : "+v"(lane));
      const int u0 = w * kTile, n_valid = min(kTile, n_wtok - u0);
      const int u = u0 + min(lane, n_valid - 1);
      const uint16_t* krow = u < nsl ? sk + (size_t)u * D : rk + (size_t)slot(u) * D;
      uint4 x[D / 8];
#pragma unroll
      for (int v = 0; v < D / 8; ++v) x[v] = reinterpret_cast<const uint4*>(krow)[v];
      if (bf) key_rows16<D, true, NRG>(sm, x, lane, p.scale_log2, sc);
      else key_rows16<D, false, NRG>(sm, x, lane, p.scale_log2, sc);
      if (p.Q > 1) {
        // row r (query token r / G) sees no later token; a masked score is a huge finite
        // negative so that a chunk with no visible token keeps a finite running max (its
        // terms vanish once a visible token, which every row has, raises it)
        const int pos = u < nsl ? u : u + body;
#pragma unroll
        for (int r = 0; r < 4 * NRG; ++r)
          if (pos > p.T - p.Q + r / G) sc[r] = kMasked;
      }
      softmax_dense<D, NRG>(sm, wave, lane, lane < n_valid, sc, st, 1.0f, bf);
      auto vrow = [&](int k) {
        const int uu = u0 + k;
        return uu < nsl ? sv + (size_t)uu * D : rv + (size_t)slot(uu) * D;
      };
      if (bf) value_rows16<D, true>(sm, wave, lane, n_valid, vrow, st);
      else value_rows16<D, false>(sm, wave, lane, n_valid, vrow, st);
      lds_order();
    }
  }

  // ---- combine the wavefronts into one partial (m, l, o) per row
  {
    const int grp = lane >> 4, n = lane & 15;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.red_o[wave][4 * grp + j][16 * nb + n] = st.o[nb][j] * kVD;
    if (n == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.red_l[wave][4 * grp + j] = st.l[j] * kV1D;
    }
    if (lane < kR) {
      float mr = st.m[0];
#pragma unroll
      for (int r = 1; r < kR; ++r)
        if (lane == r) mr = st.m[r];
      sm.red_m[wave][lane] = mr;
    }
  }
  if (pages && h == 0 && wave == kDW - 1) {
    // the tiles this workgroup read must be mapped (an unmapped one was read from a clamped
    // page): reported through the sticky flag, bit 1
    bool bad = false;
    for (int t = t0 + lane; t < t1; t += 64) {
      const int pg = pages[t];
      bad |= pg < 0 || pg >= p.n_pages;
    }
    if (__ballot(bad) && lane == 0) atomicOr(p.flag, 2u);
  }
  __syncthreads();
  const size_t rows = (size_t)p.B * p.Q * p.Hq;
  for (int idx = tid; idx < R * D; idx += kDThreads) {
    const int i = idx / D, c = idx % D;
    float mw[kDW], ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDW; ++w) {
      mw[w] = sm.red_m[w][i];
      ms = fmaxf(ms, mw[w]);
    }
    float oo = 0.0f, ll = 0.0f;
    if (ms != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDW; ++w) {
        const float f = __builtin_amdgcn_exp2f(mw[w] - ms);  // 0 for an empty wavefront (-inf)
        oo = __builtin_fmaf(f, sm.red_o[w][i][c], oo);
        ll = __builtin_fmaf(f, sm.red_l[w][i], ll);
      }
    }
    p.ws_o[((size_t)split * rows + grow(i)) * D + c] = oo;
    if (c == 0) {
      p.ws_ml[((size_t)split * rows + grow(i)) * 2] = ms;
      p.ws_ml[((size_t)split * rows + grow(i)) * 2 + 1] = ll;
    }
  }
}

}  // namespace

int launch_decode_dense(const DecodePlan& p, void* stream) {
  dim3 grid(p.n_splits, p.H, p.B);
  hipStream_t s = (hipStream_t)stream;
  const bool two = p.G * p.Q <= 8;  // rows in two groups of 4, else four
  if (p.D == 128) {
    if (two) hipLaunchKernelGGL((decode_dense_kernel<128, 2>), grid, dim3(kDThreads), 0, s, p);
    else hipLaunchKernelGGL((decode_dense_kernel<128, 4>), grid, dim3(kDThreads), 0, s, p);
  } else {
    if (two) hipLaunchKernelGGL((decode_dense_kernel<64, 2>), grid, dim3(kDThreads), 0, s, p);
    else hipLaunchKernelGGL((decode_dense_kernel<64, 4>), grid, dim3(kDThreads), 0, s, p);
  }
  return (int)hipGetLastError();
}

}  // namespace kvq
