// Split-K decode attention over the packed cache, dequantization fused into q.K^T and P.V
// (InnerQ: grouping along the inner dimension of each vector-matrix product; the decode
// structure of its "Algorithm 1 ... decode phase"); the log-sum-exp merge of the split
// partials is a second, small kernel.
//
// Grid (n_splits, KV heads, rows), 4 wavefronts per workgroup. Workgroup `split` owns a
// contiguous range of 64-token body tiles (its wavefronts take them round-robin); the 64-token
// tiles of the 16-bit sink + recent-window tokens are dealt out one per workgroup to the
// wavefronts with the fewest body tiles, so the windows cost no workgroup of their own.
//
// q.K^T runs on the 4x4x4 (16-block) f16/bf16 MFMA. Lane l belongs to block l/4 and to
// row/column l%4, and the G <= 4 query heads of a KV head are the 4-wide dimension: lane =
// token, B operand = 4 codes of the lane's token, A = the 4 matching q values of query l%4;
// output element i is query i's partial dot for that token.
// P.V of packed tiles runs on the 16x16x32 f16 MFMA: rows = (32-token block, hi/lo half of
// the weight, query), K = 16 tokens of each block per step, columns = 16 channels; the lane's
// B operand is 8 consecutive tokens of one channel. 16-bit window rows use the 4x4x4 MFMA with
// lane = channel (for D = 128 the adjacent channels 2l and 2l+1).
// Codes enter the MFMA as fp16 subnormals: one shift and one AND of a packed word leave two
// codes in the top mantissa bits of two fp16 halves, i.e. the values c * 2^(e - 24) (slot
// plans in code_plans.h). The 2^e of each slot is divided out of the matching A value (q or
// p), so every product is exact and each sum carries one known power of two.
// Each group's scale and zero are applied once to its partial sums:
//   q . k_hat = s (q . c) + z sum(q)                     key group: 32 channels of a token
//   sum_t p_t v_hat_t = s sum_t p_t c_t + z sum_t p_t    value group: 32 tokens of a channel
// Softmax weights travel as an fp16 (bf16 for bf16 windows) pair hi + lo; sum_t p_t comes
// from the same MFMA with a constant operand, so numerator and denominator use identical
// weights.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <type_traits>

#include <math.h>

#include <mutex>

#include "code_plans.h"  // slot plans and code unpacking (shared with the append kernel)
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxG = 4;
constexpr float kMaskedScore = -1e30f;  // causally masked window score (log2 units)
constexpr int kEp = 11;  // softmax weights enter the value MFMA as p * 2^(kEp - e)
// The key zero-term operand carries 2^kZShift on top of the packed-key scale, so that its
// fp16 lo half stays a normal number for the usual group sums (at most 2^8 in all)
constexpr int kZShift = 12;
// Lazy rescaling: the running max m moves only when a score exceeds it by more than kTau
// (log2 units), so weights stay below 2^kTau and p * 2^kEp * 2^kTau fits fp16.
constexpr float kTau = 4.0f;

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float4_t mfma_f16(u32x2 a, u32x2 b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma_bf16(u32x2 a, u32x2 b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(short4_t, a), __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
}
// 16x16x32 f16: lane l holds A[l % 16][8 (l / 16) + 0..7] and B[8 (l / 16) + 0..7][l % 16] (8
// halves each, as 4 registers) and D[4 (l / 16) + r][l % 16], r = 0..3
__device__ __forceinline__ float4_t mfma_f16_k32(u32x4 a, u32x4 b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                0, 0);
}
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
template <bool BF16>
__device__ __forceinline__ float4_t mfma_k32(u32x4 a, u32x4 b, float4_t c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  else
    return mfma_f16_k32(a, b, c);
}
template <bool BF16>
__device__ __forceinline__ float4_t mfma16(u32x2 a, u32x2 b, float4_t c) {
  if constexpr (BF16) return mfma_bf16(a, b, c);
  else return mfma_f16(a, b, c);
}

// Width of head h from a word-aligned per-head byte table in the kernel arguments, read a
// word at a time: a scalar load for uniform h, where a byte load would take the vector path.
__device__ __forceinline__ int head_bits(const uint8_t* table, int h) {
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

// Sums over the two 32-lane halves of a and b at once: the 16-lane rows of the result hold
// a0 + a2, a1 + a3, b0 + b2, b1 + b3 (row r of x is xr; one 32-lane swap, all VALU).
__device__ __forceinline__ float sum_halves(float a, float b) {
  const auto ab = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(ab[0]) + __uint_as_float(ab[1]);
}

// LDS traffic of one wavefront is executed in issue order, so a wavefront reading back what
// it wrote only needs the compiler not to reorder the accesses.
__device__ __forceinline__ void wave_lds_sync() { __asm__ __volatile__("" ::: "memory"); }

// Keeps global loads issued above this point from being sunk below it (software prefetch).
__device__ __forceinline__ void issue_barrier() { __asm__ __volatile__("" ::: "memory"); }

// fp16 2^(exp - 14) in the slot of token u = 0..7 of a chunk of K-step kk
template <int B>
__device__ __forceinline__ u32x4 ones_chunk(int kk) {
  auto one = [&](int u) { return (uint32_t)(VSlots<B>::exp(2 * kk + (u >> 2), u & 3) + 1) << 10; };
  return u32x4{one(0) | (one(1) << 16), one(2) | (one(3) << 16), one(4) | (one(5) << 16),
               one(6) | (one(7) << 16)};
}

template <int D>
struct Smem {
  // Query operands, one copy per wavefront: each wavefront builds its own, so no workgroup
  // barrier stands between the start of the launch and its first tiles' compute.
  // Rows of the 4 query slots are padded by 4 words so that the 4 distinct addresses of an
  // operand read fall in different LDS banks
  // (16-byte alignment lets operand reads use one ds_read_b64 with an immediate offset)
  alignas(16) uint32_t qA[kWaves][kMaxG][D / 2 + 4];  // key-MFMA A operand: fp16 q * 2^(Eq - e), slot order
  alignas(16) uint32_t qW[kWaves][kMaxG][D / 2 + 4];  // 16-bit-row A operand: q in the cache dtype
  // key zero term operand: sum of q over each key group times 2^(Eq - 24 + kZShift), as fp16
  // hi + lo halves ([hi/lo][query][group], groups past D/32 zero)
  alignas(8) uint16_t qz[kWaves][2][kMaxG][4];
  alignas(16) uint32_t pw[kWaves][2][kMaxG][36];  // per wave: hi/lo, query, 2 blocks x 16 words (+4 pad)
  // packed-body weights per wave: [32-token block][hi/lo][query][token], fp16, rows padded to
  // 40 halves; plus 32 zero halves for the operand rows of the other block
  alignas(16) uint16_t pv[kWaves][2][2][kMaxG][40];
  alignas(16) uint16_t zero16[32];
  union {
    alignas(16) float qn[kWaves][kMaxG][D];  // prologue: packed-key query, q or q * n with key normalization
    float red_o[kWaves][kMaxG][D];           // epilogue: the wavefronts' partial outputs
  };
  float red_m[kWaves][kMaxG];
  float red_l[kWaves][kMaxG];
  float new_s[kMaxG];  // fused decode step: scores of the appended token (log2 units)
};

template <int D>
struct WaveState {
  float m[kMaxG];          // running max of the scores (log2 units), uniform over the wave
  float l[kMaxG];          // weight sum of the 16-bit rows, uniform over the wave
  float o[kMaxG][D / 64];  // 16-bit rows: channel (D/64) lane + h
  // packed body: lane (g4, n) holds channel 16 nb + n of queries 2 (g4 % 2) and 2 (g4 % 2) + 1
  // over the tokens of block g4 / 2; the two blocks' lanes are added at the end
  float ob[D / 16][2];
  float lb[2];
};

// Softmax for one tile (lane = token): the weight of query i, scaled by pscl, is written to
// LDS as a hi/lo pair at wdst[i * i_stride] and wdst[hl_stride + i * i_stride]; the
// accumulators in use are rescaled when the running max moves. 16-bit rows (kBody false) are
// all processed before the first packed body tile, so then the body accumulators are still
// zero and left alone.
template <int D, bool kBody>
__device__ __forceinline__ void softmax_tile(bool valid, const float (&sc)[kMaxG], WaveState<D>& st, uint16_t* wdst,
                                             int hl_stride, int i_stride, float pscl, bool bf16_weights) {
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    const float x = valid ? sc[i] : -INFINITY;
    if (__ballot(x > st.m[i] + kTau)) {  // rare after the first tile: move the running max
      const float mn = fmaxf(st.m[i], wave_max(x));
      const float alpha = __builtin_amdgcn_exp2f(st.m[i] - mn);
      st.m[i] = mn;
      st.l[i] *= alpha;
#pragma unroll
      for (int h = 0; h < D / 64; ++h) st.o[i][h] *= alpha;
      if (kBody) {  // the lanes holding query i: query pair i / 2, slot i % 2
        const float f = ((__lane_id() >> 4) & 1) == (i >> 1) ? alpha : 1.0f;
        st.lb[i & 1] *= f;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) st.ob[nb][i & 1] *= f;
      }
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
    wdst[i * i_stride] = (uint16_t)hi;
    wdst[hl_stride + i * i_stride] = (uint16_t)lo;
  }
  wave_lds_sync();
}

// LDS destination of the softmax weights of the lane's token, for 16-bit rows (value slot
// ppos of block lane / 32) and for the packed body (token lane % 32 of block lane / 32)
template <int D>
__device__ __forceinline__ void softmax_rows16(Smem<D>& sm, int wave, int lane, bool valid, const float (&sc)[kMaxG],
                                               WaveState<D>& st, int ppos, float pscl, bool bf16_weights) {
  uint16_t* dst = reinterpret_cast<uint16_t*>(&sm.pw[wave][0][0][16 * (lane >> 5)]) + ppos;
  softmax_tile<D, false>(valid, sc, st, dst, kMaxG * 36 * 2, 36 * 2, pscl, bf16_weights);
}
template <int D>
__device__ __forceinline__ void softmax_body(Smem<D>& sm, int wave, int lane, bool valid, const float (&sc)[kMaxG],
                                             WaveState<D>& st, float pscl) {
  uint16_t* dst = &sm.pv[wave][lane >> 5][0][0][lane & 31];
  softmax_tile<D, true>(valid, sc, st, dst, kMaxG * 40, 40, pscl, false);
}

// Softmax of one packed tile for the fast loop, from the unscaled scores t1 (score = kscale *
// t1): y = score - m comes out of one FMA and is tested against kTau directly, so the common
// path costs one FMA, one compare and one exp per query. FULL: every token of the tile is in
// the body (no validity masking).
template <int D, bool FULL>
__device__ __forceinline__ void softmax_body_rel(Smem<D>& sm, int wave, int lane, bool valid, const float (&t1)[kMaxG],
                                                 float kscale, WaveState<D>& st, float pscl) {
  uint16_t* wdst = &sm.pv[wave][lane >> 5][0][0][lane & 31];
  // all four queries first, then one test: the common path has a single branch, so the four
  // score chains and exponentials can interleave
  float y[kMaxG];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    y[i] = __builtin_fmaf(kscale, t1[i], -st.m[i]);
    if (!FULL && !valid) y[i] = -INFINITY;
  }
  if (__ballot(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])) > kTau)) {
    // rare after the first tile (m = -inf gives y = +inf): move m for the queries that need it
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) {
      if (!__ballot(y[i] > kTau)) continue;
      const float x = (FULL || valid) ? kscale * t1[i] : -INFINITY;
      const float mn = fmaxf(st.m[i], wave_max(x));
      const float alpha = __builtin_amdgcn_exp2f(st.m[i] - mn);
      st.m[i] = mn;
      st.l[i] *= alpha;
#pragma unroll
      for (int h = 0; h < D / 64; ++h) st.o[i][h] *= alpha;
      const float f = ((__lane_id() >> 4) & 1) == (i >> 1) ? alpha : 1.0f;  // lanes of query i
      st.lb[i & 1] *= f;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) st.ob[nb][i & 1] *= f;
      y[i] = x - mn;
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    const float pw = __builtin_amdgcn_exp2f(y[i]) * pscl;
    const uint32_t hi = f2h(pw), lo = f2h(pw - h2f(hi));
    wdst[i * 40] = (uint16_t)hi;
    wdst[kMaxG * 40 + i * 40] = (uint16_t)lo;
  }
  wave_lds_sync();
}

// The fp16 key-MFMA A operand of a wavefront, in slot order: slot (g * 8 + s) * 4 + k of query
// row i holds q_i of channel 32 g + chan(s, k) times 2^(Eq - exp(s, k)) (q means q * n with
// key normalization), from the wavefront's packed-key query in LDS. Lane l writes slots l,
// l + 64, ... of every row; their (s, k) is (l / 4 % 8, l % 4) whatever the row and group, so
// the slot plan is read once per lane, from compile-time constants.
template <int D, int B>
__device__ __forceinline__ void build_key_operand(Smem<D>& sm, int wave, int lane, int Eq) {
  const int s = (lane >> 2) & 7, k = lane & 3;
  int ch = 0, e = 0;
#pragma unroll
  for (int ss = 0; ss < 8; ++ss)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      if (s == ss && k == kk) {
        ch = Slots<B>::chan(ss, kk);
        e = Slots<B>::exp(ss, kk);
      }
#pragma unroll
  for (int idx = lane; idx < kMaxG * D; idx += 64) {
    const int i = idx / D, slot = idx % D, g = slot / 32;
    const float qv = sm.qn[wave][i][g * 32 + ch];
    reinterpret_cast<uint16_t*>(sm.qA[wave][i])[slot] = (uint16_t)f2h(__builtin_ldexpf(qv, Eq - e));
  }
  wave_lds_sync();
}
// The same for a width known only at run time (16-bit keys have no packed operand).
template <int D>
__device__ __forceinline__ void build_key_operand_rt(Smem<D>& sm, int wave, int lane, int Eq, int kb) {
  switch (kb) {
    case 2: build_key_operand<D, 2>(sm, wave, lane, Eq); break;
    case 3: build_key_operand<D, 3>(sm, wave, lane, Eq); break;
    case 4: build_key_operand<D, 4>(sm, wave, lane, Eq); break;
    case 5: build_key_operand<D, 5>(sm, wave, lane, Eq); break;
    case 6: build_key_operand<D, 6>(sm, wave, lane, Eq); break;
    case 7: build_key_operand<D, 7>(sm, wave, lane, Eq); break;
    case 8: build_key_operand<D, 8>(sm, wave, lane, Eq); break;
    default: break;
  }
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
  static constexpr int NB = D / 16;  // 16-channel column blocks of the value MFMA
  uint32_t w[(NB / 2) * VB];         // the lane's NB/2 streams of 32 codes
  uint32_t m[NB];                    // (s|z) of channel 16 nb + lane % 16, block lane / 32
};

// Body regions read through buffer descriptors: each load is base (descriptor) + the lane's
// fixed byte offset (a VGPR computed once) + the tile's byte offset (an SGPR). No address
// register is rewritten per tile, so none can alias the destination of a load still in
// flight, and an offset past the region returns zeros instead of faulting.
constexpr int kWavePages = 64;  // page numbers one wavefront register holds (one per lane)

// Paged caches also carry the row's page table: tile t is read from page pages[t] of the
// head's pools.
struct BodySrc {
  __amdgpu_buffer_rsrc_t kc, km, vc, vm;
  const int32_t* pages;  // null for contiguous caches
  int n_pages;
};
// The page (paged caches) or region slot (contiguous caches) of body tile `tile`. An unmapped
// entry is clamped into the pools, so reading it stays in bounds (its values are meaningless).
__device__ __forceinline__ int body_page(const int32_t* pages, int n_pages, int tile) {
  if (!pages) return tile;
  const int pg = pages[tile];
  return pg < 0 ? 0 : (pg >= n_pages ? n_pages - 1 : pg);
}
// Slot of body token u (16-bit rows) in the region or pools.
__device__ __forceinline__ int body_row(const int32_t* pages, int n_pages, int u) {
  return body_page(pages, n_pages, u / kTile) * kTile + u % kTile;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t region_rsrc(const char* blob, const uint64_t* off, int r) {
  // 0x00020000: raw (untyped) buffer, 32-bit dwords
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(blob + off[r]), (short)0,
                                           (int)(uint32_t)(off[r + 1] - off[r]), 0x00020000);
}
// The body regions with zero length: every load through them returns zeros without reading
// memory, whatever its offsets (the bounds check fails for any offset).
__device__ __forceinline__ BodySrc body_src_empty(const DecodePlan& p, const uint64_t* off) {
  auto empty = [&](int r) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.blob + off[r]), (short)0, 0, 0x00020000);
  };
  return BodySrc{empty(KC), empty(KM), empty(VC), empty(VM), nullptr, 0};
}
// paged = false drops the page lookups at compile time (contiguous caches)
__device__ __forceinline__ BodySrc body_src(const DecodePlan& p, const uint64_t* off, bool paged, int b) {
  return BodySrc{region_rsrc(p.blob, off, KC), region_rsrc(p.blob, off, KM), region_rsrc(p.blob, off, VC),
                 region_rsrc(p.blob, off, VM), paged && p.pages ? p.pages + (size_t)b * p.page_stride : nullptr,
                 p.n_pages};
}
// Cache policy of the body loads: non-temporal (nt). Every packed byte is read once per
// launch, and streaming it past the caches this way measured 7 % faster than the default
// policy on the 32k-token decode.
constexpr int kStreamLoad = 2;
__device__ __forceinline__ void bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* d) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kStreamLoad);
  d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
}
__device__ __forceinline__ void bload2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* d) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kStreamLoad);
  d[0] = v[0]; d[1] = v[1];
}

template <int D, int KB>
__device__ __forceinline__ void load_k(KTile<D, KB>& t, const BodySrc& src, int tile, int lane) {
  constexpr int W = KTile<D, KB>::W;
  const int pg = body_page(src.pages, src.n_pages, tile);
  // the tile offset is uniform: keep it in a scalar register, or the compiler may wrap every
  // load in a loop over the distinct values of a vector register
  const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)pg * (kTile * W * 4));
#pragma unroll
  for (int q = 0; q < (W + 3) / 4; ++q) {
    const int nq = (W - 4 * q) < 4 ? (W - 4 * q) : 4;  // 4, or 2 for the last chunk
    const uint32_t voff = (uint32_t)(256 * q + lane * nq) * 4;
    if (nq == 4)
      bload4(src.kc, voff, soff, &t.w[4 * q]);
    else
      bload2(src.kc, voff, soff, &t.w[4 * q]);
  }
  const uint32_t msoff = __builtin_amdgcn_readfirstlane((uint32_t)pg * (kTile * (D / 32) * 4));
  const uint32_t mvoff = (uint32_t)lane * (D / 32) * 4;
  if constexpr (D == 128)
    bload4(src.km, mvoff, msoff, t.m);
  else
    bload2(src.km, mvoff, msoff, t.m);
}

// Value tile of the lane (g4, n) = (lane / 16, lane % 16): its NB/2 code streams (each 32
// codes of b bits, b words) are contiguous at word (tile * 64 + lane) * (NB/2) * b, and the
// (s|z) words of its NB channels 16 nb + n for block g4 / 2 at word tile * 2D + (g4 / 2) D +
// n NB. Both are read with 16-byte loads (8-byte ones where the count is not a multiple of 4).
template <int D, int VB>
__device__ __forceinline__ void load_v(VTile<D, VB>& t, const BodySrc& src, int tile, int lane) {
  constexpr int NB = D / 16, NW = (NB / 2) * VB;
  const int pg = body_page(src.pages, src.n_pages, tile);
  const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)pg * (2 * D * VB * 4));
  const uint32_t voff = (uint32_t)lane * NW * 4;
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int x = 0; x < NW; x += 4) bload4(src.vc, voff + 4 * x, soff, &t.w[x]);
  } else {
#pragma unroll
    for (int x = 0; x < NW; x += 2) bload2(src.vc, voff + 4 * x, soff, &t.w[x]);
  }
  const uint32_t msoff = __builtin_amdgcn_readfirstlane((uint32_t)pg * (2 * D * 4));
  const uint32_t mvoff = (uint32_t)((lane >> 5) * D + (lane & 15) * NB) * 4;
#pragma unroll
  for (int x = 0; x < NB; x += 4) bload4(src.vm, mvoff + 4 * x, msoff, &t.m[x]);
}

// Scores (log2 units) of the lane's token for the 4 query slots.
// Unscaled: the score of query i is kscale * t1[i].
template <int D, int KB>
__device__ __forceinline__ void key_phase_raw(const Smem<D>& sm, int wave, const KTile<D, KB>& t, int lane,
                                              float (&t1)[kMaxG]) {
  const int qi = lane & 3;
  constexpr int NG = D / 32;
  // the groups' MFMA chains are interleaved so that no MFMA waits for the one before it
  float4_t acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const u32x2 a = *reinterpret_cast<const u32x2*>(&sm.qA[wave][qi][(g * 8 + s) * 2]);
      acc[g] = mfma_f16(a, unpack_step<KB>(t.w, g * KB, s), acc[g]);
    }
  // sum_g z_g sum(q)_g 2^(Eq - 24 + kZShift) on the same MFMA (A = the rows' group sums as
  // fp16 hi + lo, B = the token's four fp16 zeros: exact products), scaled back by 2^-kZShift,
  // then sum_g s_g acc_g on top with the fp16 scales straight into mixed-precision FMAs
  const u32x2 zb = u32x2{__builtin_amdgcn_perm(t.m[1], t.m[0], 0x07060302u),
                         NG == 4 ? __builtin_amdgcn_perm(t.m[3], t.m[2], 0x07060302u) : 0u};
  float4_t tz = mfma_f16(*reinterpret_cast<const u32x2*>(&sm.qz[wave][0][qi][0]), zb, float4_t{0.0f, 0.0f, 0.0f, 0.0f});
  tz = mfma_f16(*reinterpret_cast<const u32x2*>(&sm.qz[wave][1][qi][0]), zb, tz);
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) t1[i] = tz[i] * (1.0f / (float)(1 << kZShift));
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float sg = h2f(t.m[g] & 0xFFFFu);
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) t1[i] = __builtin_fmaf(sg, acc[g][i], t1[i]);
  }
}
template <int D, int KB>
__device__ __forceinline__ void key_phase(const Smem<D>& sm, int wave, const KTile<D, KB>& t, int lane, float kscale,
                                          float (&sc)[kMaxG]) {
  float t1[kMaxG];
  key_phase_raw<D, KB>(sm, wave, t, lane, t1);
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) sc[i] = kscale * t1[i];
}

// P.V of one packed tile on the 16x16x32 MFMA. Rows m = (block, query pair, query bit, hi/lo)
// = 8 blk + 4 qp + 2 qb + hl for query i = 2 qp + qb; the 32 K of a step are 16 tokens of each
// block (tokens 16 kk + 0..15), the A row of a block reading zeros for the other block's
// tokens; columns are 16 channels. Two steps (kk) give D[m][n] = sum over the block's 32
// tokens; the weight sums come from the same A with the constant operand. Lane (g4, n) then
// holds the hi and lo rows of queries 2 (g4 % 2) + 0, 1 of block g4 / 2 for channel 16 nb + n:
// it adds each pair and applies that block's scale and zero. nblk: valid 32-token blocks (1
// or 2).
template <int D, int VB, bool FULL = false>
__device__ __forceinline__ void value_phase(const Smem<D>& sm, int wave, const VTile<D, VB>& t, int lane, int nblk,
                                            WaveState<D>& st) {
  constexpr int NB = D / 16;
  constexpr float kV = (float)(1 << (24 - kEp));   // code products carry 2^(kEp - 24)
  constexpr float kV1 = (float)(1 << (14 - kEp));  // weight sums carry 2^(kEp - 14)
  const int m = lane & 15, g4 = lane >> 4;
  const uint16_t* asrc = (m >> 3) == (g4 >> 1) ? &sm.pv[wave][m >> 3][m & 1][(m >> 1) & 3][8 * (g4 & 1)] : sm.zero16;
  const u32x4 a0 = *reinterpret_cast<const u32x4*>(asrc);
  const u32x4 a1 = *reinterpret_cast<const u32x4*>(asrc + 16);
  float4_t d1 = mfma_f16_k32(a0, ones_chunk<VB>(0), float4_t{0.0f, 0.0f, 0.0f, 0.0f});
  d1 = mfma_f16_k32(a1, ones_chunk<VB>(1), d1);
  // the body accumulators hold sum s D + z D1 2^-10 and sum D1; the code products carry
  // 2^(kEp - 24) and the weight sums 2^(kEp - 14), so ob * kV and lb * kV1 are the sums
  const float w0 = d1[0] + d1[1], w1 = d1[2] + d1[3];  // the lane's two queries, hi + lo
  const float w0s = w0 * (kV1 / kV), w1s = w1 * (kV1 / kV);
  const bool live = FULL || (g4 >> 1) < nblk;  // the lane's block holds body tokens
  // all MFMAs first (the kk = 1 step of a column block is issued after every kk = 0 one, so no
  // MFMA waits for its accumulator), then the scale and zero of every column block
  float4_t d[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int base = (nb >> 1) * VB, c0 = 2 * (nb & 1);  // stream, chunk of kk = 0
    const u32x2 p0 = unpack_step_v<VB>(t.w, base, 2 * c0), p1 = unpack_step_v<VB>(t.w, base, 2 * c0 + 1);
    d[nb] = mfma_f16_k32(a0, u32x4{p0.x, p0.y, p1.x, p1.y}, float4_t{0.0f, 0.0f, 0.0f, 0.0f});
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int base = (nb >> 1) * VB, c1 = 2 * (nb & 1) + 1;  // chunk of kk = 1
    const u32x2 p2 = unpack_step_v<VB>(t.w, base, 2 * c1), p3 = unpack_step_v<VB>(t.w, base, 2 * c1 + 1);
    d[nb] = mfma_f16_k32(a1, u32x4{p2.x, p2.y, p3.x, p3.y}, d[nb]);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint32_t mw = live ? t.m[nb] : 0u;
    const float sv = h2f(mw & 0xFFFFu), zv = h2f(mw >> 16);
    st.ob[nb][0] = __builtin_fmaf(sv, d[nb][0] + d[nb][1], __builtin_fmaf(zv, w0s, st.ob[nb][0]));
    st.ob[nb][1] = __builtin_fmaf(sv, d[nb][2] + d[nb][3], __builtin_fmaf(zv, w1s, st.ob[nb][1]));
  }
  st.lb[0] += w0;
  st.lb[1] += w1;
}

// Factor of the softmax weight of body token tb (0..31 of its block): 2^(kEp - e) with e the
// exponent of the token's value slot (token u = tb % 8 of its chunk)
template <int VB>
__device__ __forceinline__ float value_pscale(int tb) {
  float f = 1.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if ((tb & 7) == u)
      f = (tb & 16) ? (float)(1 << kEp) / (float)(1 << VSlots<VB>::exp(2 + (u >> 2), u & 3))
                    : (float)(1 << kEp) / (float)(1 << VSlots<VB>::exp(u >> 2, u & 3));
  return f;
}

// ---------------------------------------------------------------------------------------
// 16-bit rows (sink and recent windows; heads kept unquantized)
// ---------------------------------------------------------------------------------------
// q.K^T of 16-bit rows: lane = token, its key row x (D values, 16-byte pieces) in registers
template <int D, bool BF16>
__device__ __forceinline__ void key_phase_16(const Smem<D>& sm, int wave, const uint4 (&x)[D / 8], int lane,
                                             float scale_log2, float (&sc)[kMaxG]) {
  const int qi = lane & 3;
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int v = 0; v < D / 8; ++v) {
    const u32x2 a0 = *reinterpret_cast<const u32x2*>(&sm.qW[wave][qi][4 * v]);
    const u32x2 a1 = *reinterpret_cast<const u32x2*>(&sm.qW[wave][qi][4 * v + 2]);
    acc = mfma16<BF16>(a0, u32x2{x[v].x, x[v].y}, acc);
    acc = mfma16<BF16>(a1, u32x2{x[v].z, x[v].w}, acc);
  }
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) sc[i] = acc[i] * scale_log2;
}

// Value rows of one 64-token tile of 16-bit rows, both 32-token blocks: for token k the
// lane's D/64 adjacent channels (one dword for D = 128, one 16-bit value for D = 64); tokens
// past n_valid repeat the last valid row (their weights are zero). All loads are issued
// before any is used.
template <int D, class RowOf>
__device__ __forceinline__ void load_v16(uint32_t (&vr)[2][32], int lane, int n_valid, RowOf row_of) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint16_t* r = row_of(min(jj * 32 + k, n_valid - 1));
      if constexpr (D == 128)
        vr[jj][k] = *reinterpret_cast<const uint32_t*>(r + 2 * lane);
      else
        vr[jj][k] = r[lane];
    }
}

// fp16/bf16 pair (channel NH*lane + h of token a, same channel of token b)
template <int H>
__device__ __forceinline__ uint32_t pair16(uint32_t a, uint32_t b) {
  return H == 0 ? __builtin_amdgcn_perm(b, a, 0x05040100u) : __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// lane = channel; P.V of one tile of 16-bit rows from the operands load_v16 fetched
template <int D, bool BF16>
__device__ __forceinline__ void value_phase_16(const Smem<D>& sm, int wave, int lane, int n_valid,
                                               const uint32_t (&vr)[2][32], WaveState<D>& st) {
  const int qi = lane & 3;
  const uint32_t one1 = BF16 ? 0x3F80u : 0x3C00u;
  const u32x2 one = u32x2{one1 | (one1 << 16), one1 | (one1 << 16)};
  float4_t acc[D / 64], acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int h = 0; h < D / 64; ++h) acc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    if (jj * 32 < n_valid) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x2 ahi = *reinterpret_cast<const u32x2*>(&sm.pw[wave][0][qi][16 * jj + 2 * s]);
        const u32x2 alo = *reinterpret_cast<const u32x2*>(&sm.pw[wave][1][qi][16 * jj + 2 * s]);
        const uint32_t* r = &vr[jj][4 * s];
        const u32x2 b0 = u32x2{pair16<0>(r[0], r[1]), pair16<0>(r[2], r[3])};
        acc[0] = mfma16<BF16>(ahi, b0, acc[0]);
        acc[0] = mfma16<BF16>(alo, b0, acc[0]);
        if constexpr (D == 128) {
          const u32x2 b1 = u32x2{pair16<1>(r[0], r[1]), pair16<1>(r[2], r[3])};
          acc[1] = mfma16<BF16>(ahi, b1, acc[1]);
          acc[1] = mfma16<BF16>(alo, b1, acc[1]);
        }
        acc1 = mfma16<BF16>(ahi, one, acc1);
        acc1 = mfma16<BF16>(alo, one, acc1);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < D / 64; ++h)
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) st.o[i][h] += acc[h][i];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) st.l[i] += acc1[i];
}

// ---------------------------------------------------------------------------------------
// Tile loops
// ---------------------------------------------------------------------------------------

// One 64-token tile of 16-bit rows: for every token, the lane's value channel(s) (loaded
// ahead, possibly before the query prologue); the key rows are loaded when it is computed.
template <int D>
struct Rows16 {
  uint32_t v[2][32];
};
template <int D, class VRowOf>
__device__ __forceinline__ void rows16_issue(Rows16<D>& r, int base, int n_tok, int lane, VRowOf vrow) {
  load_v16<D>(r.v, lane, min(kTile, n_tok - base), [&](int k) { return vrow(base + k); });
}
template <int D, class KRowOf>
__device__ __forceinline__ void rows16_compute(Smem<D>& sm, const DecodePlan& p, const Rows16<D>& r, int base,
                                               int n_tok, int lane, int wave, WaveState<D>& st, KRowOf krow) {
  const int u = base + lane;
  const bool valid = u < n_tok;
  const int n_valid = min(kTile, n_tok - base);
  uint4 x[D / 8];  // the lane's key row, all loads in flight together
  const uint4* r4 = reinterpret_cast<const uint4*>(krow(valid ? u : base));
#pragma unroll
  for (int v = 0; v < D / 8; ++v) x[v] = r4[v];
  issue_barrier();
  float sc[kMaxG];
  if (p.dtype == KVQ_BF16) {
    key_phase_16<D, true>(sm, wave, x, lane, p.scale_log2, sc);
    softmax_rows16<D>(sm, wave, lane, valid, sc, st, lane & 31, 1.0f, true);
    value_phase_16<D, true>(sm, wave, lane, n_valid, r.v, st);
  } else {
    key_phase_16<D, false>(sm, wave, x, lane, p.scale_log2, sc);
    softmax_rows16<D>(sm, wave, lane, valid, sc, st, lane & 31, 1.0f, false);
    value_phase_16<D, false>(sm, wave, lane, n_valid, r.v, st);
  }
  wave_lds_sync();
}
// One window unit: kWinTile = 16 tokens of 16-bit rows, all of its loads in 32 registers.
// Keys are read cooperatively (lane (t, j): token t = lane % 16, channels 32 s + 8 j .. +7 of
// step s), which is the B operand of a 16x16x32 MFMA whose rows 0..3 are the queries; values
// are whole rows, lane = channel pair (D = 128) or channel (D = 64), as for 16-bit tiles.
// Token geometry of one row: its length, quantized body, live sink and window tokens, the
// ring's oldest slot, and how its body tiles and window units are dealt out. Uniform rows
// take it from the plan; ragged rows derive it from their length by the host's rules (the
// body is every whole 32-token block that has left the window of n_recent..n_recent + 31).
struct RowGeom {
  int T, body, nsl, n_win, ring0, n_tiles, n_wtiles, tps;
};
__device__ __forceinline__ RowGeom row_geom(const DecodePlan& p, int b) {
  if (!p.ragged)
    return RowGeom{p.T, p.body, p.n_sink_live, p.n_win, p.ring0, p.n_tiles, p.n_wtiles, p.tiles_per_split};
  RowGeom g;
  g.T = p.row_len[b];
  const int n_recent = p.ring - kGroup;
  const int r = g.T - p.n_sink_cfg - n_recent;
  g.body = r <= 0 ? 0 : (r / kGroup) * kGroup;
  g.nsl = min(g.T, p.n_sink_cfg);
  g.n_win = g.T - g.nsl - g.body;
  g.ring0 = g.body % p.ring;
  g.n_tiles = (g.body + kTile - 1) / kTile;
  g.n_wtiles = (g.nsl + g.n_win + kWinTile - 1) / kWinTile;
  g.tps = (g.n_tiles + p.n_splits - 1) / p.n_splits;
  return g;
}

template <int D>
struct WinUnit {
  u32x4 k[D / 32];
  uint32_t v[kWinTile];
};
template <int D, class KRowOf, class VRowOf>
__device__ __forceinline__ void win_issue(WinUnit<D>& w, int base, int n_valid, int lane, KRowOf krow, VRowOf vrow) {
  static_assert(kWinTile == 16, "window units are 16 tokens (one MFMA column block)");
  const uint16_t* kr = krow(base + min(lane & 15, n_valid - 1)) + 8 * (lane >> 4);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) w.k[s] = *reinterpret_cast<const u32x4*>(kr + 32 * s);
#pragma unroll
  for (int k = 0; k < kWinTile; ++k) {
    const uint16_t* r = vrow(base + min(k, n_valid - 1));
    if constexpr (D == 128)
      w.v[k] = *reinterpret_cast<const uint32_t*>(r + 2 * lane);
    else
      w.v[k] = r[lane];
  }
}
template <int D, bool BF16>
__device__ __forceinline__ void win_compute_t(Smem<D>& sm, const DecodePlan& p, const RowGeom& g, const WinUnit<D>& w,
                                              int u0, int n_valid, int lane, int wave, WaveState<D>& st) {
  // scores: lane t < 16 ends with q_i . k_t for the queries i = 0..3 of rows 0..3
  const int i = lane & 15, j = lane >> 4;
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const u32x4 a = i < kMaxG ? *reinterpret_cast<const u32x4*>(&sm.qW[wave][i][16 * s + 4 * j]) : u32x4{0u, 0u, 0u, 0u};
    acc = mfma_k32<BF16>(a, w.k[s], acc);
  }
  float sc[kMaxG];
#pragma unroll
  for (int r = 0; r < kMaxG; ++r) sc[r] = acc[r] * p.scale_log2;
  if (p.Q > 1) {
    // several query tokens: row r (query token r / G, the (T - Q + r / G)-th token) sees no
    // later token. Window token u sits at position u (sink) or u + body (recent ring). A
    // masked score is a huge finite negative rather than -inf: a wavefront whose first unit
    // is all masked for a row then keeps a finite running max, and the masked terms vanish
    // (weight 2^(-1e30 - m) = 0) once a visible token, which every row has, sets the max.
    const int u = u0 + (lane & 15);
    const int pos = u < g.nsl ? u : u + g.body;
#pragma unroll
    for (int r = 0; r < kMaxG; ++r)
      if (pos > g.T - p.Q + r / p.G) sc[r] = kMaskedScore;
  }
  softmax_rows16<D>(sm, wave, lane, lane < n_valid, sc, st, lane & 31, 1.0f, BF16);
  // P.V over the unit's 16 rows: 4 steps of 4 tokens on the 4x4x4 MFMA (lane = channel)
  const int qi = lane & 3;
  const uint32_t one1 = BF16 ? 0x3F80u : 0x3C00u;
  const u32x2 one = u32x2{one1 | (one1 << 16), one1 | (one1 << 16)};
  float4_t o[D / 64], l1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int h = 0; h < D / 64; ++h) o[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < kWinTile / 4; ++s) {
    const u32x2 ahi = *reinterpret_cast<const u32x2*>(&sm.pw[wave][0][qi][2 * s]);
    const u32x2 alo = *reinterpret_cast<const u32x2*>(&sm.pw[wave][1][qi][2 * s]);
    const uint32_t* r = &w.v[4 * s];
    const u32x2 b0 = u32x2{pair16<0>(r[0], r[1]), pair16<0>(r[2], r[3])};
    o[0] = mfma16<BF16>(ahi, b0, o[0]);
    o[0] = mfma16<BF16>(alo, b0, o[0]);
    if constexpr (D == 128) {
      const u32x2 b1 = u32x2{pair16<1>(r[0], r[1]), pair16<1>(r[2], r[3])};
      o[1] = mfma16<BF16>(ahi, b1, o[1]);
      o[1] = mfma16<BF16>(alo, b1, o[1]);
    }
    l1 = mfma16<BF16>(ahi, one, l1);
    l1 = mfma16<BF16>(alo, one, l1);
  }
#pragma unroll
  for (int h = 0; h < D / 64; ++h)
#pragma unroll
    for (int r = 0; r < kMaxG; ++r) st.o[r][h] += o[h][r];
#pragma unroll
  for (int r = 0; r < kMaxG; ++r) st.l[r] += l1[r];
  wave_lds_sync();
}
template <int D>
__device__ __forceinline__ void win_compute(Smem<D>& sm, const DecodePlan& p, const RowGeom& g, const WinUnit<D>& w,
                                            int u0, int n_valid, int lane, int wave, WaveState<D>& st) {
  if (p.dtype == KVQ_BF16)
    win_compute_t<D, true>(sm, p, g, w, u0, n_valid, lane, wave, st);
  else
    win_compute_t<D, false>(sm, p, g, w, u0, n_valid, lane, wave, st);
}

// Quantized keys and values, both widths fixed: the loads of the next tile are issued before
// the current tile is computed.
template <int D, int KB, int VB, bool PAGED, class Prologue, class WindowIssue, class Window>
__device__ __forceinline__ void body_loop(Smem<D>& sm, const DecodePlan& p, const uint64_t* off, int b, int body,
                                          int t0, int t1, int lane, int wave, Prologue prologue,
                                          WindowIssue window_issue, Window window, WaveState<D>& st) {
  // paged caches: lane i holds the page of this wavefront's tile number pbase + i (loaded 64 at
  // a time), and each tile's page is read out of that register, so the loads of the next tile
  // never wait for a page-table lookup. src then carries no table: load_k / load_v take the
  // page as the tile slot.
  const BodySrc src = body_src(p, off, false, b);
  const int32_t* row_pages = PAGED ? p.pages + (size_t)b * p.page_stride : nullptr;
  int pv = 0, pbase = -kWavePages;
  auto page_of = [&](int t) -> int {
    if constexpr (!PAGED) {
      return t;
    } else {
      const int k = (t - t0 - wave) / kWaves;  // the wavefront's k-th tile
      if (k - pbase >= kWavePages) {
        pbase = k;
        const int tl = t0 + wave + (pbase + lane) * kWaves;
        pv = tl < t1 ? body_page(row_pages, p.n_pages, tl) : 0;
      }
      return __builtin_amdgcn_readlane(pv, k - pbase);
    }
  };
  int tile = t0 + wave;
  const bool any = tile < t1;
  // Two register buffers, each always in the same registers: a buffer is refilled while the
  // other one is computed. The wavefront's first tile is in flight before the query prologue
  // runs, the second one from its end (a smaller flood ahead of the query loads lets them
  // return sooner). Every fetch is issued, so the compiler's load counts stay fixed and no
  // wait covers a load still needed in flight; a fetch past the wavefront's last tile goes
  // through zero-length descriptors and reads nothing.
  const BodySrc nul = body_src_empty(p, off);
  KTile<D, KB> kt[2];
  VTile<D, VB> vt[2];
  auto fetch = [&](KTile<D, KB>& kd, VTile<D, VB>& vd, int t) {
    const bool live = t < t1;
    const BodySrc& s = live ? src : nul;
    const int pg = page_of(live ? t : t0 + wave);
    load_k<D, KB>(kd, s, pg, lane);
    load_v<D, VB>(vd, s, pg, lane);
  };
  WinUnit<D> wt;
  window_issue(wt);
  fetch(kt[0], vt[0], tile);
  issue_barrier();
  const int Eq = prologue();
  fetch(kt[1], vt[1], tile + kWaves);
  issue_barrier();
  build_key_operand<D, KB>(sm, wave, lane, Eq);
  const float kscale = __builtin_ldexpf(p.scale_log2, 24 - Eq);
  window(wt);
  if (!any) return;
  const float pscl = value_pscale<VB>(lane & 31);
  // this workgroup's tiles below tfull hold 64 body tokens; only the row's last tile can hold
  // 32, and it is then the last tile of its wavefront: only that step masks tokens and blocks
  const int tfull = min(t1, body / kTile);
  auto step = [&](auto full, const KTile<D, KB>& kcur, const VTile<D, VB>& vcur) {
    constexpr bool FULL = decltype(full)::value;
    float kraw[kMaxG];
    key_phase_raw<D, KB>(sm, wave, kcur, lane, kraw);
    softmax_body_rel<D, FULL>(sm, wave, lane, FULL || tile * kTile + lane < body, kraw, kscale, st, pscl);
    value_phase<D, VB, FULL>(sm, wave, vcur, lane, FULL ? 2 : min(2, (body - tile * kTile) / 32), st);
    wave_lds_sync();
    tile += kWaves;
  };
  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;
  // the loop runs the full tiles; a partial tile (the wavefront's last) is computed after it,
  // from the buffer that then holds it (in1)
  bool in1 = false;
  if (tile < tfull) {
    step(Full{}, kt[0], vt[0]);
    in1 = true;
    while (tile < tfull) {
      fetch(kt[0], vt[0], tile + kWaves);  // buffer 0 is free: the tile after this one
      issue_barrier();
      step(Full{}, kt[1], vt[1]);
      in1 = false;
      if (tile >= tfull) break;
      fetch(kt[1], vt[1], tile + kWaves);
      issue_barrier();
      step(Full{}, kt[0], vt[0]);
      in1 = true;
    }
  }
  if (tile < t1) {
    if (in1)
      step(Part{}, kt[1], vt[1]);
    else
      step(Part{}, kt[0], vt[0]);
  }
}

template <int D, int KB>
__device__ __forceinline__ void key_tile_q(const Smem<D>& sm, int wave, const BodySrc& src, int tile, int lane,
                                           float kscale, float (&sc)[kMaxG]) {
  KTile<D, KB> t;
  load_k<D, KB>(t, src, tile, lane);
  key_phase<D, KB>(sm, wave, t, lane, kscale, sc);
}

template <int D, int VB>
__device__ __forceinline__ void value_tile_q(Smem<D>& sm, int wave, const BodySrc& src, int tile,
                                             int lane, bool valid, const float (&sc)[kMaxG], int nblk, WaveState<D>& st) {
  softmax_body<D>(sm, wave, lane, valid, sc, st, value_pscale<VB>(lane & 31));
  VTile<D, VB> t;
  load_v<D, VB>(t, src, tile, lane);
  value_phase<D, VB>(sm, wave, t, lane, nblk, st);
}

// Body tiles of heads with a 16-bit key or value side (one phase 16-bit, the other packed
// or 16-bit); no prefetch.
template <int D>
__device__ __forceinline__ void mixed_body_loop(Smem<D>& sm, const DecodePlan& p, const uint64_t* off, int b, int h,
                                                int body, int t0, int t1, int lane, int wave, float kscale,
                                                WaveState<D>& st) {
  const int kb = head_bits(p.k_bits, h), vb = head_bits(p.v_bits, h);
  const bool bf16 = p.dtype == KVQ_BF16;
  const uint16_t* kr = reinterpret_cast<const uint16_t*>(p.blob + off[KC]);
  const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.blob + off[VC]);
  const BodySrc src = body_src(p, off, true, b);
  for (int tile = t0 + wave; tile < t1; tile += kWaves) {
    const int tok = tile * kTile + lane;
    const bool valid = tok < body;
    const int n_valid = min(kTile, body - tile * kTile);
    const int pg = body_page(src.pages, src.n_pages, tile);
    float sc[kMaxG];
    switch (kb) {
      case 2: key_tile_q<D, 2>(sm, wave, src, tile, lane, kscale, sc); break;
      case 3: key_tile_q<D, 3>(sm, wave, src, tile, lane, kscale, sc); break;
      case 4: key_tile_q<D, 4>(sm, wave, src, tile, lane, kscale, sc); break;
      case 5: key_tile_q<D, 5>(sm, wave, src, tile, lane, kscale, sc); break;
      case 6: key_tile_q<D, 6>(sm, wave, src, tile, lane, kscale, sc); break;
      case 7: key_tile_q<D, 7>(sm, wave, src, tile, lane, kscale, sc); break;
      case 8: key_tile_q<D, 8>(sm, wave, src, tile, lane, kscale, sc); break;
      default:
        uint4 x[D / 8];
        const uint4* r4 = reinterpret_cast<const uint4*>(kr + ((size_t)pg * kTile + (valid ? lane : 0)) * D);
#pragma unroll
        for (int v = 0; v < D / 8; ++v) x[v] = r4[v];
        issue_barrier();
        if (bf16)
          key_phase_16<D, true>(sm, wave, x, lane, p.scale_log2, sc);
        else
          key_phase_16<D, false>(sm, wave, x, lane, p.scale_log2, sc);
        break;
    }
    const int nblk = n_valid / 32;
    switch (vb) {
      case 2: value_tile_q<D, 2>(sm, wave, src, tile, lane, valid, sc, nblk, st); break;
      case 3: value_tile_q<D, 3>(sm, wave, src, tile, lane, valid, sc, nblk, st); break;
      case 4: value_tile_q<D, 4>(sm, wave, src, tile, lane, valid, sc, nblk, st); break;
      case 5: value_tile_q<D, 5>(sm, wave, src, tile, lane, valid, sc, nblk, st); break;
      case 6: value_tile_q<D, 6>(sm, wave, src, tile, lane, valid, sc, nblk, st); break;
      case 7: value_tile_q<D, 7>(sm, wave, src, tile, lane, valid, sc, nblk, st); break;
      case 8: value_tile_q<D, 8>(sm, wave, src, tile, lane, valid, sc, nblk, st); break;
      default: {
        uint32_t rows[2][32];
        load_v16<D>(rows, lane, n_valid, [&](int k) { return vr + ((size_t)pg * kTile + k) * D; });
        softmax_rows16<D>(sm, wave, lane, valid, sc, st, lane & 31, 1.0f, bf16);
        if (bf16)
          value_phase_16<D, true>(sm, wave, lane, n_valid, rows, st);
        else
          value_phase_16<D, false>(sm, wave, lane, n_valid, rows, st);
        break;
      }
    }
    wave_lds_sync();
  }
}

// 16-bit rows for tokens [first, n_tok) in 64-token tiles, round-robin over the wavefronts.
template <int D, class KRowOf, class VRowOf>
__device__ __forceinline__ void rows16_loop(Smem<D>& sm, const DecodePlan& p, int first, int n_tok, int lane, int wave,
                                            WaveState<D>& st, KRowOf krow, VRowOf vrow) {
  for (int base = first + wave * kTile; base < n_tok; base += kWaves * kTile) {
    Rows16<D> r;
    rows16_issue<D>(r, base, n_tok, lane, vrow);
    rows16_compute<D>(sm, p, r, base, n_tok, lane, wave, st, krow);
  }
}

// ---------------------------------------------------------------------------------------
// Kernel
// ---------------------------------------------------------------------------------------
// WIDE: the instantiation that also holds the path for 5- to 8-bit codes and heads with one
// 16-bit side. Its register pressure would make the compiler spill in the fast loops, so
// caches whose heads all take the fast path (or are 16-bit on both sides) use the other one.
// PAGED: the instantiation for paged caches (the page lookups cost the contiguous fast loop
// registers and time, so contiguous caches use one without them; WIDE always looks them up).
template <int D, bool WIDE, bool PAGED>
// two wavefronts per SIMD (two workgroups per CU): the register budget is 256
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(const DecodePlan p) {
  __shared__ Smem<D> sm;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int R = G * p.Q;  // query rows of this KV head: row r is query token r / G of query head h G + r % G
  const int kb = head_bits(p.k_bits, h), vb = head_bits(p.v_bits, h);
  // global query row of row r: [B][Q][Hq] order
  auto grow = [&](int r) { return ((size_t)b * p.Q + r / G) * p.Hq + (size_t)h * G + r % G; };
  const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q);

  // ---- q operands, built by every wavefront for itself in its LDS slice: the raw 16-bit
  // copy, the per-group sums of q, and the fp16 key operand in slot order with q scaled by
  // 2^Eq so that max|q| * 2^Eq lies in [2^14, 2^15) (q means q * n for the packed keys of a
  // cache with key normalization). The query loads are issued first, before the region
  // table is read; the body and window loads follow as soon as the table is in. No barrier
  // stands between a wavefront's start and its first tile.
  constexpr int E = kMaxG * D / 64;  // consecutive query elements per lane (8 or 4): one 16- or 8-byte load
  const int i0 = (lane * E) / D, c0 = (lane * E) % D;
  // (rows past R read row R - 1 and are zeroed: no lane skips the load, so the compiler's
  // count of loads in flight stays exact)
  // Only loads are issued here; their values are first used in the prologue, after the window
  // and body loads, so no wait for them stands in front of those.
  const bool q_live = i0 < R;
  uint32_t qw[E / 2];  // the lane's E 16-bit query elements, two to a word
  {
    const uint16_t* src = q + grow(q_live ? i0 : R - 1) * D + c0;
    if constexpr (E == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      qw[0] = v.x; qw[1] = v.y; qw[2] = v.z; qw[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      qw[0] = v.x; qw[1] = v.y;
    }
  }
  // the region table of this (row, head), read once into scalar registers ahead of anything
  // the compiler must treat as a possible store
  const uint64_t* tab = p.off + ((size_t)b * p.H + h) * kRegions;
  uint64_t off[kRegions];
#pragma unroll
  for (int r = 0; r < kRegions; ++r) off[r] = tab[r];
  // per-channel key norms (caches with key normalization, packed key heads): the packed keys
  // hold k / n, so the packed-key operand is built from q * n
  // (only caches with norms load them: these loads are issued behind the region table, with
  // the body loads' flood, and the prologue would wait for them)
  const bool use_norm = p.key_norm && kb != 16;
  float knraw[E];
#pragma unroll
  for (int e = 0; e < E; ++e) knraw[e] = 1.0f;
  if (use_norm) {
    const float* kn = reinterpret_cast<const float*>(p.blob + off[KN]) + c0;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(kn + e);
      knraw[e] = v.x; knraw[e + 1] = v.y; knraw[e + 2] = v.z; knraw[e + 3] = v.w;
    }
  }
  issue_barrier();
  // Returns Eq; the caller builds the key operand for its width (build_key_operand) and scores
  // with the factor scale_log2 * 2^(24 - Eq). Every wavefront calls it once.
  auto prologue = [&]() -> int {
    float qmax = 0.0f, qs = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t qh = q_live ? (qw[e / 2] >> (16 * (e & 1))) & 0xFFFFu : 0u;
      reinterpret_cast<uint16_t*>(sm.qW[wave][i0])[c0 + e] = (uint16_t)qh;
      const float v = widen(qh, p.dtype) * knraw[e];
      sm.qn[wave][i0][c0 + e] = v;
      qmax = fmaxf(qmax, fabsf(v));
      qs += v;
    }
    // a 32-channel group spans 32 / E aligned lanes
#pragma unroll
    for (int o2 = 16 / E; o2 >= 1; o2 >>= 1) qs += __shfl_xor(qs, o2, 64);
    if (lane < 32) sm.zero16[lane] = 0;
    qmax = wave_max(qmax);
    int qe = 0;
    if (qmax > 0.0f) (void)frexpf(qmax, &qe);
    const int Eq = 15 - qe;
    // the key zero-term operand: |sum of q| * 2^Eq <= 2^20, so the value is at most 2^8
    if (c0 % 32 == 0) {
      const float v = __builtin_ldexpf(qs, Eq - 24 + kZShift);
      const uint32_t hi = f2h(v);
      sm.qz[wave][0][i0][c0 / 32] = (uint16_t)hi;
      sm.qz[wave][1][i0][c0 / 32] = (uint16_t)f2h(v - h2f(hi));
      if constexpr (D / 32 < 4) {
        sm.qz[wave][0][i0][c0 / 32 + 2] = 0;
        sm.qz[wave][1][i0][c0 / 32 + 2] = 0;
      }
    }
    wave_lds_sync();
    return Eq;
  };

  WaveState<D> st;
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    st.m[i] = -INFINITY;
    st.l[i] = 0.0f;
#pragma unroll
    for (int hh = 0; hh < D / 64; ++hh) st.o[i][hh] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    st.lb[k] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.ob[nb][k] = 0.0f;
  }

  // ---- this workgroup's work: body tiles [t0, t1) round-robin over the wavefronts, and the
  // window units w = split + n_splits * k (k = 0, 1, ...) of kWinTile tokens, unit k going to
  // wavefront kWaves - 1 - k % kWaves (the last wavefronts have the fewest body tiles). Small
  // units spread the 16-bit window over many wavefronts instead of loading a few of them
  // with several body tiles' worth of bytes. A wavefront's first window unit is loaded
  // before the query prologue, so its latency is hidden.
  const RowGeom g = row_geom(p, b);
  const int body = g.body;
  const int t0 = split * g.tps, t1 = min(g.n_tiles, t0 + g.tps);
  const int n_wtok = g.nsl + g.n_win;
  const int w_first = split + p.n_splits * (kWaves - 1 - wave);  // k = kWaves - 1 - wave
  const uint16_t* sk = reinterpret_cast<const uint16_t*>(p.blob + off[SK]);
  const uint16_t* sv = reinterpret_cast<const uint16_t*>(p.blob + off[SV]);
  const uint16_t* rk = reinterpret_cast<const uint16_t*>(p.blob + off[RK]);
  const uint16_t* rv = reinterpret_cast<const uint16_t*>(p.blob + off[RV]);
  // window token u < n_sink_live is sink row u, else ring slot (ring0 + u - n_sink_live) mod
  // ring, ring0 = body mod ring (the ring's oldest live slot)
  const int nsl = g.nsl, ring0 = g.ring0, ring = p.ring;
  auto slot = [=](int u) {
    const int r = ring0 + (u - nsl);
    return r >= ring ? r - ring : r;
  };
  auto krow = [=](int u) { return u < nsl ? sk + (size_t)u * D : rk + (size_t)slot(u) * D; };
  auto vrow = [=](int u) { return u < nsl ? sv + (size_t)u * D : rv + (size_t)slot(u) * D; };
  const bool has_w = w_first < g.n_wtiles;
  auto wlim = [=](int w) { return min(n_wtok, (w + 1) * kWinTile); };  // end of window unit w
  // issue the value loads of the first window tile (before the prologue); compute the window
  auto window_issue = [&](WinUnit<D>& wt) {
    if (has_w) win_issue<D>(wt, w_first * kWinTile, wlim(w_first) - w_first * kWinTile, lane, krow, vrow);
  };
  auto window = [&](const WinUnit<D>& wt) {
    if (!has_w) return;
    win_compute<D>(sm, p, g, wt, w_first * kWinTile, wlim(w_first) - w_first * kWinTile, lane, wave, st);
    for (int w = w_first + kWaves * p.n_splits; w < g.n_wtiles; w += kWaves * p.n_splits) {
      WinUnit<D> r;
      win_issue<D>(r, w * kWinTile, wlim(w) - w * kWinTile, lane, krow, vrow);
      win_compute<D>(sm, p, g, r, w * kWinTile, wlim(w) - w * kWinTile, lane, wave, st);
    }
  };

  if (kb == 16 && vb == 16) {
    WinUnit<D> wt;
    window_issue(wt);
    (void)prologue();
    window(wt);
    const uint16_t* kr = reinterpret_cast<const uint16_t*>(p.blob + off[KC]);
    const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.blob + off[VC]);
    const int32_t* pages = p.pages ? p.pages + (size_t)b * p.page_stride : nullptr;
    rows16_loop<D>(sm, p, t0 * kTile, min(body, t1 * kTile), lane, wave, st,
                   [&](int u) { return kr + (size_t)body_row(pages, p.n_pages, u) * D; },
                   [&](int u) { return vr + (size_t)body_row(pages, p.n_pages, u) * D; });
  } else if (kb <= 4 && vb <= 4) {
    // the widths the allocator hands out in {2,3,4}: prefetching loop per combination
#define KVQ_BODY(KB_, VB_) \
  case KB_ * 16 + VB_: body_loop<D, KB_, VB_, PAGED>(sm, p, off, b, body, t0, t1, lane, wave, prologue, window_issue, window, st); break;
    switch (kb * 16 + vb) {
      KVQ_BODY(2, 2) KVQ_BODY(2, 3) KVQ_BODY(2, 4) KVQ_BODY(3, 2) KVQ_BODY(3, 3) KVQ_BODY(3, 4)
      KVQ_BODY(4, 2) KVQ_BODY(4, 3) KVQ_BODY(4, 4)
      default: (void)prologue(); break;
    }
#undef KVQ_BODY
  } else if constexpr (WIDE) {
    // wider codes or a 16-bit side: one phase at a time
    WinUnit<D> wt;
    window_issue(wt);
    const int Eq = prologue();
    build_key_operand_rt<D>(sm, wave, lane, Eq, kb);
    const float kscale = __builtin_ldexpf(p.scale_log2, 24 - Eq);
    window(wt);
    mixed_body_loop<D>(sm, p, off, b, h, body, t0, t1, lane, wave, kscale, st);
  } else {
    (void)prologue();  // not reached: the host launches the WIDE instantiation for such heads
  }

  // ---- combine the wavefronts of this workgroup into one partial (m, l, o). The packed-body
  // sums of the two blocks' lanes are added with one lane swap (sum_halves), after which lane
  // (r, n) holds query qr of channels 16 nb + n; the 16-bit-row sums (lane = channel pair) are
  // added on top in LDS by the wavefronts that have any.
  const int r4 = lane >> 4, n16 = lane & 15;
  const int qr = ((r4 & 1) << 1) | (r4 >> 1);
  const float lbr = sum_halves(st.lb[0], st.lb[1]);
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    const float v = sum_halves(st.ob[nb][0], st.ob[nb][1]);
    sm.red_o[wave][qr][16 * nb + n16] = v * (float)(1 << (24 - kEp));
  }
  if (n16 == 0) {
    const float mq = qr == 0 ? st.m[0] : qr == 1 ? st.m[1] : qr == 2 ? st.m[2] : st.m[3];
    const float lq = qr == 0 ? st.l[0] : qr == 1 ? st.l[1] : qr == 2 ? st.l[2] : st.l[3];
    sm.red_m[wave][qr] = mq;
    sm.red_l[wave][qr] = __builtin_fmaf(lbr, (float)(1 << (14 - kEp)), lq);
  }
  if (has_w || !(kb <= 4 && vb <= 4)) {  // 16-bit rows seen: st.o holds sums
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < kMaxG; ++i)
#pragma unroll
      for (int hh = 0; hh < D / 64; ++hh) sm.red_o[wave][i][(D / 64) * lane + hh] += st.o[i][hh];
  }
  // fused decode step: the token being appended is not in the cache yet (the merge launch
  // writes it there). The last split adds it as one more softmax term (m = its score, l = 1,
  // o = its value row); wavefront i scores it against query i
  const bool fresh = p.new_k != nullptr && split == p.n_splits - 1;
  const size_t kv_row = ((size_t)b * p.H + h) * D;
  if (fresh && wave < G) {
    const uint16_t* nk = reinterpret_cast<const uint16_t*>(p.new_k) + kv_row;
    float acc = 0.0f;
#pragma unroll
    for (int hh = 0; hh < D / 64; ++hh) {
      const int c = (D / 64) * lane + hh;
      acc = __builtin_fmaf(widen(reinterpret_cast<const uint16_t*>(sm.qW[wave][wave])[c], p.dtype),
                           widen(nk[c], p.dtype), acc);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) sm.new_s[wave] = acc * p.scale_log2;
  }
  if (p.pages && h == 0 && wave == kWaves - 1) {
    // the tiles this workgroup read must be mapped: an unmapped one was read from a clamped
    // page (in bounds, meaningless values) and is reported through the sticky flag, bit 1
    const int32_t* row_pages = p.pages + (size_t)b * p.page_stride;
    bool bad = false;
    for (int t = t0 + lane; t < t1; t += 64) {
      const int pg = row_pages[t];
      bad |= pg < 0 || pg >= p.n_pages;
    }
    if (__ballot(bad) && lane == 0) atomicOr(p.flag, 2u);
  }
  __syncthreads();
  const size_t rows = (size_t)p.B * p.Q * p.Hq;
  for (int idx = tid; idx < R * D; idx += kThreads) {
    const int i = idx / D, c = idx % D;
    float mw[kWaves], ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = sm.red_m[w][i];
      ms = fmaxf(ms, mw[w]);
    }
    const float sn = fresh ? sm.new_s[i] : -INFINITY;
    ms = fmaxf(ms, sn);
    float oo = 0.0f, ll = 0.0f;
    if (ms != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(mw[w] - ms);  // 0 for an empty wavefront (-inf)
        oo = __builtin_fmaf(f, sm.red_o[w][i][c], oo);
        ll = __builtin_fmaf(f, sm.red_l[w][i], ll);
      }
      if (fresh) {
        const float f = __builtin_amdgcn_exp2f(sn - ms);
        oo = __builtin_fmaf(f, widen(reinterpret_cast<const uint16_t*>(p.new_v)[kv_row + c], p.dtype), oo);
        ll += f;
      }
    }
    p.ws_o[((size_t)split * rows + grow(i)) * D + c] = oo;
    if (c == 0) {
      p.ws_ml[((size_t)split * rows + grow(i)) * 2] = ms;
      p.ws_ml[((size_t)split * rows + grow(i)) * 2 + 1] = ll;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Log-sum-exp merge of the n_splits partials (m_j, l_j, o_j) of one output row:
//   out = sum_j 2^(m_j - m*) o_j / sum_j 2^(m_j - m*) l_j,  m* = max_j m_j.
// A separate launch: the kernel boundary makes every partial visible, so no workgroup has
// to write back or invalidate the L2 caches. T lanes per output element, T the smallest power
// of two with T * kMergeChunk >= n_splits, and C the smallest power of two that holds a lane's
// share: each lane loads its (at most C) partials all at once and combines them, and the T
// lane results are combined with lane shuffles, so a launch waits for one round of loads
// whatever the split count.
// ---------------------------------------------------------------------------------------
constexpr int kMergeChunk = 16;

template <int D, int T, int C>
__global__ __launch_bounds__(kThreads) void merge_kernel(const DecodePlan p) {
  const size_t rows = (size_t)p.B * p.Q * p.Hq;
  const size_t gid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (p.new_k != nullptr && gid < (size_t)p.B * p.H * (D / 4)) {
    // fused decode step: the appended token enters its ring slot once every read of the ring
    // by the decode launch is done (one 16-byte piece of its key or value row per thread)
    const size_t bh = gid / (D / 4);
    const int piece = (int)(gid % (D / 4));
    const bool kv = piece >= D / 8;
    const uint4 x = reinterpret_cast<const uint4*>(kv ? p.new_v : p.new_k)[bh * (D / 8) + piece % (D / 8)];
    const uint64_t ring_off = p.off[bh * kRegions + (kv ? RV : RK)];
    uint4* dst = reinterpret_cast<uint4*>(const_cast<char*>(p.blob) + ring_off + (size_t)p.new_slot * D * 2);
    dst[piece % (D / 8)] = x;
  }
  // T adjacent lanes share output element idx; lane `sub` of them combines the partials
  // sub, sub + T, sub + 2T, ... (at most C of them), and the T results are then
  // combined across the lanes, so every partial load of the launch is in flight at once
  const size_t idx = gid / T;
  const int sub = (int)(gid % T);
  if (idx >= rows * D) return;  // all T lanes of an element leave together
  const size_t r = idx / D;
  const int parts = p.n_splits;
  const int mine = parts > sub ? (parts - sub + T - 1) / T : 0;  // partials of this lane
  const float* op = p.ws_o + idx;
  const float* mlp = p.ws_ml + r * 2;
  float mx = -INFINITY, num = 0.0f, den = 0.0f;
  for (int k0 = 0; k0 < mine; k0 += C) {
    float m[C], l[C], o[C];
#pragma unroll
    for (int u = 0; u < C; ++u) {
      const int j = sub + T * min(k0 + u, mine - 1);  // past the end: a repeat, weighted 0 below
      const float2 ml = *reinterpret_cast<const float2*>(mlp + (size_t)j * rows * 2);
      m[u] = k0 + u < mine ? ml.x : -INFINITY;
      l[u] = ml.y;
      o[u] = op[(size_t)j * rows * D];
    }
    float cm = mx;
#pragma unroll
    for (int u = 0; u < C; ++u) cm = fmaxf(cm, m[u]);
    if (cm == -INFINITY) continue;  // nothing but empty partials so far
    const float rescale = exp2f(mx - cm);  // 0 while mx is still -inf
    num *= rescale;
    den *= rescale;
#pragma unroll
    for (int u = 0; u < C; ++u) {
      const float f = m[u] == -INFINITY ? 0.0f : exp2f(m[u] - cm);
      num += f * o[u];
      den += f * l[u];
    }
    mx = cm;
  }
#pragma unroll
  for (int x = 1; x < T; x <<= 1) {
    const float m2 = __shfl_xor(mx, x, 64), n2 = __shfl_xor(num, x, 64), d2 = __shfl_xor(den, x, 64);
    const float cm = fmaxf(mx, m2);
    if (cm != -INFINITY) {
      const float f1 = mx == -INFINITY ? 0.0f : exp2f(mx - cm);
      const float f2 = m2 == -INFINITY ? 0.0f : exp2f(m2 - cm);
      num = f1 * num + f2 * n2;
      den = f1 * den + f2 * d2;
      mx = cm;
    }
  }
  if (sub == 0) p.out[idx] = num / den;
}

}  // namespace

int launch_decode_splitk(const DecodePlan& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  dim3 grid(p.n_splits, p.H, p.B);
  bool wide = false;
  for (int h = 0; h < p.H; ++h) {
    const int kb = p.k_bits[h], vb = p.v_bits[h];
    wide |= !(kb <= 4 && vb <= 4) && !(kb == 16 && vb == 16);
  }
  const bool paged = p.pages != nullptr;
  if (p.D == 128) {
    if (wide)
      hipLaunchKernelGGL((decode_kernel<128, true, true>), grid, dim3(kThreads), 0, s, p);
    else if (paged)
      hipLaunchKernelGGL((decode_kernel<128, false, true>), grid, dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((decode_kernel<128, false, false>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (wide)
      hipLaunchKernelGGL((decode_kernel<64, true, true>), grid, dim3(kThreads), 0, s, p);
    else if (paged)
      hipLaunchKernelGGL((decode_kernel<64, false, true>), grid, dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((decode_kernel<64, false, false>), grid, dim3(kThreads), 0, s, p);
  }
  return (int)hipGetLastError();
}

// Split partials of kvq_decode_attention_noalloc: a file-scope device array instead of a
// caller workspace, for callers that cannot allocate. Every GPU the library runs on holds its
// own copy, at its own address, until the process ends; host code reaches it only through the
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

int static_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kStaticScratchBytes;
  return 0;
}

int launch_decode_merge(const DecodePlan& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  // lanes per output element (T) and partials per lane (C): C the smallest power of two that
  // holds every split, up to kMergeChunk; past that, T lanes of kMergeChunk each
  int T = 1, C = 1;
  while (C < p.n_splits && C < kMergeChunk) C *= 2;
  while (T * C < p.n_splits) T *= 2;
  // (the fused step's ring store needs B H D / 4 threads, never more than the B Hq D elements)
  const size_t threads = (size_t)p.B * p.Q * p.Hq * p.D * T;
  const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
#define KVQ_MERGE(D_, T_, C_) hipLaunchKernelGGL((merge_kernel<D_, T_, C_>), dim3(blocks), dim3(kThreads), 0, s, p)
#define KVQ_MERGE_TC(D_)                                 \
  if (T == 1) {                                          \
    switch (C) {                                         \
      case 1: KVQ_MERGE(D_, 1, 1); break;                \
      case 2: KVQ_MERGE(D_, 1, 2); break;                \
      case 4: KVQ_MERGE(D_, 1, 4); break;                \
      case 8: KVQ_MERGE(D_, 1, 8); break;                \
      default: KVQ_MERGE(D_, 1, kMergeChunk); break;     \
    }                                                    \
  } else {                                               \
    switch (T) {                                         \
      case 2: KVQ_MERGE(D_, 2, kMergeChunk); break;      \
      case 4: KVQ_MERGE(D_, 4, kMergeChunk); break;      \
      case 8: KVQ_MERGE(D_, 8, kMergeChunk); break;      \
      default: KVQ_MERGE(D_, 16, kMergeChunk); break;    \
    }                                                    \
  }
  if (p.D == 128) {
    KVQ_MERGE_TC(128)
  } else {
    KVQ_MERGE_TC(64)
  }
#undef KVQ_MERGE_TC
#undef KVQ_MERGE
  return (int)hipGetLastError();
}

}  // namespace kvq
