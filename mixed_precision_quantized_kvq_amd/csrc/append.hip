// Append kernels: quantize + pack the 32-token blocks that leave the recent window, and copy
// new sink / recent tokens into their 16-bit windows (InnerQ techniques (i) and (ii)).
// Built with -ffp-contract=off: the quantizer must round exactly as quant_device.h states.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "code_plans.h"
#include "kvq_internal.h"
#include "quant_device.h"

namespace kvq {
namespace {

// Token counts of row b for this append (uniform, or the row's own when ragged).
__device__ __forceinline__ RowAppend row_append(const AppendPlan& p, int b) {
  if (!p.ragged) return RowAppend{p.len0, p.len1, p.body0, p.body1, p.n_new};
  RowAppend a;
  a.len0 = p.row_len0[b];
  a.n = p.row_new[b];
  a.len1 = a.len0 + a.n;
  auto body = [&](int T) {
    const int r = T - p.n_sink - p.n_recent;
    return r <= 0 ? 0 : (r / kGroup) * kGroup;
  };
  a.body0 = body(a.len0);
  a.body1 = body(a.len1);
  return a;
}

// Address of absolute token t of (row, head): the ring if it was appended before this call
// (only live ring tokens are ever flushed), else the new input.
__device__ __forceinline__ const uint16_t* token_row(const AppendPlan& p, int len0, const char* base_ring,
                                                     const uint16_t* in, int t) {
  if (t < len0) {
    const int slot = (t - p.n_sink) % (p.n_recent + kGroup);
    return reinterpret_cast<const uint16_t*>(base_ring) + (size_t)slot * p.D;
  }
  return in + (size_t)(t - len0) * p.D;
}

// Range check on raw 16-bit elements (two to a word): |x| <= 2^14 and not NaN is
// (bits & 0x7FFF) <= the bits of 2^14, since non-negative values order like their patterns
// and infinities and NaNs lie above every finite value.
__device__ __forceinline__ bool raw_out_of_range(const uint32_t (&w)[16], int dtype) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int k = 1; k < 16; ++k) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[k] & 0x7FFF7FFFu));
  const unsigned lim = dtype == KVQ_BF16 ? 0x4680u : 0x7400u;  // 16384 in bf16 / fp16
  return max((unsigned)m.x, (unsigned)m.y) > lim;
}
// The same test on fp32 values (keys divided by their norms).
__device__ __forceinline__ bool f32_out_of_range(const float (&x)[32]) {
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  return m > 0x46800000u;  // 16384.0f
}

template <bool BF16>
__device__ __forceinline__ void widen_words(const uint32_t (&w)[16], float (&x)[32]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if constexpr (BF16) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    } else {
      x[2 * k] = widen16((uint16_t)(w[k] & 0xFFFFu), KVQ_F16);
      x[2 * k + 1] = widen16((uint16_t)(w[k] >> 16), KVQ_F16);
    }
  }
}

// Codes (as patterns, quant_device.h) of a group: the asymmetric quantizer, or the hybrid
// choice by float64 squared error (strictly lower wins, ties to asymmetric). The hybrid pass
// scores both variants element by element without keeping their codes, then forms the
// winner's codes; the symmetric form is the asymmetric one with zero 0 (x - 0 = x exactly).
template <int B>
__device__ __forceinline__ GroupQ quantize_patterns(const float (&x)[32], bool hybrid, uint32_t (&cb)[32]) {
  const GroupQ a = asym_params(x, B);
  FastForm f = fast_form<false>(a);
  if (hybrid) {
    const GroupQ sq = sym_params(x, B);
    const FastForm fs = fast_form<true>(sq);
    const double sa = (double)a.s, za = (double)a.z, ss = (double)sq.s, zs = (double)sq.z;
    double ea = 0.0, es = 0.0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const double xd = (double)x[i];
      const double da = xd - __fma_rn((double)(code_pattern<false>(x[i], f) - kTwo23Bits), sa, za);
      const double ds = xd - __fma_rn((double)(code_pattern<true>(x[i], fs) - kTwo23Bits), ss, zs);
      const double qa = da * da, qs = ds * ds;
      ea = ea + qa;
      es = es + qs;
    }
    if (es < ea) {
      f = fs;
      f.z = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) cb[i] = code_pattern<false>(x[i], f);
      return sq;
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) cb[i] = code_pattern<false>(x[i], f);
  return a;
}

// Value streams. Decode lane (g4, n) of a tile (g4 = 2 * block + jp) holds D/32 streams of 32
// codes; stream vg holds channels 16 nb + n for nb = 2 vg, 2 vg + 1 and, of each, the tokens
// 16 kk + 8 jp + u (kk = 0, 1; u = 0..7) of the block, element e = 8 (2 (nb % 2) + kk) + u at
// stream position vpos(e), the order in which the decode kernel's value plan reads them.
template <int B>
__host__ __device__ constexpr int vpos(int e) {
  return VSlots<B>::chan(2 * (e >> 3) + ((e & 7) >> 2), e & 3);
}
// Bit of token k of a channel of parity P (nb % 2) in its stream for jp = (k >> 3) & 1.
template <int B, int P>
__host__ __device__ constexpr int vbit(int k) {
  return vpos<B>(8 * (2 * P + (k >> 4)) + (k & 7)) * B;
}
// Widths whose parity-1 positions are the parity-0 ones plus 16: each channel then owns whole
// words of its two streams (the first or second B/2 words).
template <int B>
__host__ __device__ constexpr bool split_halves() {
  for (int e = 0; e < 16; ++e)
    if (vpos<B>(e + 16) != vpos<B>(e) + 16 || vpos<B>(e) >= 16) return false;
  return true;
}
template <int B, int P>
struct HalfTotals {  // constant parts of the two streams' words once a channel's patterns are in
  uint32_t v[2][B];
  constexpr HalfTotals() : v() {
    for (int k = 0; k < 32; ++k) {
      const int bit = vbit<B, P>(k), wi = bit >> 5, off = bit & 31, jp = (k >> 3) & 1;
      v[jp][wi] += kTwo23Bits << off;
      if (off + B > 32) v[jp][wi + 1] += kTwo23Bits >> (32 - off);
    }
  }
};
// This channel's codes in its two streams (s0: jp = 0, s1: jp = 1), zeros elsewhere.
template <int B, int P>
__device__ __forceinline__ void pack_value_halves(const uint32_t (&cb)[32], uint32_t (&s0)[B], uint32_t (&s1)[B]) {
  constexpr HalfTotals<B, P> t{};
#pragma unroll
  for (int w = 0; w < B; ++w) {
    s0[w] = 0u - t.v[0][w];
    s1[w] = 0u - t.v[1][w];
  }
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if ((k >> 3) & 1) add_at<B, B>(s1, vbit<B, P>(k), cb[k]);
    else add_at<B, B>(s0, vbit<B, P>(k), cb[k]);
  }
}

// Store of a value thread's codes. Thread xv = channel c = 16 nb + n sits in lane c % 64 of
// its wavefront, so the other channel of its streams (parity 1 - P) is 16 lanes away, in the
// paired 16-lane row.
template <int B>
__device__ __forceinline__ void store_value_streams(const uint32_t (&cb)[32], int c, int jj, int D, uint32_t* vc) {
  const int n = c & 15, nb = c >> 4, P = nb & 1, vg = nb >> 1, nv = D / 32;
  // words of stream vg of decode lane (2 jj + jp) * 16 + n
  auto dst = [&](int jp) { return vc + ((size_t)(((2 * jj + jp) * 16 + n) * nv + vg)) * B; };
  uint32_t s0[B], s1[B];
  if constexpr (split_halves<B>()) {
    pack_value_halves<B, 0>(cb, s0, s1);
    uint32_t* d0 = dst(0) + P * (B / 2);
    uint32_t* d1 = dst(1) + P * (B / 2);
#pragma unroll
    for (int w = 0; w < B / 2; ++w) {
      d0[w] = s0[w];
      d1[w] = s1[w];
    }
  } else {
    if (P) pack_value_halves<B, 1>(cb, s0, s1);
    else pack_value_halves<B, 0>(cb, s0, s1);
    // or in the paired row's halves (16-lane rows 0 <-> 1, 2 <-> 3)
#pragma unroll
    for (int w = 0; w < B; ++w) {
      const auto x0 = __builtin_amdgcn_permlane16_swap(s0[w], s0[w], false, false);
      const auto x1 = __builtin_amdgcn_permlane16_swap(s1[w], s1[w], false, false);
      s0[w] = x0[0] | x0[1];
      s1[w] = x1[0] | x1[1];
    }
    uint32_t* d = dst(P);
#pragma unroll
    for (int w = 0; w < B; ++w) d[w] = P ? s1[w] : s0[w];
  }
}

// Flush of 32-token blocks leaving the recent window: one workgroup per (block, KV head, row),
// 2*D threads (D is a template parameter, so row strides are immediate load offsets). Thread i < D quantizes key group i = (token tt of the block) * (D/32) + channel
// group g; thread D + c quantizes value channel c over the block's 32 tokens and writes its
// codes straight into the two value streams that hold them (no LDS, no barrier).
template <int D, bool ASYM>
__global__ __launch_bounds__(2 * D) void append_flush_kernel(const AppendPlan p) {
  constexpr int Gd = D / kGroup;
  const bool hybrid = !ASYM && p.hybrid != 0;
  const int h = blockIdx.y, b = blockIdx.z;
  const RowAppend ra = row_append(p, b);
  if ((int)blockIdx.x >= (ra.body1 - ra.body0) / kGroup) return;  // ragged: this row flushes fewer blocks
  const int j = ra.body0 / kGroup + blockIdx.x;                    // body block index
  // the region table of this (row, head), read into scalar registers before any store
  const uint64_t* tab = p.off + ((size_t)b * p.H + h) * kRegions;
  uint64_t off[kRegions];
#pragma unroll
  for (int r = 0; r < kRegions; ++r) off[r] = tab[r];
  const size_t in_off = ((size_t)b * p.H + h) * p.n_new * D;
  const uint16_t* kin = reinterpret_cast<const uint16_t*>(p.k_in) + in_off;
  const uint16_t* vin = reinterpret_cast<const uint16_t*>(p.v_in) + in_off;
  const int tid = threadIdx.x;
  const bool is_key = tid < D;
  const int bits = is_key ? p.k_bits[h] : p.v_bits[h];
  const int tile = j >> 1, jj = j & 1;
  // paged caches: the tile's page in this head's pools; an unmapped tile writes nothing and
  // sets flag bit 1
  int ptile = tile;
  if (p.pages) {
    ptile = p.pages[(size_t)b * p.page_stride + tile];
    if (ptile < 0 || ptile >= p.n_pages) {
      if (tid == 0) atomicOr(p.range_flag, 2u);
      return;
    }
  }
  const int pj = 2 * ptile + jj;  // the block's slot in the body region or pools
  const int t0 = p.n_sink + j * kGroup;  // first token of the block
  // the block's value rows: consecutive rows of the input or of the ring unless the block
  // straddles the append or the ring's end (uniform)
  const int slot0 = (t0 - p.n_sink) % (p.n_recent + kGroup);
  const bool in_ring = t0 + kGroup <= ra.len0 && slot0 + kGroup <= p.n_recent + kGroup;
  const bool in_input = t0 >= ra.len0;
  const uint16_t* vrows = in_ring    ? reinterpret_cast<const uint16_t*>(p.blob + off[RV]) + (size_t)slot0 * D
                          : in_input ? vin + (size_t)(t0 - ra.len0) * D
                                     : nullptr;
  if (bits == 16) {
    // unquantized head: the block's rows are copied
    if (is_key) {
      const int tt = tid / Gd, g = tid % Gd;
      const uint16_t* src = token_row(p, ra.len0, p.blob + off[RK], kin, t0 + tt) + g * kGroup;
      uint4* dst = reinterpret_cast<uint4*>(p.blob + off[KC]) + ((size_t)(pj * kGroup + tt) * D + g * kGroup) / 8;
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[v] = reinterpret_cast<const uint4*>(src)[v];
    } else {
      const int c = tid - D;
      uint16_t* dst = reinterpret_cast<uint16_t*>(p.blob + off[VC]);
#pragma unroll
      for (int k = 0; k < 32; ++k)
        dst[(size_t)(pj * kGroup + k) * D + c] = token_row(p, ra.len0, p.blob + off[RV], vin, t0 + k)[c];
    }
    return;
  }
  // the group's 32 raw elements, two to a word
  uint32_t raw[16];
  if (is_key) {
    const int tt = tid / Gd, g = tid % Gd;
    const uint4* s4 = reinterpret_cast<const uint4*>(token_row(p, ra.len0, p.blob + off[RK], kin, t0 + tt) + g * kGroup);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 u = s4[v];
      raw[4 * v] = u.x;
      raw[4 * v + 1] = u.y;
      raw[4 * v + 2] = u.z;
      raw[4 * v + 3] = u.w;
    }
  } else {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const int c = tid - D;
    if (vrows) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const u16x2 e = {vrows[(2 * k) * D + c], vrows[(2 * k + 1) * D + c]};
        raw[k] = __builtin_bit_cast(uint32_t, e);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const u16x2 e = {token_row(p, ra.len0, p.blob + off[RV], vin, t0 + 2 * k)[c],
                         token_row(p, ra.len0, p.blob + off[RV], vin, t0 + 2 * k + 1)[c]};
        raw[k] = __builtin_bit_cast(uint32_t, e);
      }
    }
  }
  // the dtype is uniform: one widening per launch, not both and a select per element
  float x[32];
  if (p.dtype == KVQ_BF16) widen_words<true>(raw, x);
  else widen_words<false>(raw, x);
  bool bad;
  if (is_key && p.key_norm) {  // the group holds k_c / n_c (IEEE fp32 division)
    const float* kn = reinterpret_cast<const float*>(p.blob + off[KN]) + (tid % Gd) * kGroup;
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = x[i] / kn[i];
    bad = f32_out_of_range(x);
  } else {
    bad = raw_out_of_range(raw, p.dtype);
  }
  if (bad) atomicOr(p.range_flag, 1u);
  bool sym = false;
  // the width is uniform over each wavefront (keys: wavefronts 0, 1; values: 2, 3)
  auto group = [&](auto bc) {
    constexpr int B = decltype(bc)::value;
    uint32_t cb[32];
    const GroupQ q = quantize_patterns<B>(x, hybrid, cb);
    sym = q.sym;
    const uint32_t meta = (uint32_t)q.s_bits | ((uint32_t)q.z_bits << 16);
    if (is_key) {
      uint32_t w[B];
      pack_patterns<B>(cb, w);
      const int tt = tid / Gd, g = tid % Gd;
      const int W = Gd * B;  // words per token
      const int t_in_tile = jj * kGroup + tt;
      uint32_t* kc = reinterpret_cast<uint32_t*>(p.blob + off[KC]) + (size_t)ptile * kTile * W;
#pragma unroll
      for (int k = 0; k < B; ++k) {
        const int wi = g * B + k;
        const int qc = wi >> 2, nq = min(4, W - 4 * qc);
        kc[256 * qc + t_in_tile * nq + (wi - 4 * qc)] = w[k];
      }
      reinterpret_cast<uint32_t*>(p.blob + off[KM])[(size_t)(pj * kGroup + tt) * Gd + g] = meta;
    } else {
      const int c = tid - D;
      store_value_streams<B>(cb, c, jj, D, reinterpret_cast<uint32_t*>(p.blob + off[VC]) + (size_t)ptile * 2 * D * B);
      // (s|z) of channel c = 16 nb + n for this block, at [tile][block][n][nb]
      reinterpret_cast<uint32_t*>(p.blob + off[VM])[(size_t)ptile * 2 * D + jj * D + (c & 15) * (D / 16) + (c >> 4)] =
          meta;
    }
  };
  switch (bits) {
    case 2: group(std::integral_constant<int, 2>{}); break;
    case 3: group(std::integral_constant<int, 3>{}); break;
    case 4: group(std::integral_constant<int, 4>{}); break;
    case 5: group(std::integral_constant<int, 5>{}); break;
    case 6: group(std::integral_constant<int, 6>{}); break;
    case 7: group(std::integral_constant<int, 7>{}); break;
    default: group(std::integral_constant<int, 8>{}); break;
  }
  if (hybrid) {
    // flag bit i of this block's key (value) words = group i of thread i (D + i)
    const unsigned long long m = __ballot(sym);
    if ((tid & 63) == 0) {
      uint32_t* fl = reinterpret_cast<uint32_t*>(p.blob + off[FL]) + (size_t)pj * 2 * Gd;
      const int wbase = (is_key ? 0 : Gd) + ((is_key ? tid : tid - D) >> 5);
      fl[wbase] = (uint32_t)m;
      fl[wbase + 1] = (uint32_t)(m >> 32);
    }
  }
}

// Per-channel key norms of the first append (InnerQ technique (iii)): n_c = the smallest power
// of two >= max |k_c| over its tokens, 1 where that max is 0. One workgroup per (row, KV head):
// thread (lane l, part r) reads 16-byte pieces l (8 channels) of tokens r, r + R, ...; the
// maxima meet in LDS (as the bit patterns of non-negative floats, which order like the
// floats). Heads kept in 16 bits have no norms.
constexpr int kNormThreads = 1024;
__global__ __launch_bounds__(kNormThreads) void key_norm_kernel(const AppendPlan p) {
  __shared__ uint32_t nmax[128];
  const int h = blockIdx.x % p.H, b = blockIdx.x / p.H, tid = threadIdx.x;
  if (p.k_bits[h] == 16) return;  // uniform over the workgroup
  if (tid < p.D) nmax[tid] = 0u;
  __syncthreads();
  const int pieces = p.D / 8, parts = kNormThreads / pieces;
  const int l = tid % pieces, r = tid / pieces;
  const uint4* k = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.k_in) +
                                                  ((size_t)b * p.H + h) * p.n_new * p.D) + l;
  float m[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  const RowAppend ra = row_append(p, b);
  if (p.ragged && !(ra.len0 == 0 && ra.n > 0)) return;  // norms come from a row's first append
  // eight tokens' loads in flight per thread (a token past the end re-reads the last one,
  // which leaves the maxima unchanged)
  constexpr int kBatch = 8;
  for (int t0 = r; t0 < ra.n; t0 += kBatch * parts) {
    uint4 u[kBatch];
#pragma unroll
    for (int v = 0; v < kBatch; ++v) u[v] = k[(size_t)min(t0 + v * parts, ra.n - 1) * pieces];
#pragma unroll
    for (int v = 0; v < kBatch; ++v) {
      const uint32_t w[4] = {u[v].x, u[v].y, u[v].z, u[v].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[2 * i] = fmaxf(m[2 * i], fabsf(widen16((uint16_t)(w[i] & 0xFFFFu), p.dtype)));
        m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(widen16((uint16_t)(w[i] >> 16), p.dtype)));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) atomicMax(&nmax[8 * l + i], __float_as_uint(m[i]));
  __syncthreads();
  if (tid < p.D) {
    const uint64_t* off = p.off + ((size_t)b * p.H + h) * kRegions;
    // the smallest power of two >= max |k_c| (1 if that is 0): dividing by it, and folding
    // it into the query, is exact
    const float m = __uint_as_float(nmax[tid]);
    int e = 0;
    const float f = frexpf(m, &e);  // m = f * 2^e, 0.5 <= f < 1
    const float n = f == 0.5f ? m : ldexpf(1.0f, e);
    reinterpret_cast<float*>(p.blob + off[KN])[tid] = m > 0.0f ? n : 1.0f;
  }
}

// Copy new tokens that land in the sink or in the recent ring: one thread per 16 bytes of a
// key or value row. Token index k < n_a is sink token len0 + k, else ring token t_b + k - n_a
// (per row: sink tokens [len0, min(len1, n_sink)), ring tokens [max(len0, n_sink + body1),
// len1)). The grid covers n_tok tokens per row, the most any row copies.
__global__ __launch_bounds__(256) void append_window_kernel(const AppendPlan p, int n_tok) {
  const int chunks = p.D / 8;                   // 16-byte chunks per row
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)p.B * p.H * n_tok * 2 * chunks;
  if (gid >= total) return;
  const int ch = (int)(gid % chunks);
  long long r = gid / chunks;
  const int kv = (int)(r % 2);
  r /= 2;
  const int k = (int)(r % n_tok);
  r /= n_tok;
  const int h = (int)(r % p.H), b = (int)(r / p.H);
  const RowAppend ra = row_append(p, b);
  const int n_a = max(0, min(ra.len1, p.n_sink) - ra.len0);
  const int t_b = max(ra.len0, p.n_sink + ra.body1);
  if (k >= n_a + max(0, ra.len1 - t_b)) return;
  const int t = k < n_a ? ra.len0 + k : t_b + (k - n_a);
  const uint64_t* off = p.off + ((size_t)b * p.H + h) * kRegions;
  const uint16_t* in = reinterpret_cast<const uint16_t*>(kv ? p.v_in : p.k_in) +
                       (((size_t)b * p.H + h) * p.n_new + (t - ra.len0)) * p.D;
  char* dst_row;
  if (t < p.n_sink) {
    dst_row = p.blob + off[kv ? SV : SK] + (size_t)t * p.D * 2;
  } else {
    const int slot = (t - p.n_sink) % (p.n_recent + kGroup);
    dst_row = p.blob + off[kv ? RV : RK] + (size_t)slot * p.D * 2;
  }
  reinterpret_cast<uint4*>(dst_row)[ch] = reinterpret_cast<const uint4*>(in)[ch];
}

}  // namespace

int launch_append_flush(const AppendPlan& p, void* stream) {
  int nblk = 0;
  for (int b = 0; b < (p.ragged ? p.B : 1); ++b) {
    const RowAppend a = host_row_append(p, b);
    nblk = max(nblk, (a.body1 - a.body0) / kGroup);
  }
  if (nblk <= 0) return (int)hipSuccess;
  dim3 grid(nblk, p.H, p.B);
  hipStream_t s = (hipStream_t)stream;
  if (p.D == 128) {
    if (p.hybrid) hipLaunchKernelGGL((append_flush_kernel<128, false>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((append_flush_kernel<128, true>), grid, dim3(256), 0, s, p);
  } else {
    if (p.hybrid) hipLaunchKernelGGL((append_flush_kernel<64, false>), grid, dim3(128), 0, s, p);
    else hipLaunchKernelGGL((append_flush_kernel<64, true>), grid, dim3(128), 0, s, p);
  }
  return (int)hipGetLastError();
}

int launch_key_norms(const AppendPlan& p, void* stream) {
  hipLaunchKernelGGL(key_norm_kernel, dim3((unsigned)(p.B * p.H)), dim3(kNormThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_append_window(const AppendPlan& p, void* stream) {
  // sink tokens [len0, min(len1, n_sink)); ring tokens [max(len0, n_sink + body1), len1)
  int n_tok = 0;
  for (int b = 0; b < (p.ragged ? p.B : 1); ++b) {
    const RowAppend a = host_row_append(p, b);
    const int n_a = max(0, min(a.len1, p.n_sink) - a.len0);
    const int t_b = max(a.len0, p.n_sink + a.body1);
    n_tok = max(n_tok, n_a + max(0, a.len1 - t_b));
  }
  if (n_tok == 0) return (int)hipSuccess;
  const long long total = (long long)p.B * p.H * n_tok * 2 * (p.D / 8);
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(append_window_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                     (hipStream_t)stream, p, n_tok);
  return (int)hipGetLastError();
}

}  // namespace kvq
