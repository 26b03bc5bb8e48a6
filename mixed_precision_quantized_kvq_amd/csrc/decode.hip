// Split-K decode attention over the packed cache, with dequantization fused into q.K^T and
// P.V (InnerQ: grouping along the inner dimension, "Algorithm 1 ... decode phase"), and the
// log-sum-exp merge of the split partials.
//
// Work decomposition: grid (n_splits + 1, KV heads, rows). Workgroup `split` < n_splits owns
// a contiguous range of 64-token body tiles; its four wavefronts take tiles round-robin.
// The last workgroup of a (row, head) takes the 16-bit sink and recent-window tokens.
// Per tile:
//   scores  lane = token. Key group g of the token holds 32 codes c and fp16 (s, z), and
//           q.k_hat = sum_g s_g (q_g . c_g) + z_g sum(q_g)  (scale/zero factored out of each
//           group's partial dot product, InnerQ Fig. 2).
//   softmax online max / sum per wavefront, in log2 units.
//   values  lane = channel. A value group is 32 tokens of one channel with one (s, z):
//           o_c += sum_t p_t (c_t s + z).
// Each workgroup writes (m, l, o) for its G query heads; the merge kernel combines them.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxG = 4;

__device__ __forceinline__ float widen(uint16_t raw, int dtype) {
  if (dtype == KVQ_BF16) return __uint_as_float((uint32_t)raw << 16);
  return __half2float(__ushort_as_half(raw));
}
__device__ __forceinline__ float half_lo(uint32_t w) { return __half2float(__ushort_as_half((uint16_t)(w & 0xFFFFu))); }
__device__ __forceinline__ float half_hi(uint32_t w) { return __half2float(__ushort_as_half((uint16_t)(w >> 16))); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Bits [pos, pos + B) of a little-endian word stream held in registers. Called only from
// fully unrolled loops, so pos is a constant and the array stays in registers.
template <int B, int N>
__device__ __forceinline__ uint32_t extract(const uint32_t (&w)[N], int pos) {
  const int wi = pos >> 5, off = pos & 31;
  const uint32_t mask = (1u << B) - 1u;
  if (off + B <= 32) return (w[wi] >> off) & mask;
  return ((w[wi] >> off) | (w[wi + 1] << (32 - off))) & mask;
}

template <int D>
struct Smem {
  float q[kMaxG][D];
  float qsum[kMaxG][D / 32];
  float p[kWaves][kMaxG][64];
  float red_o[kWaves][kMaxG][D];
  float red_m[kWaves][kMaxG];
  float red_l[kWaves][kMaxG];
};

// ---- scores for one tile, lane = token --------------------------------------------------

template <int D, int B>
__device__ __forceinline__ void key_scores_q(const Smem<D>& sm, const uint32_t* kc_tile,
                                             const uint32_t* km_tok, int lane, float (&sc)[kMaxG]) {
  constexpr int Gd = D / 32, W = Gd * B;
  uint32_t w[W];
#pragma unroll
  for (int x = 0; x < W; ++x) {
    const int qc = x >> 2, nq = (W - 4 * qc) < 4 ? (W - 4 * qc) : 4;
    w[x] = kc_tile[256 * qc + lane * nq + (x - 4 * qc)];
  }
  uint32_t meta[Gd];
#pragma unroll
  for (int g = 0; g < Gd; ++g) meta[g] = km_tok[g];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) sc[i] = 0.0f;
#pragma unroll
  for (int g = 0; g < Gd; ++g) {
    float acc[kMaxG] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float cf = (float)extract<B>(w, (g * 32 + k) * B);
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) acc[i] = fmaf(cf, sm.q[i][g * 32 + k], acc[i]);
    }
    const float s = half_lo(meta[g]), z = half_hi(meta[g]);
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) sc[i] += s * acc[i] + z * sm.qsum[i][g];
  }
}

template <int D>
__device__ __forceinline__ void key_scores_16(const Smem<D>& sm, const uint16_t* row, int dtype,
                                              float (&sc)[kMaxG]) {
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) sc[i] = 0.0f;
  const uint4* r4 = reinterpret_cast<const uint4*>(row);
#pragma unroll 4
  for (int v = 0; v < D / 8; ++v) {
    const uint4 u = r4[v];
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = widen((uint16_t)(wd[k] & 0xFFFFu), dtype);
      const float b = widen((uint16_t)(wd[k] >> 16), dtype);
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) {
        sc[i] = fmaf(a, sm.q[i][v * 8 + 2 * k], sc[i]);
        sc[i] = fmaf(b, sm.q[i][v * 8 + 2 * k + 1], sc[i]);
      }
    }
  }
}

// ---- values for one tile, lane = channel -----------------------------------------------

template <int D, int B>
__device__ __forceinline__ void value_accum_q(const Smem<D>& sm, int wave, const uint32_t* vc_tile,
                                              const uint32_t* vm_tile, int lane, int nblk,
                                              float (&o)[kMaxG][D / 64]) {
#pragma unroll
  for (int ch = 0; ch < D / 64; ++ch) {
    const int c = lane + 64 * ch;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      if (jj < nblk) {
        uint32_t w[B];
#pragma unroll
        for (int k = 0; k < B; ++k) w[k] = vc_tile[(c * 2 + jj) * B + k];
        const uint32_t meta = vm_tile[c * 2 + jj];
        const float s = half_lo(meta), z = half_hi(meta);
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const float v = fmaf((float)extract<B>(w, k * B), s, z);
#pragma unroll
          for (int i = 0; i < kMaxG; ++i) o[i][ch] = fmaf(sm.p[wave][i][jj * 32 + k], v, o[i][ch]);
        }
      }
    }
  }
}

// 16-bit values: row_of(k) gives the row of token k of the tile (k < n_valid).
template <int D, class RowOf>
__device__ __forceinline__ void value_accum_16(const Smem<D>& sm, int wave, int lane, int n_valid,
                                               int dtype, RowOf row_of, float (&o)[kMaxG][D / 64]) {
  for (int k = 0; k < n_valid; ++k) {
    const uint16_t* row = row_of(k);
#pragma unroll
    for (int ch = 0; ch < D / 64; ++ch) {
      const float v = widen(row[lane + 64 * ch], dtype);
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) o[i][ch] = fmaf(sm.p[wave][i][k], v, o[i][ch]);
    }
  }
}

// ---- online softmax bookkeeping ----------------------------------------------------------

template <int D>
__device__ __forceinline__ void softmax_update(Smem<D>& sm, int wave, int lane, bool valid,
                                               const float (&sc)[kMaxG], float (&m_run)[kMaxG],
                                               float (&l_lane)[kMaxG], float (&o)[kMaxG][D / 64],
                                               float scale_log2) {
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    const float s = valid ? sc[i] * scale_log2 : -INFINITY;
    const float mt = wave_max(s);
    const float m_new = fmaxf(m_run[i], mt);
    const float alpha = exp2f(m_run[i] - m_new);
    const float pv = valid ? exp2f(s - m_new) : 0.0f;
    l_lane[i] = l_lane[i] * alpha + pv;
#pragma unroll
    for (int ch = 0; ch < D / 64; ++ch) o[i][ch] *= alpha;
    m_run[i] = m_new;
    sm.p[wave][i][lane] = pv;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodePlan p) {
  __shared__ Smem<D> sm;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)b * p.Hq + (size_t)h * G) * D;
  for (int idx = tid; idx < kMaxG * D; idx += kThreads) {
    const int i = idx / D, c = idx % D;
    sm.q[i][c] = i < G ? widen(q[(size_t)i * D + c], p.dtype) : 0.0f;
  }
  __syncthreads();
  if (tid < kMaxG * (D / 32)) {
    const int i = tid / (D / 32), g = tid % (D / 32);
    float s = 0.0f;
    for (int k = 0; k < 32; ++k) s += sm.q[i][g * 32 + k];
    sm.qsum[i][g] = s;
  }
  __syncthreads();

  float m_run[kMaxG], l_lane[kMaxG], o[kMaxG][D / 64];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    m_run[i] = -INFINITY;
    l_lane[i] = 0.0f;
#pragma unroll
    for (int ch = 0; ch < D / 64; ++ch) o[i][ch] = 0.0f;
  }
  const uint64_t* off = p.off + ((size_t)b * p.H + h) * kRegions;
  const int kb = p.k_bits[h], vb = p.v_bits[h];

  if (split < p.n_splits) {
    const int t0 = split * p.tiles_per_split;
    const int t1 = min(p.n_tiles, t0 + p.tiles_per_split);
    for (int tile = t0 + wave; tile < t1; tile += kWaves) {
      const int tok = tile * kTile + lane;
      const bool valid = tok < p.body;
      const int tok_c = valid ? tok : p.body - 1;  // clamp loads of lanes past the end
      float sc[kMaxG];
      if (kb == 16) {
        key_scores_16<D>(sm, reinterpret_cast<const uint16_t*>(p.blob + off[KC]) + (size_t)tok_c * D, p.dtype, sc);
      } else {
        const uint32_t* kc_tile = reinterpret_cast<const uint32_t*>(p.blob + off[KC]) + (size_t)tile * kTile * (D / 32) * kb;
        const uint32_t* km_tok = reinterpret_cast<const uint32_t*>(p.blob + off[KM]) + (size_t)tok_c * (D / 32);
        // lanes past the body end read the (allocated) rest of the last tile
        switch (kb) {
          case 2: key_scores_q<D, 2>(sm, kc_tile, km_tok, lane, sc); break;
          case 3: key_scores_q<D, 3>(sm, kc_tile, km_tok, lane, sc); break;
          case 4: key_scores_q<D, 4>(sm, kc_tile, km_tok, lane, sc); break;
          case 5: key_scores_q<D, 5>(sm, kc_tile, km_tok, lane, sc); break;
          case 6: key_scores_q<D, 6>(sm, kc_tile, km_tok, lane, sc); break;
          case 7: key_scores_q<D, 7>(sm, kc_tile, km_tok, lane, sc); break;
          default: key_scores_q<D, 8>(sm, kc_tile, km_tok, lane, sc); break;
        }
      }
      softmax_update<D>(sm, wave, lane, valid, sc, m_run, l_lane, o, p.scale_log2);
      const int n_valid = min(kTile, p.body - tile * kTile);
      if (vb == 16) {
        const uint16_t* vbase = reinterpret_cast<const uint16_t*>(p.blob + off[VC]) + (size_t)tile * kTile * D;
        value_accum_16<D>(sm, wave, lane, n_valid, p.dtype,
                          [&](int k) { return vbase + (size_t)k * D; }, o);
      } else {
        const int nblk = n_valid / 32;
        const uint32_t* vc_tile = reinterpret_cast<const uint32_t*>(p.blob + off[VC]) + (size_t)tile * 2 * D * vb;
        const uint32_t* vm_tile = reinterpret_cast<const uint32_t*>(p.blob + off[VM]) + (size_t)tile * 2 * D;
        switch (vb) {
          case 2: value_accum_q<D, 2>(sm, wave, vc_tile, vm_tile, lane, nblk, o); break;
          case 3: value_accum_q<D, 3>(sm, wave, vc_tile, vm_tile, lane, nblk, o); break;
          case 4: value_accum_q<D, 4>(sm, wave, vc_tile, vm_tile, lane, nblk, o); break;
          case 5: value_accum_q<D, 5>(sm, wave, vc_tile, vm_tile, lane, nblk, o); break;
          case 6: value_accum_q<D, 6>(sm, wave, vc_tile, vm_tile, lane, nblk, o); break;
          case 7: value_accum_q<D, 7>(sm, wave, vc_tile, vm_tile, lane, nblk, o); break;
          default: value_accum_q<D, 8>(sm, wave, vc_tile, vm_tile, lane, nblk, o); break;
        }
      }
      wave_sync_lds();  // p of this tile is consumed before the next tile overwrites it
    }
  } else {
    // 16-bit windows: window token u < n_sink_live is sink row u, else the ring slot of
    // absolute token n_sink + body + (u - n_sink_live)
    const int n_tot = p.n_sink_live + p.n_win;
    const uint16_t* sk = reinterpret_cast<const uint16_t*>(p.blob + off[SK]);
    const uint16_t* sv = reinterpret_cast<const uint16_t*>(p.blob + off[SV]);
    const uint16_t* rk = reinterpret_cast<const uint16_t*>(p.blob + off[RK]);
    const uint16_t* rv = reinterpret_cast<const uint16_t*>(p.blob + off[RV]);
    auto row_index = [&](int u, bool& in_sink) {
      in_sink = u < p.n_sink_live;
      return in_sink ? u : (p.body + u - p.n_sink_live) % p.ring;
    };
    for (int base = wave * kTile; base < n_tot; base += kWaves * kTile) {
      const int u = base + lane;
      const bool valid = u < n_tot;
      bool in_sink;
      const int r = row_index(valid ? u : 0, in_sink);
      float sc[kMaxG];
      key_scores_16<D>(sm, (in_sink ? sk : rk) + (size_t)r * D, p.dtype, sc);
      softmax_update<D>(sm, wave, lane, valid, sc, m_run, l_lane, o, p.scale_log2);
      const int n_valid = min(kTile, n_tot - base);
      value_accum_16<D>(sm, wave, lane, n_valid, p.dtype,
                        [&](int k) {
                          bool s_;
                          const int rr = row_index(base + k, s_);
                          return (s_ ? sv : rv) + (size_t)rr * D;
                        },
                        o);
      wave_sync_lds();
    }
  }

  // combine the four wavefronts
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    const float l = wave_sum(l_lane[i]);
    if (lane == 0) {
      sm.red_m[wave][i] = m_run[i];
      sm.red_l[wave][i] = l;
    }
#pragma unroll
    for (int ch = 0; ch < D / 64; ++ch) sm.red_o[wave][i][lane + 64 * ch] = o[i][ch];
  }
  __syncthreads();
  const size_t rows = (size_t)p.B * p.Hq;
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
    const size_t row = (size_t)b * p.Hq + (size_t)h * G + i;
    p.ws_o[((size_t)split * rows + row) * D + c] = oo;
    if (c == 0) {
      p.ws_ml[((size_t)split * rows + row) * 2] = ms;
      p.ws_ml[((size_t)split * rows + row) * 2 + 1] = ll;
    }
  }
}

// out = sum_j 2^(m_j - m*) o_j / sum_j 2^(m_j - m*) l_j over the n_splits + 1 partials
__global__ __launch_bounds__(128) void merge_kernel(const DecodePlan p) {
  const size_t row = blockIdx.x;
  const int c = threadIdx.x;
  const size_t rows = (size_t)p.B * p.Hq;
  const int parts = p.n_splits + 1;
  float ms = -INFINITY;
  for (int j = 0; j < parts; ++j) ms = fmaxf(ms, p.ws_ml[((size_t)j * rows + row) * 2]);
  float oo = 0.0f, ll = 0.0f;
  for (int j = 0; j < parts; ++j) {
    const float mj = p.ws_ml[((size_t)j * rows + row) * 2];
    if (mj == -INFINITY) continue;
    const float f = exp2f(mj - ms);
    oo += f * p.ws_o[((size_t)j * rows + row) * p.D + c];
    ll += f * p.ws_ml[((size_t)j * rows + row) * 2 + 1];
  }
  p.out[row * p.D + c] = oo / ll;
}

}  // namespace

int launch_decode(const DecodePlan& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  dim3 grid(p.n_splits + 1, p.H, p.B);
  if (p.D == 128)
    hipLaunchKernelGGL(decode_kernel<128>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(decode_kernel<64>, grid, dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(merge_kernel, dim3(p.B * p.Hq), dim3(p.D), 0, s, p);
  return (int)hipGetLastError();
}

}  // namespace kvq
