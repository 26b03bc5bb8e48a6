// Append kernels: quantize + pack the 32-token blocks that leave the recent window, and copy
// new sink / recent tokens into their 16-bit windows (InnerQ techniques (i) and (ii)).
// Built with -ffp-contract=off: the quantizer must round exactly as quant_device.h states.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "code_plans.h"
#include "kvq_internal.h"
#include "quant_device.h"

namespace kvq {
namespace {

constexpr int kFlushWgPerCu = 4;  // persistent flush workgroups per compute unit

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

__device__ __forceinline__ void load_row32(const uint16_t* src, int dtype, float (&x)[32]) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint4 u = s4[v];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[v * 8 + 2 * k] = widen16((uint16_t)(w[k] & 0xFFFFu), dtype);
      x[v * 8 + 2 * k + 1] = widen16((uint16_t)(w[k] >> 16), dtype);
    }
  }
}

// Value stream of one decode lane: the 32 codes of virtual stream vg of lane (g4, n) of the
// block's half of the tile (g4 = 2 * (block % 2) + jp). Stream position chan(s, k) holds the
// code of token 16 kk + 8 jp + u of channel 16 nb + n, with chunk c = s / 2, nb = 2 vg + c / 2,
// kk = c % 2, u = 4 (s % 2) + k: the order the decode kernel's value plan reads.
template <int B>
__device__ __forceinline__ void pack_value_stream(const uint8_t (*codes)[36], int vg, int jp, int n,
                                                  uint32_t* dst) {
  uint64_t acc = 0;
  int nbits = 0, w = 0;
#pragma unroll
  for (int qpos = 0; qpos < kGroup; ++qpos) {
    int s = 0, k = 0;
#pragma unroll
    for (int ss = 0; ss < 8; ++ss)
#pragma unroll
      for (int kk4 = 0; kk4 < 4; ++kk4)
        if (VSlots<B>::chan(ss, kk4) == qpos) {
          s = ss;
          k = kk4;
        }
    const int c = s >> 1, nb = 2 * vg + (c >> 1), kk = c & 1, u = 4 * (s & 1) + k;
    acc |= (uint64_t)codes[16 * nb + n][16 * kk + 8 * jp + u] << nbits;
    nbits += B;
    if (nbits >= 32) {
      dst[w++] = (uint32_t)acc;
      acc >>= 32;
      nbits -= 32;
    }
  }
}

// Flush of 32-token blocks leaving the recent window. One item is one block of one (row, KV
// head); items are numbered ((row * H + head) * kmax + k), block k of the row's flushed ones
// (kmax: the most any row flushes; a ragged row's items past its own count are skipped). The
// grid is persistent: workgroup w takes items w, w + gridDim.x, ... With 2*D threads, the 32
// input rows of keys and of values of an item (2 x 8 KB at D = 128) are staged in LDS; the
// loads of the workgroup's next item are issued into registers before the current item is
// quantized, and reach LDS after it, so each workgroup keeps a block's loads in flight while
// it computes. From the stage, thread i < D quantizes key group i = (token tt of the block) *
// (D/32) + channel group g, and thread D + c value channel c over the block's 32 tokens;
// value codes go through LDS once more, to be written one (decode lane, stream) per thread in
// the decode kernel's value order.
// ASYM: the instantiation for asymmetric caches. The hybrid choice's float64 errors of both
// variants need about twice the registers, so an asymmetric cache runs at twice the
// occupancy without that code.
template <bool ASYM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ASYM ? 4 : 2))) void append_flush_kernel(
    const AppendPlan p, int kmax) {
  const bool hybrid = !ASYM && p.hybrid != 0;
  __shared__ alignas(16) uint16_t stage[2][kGroup][128];  // [keys | values][token of the block][channel]
  __shared__ alignas(4) uint8_t vcodes[128][36];          // [channel][token of the block], rows padded to 36 bytes
  const int D = p.D, Gd = D / kGroup;
  const int n_items = p.B * p.H * kmax;
  // Coordinates of an item; false for an item past its ragged row's flush count.
  auto item = [&](int it, int& b, int& h, int& j, RowAppend& ra) {
    const int k = it % kmax;
    h = (it / kmax) % p.H;
    b = it / (kmax * p.H);
    ra = row_append(p, b);
    j = ra.body0 / kGroup + k;
    return k < (ra.body1 - ra.body0) / kGroup;
  };
  // Loads of an item's key and value rows: a block is 4 D 16-byte pieces per tensor, so
  // thread t fetches pieces t and t + 2 D of each; a row still in the ring comes from the
  // cache, a new one from the input.
  uint4 rk0, rk1, rv0, rv1;
  const int ltid = threadIdx.x;  // the loads' thread index (their addresses are cheap)
  auto issue = [&](int it) {
    int b, h, j;
    RowAppend ra;
    item(it, b, h, j, ra);
    const uint64_t* off = p.off + ((size_t)b * p.H + h) * kRegions;
    const size_t in_off = ((size_t)b * p.H + h) * p.n_new * D;
    const uint16_t* kin = reinterpret_cast<const uint16_t*>(p.k_in) + in_off;
    const uint16_t* vin = reinterpret_cast<const uint16_t*>(p.v_in) + in_off;
    const int t0 = p.n_sink + j * kGroup + ltid / (D / 8), t1 = t0 + kGroup / 2, c8 = ltid % (D / 8);
    rk0 = reinterpret_cast<const uint4*>(token_row(p, ra.len0, p.blob + off[RK], kin, t0))[c8];
    rk1 = reinterpret_cast<const uint4*>(token_row(p, ra.len0, p.blob + off[RK], kin, t1))[c8];
    rv0 = reinterpret_cast<const uint4*>(token_row(p, ra.len0, p.blob + off[RV], vin, t0))[c8];
    rv1 = reinterpret_cast<const uint4*>(token_row(p, ra.len0, p.blob + off[RV], vin, t1))[c8];
  };
  auto to_lds = [&]() {
    const int tt = ltid / (D / 8), c8 = ltid % (D / 8);
    reinterpret_cast<uint4*>(&stage[0][tt][0])[c8] = rk0;
    reinterpret_cast<uint4*>(&stage[0][tt + kGroup / 2][0])[c8] = rk1;
    reinterpret_cast<uint4*>(&stage[1][tt][0])[c8] = rv0;
    reinterpret_cast<uint4*>(&stage[1][tt + kGroup / 2][0])[c8] = rv1;
  };
  int it = blockIdx.x;
  if (it >= n_items) return;  // uniform over the workgroup
  issue(it);
  to_lds();
  __syncthreads();
  while (true) {
    const int nxt = it + (int)gridDim.x;
    if (nxt < n_items) issue(nxt);  // in flight while this item is quantized
    // The thread index, opaque to the compiler for this iteration: every address below derives
    // from it, and hoisting those of all widths out of the loop would hold hundreds of
    // registers across it.
    int tid = threadIdx.x;
    __asm__ __volatile__("" : "+v"(tid));
    int b, h, j;
    RowAppend ra;
    const bool live = item(it, b, h, j, ra);
    const uint64_t* off = p.off + ((size_t)b * p.H + h) * kRegions;
    const bool is_key = tid < D;
    const int bits = is_key ? p.k_bits[h] : p.v_bits[h];
    const int vbits = p.v_bits[h];
    const int tile = j >> 1, jj = j & 1;
    // paged caches: the tile's page in this head's pools; an unmapped tile writes nothing and
    // sets flag bit 1 (uniform over the workgroup, as are live and every branch on bits below)
    int ptile = tile;
    bool mapped = true;
    if (live && p.pages) {
      ptile = p.pages[(size_t)b * p.page_stride + tile];
      if (ptile < 0 || ptile >= p.n_pages) {
        if (tid == 0) atomicOr(p.range_flag, 2u);
        mapped = false;
      }
    }
    const int pj = 2 * ptile + jj;  // the block's slot in the body region or pools
    const bool work = live && mapped;
    bool sym = false;
    if (work && bits == 16) {
      // unquantized head: the block's rows are copied
      if (is_key) {
        const int tt = tid / Gd, g = tid % Gd;
        uint4* dst = reinterpret_cast<uint4*>(p.blob + off[KC]) + ((size_t)(pj * kGroup + tt) * D + g * kGroup) / 8;
#pragma unroll
        for (int v = 0; v < 4; ++v) dst[v] = reinterpret_cast<const uint4*>(&stage[0][tt][g * kGroup])[v];
      } else {
        const int c = tid - D;
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.blob + off[VC]);
#pragma unroll
        for (int k = 0; k < 32; ++k) dst[(size_t)(pj * kGroup + k) * D + c] = stage[1][k][c];
      }
    } else if (work) {
      float x[32];
      if (is_key) {
        const int tt = tid / Gd, g = tid % Gd;
        const uint4* s4 = reinterpret_cast<const uint4*>(&stage[0][tt][g * kGroup]);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 u = s4[v];
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            x[v * 8 + 2 * k] = widen16((uint16_t)(w[k] & 0xFFFFu), p.dtype);
            x[v * 8 + 2 * k + 1] = widen16((uint16_t)(w[k] >> 16), p.dtype);
          }
        }
        if (p.key_norm) {  // the group holds k_c / n_c (IEEE fp32 division)
          const float* kn = reinterpret_cast<const float*>(p.blob + off[KN]) + g * kGroup;
#pragma unroll
          for (int i = 0; i < 32; ++i) x[i] = x[i] / kn[i];
        }
      } else {
        const int c = tid - D;
#pragma unroll
        for (int k = 0; k < 32; ++k) x[k] = widen16(stage[1][k][c], p.dtype);
      }
      if (out_of_range(x)) atomicOr(p.range_flag, 1u);
      // the width is uniform over each wavefront (keys: wavefronts 0, 1; values: 2, 3)
      auto group = [&](auto bc) {
        constexpr int B = decltype(bc)::value;
        uint32_t w[B];
        const GroupQ q = quantize_pack<B>(x, hybrid, w);
        sym = q.sym;
        const uint32_t meta = (uint32_t)q.s_bits | ((uint32_t)q.z_bits << 16);
        if (is_key) {
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
          // codes of the 32 tokens, four to a word (the rows of vcodes are 36 bytes apart)
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            uint32_t v4 = 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int pos = (4 * m + u) * B, wi = pos >> 5, o = pos & 31;
              uint32_t cd = w[wi] >> o;
              if (o + B > 32) cd |= w[wi + 1] << (32 - o);
              v4 |= (cd & ((1u << B) - 1u)) << (8 * u);
            }
            reinterpret_cast<uint32_t*>(vcodes[c])[m] = v4;
          }
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
    __syncthreads();  // vcodes complete; every read of the stage done
    if (work && vbits != 16 && !is_key) {
      // value streams of this block: 32 decode lanes (g4 = 2 jj + jp, n) x D/32 streams each
      const int xv = tid - D, nv = D / 32;
      const int lane_local = xv / nv, vg = xv % nv;
      const int jp = lane_local >> 4, n = lane_local & 15;
      const int lane = (2 * jj + jp) * 16 + n;
      uint32_t* dst = reinterpret_cast<uint32_t*>(p.blob + off[VC]) + (size_t)ptile * 2 * D * vbits +
                      ((size_t)lane * nv + vg) * vbits;
      switch (vbits) {
        case 2: pack_value_stream<2>(vcodes, vg, jp, n, dst); break;
        case 3: pack_value_stream<3>(vcodes, vg, jp, n, dst); break;
        case 4: pack_value_stream<4>(vcodes, vg, jp, n, dst); break;
        case 5: pack_value_stream<5>(vcodes, vg, jp, n, dst); break;
        case 6: pack_value_stream<6>(vcodes, vg, jp, n, dst); break;
        case 7: pack_value_stream<7>(vcodes, vg, jp, n, dst); break;
        default: pack_value_stream<8>(vcodes, vg, jp, n, dst); break;
      }
    }
    if (nxt >= n_items) break;
    to_lds();         // the next item's rows, in flight since the top of this iteration
    __syncthreads();  // vcodes free again; the stage holds the next item
    it = nxt;
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
  for (int t = r; t < ra.n; t += parts) {
    const uint4 u = k[(size_t)t * pieces];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[2 * i] = fmaxf(m[2 * i], fabsf(widen16((uint16_t)(w[i] & 0xFFFFu), p.dtype)));
      m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(widen16((uint16_t)(w[i] >> 16), p.dtype)));
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
  // persistent grid: a few workgroups per compute unit, each walking many items
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  const long long items = (long long)p.B * p.H * nblk;
  const unsigned grid = (unsigned)std::min<long long>(items, (long long)kFlushWgPerCu * cus);
  if (p.hybrid)
    hipLaunchKernelGGL(append_flush_kernel<false>, dim3(grid), dim3(2 * p.D), 0, (hipStream_t)stream, p, nblk);
  else
    hipLaunchKernelGGL(append_flush_kernel<true>, dim3(grid), dim3(2 * p.D), 0, (hipStream_t)stream, p, nblk);
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
