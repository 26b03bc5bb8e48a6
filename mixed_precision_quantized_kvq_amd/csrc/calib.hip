// Calibration kernel: squared quantization error of every group of a calibration slice at
// every candidate bit width (RateQuant: per-quantizer distortion calibration, sections 3.4
// and 4.1), summed per (head, bit width). The host adds the per-workgroup sums in order and
// fits D(b) = alpha * beta^-b. Built with -ffp-contract=off (same quantizer as the append
// path).
#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "quant_device.h"

namespace kvq {
namespace {

// One thread per (group, head): it loads its 32 elements once and evaluates every width
// b_lo..b_hi. Group order: keys (token, channel group); values (32-token block, channel).
// Each workgroup adds its groups' float64 errors per width in a fixed order (a butterfly
// within each wavefront, then the wavefronts in order) and writes one sum per width:
// part[head][width][workgroup].
template <bool ASYM>
__device__ __forceinline__ void calib_body(const CalibPlan& p) {
  __shared__ double wsum[kCalibThreads / 64][8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gi = (int64_t)blockIdx.x * kCalibThreads + tid;
  const int h = blockIdx.y;
  const bool live = gi < p.n_groups;
  const int D = p.D;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(p.x) + (size_t)h * p.n_tokens * D;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  if (live) {
    if (p.axis == KVQ_AXIS_KEY) {
      const int64_t t = gi / (D / kGroup);
      const int g = (int)(gi % (D / kGroup));
      const uint16_t* row = x + (size_t)t * D + g * kGroup;
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = widen16(row[i], p.dtype);
    } else {
      const int64_t jb = gi / D;
      const int c = (int)(gi % D);
      const uint16_t* col = x + (size_t)jb * kGroup * D + c;
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = widen16(col[(size_t)i * D], p.dtype);
    }
    if (out_of_range(v)) atomicOr(p.range_flag, 1u);
  }
  for (int bi = 0; bi < p.nb; ++bi) {
    double e = live ? group_sse(v, choose_quant(v, p.b_lo + bi, !ASYM && p.hybrid != 0)) : 0.0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) e = e + __shfl_xor(e, o, 64);
    if (lane == 0) wsum[wave][bi] = e;
  }
  __syncthreads();
  if (tid < p.nb) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kCalibThreads / 64; ++w) tot = tot + wsum[w][tid];
    p.part[((size_t)h * p.nb + tid) * p.n_blocks + blockIdx.x] = tot;
  }
}

// Two kernels: the hybrid choice's registers (248 VGPRs) would keep the asymmetric one, which
// fits 3 wavefronts per SIMD, at 2.
__global__ __launch_bounds__(kCalibThreads) void calib_kernel(const CalibPlan p) { calib_body<false>(p); }
__global__ __launch_bounds__(kCalibThreads) __attribute__((amdgpu_waves_per_eu(3))) void calib_kernel_asym(
    const CalibPlan p) {
  calib_body<true>(p);
}

}  // namespace

int launch_calib(const CalibPlan& p, void* stream) {
  dim3 grid((unsigned)p.n_blocks, (unsigned)p.n_heads);
  if (p.hybrid)
    hipLaunchKernelGGL(calib_kernel, grid, dim3(kCalibThreads), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(calib_kernel_asym, grid, dim3(kCalibThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace kvq
