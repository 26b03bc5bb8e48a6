// Calibration kernel: squared quantization error of every group of a calibration slice at
// every candidate bit width (RateQuant: per-quantizer distortion calibration, sections 3.4
// and 4.1). The host sums the per-group float64 errors in group order and fits
// D(b) = alpha * beta^-b. Built with -ffp-contract=off (same quantizer as the append path).
#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "quant_device.h"

namespace kvq {
namespace {

// One thread per (group, bit width, head). Group order: keys (token, channel group);
// values (32-token block, channel).
__global__ __launch_bounds__(256) void calib_kernel(const CalibPlan p) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= p.n_groups) return;
  const int bi = blockIdx.y, h = blockIdx.z;
  const int b = p.b_lo + bi;
  const int D = p.D;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(p.x) + (size_t)h * p.n_tokens * D;
  float v[32];
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
  const GroupQ q = choose_quant(v, b, p.hybrid != 0);
  p.sse[((size_t)h * p.nb + bi) * p.n_groups + gi] = group_sse(v, q);
}

}  // namespace

int launch_calib(const CalibPlan& p, void* stream) {
  const int threads = 256;
  dim3 grid((unsigned)((p.n_groups + threads - 1) / threads), p.nb, p.n_heads);
  hipLaunchKernelGGL(calib_kernel, grid, dim3(threads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace kvq
