// Matrix-core rate probe. Eight independent bf16 32x32x16 MFMA chains per
// wave with every operand in registers, so only the matrix cores bound it:
// the rate it reaches is what the chip sustains at the clock it holds under
// MFMA load, the ceiling the attention kernels are also quoted against
// (besides the published dense peak). It computes nothing of the method.
#include "device_common.h"
#include "kernels.h"

namespace calibatt {

constexpr int kProbeChains = 8;

__global__ void __launch_bounds__(kThreads) mfma_probe_kernel(float* sink, int64_t iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(lane + i));
    b[i] = (__bf16)(1e-3f * (float)(lane - i));
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = f32x16{};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  // The sums are data the compiler cannot see through; the store keeps the
  // chains live and practically never happens.
  if (s == 1234.5f) sink[0] = s;
}

hipError_t launch_mfma_probe(float* sink, int64_t iters, int32_t workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(kThreads), 0, stream, sink, iters);
  return hipGetLastError();
}

}  // namespace calibatt
