// Measurement kernel: the sustained bf16 MFMA rate of the part, for reporting roofline
// fractions against a measured ceiling beside the nominal one.  Every wavefront runs four
// independent chains of v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic in
// the loop) and writes one value per lane so the work stays live.
#include "common.h"

namespace zdit {

namespace {

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(1e-3f * (float)(threadIdx.x + e));
    b[e] = (bf16)(1e-3f * (float)e);
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_peak(int workgroups, int iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace zdit
