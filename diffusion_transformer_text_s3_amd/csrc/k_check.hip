// Opt-in non-finite detection (ZDIT_CHECK_FINITE).  The activations of this model outgrow half
// precision (residual stream near 6.7e3, w2 / out-projection outputs near 3.1e5; an fp16 run of
// the DiT turns to NaN by the second sampler step: Core AI model zoo, "Z-Image-Turbo port",
// section "fp16 does not work. bf16 does."), so a debug run can ask the library where the first
// NaN or infinity appeared: each checkpoint of a call scans a buffer's valid rows and raises its
// flag, and a latch records the first (step, checkpoint) whose flag is set.  Nothing here runs
// unless the flag is set in zdit_dims.
#include <algorithm>

#include "common.h"

namespace zdit {

namespace {

// Non-finite: the exponent bits all set (NaN or +-Inf).
__device__ __forceinline__ bool bad(float v) { return (__float_as_uint(v) & 0x7f800000u) == 0x7f800000u; }

// One thread per 4 consecutive values of a valid row; a wavefront that saw one raises the flag
// with a plain store (every writer stores the same 1).
__global__ __launch_bounds__(256) void finite_check_kernel(FiniteArgs a) {
  const int q = a.width >> 2;  // float4 per row
  const int64_t per_branch = (int64_t)a.rows_per_batch * q;
  const int64_t total = per_branch * a.batch;
  bool hit = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int b = (int)(i / per_branch);
    const int64_t rem = i - b * per_branch;
    const int r = (int)(rem / q), c = (int)(rem - (int64_t)r * q);
    if (r >= a.valid[b]) continue;
    const float4 v = *(const float4*)(a.p + b * a.bstride + (int64_t)r * a.ld + 4 * c);
    hit |= bad(v.x) | bad(v.y) | bad(v.z) | bad(v.w);
  }
  if (__any(hit) && (threadIdx.x & 63) == 0) *a.flag = 1;
}

// Sequential: the first set flag of this call, if no earlier one was latched; then the flags
// are cleared for the next step.
__global__ __launch_bounds__(64) void finite_latch_kernel(int* flags, int n, int step, int* first) {
  if (threadIdx.x != 0) return;
  if (first[0] < 0) {
    for (int k = 0; k < n; ++k)
      if (flags[k]) {
        first[0] = step;
        first[1] = k;
        break;
      }
  }
  for (int k = 0; k < n; ++k) flags[k] = 0;
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int* p, int n, int v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_finite_check(const FiniteArgs& a, hipStream_t s) {
  const int64_t n4 = (int64_t)a.batch * a.rows_per_batch * (a.width >> 2);
  if (n4 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(finite_check_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finite_latch(int* flags, int n, int step, int* first, hipStream_t s) {
  hipLaunchKernelGGL(finite_latch_kernel, dim3(1), dim3(64), 0, s, flags, n, step, first);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, int n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace zdit
