// Kernels of the text encoder that only it uses: the token-embedding gather, the per-head
// q/k RMSNorm followed by RoPE over dimension pairs (i, i + 64), and the list of valid rows
// that lets the projections skip the padding.  The encoder's projections,
// pre-norms, attention and residual adds run on the DiT's kernels.
#include <algorithm>

#include "common.h"

namespace zdit {

namespace {

// One thread per 8 elements of an output row: a 16-byte bf16 load, two 16-byte fp32 stores.
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  const int b = blockIdx.y;
  const int chunks = a.dim >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.s_max * chunks) return;
  const int r = (int)(i / chunks), c = (int)(i % chunks);
  float* o = a.out + ((int64_t)b * a.s_max + r) * a.dim + c * 8;
  float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
  if (r < a.len[b]) {
    const int64_t k = (int64_t)b * a.s_max + r;
    const int id = a.n_inline ? a.inline_ids[k] : a.ids[k];
    const uint4 v = *(const uint4*)((const bf16*)a.table + (int64_t)id * a.dim + c * 8);
    // bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 pattern
    lo = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
    hi = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u),
                     __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xFFFF0000u));
  }
  *(float4*)o = lo;
  *(float4*)(o + 4) = hi;
}

// 16 lanes per (row, head): lane j holds dims 8j .. 8j+7.  The partner of dim i < 64 is dim
// i + 64, held by lane j ^ 8 of the same 16-lane group.  Mean of squares reduced over the 16
// lanes in fp32; y = x / sqrt(ms + eps) * g (divided, then scaled); then y_i' = y_i c - y_{i+64} s and
// y_{i+64}' = y_{i+64} c + y_i s with (c, s) of pair i, each product and sum rounded
// separately; one rounding to bf16 at the end.
__global__ __launch_bounds__(256) void qknorm_rope_kernel(QkNormRopeArgs a) {
#pragma clang fp contract(off)
  const int b = blockIdx.y;
  const int nh = a.n_heads + a.n_kv_heads;
  const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int j = threadIdx.x & 15;
  if (item >= (int64_t)a.s_max * nh) return;  // whole 16-lane groups leave together
  const int r = (int)(item / nh), hh = (int)(item % nh);
  if (r >= a.seq_len[b]) return;
  const bool is_q = hh < a.n_heads;
  const int col = is_q ? hh * kHeadDim : a.k_col + (hh - a.n_heads) * kHeadDim;
  bf16* p = (bf16*)a.qkv + ((int64_t)b * a.s_max + r) * a.row_stride + col + j * 8;
  const uint4 raw = *(const uint4*)p;
  float x[8];
  {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m, 64);
  const float den = sqrtf(ss / (float)kHeadDim + a.eps);
  const float* g = (is_q ? a.gq : a.gk) + j * 8;
  float y[8], yp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = x[e] / den * g[e];
#pragma unroll
  for (int e = 0; e < 8; ++e) yp[e] = __shfl_xor(y[e], 8, 64);
  const int64_t tb = (int64_t)b * a.tab_bstride + (int64_t)r * 64 + (j & 7) * 8;
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c = a.cos[tb + e], s = a.sin[tb + e];
    const float t0 = y[e] * c, t1 = yp[e] * s;
    out[e] = (bf16)(j < 8 ? t0 - t1 : t0 + t1);
  }
  *(bf16x8*)p = out;
}

struct RowsArgs {
  int batch, s_max;
  int len[kMaxBatch];
};

// One thread per padded row (b, r): rows below len[b] write their compact index.
__global__ __launch_bounds__(256) void valid_rows_kernel(RowsArgs a, int* rows) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.batch * a.s_max) return;
  const int b = i / a.s_max, r = i - b * a.s_max;
  if (r >= a.len[b]) return;
  int before = 0;
  for (int k = 0; k < b; ++k) before += a.len[k];
  rows[before + r] = i;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

hipError_t launch_embed(const EmbedArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.s_max == 0) return hipSuccess;
  dim3 grid(blocks_for((int64_t)a.s_max * (a.dim >> 3)), a.batch);
  hipLaunchKernelGGL(embed_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_valid_rows(int batch, int s_max, const int* len, int* rows, hipStream_t s) {
  RowsArgs a;
  a.batch = batch; a.s_max = s_max;
  for (int b = 0; b < kMaxBatch; ++b) a.len[b] = b < batch ? len[b] : 0;
  hipLaunchKernelGGL(valid_rows_kernel, dim3(blocks_for((int64_t)batch * s_max)), dim3(256), 0, s, a, rows);
  return hipGetLastError();
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 2048)), dim3(256), 0, s,
                     (uint4*)p, n);
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(const QkNormRopeArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.s_max == 0) return hipSuccess;
  dim3 grid(blocks_for((int64_t)a.s_max * (a.n_heads + a.n_kv_heads) * 16), a.batch);
  hipLaunchKernelGGL(qknorm_rope_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace zdit
