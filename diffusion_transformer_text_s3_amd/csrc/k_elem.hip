// Bandwidth-bound kernels of the S3-DiT path on gfx950: RMSNorm + adaLN modulation, RoPE
// (bit-exact real interleaved form) and its tables, patchify / unpatchify, learned caption
// pad, the negated-CFG Euler update, the timestep MLP and the adaLN projection.
//
// Every kernel reads and writes with 16-byte (or wider) coalesced accesses where the layout
// allows, reduces in fp32 across a 64-wide wavefront, and never writes fp16.
#include "common.h"

namespace zdit {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T> __device__ __forceinline__ T to_act(float v);
template <> __device__ __forceinline__ float to_act<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 to_act<bf16>(float v) { return (bf16)v; }

template <typename T> __device__ __forceinline__ float from_act(T v);
template <> __device__ __forceinline__ float from_act<float>(float v) { return v; }
template <> __device__ __forceinline__ float from_act<bf16>(bf16 v) { return (float)v; }

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// ---------------------------------------------------------------------------------------
// RMSNorm (fp32 reduction) * gain * (1 + scale) + shift.  A workgroup of 4 wavefronts takes 4
// rows of one branch; gain, shift and scale of that branch are staged in LDS once, then each
// wavefront normalises one row, keeping it in registers (dim <= 4096: at most 16 float4 per
// lane).  One row per wavefront keeps more rows in flight than a wavefront looping over rows
// (55 against 61 us at 8320 x 3840 with 4 rows per wavefront, same box).  Four wavefronts per
// workgroup rather than 8: with ~150 registers a CU holds 12 wavefronts and with 46 KB of
// staged vectors 3 workgroups, so 4-wave workgroups fill it where 8-wave ones leave it at 8
// (8320 x 3840: 47.5 -> 41.5 us; 16 waves 61.5 us).
// ---------------------------------------------------------------------------------------
constexpr int kNormMaxChunks = 16;
constexpr int kNormRowsPerBlock = 4;

// STAGED: 4 rows per workgroup with gain / shift / scale staged in LDS (many rows).  Else one
// row per wavefront, 4 per workgroup, the vectors read from global memory where they stay in
// L2 (few rows: more workgroups, no staging to amortise).
constexpr int kNormWaves = 4;

template <typename TO, bool STAGED>
__global__ __launch_bounds__(STAGED ? 64 * kNormWaves : 256) void rmsnorm_mod_kernel(NormArgs a) {
  constexpr int kRows = STAGED ? kNormRowsPerBlock : 4;
  constexpr int kW = STAGED ? kNormWaves : 4;
  constexpr int kT = 64 * kW;
  __shared__ float4 vg_[STAGED ? 1024 : 1], vsh_[STAGED ? 1024 : 1], vsc_[STAGED ? 1024 : 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int nchunk = a.dim >> 2;
  const bool mod = a.shift != nullptr;
  const float4* vg = (const float4*)a.gain;
  const float4* vsh = mod ? (const float4*)(a.shift + b * a.mod_bstride) : nullptr;
  const float4* vsc = mod ? (const float4*)(a.scale + b * a.mod_bstride) : nullptr;
  if constexpr (STAGED) {
    for (int c = threadIdx.x; c < nchunk; c += kT) {
      vg_[c] = vg[c];
      if (mod) { vsh_[c] = vsh[c]; vsc_[c] = vsc[c]; }
    }
    __syncthreads();
    vg = vg_; vsh = vsh_; vsc = vsc_;
  }
  for (int i = 0; i < kRows / kW; ++i) {
    const int r = blockIdx.x * kRows + i * kW + wave;
    if (r >= a.rows_per_batch) break;
    const int64_t m = (int64_t)b * a.rows_per_batch + r;
    TO* out = (TO*)a.out + m * a.dim;
    if (r >= a.valid[b]) {
      for (int c = lane; c < nchunk; c += 64) {
        out[4 * c + 0] = to_act<TO>(0.f); out[4 * c + 1] = to_act<TO>(0.f);
        out[4 * c + 2] = to_act<TO>(0.f); out[4 * c + 3] = to_act<TO>(0.f);
      }
      continue;
    }
    const float4* x = (const float4*)(a.x + b * a.x_bstride + (int64_t)r * a.dim);
    // Every load is issued before the first is used: the index is clamped into the row (a lane
    // past its end reloads the last chunk) and the value zeroed by a select, so no branch
    // separates the loads (guarded loads made the compiler wait for each one in turn).  Adding
    // the zeros leaves the sum of squares unchanged, term for term.
    float4 v[kNormMaxChunks];
#pragma unroll
    for (int j = 0; j < kNormMaxChunks; ++j) v[j] = x[min(lane + 64 * j, nchunk - 1)];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kNormMaxChunks; ++j) {
      if (lane + 64 * j >= nchunk) v[j] = float4{0.f, 0.f, 0.f, 0.f};
      ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    }
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / (float)a.dim + a.eps);
    // gain / shift / scale of four chunks at a time, loaded together (clamped like x)
#pragma unroll
    for (int j0 = 0; j0 < kNormMaxChunks; j0 += 4) {
      float4 gg[4], s1[4], s2[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = min(lane + 64 * (j0 + q), nchunk - 1);
        gg[q] = vg[c];
        if (mod) { s1[q] = vsh[c]; s2[q] = vsc[c]; }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = lane + 64 * (j0 + q);
        if (c >= nchunk) continue;
        const float4 w = v[j0 + q];
        float4 o;
        o.x = w.x * rinv * gg[q].x; o.y = w.y * rinv * gg[q].y;
        o.z = w.z * rinv * gg[q].z; o.w = w.w * rinv * gg[q].w;
        if (mod) {
          o.x = o.x * (1.f + s2[q].x) + s1[q].x; o.y = o.y * (1.f + s2[q].y) + s1[q].y;
          o.z = o.z * (1.f + s2[q].z) + s1[q].z; o.w = o.w * (1.f + s2[q].w) + s1[q].w;
        }
        if constexpr (sizeof(TO) == 2) {
          bf16x4 ob = {(bf16)o.x, (bf16)o.y, (bf16)o.z, (bf16)o.w};
          *(bf16x4*)(out + 4 * c) = ob;
        } else {
          *(float4*)(out + 4 * c) = o;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// RoPE on q and k of a fused qkv row.  One thread turns 4 pairs (8 values) of one head row.
// Products and sums are rounded separately (no FMA contraction).
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
#pragma clang fp contract(off)
  const int b = blockIdx.y;
  const int units_per_row = 2 * a.n_heads * 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.s_max * units_per_row) return;
  const int s = (int)(idx / units_per_row);
  const int u = (int)(idx % units_per_row);
  if (s >= a.seq_len[b]) return;
  const int hh = u >> 4, unit = u & 15;
  const int D = a.n_heads * kHeadDim;
  T* p = (T*)a.qkv + ((int64_t)b * a.s_max + s) * 3 * D + hh * kHeadDim + unit * 8;
  const float4 c = *(const float4*)(a.cos + b * a.tab_bstride + (int64_t)s * 64 + unit * 4);
  const float4 sn = *(const float4*)(a.sin + b * a.tab_bstride + (int64_t)s * 64 + unit * 4);
  float x[8];
  if constexpr (sizeof(T) == 2) {
    bf16x8 v = *(const bf16x8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  } else {
    float4 v0 = *(const float4*)p, v1 = *(const float4*)(p + 4);
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
  }
  const float cc[4] = {c.x, c.y, c.z, c.w};
  const float ss[4] = {sn.x, sn.y, sn.z, sn.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = x[2 * i], x1 = x[2 * i + 1];
    const float p0 = x0 * cc[i];
    const float p1 = x1 * ss[i];
    const float p2 = x0 * ss[i];
    const float p3 = x1 * cc[i];
    y[2 * i] = p0 - p1;
    y[2 * i + 1] = p2 + p3;
  }
  if constexpr (sizeof(T) == 2) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)y[i];
    *(bf16x8*)p = o;
  } else {
    *(float4*)p = make_float4(y[0], y[1], y[2], y[3]);
    *(float4*)(p + 4) = make_float4(y[4], y[5], y[6], y[7]);
  }
}

// ---------------------------------------------------------------------------------------
// RoPE tables: angles and cos/sin in double, stored fp32.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_tables_kernel(RopeTabArgs a) {
  const int b = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int npairs = (a.axes[0] + a.axes[1] + a.axes[2]) / 2;
  if (idx >= (int64_t)a.s_max * npairs) return;
  const int s = (int)(idx / npairs), k = (int)(idx % npairs);
  const int nimg = a.grid_h * a.grid_w;
  int len, pos[3] = {0, 0, 0};
  if (a.kind == 0) {  // image
    len = nimg;
    pos[1] = s / a.grid_w; pos[2] = s % a.grid_w;
  } else if (a.kind == 1) {  // caption
    len = a.n_cap[b];
    pos[0] = 1 + s;
  } else if (a.kind == 3) {  // text encoder tokens: position = index from 0
    len = a.n_cap[b];
    pos[0] = s;
  } else {  // joint: image tokens then caption tokens
    len = nimg + a.n_cap[b];
    if (s < nimg) { pos[1] = s / a.grid_w; pos[2] = s % a.grid_w; }
    else pos[0] = 1 + (s - nimg);
  }
  float cv = 1.f, sv = 0.f;
  if (s < len) {
    int axis = 0, p = k;
    if (p >= a.axes[0] / 2) { p -= a.axes[0] / 2; axis = 1;
      if (p >= a.axes[1] / 2) { p -= a.axes[1] / 2; axis = 2; } }
    const double omega = pow((double)a.theta, -2.0 * (double)p / (double)a.axes[axis]);
    const double ang = (double)pos[axis] * omega;
    cv = (float)cos(ang);
    sv = (float)sin(ang);
  }
  const int64_t o = ((int64_t)b * a.s_max + s) * npairs + k;
  a.cos[o] = cv;
  a.sin[o] = sv;
}

// ---------------------------------------------------------------------------------------
// patchify / unpatchify (2x2 patch), feature f = (dy*2 + dx)*C + ch, token r*(w/2) + c
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void patchify_kernel(int C, int h, int w, const float* lat,
                                                        int64_t lat_bstride, T* tokens) {
  const int b = blockIdx.y;
  const int gw = w / 2, ntok = (h / 2) * gw, F = 4 * C;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)ntok * F) return;
  const int n = (int)(idx / F), f = (int)(idx % F);
  const int r = n / gw, c = n % gw;
  const int q = f / C, ch = f % C;
  const int dy = q >> 1, dx = q & 1;
  const float v = lat[b * lat_bstride + ((int64_t)ch * h + 2 * r + dy) * w + 2 * c + dx];
  tokens[(int64_t)b * ntok * F + idx] = to_act<T>(v);
}

__global__ __launch_bounds__(256) void unpatchify_kernel(int C, int h, int w, const float* tokens,
                                                          float* lat) {
  const int b = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)C * h * w) return;
  const int ch = (int)(idx / ((int64_t)h * w));
  const int rem = (int)(idx % ((int64_t)h * w));
  const int y = rem / w, x = rem % w;
  const int gw = w / 2, ntok = (h / 2) * gw, F = 4 * C;
  const int n = (y >> 1) * gw + (x >> 1);
  const int f = ((y & 1) * 2 + (x & 1)) * C + ch;
  lat[(int64_t)b * C * h * w + idx] = tokens[((int64_t)b * ntok + n) * F + f];
}

// Learned caption pad: rows row0 + j, cap_len[b] <= j < round_up(cap_len[b], multiple).
struct PadArgs { int cap_len[kMaxBatch]; };
__global__ __launch_bounds__(256) void cap_pad_kernel(int s_max, int dim, int row0, int multiple,
                                                       PadArgs pa, const float* pad, float* x) {
  const int b = blockIdx.z;
  const int j = blockIdx.y;
  const int L = pa.cap_len[b];
  const int nc = ((L + multiple - 1) / multiple) * multiple;
  if (j < L || j >= nc) return;
  float* row = x + ((int64_t)b * s_max + row0 + j) * dim;
  for (int k = blockIdx.x * 256 + threadIdx.x; k < dim; k += gridDim.x * 256) row[k] = pad[k];
}

template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* in, T* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = to_act<T>(in[i]);
}

// ---------------------------------------------------------------------------------------
// Negated CFG + Euler (+ decode unscale), fp32, products and sums rounded separately.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void euler_kernel(float* x, const float* vc, const float* vu,
                                                     int64_t n, float g, float sigma,
                                                     float sigma_next, float* dec) {
#pragma clang fp contract(off)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float pos = vc[i];
  float np;
  if (vu) {
    const float dd = pos - vu[i];
    const float e = g * dd;
    const float u = pos + e;
    np = -u;
  } else {
    np = -pos;
  }
  const float ds = sigma_next - sigma;
  const float step = ds * np;
  const float xn = x[i] + step;
  x[i] = xn;
  if (dec) {
    const float q = xn / 0.3611f;
    dec[i] = q + 0.1159f;
  }
}

// ---------------------------------------------------------------------------------------
// Timestep MLP: c = W2 SiLU(W1 e + b1) + b2; one block per branch.
// ---------------------------------------------------------------------------------------
struct TArgs { float t[kMaxBatch]; };
__global__ __launch_bounds__(256) void temb_kernel(TArgs ta, int t_freq, int c_dim, float t_scale,
                                                    const float* w1, const float* b1,
                                                    const float* w2, const float* b2, float* c) {
  __shared__ float e[1024];
  __shared__ float hd[1024];
  const int b = blockIdx.x;
  const int half = t_freq / 2;
  const float tau = ta.t[b] * t_scale;
  for (int k = threadIdx.x; k < half; k += blockDim.x) {
    const float f = powf(10000.0f, -(float)k / (float)half);
    const float arg = tau * f;
    e[k] = cosf(arg);
    e[half + k] = sinf(arg);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < c_dim; j += blockDim.x) {
    float acc = 0.f;
    const float* wr = w1 + (int64_t)j * t_freq;
    for (int k = 0; k < t_freq; ++k) acc += wr[k] * e[k];
    hd[j] = silu(acc + b1[j]);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < c_dim; j += blockDim.x) {
    float acc = 0.f;
    const float* wr = w2 + (int64_t)j * c_dim;
    for (int k = 0; k < c_dim; ++k) acc += wr[k] * hd[k];
    c[(int64_t)b * c_dim + j] = acc + b2[j];
  }
}

// ---------------------------------------------------------------------------------------
// adaLN projection out[b, j] = sum_k W[j, k] SiLU(c[b, k]) + bias[j], all branches at once,
// SiLU(c) staged in LDS.  Weight rows are read coalesced: a group of L lanes (L a power of two,
// 8 L >= min(c_dim, 512)) covers one row in 8-element chunks, a wavefront 64 / L rows at a
// time, each lane with ADA_U rows' loads in flight; the group's partial sums meet by xor
// shuffles.
// ---------------------------------------------------------------------------------------
constexpr int ADA_U = 4;

// Several projections of the same c in one launch: blockIdx.y selects one (weights, bias,
// output) triple.
struct AdaJobs {
  const void* w[kMaxAdaJobs];
  const float* b[kMaxAdaJobs];
  float* out[kMaxAdaJobs];
};

template <typename TW>
__global__ __launch_bounds__(256) void adaln_kernel(int batch, int c_dim, int n_out, int lanes_per_row,
                                                     const float* c, AdaJobs jobs) {
  const TW* w = (const TW*)jobs.w[blockIdx.y];
  const float* bias = jobs.b[blockIdx.y];
  float* out = jobs.out[blockIdx.y];
  extern __shared__ float sc[];  // [batch][c_dim]
  for (int i = threadIdx.x; i < batch * c_dim; i += blockDim.x) sc[i] = silu(c[i]);
  __syncthreads();
  const int L = lanes_per_row, R = 64 / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane / L, li = lane % L;
  const int row0 = (blockIdx.x * 4 + wave) * R * ADA_U + g;  // rows row0 + u R
  float acc[ADA_U][kMaxBatch];
#pragma unroll
  for (int u = 0; u < ADA_U; ++u)
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) acc[u][b] = 0.f;
  for (int k = li * 8; k < c_dim; k += L * 8) {
    float wv[ADA_U][8];
#pragma unroll
    for (int u = 0; u < ADA_U; ++u) {
      const int row = row0 + u * R;
      const TW* wr = w + (int64_t)min(row, n_out - 1) * c_dim + k;
      if constexpr (sizeof(TW) == 2) {
        const bf16x8 v = *(const bf16x8*)wr;
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[u][i] = (float)v[i];
      } else {
        const float4 v0 = *(const float4*)wr, v1 = *(const float4*)(wr + 4);
        wv[u][0] = v0.x; wv[u][1] = v0.y; wv[u][2] = v0.z; wv[u][3] = v0.w;
        wv[u][4] = v1.x; wv[u][5] = v1.y; wv[u][6] = v1.z; wv[u][7] = v1.w;
      }
    }
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      if (b < batch) {
        const float4 s0 = *(const float4*)(sc + b * c_dim + k), s1 = *(const float4*)(sc + b * c_dim + k + 4);
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int u = 0; u < ADA_U; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[u][b] += wv[u][i] * sv[i];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < ADA_U; ++u) {
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      if (b < batch) {
        for (int m = L >> 1; m >= 1; m >>= 1) acc[u][b] += __shfl_xor(acc[u][b], m, 64);
      }
    }
    const int row = row0 + u * R;
    if (li == 0 && row < n_out) {
      const float bj = bias[row];
#pragma unroll
      for (int b = 0; b < kMaxBatch; ++b)
        if (b < batch) out[(int64_t)b * n_out + row] = acc[u][b] + bj;
    }
  }
}

__global__ __launch_bounds__(256) void copy_rows_kernel(const float4* src, int64_t src_bstride4,
                                                         float4* dst, int64_t dst_bstride4,
                                                         int64_t n4) {
  const int b = blockIdx.y;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    dst[b * dst_bstride4 + i] = src[b * src_bstride4 + i];
}

inline unsigned blocks_for(int64_t n, int per = 256) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_rmsnorm_mod(int precision, const NormArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.rows_per_batch;
  if (rows == 0) return hipSuccess;
  if (rows >= 2048) {
    dim3 grid((a.rows_per_batch + kNormRowsPerBlock - 1) / kNormRowsPerBlock, a.batch);
    if (precision == 0) hipLaunchKernelGGL((rmsnorm_mod_kernel<bf16, true>), grid, dim3(64 * kNormWaves), 0, s, a);
    else hipLaunchKernelGGL((rmsnorm_mod_kernel<float, true>), grid, dim3(64 * kNormWaves), 0, s, a);
  } else {
    dim3 grid((a.rows_per_batch + 3) / 4, a.batch);
    if (precision == 0) hipLaunchKernelGGL((rmsnorm_mod_kernel<bf16, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rmsnorm_mod_kernel<float, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_rope(int precision, const RopeArgs& a, hipStream_t s) {
  dim3 grid(blocks_for((int64_t)a.s_max * 2 * a.n_heads * 16), a.batch);
  if (precision == 0) hipLaunchKernelGGL(rope_kernel<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rope_tables(const RopeTabArgs& a, hipStream_t s) {
  const int npairs = (a.axes[0] + a.axes[1] + a.axes[2]) / 2;
  dim3 grid(blocks_for((int64_t)a.s_max * npairs), a.batch);
  hipLaunchKernelGGL(rope_tables_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_patchify(int precision, int batch, int C, int h, int w, const float* lat,
                           int64_t lat_bstride, void* tokens, hipStream_t s) {
  const int64_t n = (int64_t)(h / 2) * (w / 2) * 4 * C;
  dim3 grid(blocks_for(n), batch);
  if (precision == 0)
    hipLaunchKernelGGL(patchify_kernel<bf16>, grid, dim3(256), 0, s, C, h, w, lat, lat_bstride, (bf16*)tokens);
  else
    hipLaunchKernelGGL(patchify_kernel<float>, grid, dim3(256), 0, s, C, h, w, lat, lat_bstride, (float*)tokens);
  return hipGetLastError();
}

hipError_t launch_unpatchify(int batch, int C, int h, int w, const float* tokens, float* lat,
                             hipStream_t s) {
  dim3 grid(blocks_for((int64_t)C * h * w), batch);
  hipLaunchKernelGGL(unpatchify_kernel, grid, dim3(256), 0, s, C, h, w, tokens, lat);
  return hipGetLastError();
}

hipError_t launch_cap_pad(int batch, int s_max, int dim, int row0, const int* cap_len,
                          int multiple, const float* pad, float* x, hipStream_t s) {
  PadArgs pa;
  int maxnc = 0;
  for (int b = 0; b < batch; ++b) {
    pa.cap_len[b] = cap_len[b];
    const int nc = ((cap_len[b] + multiple - 1) / multiple) * multiple;
    if (nc > maxnc) maxnc = nc;
  }
  if (maxnc == 0) return hipSuccess;
  dim3 grid(blocks_for(dim), maxnc, batch);
  hipLaunchKernelGGL(cap_pad_kernel, grid, dim3(256), 0, s, s_max, dim, row0, multiple, pa, pad, x);
  return hipGetLastError();
}

hipError_t launch_convert(int precision, const float* in, void* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (precision == 0) hipLaunchKernelGGL(convert_kernel<bf16>, dim3(blocks_for(n)), dim3(256), 0, s, in, (bf16*)out, n);
  else hipLaunchKernelGGL(convert_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, s, in, (float*)out, n);
  return hipGetLastError();
}

hipError_t launch_euler(float* x, const float* vc, const float* vu, int64_t n, float g,
                        float sigma, float sigma_next, float* dec, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(euler_kernel, dim3(blocks_for(n)), dim3(256), 0, s, x, vc, vu, n, g, sigma,
                     sigma_next, dec);
  return hipGetLastError();
}

hipError_t launch_temb(int batch, const float* t, int t_freq, int c_dim, float t_scale,
                       const float* w1, const float* b1, const float* w2, const float* b2,
                       float* c, hipStream_t s) {
  TArgs ta;
  for (int b = 0; b < batch; ++b) ta.t[b] = t[b];
  hipLaunchKernelGGL(temb_kernel, dim3(batch), dim3(256), 0, s, ta, t_freq, c_dim, t_scale, w1,
                     b1, w2, b2, c);
  return hipGetLastError();
}

hipError_t launch_adaln_multi(int precision, int batch, int c_dim, int n_out, const float* c, const void* const* w,
                              const float* const* b, float* const* out, int n_jobs, hipStream_t s) {
  if (n_jobs < 1 || n_jobs > kMaxAdaJobs) return hipErrorInvalidValue;
  AdaJobs jobs{};
  for (int i = 0; i < n_jobs; ++i) { jobs.w[i] = w[i]; jobs.b[i] = b[i]; jobs.out[i] = out[i]; }
  const size_t shm = (size_t)batch * c_dim * sizeof(float);
  int L = 1;
  while (L < 64 && 8 * L < c_dim) L <<= 1;
  const int rows_per_block = 4 * (64 / L) * ADA_U;
  dim3 grid((unsigned)((n_out + rows_per_block - 1) / rows_per_block), (unsigned)n_jobs);
  if (precision == 0)
    hipLaunchKernelGGL(adaln_kernel<bf16>, grid, dim3(256), shm, s, batch, c_dim, n_out, L, c, jobs);
  else
    hipLaunchKernelGGL(adaln_kernel<float>, grid, dim3(256), shm, s, batch, c_dim, n_out, L, c, jobs);
  return hipGetLastError();
}

hipError_t launch_adaln(int precision, int batch, int c_dim, int n_out, const float* c,
                        const void* w, const float* b, float* out, hipStream_t s) {
  return launch_adaln_multi(precision, batch, c_dim, n_out, c, &w, &b, &out, 1, s);
}

hipError_t launch_copy_rows(const float* src, int64_t src_bstride, float* dst,
                            int64_t dst_bstride, int batch, int64_t n, hipStream_t s) {
  if (n == 0 || batch == 0) return hipSuccess;
  const int64_t n4 = n / 4;
  unsigned g = blocks_for(n4);
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(g, batch), dim3(256), 0, s, (const float4*)src,
                     src_bstride / 4, (float4*)dst, dst_bstride / 4, n4);
  return hipGetLastError();
}

}  // namespace zdit
