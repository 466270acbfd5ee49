// Joint (bidirectional) softmax attention over the single-stream sequence, head_dim 128,
// ragged per branch: keys j >= seq_len[b] are masked (batch-alignment padding), every key
// below it (image tokens, caption tokens and learned caption pads) is context.
//
// bf16 path on gfx950.  A 256-thread workgroup owns 128 queries of one (branch, head); each
// wavefront owns 32 of them and keeps their 128-dim rows in registers as MFMA B operands.
// Key blocks of 64 are staged in LDS: K as [key][dim] and V as [dim][key] (V is transposed
// once per layer by vtrans_kernel).  Scores are formed transposed, S^T = K Q^T, so each lane
// holds 32 scores of a single query: the running max needs one cross-lane step (lane ^ 32)
// and the rescale of the output accumulator is a per-lane scalar.  The output is formed
// transposed too, O^T += V^T P^T, where the bf16 P^T operand is taken straight from the
// score registers: in a 32x32 MFMA result, lane half h holds keys {8g + 4h + 0..3}, so for
// each group of 16 keys both operands use the key order {4h..4h+3, 8+4h..8+4h+3}.
// Online softmax in fp32 with exp2 and the 1/sqrt(128) scale folded into log2(e).
#include "common.h"

namespace zdit {

namespace {

constexpr int QT = 128;  // queries per workgroup
constexpr int KT = 64;   // keys per LDS block
constexpr int KROW = 17; // 16-byte chunks per K row in LDS (16 + 1 pad)
constexpr int VROW = 9;  // 16-byte chunks per V^T row in LDS (8 + 1 pad)

__global__ __launch_bounds__(256) void vtrans_kernel(AttnArgs a) {
  __shared__ uint4 t[64 * KROW];
  const int b = blockIdx.z, h = blockIdx.y, s0 = blockIdx.x * 64;
  const int D = a.n_heads * kHeadDim;
  const int S = a.seq_len[b];
  const bf16* qkv = (const bf16*)a.qkv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int tok = c >> 4, dc = c & 15;
    const int s = s0 + tok;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (s < S) v = *(const uint4*)(qkv + ((int64_t)b * a.s_max + s) * 3 * D + 2 * D + h * kHeadDim + dc * 8);
    t[tok * KROW + dc] = v;
  }
  __syncthreads();
  const bf16* tb = (const bf16*)t;
  bf16* vt = (bf16*)a.vt + ((int64_t)(b * a.n_heads + h) * kHeadDim) * a.s_pad;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int d = c >> 3, sc = c & 7;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = tb[(sc * 8 + e) * (KROW * 8) + d];
    *(bf16x8*)(vt + (int64_t)d * a.s_pad + s0 + sc * 8) = o;
  }
}

__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  __shared__ uint4 Ks[KT * KROW];
  __shared__ uint4 Vs[kHeadDim * VROW];
  const int b = blockIdx.z, h = blockIdx.y, q0 = blockIdx.x * QT;
  const int D = a.n_heads * kHeadDim;
  const int S = a.seq_len[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int q = q0 + wave * 32 + fr;
  const bf16* qkv = (const bf16*)a.qkv;
  bf16* out = (bf16*)a.out;

  if (q0 >= S) {  // whole tile is padding: write zeros
    for (int i = tid; i < QT * 16; i += 256) {
      const int r = q0 + (i >> 4), c = i & 15;
      if (r < a.s_max) *(uint4*)(out + ((int64_t)b * a.s_max + r) * D + h * kHeadDim + c * 8) = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  bf16x8 qf[8];
  {
    const bf16* qp = qkv + ((int64_t)b * a.s_max + min(q, S - 1)) * 3 * D + h * kHeadDim + 8 * fh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
  }

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = 1.4426950408889634f / sqrtf((float)kHeadDim);
  const int nkt = (S + KT - 1) / KT;
  const bf16* vt = (const bf16*)a.vt + ((int64_t)(b * a.n_heads + h) * kHeadDim) * a.s_pad;
  const bf16* Vb = (const bf16*)Vs;

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * KT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int key = c >> 4, dc = c & 15;
      const int kk = k0 + key;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kk < S) v = *(const uint4*)(qkv + ((int64_t)b * a.s_max + kk) * 3 * D + D + h * kHeadDim + dc * 8);
      Ks[key * KROW + dc] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int d = c >> 3, kc = c & 7;
      Vs[d * VROW + kc] = *(const uint4*)(vt + (int64_t)d * a.s_pad + k0 + kc * 8);
    }
    __syncthreads();

    f32x16 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[t][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, Ks[(t * 32 + fr) * KROW + 2 * s + fh]);
        st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[t], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + t * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
        const float v = (key < S) ? st[t][r] * sc : -INFINITY;
        st[t][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    bf16x8 pb[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(st[t][r] - m_new);
        l_run += p;
        pb[t][r >> 3][r & 7] = (bf16)p;
      }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16* vrow = Vb + (dt * 32 + fr) * (VROW * 8);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int base = t * 32 + 16 * j + 4 * fh;
          const bf16x4 lo = *(const bf16x4*)(vrow + base);
          const bf16x4 hi = *(const bf16x4*)(vrow + base + 8);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t][j], o[dt], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l;
  if (q < a.s_max) {
    bf16* op = out + ((int64_t)b * a.s_max + q) * D + h * kHeadDim;
    const bool valid = q < S;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = valid ? (bf16)(o[dt][4 * gq + e] * inv) : (bf16)0.f;
        *(bf16x4*)(op + dt * 32 + 8 * gq + 4 * fh) = v;
      }
  }
}

// fp32 debug attention: one wavefront per (query, head, branch); lane owns dims 2l, 2l+1.
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const int b = blockIdx.z, h = blockIdx.y, q = blockIdx.x, lane = threadIdx.x;
  const int D = a.n_heads * kHeadDim;
  const int S = a.seq_len[b];
  const float* qkv = (const float*)a.qkv;
  float* op = (float*)a.out + ((int64_t)b * a.s_max + q) * D + h * kHeadDim + 2 * lane;
  if (q >= S) { op[0] = 0.f; op[1] = 0.f; return; }
  const float* qp = qkv + ((int64_t)b * a.s_max + q) * 3 * D + h * kHeadDim + 2 * lane;
  const float q0 = qp[0], q1 = qp[1];
  const float scale = 1.0f / sqrtf((float)kHeadDim);
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j = 0; j < S; ++j) {
    const float* kp = qkv + ((int64_t)b * a.s_max + j) * 3 * D + D + h * kHeadDim + 2 * lane;
    float s = q0 * kp[0] + q1 * kp[1];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    s *= scale;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    const float* vp = kp + D;
    l = l * al + p;
    o0 = o0 * al + p * vp[0];
    o1 = o1 * al + p * vp[1];
    m = mn;
  }
  op[0] = o0 / l;
  op[1] = o1 / l;
}

}  // namespace

size_t attn_vt_bytes(int precision, int batch, int s_max, int n_heads) {
  if (precision != 0) return 0;
  const int s_pad = (s_max + 63) / 64 * 64;
  return (size_t)batch * n_heads * kHeadDim * s_pad * sizeof(bf16);
}

hipError_t launch_attn(int precision, const AttnArgs& a, hipStream_t s) {
  if (precision == 0) {
    hipLaunchKernelGGL(vtrans_kernel, dim3(a.s_pad / 64, a.n_heads, a.batch), dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_bf16_kernel, dim3((a.s_max + QT - 1) / QT, a.n_heads, a.batch),
                       dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.s_max, a.n_heads, a.batch), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace zdit
