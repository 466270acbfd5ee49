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
// each group of 16 keys both operands use the key order {4h..4h+3, 8+4h..8+4h+3}; V^T is
// stored with each 16-key group in that order, so a lane reads its 8 keys in one 16-byte load.
// Online softmax in fp32 with exp2 and the 1/sqrt(128) scale folded into log2(e).
#include <type_traits>

#include "common.h"

namespace zdit {

namespace {

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
  // Within every 16-key group the keys are stored in the order the 32x32 MFMA result hands
  // them to a lane half: chunk 2g holds keys {0-3, 8-11} of group g, chunk 2g+1 holds keys
  // {4-7, 12-15}, so the attention kernel reads a lane's 8 keys as one 16-byte chunk.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int d = c >> 3, sc = c & 7;
    const int kbase = (sc >> 1) * 16 + (sc & 1) * 4;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = tb[(kbase + (e & 3) + 8 * (e >> 2)) * (KROW * 8) + d];
    *(bf16x8*)(vt + (int64_t)d * a.s_pad + s0 + sc * 8) = o;
  }
}

// 8 wavefronts x 32 queries = 256 queries per workgroup (two wavefronts per SIMD, so one's
// softmax overlaps the other's MFMAs).  K and V^T key blocks are double-buffered in LDS and
// prefetched through registers one block ahead.  Per key block t: softmax of the scores of
// block t, O^T += V^T P^T, then the QK^T MFMAs of block t+1 (built with ZDIT_ATTN_PIPELINE
// the QK^T of block t+1 is issued before the softmax instead; measured slower on gfx950).
#ifndef ZDIT_ATTN_WAVES
#define ZDIT_ATTN_WAVES 8
#endif
constexpr int NWAVE = ZDIT_ATTN_WAVES;
constexpr int QTILE = 32 * NWAVE;
constexpr int ATT_NT = 64 * NWAVE;           // threads per workgroup
constexpr int KCH = KT * 16 / ATT_NT;        // 16-byte K chunks per thread per key block
constexpr int VCH = kHeadDim * 8 / ATT_NT;   // 16-byte V^T chunks per thread per key block

// Workgroups are dispatched round-robin over the 8 XCDs.  The 1-D grid is renumbered so that
// consecutive logical ids (the query tiles of one (branch, head), which share its K and V)
// run on the same XCD and hit its L2.
__device__ __forceinline__ int xcd_logical_id(int pid, int nwg) {
  const int xcd = pid & 7, idx = pid >> 3;
  const int full = nwg >> 3, rem = nwg & 7;
  return (xcd < rem) ? xcd * (full + 1) + idx : rem * (full + 1) + (xcd - rem) * full + idx;
}

// two wavefronts per SIMD in either shape (8-wave workgroups: one per CU; 4-wave: two per CU)
__global__ __launch_bounds__(ATT_NT) __attribute__((amdgpu_waves_per_eu(2))) void attn_bf16_kernel(AttnArgs a) {
  __shared__ uint4 Ks[2][KT * KROW];
  __shared__ uint4 Vs[2][kHeadDim * VROW];
  const int nqt = (a.s_max + QTILE - 1) / QTILE;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int qt = lid % nqt, bh = lid / nqt;
  const int h = bh % a.n_heads, b = bh / a.n_heads, q0 = qt * QTILE;
  const int D = a.n_heads * kHeadDim;
  const int S = a.seq_len[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int q = q0 + wave * 32 + fr;
  const bf16* qkv = (const bf16*)a.qkv;
  bf16* out = (bf16*)a.out;

  if (q0 >= S) {  // the whole tile is padding: write zeros
    for (int i = tid; i < QTILE * 16; i += ATT_NT) {
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

  const bf16* kbase = qkv + (int64_t)b * a.s_max * 3 * D + D + h * kHeadDim;
  const bf16* vbase = (const bf16*)a.vt + ((int64_t)(b * a.n_heads + h) * kHeadDim) * a.s_pad;
  // prefetch assignment: K chunk c = tid + ATT_NT i -> key c / 16, 16-byte chunk c % 16;
  // V^T chunk c -> dim c / 8, chunk c % 8
  uint4 rk[KCH], rv[VCH];
  auto gload_k = [&](int t) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + ATT_NT * i, key = t * KT + (c >> 4);
      rk[i] = key < S ? *(const uint4*)(kbase + (int64_t)key * 3 * D + (c & 15) * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto gload_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + ATT_NT * i;
      rv[i] = *(const uint4*)(vbase + (int64_t)(c >> 3) * a.s_pad + t * KT + (c & 7) * 8);
    }
  };
  auto sstore_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + ATT_NT * i;
      Ks[buf][(c >> 4) * KROW + (c & 15)] = rk[i];
    }
  };
  auto sstore_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + ATT_NT * i;
      Vs[buf][(c >> 3) * VROW + (c & 7)] = rv[i];
    }
  };
  auto qk = [&](int buf, f32x16 (&st)[2]) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[t2][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, Ks[buf][(t2 * 32 + fr) * KROW + 2 * s + fh]);
        st[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[t2], 0, 0, 0);
      }
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = 1.4426950408889634f / sqrtf((float)kHeadDim);
  const int nkt = (S + KT - 1) / KT;

  // One key block: softmax of block t (held in `cur`), O^T += V^T P^T, QK^T of block t+1
  // into `nxt`.  Two copies alternate the roles of the score registers, so no copy is
  // needed between iterations.  Only the final block can hold keys >= S (masked).
  auto step = [&](auto masked, int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    const bool more = t + 1 < nkt;
    if (more) gload_v(t + 1);
#ifdef ZDIT_ATTN_PIPELINE
    if (more) qk((t + 1) & 1, nxt);
#endif

    float mx = -INFINITY;
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * KT + t2 * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
          if (key >= S) cur[t2][r] = -INFINITY;
        }
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[t2][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * sc);
    // Lazy rescale: the reference max moves only when some lane's max rose by more than 8
    // (log2 units), so p = exp2(s - m_run) stays below 2^8; O and l share the reference, so
    // the result O / l is the same softmax.
    if (__any(m_new > m_run + 8.0f)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      m_run = m_new;
    }
    bf16x8 pb[2][2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[t2][r], sc, -m_run));
        l_run += p;
        pb[t2][r >> 3][r & 7] = (bf16)p;
      }
    // the K prefetch is issued once this block's scores are dead (keeps the register peak low)
    if (t + 2 < nkt) gload_k(t + 2);
    const uint4* Vb = Vs[t & 1];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // 16-byte chunk (t2 * 4 + j * 2 + fh) of the V^T row holds this lane half's 8 keys
          const bf16x8 vf = __builtin_bit_cast(bf16x8, Vb[(dt * 32 + fr) * VROW + t2 * 4 + j * 2 + fh]);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t2][j], o[dt], 0, 0, 0);
        }
    }
#ifndef ZDIT_ATTN_PIPELINE
    if (more) qk((t + 1) & 1, nxt);
#endif
    if (t + 2 < nkt) sstore_k(t & 1);
    if (more) sstore_v((t + 1) & 1);
    __syncthreads();
  };

  gload_k(0); sstore_k(0);
  gload_v(0); sstore_v(0);
  if (nkt > 1) { gload_k(1); sstore_k(1); }
  __syncthreads();
  f32x16 sA[2], sB[2];
  qk(0, sA);
  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  int t = 0;
  for (; t + 2 < nkt; t += 2) {
    step(Plain{}, t, sA, sB);
    step(Plain{}, t + 1, sB, sA);
  }
  if (nkt - t == 2) {
    step(Plain{}, t, sA, sB);
    step(Masked{}, t + 1, sB, sA);
  } else {
    step(Masked{}, t, sA, sB);
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
    hipLaunchKernelGGL(attn_bf16_kernel, dim3(((a.s_max + QTILE - 1) / QTILE) * a.n_heads * a.batch),
                       dim3(ATT_NT), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.s_max, a.n_heads, a.batch), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace zdit
