// C = A B^T for few rows (M <= 256): the text encoder's projections at 2 x 64 tokens, where
// the 256 x 256 tiles of the main GEMM would occupy a few dozen of the 256 CUs while the time
// goes into streaming the weights from HBM.
//
// Split-K.  A 256-thread workgroup owns 128 rows x 64 columns of C and a K range of ks
// columns; the number of ranges depends on N and K only (about 512 workgroups for one row
// tile), so every output's sum has the same K split and the same order whatever M is.  Each
// wavefront owns 32 rows x 64 columns (2 x 4 tiles of v_mfma_f32_16x16x32_bf16).  K advances in
// 32-wide slabs through a ring of four LDS stages filled by direct-to-LDS buffer loads three
// slabs ahead (rows past M or N load as zero from the bounds-checked buffer resource).  The
// fp32 partial tiles go to a workspace [splits][M][Nv]; a second kernel sums them in split
// order and applies the epilogue: bf16 store, fp32 gated residual add, or SwiGLU on the
// paired W1 / W3 partials (Nv = 2N: the W3 columns follow the W1 columns).
#include "common.h"

namespace zdit {

namespace {

constexpr int SBM = 128, SBN = 64, SBK = 32;
constexpr int SA_CHUNKS = SBM * (SBK / 8);          // 512 16-byte chunks of A per slab
constexpr int SB_CHUNKS = SBN * (SBK / 8);          // 256 of B
constexpr int S_CHUNKS = SA_CHUNKS + SB_CHUNKS;     // 768 (12 KB) per stage
constexpr int S_DMA = S_CHUNKS / 64 / 4;            // 3 wave loads per wave per slab
constexpr int kSBufFlags = 0x00020000;
constexpr int s_waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// slot (16-byte units from the operand's first row) of logical chunk c of row r
__device__ __forceinline__ int sswz(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

__device__ __forceinline__ void sdma_16(const __amdgpu_buffer_rsrc_t rs, const uint4* lds_base, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff,
                                           0, 0);
}

__device__ __forceinline__ float ssilu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

__global__ __launch_bounds__(256) void gemm_splitk_kernel(SplitKArgs a) {
  // four separate objects, so reads of one stage are not ordered behind the in-flight
  // direct-to-LDS writes of another
  __shared__ uint4 L0[S_CHUNKS], L1[S_CHUNKS], L2[S_CHUNKS], L3[S_CHUNKS];
  const int ct = blockIdx.x, split = blockIdx.y, m0 = blockIdx.z * SBM;
  const bool second = ct >= a.col_tiles;  // SwiGLU: the W3 half of the virtual columns
  const int n0 = (second ? ct - a.col_tiles : ct) * SBN;
  const int k0 = split * a.ks;
  const int nk = (min(a.K, k0 + a.ks) - k0) / SBK;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const bf16* ab = (const bf16*)a.A + (int64_t)m0 * a.lda;
  const bf16* bb = (const bf16*)(second ? a.B2 : a.B) + (int64_t)n0 * a.ldb;
  const __amdgpu_buffer_rsrc_t ars =
      __builtin_amdgcn_make_buffer_rsrc((void*)ab, 0, (a.M - m0) * a.lda * 2, kSBufFlags);
  const __amdgpu_buffer_rsrc_t brs =
      __builtin_amdgcn_make_buffer_rsrc((void*)bb, 0, (a.N - n0) * a.ldb * 2, kSBufFlags);

  // wave load j of this wave fills stage slots (3 wave + j) * 64 + lane: slots below 512 are A
  // (row s / 4), the rest B; the lane fetches the logical chunk that belongs in its slot
  int voff[S_DMA];
#pragma unroll
  for (int j = 0; j < S_DMA; ++j) {
    const int s = (S_DMA * wave + j) * 64 + lane;
    const int sb = s < SA_CHUNKS ? s : s - SA_CHUNKS;
    const int r = sb >> 2, c = (sb & 3) ^ ((r >> 2) & 3);
    voff[j] = r * (s < SA_CHUNKS ? a.lda : a.ldb) * 2 + c * 16;
  }
  auto issue = [&](int kt, uint4* st) {
    const int soff = (k0 + kt * SBK) * 2;
#pragma unroll
    for (int j = 0; j < S_DMA; ++j) {
      const int w = S_DMA * wave + j;  // wave-uniform: A for w < 8
      sdma_16(w < SA_CHUNKS / 64 ? ars : brs, st + w * 64, voff[j], soff);
    }
  };

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fh = lane >> 4;
  const int arow = wave * 32 + fr;

  // Slab T is in stage CUR; the stage of slab T - 1 (NXT, free after this slab's barrier)
  // receives slab T + 3.  The body has no branch (a branch would make the wait insertion
  // forget which stage each in-flight load targets): past the last slab the load repeats the
  // last one into a stage that is not read again, and the wait always leaves the two newer
  // slabs' loads in flight.  A macro, so that each LDS access names its own stage object.
#define ZDIT_SPLITK_SLAB(T, CUR, NXT)                                                                  \
  {                                                                                                   \
    const int t_ = (T);                                                                               \
    __builtin_amdgcn_s_waitcnt(s_waitcnt_vm(2 * S_DMA));                                              \
    /* every wave's loads of slab T are complete (each waited for its own): a bare barrier,           \
       without the fence that would also wait for the slabs still in flight */                       \
    __builtin_amdgcn_sched_barrier(0);                                                                \
    __builtin_amdgcn_s_barrier();                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                                \
    bf16x8 fa[2], fb[4];                                                                              \
    for (int i = 0; i < 2; ++i) fa[i] = __builtin_bit_cast(bf16x8, CUR[sswz(arow + 16 * i, fh)]);    \
    for (int j = 0; j < 4; ++j) fb[j] = __builtin_bit_cast(bf16x8, CUR[SA_CHUNKS + sswz(16 * j + fr, fh)]); \
    issue(min(t_ + 3, nk - 1), NXT);                                                                  \
    for (int i = 0; i < 2; ++i)                                                                       \
      for (int j = 0; j < 4; ++j)                                                                     \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);       \
  }

  issue(0, L0);
  issue(min(1, nk - 1), L1);
  issue(min(2, nk - 1), L2);
  int t = 0;
  for (; t + 4 <= nk; t += 4) {
    ZDIT_SPLITK_SLAB(t, L0, L3)
    ZDIT_SPLITK_SLAB(t + 1, L1, L0)
    ZDIT_SPLITK_SLAB(t + 2, L2, L1)
    ZDIT_SPLITK_SLAB(t + 3, L3, L2)
  }
  if (t < nk) ZDIT_SPLITK_SLAB(t, L0, L3)
  if (t + 1 < nk) ZDIT_SPLITK_SLAB(t + 1, L1, L0)
  if (t + 2 < nk) ZDIT_SPLITK_SLAB(t + 2, L2, L1)
#undef ZDIT_SPLITK_SLAB
  // the repeated loads past the last slab are still landing
  __builtin_amdgcn_s_waitcnt(s_waitcnt_vm(0));

  // partial tile: lane holds rows 4 (lane / 16) + e of each 16 x 16 tile, column lane % 16
  const int nv0 = (second ? a.N : 0) + n0;
  float* part = a.part + (int64_t)split * a.M * a.Nv;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 16 * j + fr;
      if (n >= a.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wave * 32 + 16 * i + 4 * fh + e;
        if (m < a.M) part[(int64_t)m * a.Nv + nv0 + 16 * j + fr] = acc[i][j][e];
      }
    }
}

// One thread per 4 consecutive output columns of a row: the partials summed in split order,
// then the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(SplitKArgs a, GemmArgs g) {
  const int nq = a.N >> 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.M * nq) return;
  const int m = (int)(i / nq), n = (int)(i % nq) * 4;
  const int64_t plane = (int64_t)a.M * a.Nv;
  const float* p = a.part + (int64_t)m * a.Nv + n;
  float4 s = *(const float4*)p;
  for (int k = 1; k < a.splits; ++k) {
    const float4 v = *(const float4*)(p + k * plane);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  const RowMap& rm = g.out;
  const int b = m / rm.rows_per_batch, r = m - b * rm.rows_per_batch;
  if (r >= rm.valid[b]) return;
  const int64_t off = b * rm.batch_stride + (int64_t)r * rm.ld + n;
  if constexpr (EPI == EPI_RESID) {
    float* x = (float*)g.C + off;
    float4 xv = *(float4*)x;
    if (g.vec) {
      const float* gv = g.vec + b * g.vec_bstride + n;
      xv.x += gv[0] * s.x; xv.y += gv[1] * s.y; xv.z += gv[2] * s.z; xv.w += gv[3] * s.w;
    } else {
      xv.x += s.x; xv.y += s.y; xv.z += s.z; xv.w += s.w;
    }
    *(float4*)x = xv;
  } else {
    float o[4] = {s.x, s.y, s.z, s.w};
    if constexpr (EPI == EPI_SWIGLU) {
      float4 u = *(const float4*)(p + a.N);
      for (int k = 1; k < a.splits; ++k) {
        const float4 v = *(const float4*)(p + a.N + k * plane);
        u.x += v.x; u.y += v.y; u.z += v.z; u.w += v.w;
      }
      o[0] = ssilu(s.x) * u.x; o[1] = ssilu(s.y) * u.y; o[2] = ssilu(s.z) * u.z; o[3] = ssilu(s.w) * u.w;
    }
    bf16x4 ob;
#pragma unroll
    for (int e = 0; e < 4; ++e) ob[e] = (bf16)o[e];
    *(bf16x4*)((bf16*)g.C + off) = ob;
  }
}

}  // namespace

SplitKArgs splitk_plan(int epi, int M, int N, int K) {
  SplitKArgs a{};
  a.M = M; a.N = N; a.K = K;
  a.col_tiles = (N + SBN - 1) / SBN;
  a.Nv = epi == EPI_SWIGLU ? 2 * N : N;
  const int vtiles = epi == EPI_SWIGLU ? 2 * a.col_tiles : a.col_tiles;
  // about 512 workgroups for one 128-row tile; ranges of at least 128 columns of K
  int splits = (512 + vtiles - 1) / vtiles;
  splits = max(1, min(splits, K / 128));
  a.ks = ((K + splits - 1) / splits + SBK - 1) / SBK * SBK;
  a.splits = (K + a.ks - 1) / a.ks;
  return a;
}

size_t splitk_workspace(int epi, int M, int N, int K) {
  const SplitKArgs a = splitk_plan(epi, M, N, K);
  return (size_t)a.splits * M * a.Nv * sizeof(float);
}

hipError_t launch_gemm_splitk(int epi, const GemmArgs& g, float* part, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  SplitKArgs a = splitk_plan(epi, g.M, g.N, g.K);
  a.A = g.A; a.B = g.B; a.B2 = g.B2; a.part = part; a.lda = (int)g.lda; a.ldb = (int)g.ldb;
  const int vtiles = epi == EPI_SWIGLU ? 2 * a.col_tiles : a.col_tiles;
  dim3 grid(vtiles, a.splits, (g.M + SBM - 1) / SBM);
  hipLaunchKernelGGL(gemm_splitk_kernel, grid, dim3(256), 0, s, a);
  const unsigned rb = (unsigned)(((int64_t)g.M * (g.N / 4) + 255) / 256);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_STORE>, dim3(rb), dim3(256), 0, s, a, g); break;
    case EPI_RESID: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_RESID>, dim3(rb), dim3(256), 0, s, a, g); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_SWIGLU>, dim3(rb), dim3(256), 0, s, a, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace zdit
