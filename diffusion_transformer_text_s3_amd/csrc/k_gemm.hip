// Dense contractions of the S3-DiT block on gfx950: C = A B^T with A [M, K] and B [N, K]
// both K-contiguous (activations [tokens, features] and weights [out, in]).
//
// bf16 path: v_mfma_f32_32x32x16_bf16, fp32 accumulation.  One 256-thread workgroup owns a
// 256 x 256 tile of C; its four wavefronts each own 128 x 128 (4 x 4 MFMA tiles, 256 fp32
// accumulators per lane).  K advances in steps of 64 through two LDS buffers (2 x 64 KB):
// the next K-slab is fetched from global into registers while the current one feeds the
// MFMAs, then written to the other buffer.  LDS rows are 128 B (64 bf16); the eight 16-byte
// chunks of row r are stored at chunk ^ (r & 7), so both the 16-byte stores of a row and
// the 16-byte fragment reads of eight consecutive rows hit distinct banks.
//
// Workgroups are numbered so that the ones dispatched to the same XCD (round-robin over 8)
// get consecutive tiles, and tiles are walked in groups of 8 row-panels, so each XCD's L2
// sees a compact set of A and B panels.
//
// Epilogues run on the accumulators in registers: plain bf16 store (QKV), bias + fp32 store
// into a branch-strided buffer (embeds, final layer), fp32 gated residual read-modify-write
// (out projection, w2), and SwiGLU on paired W1 / W3 tiles (w1/w3).  There is no split-K:
// each output's sum runs over K in one fixed order, independent of M and of the tile.
#include "common.h"

namespace zdit {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 256;  // threads
// buffer resource word 3 for raw (untyped, offset-addressed) buffer loads
constexpr int kBufFlags = 0x00020000;

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

__device__ __forceinline__ int swz(int row, int kc) { return row * 8 + (kc ^ (row & 7)); }

// Physical workgroup id -> (tile row, tile col).
__device__ __forceinline__ void tile_coords(int pid, int nwg, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  // XCD-aware renumbering: consecutive logical ids on the same XCD.
  const int xcd = pid & 7, idx = pid >> 3;
  const int full = nwg >> 3, rem = nwg & 7;
  const int lid = (xcd < rem) ? xcd * (full + 1) + idx : rem * (full + 1) + (xcd - rem) * full + idx;
  constexpr int G = 8;
  const int per_group = G * tiles_n;
  const int group = lid / per_group;
  const int first_m = group * G;
  const int gsz = min(tiles_m - first_m, G);
  const int in_group = lid % per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

struct RowAddr {
  int64_t off;
  bool ok;
};

__device__ __forceinline__ RowAddr map_row(const RowMap& rm, int m) {
  const int b = m / rm.rows_per_batch, r = m - b * rm.rows_per_batch;
  RowAddr ra;
  ra.ok = r < rm.valid[b];
  ra.off = b * rm.batch_stride + (int64_t)r * rm.ld;
  return ra;
}

template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ uint4 smem[2][2][BM * BK / 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nout_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + nout_tile - 1) / nout_tile;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * nout_tile;

  // Operands are read through buffer resources based at the tile's first row: rows past M
  // (or N) fall outside the resource and load as zero.  Thread t covers rows (t / 8) + 32 i,
  // i = 0..7, 16-byte chunk t % 8 of each 64-wide K slab.
  const int lrow = tid >> 3, lkc = tid & 7;
  const bf16* A0 = (const bf16*)g.A + (int64_t)m0 * g.lda;
  const __amdgpu_buffer_rsrc_t ra_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)A0, 0, (int)min((int64_t)(g.M - m0) * g.lda * 2, (int64_t)0x7fffffff), kBufFlags);
  const bf16* B0 = (const bf16*)g.B + (int64_t)n0 * g.ldb;
  const int brec = (int)min((int64_t)(g.N - n0) * g.ldb * 2, (int64_t)0x7fffffff);
  const __amdgpu_buffer_rsrc_t rb_rs = __builtin_amdgcn_make_buffer_rsrc((void*)B0, 0, brec, kBufFlags);
  __amdgpu_buffer_rsrc_t rb2_rs = rb_rs;
  if constexpr (EPI == EPI_SWIGLU)
    rb2_rs = __builtin_amdgcn_make_buffer_rsrc((void*)((const bf16*)g.B2 + (int64_t)n0 * g.ldb), 0, brec, kBufFlags);
  const int va = (lrow * (int)g.lda + lkc * 8) * 2;
  const int vb = (lrow * (int)g.ldb + lkc * 8) * 2;
  // uniform row offsets (bytes) of the 8 rows a thread loads
  auto a_soff = [&](int i) { return 32 * i * (int)g.lda * 2; };
  auto b_soff = [&](int i) {
    if constexpr (EPI == EPI_SWIGLU) return ((i >> 2) * 64 + ((i & 3) >> 1) * 32) * (int)g.ldb * 2;
    else return 32 * i * (int)g.ldb * 2;
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[8], rb[8];
  const int nk = g.K / BK;

  auto load_slab = [&](int kt) {
    const int kb = kt * BK * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra_rs, va, a_soff(i) + kb, 0));
      const __amdgpu_buffer_rsrc_t rsb = (EPI == EPI_SWIGLU && (i & 1)) ? rb2_rs : rb_rs;
      rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsb, vb, b_soff(i) + kb, 0));
    }
  };

  load_slab(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    smem[0][0][swz(lrow + 32 * i, lkc)] = ra[i];
    smem[0][1][swz(lrow + 32 * i, lkc)] = rb[i];
  }
  __syncthreads();

  const int fr = lane & 31, fh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_slab(kt + 1);
    const uint4* sa = smem[cur][0];
    const uint4* sb = smem[cur][1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kc = 2 * s + fh;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = wm * 128 + mt * 32 + fr;
        af[mt] = __builtin_bit_cast(bf16x8, sa[swz(row, kc)]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = wn * 128 + nt * 32 + fr;
        bfr[nt] = __builtin_bit_cast(bf16x8, sb[swz(row, kc)]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
    }
    if (kt + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        smem[cur ^ 1][0][swz(lrow + 32 * i, lkc)] = ra[i];
        smem[cur ^ 1][1][swz(lrow + 32 * i, lkc)] = rb[i];
      }
    }
    __syncthreads();
  }

  // ---- epilogue.  Accumulator (mt, nt) element r of this lane is C[row][col] with
  // row = 8 (r / 4) + 4 (lane / 32) + r % 4 and col = lane % 32 within the 32 x 32 tile.
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * 128 + mt * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
      if (m >= g.M) continue;
      const RowAddr ro = map_row(g.out, m);
      if (!ro.ok) continue;
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int np = 0; np < 2; ++np) {
          const int n = n0 + wn * 64 + np * 32 + fr;
          if (n < g.N) {
            const float u = silu(acc[mt][2 * np][r]) * acc[mt][2 * np + 1][r];
            ((bf16*)g.C)[ro.off + n] = (bf16)u;
          }
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int n = n0 + wn * 128 + nt * 32 + fr;
          if (n >= g.N) continue;
          const float v = acc[mt][nt][r];
          if constexpr (EPI == EPI_STORE) {
            ((bf16*)g.C)[ro.off + n] = (bf16)v;
          } else if constexpr (EPI == EPI_BIAS) {
            ((float*)g.C)[ro.off + n] = v + g.vec[n];
          } else {  // EPI_RESID
            const int b = m / g.out.rows_per_batch;
            const float gate = g.vec ? g.vec[b * g.vec_bstride + n] : 1.0f;
            float* p = (float*)g.C + ro.off + n;
            *p = *p + gate * v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// fp32 debug GEMM: 64 x 64 tiles, K step 16, 4 x 4 outputs per thread, plain FMA.
// ---------------------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int T = 64, TK = 16;
  __shared__ float As[TK][T + 4];
  __shared__ float Bs[TK][T + 4];
  __shared__ float B2s[TK][T + 4];
  const float* A = (const float*)g.A;
  const float* B = (const float*)g.B;
  const float* B2 = (const float*)g.B2;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {}, acc3[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += TK) {
    for (int i = threadIdx.x; i < T * TK; i += 256) {
      const int r = i / TK, kk = i % TK;
      const int m = m0 + r, n = n0 + r, k = k0 + kk;
      As[kk][r] = (m < g.M && k < g.K) ? A[(int64_t)m * g.lda + k] : 0.f;
      Bs[kk][r] = (n < g.N && k < g.K) ? B[(int64_t)n * g.ldb + k] : 0.f;
      if constexpr (EPI == EPI_SWIGLU) B2s[kk][r] = (n < g.N && k < g.K) ? B2[(int64_t)n * g.ldb + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4], b3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; b[i] = Bs[kk][tx * 4 + i]; }
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) b3[i] = B2s[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] += a[i] * b[j];
          if constexpr (EPI == EPI_SWIGLU) acc3[i][j] += a[i] * b3[j];
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
    const RowAddr ro = map_row(g.out, m);
    if (!ro.ok) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      const float v = acc[i][j];
      float* C = (float*)g.C;
      if constexpr (EPI == EPI_STORE) C[ro.off + n] = v;
      else if constexpr (EPI == EPI_BIAS) C[ro.off + n] = v + g.vec[n];
      else if constexpr (EPI == EPI_SWIGLU) C[ro.off + n] = silu(v) * acc3[i][j];
      else {
        const int b = m / g.out.rows_per_batch;
        const float gate = g.vec ? g.vec[b * g.vec_bstride + n] : 1.0f;
        C[ro.off + n] = C[ro.off + n] + gate * v;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(int epi, const GemmArgs& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const int nout_tile = (epi == EPI_SWIGLU) ? BN / 2 : BN;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + nout_tile - 1) / nout_tile);
  dim3 grid(tiles), block(NT);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_STORE>, grid, block, 0, s, g); break;
    case EPI_BIAS: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_BIAS>, grid, block, 0, s, g); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_RESID>, grid, block, 0, s, g); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_SWIGLU>, grid, block, 0, s, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32(int epi, const GemmArgs& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  dim3 grid((g.N + 63) / 64, (g.M + 63) / 64), block(256);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, grid, block, 0, s, g); break;
    case EPI_BIAS: hipLaunchKernelGGL(gemm_f32_kernel<EPI_BIAS>, grid, block, 0, s, g); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID>, grid, block, 0, s, g); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, grid, block, 0, s, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace zdit
