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
// buffer resource word 3 for raw (untyped, offset-addressed) buffer loads
constexpr int kBufFlags = 0x00020000;
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kVmcnt0 = 0x0F70;

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// Chunk kc of row r sits at slot kc ^ g(r), g(r) = (r & 7) ^ ((r >> 3) & 1): any 8 aligned
// consecutive rows, and the rows of either parity among 16 consecutive rows, see distinct
// slots, so 16-byte fragment reads of 16 consecutive rows touch distinct banks.
__device__ __forceinline__ int swz(int row, int kc) { return row * 8 + (kc ^ (row & 7) ^ ((row >> 3) & 1)); }

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

// LDS stage: A tile [256 rows][8 x 16-byte chunks] then B tile, 64 KB.  Chunk kc of row r
// sits at slot kc ^ (r & 7).
__device__ __forceinline__ void lds_dma_16(const __amdgpu_buffer_rsrc_t rs, const uint4* lds_base,
                                           int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16, voff,
                                           soff, 0, 0);
}

// Fragments of one k16 step (16-byte chunk kc) of a stage for this wave's MT A tiles and 4 B
// tiles (each 32 rows).
template <int MT>
__device__ __forceinline__ void load_frags(const uint4* sa, const uint4* sb, int arow, int brow, int kc,
                                           bf16x8 (&af)[MT], bf16x8 (&bf)[4]) {
#pragma unroll
  for (int i = 0; i < MT; ++i) af[i] = __builtin_bit_cast(bf16x8, sa[swz(arow + i * 32, kc)]);
#pragma unroll
  for (int i = 0; i < 4; ++i) bf[i] = __builtin_bit_cast(bf16x8, sb[swz(brow + i * 32, kc)]);
}

template <int MT>
__device__ __forceinline__ void mma_step(const bf16x8 (&af)[MT], const bf16x8 (&bf)[4], f32x16 (&acc)[MT][4]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
}

// scheduling hint for one step's 4*MT MFMAs with the next step's MT + 4 LDS reads interleaved
template <int MT>
__device__ __forceinline__ void sched_mma_ds() {
#ifndef ZDIT_GEMM_NO_SCHED
  if constexpr (MT == 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
#endif
}

// WAVES = 4: each wavefront owns 128 x 128 of the tile (4 x 4 MFMA tiles, one wave per SIMD).
// WAVES = 8: each owns 64 x 128 (2 x 4 MFMA tiles, two waves per SIMD, so one wave's LDS and
// barrier waits are covered by the other's MFMAs).
template <int EPI, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int MT = 16 / WAVES;          // 32-row MFMA tiles per wave along M
  constexpr int BLK = 32 / WAVES;         // 8-row DMA blocks per wave per operand
  // two stages as separate objects, so reads of one stage are not ordered behind the
  // in-flight direct-to-LDS loads of the other
  __shared__ uint4 st0[2][BM * BK / 8];
  __shared__ uint4 st1[2][BM * BK / 8];

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform: keep it in a scalar register (LDS bases and buffer offsets
  // derived from it must be scalar)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // wm: MT*32-row band, wn: 128-column half
  const int nout_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + nout_tile - 1) / nout_tile;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * nout_tile;

  // Operands are read through buffer resources based at the tile's first row: rows past M
  // (or N) fall outside the resource and load as zero.
  const bf16* A0 = (const bf16*)g.A + (int64_t)m0 * g.lda;
  const __amdgpu_buffer_rsrc_t ra_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)A0, 0, (int)min((int64_t)(g.M - m0) * g.lda * 2, (int64_t)0x7fffffff), kBufFlags);
  const bf16* B0 = (const bf16*)g.B + (int64_t)n0 * g.ldb;
  const int brec = (int)min((int64_t)(g.N - n0) * g.ldb * 2, (int64_t)0x7fffffff);
  const __amdgpu_buffer_rsrc_t rb_rs = __builtin_amdgcn_make_buffer_rsrc((void*)B0, 0, brec, kBufFlags);
  __amdgpu_buffer_rsrc_t rb2_rs = rb_rs;
  if constexpr (EPI == EPI_SWIGLU)
    rb2_rs = __builtin_amdgcn_make_buffer_rsrc((void*)((const bf16*)g.B2 + (int64_t)n0 * g.ldb), 0, brec, kBufFlags);

  // Direct-to-LDS: one wave instruction writes 1 KB = 8 rows (blk * 8 ..) of the tile, lane L
  // landing at slot L % 8 of row L / 8; it therefore fetches chunk (L % 8) ^ g(row), where
  // g(row) = (L / 8) ^ (blk & 1).  The row offset goes into the per-lane (bounds-checked)
  // offset, so rows past the resource read as zero; only the K offset is scalar (the scalar
  // offset is not bounds-checked, and K offsets always stay inside a row).
  const int lr = lane >> 3;
  const int lkc0 = (lane & 7) ^ lr, lkc1 = lkc0 ^ 1;
  const int va0 = (lr * (int)g.lda + lkc0 * 8) * 2, va1 = (lr * (int)g.lda + lkc1 * 8) * 2;
  const int vb0 = (lr * (int)g.ldb + lkc0 * 8) * 2, vb1 = (lr * (int)g.ldb + lkc1 * 8) * 2;

  auto issue = [&](int kt, uint4 (&stage)[2][BM * BK / 8]) {
    const int kb = kt * BK * 2;
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
      const int blk = wave * BLK + i;        // rows blk*8 .. blk*8+7 of the tile
      lds_dma_16(ra_rs, &stage[0][blk * 64], ((i & 1) ? va1 : va0) + blk * 8 * (int)g.lda * 2, kb);
      int brow;
      __amdgpu_buffer_rsrc_t rsb = rb_rs;
      if constexpr (EPI == EPI_SWIGLU) {
        // tile row t = blk*8 + r: wave column t / 128, MFMA tile (t % 128) / 32 (even: W1,
        // odd: W3), output column (t / 128) * 64 + (tile / 2) * 32 + t % 32
        const int t = blk * 8, wc = t >> 7, mt = (t & 127) >> 5;
        brow = wc * 64 + (mt >> 1) * 32 + (t & 31);
        if (mt & 1) rsb = rb2_rs;
      } else {
        brow = blk * 8;
      }
      lds_dma_16(rsb, &stage[1][blk * 64], ((i & 1) ? vb1 : vb0) + brow * (int)g.ldb * 2, kb);
    }
  };

  f32x16 acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = g.K / BK;
  const int fr = lane & 31, fh = lane >> 5;

  const uint4* s0a = st0[0];
  const uint4* s0b = st0[1];
  const uint4* s1a = st1[0];
  const uint4* s1b = st1[1];
  const int arow = wm * (32 * MT) + fr, brow = wn * 128 + fr;
  bf16x8 fa0[MT], fb0[4], fa1[MT], fb1[4];

  // One 64-wide K slab from stage `cur` (its step-0 fragments already in fa0/fb0).  The
  // barrier comes once the slab's last fragments are in registers: after it, the DMA of the
  // slab two ahead goes into `cur`, and the next slab's step-0 fragments are read from `nxt`
  // while the last 16 MFMAs of this slab run.
#define ZDIT_SLAB(CA, CB, NA, NB, CUR_ST, HAS_NEXT, NEXT2)                                    \
  {                                                                                           \
    load_frags<MT>(CA, CB, arow, brow, 2 + fh, fa1, fb1);                                     \
    mma_step<MT>(fa0, fb0, acc);                                                              \
    sched_mma_ds<MT>();                                                                       \
    load_frags<MT>(CA, CB, arow, brow, 4 + fh, fa0, fb0);                                     \
    mma_step<MT>(fa1, fb1, acc);                                                              \
    sched_mma_ds<MT>();                                                                       \
    load_frags<MT>(CA, CB, arow, brow, 6 + fh, fa1, fb1);                                     \
    mma_step<MT>(fa0, fb0, acc);                                                              \
    sched_mma_ds<MT>();                                                                       \
    if (HAS_NEXT) {                                                                           \
      __builtin_amdgcn_s_waitcnt(kVmcnt0);                                                    \
      __syncthreads();                                                                        \
      if (NEXT2) issue(kt + 2, CUR_ST);                                                       \
      load_frags<MT>(NA, NB, arow, brow, fh, fa0, fb0);                                       \
    }                                                                                         \
    mma_step<MT>(fa1, fb1, acc);                                                              \
  }

  issue(0, st0);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  if (nk > 1) issue(1, st1);
  load_frags<MT>(s0a, s0b, arow, brow, fh, fa0, fb0);
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    ZDIT_SLAB(s0a, s0b, s1a, s1b, st0, true, kt + 2 < nk)
    ++kt;
    ZDIT_SLAB(s1a, s1b, s0a, s0b, st1, kt + 1 < nk, kt + 2 < nk)
    --kt;
  }
  if (kt < nk) ZDIT_SLAB(s0a, s0b, s1a, s1b, st0, false, false)
#undef ZDIT_SLAB

  // ---- epilogue.  Accumulator (mt, nt) element r of this lane is C[row][col] with
  // row = 8 (r / 4) + 4 (lane / 32) + r % 4 and col = lane % 32 within the 32 x 32 tile.
  // Row addressing is resolved once per row; loads of a tile's 16 values are issued together
  // before any store, so their latencies overlap.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int64_t roff[16];
    bool rok[16];
    int rb[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * (32 * MT) + mt * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
      const int mm = min(m, g.M - 1);
      const RowAddr ro = map_row(g.out, mm);
      roff[r] = ro.off;
      rok[r] = (m < g.M) && ro.ok;
      rb[r] = mm / g.out.rows_per_batch;
    }
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int np = 0; np < 2; ++np) {
        const int n = n0 + wn * 64 + np * 32 + fr;
        if (n >= g.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (rok[r]) ((bf16*)g.C)[roff[r] + n] = (bf16)(silu(acc[mt][2 * np][r]) * acc[mt][2 * np + 1][r]);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int n = n0 + wn * 128 + nt * 32 + fr;
        if (n >= g.N) continue;
        if constexpr (EPI == EPI_STORE) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (rok[r]) ((bf16*)g.C)[roff[r] + n] = (bf16)acc[mt][nt][r];
        } else if constexpr (EPI == EPI_BIAS) {
          const float bias = g.vec[n];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (rok[r]) ((float*)g.C)[roff[r] + n] = acc[mt][nt][r] + bias;
        } else {  // EPI_RESID: x += gate * (A B^T)
          float* C = (float*)g.C;
          float cur[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) cur[r] = rok[r] ? C[roff[r] + n] : 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (!rok[r]) continue;
            const float gate = g.vec ? g.vec[rb[r] * g.vec_bstride + n] : 1.0f;
            C[roff[r] + n] = cur[r] + gate * acc[mt][nt][r];
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
  dim3 grid(tiles);
#ifdef ZDIT_GEMM_4WAVE
  constexpr int W = 4;
#else
  constexpr int W = 8;
#endif
  dim3 block(64 * W);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_bf16_kernel<EPI_STORE, W>), grid, block, 0, s, g); break;
    case EPI_BIAS: hipLaunchKernelGGL((gemm_bf16_kernel<EPI_BIAS, W>), grid, block, 0, s, g); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_bf16_kernel<EPI_RESID, W>), grid, block, 0, s, g); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_bf16_kernel<EPI_SWIGLU, W>), grid, block, 0, s, g); break;
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
