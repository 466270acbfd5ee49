// Dense contractions of the S3-DiT block on gfx950: C = A B^T with A [M, K] and B [N, K]
// both K-contiguous (activations [tokens, features] and weights [out, in]).
//
// bf16 path: v_mfma_f32_16x16x32_bf16, fp32 accumulation.  One 512-thread workgroup owns a
// 256 x 256 tile of C; each of its eight wavefronts owns 64 x 128 of it (4 x 8 MFMA tiles of
// 16 x 16, 128 fp32 accumulators per lane).  K advances in 32-wide slabs (one MFMA k-step)
// through a ring of four LDS stages of 32 KB filled by direct-to-LDS buffer loads, issued three
// slabs ahead.  (The 16 x 16 x 32 form moves less accumulator data per flop than 32 x 32 x 16;
// under the chip's power limit that runs at a higher clock for the same work.)
//
// The eight wavefronts form two groups of four, one wave of each group per SIMD (waves w and
// w + 4 share a SIMD), run half a period apart ("ping-pong"): while one group issues the
// thirty-two MFMAs of a slab (with its share of the global loads spread between them), the other
// reads the fragments of its next slab from LDS.  A workgroup barrier separates the phases, so
// each SIMD's matrix pipe is fed by one wave while the other waits on LDS.
//
// LDS rows are 64 B (32 bf16 = four 16-byte chunks); chunk c of row r sits at slot
// c ^ ((r >> 2) & 3), so the 16-byte fragment reads of 16 consecutive rows cover all 64 banks.
//
// Workgroups are numbered so that the ones dispatched to the same XCD (round-robin over 8)
// get consecutive tiles, and tiles are walked in groups of 5 row-panels, so each XCD's L2
// sees a compact set of A and B panels (the 32 tiles an XCD runs together span 5 row panels
// and 7 column panels).  On the 1024^2 pair stack, groups of 4, 6, 7 and 8 rows were 0.9, 0.3,
// 0.5 and ~3 % slower, of 16 rows slower still.
//
// Epilogues work from the accumulators, staged through LDS into 16-byte row chunks: plain bf16
// store (QKV), bias + fp32 store into a branch-strided buffer (embeds, final layer), fp32 gated
// residual read-modify-write (out projection, w2), and SwiGLU on paired W1 / W3 tiles (w1/w3).  There is no split-K:
// each output's sum runs over K in one fixed order, independent of M and of the tile.
#include "common.h"

namespace zdit {

namespace {

constexpr int BM = 256, BN = 256, BK = 32, NST = 4;
constexpr int STAGE_CHUNKS = 2 * BM * (BK / 8);  // A rows then B rows, 16-byte chunks (32 KB)
constexpr int DMA_PER_WAVE = 4;                  // 1 KB direct-to-LDS loads per wave per slab
// buffer resource word 3 for raw (untyped, offset-addressed) buffer loads
constexpr int kBufFlags = 0x00020000;
// s_waitcnt immediates: vmcnt in bits 3:0 (low) and 15:14 (high), expcnt in 6:4, lgkmcnt in
// 11:8; a field at its maximum does not wait
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kVmcnt0 = waitcnt_vm(0);
// all but the loads of the last NST - 2 slabs a wave issued
constexpr int kVmcntRing = waitcnt_vm((NST - 2) * DMA_PER_WAVE);
// group 1 at the end of its memory phase of slab k has issued up to slab k + NST - 2
constexpr int kVmcntG1 = waitcnt_vm((NST - 3) * DMA_PER_WAVE);
constexpr int kLgkmcnt0 = 0xC07F;                     // lgkmcnt(0)

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }
// v * sigmoid(v) with the hardware reciprocal (about 1 ulp): the product is rounded to bf16
__device__ __forceinline__ float silu_fast(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// Slot (16-byte units from the operand's first row) of logical chunk c of row r.
__device__ __forceinline__ int swz(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// Physical workgroup id -> (tile row, tile col).
__device__ __forceinline__ void tile_coords(int pid, int nwg, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  // XCD-aware renumbering: consecutive logical ids on the same XCD.
  const int xcd = pid & 7, idx = pid >> 3;
  const int full = nwg >> 3, rem = nwg & 7;
  const int lid = (xcd < rem) ? xcd * (full + 1) + idx : rem * (full + 1) + (xcd - rem) * full + idx;
  constexpr int G = 5;
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

// m / rpb for 0 <= m < 2^24 through a float reciprocal (rinv = 1 / rpb, rounded), corrected
// to the exact quotient: the float estimate is off by at most one.
__device__ __forceinline__ int div_rows(int m, int rpb, float rinv) {
  int b = (int)((float)m * rinv);
  const int r = m - b * rpb;
  b += (r >= rpb) - (r < 0);
  return b;
}

__device__ __forceinline__ void lds_dma_16(const __amdgpu_buffer_rsrc_t rs, const uint4* lds_base,
                                           int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16, voff,
                                           soff, 0, 0);
}

__device__ __forceinline__ void barrier_fenced() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Per-wave state of the main loop.
// v_mfma_f32_16x16x32_bf16: a wave's 64 x 128 is 4 x 8 tiles of 16 x 16; a fragment is 16 rows
// x 32 k (lane l: row l % 16, k 8 (l / 16) .. + 7), i.e. one whole 32-wide slab.
struct Frags {
  bf16x8 a[4];  // [16-row A tile]
  bf16x8 b[8];  // [16-row B tile]
};
typedef f32x4 AccT;
constexpr int ACC_I = 4, ACC_J = 8;

__device__ __forceinline__ void read_frags(const uint4* st, int arow, int brow, int fh, Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = __builtin_bit_cast(bf16x8, st[swz(arow + 16 * i, fh)]);
#pragma unroll
  for (int j = 0; j < 8; ++j) f.b[j] = __builtin_bit_cast(bf16x8, st[BM * 4 + swz(brow + 16 * j, fh)]);
}

__device__ __forceinline__ void mma_slab(const Frags& f, AccT (&acc)[4][8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Epilogue of one wave: its MT x 4 accumulator tiles cover rows m_wave .. m_wave + 32 MT - 1 and
// 128 columns from ncol_wave (SwiGLU: 64 output columns, W1 / W3 tiles paired).  stg is this
// wave's private staging space in LDS (at least 9216 bytes).
// Epilogue write-out of one wave's NBAND x 32 rows from m_wave and 64 NSUB columns from
// ncol_wave (SwiGLU: 64 output columns).  stage(band, sub, stg) writes the 32 x 64 sub-tile into
// the wave's private LDS staging space stg (row stride 288 B for fp32, 144 B for bf16, at least
// 9216 bytes); the rows are then written out as 16-byte chunks: fp32 4 values, bf16 8 values
// per lane, one row address per chunk.  The row padding keeps both the staging writes and the
// 16-byte read-back free of bank conflicts.
template <int EPI>
struct EpiFmt {
  static constexpr bool kPart = (EPI == EPI_PART || EPI == EPI_PART_SWIGLU);
  static constexpr bool kF32 = (EPI == EPI_BIAS || EPI == EPI_RESID || kPart);
  static constexpr int ES = kF32 ? 4 : 2;             // bytes per staged element
  static constexpr int VW = 16 / ES;                  // elements per 16-byte chunk
  static constexpr int CPR = 64 / VW;                 // chunks per 64-wide row
  static constexpr int STRIDE = 64 * ES + 16 * (ES / 2);  // fp32: 288 B, bf16: 144 B
  // 64-column sub-tiles per band (PART_SWIGLU: the W1 sums, then the W3 sums of 64 outputs)
  static constexpr int NSUB = (EPI == EPI_SWIGLU) ? 1 : 2;
};

// The B tile holds W1 and W3 rows in pairs (SwiGLU and its partial form).
template <int EPI>
constexpr bool kPaired = (EPI == EPI_SWIGLU || EPI == EPI_PART_SWIGLU);

// RoPE on 4 (x0, x1) pairs of a bf16 q or k chunk: y0 = x0 c - x1 s, y1 = x0 s + x1 c in fp32,
// each product and sum rounded (no contraction), then rounded to bf16 -- the same arithmetic
// as the stand-alone RoPE kernel.
__device__ __forceinline__ uint4 rope_chunk(uint4 v, float4 c4, float4 s4) {
#pragma clang fp contract(off)
  const bf16x8 x = __builtin_bit_cast(bf16x8, v);
  const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
  const float ss[4] = {s4.x, s4.y, s4.z, s4.w};
  bf16x8 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = (float)x[2 * i], x1 = (float)x[2 * i + 1];
    const float p0 = x0 * cc[i];
    const float p1 = x1 * ss[i];
    const float p2 = x0 * ss[i];
    const float p3 = x1 * cc[i];
    y[2 * i] = (bf16)(p0 - p1);
    y[2 * i + 1] = (bf16)(p2 + p3);
  }
  return __builtin_bit_cast(uint4, y);
}

template <int EPI, int NBAND, class Stage>
__device__ __forceinline__ void epilogue_out(const GemmArgs& g, void* Cbase, int m_wave, int ncol_wave, char* stg,
                                             int lane, Stage stage) {
  constexpr bool kF32 = EpiFmt<EPI>::kF32;
  constexpr int VW = EpiFmt<EPI>::VW, CPR = EpiFmt<EPI>::CPR, STRIDE = EpiFmt<EPI>::STRIDE;
  constexpr int NSUB = EpiFmt<EPI>::NSUB;
  const int rpb = g.out.rows_per_batch;
  const float rinv = 1.0f / (float)rpb;
  // 16-byte row chunks need 16-byte aligned rows
  const bool vec_ok = ((g.out.ld | g.out.batch_stride) % VW == 0) && (((uintptr_t)Cbase & 15) == 0) &&
                      (EPI != EPI_RESID || g.vec == nullptr || (g.vec_bstride % VW == 0 && ((uintptr_t)g.vec & 15) == 0)) &&
                      (EPI != EPI_BIAS || ((uintptr_t)g.vec & 15) == 0);
#pragma unroll
  for (int mt = 0; mt < NBAND; ++mt) {
#pragma unroll
    for (int p = 0; p < NSUB; ++p) {
      stage(mt, p, stg);
      // PART_SWIGLU's two sub-tiles are the W1 and W3 sums of the same 64 outputs
      const int ncol0 = ncol_wave + (EPI == EPI_PART_SWIGLU ? 0 : p * 64);
      if constexpr (EPI == EPI_QKV) {
        // v columns: the 32 rows of the sub-tile are 32 consecutive tokens of one branch
        // (rows per branch are a multiple of 32); write them transposed into V^T, 8 keys per
        // 16-byte chunk in the attention kernel's key order (chunk 2q of a 16-key group holds
        // keys 0-3 and 8-11, chunk 2q + 1 keys 4-7 and 12-15), zero at or past seq[b].
        const int D = g.N / 3;
        if (ncol0 >= 2 * D) {
          const int mrow = m_wave + mt * 32;
          if (mrow >= g.M || ncol0 >= g.N) continue;  // rows past M, columns past the last head
          const int b0 = div_rows(mrow, rpb, rinv), t0 = mrow - b0 * rpb;
          const int hd = (ncol0 - 2 * D) >> 7, d0 = (ncol0 - 2 * D) & 127;
          bf16* vt = (bf16*)g.vt + ((int64_t)(b0 * g.n_heads + hd) * kHeadDim + d0) * g.vt_pad + t0;
          const int sq = g.seq[b0];
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int c = it * 64 + lane, d = c >> 2, ch = c & 3;
            const int kb = (ch >> 1) * 16 + (ch & 1) * 4;
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int t = kb + (e & 3) + 8 * (e >> 2);
              const bf16 val = *(const bf16*)(stg + t * STRIDE + d * 2);
              o[e] = (t0 + t < sq) ? val : (bf16)0.f;
            }
            *(bf16x8*)(vt + (int64_t)d * g.vt_pad + ch * 8) = o;
          }
          continue;
        }
      }
      constexpr int NIT = 32 * CPR / 64;
      // PART_SWIGLU: the second sub-tile holds W3 sums, stored N columns further on
      const int64_t cadd = (EPI == EPI_PART_SWIGLU && p == 1) ? (int64_t)g.N : 0;
      // addresses of this lane's chunks; all global loads are issued before any is used
      int64_t off[NIT];
      int nn[NIT], bq[NIT], rq[NIT];
      bool ok[NIT], full[NIT];
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int c = it * 64 + lane, row = c / CPR, ch = c % CPR;
        const int m = m_wave + mt * 32 + row;
        nn[it] = ncol0 + ch * VW;
        const int mm = min(m, g.M - 1);
        bq[it] = div_rows(mm, rpb, rinv);
        const int rr = mm - bq[it] * rpb;
        rq[it] = rr;
        ok[it] = m < g.M && nn[it] < g.N && rr < g.out.valid[bq[it]];
        off[it] = bq[it] * g.out.batch_stride + (int64_t)rr * g.out.ld + nn[it] + cadd;
        full[it] = vec_ok && nn[it] + VW <= g.N;
      }
      if constexpr (EPI == EPI_RESID) {
        // All eight x chunks of the lane are in flight before the first use.  A lane's column
        // chunk is the same in every iteration, so its gate depends on the row's branch only:
        // with at least 32 rows per branch the sub-tile's rows span at most two branches, whose
        // gates are loaded once.
        float4 x[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          x[it] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (ok[it] && full[it]) x[it] = *(const float4*)((const float*)Cbase + off[it]);
        }
        const bool two = g.vec && rpb >= 32 && full[0];
        float4 g_lo = make_float4(1.f, 1.f, 1.f, 1.f), g_hi = g_lo;
        if (two) {
          g_lo = *(const float4*)(g.vec + bq[0] * g.vec_bstride + nn[0]);
          g_hi = *(const float4*)(g.vec + bq[NIT - 1] * g.vec_bstride + nn[0]);
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          if (!ok[it]) continue;
          const int c = it * 64 + lane, row = c / CPR, ch = c % CPR;
          const uint4 v = *(const uint4*)(stg + row * STRIDE + ch * 16);
          const float* vf = (const float*)&v;
          float* C = (float*)Cbase + off[it];
          if (full[it]) {
            float4 gv = bq[it] == bq[0] ? g_lo : g_hi;
            if (g.vec && !two) gv = *(const float4*)(g.vec + bq[it] * g.vec_bstride + nn[it]);
            *(float4*)C = make_float4(x[it].x + gv.x * vf[0], x[it].y + gv.y * vf[1],
                                      x[it].z + gv.z * vf[2], x[it].w + gv.w * vf[3]);
          } else {
            const float* gt = g.vec ? g.vec + bq[it] * g.vec_bstride + nn[it] : nullptr;
            for (int e = 0; e < VW && nn[it] + e < g.N; ++e) C[e] = C[e] + (gt ? gt[e] : 1.0f) * vf[e];
          }
        }
      } else {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          if (!ok[it]) continue;
          const int c = it * 64 + lane, row = c / CPR, ch = c % CPR;
          const uint4 v = *(const uint4*)(stg + row * STRIDE + ch * 16);
          const int n = nn[it];
          if constexpr (EPI == EPI_BIAS) {
            const float* vf = (const float*)&v;
            float* C = (float*)Cbase + off[it];
            if (full[it]) {
              const float4 bi = *(const float4*)(g.vec + n);
              *(float4*)C = make_float4(vf[0] + bi.x, vf[1] + bi.y, vf[2] + bi.z, vf[3] + bi.w);
            } else {
              for (int e = 0; e < VW && n + e < g.N; ++e) C[e] = vf[e] + g.vec[n + e];
            }
          } else if constexpr (EpiFmt<EPI>::kPart) {
            const float* vf = (const float*)&v;
            float* C = (float*)Cbase + off[it];
            if (full[it]) {
              *(uint4*)C = v;
            } else {
              for (int e = 0; e < VW && n + e < g.N; ++e) C[e] = vf[e];
            }
          } else if constexpr (EPI == EPI_QKV) {
            // q / k columns (rows per branch, head dim and N are multiples of 8: always full)
            const int b = bq[it], rr = rq[it];
            uint4 y = v;
            if (rr < g.seq[b]) {
              const int64_t toff = b * g.rope_bstride + (int64_t)rr * 64 + ((n & 127) >> 1);
              y = rope_chunk(v, *(const float4*)(g.rope_cos + toff), *(const float4*)(g.rope_sin + toff));
            }
            *(uint4*)((bf16*)Cbase + off[it]) = y;
          } else {
            bf16* C = (bf16*)Cbase + off[it];
            if (full[it]) {
              *(uint4*)C = v;
            } else {
              const bf16* vb = (const bf16*)&v;
              for (int e = 0; e < VW && n + e < g.N; ++e) C[e] = vb[e];
            }
          }
        }
      }
    }
  }
}


// Epilogue from 16 x 16 MFMA accumulators of a 16 NI x 128 wave tile: tile (i, j) element r of
// this lane is C[4 (lane / 16) + r][lane % 16] within the tile.  For SwiGLU, B tiles j and j + 2
// (j % 4 < 2) are the W1 and W3 rows of the same 16 outputs.
template <int EPI, int NI>
__device__ __forceinline__ void epilogue16(const GemmArgs& g, void* Cbase, const f32x4 (&acc)[NI][8], int m_wave,
                                           int ncol_wave, char* stg, int lane) {
  const int c16 = lane & 15, q4 = lane >> 4;
  constexpr int ES = EpiFmt<EPI>::ES, STRIDE = EpiFmt<EPI>::STRIDE;
  epilogue_out<EPI, NI / 2>(g, Cbase, m_wave, ncol_wave, stg, lane, [&](int mt, int p, char* st) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = ii * 16 + 4 * q4 + r;
          char* dst = st + row * STRIDE + (jj * 16 + c16) * ES;
          const int i = 2 * mt + ii;
          if constexpr (EPI == EPI_SWIGLU) {
            const int j1 = (jj >> 1) * 4 + (jj & 1);
            *(bf16*)dst = (bf16)(silu_fast(acc[i][j1][r]) * acc[i][j1 + 2][r]);
          } else if constexpr (EPI == EPI_PART_SWIGLU) {
            // sub-tile 0: the W1 tiles (0, 1, 4, 5), sub-tile 1: the W3 tiles (2, 3, 6, 7)
            const int j1 = (jj >> 1) * 4 + (jj & 1) + 2 * p;
            *(float*)dst = acc[i][j1][r];
          } else if constexpr (EPI == EPI_STORE || EPI == EPI_QKV) {
            *(bf16*)dst = (bf16)acc[i][4 * p + jj][r];
          } else {
            *(float*)dst = acc[i][4 * p + jj][r];
          }
        }
      }
    }
  });
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_bf16_kernel(GemmArgs g) {
  // one object per stage, so LDS reads of one stage are not ordered behind the in-flight
  // direct-to-LDS loads of another
  __shared__ uint4 st0[STAGE_CHUNKS];
  __shared__ uint4 st1[STAGE_CHUNKS];
  __shared__ uint4 st2[STAGE_CHUNKS];
  __shared__ uint4 st3[STAGE_CHUNKS];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform values live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, sw = wave & 3;   // group; the group's wave on SIMD sw
  const int wm = grp * 2 + (sw >> 1), wn = sw & 1;  // 64-row band, 128-column half
  const int nout_tile = kPaired<EPI> ? BN / 2 : BN;
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
  if constexpr (kPaired<EPI>)
    rb2_rs = __builtin_amdgcn_make_buffer_rsrc((void*)((const bf16*)g.B2 + (int64_t)n0 * g.ldb), 0, brec, kBufFlags);

  // Direct-to-LDS loads: group 0 fetches the A rows of a slab, group 1 the B rows, each wave
  // four 16-row blocks (1 KB each).  One instruction writes lane L at slot L of the block (row
  // L / 4, slot L % 4), so lane L fetches logical chunk (L % 4) ^ ((L / 16) % 4) of its row.
  // The row offset is in the per-lane (bounds-checked) offset; the K offset is scalar.
  // K range: the whole of K, or split blockIdx.y's range for the partial forms
  const int k_begin = EpiFmt<EPI>::kPart ? (int)blockIdx.y * g.k_split : 0;
  const int nk = (EpiFmt<EPI>::kPart ? min(g.K, k_begin + g.k_split) - k_begin : g.K) / BK;
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const int64_t ld = grp == 0 ? g.lda : g.ldb;
  int voff[DMA_PER_WAVE];
  __amdgpu_buffer_rsrc_t drs[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int blk = sw * DMA_PER_WAVE + i;  // tile rows blk*16 .. blk*16+15
    int row = blk * 16;
    drs[i] = grp == 0 ? ra_rs : rb_rs;
    if constexpr (kPaired<EPI>) {
      if (grp == 1) {
        // tile row t: wave column t / 128, MFMA tile (t % 128) / 32 (even: W1, odd: W3),
        // output column (t / 128) * 64 + (tile / 2) * 32 + t % 32
        const int t = blk * 16, wc = t >> 7, mt = (t & 127) >> 5;
        row = wc * 64 + (mt >> 1) * 32 + (t & 31);
        if (mt & 1) drs[i] = rb2_rs;
      }
    }
    voff[i] = (int)((row + (lane >> 2)) * ld * 2) + lchunk * 16;
  }
  const int dma_dst = (grp * BM + sw * DMA_PER_WAVE * 16) * 4;  // first chunk of this wave's blocks

  auto issue = [&](int kt, uint4* stage) {
    // past the end: reload the last slab into a dead stage
    const int kb = (k_begin + min(kt, nk - 1) * BK) * 2;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) lds_dma_16(drs[i], stage + dma_dst + i * 64, voff[i], kb);
  };

  AccT acc[ACC_I][ACC_J];
#pragma unroll
  for (int i = 0; i < ACC_I; ++i)
#pragma unroll
    for (int j = 0; j < ACC_J; ++j)
#pragma unroll
      for (int r = 0; r < (int)(sizeof(AccT) / 4); ++r) acc[i][j][r] = 0.f;

  const int fr = lane & 15, fh = lane >> 4;  // fragment row, 8-wide k group
  const int arow = wm * 64 + fr, brow = wn * 128 + fr;
  Frags f;

  // Prologue: slabs 0..NST-2 in flight, slab 0 landed and visible.
  issue(0, st0);
  issue(1, st1);
  issue(2, st2);
  __builtin_amdgcn_s_waitcnt(kVmcntRing);
  barrier_fenced();
  if (grp == 1) barrier_fenced();  // group 1 runs one phase behind

  // One slab: memory phase (read this slab's fragments), barrier, compute phase (the MFMAs,
  // with this wave's loads of slab kt+NST-1 into the stage freed by slab kt-1 spread between
  // them), barrier.  Group 0's loads of slab kt+1 are complete after its compute phase of slab
  // kt, group 1's after its memory phase of slab kt; both before the barrier that precedes
  // group 0's reads of slab kt+1.
#define ZDIT_SLAB(CUR, FREE, KT, MMA)                              \
  {                                                                \
    read_frags(CUR, arow, brow, fh, f);                            \
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);                         \
    if (grp == 1) __builtin_amdgcn_s_waitcnt(kVmcntG1);            \
    barrier_fenced();                                              \
    if (MMA) mma_slab(f, acc);                                     \
    issue((KT) + NST - 1, FREE);                                   \
    for (int q = 0; q < DMA_PER_WAVE; ++q) {                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);           \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);           \
    }                                                              \
    if (grp == 0) __builtin_amdgcn_s_waitcnt(kVmcntRing);          \
    if (grp == 0 || (KT) + 1 < nk) barrier_fenced();               \
  }

  // Whole turns of the ring, then the remaining slabs.  (The loop body is branch-free, so the
  // compiler sees every stage's last load exactly.)  Rows past M load as zero and are summed
  // like the others: skipping the MFMAs of waves whose rows all lie past M (a separate loop
  // copy for them) made the block's GEMMs 4-5 % slower on the same box, so they run as well.
#define ZDIT_LOOP(MMA)                                             \
  {                                                                \
    int kt = 0;                                                    \
    for (; kt + 4 <= nk; kt += 4) {                                \
      ZDIT_SLAB(st0, st3, kt, MMA)                                 \
      ZDIT_SLAB(st1, st0, kt + 1, MMA)                             \
      ZDIT_SLAB(st2, st1, kt + 2, MMA)                             \
      ZDIT_SLAB(st3, st2, kt + 3, MMA)                             \
    }                                                              \
    if (kt < nk) ZDIT_SLAB(st0, st3, kt, MMA)                      \
    if (kt + 1 < nk) ZDIT_SLAB(st1, st0, kt + 1, MMA)              \
    if (kt + 2 < nk) ZDIT_SLAB(st2, st1, kt + 2, MMA)              \
  }
  ZDIT_LOOP(true)
#undef ZDIT_LOOP
#undef ZDIT_SLAB
  // Loads of the slabs past the end are still landing in dead stages.  Once every wave has
  // drained its loads and passed this barrier, the LDS stages are free for the epilogue.
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  barrier_fenced();

  const int sidx = wave >> 1;
  char* const stg = (char*)(sidx == 0 ? st0 : sidx == 1 ? st1 : sidx == 2 ? st2 : st3) + (wave & 1) * 16384;
  // the partial forms write split blockIdx.y's plane [M][part_ld]
  void* Cbase = EpiFmt<EPI>::kPart ? (void*)(g.part + (int64_t)blockIdx.y * g.M * g.part_ld) : g.C;
  epilogue16<EPI, 4>(g, Cbase, acc, m0 + wm * 64, n0 + wn * (kPaired<EPI> ? 64 : 128), stg, lane);
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
  dim3 grid(tiles), block(512);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_STORE>, grid, block, 0, s, g); break;
    case EPI_BIAS: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_BIAS>, grid, block, 0, s, g); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_RESID>, grid, block, 0, s, g); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_SWIGLU>, grid, block, 0, s, g); break;
    case EPI_QKV: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_QKV>, grid, block, 0, s, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

SplitPlan tile_split_plan(int epi, int N, int K) {
  // At most 128 workgroups per 256-row panel, so that a branch of up to 512 rows (two panels)
  // runs in one round on 256 CUs; at most 8 ranges and ranges of at least 16 slabs.  More ranges
  // spread the work over more CUs but write and read one more fp32 partial plane each, and a
  // second round of workgroups costs a whole tile time: on the 256 px block (two panels) two
  // ranges instead of four for q/k/v and one instead of two for w1/w3 took the block from 0.366
  // to 0.326 ms.  From N and K only, so a row's sums do not depend on M.
  SplitPlan p;
  const bool paired = epi == EPI_SWIGLU;
  const int n_tiles = (N + (paired ? BN / 2 : BN) - 1) / (paired ? BN / 2 : BN);
  const int max_splits = std::max(1, std::min(8, K / 512));
  const int splits = std::min(max_splits, std::max(1, 128 / n_tiles));
  p.k_split = ((K + splits - 1) / splits + BK - 1) / BK * BK;
  p.splits = (K + p.k_split - 1) / p.k_split;
  p.Nv = paired ? 2 * N : N;
  return p;
}

size_t tile_split_workspace(int epi, int M, int N, int K) {
  const SplitPlan p = tile_split_plan(epi, N, K);
  return p.splits == 1 ? 0 : (size_t)p.splits * M * p.Nv * sizeof(float);
}

hipError_t launch_gemm_bf16_split(int epi, const GemmArgs& g, float* part, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (epi != EPI_STORE && epi != EPI_RESID && epi != EPI_SWIGLU) return hipErrorInvalidValue;
  const SplitPlan p = tile_split_plan(epi, g.N, g.K);
  // one range: the whole-K kernel with the epilogue itself (no partial plane, no reduction)
  if (p.splits == 1) return launch_gemm_bf16(epi, g, s);
  GemmArgs pg = g;
  pg.C = part;
  pg.part = part;
  pg.k_split = p.k_split;
  pg.part_ld = p.Nv;
  pg.out.rows_per_batch = g.M;
  pg.out.batch_stride = 0;
  pg.out.ld = p.Nv;
  for (int b = 0; b < kMaxBatch; ++b) pg.out.valid[b] = g.M;
  const bool paired = epi == EPI_SWIGLU;
  const int nout_tile = paired ? BN / 2 : BN;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + nout_tile - 1) / nout_tile);
  dim3 grid(tiles, p.splits), block(512);
  // one partial plane per split: the kernel offsets C by split * M * Nv itself
  if (paired) hipLaunchKernelGGL(gemm_bf16_kernel<EPI_PART_SWIGLU>, grid, block, 0, s, pg);
  else hipLaunchKernelGGL(gemm_bf16_kernel<EPI_PART>, grid, block, 0, s, pg);
  if (hipError_t e = hipGetLastError()) return e;
  SplitKArgs a{};
  a.part = part;
  a.M = g.M;
  a.N = g.N;
  a.Nv = p.Nv;
  a.splits = p.splits;
  return launch_splitk_reduce(epi, a, g, s);
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
