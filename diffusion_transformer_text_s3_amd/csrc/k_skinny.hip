// C = A B^T for few rows (M <= 256): the text encoder's projections on its valid tokens, where
// the 256 x 256 tiles of the main GEMM would occupy a few dozen of the 256 CUs while the time
// goes into streaming the weights from HBM.
//
// Split-K with the weights streamed into registers.  A 512-thread workgroup owns one tile of up
// to 64 rows, 128 columns of C and one K range; wavefront w owns columns n0 + 16 w .. + 15.  Per
// 32-wide slab a lane loads 16 bytes of its weight row (the B fragment of
// v_mfma_f32_16x16x32_bf16: row l % 16, k 8 (l / 16) ..) KU_B slabs ahead, so each wavefront
// keeps 16 KB of weights in flight, reads the four A fragments (16-row tiles) from LDS and
// issues four MFMAs.  A arrives in LDS in chunks of 256 columns (32 KB), double-buffered and
// fetched one chunk ahead by direct-to-LDS loads; one barrier per chunk.  The K ranges are whole
// multiples of 256 columns except the last, their number depends on N and K only (at most
// about 256 workgroups per row tile, one per CU), so every output's sum has the same K split and
// order whatever M is.  The fp32 partial tiles go to a workspace [splits][M][Nv]; a second
// kernel sums them in split order and applies the epilogue: bf16 store, fp32 gated residual add, or SwiGLU on the
// paired W1 / W3 partials (Nv = 2N: the W3 columns follow the W1 columns).  Optional row maps
// gather the rows of A and scatter the rows of C, so a caller can run only the valid rows of a
// padded batch.  The reduction can also carry the work that follows it (SplitKFuse): the
// encoder's q/k RMSNorm + RoPE after the q/k/v projection, or the RMSNorm after a residual add.
// Buffer resources make rows past M or N read as zero.
//
// The weights may also come packed (pack_bfrag_kernel): each band of 16 rows stored slab after
// slab, a slab being the 64 lanes' 16-byte fragments in lane order, so a wavefront reads one
// contiguous 1 KB run per slab instead of 16 pieces of 64 bytes K * 2 bytes apart.  Only the
// weight addresses change: same fragments, same order, bit-identical results.
#include "common.h"

namespace zdit {

namespace {

constexpr int KM = 64;                  // rows per tile
constexpr int KNW = 16;                 // columns per wavefront
constexpr int KWG = 8 * KNW;            // columns per workgroup
constexpr int KSL = 32;                 // slab width (one MFMA k-step)
constexpr int KU_B = 16;                // weight slabs in flight per lane
constexpr int KCH = 256;                // A chunk width (K columns)
constexpr int KCH_SL = KCH / KSL;       // 8 slabs per chunk
constexpr int KCH_CPR = KCH / 8;        // 32 16-byte chunks per A row of a chunk
constexpr int KCH_CHUNKS = KM * KCH_CPR;  // 2048 (32 KB)
constexpr int KCH_DMA = KCH_CHUNKS / 64 / 8;  // 4 wave loads per wave per chunk
constexpr int kSBufFlags = 0x00020000;
constexpr int s_waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ssilu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// LDS slot of logical 16-byte chunk c of A row r within a chunk buffer: the 16 rows of one
// fragment read hit 16 distinct bank groups
__device__ __forceinline__ int aslot(int r, int c) { return r * KCH_CPR + (c ^ (r & 15)); }

__device__ __forceinline__ void sdma_16(const __amdgpu_buffer_rsrc_t rs, const uint4* lds_base, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff,
                                           0, 0);
}

// RES = 0: A chunks double-buffered, one barrier per chunk.  RES = 2 or 4: a K range of at most
// RES chunks has all of them resident (RES x 32 KB of LDS), loaded together with the first
// weight slabs; one barrier, then every slab of the range with no further wait for A, so the
// weight stream keeps KU_B slabs in flight throughout (the double-buffered form drops to 8 at each
// chunk boundary, where its wait for the next chunk's loads also covers the older weight loads).
template <int RES>
__global__ __launch_bounds__(512) void gemm_splitk_kernel(SplitKArgs a) {
  // separate objects, so reads of one chunk buffer are not ordered behind the in-flight
  // direct-to-LDS writes of another
  __shared__ uint4 A0[KCH_CHUNKS], A1[KCH_CHUNKS];
  __shared__ uint4 A2[RES > 2 ? KCH_CHUNKS : 1], A3[RES > 2 ? KCH_CHUNKS : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ct = blockIdx.x, split = blockIdx.y, m0 = blockIdx.z * KM;
  const bool direct = a.swiglu_direct != 0;
  // SwiGLU: the W3 half of the virtual columns (direct: of the workgroup's waves)
  const bool second = direct ? wave >= 4 : ct >= a.col_tiles;
  const int n0 = direct ? ct * (KWG / 2) + (wave & 3) * KNW : (second ? ct - a.col_tiles : ct) * KWG + wave * KNW;
  const int k0 = split * a.ks;
  const int kr = min(a.K, k0 + a.ks) - k0;  // K columns of this range
  const int nk = kr / KSL;                  // slabs (>= 1)
  const int nch = (kr + KCH - 1) / KCH;     // A chunks
  const int fr = lane & 15, fh = lane >> 4;

  // weight rows n0 .. n0 + 15; rows past N fall outside the resource.  Offsets are unsigned.
  const bf16* bb = (const bf16*)(second ? a.B2 : a.B) + (int64_t)min(n0, a.N) * a.ldb;
  const __amdgpu_buffer_rsrc_t brs =
      __builtin_amdgcn_make_buffer_rsrc((void*)bb, 0, max(0, a.N - n0) * a.ldb * 2, kSBufFlags);
  // row-major: lane l reads 16 bytes of row fr at column k0 + 32 t + 8 fh (16 rows of 64 bytes per
  // slab); packed: slab k0 / 32 + t of the band is 1 KB in a row, the lane's chunk at 16 l
  const unsigned bvo = a.packed ? (unsigned)(k0 * 32 + lane * 16) : (unsigned)(fr * a.ldb * 2 + fh * 16 + k0 * 2);
  const unsigned bstep = a.packed ? 1024u : (unsigned)(KSL * 2);
  // slabs past the range reload the last one (branch-free); no MFMA uses them
  auto ldb = [&](int t) {
    return __builtin_amdgcn_raw_buffer_load_b128(brs, (int)(bvo + (unsigned)min(t, nk - 1) * bstep), 0, 0);
  };

  // A chunk loads: wave load j of this wave fills slots 64 (KCH_DMA wave + j) + lane, i.e. row
  // 2 (KCH_DMA wave + j) + lane / 32 and physical chunk lane % 32; the lane fetches the logical chunk
  // that belongs there.  A row past M gets an offset past the end of the resource (2^31 + k
  // stays out of range), so it loads as zero.
  const bool gather = a.a_rows != nullptr;
  const bf16* ab = (const bf16*)a.A + (gather ? 0 : (int64_t)m0 * a.lda);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ab, 0, (gather ? a.a_phys_rows : max(0, a.M - m0)) * a.lda * 2, kSBufFlags);
  unsigned avo[KCH_DMA];
#pragma unroll
  for (int j = 0; j < KCH_DMA; ++j) {
    const int r = 2 * (KCH_DMA * wave + j) + (lane >> 5);
    const int c = (lane & 31) ^ (r & 15);
    const int m = m0 + r;
    const unsigned row = m < a.M ? (unsigned)(gather ? a.a_rows[m] : r) * (unsigned)(a.lda * 2) : 0x80000000u;
    avo[j] = row + (unsigned)(c * 16);
  }
  // The chunk's K offset goes into the per-lane offset, which the hardware checks against the
  // resource: in the last range's last chunk, columns past K of the last row lie past the end of
  // A and load as zero instead of reading whatever follows A (the scalar offset is not checked).
  // An invalid row's 2^31 base plus the offset (< 2^31) stays out of range.
  auto dma_a = [&](int ch, uint4* buf) {
    const unsigned coff = (unsigned)(k0 + min(ch, nch - 1) * KCH) * 2u;
#pragma unroll
    for (int j = 0; j < KCH_DMA; ++j) sdma_16(ars, buf + (KCH_DMA * wave + j) * 64, (int)(avo[j] + coff), 0);
  };

  u32x4 bq[KU_B];
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One chunk of A in buffer CUR (every wave's loads landed), the next one's loads go to NXT
  // (every wave finished reading it before the barrier that ended the previous chunk).  Its 8
  // slabs: the weights of slab T from bq, the A fragments from CUR, four MFMAs, then the weight
  // load of slab T + KU_B.  Slabs past the range (in its last chunk) issue no MFMA, so the A
  // columns there never enter a sum.  At the end: this wave's chunk loads (issued before the
  // chunk's 8 weight loads) are complete, then the barrier.  A macro, so that each LDS access
  // names its own buffer object.
#define ZDIT_SK_CHUNK(CH, CUR, NXT)                                                                    \
  {                                                                                                   \
    const int ch_ = (CH);                                                                             \
    dma_a(ch_ + 1, NXT);                                                                              \
    _Pragma("unroll") for (int s = 0; s < KCH_SL; ++s) {                                              \
      const int tt = ch_ * KCH_SL + s;                                                                \
      const int q = (ch_ & 1) * KCH_SL + s; /* ring slot: chunks alternate halves of bq */           \
      if (tt < nk) {                                                                                  \
        const bf16x8 bf = __builtin_bit_cast(bf16x8, bq[q]);                                          \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                               \
          const int r = 16 * i + fr;                                                                  \
          const bf16x8 af = __builtin_bit_cast(bf16x8, CUR[aslot(r, s * 4 + fh)]);                    \
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[i], 0, 0, 0);                  \
        }                                                                                             \
      }                                                                                               \
      bq[q] = ldb(tt + KU_B);                                                                         \
    }                                                                                                 \
    __builtin_amdgcn_s_waitcnt(s_waitcnt_vm(KCH_SL));                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                                \
    __builtin_amdgcn_s_barrier();                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                                \
  }

  // The slabs of one resident chunk CH in buffer CUR (RES > 0): no loads of A, no barrier.
#define ZDIT_SK_RESIDENT(CH, CUR)                                                                      \
  {                                                                                                   \
    _Pragma("unroll") for (int s = 0; s < KCH_SL; ++s) {                                              \
      const int tt = (CH) * KCH_SL + s;                                                               \
      const int q = ((CH) & 1) * KCH_SL + s;                                                          \
      if (tt < nk) {                                                                                  \
        const bf16x8 bf = __builtin_bit_cast(bf16x8, bq[q]);                                          \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                               \
          const int r = 16 * i + fr;                                                                  \
          const bf16x8 af = __builtin_bit_cast(bf16x8, CUR[aslot(r, s * 4 + fh)]);                    \
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[i], 0, 0, 0);                  \
        }                                                                                             \
      }                                                                                               \
      bq[q] = ldb(tt + KU_B);                                                                         \
    }                                                                                                 \
  }

  if constexpr (RES == 0) {
    dma_a(0, A0);
#pragma unroll
    for (int u = 0; u < KU_B; ++u) bq[u] = ldb(u);
    __builtin_amdgcn_s_waitcnt(s_waitcnt_vm(KU_B));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    int ch = 0;
    for (; ch + 2 <= nch; ch += 2) {
      ZDIT_SK_CHUNK(ch, A0, A1)
      ZDIT_SK_CHUNK(ch + 1, A1, A0)
    }
    if (ch < nch) ZDIT_SK_CHUNK(ch, A0, A1)
  } else {
    // every chunk of the range (nch <= RES), then the first weight slabs; waiting until at most
    // KU_B loads are in flight leaves exactly those weight loads, so all of A has landed
    dma_a(0, A0);
    if (nch > 1) dma_a(1, A1);
    if constexpr (RES > 2) {
      if (nch > 2) dma_a(2, A2);
      if (nch > 3) dma_a(3, A3);
    }
#pragma unroll
    for (int u = 0; u < KU_B; ++u) bq[u] = ldb(u);
    __builtin_amdgcn_s_waitcnt(s_waitcnt_vm(KU_B));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    ZDIT_SK_RESIDENT(0, A0)
    if (nch > 1) ZDIT_SK_RESIDENT(1, A1)
    if constexpr (RES > 2) {
      if (nch > 2) ZDIT_SK_RESIDENT(2, A2)
      if (nch > 3) ZDIT_SK_RESIDENT(3, A3)
    }
  }
#undef ZDIT_SK_CHUNK
#undef ZDIT_SK_RESIDENT
  // the loads past the range are still landing
  __builtin_amdgcn_s_waitcnt(s_waitcnt_vm(0));

  // lane holds rows 4 (lane / 16) + e of each 16 x 16 tile, column lane % 16
  if (direct) {
    // after this barrier every chunk read and every direct-to-LDS write has completed, so A0
    // carries the W3 sums of waves 4-7 to waves 0-3 (same lane, same rows and columns)
    float* w3s = (float*)A0;
    __syncthreads();
    if (wave >= 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) w3s[((wave - 4) * 16 + i * 4 + e) * 64 + lane] = acc[i][e];
    }
    __syncthreads();
    const int n = n0 + fr;
    if (wave < 4 && n < a.N) {
      bf16* u = (bf16*)a.u_out + n;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + 16 * i + 4 * fh + e;
          const float w3 = w3s[(wave * 16 + i * 4 + e) * 64 + lane];
          if (m < a.M) u[(int64_t)m * a.u_ld] = (bf16)(ssilu(acc[i][e]) * w3);
        }
    }
    return;
  }
  // partial tile
  const int n = n0 + fr;
  if (n >= a.N) return;
  float* part = a.part + (int64_t)split * a.M * a.Nv + (second ? a.N : 0) + n;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + 16 * i + 4 * fh + e;
      if (m < a.M) part[(int64_t)m * a.Nv] = acc[i][e];
    }
}

// One thread per 4 consecutive output columns of a row: the partials summed in split order,
// then the epilogue.
// Sums of the float4 at p0 + k * plane (and at p1 + k * plane) over the ranges k, in order;
// the loads of up to 16 ranges are issued before their adds.
__device__ __forceinline__ void sum_ranges(const float* p0, const float* p1, int64_t plane, int splits, float4& s0,
                                           float4& s1) {
  constexpr int KB = 16;
  s0 = s1 = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < splits; k0 += KB) {
    float4 t0[KB], t1[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i)
      if (k0 + i < splits) {
        t0[i] = *(const float4*)(p0 + (k0 + i) * plane);
        if (p1) t1[i] = *(const float4*)(p1 + (k0 + i) * plane);
      }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if (k0 + i >= splits) break;
      if (k0 + i == 0) {
        s0 = t0[i];
        if (p1) s1 = t1[i];
      } else {
        s0.x += t0[i].x; s0.y += t0[i].y; s0.z += t0[i].z; s0.w += t0[i].w;
        if (p1) { s1.x += t1[i].x; s1.y += t1[i].y; s1.z += t1[i].z; s1.w += t1[i].w; }
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(SplitKArgs a, GemmArgs g) {
  const int nq = a.N >> 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.M * nq) return;
  const int m = (int)(i / nq), n = (int)(i % nq) * 4;
  const int64_t plane = (int64_t)a.M * a.Nv;
  const float* p = a.part + (int64_t)m * a.Nv + n;
  float4 s, u;
  sum_ranges(p, EPI == EPI_SWIGLU ? p + a.N : nullptr, plane, a.splits, s, u);
  const RowMap& rm = g.out;
  int b;
  int64_t off;
  if (a.c_rows) {
    const int row = a.c_rows[m];
    b = row / rm.rows_per_batch;
    off = (int64_t)row * rm.ld + n;
  } else {
    b = m / rm.rows_per_batch;
    const int r = m - b * rm.rows_per_batch;
    if (r >= rm.valid[b]) return;
    off = b * rm.batch_stride + (int64_t)r * rm.ld + n;
  }
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
      o[0] = ssilu(s.x) * u.x; o[1] = ssilu(s.y) * u.y; o[2] = ssilu(s.z) * u.z; o[3] = ssilu(s.w) * u.w;
    }
    bf16x4 ob;
#pragma unroll
    for (int e = 0; e < 4; ++e) ob[e] = (bf16)o[e];
    *(bf16x4*)((bf16*)g.C + off) = ob;
  }
}

// The q/k/v reduction with the encoder's per-head RMSNorm and RoPE: 16 lanes per (row, head),
// lane j holding dims 8 j .. 8 j + 7; the partner of dim i < 64 is dim i + 64, in lane j ^ 8.
// Sums in split order, then for q and k heads y = x / sqrt(mean(x^2) + eps) * g and
// y_i c - y_{i+64} s, y_{i+64} c + y_i s (each product and sum rounded separately), one rounding
// to bf16; v heads are rounded as summed.
__global__ __launch_bounds__(256) void splitk_reduce_qkv_kernel(SplitKArgs a, GemmArgs g, SplitKFuse f) {
#pragma clang fp contract(off)
  const int nh = f.n_heads + 2 * f.n_kv_heads;
  const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int j = threadIdx.x & 15;
  if (item >= (int64_t)a.M * nh) return;  // whole 16-lane groups leave together
  const int m = (int)(item / nh), hh = (int)(item % nh);
  const int col = hh * kHeadDim + j * 8;
  const int64_t plane = (int64_t)a.M * a.Nv;
  const float* p = a.part + (int64_t)m * a.Nv + col;
  float4 lo, hi;
  sum_ranges(p, p + 4, plane, a.splits, lo, hi);
  const float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  const int row = a.c_rows[m];
  bf16x8 out;
  if (hh < f.n_heads + f.n_kv_heads) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) ss += __shfl_xor(ss, d, 64);
    const float den = sqrtf(ss / (float)kHeadDim + f.eps);
    const float* gv = (hh < f.n_heads ? f.gq : f.gk) + j * 8;
    float y[8], yp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[e] / den * gv[e];
#pragma unroll
    for (int e = 0; e < 8; ++e) yp[e] = __shfl_xor(y[e], 8, 64);
    const int b = row / f.L, r = row - b * f.L;
    const int64_t tb = b * f.tab_bstride + (int64_t)r * 64 + (j & 7) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = f.cos[tb + e], sn = f.sin[tb + e];
      const float t0 = y[e] * c, t1 = yp[e] * sn;
      out[e] = (bf16)(j < 8 ? t0 - t1 : t0 + t1);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (bf16)x[e];
    if (f.vt) {
      // value head hk, token r of branch b -> V^T row (b, hk, d), key position: within each
      // 16-key group, key t sits in chunk (t >> 2) & 1 at element (t & 3) + 4 (t >> 3)
      const int b = row / f.L, r = row - b * f.L;
      const int hk = hh - f.n_heads - f.n_kv_heads;
      const int t = r & 15;
      const int pos = ((r >> 4) * 2 + ((t >> 2) & 1)) * 8 + (t & 3) + 4 * (t >> 3);
      bf16* vt = (bf16*)f.vt + ((int64_t)(b * f.n_kv_heads + hk) * kHeadDim + j * 8) * f.s_pad + pos;
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(int64_t)e * f.s_pad] = out[e];
      return;
    }
  }
  *(bf16x8*)((bf16*)g.C + (int64_t)row * g.out.ld + col) = out;
}

// The residual reduction with the following RMSNorm: one workgroup per row.  x += sum of the
// partials (times the gate if any), then h = x / sqrt(mean(x^2) + eps) * gain as bf16 (the same
// formula as the RMSNorm kernel).  Rows up to 4096 wide: one 4-column group per thread
// (blockDim = N / 4 rounded up to a wavefront), the row's x and gate loads issued before the sums.
__global__ __launch_bounds__(1024) void splitk_reduce_resid_norm_kernel(SplitKArgs a, GemmArgs g, SplitKFuse f) {
  __shared__ float wsum[16];
  const int m = blockIdx.x, c = threadIdx.x;
  const int nq = a.N >> 2;
  const bool on = c < nq;
  const int64_t plane = (int64_t)a.M * a.Nv;
  const int row = a.c_rows[m];
  const int b = row / g.out.rows_per_batch;
  float* x = (float*)g.C + (int64_t)row * g.out.ld + 4 * c;
  const float* gate = g.vec ? g.vec + b * g.vec_bstride + 4 * c : nullptr;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f), gv = make_float4(1.f, 1.f, 1.f, 1.f);
  float ss = 0.f;
  if (on) {
    v = *(const float4*)x;
    if (gate) gv = *(const float4*)gate;
    float4 s4, unused;
    sum_ranges(a.part + (int64_t)m * a.Nv + 4 * c, nullptr, plane, a.splits, s4, unused);
    if (gate) {
      v.x += gv.x * s4.x; v.y += gv.y * s4.y; v.z += gv.z * s4.z; v.w += gv.w * s4.w;
    } else {
      v.x += s4.x; v.y += s4.y; v.z += s4.z; v.w += s4.w;
    }
    *(float4*)x = v;
    ss = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((c & 63) == 0) wsum[c >> 6] = ss;
  __syncthreads();
  const int nw = blockDim.x >> 6;
  ss = wsum[0];
  for (int w = 1; w < nw; ++w) ss += wsum[w];
  const float rinv = 1.0f / sqrtf(ss / (float)a.N + f.eps);
  if (on) {
    const float4 gg = *(const float4*)(f.gain + 4 * c);
    bf16x4 o;
    o[0] = (bf16)(v.x * rinv * gg.x); o[1] = (bf16)(v.y * rinv * gg.y);
    o[2] = (bf16)(v.z * rinv * gg.z); o[3] = (bf16)(v.w * rinv * gg.w);
    *(bf16x4*)((bf16*)f.h + (int64_t)row * a.N + 4 * c) = o;
  }
}

}  // namespace

SplitKArgs splitk_plan(int epi, int M, int N, int K) {
  SplitKArgs a{};
  a.M = M; a.N = N; a.K = K;
  a.col_tiles = (N + KWG - 1) / KWG;
  a.Nv = epi == EPI_SWIGLU ? 2 * N : N;
  const int vtiles = epi == EPI_SWIGLU ? 2 * a.col_tiles : a.col_tiles;
  // at most about 256 workgroups for one row tile (one per CU); ranges of whole 256-column
  // chunks
  const int units = (K + KCH - 1) / KCH;
  const int ranges = max(1, 256 / vtiles);
  a.ks = ((units + ranges - 1) / ranges) * KCH;
  a.splits = (K + a.ks - 1) / a.ks;
  return a;
}

namespace {
// one thread per 16-byte chunk of the packed matrix, in packed order (coalesced writes)
__global__ __launch_bounds__(256) void pack_bfrag_kernel(const uint4* src, uint4* dst, int N, int K) {
  const int64_t n = (int64_t)N * K / 8;
  const int slabs = K / KSL;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int l = (int)(i & 63);
    const int64_t bt = i >> 6;
    const int t = (int)(bt % slabs);
    const int64_t band = bt / slabs;
    const int64_t row = band * 16 + (l & 15);
    const int col = t * KSL + 8 * (l >> 4);
    dst[i] = src[(row * K + col) >> 3];
  }
}
}  // namespace

hipError_t launch_pack_bfrag(const void* src, void* dst, int N, int K, hipStream_t s) {
  if (N % 16 || K % KSL) return hipErrorInvalidValue;
  const int64_t n = (int64_t)N * K / 8;
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(pack_bfrag_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint4*)src, (uint4*)dst, N, K);
  return hipGetLastError();
}

size_t splitk_workspace(int epi, int M, int N, int K) {
  const SplitKArgs a = splitk_plan(epi, M, N, K);
  return (size_t)a.splits * M * a.Nv * sizeof(float);
}

hipError_t launch_splitk_reduce(int epi, const SplitKArgs& a, const GemmArgs& g, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const unsigned rb = (unsigned)(((int64_t)a.M * (a.N / 4) + 255) / 256);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_STORE>, dim3(rb), dim3(256), 0, s, a, g); break;
    case EPI_RESID: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_RESID>, dim3(rb), dim3(256), 0, s, a, g); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_SWIGLU>, dim3(rb), dim3(256), 0, s, a, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_splitk(int epi, const GemmArgs& g, float* part, hipStream_t s, const int* a_rows,
                              int a_phys_rows, const int* c_rows, const SplitKFuse* fuse, bool b_packed) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (b_packed && (g.N % 16 || g.K % KSL || g.ldb != g.K)) return hipErrorInvalidValue;
  SplitKArgs a = splitk_plan(epi, g.M, g.N, g.K);
  a.packed = b_packed ? 1 : 0;
  a.A = g.A; a.B = g.B; a.B2 = g.B2; a.part = part; a.lda = (int)g.lda; a.ldb = (int)g.ldb;
  a.a_rows = a_rows; a.a_phys_rows = a_phys_rows; a.c_rows = c_rows;
  const int vtiles = epi == EPI_SWIGLU ? 2 * a.col_tiles : a.col_tiles;
  const bool direct = epi == EPI_SWIGLU && a.splits == 1 && !c_rows && (!fuse || fuse->kind == SplitKFuse::NONE) &&
                      g.out.rows_per_batch >= g.M && g.out.valid[0] >= g.M;
  if (direct) {
    a.swiglu_direct = 1;
    a.u_out = g.C;
    a.u_ld = g.out.ld;
  }
  dim3 grid(direct ? (g.N + KWG / 2 - 1) / (KWG / 2) : vtiles, a.splits, (g.M + KM - 1) / KM);
  const int nch = a.ks / KCH;  // chunks of a full range
  if (nch <= 2)
    hipLaunchKernelGGL(gemm_splitk_kernel<2>, grid, dim3(512), 0, s, a);
  else if (nch <= 4)
    hipLaunchKernelGGL(gemm_splitk_kernel<4>, grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_splitk_kernel<0>, grid, dim3(512), 0, s, a);
  if (direct) return hipGetLastError();
  if (fuse && fuse->kind == SplitKFuse::QK_NORM_ROPE) {
    if (epi != EPI_STORE || !c_rows) return hipErrorInvalidValue;
    const int64_t lanes = (int64_t)g.M * (fuse->n_heads + 2 * fuse->n_kv_heads) * 16;
    hipLaunchKernelGGL(splitk_reduce_qkv_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, a, g, *fuse);
    return hipGetLastError();
  }
  if (fuse && fuse->kind == SplitKFuse::RESID_NORM) {
    if (epi != EPI_RESID || !c_rows || g.N > 4096 || g.N % 4) return hipErrorInvalidValue;
    const unsigned threads = (unsigned)((g.N / 4 + 63) / 64 * 64);
    hipLaunchKernelGGL(splitk_reduce_resid_norm_kernel, dim3(g.M), dim3(threads), 0, s, a, g, *fuse);
    return hipGetLastError();
  }
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
