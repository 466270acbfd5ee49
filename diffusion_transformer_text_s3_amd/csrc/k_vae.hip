// fp32 kernels of the 16-channel AutoencoderKL decoder (Core AI model zoo, "Z-Image-Turbo
// port", table "Architecture -> export mapping", row VAE: the decoder runs in fp32 and
// upsamples by nearest neighbour).  Activations are NHWC fp32 so that a pixel's channels are
// contiguous: the 3x3 convolutions run as implicit GEMMs on the fp32 MFMA (v_mfma_f32_16x16x4
// _f32), reading each (pixel, tap) as a 64-byte channel slice and the 2x nearest upsample as
// input addresses at half the coordinates.  Two forms: the direct one loads its tiles straight
// into LDS and takes inputs that need no transform (the decoder writes SiLU(GroupNorm(x)) once
// per convolution input, vact_kernel, and takes the GroupNorm statistics from the producing
// convolution's epilogue); the staged one applies a GroupNorm affine and SiLU while it stages
// the input tile through registers.  Both sum in the same order.
#include <math.h>

#include <algorithm>

#include "vae.h"

namespace zdit {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kVM = 128;     // output pixels per tile
constexpr int kVN = 128;     // output channels per tile
constexpr int kVK = 16;      // channels of one tap per K step
constexpr int kVLd = 16;     // LDS row: the 16 channels of a K step, 64 bytes

// 16-byte chunk c of LDS row r sits at chunk c ^ ((r >> 2) & 3), as in the bf16 GEMM: a wave's
// fragment reads (16 consecutive rows, one chunk each) cover all banks.
__device__ inline int vlds(int r, int c) { return r * kVLd + ((c ^ ((r >> 2) & 3)) << 2); }

// SiLU with the hardware exp2 and reciprocal (each within a few ulp): t / (1 + e^-t)
__device__ inline float silu_f(float t) { return t * __builtin_amdgcn_rcpf(1.0f + __expf(-t)); }

// The result tile of one wave: rows m_base + 16 i + 4 (l / 16) + e, columns n_base + 16 j + l % 16
// of each 16 x 16 MFMA tile (lane l, register e): alpha * acc + bias (+ the residual), NHWC rows of
// ldc floats or NCHW planes.  The residual values of a 16-row slice are loaded before its first
// store, so those loads are in flight together (each element is read and written by its own lane
// only, so a residual that aliases the output is still read before it is overwritten).
template <int RJ, bool STATS = false>
__device__ __forceinline__ void vconv_epilogue(const VConvArgs& a, f4 (&acc)[4][RJ], int m_base, int n_base,
                                               int lane) {
  const int fr = lane & 15, fk = 4 * (lane >> 4);
  const int hw = a.H * a.W;
  auto offset = [&](int m, int n) -> int64_t {
    if (a.out_nchw) {
      const int im = m / hw;
      return ((int64_t)im * a.N + n) * hw + (m - im * hw);
    }
    return (int64_t)m * a.ldc + n;
  };
  float bv[RJ];
#pragma unroll
  for (int j = 0; j < RJ; ++j) {
    const int n = n_base + 16 * j + fr;
    bv[j] = a.bias && n < a.N ? a.bias[n] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the residual of one 16-row slice: 4 RJ loads in flight, then the stores
    f4 rv[RJ];
    if (a.res) {
#pragma unroll
      for (int j = 0; j < RJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m_base + 16 * i + fk + e, n = n_base + 16 * j + fr;
          rv[j][e] = m < a.M && n < a.N ? a.res[offset(m, n)] : 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int n = n_base + 16 * j + fr;
      if (n >= a.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m_base + 16 * i + fk + e;
        if (m >= a.M) continue;
        float v = a.alpha * acc[i][j][e] + bv[j];
        if (a.res) v = rv[j][e] + v;
        a.C[offset(m, n)] = v;
        if constexpr (STATS) acc[i][j][e] = v;
      }
    }
  }
  if constexpr (STATS) {
    if (!a.gn_part) return;
    // GroupNorm statistics of this wave's 64 rows (a half tile), per column: the mean of the
    // valid rows, then the sum of squared deviations from it.  A column's 64 rows are 16 values
    // in each of the four lanes l % 16 + 16 g; the lanes combine by two xor exchanges, which
    // leave the same sum in all four.
    const int nv = min(max(a.M - m_base, 0), 64);
    if (nv == 0) return;
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) t += 16 * i + fk + e < nv ? acc[i][j][e] : 0.f;
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
      const float mean = t / (float)nv;
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d = 16 * i + fk + e < nv ? acc[i][j][e] - mean : 0.f;
          q = fmaf(d, d, q);
        }
      q += __shfl_xor(q, 16);
      q += __shfl_xor(q, 32);
      const int n = n_base + 16 * j + fr;
      if (lane < 16 && n < a.N) a.gn_part[(int64_t)(m_base >> 6) * a.N + n] = make_float2(mean, q);
    }
  }
}

// 256 threads = 4 wavefronts, each owning 64 rows x (BN / (4 / (BM / 64))) columns of the
// BM x BN output tile as 16 x 16 MFMA tiles: BM = BN = 128 (a 2 x 2 wave grid, 64 x 64 per
// wave, 64 fp32 accumulators per lane) for the convolutions and GEMMs, BM = 256, BN = 16 (4 x 1,
// 64 x 16 per wave) for the output conv to 3 channels.  One K step = 16 channels of one tap:
// the A tile (BM pixels x 16) and the B tile (BN output channels x 16) are loaded into
// registers one step ahead, transformed, and written to the other half of a double-buffered
// LDS ring; one barrier per step.  A lane reads its fragment as one 16-byte row chunk: lane l
// feeds k = 4 * (l / 16) + kk of the step in the kk-th MFMA, for A and B alike.
template <int BM, int BN>
__global__ __launch_bounds__(256) void vconv_kernel(VConvArgs a) {
  constexpr int TA = 256 / BM;          // loader threads per A row
  constexpr int FA = 4 / TA;            // float4 of one A row per loader thread
  constexpr int WGM = BM / 64;          // wave grid rows
  constexpr int WGN = 4 / WGM;          // wave grid columns
  constexpr int RJ = BN / WGN / 16;     // 16-wide column tiles per wave
  constexpr int FB = 4 * BN >= 256 ? 4 * BN / 256 : 1;  // float4 of B per loader thread
  constexpr int TB = 4 / FB;            // loader threads per B row
  __shared__ __attribute__((aligned(16))) float sA[2][BM * kVLd];
  __shared__ __attribute__((aligned(16))) float sB[2][BN * kVLd];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const float* A = a.A;
  const float* B = a.B;
  const int hw = a.H * a.W;

  // A loader: tile row lr, channels 4 FA lh .. of the step; B loader: row br, part bh
  const int lr = tid / TA, lh = tid % TA;
  const int am = m0 + lr;
  const bool arow = am < a.M;
  int img = 0, py = 0, px = 0;
  if (arow) {
    img = am / hw;
    const int rem = am - img * hw;
    py = rem / a.W;
    px = rem - py * a.W;
  }
  const int br = tid / TB, bh = tid % TB;
  const bool bload = br < BN;
  const int bn = n0 + br;
  const bool brow = bload && bn < a.N;
  const float* Brow = B + (int64_t)(brow ? bn : 0) * a.ldb;
  const int rad = a.ksize >> 1;
  const int Hs = a.upsample ? a.H >> 1 : a.H, Ws = a.upsample ? a.W >> 1 : a.W;
  const int csteps = (a.K + kVK - 1) / kVK;
  const int nsteps = a.ksize * a.ksize * csteps;
  const float* aff = a.affine ? a.affine + (int64_t)img * a.K * 2 : nullptr;

  f4 ra[FA], rb[FB], rf[2 * FA];  // rf: (a, d) pairs of the A channels
  bool aval = false;
  int ac = 0;
  // position of the next step to load: tap (ky, kx) and channel step cst, advanced in order
  int ky = 0, kx = 0, tap = 0, cst = 0;
  auto load = [&]() {
    const int cs = cst * kVK;
    const int c0 = cs + 4 * FA * lh;
    const int yy = py + ky - rad, xx = px + kx - rad;
    aval = arow && yy >= 0 && yy < a.H && xx >= 0 && xx < a.W;
    ac = c0;
    const float* src = A;
    if (aval) {
      const int ys = a.upsample ? yy >> 1 : yy, xs = a.upsample ? xx >> 1 : xx;
      src = A + ((int64_t)(img * Hs + ys) * Ws + xs) * a.lda + c0;
    }
#pragma unroll
    for (int j = 0; j < FA; ++j) {
      const bool cin = c0 + 4 * j < a.K;  // K % 4 == 0: a 4-channel group is all in or all out
      ra[j] = (aval && cin) ? *(const f4*)(src + 4 * j) : f4{0.f, 0.f, 0.f, 0.f};
      if (aff) {
        rf[2 * j] = cin ? *(const f4*)(aff + 2 * (c0 + 4 * j)) : f4{0.f, 0.f, 0.f, 0.f};
        rf[2 * j + 1] = cin ? *(const f4*)(aff + 2 * (c0 + 4 * j) + 4) : f4{0.f, 0.f, 0.f, 0.f};
      }
    }
    const int cb = cs + 4 * FB * bh;
    const float* wsrc = Brow + (int64_t)tap * a.K + cb;
#pragma unroll
    for (int j = 0; j < FB; ++j)
      rb[j] = (brow && cb + 4 * j < a.K) ? *(const f4*)(wsrc + 4 * j) : f4{0.f, 0.f, 0.f, 0.f};
    if (++cst == csteps) {
      cst = 0;
      ++tap;
      if (++kx == a.ksize) {
        kx = 0;
        ++ky;
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < FA; ++j) {
      f4 v = ra[j];
      if (aff) {  // uniform; the per-lane choice is a select, so no copies of v are made early
        const bool tr = aval && ac + 4 * j < a.K;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f4 ad = rf[2 * j + (e >> 1)];
          const float t = fmaf(ad[2 * (e & 1)], v[e], ad[2 * (e & 1) + 1]);
          float y = a.silu ? silu_f(t) : t;
          asm volatile("" : "+v"(y));  // computed on every lane: the choice below stays a select
          v[e] = tr ? y : v[e];
        }
      }
      *(f4*)&sA[buf][vlds(lr, FA * lh + j)] = v;
    }
    if (bload) {
#pragma unroll
      for (int j = 0; j < FB; ++j) *(f4*)&sB[buf][vlds(br, FB * bh + j)] = rb[j];
    }
  };

  const int wm0 = (wave % WGM) * 64, wn0 = (wave / WGM) * (BN / WGN);
  const int fr = lane & 15, fc = lane >> 4;
  f4 acc[4][RJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < RJ; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  load();
  store(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load();
    f4 af[4], bf[RJ];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *(const f4*)&sA[buf][vlds(wm0 + 16 * i + fr, fc)];
#pragma unroll
    for (int j = 0; j < RJ; ++j) bf[j] = *(const f4*)&sB[buf][vlds(wn0 + 16 * j + fr, fc)];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < RJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][kk], bf[j][kk], acc[i][j], 0, 0, 0);
    // The wait for the next step's loads stays below the MFMAs.  The transform and LDS stores
    // run at raised wave priority: the other workgroups on the CU are then in their MFMA
    // phases, and this wave gets back to its own MFMAs sooner.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    if (s + 1 < nsteps) store(buf ^ 1);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }

  vconv_epilogue<RJ>(a, acc, m0 + wm0, n0 + wn0, lane);
}

// ------------------------------------------------------------ convolution, direct-to-LDS form
// The same tiles, K steps, LDS layout, fragment reads and MFMA order as vconv_kernel<BM, BN>
// (so the same sums in the same order), for inputs that need no transform: the A and B tiles
// go from memory straight into LDS with buffer loads (buffer_load_dword ... lds), no staging
// registers, selects or LDS stores, and two steps ahead through a ring of three stages.
// The fp32 MFMA shares its issue cycles with the vector ALU, so the fewer vector instructions
// per MFMA the better.
// Each operand is read through a buffer resource over the rows one tile can touch (bounds
// checked by the hardware): a lane's offset is past the end for output rows past M, for taps
// outside the image and for weight rows past N, and such a load returns zeros.  A lane's A
// offsets change only when the tap does; the channel step is the scalar offset.
// Tile shapes: 128 x 128 (2 x 2 waves of 64 x 64; each wave loads two 16-row blocks of A and two
// of B per step) and 256 x 16 for the output conv (4 x 1 waves of 64 x 16; each wave loads four A
// blocks and its own copy of the one B block, so every wave issues the same number of loads).
template <int BM, int BN>
struct VDirect {
  static constexpr int WGM = BM / 64, WGN = 4 / WGM;
  static constexpr int RJ = BN / WGN / 16;           // 16-wide column tiles per wave
  static constexpr int ABLK = BM / 64;               // A blocks per wave
  static constexpr bool PRIV_B = BN < 64;            // B private to each wave
  static constexpr int BBLK = PRIV_B ? BN / 16 : BN / 64;
  static constexpr int LOADS = ABLK + BBLK;          // loads per wave per step
  static constexpr int BROWS = PRIV_B ? 4 * BN : BN;  // B rows in a stage
  static constexpr int STAGE = (BM + BROWS) * kVLd;   // floats: A rows, then B rows
};
constexpr int kBufFlags = 0x00020000;   // raw (offset-addressed) buffer, word 3
constexpr int kOob = 0x7ffffff0;        // an offset past every resource's end
// s_waitcnt immediate waiting for vmcnt <= n only (expcnt and lgkmcnt fields at their maximum)
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

__device__ __forceinline__ void vdma16(__amdgpu_buffer_rsrc_t rs, float* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void vbarrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Source pixels (within the tile's image) that the tile's output rows read: [lo, hi).
struct VSpan {
  int img, lo, hi;
};
template <int BM>
__device__ __forceinline__ VSpan vconv_span(const VConvArgs& a, int m0) {
  const int hw = a.H * a.W;
  VSpan sp;
  sp.img = m0 / hw;
  const int p0 = m0 - sp.img * hw;                   // first output pixel in the image
  const int p1 = min(m0 + BM, min(a.M, (sp.img + 1) * hw)) - 1 - sp.img * hw;  // last
  const int rad = a.ksize >> 1;
  const int Ws = a.upsample ? a.W >> 1 : a.W;
  if (a.H == 1) {  // one row per image (GEMM mode): columns
    int x0 = max(0, p0 - rad), x1 = min(a.W - 1, p1 + rad);
    if (a.upsample) { x0 >>= 1; x1 >>= 1; }
    sp.lo = x0;
    sp.hi = x1 + 1;
  } else {
    int y0 = max(0, p0 / a.W - rad), y1 = min(a.H - 1, p1 / a.W + rad);
    if (a.upsample) { y0 >>= 1; y1 >>= 1; }
    sp.lo = y0 * Ws;
    sp.hi = (y1 + 1) * Ws;
  }
  return sp;
}

template <int BM, int BN>
__global__ __launch_bounds__(256, BM == 128 ? 3 : 2) void vconv_direct_kernel(VConvArgs a) {
  using D = VDirect<BM, BN>;
  __shared__ __attribute__((aligned(16))) float st0[D::STAGE];
  __shared__ __attribute__((aligned(16))) float st1[D::STAGE];
  __shared__ __attribute__((aligned(16))) float st2[D::STAGE];
  const int tid = threadIdx.x;
  // the wave index in a scalar register: the LDS destinations of the loads are then scalar
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int hw = a.H * a.W;
  const int rad = a.ksize >> 1;
  const int Hs = a.upsample ? a.H >> 1 : a.H, Ws = a.upsample ? a.W >> 1 : a.W;
  const int csteps = a.K / kVK;  // K % 16 == 0 on this path
  const int nsteps = a.ksize * a.ksize * csteps;

  const VSpan sp = vconv_span<BM>(a, m0);
  const float* Abase = a.A + ((int64_t)sp.img * Hs * Ws + sp.lo) * a.lda;
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void*)Abase, 0, (int)((int64_t)(sp.hi - sp.lo) * a.lda * 4), kBufFlags);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.B + (int64_t)n0 * a.ldb), 0, (int)((int64_t)min(a.N - n0, BN) * a.ldb * 4), kBufFlags);

  // This wave loads A blocks ABLK wave + i and B blocks BBLK wave + i (or, B private, all of B
  // into its own copy); one instruction puts lane L at slot L of a 16-row block (row L / 4,
  // 16-byte slot L % 4), so lane L fetches the logical chunk whose swizzled slot that is.
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  int py[D::ABLK], px[D::ABLK], voa[D::ABLK], vob[D::BBLK];
  bool mok[D::ABLK];
#pragma unroll
  for (int i = 0; i < D::ABLK; ++i) {
    const int r = (D::ABLK * wave + i) * 16 + (lane >> 2);
    const int m = m0 + r;
    mok[i] = m < a.M;
    const int p = m - sp.img * hw;
    py[i] = p / a.W;
    px[i] = p - py[i] * a.W;
  }
#pragma unroll
  for (int i = 0; i < D::BBLK; ++i) {
    const int r = ((D::PRIV_B ? 0 : D::BBLK * wave) + i) * 16 + (lane >> 2);
    vob[i] = n0 + r < a.N ? (int)(r * a.ldb * 4) + lchunk * 16 : kOob;
  }
  const int bdst = D::PRIV_B ? BM + wave * BN : BM + D::BBLK * wave * 16;  // first B row this wave loads
  // A offsets of the tap (ky, kx)
  auto tap_offsets = [&](int ky, int kx) {
#pragma unroll
    for (int i = 0; i < D::ABLK; ++i) {
      const int yy = py[i] + ky - rad, xx = px[i] + kx - rad;
      const bool ok = mok[i] && yy >= 0 && yy < a.H && xx >= 0 && xx < a.W;
      const int ys = a.upsample ? yy >> 1 : yy, xs = a.upsample ? xx >> 1 : xx;
      voa[i] = ok ? (ys * Ws + xs - sp.lo) * (int)a.lda * 4 + lchunk * 16 : kOob;
    }
  };

  // issue position: tap (iky, ikx), channel step ics; past the last step the last one repeats
  // (into a stage no one reads again) so that every step has the same number of loads
  int iky = 0, ikx = 0, itap = 0, ics = 0, issued = 0;
  tap_offsets(0, 0);
  auto issue = [&](float* stage) {
    const int soa = ics * kVK * 4, sob = (itap * a.K + ics * kVK) * 4;
#pragma unroll
    for (int i = 0; i < D::ABLK; ++i) vdma16(rsa, stage + (D::ABLK * wave + i) * 16 * kVLd, voa[i], soa);
#pragma unroll
    for (int i = 0; i < D::BBLK; ++i) vdma16(rsb, stage + (bdst + i * 16) * kVLd, vob[i], sob);
    if (++issued < nsteps) {
      if (++ics == csteps) {
        ics = 0;
        ++itap;
        if (++ikx == a.ksize) {
          ikx = 0;
          ++iky;
        }
        tap_offsets(iky, ikx);
      }
    }
  };

  const int wm0 = (wave % D::WGM) * 64, wn0 = (wave / D::WGM) * (BN / D::WGN);
  const int fr = lane & 15, fc = lane >> 4;
  f4 acc[4][D::RJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < D::RJ; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  // one step: this wave's loads of the step have landed (the next step's may still be in
  // flight), the barrier makes every wave's visible and frees the stage read in the step
  // before, which takes the loads of two steps ahead
  auto step = [&](const float* cur, float* freed) {
    __builtin_amdgcn_s_waitcnt(vm_wait(D::LOADS));
    vbarrier();
    issue(freed);
    const float* sA = cur;
    const float* sB = cur + (D::PRIV_B ? BM + wave * BN : BM) * kVLd;
    f4 af[4], bf[D::RJ];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *(const f4*)&sA[vlds(wm0 + 16 * i + fr, fc)];
#pragma unroll
    for (int j = 0; j < D::RJ; ++j) bf[j] = *(const f4*)&sB[vlds(wn0 + 16 * j + fr, fc)];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < D::RJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][kk], bf[j][kk], acc[i][j], 0, 0, 0);
  };

  issue(st0);
  issue(st1);
  int s = 0;
  for (; s + 3 <= nsteps; s += 3) {
    step(st0, st2);
    step(st1, st0);
    step(st2, st1);
  }
  if (s < nsteps) step(st0, st2);
  if (s + 1 < nsteps) step(st1, st0);
  // the loads past the end are still landing in dead stages: drain them before the wave ends
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  vconv_epilogue<D::RJ, true>(a, acc, m0 + wm0, n0 + wn0, lane);
}

// GroupNorm from the half-tile statistics of a convolution (mean_h, M2_h over n_h rows per
// channel), combined in float64 with the pairwise update of Chan, Golub and LeVeque: merging
// (n_a, m_a, M2_a) and (n_b, m_b, M2_b) gives n = n_a + n_b, m = m_a + (m_b - m_a) n_b / n and
// M2 = M2_a + M2_b + (m_b - m_a)^2 n_a n_b / n.  Every merge runs in a fixed order.
__device__ __forceinline__ void chan_merge(double& n, double& m, double& q, double nb, double mb, double qb) {
  if (nb == 0.0) return;  // an empty set (a thread with no chunks)
  const double t = n + nb, d = mb - m;
  m += d * nb / t;
  q += qb + d * d * n * nb / t;
  n = t;
}

constexpr int kGnChunk = 16;  // half tiles per workgroup of the first level

// First level, one workgroup per (chunk of kGnChunk half tiles, image): per channel (one thread,
// coalesced over the channels) the chunk's count, mean and M2 (the exact two-sum identity
// M2 = sum of M2_h + n_h (m_h - m)^2), then per group the channels merged in order.
__global__ __launch_bounds__(256) void vgn_conv_chunk_kernel(const float2* part, VGnArgs a, double* chunk) {
  __shared__ double cs[3][1024];
  const int tid = threadIdx.x;
  const int ck = blockIdx.x, img = blockIdx.y;
  const int hpi = (a.HW + 63) / 64;
  const int h0 = ck * kGnChunk, h1 = min(h0 + kGnChunk, hpi);
  const float2* p = part + (int64_t)img * hpi * a.C;
  for (int c = tid; c < a.C; c += 256) {
    double n = 0.0, sum = 0.0;
    for (int h = h0; h < h1; ++h) {
      const double nh = (double)min(64, a.HW - 64 * h);
      n += nh;
      sum += nh * (double)p[(int64_t)h * a.C + c].x;
    }
    const double m = sum / n;
    double q = 0.0;
    for (int h = h0; h < h1; ++h) {
      const double nh = (double)min(64, a.HW - 64 * h);
      const float2 v = p[(int64_t)h * a.C + c];
      const double d = (double)v.x - m;
      q += (double)v.y + nh * d * d;
    }
    cs[0][c] = n;
    cs[1][c] = m;
    cs[2][c] = q;
  }
  __syncthreads();
  const int cpg = a.C / a.groups;
  for (int g = tid; g < a.groups; g += 256) {
    const int c0 = g * cpg;
    double n = cs[0][c0], m = cs[1][c0], q = cs[2][c0];
    for (int cc = 1; cc < cpg; ++cc) chan_merge(n, m, q, cs[0][c0 + cc], cs[1][c0 + cc], cs[2][c0 + cc]);
    double* o = chunk + (((int64_t)img * gridDim.x + ck) * a.groups + g) * 3;
    o[0] = n;
    o[1] = m;
    o[2] = q;
  }
}

// Second level, one workgroup per (group, image): thread t merges chunks t, t + 256, ... in
// order, then the 256 results merge pairwise in a fixed tree; then 1/sqrt(M2 / n + eps) and the
// per-channel affine, as vgn_finalize_kernel.
__global__ __launch_bounds__(256) void vgn_conv_final_kernel(const double* chunk, int nck, VGnArgs a) {
  __shared__ double rn[256], rm[256], rq[256];
  const int tid = threadIdx.x;
  const int g = blockIdx.x, img = blockIdx.y;
  const double* c = chunk + ((int64_t)img * nck * a.groups + g) * 3;
  double n = 0.0, m = 0.0, q = 0.0;
  for (int k = tid; k < nck; k += 256) {
    const double* e = c + (int64_t)k * a.groups * 3;
    chan_merge(n, m, q, e[0], e[1], e[2]);
  }
  rn[tid] = n;
  rm[tid] = m;
  rq[tid] = q;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      double n2 = rn[tid], m2 = rm[tid], q2 = rq[tid];
      chan_merge(n2, m2, q2, rn[tid + w], rm[tid + w], rq[tid + w]);
      rn[tid] = n2;
      rm[tid] = m2;
      rq[tid] = q2;
    }
    __syncthreads();
  }
  const double mean = rm[0], rstd = 1.0 / sqrt(rq[0] / rn[0] + (double)a.eps);
  if (tid == 0) {
    double* st = a.stat + ((int64_t)img * a.groups + g) * 2;
    st[0] = mean;
    st[1] = rstd;
  }
  const int cpg = a.C / a.groups;
  for (int cc = tid; cc < cpg; cc += 256) {
    const int ch = g * cpg + cc;
    const double ga = (double)a.gamma[ch] * rstd;
    a.affine[((int64_t)img * a.C + ch) * 2] = (float)ga;
    a.affine[((int64_t)img * a.C + ch) * 2 + 1] = (float)((double)a.beta[ch] - mean * ga);
  }
}

// out = SiLU(a x + d) (silu != 0) or a x + d per (image, channel), with the affine of
// [images][C][2]; the same arithmetic as the transform of vconv_kernel.  out may alias x.
__global__ __launch_bounds__(256) void vact_kernel(const float* x, const float* affine, int64_t quads_per_image,
                                                   int cq, int64_t quads, int silu, float* out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < quads; i += (int64_t)gridDim.x * 256) {
    const int64_t img = i / quads_per_image;
    const int q = (int)(i & (cq - 1));
    const float* ad = affine + (img * cq * 4 + 4 * q) * 2;
    const f4 ad0 = *(const f4*)ad, ad1 = *(const f4*)(ad + 4);
    f4 v = *(const f4*)(x + 4 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f4 p = e < 2 ? ad0 : ad1;
      const float t = fmaf(p[2 * (e & 1)], v[e], p[2 * (e & 1) + 1]);
      v[e] = silu ? silu_f(t) : t;
    }
    *(f4*)(out + 4 * i) = v;
  }
}

// ------------------------------------------------------------------------------ GroupNorm
// Partial sums over one chunk of pixels of one image: pass 0 sums x, pass 1 sums (x - mean)^2
// with the group's mean from the first pass.  256 threads: C / 4 channel quads across, 256 /
// (C / 4) pixels down; the per-thread sums are added per channel in a fixed order.
__global__ __launch_bounds__(256) void vgn_partial_kernel(VGnArgs a, int pass) {
  __shared__ f4 red[256];
  const int tid = threadIdx.x;
  const int img = blockIdx.y, chunk = blockIdx.x;
  const int Q = a.C >> 2, rows = 256 / Q;
  const int q = tid % Q, r = tid / Q;
  const int p0 = chunk * a.chunk, p1 = min(p0 + a.chunk, a.HW);
  const int cpg = a.C / a.groups;
  f4 m = f4{0.f, 0.f, 0.f, 0.f};
  if (pass) {
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] = (float)a.stat[((int64_t)img * a.groups + (4 * q + e) / cpg) * 2];
  }
  f4 s = f4{0.f, 0.f, 0.f, 0.f};
  const float* x = a.x + (int64_t)img * a.HW * a.C + 4 * q;
  for (int p = p0 + r; p < p1; p += rows) {
    const f4 v = *(const f4*)(x + (int64_t)p * a.C);
    if (pass) {
      const f4 d = v - m;
      s += d * d;
    } else {
      s += v;
    }
  }
  red[tid] = s;
  __syncthreads();
  const int nch = gridDim.x;
  for (int c = tid; c < a.C; c += 256) {
    float t = 0.f;
    for (int rr = 0; rr < rows; ++rr) t += red[rr * Q + (c >> 2)][c & 3];
    a.part[((int64_t)img * nch + chunk) * a.C + c] = t;
  }
}

// One workgroup per (group, image): the chunk partials of the group's channels summed in
// float64 in a fixed order; pass 0 stores the mean, pass 1 1/sqrt(var + eps) and the
// per-channel affine (a, d) = (gamma rstd, beta - mean gamma rstd).
__global__ __launch_bounds__(256) void vgn_finalize_kernel(VGnArgs a, int nch, int pass) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int g = blockIdx.x, img = blockIdx.y;
  const int cpg = a.C / a.groups;
  const int n = nch * cpg;
  double t = 0.0;
  for (int i = tid; i < n; i += 256) {
    const int ch = i / cpg, cc = i - ch * cpg;
    t += (double)a.part[((int64_t)img * nch + ch) * a.C + g * cpg + cc];
  }
  red[tid] = t;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const double cnt = (double)a.HW * cpg;
  double* st = a.stat + ((int64_t)img * a.groups + g) * 2;
  if (pass == 0) {
    if (tid == 0) st[0] = red[0] / cnt;
    return;
  }
  const double mean = st[0];
  const double rstd = 1.0 / sqrt(red[0] / cnt + (double)a.eps);
  if (tid == 0) st[1] = rstd;
  for (int cc = tid; cc < cpg; cc += 256) {
    const int c = g * cpg + cc;
    const double ga = (double)a.gamma[c] * rstd;
    a.affine[((int64_t)img * a.C + c) * 2] = (float)ga;
    a.affine[((int64_t)img * a.C + c) * 2 + 1] = (float)((double)a.beta[c] - mean * ga);
  }
}

// ------------------------------------------------------------------------------ small kernels
__global__ void vlatent_in_kernel(const float* z, float* out, int images, int ch, int h, int w, int unscale,
                                  float scale, float shift) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)images * ch * h * w;
  if (i >= n) return;
  // i indexes the NHWC output: ((img * h + y) * w + x) * ch + c
  const int c = (int)(i % ch);
  const int64_t pix = i / ch;
  const int x = (int)(pix % w);
  const int64_t t = pix / w;
  const int y = (int)(t % h);
  const int img = (int)(t / h);
  const float v = z[(((int64_t)img * ch + c) * h + y) * w + x];
  out[i] = unscale ? v / scale + shift : v;
}

// one workgroup per row: max, then the sum of exp(s - max), then exp(s - max) / sum
// A row of at most 1024 Q values per workgroup held in registers (Q float4 per thread, columns
// 4 (t + 256 k) .. + 3): one read and one write of the row, the same arithmetic as
// vsoftmax_kernel (expf of s - max, then an IEEE division by the sum; the sum's order differs).
template <int Q>
__global__ __launch_bounds__(256) void vsoftmax_reg_kernel(float* S, int n) {
  __shared__ float red[8];
  float* row = S + (int64_t)blockIdx.x * n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nq = n >> 2;
  f4 v[Q];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const int q = tid + 256 * k;
    v[k] = q < nq ? *(const f4*)(row + 4 * q) : f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    mx = fmaxf(mx, fmaxf(fmaxf(v[k][0], v[k][1]), fmaxf(v[k][2], v[k][3])));
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float sm = 0.f;
#pragma unroll
  for (int k = 0; k < Q; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[k][e] = expf(v[k][e] - mx);  // exp(-inf) = 0 past the row's end
      sm += v[k][e];
    }
  for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o);
  if (lane == 0) red[4 + wave] = sm;
  __syncthreads();
  sm = (red[4] + red[5]) + (red[6] + red[7]);
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const int q = tid + 256 * k;
    if (q < nq) *(f4*)(row + 4 * q) = v[k] / sm;
  }
}

__global__ __launch_bounds__(256) void vsoftmax_kernel(float* S, int n) {
  __shared__ float red[256];
  float* row = S + (int64_t)blockIdx.x * n;
  const int tid = threadIdx.x;
  float mx = -INFINITY;
  for (int j = tid; j < n; j += 256) mx = fmaxf(mx, row[j]);
  red[tid] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float sm = 0.f;
  for (int j = tid; j < n; j += 256) sm += expf(row[j] - mx);
  red[tid] = sm;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  sm = red[0];
  for (int j = tid; j < n; j += 256) row[j] = expf(row[j] - mx) / sm;
}

__global__ void vtranspose_kernel(const float* in, int64_t ld, int c0, float* out, int n, int C) {
  __shared__ float t[32][33];
  const int j0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
  const float* src = in + c0;
  for (int r = threadIdx.y; r < 32; r += 8) {
    const int j = j0 + r, c = k0 + threadIdx.x;
    t[r][threadIdx.x] = (j < n && c < C) ? src[(int64_t)j * ld + c] : 0.f;
  }
  __syncthreads();
  float* dst = out;
  for (int r = threadIdx.y; r < 32; r += 8) {
    const int c = k0 + r, j = j0 + threadIdx.x;
    if (c < C && j < n) dst[(int64_t)c * n + j] = t[threadIdx.x][r];
  }
}

}  // namespace

namespace {
bool direct_ok(const VConvArgs& a, int BM, int BN) {
  if (a.affine || a.K % kVK || a.lda % 4 || a.ldb % 4) return false;
  if (((uintptr_t)a.A | (uintptr_t)a.B) & 15) return false;
  const int64_t hw = (int64_t)a.H * a.W;
  if (a.M != hw && hw % BM) return false;  // a tile lies in one image
  // the largest span of source rows a tile can read, in bytes, within a 32-bit buffer offset
  const int64_t Ws = a.upsample ? a.W / 2 : a.W;
  const int rad = a.ksize / 2;
  const int64_t px = a.H == 1 ? BM + 2 * rad : (BM / a.W + 2 + 2 * rad) * Ws;
  const int64_t limit = (int64_t)0x7fffffff - 4096;
  if (px * a.lda * 4 > limit || (int64_t)BN * a.ldb * 4 > limit) return false;
  if ((int64_t)a.ksize * a.ksize * a.K * 4 > limit) return false;
  return true;
}
}  // namespace

bool vconv_direct_ok(const VConvArgs& a) { return a.N <= 16 ? direct_ok(a, 256, 16) : direct_ok(a, kVM, kVN); }

hipError_t launch_vconv(const VConvArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const bool direct = vconv_direct_ok(a);
  if (a.N <= 16) {  // the output conv (3 channels): 256 x 16 tiles
    dim3 grid((a.M + 255) / 256, 1);
    if (direct)
      hipLaunchKernelGGL((vconv_direct_kernel<256, 16>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((vconv_kernel<256, 16>), grid, dim3(256), 0, s, a);
  } else {
    dim3 grid((a.M + kVM - 1) / kVM, (a.N + kVN - 1) / kVN);
    if (direct)
      hipLaunchKernelGGL((vconv_direct_kernel<kVM, kVN>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((vconv_kernel<kVM, kVN>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_vact(const float* x, const float* affine, int images, int64_t hw, int C, int silu, float* out,
                       hipStream_t s) {
  const int64_t quads = (int64_t)images * hw * C / 4;
  if (quads == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((quads + 255) / 256, 256 * 64);
  hipLaunchKernelGGL(vact_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, affine, hw * C / 4, C / 4, quads,
                     silu, out);
  return hipGetLastError();
}

int vgn_chunks(int HW, int C) {
  const int chunk = std::max(256 / (C / 4), 65536 / C);
  return (HW + chunk - 1) / chunk;
}

size_t vgn_part_floats(int images, int HW, int C) { return (size_t)images * vgn_chunks(HW, C) * C; }

size_t vgn_conv_chunk_doubles(int images, int HW, int groups) {
  const int hpi = (HW + 63) / 64;
  return (size_t)images * ((hpi + kGnChunk - 1) / kGnChunk) * groups * 3;
}

hipError_t launch_vgn_from_conv(const float2* part, double* chunk, const VGnArgs& a, hipStream_t s) {
  const int hpi = (a.HW + 63) / 64;
  const int nck = (hpi + kGnChunk - 1) / kGnChunk;
  hipLaunchKernelGGL(vgn_conv_chunk_kernel, dim3(nck, a.images), dim3(256), 0, s, part, a, chunk);
  hipLaunchKernelGGL(vgn_conv_final_kernel, dim3(a.groups, a.images), dim3(256), 0, s, chunk, nck, a);
  return hipGetLastError();
}

hipError_t launch_vgn(VGnArgs a, hipStream_t s) {
  a.chunk = std::max(256 / (a.C / 4), 65536 / a.C);
  const int nch = vgn_chunks(a.HW, a.C);
  for (int pass = 0; pass < 2; ++pass) {
    hipLaunchKernelGGL(vgn_partial_kernel, dim3(nch, a.images), dim3(256), 0, s, a, pass);
    hipLaunchKernelGGL(vgn_finalize_kernel, dim3(a.groups, a.images), dim3(256), 0, s, a, nch, pass);
  }
  return hipGetLastError();
}

hipError_t launch_vlatent_in(const float* z, float* out, int images, int ch, int h, int w, int unscale,
                             float scale, float shift, hipStream_t s) {
  const int64_t n = (int64_t)images * ch * h * w;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(vlatent_in_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, z, out, images, ch, h, w,
                     unscale, scale, shift);
  return hipGetLastError();
}

hipError_t launch_vsoftmax(float* S, int64_t rows, int n, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 g((unsigned)rows), b(256);
  if (n % 4 || ((uintptr_t)S & 15) || n > 16384)
    hipLaunchKernelGGL(vsoftmax_kernel, g, b, 0, s, S, n);
  else if (n <= 1024)
    hipLaunchKernelGGL(vsoftmax_reg_kernel<1>, g, b, 0, s, S, n);
  else if (n <= 4096)
    hipLaunchKernelGGL(vsoftmax_reg_kernel<4>, g, b, 0, s, S, n);
  else
    hipLaunchKernelGGL(vsoftmax_reg_kernel<16>, g, b, 0, s, S, n);
  return hipGetLastError();
}

hipError_t launch_vtranspose(const float* in, int64_t ld, int c0, float* out, int n, int C, hipStream_t s) {
  dim3 grid((n + 31) / 32, (C + 31) / 32);
  hipLaunchKernelGGL(vtranspose_kernel, grid, dim3(32, 8), 0, s, in, ld, c0, out, n, C);
  return hipGetLastError();
}

}  // namespace zdit
