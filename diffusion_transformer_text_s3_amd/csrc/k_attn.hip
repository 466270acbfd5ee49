// Softmax attention, head_dim 128, ragged per branch: keys j >= seq_len[b] are masked
// (batch-alignment padding).  The DiT's joint attention is bidirectional: every key below
// seq_len[b] (image tokens, caption tokens and learned caption pads) is context.  The text
// encoder's is causal (key j visible to query i only when j <= i) with grouped key/value
// heads (query head h reads key/value head h / (n_heads / n_kv_heads)).
//
// bf16 path on gfx950.  A 512-thread workgroup owns 256 queries of one (branch, head); each
// wavefront owns 32 of them and keeps their 128-dim rows in registers as MFMA B operands.
// Key blocks of 64 are staged in LDS by direct-to-LDS buffer loads: K as [key][dim] and V as
// [dim][key] (V is transposed once per layer by vtrans_kernel).  Scores are formed
// transposed, S^T = K Q^T, so each lane holds 32 scores of a single query: the running max
// needs one cross-lane step (lane ^ 32) and the rescale of the output accumulator is a
// per-lane scalar.  The output is formed transposed too, O^T += V^T P^T, where the bf16 P^T
// operand is taken straight from the score registers: in a 32x32 MFMA result, lane half h
// holds keys {8g + 4h + 0..3}, so for each group of 16 keys both operands use the key order
// {4h..4h+3, 8+4h..8+4h+3}; V^T is stored with each 16-key group in that order, so a lane
// reads its 8 keys in one 16-byte load.
// Online softmax in fp32 with exp2 and the 1/sqrt(128) scale folded into log2(e).
#include <type_traits>

#include "common.h"

namespace zdit {

namespace {

constexpr int KT = 64;   // keys per LDS block
constexpr int KROW = 17; // 16-byte chunks per row of the V transpose staging tile (16 + 1 pad)

// One workgroup per (64 tokens, key/value head, branch).
__global__ __launch_bounds__(256) void vtrans_kernel(AttnArgs a) {
  __shared__ uint4 t[64 * KROW];
  const int b = blockIdx.z, h = blockIdx.y, s0 = blockIdx.x * 64;
  const int S = a.seq_len[b];
  const bf16* qkv = (const bf16*)a.qkv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int tok = c >> 4, dc = c & 15;
    const int s = s0 + tok;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (s < S)
      v = *(const uint4*)(qkv + ((int64_t)b * a.s_max + s) * a.row_stride + a.v_col + h * kHeadDim + dc * 8);
    t[tok * KROW + dc] = v;
  }
  __syncthreads();
  const bf16* tb = (const bf16*)t;
  bf16* vt = (bf16*)a.vt + ((int64_t)(b * a.n_kv_heads + h) * kHeadDim) * a.s_pad;
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

// V^T tokens s_max .. s_pad - 1 (past every branch's rows) read as zero keys: one thread per
// 16-byte chunk of those columns in every (branch, head, dim) row.
__global__ __launch_bounds__(256) void vt_tail_zero_kernel(AttnArgs a) {
  const int tail = (a.s_pad - a.s_max) >> 3;  // chunks per row
  const int64_t rows = (int64_t)a.batch * a.n_kv_heads * kHeadDim;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * tail) return;
  const int64_t row = i / tail;
  const int c = (int)(i % tail);
  *(uint4*)((bf16*)a.vt + row * a.s_pad + a.s_max + c * 8) = make_uint4(0, 0, 0, 0);
}

// 8 wavefronts x 32 queries = 256 queries per workgroup (two wavefronts per SIMD, so one's
// softmax can overlap the other's MFMAs).  K and V^T key blocks are double-buffered in LDS and
// fetched with direct-to-LDS buffer loads (no staging registers): V^T one block ahead, K two
// (QK^T runs a block ahead of PV).  Per key block t, within one wavefront: the QK^T MFMAs of
// block t+1 interleaved with the exponentials of block t, then the PV MFMAs of block t
// interleaved with its row sums and the maximum of block t+1.
constexpr int NWAVE = 8;
constexpr int QTILE = 32 * NWAVE;
constexpr int ATT_NT = 64 * NWAVE;  // threads per workgroup
// buffer resource word 3 for raw (untyped, offset-addressed) buffer loads
constexpr int kAttBufFlags = 0x00020000;
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kAttVmcnt0 = 0x0F70;

// Workgroups are dispatched round-robin over the 8 XCDs.  The 1-D grid is renumbered so that
// consecutive logical ids (the query tiles of one (branch, head), which share its K and V)
// run on the same XCD and hit its L2.
__device__ __forceinline__ int xcd_logical_id(int pid, int nwg) {
  const int xcd = pid & 7, idx = pid >> 3;
  const int full = nwg >> 3, rem = nwg & 7;
  return (xcd < rem) ? xcd * (full + 1) + idx : rem * (full + 1) + (xcd - rem) * full + idx;
}

// One lane's 16 bytes of a direct-to-LDS load: lane L writes LDS at lds_base + 16 L.  voff is
// bounds-checked against the resource (out of range loads zero); soff is not.
__device__ __forceinline__ void att_dma_16(const __amdgpu_buffer_rsrc_t rs, const uint4* lds_base, int voff,
                                           int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16, voff,
                                           soff, 0, 0);
}

// f(v[lane], v[lane ^ 32]) for a symmetric f, on the VALU: v_permlane32_swap of (v, v) gives
// {v[lane & 31], v[32 + (lane & 31)]}.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS layouts (16-byte chunks).  K block: row = key (16 chunks = 128 dims), chunk c of key k
// at slot c ^ (k & 15).  V^T block: row = dim (8 chunks = 64 keys), chunk c of dim d at slot
// c ^ (d & 7) ^ ((d >> 3) & 1).  Either way the 16 lanes that one 16-byte LDS read serves in
// a cycle (16 consecutive rows, one logical chunk) hit 16 distinct bank groups.
__device__ __forceinline__ int k_slot(int key, int c) { return key * 16 + (c ^ (key & 15)); }
__device__ __forceinline__ int v_slot(int d, int c) { return d * 8 + (c ^ (d & 7) ^ ((d >> 3) & 1)); }

__global__ __launch_bounds__(ATT_NT) __attribute__((amdgpu_waves_per_eu(2))) void attn_bf16_kernel(AttnArgs a) {
  // four separate objects, so reads of one buffer are not ordered behind the in-flight
  // direct-to-LDS writes of another
  __shared__ uint4 K0[KT * 16], K1[KT * 16];
  __shared__ uint4 V0[kHeadDim * 8], V1[kHeadDim * 8];
  const int nqt = (a.s_max + QTILE - 1) / QTILE;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int qt = lid % nqt, bh = lid / nqt;
  const int h = bh % a.n_heads, b = bh / a.n_heads, q0 = qt * QTILE;
  const int hk = h / (a.n_heads / a.n_kv_heads);  // key/value head of this query head
  const int D = a.n_heads * kHeadDim;              // output row width
  const int rs = a.row_stride;
  const int S = a.seq_len[b];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const bf16* qp = qkv + ((int64_t)b * a.s_max + min(q, S - 1)) * rs + h * kHeadDim + 8 * fh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
  }

  // K rows of this (branch, key head): key k at k * row_stride elements from kbase.  The
  // resource ends after key S - 1's 128 dims, so keys >= S load as zero.
  const int krow = rs * 2;  // bytes between consecutive keys
  const bf16* kbase = qkv + (int64_t)b * a.s_max * rs + a.k_col + hk * kHeadDim;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, (S - 1) * krow + kHeadDim * 2, kAttBufFlags);
  const bf16* vbase = (const bf16*)a.vt + ((int64_t)(b * a.n_kv_heads + hk) * kHeadDim) * a.s_pad;
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, kHeadDim * a.s_pad * 2, kAttBufFlags);
  // Each key block is 16 KB of K and 16 KB of V^T: 16 wave loads of 1 KB each, two per wave.
  // K load j covers keys 4j .. 4j+3 (lane L: key 4j + L / 16, slot L % 16); V^T load j covers
  // dims 8j .. 8j+7 (lane L: dim 8j + L / 8, slot L % 8).  Lanes fetch the chunk that belongs
  // in their slot.
  int kvo[2], vvo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = wave * 2 + i;
    const int key = 4 * j + (lane >> 4), ks = lane & 15;
    kvo[i] = key * krow + (ks ^ (key & 15)) * 16;
    const int d = 8 * j + (lane >> 3), vs = lane & 7;
    vvo[i] = d * a.s_pad * 2 + (vs ^ (d & 7) ^ ((d >> 3) & 1)) * 16;
  }
  auto dma_k = [&](int t, uint4* dst) {
#pragma unroll
    for (int i = 0; i < 2; ++i) att_dma_16(krs, dst + (wave * 2 + i) * 64, kvo[i] + t * KT * krow, 0);
  };
  auto dma_v = [&](int t, uint4* dst) {
#pragma unroll
    for (int i = 0; i < 2; ++i) att_dma_16(vrs, dst + (wave * 2 + i) * 64, vvo[i], t * KT * 2);
  };
  auto qk = [&](const uint4* Kb, f32x16 (&st)[2]) {
    const f32x16 zero = {};
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, Kb[k_slot(t2 * 32 + fr, 2 * s + fh)]);
        // the first k-step starts from a zero accumulator operand (no register clearing)
        st[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s == 0 ? zero : st[t2], 0, 0, 0);
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
  // causal: no key past the tile's last valid query is needed
  const int nkt = (a.causal ? min(q0 + QTILE, S) + KT - 1 : S + KT - 1) / KT;
  // largest key this lane's query sees (key 0 is always visible)
  const int klim = a.causal ? min(S - 1, q) : S - 1;

  // Scores of one block as a lane holds them: keys past the lane's limit set to -inf when
  // `masked`, then the maximum over the lane pair, in log2 units.
  auto block_max = [&](auto masked, int t, f32x16 (&st)[2]) {
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * KT + t2 * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
          if (key > klim) st[t2][r] = -INFINITY;
        }
    }
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], st[t2][r]);
    return xor32_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * sc;
  };

  // One key block t: K(t+1) is in Kn, V^T(t) in Vc, block t's scores in `cur`, and m_run
  // already covers them.  Loads of V^T block t+1 (into Vn) and K block t+2 (into Kc, last
  // read in the previous step) start first; past the last block they repeat it into buffers
  // no one reads again, so the step has no branch before its end.  Within one wave the MFMAs
  // run beside independent VALU and transcendental work, so the instruction stream
  // interleaves them: the 16 QK^T MFMAs of block t+1 with the exponentials of block t, then
  // the 16 PV MFMAs of block t with the row sums and the maximum of block t+1; fragment reads
  // run four ahead.  The (rare) rescale for block t+1 comes last.  NextMasked: block t+1 may
  // hold keys past a lane's limit.  Last: block t is the final one (no block t+1).
  auto step = [&](auto next_masked, auto last, int t, uint4* Kc, uint4* Vc, uint4* Kn, uint4* Vn,
                  f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    constexpr bool LAST = decltype(last)::value;
    dma_v(min(t + 1, nkt - 1), Vn);
    dma_k(min(t + 2, nkt - 1), Kc);
    if constexpr (!LAST) qk(Kn, nxt);
    bf16x8 pb[2][2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pb[t2][r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(cur[t2][r], sc, -m_run));
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // logical chunk (t2 * 4 + j * 2 + fh) of the V^T row holds this lane half's 8 keys
          const bf16x8 vf = __builtin_bit_cast(bf16x8, Vc[v_slot(dt * 32 + fr, t2 * 4 + j * 2 + fh)]);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t2][j], o[dt], 0, 0, 0);
        }
    // row sum of the bf16 probabilities that enter O (so O / l weighs the values exactly as
    // P V does), in four dot2 chains
    const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
    float l4[4] = {l_run, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pp = {pb[t2][j][2 * e], pb[t2][j][2 * e + 1]};
          l4[2 * t2 + j] = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, l4[2 * t2 + j], false);
        }
    l_run = (l4[0] + l4[1]) + (l4[2] + l4[3]);
    if constexpr (!LAST) {
      const float m_new = fmaxf(m_run, block_max(next_masked, t + 1, nxt));
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
      }
      // Lazy rescale: a query's reference max moves only when its max rose by more than 8
      // (log2 units), so p = exp2(s - m_run) stays below 2^8; O and l share the reference,
      // so the result O / l is the same softmax.  The branch is taken when any lane needs
      // it; the other lanes scale by exactly 1, so every query's arithmetic depends on its
      // own scores only.
      const bool move = m_new > m_run + 8.0f;
      if (__any(move)) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
        m_run = move ? m_new : m_run;
      }
    }
    __builtin_amdgcn_s_waitcnt(kAttVmcnt0);
    __syncthreads();
  };

  // steps from tm on may hold keys past a lane's limit: the last block (keys >= S), and with
  // causal masking every block from the one holding the tile's first query (tm is even)
  const int tm = (a.causal ? min(nkt - 1, q0 / KT) : nkt - 1) & ~1;
  dma_k(0, K0);
  dma_v(0, V0);
  dma_k(min(1, nkt - 1), K1);
  __builtin_amdgcn_s_waitcnt(kAttVmcnt0);
  __syncthreads();
  if (q0 + wave * 32 >= S) {
    // Every query of this wavefront is padding (the tile's last rows): it keeps loading its
    // share of each key block and meets every barrier of the working wavefronts (the prologue's
    // second one and one per step), and writes zeros.
    __syncthreads();
    for (int t = 0; t < nkt; ++t) {
      dma_v(min(t + 1, nkt - 1), (t & 1) ? V0 : V1);
      dma_k(min(t + 2, nkt - 1), (t & 1) ? K1 : K0);
      __builtin_amdgcn_s_waitcnt(kAttVmcnt0);
      __syncthreads();
    }
    if (q < a.s_max) {
      bf16* op = out + ((int64_t)b * a.s_max + q) * D + h * kHeadDim;
#pragma unroll
      for (int c = 0; c < 16; ++c) *(bf16x4*)(op + 8 * c + 4 * fh) = bf16x4{};
    }
    return;
  }
  f32x16 sA[2], sB[2];
  qk(K0, sA);
  m_run = tm == 0 ? block_max(std::true_type{}, 0, sA) : block_max(std::false_type{}, 0, sA);
  // step 0 loads key block 2 into K0: every wave's reads of K0 must be done
  __syncthreads();
  using P = std::false_type;
  using M = std::true_type;
  // step t masks block t + 1 from t = tp on (tp even, at most tm - 1)
  const int tp = max(tm - 1, 0) & ~1;
  int t = 0;
  for (; t < tp; t += 2) {
    step(P{}, P{}, t, K0, V0, K1, V1, sA, sB);
    step(P{}, P{}, t + 1, K1, V1, K0, V0, sB, sA);
  }
  for (; t + 2 <= nkt - 1; t += 2) {
    step(M{}, P{}, t, K0, V0, K1, V1, sA, sB);
    step(M{}, P{}, t + 1, K1, V1, K0, V0, sB, sA);
  }
  if (t == nkt - 1) {
    step(M{}, M{}, t, K0, V0, K1, V1, sA, sB);
  } else {
    step(M{}, P{}, t, K0, V0, K1, V1, sA, sB);
    step(M{}, M{}, t + 1, K1, V1, K0, V0, sB, sA);
  }

  const float l = xor32_sum(l_run);
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
  const int hk = h / (a.n_heads / a.n_kv_heads);
  const int S = a.seq_len[b];
  const float* qkv = (const float*)a.qkv;
  float* op = (float*)a.out + ((int64_t)b * a.s_max + q) * D + h * kHeadDim + 2 * lane;
  if (q >= S) { op[0] = 0.f; op[1] = 0.f; return; }
  const float* qp = qkv + ((int64_t)b * a.s_max + q) * a.row_stride + h * kHeadDim + 2 * lane;
  const float q0 = qp[0], q1 = qp[1];
  const float scale = 1.0f / sqrtf((float)kHeadDim);
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  const int nk = a.causal ? q + 1 : S;
  for (int j = 0; j < nk; ++j) {
    const float* row = qkv + ((int64_t)b * a.s_max + j) * a.row_stride;
    const float* kp = row + a.k_col + hk * kHeadDim + 2 * lane;
    float s = q0 * kp[0] + q1 * kp[1];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    s *= scale;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    const float* vp = row + a.v_col + hk * kHeadDim + 2 * lane;
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

hipError_t launch_vt_tail_zero(const AttnArgs& args, hipStream_t s) {
  AttnArgs a = args;
  attn_layout_defaults(a);
  const int64_t n = (int64_t)a.batch * a.n_kv_heads * kHeadDim * ((a.s_pad - a.s_max) >> 3);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(vt_tail_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn(int precision, const AttnArgs& args, hipStream_t s) {
  AttnArgs a = args;
  attn_layout_defaults(a);
  if (precision == 0) {
    if (!a.vt_ready)
      hipLaunchKernelGGL(vtrans_kernel, dim3(a.s_pad / 64, a.n_kv_heads, a.batch), dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_bf16_kernel, dim3(((a.s_max + QTILE - 1) / QTILE) * a.n_heads * a.batch),
                       dim3(ATT_NT), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.s_max, a.n_heads, a.batch), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace zdit
