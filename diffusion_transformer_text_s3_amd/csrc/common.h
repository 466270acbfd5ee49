// Internal types and kernel launchers of the gfx950 S3-DiT library.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace zdit {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxBatch = 16;
constexpr int kHeadDim = 128;

// Maps a compact row index m (0..rows-1, `rows_per_batch` rows per branch) to a row of a
// branch-strided buffer: address = base + b * batch_stride + r * ld, written only when
// r < valid[b].
struct RowMap {
  int rows_per_batch;
  int64_t batch_stride;
  int64_t ld;
  int valid[kMaxBatch];
};

// EPI_QKV: the fused q/k/v projection of a block (bf16 only): q and k columns are rotated by
// RoPE on rows below seq[b] and stored, v columns are not stored in C but written transposed
// into vt (see k_attn.hip for its layout), zero on rows at or past seq[b].
// EPI_PART / EPI_PART_SWIGLU: the K range [k0, k0 + k_split) of split blockIdx.y, its fp32
// partial product stored to part + split * M * part_ld (row m at m * part_ld; SwiGLU: the W1 sums
// at columns n, the W3 sums at N + n), for a fixed-order sum by the split-K reduction.
enum Epi { EPI_STORE = 0, EPI_BIAS = 1, EPI_RESID = 2, EPI_SWIGLU = 3, EPI_QKV = 4, EPI_PART = 5,
           EPI_PART_SWIGLU = 6 };

struct GemmArgs {
  const void* A;
  const void* B;
  const void* B2;        // second weight (SwiGLU up projection)
  void* C;
  const float* vec;      // bias [N] (EPI_BIAS) or gate (EPI_RESID; NULL = 1)
  int64_t vec_bstride;   // gate branch stride in floats
  int M, N, K;
  int64_t lda, ldb;
  RowMap out;
  // EPI_QKV only: RoPE tables [batch][rows_per_batch][64] (rope_bstride floats between
  // branches), valid rows per branch, V^T destination [batch][n_heads][128][vt_pad]
  const float* rope_cos;
  const float* rope_sin;
  int64_t rope_bstride;
  void* vt;
  int vt_pad, n_heads;
  int seq[kMaxBatch];
  // EPI_PART / EPI_PART_SWIGLU only
  float* part;
  int k_split, part_ld;
};

// ---- launchers (return hipError_t of the launch) ----
hipError_t launch_gemm_bf16(int epi, const GemmArgs& g, hipStream_t s);
// The main GEMM split over K for few rows: `splits` ranges of g.k_split columns (a multiple of
// 32, from N and K only) computed by gemm_bf16_kernel into fp32 partials `part`
// [splits][M][Nv] (Nv = N, or 2N for SwiGLU), then summed in range order by the split-K
// reduction with the epilogue (EPI_STORE, EPI_RESID, EPI_SWIGLU) through g.out.
struct SplitPlan {
  int splits, k_split, Nv;
};
SplitPlan tile_split_plan(int epi, int N, int K);
size_t tile_split_workspace(int epi, int M, int N, int K);
hipError_t launch_gemm_bf16_split(int epi, const GemmArgs& g, float* part, hipStream_t s);
hipError_t launch_gemm_f32(int epi, const GemmArgs& g, hipStream_t s);

// Split-K GEMM for few rows (M <= 256; N % 8 == 0, K % 64 == 0): fp32 partials of
// [splits][M][Nv] in `part`, then a fixed-order sum and the epilogue (EPI_STORE, EPI_RESID,
// EPI_SWIGLU; output through g.out as in the main GEMM).  The split of K depends on N and K
// only.
struct SplitKArgs {
  const void* A;
  const void* B;
  const void* B2;
  float* part;
  int M, N, K, lda, ldb;
  int ks;         // K columns per split (multiple of 32)
  int splits;
  int col_tiles;  // 64-column tiles per weight
  int Nv;         // partial row width: N, or 2N for SwiGLU (W3 columns after W1's)
  // Row gather / scatter (NULL: row m is row m).  A row m is row a_rows[m] of A, which has
  // a_phys_rows rows; output row m goes to row c_rows[m] of C (RowMap ld, no batch stride).
  const int* a_rows;
  int a_phys_rows;
  const int* c_rows;
  // SwiGLU over one K range with unmapped output rows: a workgroup's waves 0-3 take 64 W1
  // columns and waves 4-7 the same 64 W3 columns, and the GEMM writes u (bf16, row m at
  // u_out + m * u_ld) itself; no partials, no reduction launch
  int swiglu_direct;
  void* u_out;
  int64_t u_ld;
  // B and B2 in the packed band layout of launch_pack_bfrag (ldb == K, N % 16 == 0): slab t of
  // the 16-row band of a wavefront is 1 KB in a row, chunk lane at t * 1024 + 16 lane
  int packed;
};
SplitKArgs splitk_plan(int epi, int M, int N, int K);
size_t splitk_workspace(int epi, int M, int N, int K);
// Work folded into the split-K reduction.  QK_NORM_ROPE (with EPI_STORE and a row scatter map
// into rows b * L + r of C): the q and k heads of each row are RMS-normalised over their 128 dims
// (gains gq / gk, in fp32 from the summed projection) and rotated by RoPE over dimension pairs
// (i, i + 64) at position r (cos / sin [b][r][64]); v heads are rounded as they are.
// RESID_NORM (with EPI_RESID and a row scatter map): after the residual add, each row of the
// residual stream is RMS-normalised with `gain` and written as bf16 to row c_rows[m] of h.
struct SplitKFuse {
  enum Kind { NONE = 0, QK_NORM_ROPE = 1, RESID_NORM = 2 } kind = NONE;
  const float* gq = nullptr;
  const float* gk = nullptr;
  const float* cos = nullptr;
  const float* sin = nullptr;
  int64_t tab_bstride = 0;
  int n_heads = 0, n_kv_heads = 0, L = 0;
  const float* gain = nullptr;
  void* h = nullptr;
  float eps = 0.f;
  // QK_NORM_ROPE: when set, v heads go transposed into vt [b][n_kv_heads][128][s_pad] in the
  // attention kernel's key order (and not into C)
  void* vt = nullptr;
  int s_pad = 0;
};
hipError_t launch_gemm_splitk(int epi, const GemmArgs& g, float* part, hipStream_t s, const int* a_rows = nullptr,
                              int a_phys_rows = 0, const int* c_rows = nullptr, const SplitKFuse* fuse = nullptr,
                              bool b_packed = false);
// bf16 [N][K] row-major -> bands of 16 rows, each a run of 32-column slabs of 64 16-byte chunks,
// chunk l of slab t of band b = columns 32 t + 8 (l / 16) .. + 7 of row 16 b + l % 16 (the B
// fragment of v_mfma_f32_16x16x32_bf16); N % 16 == 0, K % 32 == 0
hipError_t launch_pack_bfrag(const void* src, void* dst, int N, int K, hipStream_t s);
// The split-K reduction alone: sums a.splits partial planes [splits][M][Nv] of a.part in order
// and applies the epilogue (EPI_STORE, EPI_RESID, EPI_SWIGLU) through g.out (a.c_rows NULL).
hipError_t launch_splitk_reduce(int epi, const SplitKArgs& a, const GemmArgs& g, hipStream_t s);

// q, k, v rows: row r of branch b at qkv + (b * s_max + r) * row_stride elements, query head
// h at column h * 128, key head j at k_col + j * 128, value head j at v_col + j * 128.  Query
// head h reads key/value head h / (n_heads / n_kv_heads).  Zero row_stride / k_col / v_col /
// n_kv_heads mean the DiT layout: n_kv_heads = n_heads, row_stride 3D, k_col D, v_col 2D
// (D = n_heads * 128).  causal: key j is visible to query i only when j <= i.
struct AttnArgs {
  const void* qkv;
  void* vt;          // bf16 path: [B, n_kv_heads, 128, s_pad] transposed values (workspace)
  void* out;         // [B, s_max, n_heads * 128]
  int batch, s_max, s_pad, n_heads;
  int n_kv_heads, row_stride, k_col, v_col;
  int causal;
  int vt_ready;      // vt already holds V^T (written by the QKV GEMM epilogue)
  int seq_len[kMaxBatch];
};
// DiT defaults filled in for zero fields (see AttnArgs)
inline void attn_layout_defaults(AttnArgs& a) {
  const int D = a.n_heads * kHeadDim;
  if (a.n_kv_heads == 0) a.n_kv_heads = a.n_heads;
  if (a.row_stride == 0) a.row_stride = 3 * D;
  if (a.k_col == 0) a.k_col = D;
  if (a.v_col == 0) a.v_col = 2 * D;
}
size_t attn_vt_bytes(int precision, int batch, int s_max, int n_heads);
hipError_t launch_attn(int precision, const AttnArgs& a, hipStream_t s);
// Zero V^T tokens s_max .. s_pad - 1 of every (branch, head, dim) row (after the QKV epilogue
// wrote tokens below s_max).
hipError_t launch_vt_tail_zero(const AttnArgs& a, hipStream_t s);

// Row r of branch b is x + b * x_bstride + r * dim; out is compact [batch * rows, dim].
// shift / scale: fp32 [dim] vectors of branch 0, branch b at + b * mod_bstride; both NULL
// for no modulation.  Rows with r >= valid[b] are written as 0.
struct NormArgs {
  const float* x;
  int64_t x_bstride;
  int rows_per_batch;
  int batch;
  int dim;
  const float* gain;
  const float* shift;
  const float* scale;
  int64_t mod_bstride;
  float eps;
  void* out;
  int valid[kMaxBatch];
};
hipError_t launch_rmsnorm_mod(int precision, const NormArgs& a, hipStream_t s);

// Per-head RMSNorm (gain gq for query heads, gk for key heads, over the 128 dims of a head)
// followed by RoPE that turns dims (i, i + 64) by the row's angle i, in place on the bf16
// q and k heads of rows r < seq_len[b] (rows laid out as in AttnArgs).  cos / sin: fp32
// [batch][s_max][64] with tab_bstride floats between branches (0 = shared).
struct QkNormRopeArgs {
  void* qkv;
  int64_t row_stride;
  int k_col;
  int n_heads, n_kv_heads;
  const float* gq;
  const float* gk;
  const float* cos;
  const float* sin;
  int64_t tab_bstride;
  float eps;
  int batch, s_max;
  int seq_len[kMaxBatch];
};
hipError_t launch_qknorm_rope(const QkNormRopeArgs& a, hipStream_t s);

// out[b][r][:] = table[ids[b * s_max + r]][:] (bf16 table, fp32 out) for r < len[b], 0 for
// r >= len[b] (ids there are not read).  dim a multiple of 8.
// Ids of at most kInlineIds tokens (batch * s_max) travel in the kernel arguments (n_inline > 0),
// so the call makes no host-to-device copy; otherwise they are read from `ids` (device).
constexpr int kInlineIds = 512;
struct EmbedArgs {
  const int* ids;
  const void* table;
  float* out;
  int batch, s_max, dim;
  int len[kMaxBatch];
  int n_inline;
  int inline_ids[kInlineIds];
};
hipError_t launch_embed(const EmbedArgs& a, hipStream_t s);

// The valid rows of a padded batch in order: entry i (i < sum of len) is b * s_max + r for
// the i-th pair (b, r < len[b]).
hipError_t launch_valid_rows(int batch, int s_max, const int* len, int* rows, hipStream_t s);

// Opt-in non-finite detection: flag = 1 when any value of the valid rows (r < valid[b]) of a
// branch-strided fp32 buffer is NaN or +-Inf.  Row r of branch b: p + b * bstride + r * ld,
// `width` values (a multiple of 4, 16-byte aligned rows).
struct FiniteArgs {
  const float* p;
  int64_t bstride, ld;
  int rows_per_batch, batch, width;
  int valid[kMaxBatch];
  int* flag;
};
hipError_t launch_finite_check(const FiniteArgs& a, hipStream_t s);
// When first[0] < 0 and one of flags[0..n) is set: first = {step, index of the first set flag}.
// Then every flag is cleared.  One thread, in stream order.
hipError_t launch_finite_latch(int* flags, int n, int step, int* first, hipStream_t s);
// p[0..n) = v
hipError_t launch_fill_i32(int* p, int n, int v, hipStream_t s);

// zero `bytes` (a multiple of 16) at 16-byte aligned p
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s);

// measurement: `workgroups` x 256 threads, each wave 4 x iters bf16 32x32x16 MFMAs; out
// [workgroups * 256] fp32
hipError_t launch_mfma_peak(int workgroups, int iters, float* out, hipStream_t s);

struct RopeArgs {
  void* qkv;
  const float* cos;
  const float* sin;
  int64_t tab_bstride;   // floats between branches of the tables (0 = shared)
  int batch, s_max, n_heads;
  int seq_len[kMaxBatch];
};
hipError_t launch_rope(int precision, const RopeArgs& a, hipStream_t s);

struct RopeTabArgs {
  float* cos;
  float* sin;
  int kind, batch, s_max, grid_h, grid_w;
  int axes[3];
  float theta;
  int n_cap[kMaxBatch];
};
hipError_t launch_rope_tables(const RopeTabArgs& a, hipStream_t s);

hipError_t launch_patchify(int precision, int batch, int C, int h, int w, const float* lat,
                           int64_t lat_bstride, void* tokens, hipStream_t s);
hipError_t launch_unpatchify(int batch, int C, int h, int w, const float* tokens, float* lat,
                             hipStream_t s);
hipError_t launch_cap_pad(int batch, int s_max, int dim, int row0, const int* cap_len,
                          int multiple, const float* pad, float* x, hipStream_t s);
hipError_t launch_convert(int precision, const float* in, void* out, int64_t n, hipStream_t s);
hipError_t launch_euler(float* x, const float* vc, const float* vu, int64_t n, float g,
                        float sigma, float sigma_next, float* dec, hipStream_t s);
hipError_t launch_temb(int batch, const float* t, int t_freq, int c_dim, float t_scale,
                       const float* w1, const float* b1, const float* w2, const float* b2,
                       float* c, hipStream_t s);
hipError_t launch_adaln(int precision, int batch, int c_dim, int n_out, const float* c,
                        const void* w, const float* b, float* out, hipStream_t s);
// up to kMaxAdaJobs projections of the same c (weights w[i], bias b[i] -> out[i]) in one launch
constexpr int kMaxAdaJobs = 40;
hipError_t launch_adaln_multi(int precision, int batch, int c_dim, int n_out, const float* c, const void* const* w,
                              const float* const* b, float* const* out, int n_jobs, hipStream_t s);
hipError_t launch_copy_rows(const float* src, int64_t src_bstride, float* dst,
                            int64_t dst_bstride, int batch, int64_t n, hipStream_t s);

}  // namespace zdit
