// C ABI of the text encoder (a Qwen3-shaped causal decoder read out at hidden_states[-2]):
// argument validation, workspace planning and the launch sequence of its blocks.  Every
// argument is checked before the first launch; on error nothing is enqueued.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "api_util.h"

using namespace zdit;

namespace {

// Shapes the kernels implement; the checks name the limit that fails.
zdit_status check_enc_cfg(const zdit_enc_cfg* c) {
  if (!c) return fail(ZDIT_EINVAL, "cfg is NULL");
  if (c->head_dim != kHeadDim) return fail(ZDIT_EUNSUPPORTED, "head_dim %d (only 128)", c->head_dim);
  if (c->n_layers < 2) return fail(ZDIT_EINVAL, "n_layers %d (at least 2: the output is after n_layers - 1)", c->n_layers);
  if (c->hidden < 128 || c->hidden % 128 || c->hidden > 4096)
    return fail(ZDIT_EUNSUPPORTED, "hidden %d (multiple of 128, <= 4096)", c->hidden);
  if (c->inter < 128 || c->inter % 128) return fail(ZDIT_EUNSUPPORTED, "inter %d (positive multiple of 128)", c->inter);
  if (c->n_heads < 1 || c->n_heads > 64) return fail(ZDIT_EUNSUPPORTED, "n_heads %d (1..64)", c->n_heads);
  if (c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads)
    return fail(ZDIT_EINVAL, "n_kv_heads %d must divide n_heads %d", c->n_kv_heads, c->n_heads);
  if (c->vocab < 1) return fail(ZDIT_EINVAL, "vocab %d", c->vocab);
  if (!(c->rope_theta > 0.f) || !isfinite(c->rope_theta)) return fail(ZDIT_EINVAL, "rope_theta must be finite and > 0");
  if (!(c->norm_eps >= 0.f) || !isfinite(c->norm_eps)) return fail(ZDIT_EINVAL, "norm_eps must be finite and >= 0");
  if (c->flags & ~ZDIT_ENC_PACKED_WEIGHTS) return fail(ZDIT_EINVAL, "unknown flags 0x%x", c->flags);
  return ZDIT_OK;
}

int qkv_width(const zdit_enc_cfg& c) { return (c.n_heads + 2 * c.n_kv_heads) * kHeadDim; }

// the K resource of the attention kernel spans s_max rows of the qkv buffer in bytes
bool qkv_fits(int64_t s_max, int64_t width) { return s_max * width * 2 <= INT32_MAX; }

// Rows up to which the projections run as split-K GEMMs (the weights then stream from HBM
// through ~512 workgroups instead of a few dozen 256 x 256 tiles).
constexpr int kSplitKMaxRows = 256;

struct EncPlan {
  size_t ids, rows, cos, sin, h, qkv, vt, o, u, part, total;
  bool splitk;
  bool packed;  // projection weights in the packed band layout (split-K path only)
};

size_t enc_part_bytes(const zdit_enc_cfg& c, int M) {
  const int D = c.hidden, Dq = c.n_heads * kHeadDim;
  size_t b = splitk_workspace(EPI_STORE, M, qkv_width(c), D);
  b = std::max(b, splitk_workspace(EPI_RESID, M, D, Dq));
  b = std::max(b, splitk_workspace(EPI_SWIGLU, M, c.inter, D));
  b = std::max(b, splitk_workspace(EPI_RESID, M, D, c.inter));
  return b;
}

EncPlan plan_enc(const zdit_enc_cfg& c, int B, int L) {
  const size_t M = (size_t)B * L;
  EncPlan p;
  p.splitk = M <= (size_t)kSplitKMaxRows;
  p.packed = (c.flags & ZDIT_ENC_PACKED_WEIGHTS) != 0;
  size_t off = 0;
  p.ids = off; off += al256(M * 4);
  p.rows = off; off += al256(M * 4);
  p.cos = off; off += al256(M * 64 * 4);
  p.sin = off; off += al256(M * 64 * 4);
  p.h = off;   off += al256(M * c.hidden * 2);
  const size_t r0 = off;
  p.qkv = off; off += al256(M * qkv_width(c) * 2);
  p.vt = off;  off += al256(attn_vt_bytes(0, B, L, c.n_kv_heads));
  p.o = off;   off += al256(M * c.n_heads * kHeadDim * 2);
  if (p.splitk) {
    // V^T is written by the q/k/v reduction and its padding is zeroed once per forward, so
    // nothing else may write there
    p.u = off;
    off += al256(M * (size_t)c.inter * 2);
  } else {
    p.u = r0;  // the SwiGLU activation reuses the attention region (dead by then)
    off = std::max(off, r0 + al256(M * (size_t)c.inter * 2));
  }
  p.part = off;
  if (p.splitk) off += al256(enc_part_bytes(c, (int)M));
  p.total = off;
  return p;
}

// A projection of the block.  Few rows: split-K over the valid rows only (A_GATHER: A is the
// padded [B * L] layout, read through the valid-row list; C_SCATTER: C too), with M the
// number of valid rows.  Else the main GEMM over the padded rows (the RowMap skips padding).
hipError_t enc_gemm(int epi, GemmArgs g, bool a_gather, bool c_scatter, int B, int L, int Mc, const EncPlan& pl,
                    char* ws, hipStream_t st, const SplitKFuse* fuse = nullptr) {
  if (!pl.splitk) return launch_gemm_bf16(epi, g, st);
  const int* rows = (const int*)(ws + pl.rows);
  g.M = Mc;
  if (!c_scatter) g.out = compact_rows(Mc, g.out.ld);
  return launch_gemm_splitk(epi, g, (float*)(ws + pl.part), st, a_gather ? rows : nullptr, B * L,
                            c_scatter ? rows : nullptr, fuse, pl.packed);
}

zdit_status check_ids(int batch, int max_len, int vocab, const int32_t* ids, const int32_t* len) {
  if (!ids || !len) return fail(ZDIT_EINVAL, "ids or len NULL");
  for (int b = 0; b < batch; ++b) {
    if (len[b] < 1 || len[b] > max_len) return fail(ZDIT_EINVAL, "len[%d] = %d (1..max_len %d)", b, len[b], max_len);
    for (int r = 0; r < len[b]; ++r) {
      const int id = ids[(int64_t)b * max_len + r];
      if (id < 0 || id >= vocab) return fail(ZDIT_EINVAL, "ids[%d][%d] = %d outside [0, %d)", b, r, id, vocab);
    }
  }
  return ZDIT_OK;
}

zdit_status check_layer_w(const zdit_enc_layer_w& w, int i) {
  const void* ptrs[] = {w.in_norm, w.w_qkv, w.q_norm, w.k_norm, w.w_o, w.post_norm, w.w_gate, w.w_up, w.w_down};
  const char* names[] = {"in_norm", "w_qkv", "q_norm", "k_norm", "w_o", "post_norm", "w_gate", "w_up", "w_down"};
  for (int j = 0; j < 9; ++j) {
    if (!ptrs[j]) return fail(ZDIT_EINVAL, "layer %d weight %s is NULL", i, names[j]);
    if (!aligned16(ptrs[j])) return fail(ZDIT_EINVAL, "layer %d weight %s not 16-byte aligned", i, names[j]);
  }
  return ZDIT_OK;
}

AttnArgs enc_attn_args(const zdit_enc_cfg& c, int B, int L, const int32_t* len, const void* qkv, void* vt, void* o) {
  AttnArgs aa{};
  aa.qkv = qkv; aa.vt = vt; aa.out = o; aa.batch = B; aa.s_max = L; aa.s_pad = round_up(L, 64);
  aa.n_heads = c.n_heads; aa.n_kv_heads = c.n_kv_heads; aa.row_stride = qkv_width(c);
  aa.k_col = c.n_heads * kHeadDim; aa.v_col = (c.n_heads + c.n_kv_heads) * kHeadDim;
  aa.causal = 1;
  for (int b = 0; b < kMaxBatch; ++b) aa.seq_len[b] = b < B ? len[b] : 0;
  return aa;
}

// One block on B branches of L rows (x fp32 [B * L, hidden], rows >= len[b] stay 0).  On the
// split-K path the q/k norm + RoPE ride on the q/k/v reduction and each residual reduction also
// writes the RMSNorm that follows it: the post-attention norm, and the next block's input norm
// (next_in_norm; NULL after the last block).  There the input norm of this block is already in h
// except for the first block (in_normed false).
zdit_status enc_block(const zdit_enc_cfg& c, const zdit_enc_layer_w& w, int B, int L, const int32_t* len,
                      float* x, const EncPlan& pl, char* ws, hipStream_t st, bool in_normed,
                      const float* next_in_norm) {
  const int D = c.hidden, I = c.inter, M = B * L, W = qkv_width(c), Dq = c.n_heads * kHeadDim;
  int Mc = 0;  // valid rows
  for (int b = 0; b < B; ++b) Mc += len[b];
  void* h = ws + pl.h;
  void* qkv = ws + pl.qkv;
  void* vt = ws + pl.vt;
  void* o = ws + pl.o;
  void* u = ws + pl.u;

  NormArgs na;
  na.x = x; na.x_bstride = (int64_t)L * D; na.rows_per_batch = L; na.batch = B; na.dim = D;
  na.gain = w.in_norm; na.shift = nullptr; na.scale = nullptr; na.mod_bstride = 0;
  na.eps = c.norm_eps; na.out = h;
  for (int b = 0; b < kMaxBatch; ++b) na.valid[b] = b < B ? len[b] : 0;
  if (!pl.splitk || !in_normed) HIP_TRY(launch_rmsnorm_mod(ZDIT_BF16, na, st));

  GemmArgs g{};
  g.A = h; g.B = w.w_qkv; g.C = qkv; g.M = M; g.N = W; g.K = D; g.lda = D; g.ldb = D;
  g.out = compact_rows(M, W);
  if (pl.splitk) {
    SplitKFuse f;
    f.kind = SplitKFuse::QK_NORM_ROPE;
    f.gq = w.q_norm; f.gk = w.k_norm; f.cos = (const float*)(ws + pl.cos); f.sin = (const float*)(ws + pl.sin);
    f.tab_bstride = (int64_t)L * 64; f.n_heads = c.n_heads; f.n_kv_heads = c.n_kv_heads; f.L = L; f.eps = c.norm_eps;
    f.vt = vt; f.s_pad = round_up(L, 64);
    HIP_TRY(enc_gemm(EPI_STORE, g, true, true, B, L, Mc, pl, ws, st, &f));
  } else {
    HIP_TRY(enc_gemm(EPI_STORE, g, true, true, B, L, Mc, pl, ws, st));
    QkNormRopeArgs qa;
    qa.qkv = qkv; qa.row_stride = W; qa.k_col = Dq; qa.n_heads = c.n_heads; qa.n_kv_heads = c.n_kv_heads;
    qa.gq = w.q_norm; qa.gk = w.k_norm; qa.cos = (const float*)(ws + pl.cos); qa.sin = (const float*)(ws + pl.sin);
    qa.tab_bstride = (int64_t)L * 64; qa.eps = c.norm_eps; qa.batch = B; qa.s_max = L;
    for (int b = 0; b < kMaxBatch; ++b) qa.seq_len[b] = b < B ? len[b] : 0;
    HIP_TRY(launch_qknorm_rope(qa, st));
  }

  AttnArgs aa = enc_attn_args(c, B, L, len, qkv, vt, o);
  aa.vt_ready = pl.splitk ? 1 : 0;  // the q/k/v reduction wrote V^T
  HIP_TRY(launch_attn(ZDIT_BF16, aa, st));

  RowMap xr;
  xr.rows_per_batch = L; xr.batch_stride = (int64_t)L * D; xr.ld = D;
  for (int b = 0; b < kMaxBatch; ++b) xr.valid[b] = b < B ? len[b] : 0;
  SplitKFuse rn;  // residual reduction + the RMSNorm after it (split-K path)
  rn.kind = SplitKFuse::RESID_NORM;
  rn.h = h; rn.eps = c.norm_eps;
  g = GemmArgs{};
  g.A = o; g.B = w.w_o; g.C = x; g.M = M; g.N = D; g.K = Dq; g.lda = Dq; g.ldb = Dq; g.out = xr;
  if (pl.splitk) {
    rn.gain = w.post_norm;
    HIP_TRY(enc_gemm(EPI_RESID, g, true, true, B, L, Mc, pl, ws, st, &rn));
  } else {
    HIP_TRY(enc_gemm(EPI_RESID, g, true, true, B, L, Mc, pl, ws, st));
    na.gain = w.post_norm;
    HIP_TRY(launch_rmsnorm_mod(ZDIT_BF16, na, st));
  }

  g = GemmArgs{};
  g.A = h; g.B = w.w_gate; g.B2 = w.w_up; g.C = u; g.M = M; g.N = I; g.K = D; g.lda = D; g.ldb = D;
  g.out = compact_rows(M, I);
  // split-K: u holds the valid rows only, in order
  HIP_TRY(enc_gemm(EPI_SWIGLU, g, true, false, B, L, Mc, pl, ws, st));

  g = GemmArgs{};
  g.A = u; g.B = w.w_down; g.C = x; g.M = M; g.N = D; g.K = I; g.lda = I; g.ldb = I; g.out = xr;
  if (pl.splitk && next_in_norm) {
    rn.gain = next_in_norm;
    HIP_TRY(enc_gemm(EPI_RESID, g, false, true, B, L, Mc, pl, ws, st, &rn));
  } else {
    HIP_TRY(enc_gemm(EPI_RESID, g, false, true, B, L, Mc, pl, ws, st));
  }
  return ZDIT_OK;
}

// The embedding gather of the host ids into out: up to kInlineIds tokens the ids ride in the
// kernel arguments (no copy, so the call can be captured into a graph), more are copied into
// the workspace first.
zdit_status embed_rows(int B, int L, int dim, const int32_t* ids, const int32_t* len, const void* table,
                       float* out, int* ids_dev, hipStream_t st) {
  EmbedArgs ea;
  const int64_t n = (int64_t)B * L;
  ea.n_inline = n <= kInlineIds ? (int)n : 0;
  if (ea.n_inline) {
    for (int64_t i = 0; i < n; ++i) {
      const int r = (int)(i % L);
      ea.inline_ids[i] = r < len[i / L] ? ids[i] : 0;  // only valid rows' ids are read
    }
    ea.ids = nullptr;
  } else {
    HIP_TRY(hipMemcpyAsync(ids_dev, ids, (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice, st));
    ea.ids = ids_dev;
  }
  ea.table = table; ea.out = out; ea.batch = B; ea.s_max = L; ea.dim = dim;
  for (int b = 0; b < kMaxBatch; ++b) ea.len[b] = b < B ? len[b] : 0;
  HIP_TRY(launch_embed(ea, st));
  return ZDIT_OK;
}

}  // namespace

extern "C" {

size_t zdit_encoder_workspace(const zdit_enc_cfg* cfg, int32_t batch, int32_t max_len) {
  if (!cfg || check_enc_cfg(cfg) != ZDIT_OK || batch < 1 || batch > ZDIT_MAX_BATCH || max_len < 1) return 0;
  return plan_enc(*cfg, batch, max_len).total + 256;
}

zdit_status zdit_encoder_fwd(const zdit_enc_cfg* cfg, const zdit_enc_w* w, int32_t batch, int32_t max_len,
                             const int32_t* ids, const int32_t* len, float* hidden_out, void* ws, size_t ws_bytes,
                             void* hip_stream) {
  if (zdit_status s = check_enc_cfg(cfg)) return s;
  const zdit_enc_cfg& c = *cfg;
  if (batch < 1 || batch > ZDIT_MAX_BATCH || max_len < 1) return fail(ZDIT_EINVAL, "batch %d / max_len %d", batch, max_len);
  if ((int64_t)batch * max_len > (1 << 24) || !qkv_fits(max_len, qkv_width(c)))
    return fail(ZDIT_EUNSUPPORTED, "batch %d x max_len %d too large", batch, max_len);
  if (!w || !w->embed || !w->layers) return fail(ZDIT_EINVAL, "weights NULL");
  if (!aligned16(w->embed)) return fail(ZDIT_EINVAL, "embed not 16-byte aligned");
  for (int i = 0; i < c.n_layers - 1; ++i)
    if (zdit_status s = check_layer_w(w->layers[i], i)) return s;
  if (zdit_status s = check_ids(batch, max_len, c.vocab, ids, len)) return s;
  if (!hidden_out || !aligned16(hidden_out)) return fail(ZDIT_EINVAL, "hidden_out NULL or not 16-byte aligned");
  const EncPlan pl = plan_enc(c, batch, max_len);
  if (pl.packed && !pl.splitk)
    return fail(ZDIT_EUNSUPPORTED, "packed weights need batch * max_len <= %d (got %d x %d)", kSplitKMaxRows, batch,
                max_len);
  if (!ws || ws_bytes < pl.total + 256) return fail(ZDIT_EWORKSPACE, "workspace %zu < %zu", ws_bytes, pl.total + 256);
  char* base = (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  const hipStream_t st = (hipStream_t)hip_stream;

  RopeTabArgs rt;
  rt.cos = (float*)(base + pl.cos); rt.sin = (float*)(base + pl.sin); rt.kind = ZDIT_SEQ_TEXT;
  rt.batch = batch; rt.s_max = max_len; rt.grid_h = 0; rt.grid_w = 0;
  rt.axes[0] = kHeadDim; rt.axes[1] = 0; rt.axes[2] = 0; rt.theta = c.rope_theta;
  for (int b = 0; b < kMaxBatch; ++b) rt.n_cap[b] = b < batch ? len[b] : 0;
  HIP_TRY(launch_rope_tables(rt, st));

  if (zdit_status s = embed_rows(batch, max_len, c.hidden, ids, len, w->embed, hidden_out, (int*)(base + pl.ids), st))
    return s;
  if (pl.splitk) {
    HIP_TRY(launch_valid_rows(batch, max_len, len, (int*)(base + pl.rows), st));
    // V^T positions of padding keys (never written by the q/k/v reduction) read as zero
    HIP_TRY(launch_zero_fill(base + pl.vt, al256(attn_vt_bytes(0, batch, max_len, c.n_kv_heads)), st));
  }
  const int nb = c.n_layers - 1;
  for (int i = 0; i < nb; ++i) {
    const float* next = i + 1 < nb ? w->layers[i + 1].in_norm : nullptr;
    if (zdit_status s = enc_block(c, w->layers[i], batch, max_len, len, hidden_out, pl, base, st, i > 0, next))
      return s;
  }
  return ok();
}

size_t zdit_op_gemm_splitk_workspace(int32_t epilogue, int32_t M, int32_t N, int32_t K) {
  if (M < 1 || M > kSplitKMaxRows || N < 8 || N % 8 || K < 64 || K % 64 || (int64_t)N * K * 2 > INT32_MAX) return 0;
  if (epilogue != ZDIT_EPI_STORE && epilogue != ZDIT_EPI_RESID && epilogue != ZDIT_EPI_SWIGLU) return 0;
  return splitk_workspace(epilogue, M, N, K) + 256;
}

}  // extern "C"

namespace {
zdit_status gemm_splitk_op(bool packed, int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A,
                           const void* B, const void* B2, const float* vec, void* C, void* ws, size_t ws_bytes,
                           void* hip_stream) {
  if (epilogue != ZDIT_EPI_STORE && epilogue != ZDIT_EPI_RESID && epilogue != ZDIT_EPI_SWIGLU)
    return fail(ZDIT_EINVAL, "epilogue %d", epilogue);
  if (M < 1 || N < 1 || K < 1) return fail(ZDIT_EINVAL, "M %d N %d K %d", M, N, K);
  if (M > kSplitKMaxRows || N % 8 || K % 64 || (int64_t)N * K * 2 > INT32_MAX)
    return fail(ZDIT_EUNSUPPORTED, "M %d (<= %d), N %d (multiple of 8), K %d (multiple of 64)", M, kSplitKMaxRows,
                N, K);
  if (packed && N % 16) return fail(ZDIT_EUNSUPPORTED, "packed weights: N %d must be a multiple of 16", N);
  if (!A || !B || !C || (epilogue == ZDIT_EPI_SWIGLU && !B2)) return fail(ZDIT_EINVAL, "NULL operand");
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || (B2 && !aligned16(B2)) || (vec && !aligned16(vec)))
    return fail(ZDIT_EINVAL, "operand not 16-byte aligned");
  if (!ws || ws_bytes < zdit_op_gemm_splitk_workspace(epilogue, M, N, K)) return fail(ZDIT_EWORKSPACE, "workspace too small");
  GemmArgs g{};
  g.A = A; g.B = B; g.B2 = B2; g.C = C; g.M = M; g.N = N; g.K = K; g.lda = K; g.ldb = K;
  g.vec = epilogue == ZDIT_EPI_RESID ? vec : nullptr;
  g.out = compact_rows(M, N);
  float* part = (float*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  HIP_TRY(launch_gemm_splitk(epilogue, g, part, (hipStream_t)hip_stream, nullptr, 0, nullptr, nullptr, packed));
  return ok();
}
}  // namespace

extern "C" {

zdit_status zdit_op_gemm_splitk(int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A, const void* B,
                                const void* B2, const float* vec, void* C, void* ws, size_t ws_bytes,
                                void* hip_stream) {
  return gemm_splitk_op(false, epilogue, M, N, K, A, B, B2, vec, C, ws, ws_bytes, hip_stream);
}

zdit_status zdit_op_gemm_splitk_packed(int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A,
                                       const void* B, const void* B2, const float* vec, void* C, void* ws,
                                       size_t ws_bytes, void* hip_stream) {
  return gemm_splitk_op(true, epilogue, M, N, K, A, B, B2, vec, C, ws, ws_bytes, hip_stream);
}

zdit_status zdit_op_pack_weights(int32_t N, int32_t K, const void* src, void* dst, void* hip_stream) {
  if (N < 16 || K < 32 || N % 16 || K % 32) return fail(ZDIT_EUNSUPPORTED, "N %d (multiple of 16), K %d (multiple of 32)", N, K);
  if ((int64_t)N * K * 2 > INT32_MAX) return fail(ZDIT_EUNSUPPORTED, "matrix larger than 2 GiB");
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return fail(ZDIT_EINVAL, "NULL or misaligned pointer");
  const uintptr_t a0 = (uintptr_t)src, b0 = (uintptr_t)dst, n = (uintptr_t)N * K * 2;
  if (a0 < b0 + n && b0 < a0 + n) return fail(ZDIT_EINVAL, "src and dst overlap");
  HIP_TRY(launch_pack_bfrag(src, dst, N, K, (hipStream_t)hip_stream));
  return ok();
}

size_t zdit_op_embed_workspace(int32_t batch, int32_t max_len) {
  if (batch < 1 || max_len < 1) return 0;
  return al256((size_t)batch * max_len * 4) + 256;
}

zdit_status zdit_op_embed(int32_t batch, int32_t max_len, int32_t dim, int32_t vocab, const int32_t* ids,
                          const int32_t* len, const void* table, float* out, void* ws, size_t ws_bytes,
                          void* hip_stream) {
  if (batch < 1 || batch > ZDIT_MAX_BATCH || max_len < 1 || dim < 8 || dim % 8 || vocab < 1)
    return fail(ZDIT_EINVAL, "batch %d / max_len %d / dim %d / vocab %d", batch, max_len, dim, vocab);
  if (zdit_status s = check_ids(batch, max_len, vocab, ids, len)) return s;
  if (!table || !out || !aligned16(table) || !aligned16(out)) return fail(ZDIT_EINVAL, "table / out NULL or misaligned");
  if (!ws || ws_bytes < zdit_op_embed_workspace(batch, max_len)) return fail(ZDIT_EWORKSPACE, "workspace too small");
  char* base = (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  if (zdit_status s = embed_rows(batch, max_len, dim, ids, len, table, out, (int*)base, (hipStream_t)hip_stream))
    return s;
  return ok();
}

zdit_status zdit_op_qknorm_rope(int32_t batch, int32_t s_max, int32_t n_heads, int32_t n_kv_heads,
                                const int32_t* seq_len, void* qkv, const float* q_norm, const float* k_norm,
                                const float* cos, const float* sin, float eps, void* hip_stream) {
  if (batch < 1 || batch > ZDIT_MAX_BATCH || s_max < 1) return fail(ZDIT_EINVAL, "batch %d / s_max %d", batch, s_max);
  if (n_heads < 1 || n_kv_heads < 1 || n_heads > 64 || n_kv_heads > 64) return fail(ZDIT_EINVAL, "head counts");
  if (!seq_len || !qkv || !q_norm || !k_norm || !cos || !sin) return fail(ZDIT_EINVAL, "NULL pointer argument");
  if (!aligned16(qkv)) return fail(ZDIT_EINVAL, "qkv not 16-byte aligned");
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(ZDIT_EINVAL, "eps must be finite and >= 0");
  for (int b = 0; b < batch; ++b)
    if (seq_len[b] < 0 || seq_len[b] > s_max) return fail(ZDIT_EINVAL, "seq_len[%d] = %d", b, seq_len[b]);
  QkNormRopeArgs qa;
  qa.qkv = qkv; qa.row_stride = (int64_t)(n_heads + 2 * n_kv_heads) * kHeadDim; qa.k_col = n_heads * kHeadDim;
  qa.n_heads = n_heads; qa.n_kv_heads = n_kv_heads; qa.gq = q_norm; qa.gk = k_norm; qa.cos = cos; qa.sin = sin;
  qa.tab_bstride = (int64_t)s_max * 64; qa.eps = eps; qa.batch = batch; qa.s_max = s_max;
  for (int b = 0; b < kMaxBatch; ++b) qa.seq_len[b] = b < batch ? seq_len[b] : 0;
  HIP_TRY(launch_qknorm_rope(qa, (hipStream_t)hip_stream));
  return ok();
}

size_t zdit_op_attn_gqa_workspace(int32_t precision, int32_t batch, int32_t s_max, int32_t n_kv_heads) {
  if (batch < 1 || s_max < 1 || n_kv_heads < 1) return 0;
  return al256(attn_vt_bytes(precision, batch, s_max, n_kv_heads)) + 256;
}

zdit_status zdit_op_attn_gqa(int32_t precision, int32_t batch, int32_t s_max, int32_t n_heads, int32_t n_kv_heads,
                             int32_t causal, const int32_t* seq_len, const void* qkv, void* out, void* ws,
                             size_t ws_bytes, void* hip_stream) {
  if (precision != ZDIT_BF16 && precision != ZDIT_FP32_DEBUG) return fail(ZDIT_EINVAL, "precision %d", precision);
  if (batch < 1 || batch > ZDIT_MAX_BATCH || s_max < 1) return fail(ZDIT_EINVAL, "batch %d / s_max %d", batch, s_max);
  if (n_heads < 1 || n_heads > 64) return fail(ZDIT_EUNSUPPORTED, "n_heads %d (1..64)", n_heads);
  if (n_kv_heads < 1 || n_heads % n_kv_heads) return fail(ZDIT_EINVAL, "n_kv_heads %d must divide n_heads %d", n_kv_heads, n_heads);
  const int width = (n_heads + 2 * n_kv_heads) * kHeadDim;
  if (!qkv_fits(s_max, width * (precision == ZDIT_BF16 ? 1 : 2))) return fail(ZDIT_EUNSUPPORTED, "s_max %d too large", s_max);
  if (!seq_len || !qkv || !out) return fail(ZDIT_EINVAL, "NULL pointer argument");
  if (!aligned16(qkv) || !aligned16(out)) return fail(ZDIT_EINVAL, "qkv / out not 16-byte aligned");
  for (int b = 0; b < batch; ++b)
    if (seq_len[b] < 1 || seq_len[b] > s_max) return fail(ZDIT_EINVAL, "seq_len[%d] = %d", b, seq_len[b]);
  if (ws_bytes < zdit_op_attn_gqa_workspace(precision, batch, s_max, n_kv_heads) || (precision == ZDIT_BF16 && !ws))
    return fail(ZDIT_EWORKSPACE, "workspace too small");
  AttnArgs aa{};
  aa.qkv = qkv; aa.vt = ws; aa.out = out; aa.batch = batch; aa.s_max = s_max; aa.s_pad = round_up(s_max, 64);
  aa.n_heads = n_heads; aa.n_kv_heads = n_kv_heads; aa.row_stride = width;
  aa.k_col = n_heads * kHeadDim; aa.v_col = (n_heads + n_kv_heads) * kHeadDim; aa.causal = causal ? 1 : 0;
  for (int b = 0; b < kMaxBatch; ++b) aa.seq_len[b] = b < batch ? seq_len[b] : 0;
  HIP_TRY(launch_attn(precision, aa, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_device_info(int32_t device, int32_t* cu_count, int32_t* max_sclk_khz, int32_t* l2_bytes) {
  if (!cu_count || !max_sclk_khz || !l2_bytes) return fail(ZDIT_EINVAL, "NULL output");
  HIP_TRY(hipDeviceGetAttribute(cu_count, hipDeviceAttributeMultiprocessorCount, device));
  HIP_TRY(hipDeviceGetAttribute(max_sclk_khz, hipDeviceAttributeClockRate, device));
  HIP_TRY(hipDeviceGetAttribute(l2_bytes, hipDeviceAttributeL2CacheSize, device));
  return ok();
}

zdit_status zdit_op_mfma_peak(int32_t workgroups, int32_t iters, float* out, void* hip_stream) {
  if (workgroups < 1 || iters < 1) return fail(ZDIT_EINVAL, "workgroups %d / iters %d", workgroups, iters);
  if (!out || !aligned16(out)) return fail(ZDIT_EINVAL, "out NULL or not 16-byte aligned");
  HIP_TRY(launch_mfma_peak(workgroups, iters, out, (hipStream_t)hip_stream));
  return ok();
}

}  // extern "C"
