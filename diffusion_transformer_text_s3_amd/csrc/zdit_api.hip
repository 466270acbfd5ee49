// C ABI of the S3-DiT hot path: argument validation, workspace planning and the launch
// sequences of the block, the stack and the sampler.  Every argument is checked before the
// first launch; on error nothing is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "api_util.h"

using namespace zdit;

// Scratch memory of zdit_block_fwd_noalloc: a file-scope device array, one copy per device (the
// runtime places it when the code object loads on that device; it stays until the process
// ends).  Host code never passes the array's name to a kernel: its device address on each
// device comes from hipGetSymbolAddress with that device current, kept below.
static constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known
}  // namespace

std::string& zdit::api_error_text() {
  thread_local std::string text;
  return text;
}

namespace {

zdit_status check_dims(const zdit_dims* d) {
  if (!d) return fail(ZDIT_EINVAL, "dims is NULL");
  if (d->precision != ZDIT_BF16 && d->precision != ZDIT_FP32_DEBUG)
    return fail(ZDIT_EINVAL, "precision %d is neither ZDIT_BF16 nor ZDIT_FP32_DEBUG", d->precision);
  if (d->head_dim != kHeadDim) return fail(ZDIT_EUNSUPPORTED, "head_dim %d (only 128)", d->head_dim);
  if (d->n_heads < 1 || d->dim != d->n_heads * d->head_dim)
    return fail(ZDIT_EUNSUPPORTED, "dim %d != n_heads %d * head_dim", d->dim, d->n_heads);
  if (d->dim % 128 != 0 || d->dim > 4096) return fail(ZDIT_EUNSUPPORTED, "dim %d (multiple of 128, <= 4096)", d->dim);
  if (d->ffn_hidden < 128 || d->ffn_hidden % 128 != 0)
    return fail(ZDIT_EUNSUPPORTED, "ffn_hidden %d (positive multiple of 128)", d->ffn_hidden);
  const int* ax = d->rope_axes;
  if (ax[0] < 0 || ax[1] < 0 || ax[2] < 0 || (ax[0] | ax[1] | ax[2]) & 1 || ax[0] + ax[1] + ax[2] != d->head_dim)
    return fail(ZDIT_EUNSUPPORTED, "rope_axes %d/%d/%d must be even and sum to head_dim", ax[0], ax[1], ax[2]);
  if (d->c_dim < 64 || d->c_dim % 64 != 0 || d->c_dim > 1024)
    return fail(ZDIT_EUNSUPPORTED, "c_dim %d (multiple of 64, <= 1024)", d->c_dim);
  if (!(d->norm_eps >= 0.f) || !isfinite(d->norm_eps)) return fail(ZDIT_EINVAL, "norm_eps must be finite and >= 0");
  if (d->flags & ~ZDIT_CHECK_FINITE) return fail(ZDIT_EINVAL, "unknown flag bits 0x%x", (unsigned)d->flags);
  return ZDIT_OK;
}

// ------------------------------------------------------------------ non-finite checks
// ZDIT_CHECK_FINITE: checkpoints of one call raise flags[k]; after each step the latch keeps the
// first (step, checkpoint) whose flag is set in first[0..1].  The region holds n flags + 2.
struct Check {
  int* flags = nullptr;  // nullptr: checking off
  int* first = nullptr;
  int n = 0;
};

size_t check_bytes(int n) { return al256((size_t)(n + 2) * 4); }

Check check_at(const zdit_dims& d, char* region, int n) {
  Check c;
  if (d.flags & ZDIT_CHECK_FINITE) {
    c.flags = (int*)region;
    c.first = c.flags + n;
    c.n = n;
  }
  return c;
}

// flags = 0, first = {-1, -1}
hipError_t check_begin(const Check& c, hipStream_t st) {
  if (!c.flags) return hipSuccess;
  if (hipError_t e = launch_fill_i32(c.flags, c.n, 0, st)) return e;
  return launch_fill_i32(c.first, 2, -1, st);
}

// flags[k] |= any non-finite value in the valid rows of a branch-strided fp32 buffer
hipError_t check_rows(const Check& c, int k, const float* p, int64_t bstride, int64_t ld, int rows_per_batch,
                      int batch, int width, const int* valid, hipStream_t st) {
  if (!c.flags) return hipSuccess;
  FiniteArgs a;
  a.p = p; a.bstride = bstride; a.ld = ld; a.rows_per_batch = rows_per_batch; a.batch = batch; a.width = width;
  for (int b = 0; b < kMaxBatch; ++b) a.valid[b] = b < batch ? (valid ? valid[b] : rows_per_batch) : 0;
  a.flag = c.flags + k;
  return launch_finite_check(a, st);
}

hipError_t check_latch(const Check& c, int step, hipStream_t st) {
  if (!c.flags) return hipSuccess;
  return launch_finite_latch(c.flags, c.n, step, c.first, st);
}

// Reads the verdict back (synchronising the stream); *step / *where = -1 when every value was
// finite.
zdit_status check_read(const Check& c, hipStream_t st, int* step, int* where) {
  int h[2] = {-1, -1};
  if (c.flags) {
    HIP_TRY(hipMemcpyAsync(h, c.first, sizeof h, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
  }
  *step = h[0];
  *where = h[1];
  return ZDIT_OK;
}

// ------------------------------------------------------------------ block workspace plan
// Rows per branch up to which the block's four GEMMs split K into fp32 partials summed in a
// fixed order (tile_split_plan): with a few hundred rows the 256 x 256 tiles would occupy a
// small part of the chip (the 256 px and 512 px images, the caption refiners).  The choice
// depends on the rows per branch and the split on N and K only, so a branch computed alone and
// the same branch in a batch (or the shared image path and its per-branch copies) agree to the
// bit.
constexpr int kSplitRows = 512;

bool use_split(const zdit_dims& d, int s) { return d.precision == ZDIT_BF16 && s <= kSplitRows; }

// fp32 partial planes of the largest of the block's four split GEMMs at M rows
size_t split_part_bytes(const zdit_dims& d, int M) {
  const int D = d.dim, H = d.ffn_hidden;
  size_t m = tile_split_workspace(EPI_STORE, M, 3 * D, D);
  m = std::max(m, tile_split_workspace(EPI_RESID, M, D, D));
  m = std::max(m, tile_split_workspace(EPI_SWIGLU, M, H, D));
  m = std::max(m, tile_split_workspace(EPI_RESID, M, D, H));
  return m;
}

struct BlockPlan {
  size_t mod, chk, part, h, qkv, vt, o, u, total;
};

// A GEMM of the block: the whole-K kernel, or the K-split one with partials in `part`.
hipError_t block_gemm(const zdit_dims& d, bool split, int epi, const GemmArgs& g, void* part, hipStream_t st) {
  if (split) return launch_gemm_bf16_split(epi, g, (float*)part, st);
  return gemm(d.precision, epi, g, st);
}

// checkpoints of zdit_block_fwd: the input rows, the output rows
constexpr int kBlockChecks = 2;

BlockPlan plan_block(const zdit_dims& d, int B, int s) {
  const size_t M = (size_t)B * s, ab = act_bytes(d.precision);
  BlockPlan p;
  size_t off = 0;
  p.mod = off; off += al256((size_t)B * 6 * d.dim * 4);
  p.chk = off; off += check_bytes(kBlockChecks);
  p.part = off; off += use_split(d, s) ? al256(split_part_bytes(d, (int)M)) : 0;
  p.h = off;   off += al256(M * d.dim * ab);
  const size_t r0 = off;
  p.qkv = off; off += al256(M * 3 * d.dim * ab);
  p.vt = off;  off += al256(attn_vt_bytes(d.precision, B, s, d.n_heads));
  p.o = off;   off += al256(M * d.dim * ab);
  p.u = r0;  // the SwiGLU activation reuses the attention region (dead by then)
  off = std::max(off, r0 + al256(M * (size_t)d.ffn_hidden * ab));
  p.total = off;
  return p;
}


// q, k, v projection of h [B * s, nh * 128] (rows of branch b at b * s), RoPE on q and k,
// and joint attention into o.  In bf16 with s % 32 == 0 the projection's epilogue rotates q, k
// and writes V^T itself (one kernel instead of GEMM + RoPE + transpose); otherwise the GEMM
// stores q, k, v and separate kernels rotate and transpose.  The results are bit-identical.
zdit_status qkv_attention(int P, int nh, int B, int s, const int* seq_len, const void* h, const void* w_qkv,
                          void* qkv, void* vt, void* o, const float* cosT, const float* sinT,
                          int64_t tab_bstride, hipStream_t st, void* part = nullptr) {
  const int D = nh * kHeadDim, M = B * s;
  AttnArgs aa{};
  aa.qkv = qkv; aa.vt = vt; aa.out = o; aa.batch = B; aa.s_max = s; aa.s_pad = round_up(s, 64);
  aa.n_heads = nh;
  for (int b = 0; b < kMaxBatch; ++b) aa.seq_len[b] = b < B ? seq_len[b] : 0;

  GemmArgs g{};
  g.A = h; g.B = w_qkv; g.C = qkv; g.M = M; g.N = 3 * D; g.K = D; g.lda = D; g.ldb = D;
  if (P == ZDIT_BF16 && s % 32 == 0 && !part) {
    g.out.rows_per_batch = s; g.out.batch_stride = (int64_t)s * 3 * D; g.out.ld = 3 * D;
    for (int b = 0; b < kMaxBatch; ++b) { g.out.valid[b] = b < B ? s : 0; g.seq[b] = b < B ? seq_len[b] : 0; }
    g.rope_cos = cosT; g.rope_sin = sinT; g.rope_bstride = tab_bstride;
    g.vt = vt; g.vt_pad = aa.s_pad; g.n_heads = nh;
    HIP_TRY(launch_gemm_bf16(EPI_QKV, g, st));
    HIP_TRY(launch_vt_tail_zero(aa, st));
    aa.vt_ready = 1;
  } else {
    g.out = compact_rows(M, 3LL * D);
    if (part) HIP_TRY(launch_gemm_bf16_split(EPI_STORE, g, (float*)part, st));
    else HIP_TRY(gemm(P, EPI_STORE, g, st));
    RopeArgs ra;
    ra.qkv = qkv; ra.cos = cosT; ra.sin = sinT; ra.tab_bstride = tab_bstride;
    ra.batch = B; ra.s_max = s; ra.n_heads = nh;
    for (int b = 0; b < kMaxBatch; ++b) ra.seq_len[b] = b < B ? seq_len[b] : 0;
    HIP_TRY(launch_rope(P, ra, st));
  }
  HIP_TRY(launch_attn(P, aa, st));
  return ZDIT_OK;
}

// One block on B branches of s rows each.  x rows are x + b * x_bstride + r * dim.
// mod: [B][6][dim] fp32 already computed, or NULL (no adaLN).
zdit_status block_forward(const zdit_dims& d, const zdit_block_w& w, int B, int s,
                          const int* seq_len, float* x, int64_t x_bstride, const float* mod,
                          const float* cosT, const float* sinT, int64_t tab_bstride, char* ws,
                          hipStream_t st) {
  const int P = d.precision, D = d.dim, H = d.ffn_hidden, M = B * s;
  const BlockPlan pl = plan_block(d, B, s);
  const bool split = use_split(d, s);
  void* part = split ? ws + pl.part : nullptr;
  void* h = ws + pl.h;
  void* qkv = ws + pl.qkv;
  void* vt = ws + pl.vt;
  void* o = ws + pl.o;
  void* u = ws + pl.u;

  NormArgs na;
  na.x = x; na.x_bstride = x_bstride; na.rows_per_batch = s; na.batch = B; na.dim = D;
  na.gain = w.norm1; na.mod_bstride = 6LL * D;
  na.shift = mod ? mod : nullptr; na.scale = mod ? mod + D : nullptr;
  na.eps = d.norm_eps; na.out = h;
  for (int b = 0; b < kMaxBatch; ++b) na.valid[b] = b < B ? seq_len[b] : 0;
  HIP_TRY(launch_rmsnorm_mod(P, na, st));

  {
    // a one-range plan runs the whole-K GEMM, so the q/k/v projection then takes the fused form
    const bool qkv_split = split && tile_split_plan(EPI_STORE, 3 * D, D).splits > 1;
    const zdit_status rc = qkv_attention(P, d.n_heads, B, s, seq_len, h, w.w_qkv, qkv, vt, o, cosT, sinT,
                                         tab_bstride, st, qkv_split ? part : nullptr);
    if (rc != ZDIT_OK) return rc;
  }

  RowMap xr;
  xr.rows_per_batch = s; xr.batch_stride = x_bstride; xr.ld = D;
  for (int b = 0; b < kMaxBatch; ++b) xr.valid[b] = b < B ? seq_len[b] : 0;

  GemmArgs g{};
  g.A = o; g.B = w.w_out; g.C = x; g.M = M; g.N = D; g.K = D; g.lda = D; g.ldb = D;
  g.vec = mod ? mod + 2LL * D : nullptr; g.vec_bstride = 6LL * D; g.out = xr;
  HIP_TRY(block_gemm(d, split, EPI_RESID, g, part, st));

  na.gain = w.norm2;
  na.shift = mod ? mod + 3LL * D : nullptr; na.scale = mod ? mod + 4LL * D : nullptr;
  HIP_TRY(launch_rmsnorm_mod(P, na, st));

  g = GemmArgs{};
  g.A = h; g.B = w.w1; g.B2 = w.w3; g.C = u; g.M = M; g.N = H; g.K = D; g.lda = D; g.ldb = D;
  g.out = compact_rows(M, H);
  HIP_TRY(block_gemm(d, split, EPI_SWIGLU, g, part, st));

  g = GemmArgs{};
  g.A = u; g.B = w.w2; g.C = x; g.M = M; g.N = D; g.K = H; g.lda = H; g.ldb = H;
  g.vec = mod ? mod + 5LL * D : nullptr; g.vec_bstride = 6LL * D; g.out = xr;
  HIP_TRY(block_gemm(d, split, EPI_RESID, g, part, st));
  return ZDIT_OK;
}

zdit_status check_block_w(const zdit_block_w* w, bool need_ada) {
  if (!w) return fail(ZDIT_EINVAL, "block weights NULL");
  const void* ptrs[] = {w->w_qkv, w->w_out, w->w1, w->w3, w->w2, w->norm1, w->norm2};
  const char* names[] = {"w_qkv", "w_out", "w1", "w3", "w2", "norm1", "norm2"};
  for (int i = 0; i < 7; ++i) {
    if (!ptrs[i]) return fail(ZDIT_EINVAL, "block weight %s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(ZDIT_EINVAL, "block weight %s not 16-byte aligned", names[i]);
  }
  if ((w->w_ada == nullptr) != (w->b_ada == nullptr)) return fail(ZDIT_EINVAL, "w_ada and b_ada must both be set or both NULL");
  if (need_ada && !w->w_ada) return fail(ZDIT_EINVAL, "this block needs adaLN weights");
  if (w->w_ada && (!aligned16(w->w_ada) || !aligned16(w->b_ada))) return fail(ZDIT_EINVAL, "adaLN weights not 16-byte aligned");
  return ZDIT_OK;
}

// ------------------------------------------------------------------ stack
struct StackPlan {
  int nimg, gh, gw, max_nc, s_max;
  int nc[kMaxBatch], S[kMaxBatch];
  size_t x, c, mod, fmod, chk, tab_img_c, tab_img_s, tab_cap_c, tab_cap_s, tab_j_c, tab_j_s, tok,
      capa, ftok, blk, total;
  BlockPlan bp;
};

// Checkpoints of a stack forward: 0 the latents, 1 the caption features, then the residual
// stream after each noise refiner, context refiner and main block, then the velocity.
int stack_checks(const zdit_model_cfg& cfg) { return 3 + cfg.n_noise_ref + cfg.n_ctx_ref + cfg.n_main; }

// The place a stack checkpoint names, for zdit_last_error().
std::string stack_check_name(const zdit_model_cfg& cfg, int k) {
  char buf[96];
  const int nr = cfg.n_noise_ref, cr = cfg.n_ctx_ref, nm = cfg.n_main;
  if (k == 0) return "the input latents";
  if (k == 1) return "the caption features (valid rows)";
  k -= 2;
  if (k < nr) { snprintf(buf, sizeof buf, "the image rows after noise refiner %d", k); return buf; }
  k -= nr;
  if (k < cr) { snprintf(buf, sizeof buf, "the caption rows after context refiner %d", k); return buf; }
  k -= cr;
  if (k < nm) { snprintf(buf, sizeof buf, "the residual stream after main block %d", k); return buf; }
  return "the velocity";
}

// The adaLN modulations of the n blocks of a stage (the same c for all), in launches of up to
// kMaxAdaJobs blocks: block i's six vectors at mod + i * batch * 6 * dim.
hipError_t stage_adaln(int precision, int batch, const zdit_dims& d, const float* c, const zdit_block_w* blocks, int n,
                       float* mod, hipStream_t st) {
  const int D = d.dim;
  for (int i0 = 0; i0 < n; i0 += kMaxAdaJobs) {
    const int nj = std::min(kMaxAdaJobs, n - i0);
    const void* w[kMaxAdaJobs];
    const float* b[kMaxAdaJobs];
    float* out[kMaxAdaJobs];
    for (int j = 0; j < nj; ++j) {
      w[j] = blocks[i0 + j].w_ada;
      b[j] = blocks[i0 + j].b_ada;
      out[j] = mod + (size_t)(i0 + j) * batch * 6 * D;
    }
    if (hipError_t e = launch_adaln_multi(precision, batch, d.c_dim, 6 * D, c, w, b, out, nj, st)) return e;
  }
  return hipSuccess;
}

StackPlan plan_stack(const zdit_model_cfg& cfg, int B, int lat_h, int lat_w, int max_cap_len,
                     const int* cap_len) {
  StackPlan p;
  const zdit_dims& d = cfg.d;
  const int ab = act_bytes(d.precision), D = d.dim, hp = d.head_dim / 2;
  p.gh = lat_h / cfg.patch; p.gw = lat_w / cfg.patch; p.nimg = p.gh * p.gw;
  p.max_nc = 0;
  for (int b = 0; b < kMaxBatch; ++b) { p.nc[b] = 0; p.S[b] = 0; }
  if (cap_len) {
    for (int b = 0; b < B; ++b) {
      p.nc[b] = round_up(cap_len[b], cfg.seq_multiple);
      p.max_nc = std::max(p.max_nc, p.nc[b]);
      p.S[b] = p.nimg + p.nc[b];
    }
  } else {
    p.max_nc = round_up(std::min(max_cap_len, cfg.max_cap_len), cfg.seq_multiple);  // upper bound
  }
  p.s_max = p.nimg + p.max_nc;
  const int F = cfg.patch * cfg.patch * cfg.latent_ch;
  size_t off = 0;
  // first, so that its offset does not depend on the caption lengths
  p.chk = off; off += check_bytes(stack_checks(cfg));
  p.x = off; off += al256((size_t)B * p.s_max * D * 4);
  p.c = off; off += al256((size_t)B * d.c_dim * 4);
  // one modulation set per adaLN block of a stage (noise refiners, or main blocks), computed by one launch
  const int nmod = std::max(1, std::max(cfg.n_noise_ref, cfg.n_main));
  p.mod = off; off += al256((size_t)nmod * B * 6 * D * 4);
  p.fmod = off; off += al256((size_t)B * 2 * D * 4);
  p.tab_img_c = off; off += al256((size_t)p.nimg * hp * 4);
  p.tab_img_s = off; off += al256((size_t)p.nimg * hp * 4);
  p.tab_cap_c = off; off += al256((size_t)p.max_nc * hp * 4);
  p.tab_cap_s = off; off += al256((size_t)p.max_nc * hp * 4);
  p.tab_j_c = off; off += al256((size_t)p.s_max * hp * 4);
  p.tab_j_s = off; off += al256((size_t)p.s_max * hp * 4);
  p.tok = off; off += al256((size_t)B * p.nimg * F * ab);
  p.capa = off; off += al256((size_t)B * max_cap_len * cfg.cap_dim * ab);
  p.ftok = off; off += al256((size_t)B * p.nimg * F * 4);
  p.bp = plan_block(d, B, p.s_max);  // the largest block call (main blocks)
  p.blk = off; off += p.bp.total;
  p.total = off;
  return p;
}

zdit_status check_cfg(const zdit_model_cfg* cfg) {
  if (!cfg) return fail(ZDIT_EINVAL, "cfg is NULL");
  zdit_status s = check_dims(&cfg->d);
  if (s) return s;
  if (cfg->latent_ch != 16 || cfg->patch != 2)
    return fail(ZDIT_EUNSUPPORTED, "latent_ch %d / patch %d (only 16 / 2)", cfg->latent_ch, cfg->patch);
  if (cfg->cap_dim < 64 || cfg->cap_dim % 64) return fail(ZDIT_EUNSUPPORTED, "cap_dim %d (multiple of 64)", cfg->cap_dim);
  if (cfg->t_freq != cfg->d.c_dim) return fail(ZDIT_EUNSUPPORTED, "t_freq %d must equal c_dim %d", cfg->t_freq, cfg->d.c_dim);
  if (cfg->seq_multiple < 1 || cfg->seq_multiple > 512) return fail(ZDIT_EINVAL, "seq_multiple %d", cfg->seq_multiple);
  if (cfg->max_cap_len < 1 || cfg->max_cap_len > 4096) return fail(ZDIT_EINVAL, "max_cap_len %d", cfg->max_cap_len);
  if (cfg->n_noise_ref < 0 || cfg->n_ctx_ref < 0 || cfg->n_main < 0) return fail(ZDIT_EINVAL, "negative block count");
  if (!(cfg->rope_theta > 0.f) || !(cfg->t_scale > 0.f)) return fail(ZDIT_EINVAL, "rope_theta and t_scale must be > 0");
  return ZDIT_OK;
}

zdit_status check_model_w(const zdit_model_cfg& cfg, const zdit_model_w* w) {
  if (!w) return fail(ZDIT_EINVAL, "model weights NULL");
  const void* ptrs[] = {w->x_emb_w, w->x_emb_b, w->cap_emb_w, w->cap_emb_b, w->cap_pad, w->t_w1, w->t_b1,
                        w->t_w2, w->t_b2, w->final_norm, w->final_ada_w, w->final_ada_b, w->final_w, w->final_b};
  for (const void* p : ptrs) {
    if (!p) return fail(ZDIT_EINVAL, "a model weight pointer is NULL");
    if (!aligned16(p)) return fail(ZDIT_EINVAL, "a model weight pointer is not 16-byte aligned");
  }
  if ((cfg.n_noise_ref && !w->noise_ref) || (cfg.n_ctx_ref && !w->ctx_ref) || (cfg.n_main && !w->main))
    return fail(ZDIT_EINVAL, "block weight array NULL");
  for (int i = 0; i < cfg.n_noise_ref; ++i) if (zdit_status s = check_block_w(&w->noise_ref[i], true)) return s;
  for (int i = 0; i < cfg.n_ctx_ref; ++i) if (zdit_status s = check_block_w(&w->ctx_ref[i], false)) return s;
  for (int i = 0; i < cfg.n_main; ++i) if (zdit_status s = check_block_w(&w->main[i], true)) return s;
  return ZDIT_OK;
}

// The attention kernel addresses one branch's qkv rows ([s_max, 3 dim] bf16) with 32-bit byte
// offsets.
bool seq_fits(int64_t s_max, int dim) { return s_max * 6 * dim <= INT32_MAX; }

zdit_status check_stack_args(const zdit_model_cfg* cfg, const zdit_model_w* w, int batch, int lat_h,
                             int lat_w, const float* latents, const float* cap_feats, int max_cap_len,
                             const int* cap_len, const float* t, const float* velocity) {
  if (zdit_status s = check_cfg(cfg)) return s;
  if (zdit_status s = check_model_w(*cfg, w)) return s;
  if (batch < 1 || batch > ZDIT_MAX_BATCH) return fail(ZDIT_EINVAL, "batch %d (1..%d)", batch, ZDIT_MAX_BATCH);
  if (lat_h < 2 || lat_w < 2 || lat_h % 2 || lat_w % 2) return fail(ZDIT_EINVAL, "lat_h %d / lat_w %d must be even and >= 2", lat_h, lat_w);
  if ((int64_t)(lat_h / 2) * (lat_w / 2) > (1 << 20)) return fail(ZDIT_EUNSUPPORTED, "too many image tokens");
  if (max_cap_len < 1) return fail(ZDIT_EINVAL, "max_cap_len %d", max_cap_len);
  const int64_t s_bound = (int64_t)(lat_h / 2) * (lat_w / 2) +
                          round_up(std::min(max_cap_len, cfg->max_cap_len), cfg->seq_multiple);
  if (!seq_fits(s_bound, cfg->d.dim)) return fail(ZDIT_EUNSUPPORTED, "sequence of %lld tokens too long", (long long)s_bound);
  if (!latents || !cap_feats || !velocity || !cap_len || !t) return fail(ZDIT_EINVAL, "NULL pointer argument");
  if (!aligned16(latents) || !aligned16(cap_feats) || !aligned16(velocity)) return fail(ZDIT_EINVAL, "device pointer not 16-byte aligned");
  const int lim = std::min(max_cap_len, cfg->max_cap_len);
  for (int b = 0; b < batch; ++b) {
    if (cap_len[b] < 1 || cap_len[b] > lim) return fail(ZDIT_EINVAL, "cap_len[%d] = %d outside 1..%d", b, cap_len[b], lim);
    if (!isfinite(t[b])) return fail(ZDIT_EINVAL, "t[%d] is not finite", b);
  }
  return ZDIT_OK;
}

// Caption cache: the caption rows after the context refiners depend only on the caption
// features (no timestep, no latent), so a caller running several steps on the same captions
// can pass cap_out on the first call ([B][max n_cap][dim] fp32, filled) and cap_in on the
// later ones (copied in place of cap-embed, learned pad and context refiners).
struct CapCache {
  const float* in = nullptr;
  float* out = nullptr;
};

// chk / step: the ZDIT_CHECK_FINITE checkpoints (off when chk.flags is NULL) and the sampler
// step they are latched under.
zdit_status stack_forward(const zdit_model_cfg& cfg, const zdit_model_w& w, int B, int lat_h, int lat_w,
                          const float* latents, int64_t lat_bstride, const float* cap_feats,
                          int max_cap_len, const int* cap_len, const float* t, float* velocity,
                          char* ws, hipStream_t st, CapCache cache = CapCache{}, Check chk = Check{},
                          int step = 0) {
  const zdit_dims& d = cfg.d;
  const int P = d.precision, D = d.dim, F = cfg.patch * cfg.patch * cfg.latent_ch;
  const StackPlan p = plan_stack(cfg, B, lat_h, lat_w, max_cap_len, cap_len);
  float* x = (float*)(ws + p.x);
  float* c = (float*)(ws + p.c);
  float* mod = (float*)(ws + p.mod);
  float* fmod = (float*)(ws + p.fmod);
  char* bws = ws + p.blk;
  const int64_t xb = (int64_t)p.s_max * D;

  const int64_t lat_n = (int64_t)cfg.latent_ch * lat_h * lat_w;
  const int nr = cfg.n_noise_ref, cr = cfg.n_ctx_ref;
  HIP_TRY(check_rows(chk, 0, latents, lat_bstride, lat_n, 1, lat_bstride == 0 ? 1 : B, (int)lat_n, nullptr, st));
  if (!cache.in)
    HIP_TRY(check_rows(chk, 1, cap_feats, (int64_t)max_cap_len * cfg.cap_dim, cfg.cap_dim, max_cap_len, B,
                       cfg.cap_dim, cap_len, st));

  // conditioning
  HIP_TRY(launch_temb(B, t, cfg.t_freq, d.c_dim, cfg.t_scale, w.t_w1, w.t_b1, w.t_w2, w.t_b2, c, st));

  // Image tokens -> rows [0, nimg) of every branch.  When every branch sees the same latent
  // (branch stride 0) at the same model time, the image rows through the noise refiners are
  // identical per branch (no kernel mixes branches, and each output's arithmetic does not
  // depend on the batch), so they are computed for branch 0 and copied.
  bool same_img = B > 1 && lat_bstride == 0;
  for (int b = 1; b < B && same_img; ++b) same_img = (t[b] == t[0]);
  const int Bi = same_img ? 1 : B;
  HIP_TRY(launch_patchify(P, Bi, cfg.latent_ch, lat_h, lat_w, latents, lat_bstride, ws + p.tok, st));
  GemmArgs g{};
  g.A = ws + p.tok; g.B = w.x_emb_w; g.C = x; g.vec = w.x_emb_b;
  g.M = Bi * p.nimg; g.N = D; g.K = F; g.lda = F; g.ldb = F;
  g.out.rows_per_batch = p.nimg; g.out.batch_stride = xb; g.out.ld = D;
  for (int b = 0; b < kMaxBatch; ++b) g.out.valid[b] = p.nimg;
  HIP_TRY(gemm(P, EPI_BIAS, g, st));

  // RoPE tables, shared by every branch (positions of valid rows do not depend on the branch)
  RopeTabArgs rt;
  rt.batch = 1; rt.grid_h = p.gh; rt.grid_w = p.gw; rt.theta = cfg.rope_theta;
  for (int i = 0; i < 3; ++i) rt.axes[i] = d.rope_axes[i];
  rt.n_cap[0] = p.max_nc;
  float* ti_c = (float*)(ws + p.tab_img_c); float* ti_s = (float*)(ws + p.tab_img_s);
  float* tc_c = (float*)(ws + p.tab_cap_c); float* tc_s = (float*)(ws + p.tab_cap_s);
  float* tj_c = (float*)(ws + p.tab_j_c); float* tj_s = (float*)(ws + p.tab_j_s);
  rt.kind = ZDIT_SEQ_IMAGE; rt.s_max = p.nimg; rt.cos = ti_c; rt.sin = ti_s;
  HIP_TRY(launch_rope_tables(rt, st));
  rt.kind = ZDIT_SEQ_CAPTION; rt.s_max = p.max_nc; rt.cos = tc_c; rt.sin = tc_s;
  HIP_TRY(launch_rope_tables(rt, st));
  rt.kind = ZDIT_SEQ_JOINT; rt.s_max = p.s_max; rt.cos = tj_c; rt.sin = tj_s;
  HIP_TRY(launch_rope_tables(rt, st));

  int len[kMaxBatch];
  // noise refiners: image rows only (branch 0 only when the image rows are shared)
  for (int b = 0; b < B; ++b) len[b] = p.nimg;
  HIP_TRY(stage_adaln(P, Bi, d, c, w.noise_ref, cfg.n_noise_ref, mod, st));
  for (int i = 0; i < cfg.n_noise_ref; ++i) {
    const zdit_block_w& bw = w.noise_ref[i];
    float* mod_i = mod + (size_t)i * Bi * 6 * D;
    if (zdit_status s = block_forward(d, bw, Bi, p.nimg, len, x, xb, mod_i, ti_c, ti_s, 0, bws, st)) return s;
    HIP_TRY(check_rows(chk, 2 + i, x, xb, D, p.nimg, Bi, D, nullptr, st));
  }
  if (same_img)
    HIP_TRY(launch_copy_rows(x, 0, x + xb, xb, B - 1, (int64_t)p.nimg * D, st));

  // caption tokens -> rows [nimg, nimg + n_cap_b): cap-embed, learned pad, context refiners
  float* xcap = x + (int64_t)p.nimg * D;
  const int64_t cache_bstride = (int64_t)p.max_nc * D;
  if (cache.in) {
    HIP_TRY(launch_copy_rows(cache.in, cache_bstride, xcap, xb, B, cache_bstride, st));
  } else {
    HIP_TRY(launch_convert(P, cap_feats, ws + p.capa, (int64_t)B * max_cap_len * cfg.cap_dim, st));
    g = GemmArgs{};
    g.A = ws + p.capa; g.B = w.cap_emb_w; g.C = xcap; g.vec = w.cap_emb_b;
    g.M = B * max_cap_len; g.N = D; g.K = cfg.cap_dim; g.lda = cfg.cap_dim; g.ldb = cfg.cap_dim;
    g.out.rows_per_batch = max_cap_len; g.out.batch_stride = xb; g.out.ld = D;
    for (int b = 0; b < kMaxBatch; ++b) g.out.valid[b] = b < B ? cap_len[b] : 0;
    HIP_TRY(gemm(P, EPI_BIAS, g, st));
    HIP_TRY(launch_cap_pad(B, p.s_max, D, p.nimg, cap_len, cfg.seq_multiple, w.cap_pad, x, st));
    // context refiners: caption rows only, no adaLN
    for (int b = 0; b < B; ++b) len[b] = p.nc[b];
    for (int i = 0; i < cfg.n_ctx_ref; ++i) {
      if (zdit_status s = block_forward(d, w.ctx_ref[i], B, p.max_nc, len, xcap, xb, nullptr, tc_c, tc_s, 0, bws, st))
        return s;
      HIP_TRY(check_rows(chk, 2 + nr + i, xcap, xb, D, p.max_nc, B, D, p.nc, st));
    }
    if (cache.out) HIP_TRY(launch_copy_rows(xcap, xb, cache.out, cache_bstride, B, cache_bstride, st));
  }

  // main blocks on the joint sequence
  for (int b = 0; b < B; ++b) len[b] = p.S[b];
  HIP_TRY(stage_adaln(P, B, d, c, w.main, cfg.n_main, mod, st));
  for (int i = 0; i < cfg.n_main; ++i) {
    const zdit_block_w& bw = w.main[i];
    float* mod_i = mod + (size_t)i * B * 6 * D;
    if (zdit_status s = block_forward(d, bw, B, p.s_max, len, x, xb, mod_i, tj_c, tj_s, 0, bws, st)) return s;
    HIP_TRY(check_rows(chk, 2 + nr + cr + i, x, xb, D, p.s_max, B, D, p.S, st));
  }
  // final layer on the image rows
  HIP_TRY(launch_adaln(P, B, d.c_dim, 2 * D, c, w.final_ada_w, w.final_ada_b, fmod, st));
  NormArgs na;
  na.x = x; na.x_bstride = xb; na.rows_per_batch = p.nimg; na.batch = B; na.dim = D;
  na.gain = w.final_norm; na.shift = fmod; na.scale = fmod + D; na.mod_bstride = 2LL * D;
  na.eps = d.norm_eps; na.out = bws + p.bp.h;
  for (int b = 0; b < kMaxBatch; ++b) na.valid[b] = p.nimg;
  HIP_TRY(launch_rmsnorm_mod(P, na, st));
  g = GemmArgs{};
  g.A = bws + p.bp.h; g.B = w.final_w; g.C = ws + p.ftok; g.vec = w.final_b;
  g.M = B * p.nimg; g.N = F; g.K = D; g.lda = D; g.ldb = D;
  g.out = compact_rows(B * p.nimg, F);
  HIP_TRY(gemm(P, EPI_BIAS, g, st));
  HIP_TRY(launch_unpatchify(B, cfg.latent_ch, lat_h, lat_w, (const float*)(ws + p.ftok), velocity, st));
  HIP_TRY(check_rows(chk, 2 + nr + cr + cfg.n_main, velocity, lat_n, lat_n, 1, B, (int)lat_n, nullptr, st));
  HIP_TRY(check_latch(chk, step, st));
  return ZDIT_OK;
}

// Arguments of a block forward other than the workspace.
zdit_status check_block_args(const zdit_dims* dims, const zdit_block_w* w, int batch, int s_max, const int* seq_len,
                             const float* x, const float* c, const float* rope_cos, const float* rope_sin) {
  if (zdit_status s = check_dims(dims)) return s;
  if (zdit_status s = check_block_w(w, false)) return s;
  if (batch < 1 || batch > ZDIT_MAX_BATCH) return fail(ZDIT_EINVAL, "batch %d (1..%d)", batch, ZDIT_MAX_BATCH);
  if (s_max < 1 || (int64_t)batch * s_max > (1 << 24)) return fail(ZDIT_EINVAL, "s_max %d", s_max);
  if (!seq_fits(s_max, dims->dim)) return fail(ZDIT_EUNSUPPORTED, "s_max %d too long for dim %d", s_max, dims->dim);
  if (!seq_len) return fail(ZDIT_EINVAL, "seq_len is NULL");
  for (int b = 0; b < batch; ++b)
    if (seq_len[b] < 1 || seq_len[b] > s_max) return fail(ZDIT_EINVAL, "seq_len[%d] = %d outside 1..%d", b, seq_len[b], s_max);
  if (!x || !rope_cos || !rope_sin) return fail(ZDIT_EINVAL, "NULL pointer argument");
  if (w->w_ada && !c) return fail(ZDIT_EINVAL, "c is NULL but the block has adaLN weights");
  if (!aligned16(x) || !aligned16(rope_cos) || !aligned16(rope_sin) || (c && !aligned16(c)))
    return fail(ZDIT_EINVAL, "device pointer not 16-byte aligned");
  return ZDIT_OK;
}

// The launch sequence of zdit_block_fwd on a validated call, with workspace ws (at least
// plan_block().total bytes, 256-aligned).
zdit_status run_block(const zdit_dims& d, const zdit_block_w& w, int batch, int s_max, const int* seq_len, float* x,
                      const float* c, const float* rope_cos, const float* rope_sin, char* ws, hipStream_t st) {
  const BlockPlan pl = plan_block(d, batch, s_max);
  const int D = d.dim;
  const Check chk = check_at(d, ws + pl.chk, kBlockChecks);
  HIP_TRY(check_begin(chk, st));
  HIP_TRY(check_rows(chk, 0, x, (int64_t)s_max * D, D, s_max, batch, D, seq_len, st));
  float* mod = nullptr;
  if (w.w_ada) {
    mod = (float*)(ws + pl.mod);
    HIP_TRY(launch_adaln(d.precision, batch, d.c_dim, 6 * D, c, w.w_ada, w.b_ada, mod, st));
  }
  if (zdit_status s = block_forward(d, w, batch, s_max, seq_len, x, (int64_t)s_max * D, mod, rope_cos, rope_sin,
                                    (int64_t)s_max * (d.head_dim / 2), ws, st))
    return s;
  HIP_TRY(check_rows(chk, 1, x, (int64_t)s_max * D, D, s_max, batch, D, seq_len, st));
  HIP_TRY(check_latch(chk, 0, st));
  int step, where;
  if (zdit_status s = check_read(chk, st, &step, &where)) return s;
  if (where == 0) return fail(ZDIT_ENONFINITE, "non-finite value in the valid rows of the input x");
  if (where == 1) return fail(ZDIT_ENONFINITE, "non-finite value in the block output (residual stream)");
  return ok();
}

double sigma_at(int i, int n, double shift) {
  const double t = (double)i / (double)n;
  return shift * (1.0 - t) / (shift * (1.0 - t) + t);
}

}  // namespace

extern "C" {

const char* zdit_last_error(void) { return api_error_text().c_str(); }
int32_t zdit_abi_version(void) { return ZDIT_ABI_VERSION; }

size_t zdit_block_workspace(const zdit_dims* dims, int32_t batch, int32_t s_max) {
  if (check_dims(dims) || batch < 1 || batch > ZDIT_MAX_BATCH || s_max < 1) return 0;
  return plan_block(*dims, batch, s_max).total;
}

zdit_status zdit_block_fwd(const zdit_dims* dims, const zdit_block_w* w, int32_t batch, int32_t s_max,
                           const int32_t* seq_len, float* x, const float* c, const float* rope_cos,
                           const float* rope_sin, void* ws, size_t ws_bytes, void* hip_stream) {
  if (zdit_status s = check_block_args(dims, w, batch, s_max, seq_len, x, c, rope_cos, rope_sin)) return s;
  if (!ws) return fail(ZDIT_EINVAL, "NULL pointer argument");
  if (((uintptr_t)ws & 255u) != 0) return fail(ZDIT_EINVAL, "workspace not 256-byte aligned");
  const size_t need = plan_block(*dims, batch, s_max).total;
  if (ws_bytes < need) return fail(ZDIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return run_block(*dims, *w, batch, s_max, seq_len, x, c, rope_cos, rope_sin, (char*)ws, (hipStream_t)hip_stream);
}

zdit_status zdit_block_fwd_noalloc(const zdit_dims* dims, const zdit_block_w* w, int32_t batch, int32_t s_max,
                                   const int32_t* seq_len, float* x, const float* c, const float* rope_cos,
                                   const float* rope_sin, void* hip_stream) {
  if (zdit_status s = check_block_args(dims, w, batch, s_max, seq_len, x, c, rope_cos, rope_sin)) return s;
  const size_t need = plan_block(*dims, batch, s_max).total;
  if (need > kNoAllocScratchBytes)
    return fail(ZDIT_EUNSUPPORTED, "this shape needs %zu bytes of scratch; zdit_block_fwd_noalloc holds %zu "
                "(use zdit_block_fwd with a workspace)", need, kNoAllocScratchBytes);
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(ZDIT_EUNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
      if (!p) return fail(ZDIT_EHIP, "hipGetSymbolAddress returned NULL for the scratch array");
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return run_block(*dims, *w, batch, s_max, seq_len, x, c, rope_cos, rope_sin, (char*)ws, (hipStream_t)hip_stream);
}

size_t zdit_stack_workspace(const zdit_model_cfg* cfg, int32_t batch, int32_t lat_h, int32_t lat_w,
                            int32_t max_cap_len) {
  if (check_cfg(cfg) || batch < 1 || batch > ZDIT_MAX_BATCH || lat_h < 2 || lat_w < 2 || max_cap_len < 1) return 0;
  return plan_stack(*cfg, batch, lat_h, lat_w, max_cap_len, nullptr).total;
}

zdit_status zdit_stack_fwd(const zdit_model_cfg* cfg, const zdit_model_w* w, int32_t batch, int32_t lat_h,
                           int32_t lat_w, const float* latents, int64_t latent_batch_stride,
                           const float* cap_feats, int32_t max_cap_len, const int32_t* cap_len,
                           const float* t, float* velocity, void* ws, size_t ws_bytes, void* hip_stream) {
  if (zdit_status s = check_stack_args(cfg, w, batch, lat_h, lat_w, latents, cap_feats, max_cap_len, cap_len, t, velocity))
    return s;
  if (latent_batch_stride < 0 || latent_batch_stride % 4) return fail(ZDIT_EINVAL, "latent_batch_stride %lld", (long long)latent_batch_stride);
  if (!ws || ((uintptr_t)ws & 255u)) return fail(ZDIT_EINVAL, "workspace NULL or not 256-byte aligned");
  const StackPlan pl = plan_stack(*cfg, batch, lat_h, lat_w, max_cap_len, nullptr);
  if (ws_bytes < pl.total) return fail(ZDIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, pl.total);
  hipStream_t st = (hipStream_t)hip_stream;
  const Check chk = check_at(cfg->d, (char*)ws + pl.chk, stack_checks(*cfg));
  HIP_TRY(check_begin(chk, st));
  if (zdit_status s = stack_forward(*cfg, *w, batch, lat_h, lat_w, latents, latent_batch_stride, cap_feats,
                                    max_cap_len, cap_len, t, velocity, (char*)ws, st, CapCache{}, chk, 0))
    return s;
  int step, where;
  if (zdit_status s = check_read(chk, st, &step, &where)) return s;
  if (where >= 0) return fail(ZDIT_ENONFINITE, "non-finite value in %s", stack_check_name(*cfg, where).c_str());
  return ok();
}

zdit_status zdit_sigmas(int32_t num_steps, float shift, float* out) {
  if (num_steps < 1 || num_steps > 1000) return fail(ZDIT_EINVAL, "num_steps %d (1..1000)", num_steps);
  if (!(shift > 0.f) || !isfinite(shift)) return fail(ZDIT_EINVAL, "shift must be finite and > 0");
  if (!out) return fail(ZDIT_EINVAL, "out is NULL");
  for (int i = 0; i <= num_steps; ++i) out[i] = (float)sigma_at(i, num_steps, (double)shift);
  return ok();
}

zdit_status zdit_n_cap(int32_t cap_len, int32_t multiple, int32_t* out) {
  if (cap_len < 1 || cap_len > 512) return fail(ZDIT_EINVAL, "cap_len %d (1..512)", cap_len);
  if (multiple < 1 || multiple > 512) return fail(ZDIT_EINVAL, "multiple %d (1..512)", multiple);
  if (!out) return fail(ZDIT_EINVAL, "out is NULL");
  *out = round_up(cap_len, multiple);
  return ok();
}

zdit_status zdit_euler_step(float* x, const float* v_cond, const float* v_uncond, int64_t n, float guidance,
                            float sigma, float sigma_next, float* decode_out, void* hip_stream) {
  if (n < 0) return fail(ZDIT_EINVAL, "n %lld < 0", (long long)n);
  if (!isfinite(guidance) || !isfinite(sigma) || !isfinite(sigma_next)) return fail(ZDIT_EINVAL, "non-finite scalar");
  if (!v_uncond && guidance != 0.f) return fail(ZDIT_EINVAL, "v_uncond is NULL but guidance != 0");
  if (n == 0) return ok();
  if (!x || !v_cond) return fail(ZDIT_EINVAL, "NULL pointer argument");
  HIP_TRY(launch_euler(x, v_cond, v_uncond, n, guidance, sigma, sigma_next, decode_out, (hipStream_t)hip_stream));
  return ok();
}

// Caption rows after the context refiners, kept across sampler steps: [nb][n_cap max][dim]
// fp32 (n_cap of any valid length is at most max_cap_len rounded up to the multiple).
static size_t sample_cap_cache_bytes(const zdit_model_cfg* cfg, int nb, int max_cap_len) {
  const int m = cfg->seq_multiple;
  const size_t nc = (size_t)((max_cap_len + m - 1) / m) * m;
  return al256((size_t)nb * nc * cfg->d.dim * 4);
}

size_t zdit_sample_workspace(const zdit_model_cfg* cfg, int32_t lat_h, int32_t lat_w, int32_t max_cap_len,
                             float guidance) {
  const int nb = guidance != 0.f ? 2 : 1;
  const size_t st = zdit_stack_workspace(cfg, nb, lat_h, lat_w, max_cap_len);
  if (!st) return 0;
  return st + al256((size_t)nb * cfg->latent_ch * lat_h * lat_w * 4) + sample_cap_cache_bytes(cfg, nb, max_cap_len);
}

zdit_status zdit_sample(const zdit_model_cfg* cfg, const zdit_model_w* w, int32_t lat_h, int32_t lat_w, float* x,
                        const float* cap_feats, int32_t max_cap_len, const int32_t* cap_len, float guidance,
                        int32_t num_steps, float shift, float* decode_out, void* ws, size_t ws_bytes,
                        void* hip_stream) {
  const int nb = guidance != 0.f ? 2 : 1;
  if (!isfinite(guidance)) return fail(ZDIT_EINVAL, "guidance not finite");
  if (num_steps < 1 || num_steps > 1000) return fail(ZDIT_EINVAL, "num_steps %d (1..1000)", num_steps);
  if (!(shift > 0.f) || !isfinite(shift)) return fail(ZDIT_EINVAL, "shift must be finite and > 0");
  float tt[2] = {0.5f, 0.5f};
  if (zdit_status s = check_stack_args(cfg, w, nb, lat_h, lat_w, x, cap_feats, max_cap_len, cap_len, tt, x)) return s;
  if (decode_out && !aligned16(decode_out)) return fail(ZDIT_EINVAL, "decode_out not 16-byte aligned");
  if (!ws || ((uintptr_t)ws & 255u)) return fail(ZDIT_EINVAL, "workspace NULL or not 256-byte aligned");
  const size_t need = zdit_sample_workspace(cfg, lat_h, lat_w, max_cap_len, guidance);
  if (ws_bytes < need) return fail(ZDIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t st = (hipStream_t)hip_stream;
  const int64_t n = (int64_t)cfg->latent_ch * lat_h * lat_w;
  float* vel = (float*)ws;
  float* cap_cache = (float*)((char*)ws + al256((size_t)nb * n * 4));
  char* sws = (char*)cap_cache + sample_cap_cache_bytes(cfg, nb, max_cap_len);
  std::vector<float> sg(num_steps + 1);
  for (int i = 0; i <= num_steps; ++i) sg[i] = (float)sigma_at(i, num_steps, (double)shift);
  // the stack's own check region inside its workspace; checkpoints latched per step
  const StackPlan spl = plan_stack(*cfg, nb, lat_h, lat_w, max_cap_len, nullptr);
  const Check chk = check_at(cfg->d, sws + spl.chk, stack_checks(*cfg));
  HIP_TRY(check_begin(chk, st));
  for (int i = 0; i < num_steps; ++i) {
    const float ti = 1.0f - sg[i];
    const float tv[2] = {ti, ti};
    // the caption rows do not depend on the step: context refiners run in step 0 only
    CapCache cc;
    if (i == 0) cc.out = cap_cache; else cc.in = cap_cache;
    if (zdit_status s = stack_forward(*cfg, *w, nb, lat_h, lat_w, x, 0, cap_feats, max_cap_len, cap_len, tv, vel,
                                      sws, st, cc, chk, i)) return s;
    HIP_TRY(launch_euler(x, vel, nb == 2 ? vel + n : nullptr, n, guidance, sg[i], sg[i + 1],
                         i == num_steps - 1 ? decode_out : nullptr, st));
  }
  int step, where;
  if (zdit_status s = check_read(chk, st, &step, &where)) return s;
  if (where >= 0)
    return fail(ZDIT_ENONFINITE, "sampler step %d: non-finite value in %s", step, stack_check_name(*cfg, where).c_str());
  return ok();
}

zdit_status zdit_rope_tables(int32_t kind, const int32_t rope_axes[3], float theta, int32_t batch, int32_t s_max,
                             int32_t grid_h, int32_t grid_w, const int32_t* n_cap, float* cos_out, float* sin_out,
                             void* hip_stream) {
  if (kind < ZDIT_SEQ_IMAGE || kind > ZDIT_SEQ_TEXT) return fail(ZDIT_EINVAL, "kind %d", kind);
  if (!rope_axes) return fail(ZDIT_EINVAL, "rope_axes NULL");
  for (int i = 0; i < 3; ++i)
    if (rope_axes[i] < 0 || rope_axes[i] % 2) return fail(ZDIT_EINVAL, "rope_axes[%d] = %d", i, rope_axes[i]);
  if (rope_axes[0] + rope_axes[1] + rope_axes[2] < 2) return fail(ZDIT_EINVAL, "rope axes sum < 2");
  if (!(theta > 0.f)) return fail(ZDIT_EINVAL, "theta must be > 0");
  if (batch < 1 || batch > ZDIT_MAX_BATCH || s_max < 1) return fail(ZDIT_EINVAL, "batch %d / s_max %d", batch, s_max);
  if (grid_h < 0 || grid_w < 0) return fail(ZDIT_EINVAL, "grid %d x %d", grid_h, grid_w);
  if (kind != ZDIT_SEQ_IMAGE && !n_cap) return fail(ZDIT_EINVAL, "n_cap NULL");
  if (!cos_out || !sin_out) return fail(ZDIT_EINVAL, "NULL output");
  RopeTabArgs rt;
  rt.cos = cos_out; rt.sin = sin_out; rt.kind = kind; rt.batch = batch; rt.s_max = s_max;
  rt.grid_h = grid_h; rt.grid_w = grid_w; rt.theta = theta;
  for (int i = 0; i < 3; ++i) rt.axes[i] = rope_axes[i];
  for (int b = 0; b < kMaxBatch; ++b) rt.n_cap[b] = (kind != ZDIT_SEQ_IMAGE && b < batch) ? n_cap[b] : 0;
  for (int b = 0; b < batch; ++b)
    if (kind != ZDIT_SEQ_IMAGE && n_cap[b] < 0) return fail(ZDIT_EINVAL, "n_cap[%d] < 0", b);
  HIP_TRY(launch_rope_tables(rt, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_gemm(int32_t precision, int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A,
                         const void* B, const void* B2, const float* vec, void* C, void* hip_stream) {
  if (precision != ZDIT_BF16 && precision != ZDIT_FP32_DEBUG) return fail(ZDIT_EINVAL, "precision %d", precision);
  if (epilogue < ZDIT_EPI_STORE || epilogue > ZDIT_EPI_SWIGLU) return fail(ZDIT_EINVAL, "epilogue %d", epilogue);
  if (M < 0 || N < 1 || K < 1) return fail(ZDIT_EINVAL, "M %d N %d K %d", M, N, K);
  if (M > (1 << 24)) return fail(ZDIT_EUNSUPPORTED, "M %d (at most 2^24 rows)", M);
  if (precision == ZDIT_BF16 && K % 64) return fail(ZDIT_EUNSUPPORTED, "K %d not a multiple of 64", K);
  if (K % 8) return fail(ZDIT_EUNSUPPORTED, "K %d not a multiple of 8", K);
  if (!A || !B || !C) return fail(ZDIT_EINVAL, "NULL operand");
  if (epilogue == ZDIT_EPI_SWIGLU && !B2) return fail(ZDIT_EINVAL, "B2 NULL for SwiGLU");
  if (epilogue == ZDIT_EPI_BIAS && !vec) return fail(ZDIT_EINVAL, "bias NULL");
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || (B2 && !aligned16(B2))) return fail(ZDIT_EINVAL, "operand not 16-byte aligned");
  GemmArgs g{};
  g.A = A; g.B = B; g.B2 = B2; g.C = C; g.vec = vec; g.vec_bstride = 0;
  g.M = M; g.N = N; g.K = K; g.lda = K; g.ldb = K;
  g.out = compact_rows(M, N);
  HIP_TRY(gemm(precision, epilogue, g, (hipStream_t)hip_stream));
  return ok();
}

size_t zdit_op_gemm_ksplit_workspace(int32_t epilogue, int32_t M, int32_t N, int32_t K) {
  if ((epilogue != ZDIT_EPI_STORE && epilogue != ZDIT_EPI_RESID && epilogue != ZDIT_EPI_SWIGLU) || M < 1 ||
      M > (1 << 24) || N < 8 || N % 8 || K < 64 || K % 64)
    return 0;
  return al256(tile_split_workspace(epilogue, M, N, K)) + 256;  // never 0 for an accepted shape
}

zdit_status zdit_op_gemm_ksplit(int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A, const void* B,
                                const void* B2, const float* vec, void* C, void* ws, size_t ws_bytes,
                                void* hip_stream) {
  if (epilogue != ZDIT_EPI_STORE && epilogue != ZDIT_EPI_RESID && epilogue != ZDIT_EPI_SWIGLU)
    return fail(ZDIT_EUNSUPPORTED, "epilogue %d (STORE, RESID or SWIGLU)", epilogue);
  if (M < 0 || N < 1 || K < 1) return fail(ZDIT_EINVAL, "M %d N %d K %d", M, N, K);
  if (M > (1 << 24) || N % 8 || K % 64) return fail(ZDIT_EUNSUPPORTED, "M %d / N %d / K %d", M, N, K);
  if (!A || !B || !C || (epilogue == ZDIT_EPI_SWIGLU && !B2)) return fail(ZDIT_EINVAL, "NULL operand");
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || (B2 && !aligned16(B2)) || (vec && !aligned16(vec)))
    return fail(ZDIT_EINVAL, "operand not 16-byte aligned");
  if (M == 0) return ok();
  if (!ws || !aligned16(ws) || ws_bytes < zdit_op_gemm_ksplit_workspace(epilogue, M, N, K))
    return fail(ZDIT_EWORKSPACE, "workspace too small");
  GemmArgs g{};
  g.A = A; g.B = B; g.B2 = B2; g.C = C; g.vec = vec; g.vec_bstride = 0;
  g.M = M; g.N = N; g.K = K; g.lda = K; g.ldb = K;
  g.out = compact_rows(M, N);
  HIP_TRY(launch_gemm_bf16_split(epilogue, g, (float*)ws, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_rmsnorm_mod(int32_t precision, int32_t rows, int32_t dim, const float* x, const float* gain,
                                const float* shift, const float* scale, float eps, void* out, void* hip_stream) {
  if (precision != ZDIT_BF16 && precision != ZDIT_FP32_DEBUG) return fail(ZDIT_EINVAL, "precision %d", precision);
  if (rows < 0 || dim < 128 || dim % 128 || dim > 4096) return fail(ZDIT_EUNSUPPORTED, "rows %d dim %d", rows, dim);
  if (!x || !gain || !out || (!shift) != (!scale)) return fail(ZDIT_EINVAL, "NULL pointer argument");
  if (!aligned16(x) || !aligned16(gain) || !aligned16(out) || (shift && (!aligned16(shift) || !aligned16(scale))))
    return fail(ZDIT_EINVAL, "pointer not 16-byte aligned");
  if (rows == 0) return ok();
  NormArgs na;
  na.x = x; na.x_bstride = 0; na.rows_per_batch = rows; na.batch = 1; na.dim = dim; na.gain = gain;
  na.shift = shift; na.scale = scale; na.mod_bstride = 0; na.eps = eps; na.out = out;
  for (int b = 0; b < kMaxBatch; ++b) na.valid[b] = rows;
  HIP_TRY(launch_rmsnorm_mod(precision, na, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_rope(int32_t precision, int32_t batch, int32_t s_max, int32_t n_heads, const int32_t* seq_len,
                         void* qkv, const float* cos, const float* sin, void* hip_stream) {
  if (precision != ZDIT_BF16 && precision != ZDIT_FP32_DEBUG) return fail(ZDIT_EINVAL, "precision %d", precision);
  if (batch < 1 || batch > ZDIT_MAX_BATCH || s_max < 1 || n_heads < 1) return fail(ZDIT_EINVAL, "batch/s_max/n_heads");
  if (!seq_len || !qkv || !cos || !sin) return fail(ZDIT_EINVAL, "NULL pointer argument");
  if (!aligned16(qkv) || !aligned16(cos) || !aligned16(sin)) return fail(ZDIT_EINVAL, "pointer not 16-byte aligned");
  RopeArgs ra;
  ra.qkv = qkv; ra.cos = cos; ra.sin = sin; ra.tab_bstride = (int64_t)s_max * 64;
  ra.batch = batch; ra.s_max = s_max; ra.n_heads = n_heads;
  for (int b = 0; b < kMaxBatch; ++b) ra.seq_len[b] = b < batch ? seq_len[b] : 0;
  for (int b = 0; b < batch; ++b)
    if (seq_len[b] < 0 || seq_len[b] > s_max) return fail(ZDIT_EINVAL, "seq_len[%d]", b);
  HIP_TRY(launch_rope(precision, ra, (hipStream_t)hip_stream));
  return ok();
}

size_t zdit_op_attn_workspace(int32_t precision, int32_t batch, int32_t s_max, int32_t n_heads) {
  return al256(attn_vt_bytes(precision, batch, s_max, n_heads)) + 256;
}

zdit_status zdit_op_attn(int32_t precision, int32_t batch, int32_t s_max, int32_t n_heads, const int32_t* seq_len,
                         const void* qkv, void* out, void* ws, size_t ws_bytes, void* hip_stream) {
  if (precision != ZDIT_BF16 && precision != ZDIT_FP32_DEBUG) return fail(ZDIT_EINVAL, "precision %d", precision);
  if (batch < 1 || batch > ZDIT_MAX_BATCH || s_max < 1 || n_heads < 1) return fail(ZDIT_EINVAL, "batch/s_max/n_heads");
  if (n_heads > 32 || !seq_fits(s_max, n_heads * kHeadDim)) return fail(ZDIT_EUNSUPPORTED, "s_max %d / n_heads %d too large", s_max, n_heads);
  if (!seq_len || !qkv || !out) return fail(ZDIT_EINVAL, "NULL pointer argument");
  for (int b = 0; b < batch; ++b)
    if (seq_len[b] < 1 || seq_len[b] > s_max) return fail(ZDIT_EINVAL, "seq_len[%d] = %d", b, seq_len[b]);
  if (ws_bytes < zdit_op_attn_workspace(precision, batch, s_max, n_heads) || (precision == ZDIT_BF16 && !ws))
    return fail(ZDIT_EWORKSPACE, "workspace too small");
  AttnArgs aa{};
  aa.qkv = qkv; aa.vt = ws; aa.out = out; aa.batch = batch; aa.s_max = s_max; aa.s_pad = round_up(s_max, 64);
  aa.n_heads = n_heads;
  for (int b = 0; b < kMaxBatch; ++b) aa.seq_len[b] = b < batch ? seq_len[b] : 0;
  HIP_TRY(launch_attn(precision, aa, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_qkv_attn(int32_t batch, int32_t s_max, int32_t n_heads, const int32_t* seq_len, const void* h,
                             const void* w_qkv, const float* cos, const float* sin, void* qkv, void* out, void* ws,
                             size_t ws_bytes, void* hip_stream) {
  if (batch < 1 || batch > ZDIT_MAX_BATCH || s_max < 1 || n_heads < 1) return fail(ZDIT_EINVAL, "batch/s_max/n_heads");
  if (s_max % 32) return fail(ZDIT_EUNSUPPORTED, "s_max %d not a multiple of 32", s_max);
  if (n_heads > 32 || !seq_fits(s_max, n_heads * kHeadDim) || (int64_t)batch * s_max > (1 << 24))
    return fail(ZDIT_EUNSUPPORTED, "s_max %d / n_heads %d too large", s_max, n_heads);
  if (!seq_len || !h || !w_qkv || !cos || !sin || !qkv || !out) return fail(ZDIT_EINVAL, "NULL pointer argument");
  if (!aligned16(h) || !aligned16(w_qkv) || !aligned16(cos) || !aligned16(sin) || !aligned16(qkv) || !aligned16(out))
    return fail(ZDIT_EINVAL, "pointer not 16-byte aligned");
  for (int b = 0; b < batch; ++b)
    if (seq_len[b] < 1 || seq_len[b] > s_max) return fail(ZDIT_EINVAL, "seq_len[%d] = %d", b, seq_len[b]);
  if (!ws || !aligned16(ws) || ws_bytes < zdit_op_attn_workspace(ZDIT_BF16, batch, s_max, n_heads))
    return fail(ZDIT_EWORKSPACE, "workspace too small");
  const zdit_status rc = qkv_attention(ZDIT_BF16, n_heads, batch, s_max, seq_len, h, w_qkv, qkv, ws, out, cos, sin,
                                       (int64_t)s_max * 64, (hipStream_t)hip_stream);
  return rc == ZDIT_OK ? ok() : rc;
}

zdit_status zdit_op_patchify(int32_t batch, int32_t C, int32_t h, int32_t w, const float* lat,
                             int64_t lat_batch_stride, float* tokens, void* hip_stream) {
  if (batch < 1 || C < 1 || h < 2 || w < 2 || h % 2 || w % 2) return fail(ZDIT_EINVAL, "shape");
  if (!lat || !tokens) return fail(ZDIT_EINVAL, "NULL pointer argument");
  HIP_TRY(launch_patchify(ZDIT_FP32_DEBUG, batch, C, h, w, lat, lat_batch_stride, tokens, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_unpatchify(int32_t batch, int32_t C, int32_t h, int32_t w, const float* tokens, float* lat,
                               void* hip_stream) {
  if (batch < 1 || C < 1 || h < 2 || w < 2 || h % 2 || w % 2) return fail(ZDIT_EINVAL, "shape");
  if (!lat || !tokens) return fail(ZDIT_EINVAL, "NULL pointer argument");
  HIP_TRY(launch_unpatchify(batch, C, h, w, tokens, lat, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_cap_pad(int32_t batch, int32_t s_max, int32_t dim, int32_t row0, const int32_t* cap_len,
                            const float* cap_pad, float* x, void* hip_stream) {
  if (batch < 1 || batch > ZDIT_MAX_BATCH || s_max < 1 || dim < 1 || row0 < 0) return fail(ZDIT_EINVAL, "shape");
  if (!cap_len || !cap_pad || !x) return fail(ZDIT_EINVAL, "NULL pointer argument");
  for (int b = 0; b < batch; ++b) {
    if (cap_len[b] < 1 || cap_len[b] > 512) return fail(ZDIT_EINVAL, "cap_len[%d] = %d", b, cap_len[b]);
    if (row0 + round_up(cap_len[b], 32) > s_max) return fail(ZDIT_EINVAL, "padded caption of branch %d exceeds s_max", b);
  }
  HIP_TRY(launch_cap_pad(batch, s_max, dim, row0, cap_len, 32, cap_pad, x, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_temb(int32_t batch, const float* t, int32_t t_freq, int32_t c_dim, float t_scale,
                         const float* w1, const float* b1, const float* w2, const float* b2, float* c_out,
                         void* hip_stream) {
  if (batch < 1 || batch > ZDIT_MAX_BATCH) return fail(ZDIT_EINVAL, "batch %d", batch);
  if (t_freq < 2 || t_freq % 2 || t_freq > 1024 || c_dim < 1 || c_dim > 1024) return fail(ZDIT_EUNSUPPORTED, "t_freq / c_dim");
  if (!t || !w1 || !b1 || !w2 || !b2 || !c_out) return fail(ZDIT_EINVAL, "NULL pointer argument");
  HIP_TRY(launch_temb(batch, t, t_freq, c_dim, t_scale, w1, b1, w2, b2, c_out, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_adaln(int32_t precision, int32_t batch, int32_t c_dim, int32_t n_out, const float* c,
                          const void* w, const float* b, float* out, void* hip_stream) {
  if (precision != ZDIT_BF16 && precision != ZDIT_FP32_DEBUG) return fail(ZDIT_EINVAL, "precision %d", precision);
  if (batch < 1 || batch > ZDIT_MAX_BATCH || c_dim < 8 || c_dim % 8 || c_dim > 1024 || n_out < 1)
    return fail(ZDIT_EINVAL, "batch / c_dim / n_out");
  if (!c || !w || !b || !out) return fail(ZDIT_EINVAL, "NULL pointer argument");
  if (!aligned16(c) || !aligned16(w) || !aligned16(b) || !aligned16(out))
    return fail(ZDIT_EINVAL, "pointer not 16-byte aligned");
  HIP_TRY(launch_adaln(precision, batch, c_dim, n_out, c, w, b, out, (hipStream_t)hip_stream));
  return ok();
}

}  // extern "C"
