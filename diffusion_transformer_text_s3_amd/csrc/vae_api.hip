// C ABI of the 16-channel AutoencoderKL decoder (Core AI model zoo, "Z-Image-Turbo port",
// table "Architecture -> export mapping", row VAE): argument validation, workspace planning
// and the launch sequence.  Every argument is checked before the first launch; on error
// nothing is enqueued.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <utility>

#include "api_util.h"
#include "vae.h"

using namespace zdit;

namespace {

constexpr int kVaeMaxLat = 256;  // latent side (a 2048-pixel image side)

bool pow2_width(int c) { return c >= 32 && c <= 1024 && (c & (c - 1)) == 0; }

zdit_status check_vae_cfg(const zdit_vae_cfg* c) {
  if (!c) return fail(ZDIT_EINVAL, "cfg is NULL");
  if (c->latent_ch < 4 || c->latent_ch % 4) return fail(ZDIT_EUNSUPPORTED, "latent_ch %d (a multiple of 4)", c->latent_ch);
  if (c->out_ch < 1 || c->out_ch > 4) return fail(ZDIT_EUNSUPPORTED, "out_ch %d (1..4)", c->out_ch);
  if (c->groups < 1) return fail(ZDIT_EINVAL, "groups %d", c->groups);
  for (int i = 0; i < 4; ++i) {
    if (!pow2_width(c->widths[i]))
      return fail(ZDIT_EUNSUPPORTED, "widths[%d] = %d (a power of two in 32..1024)", i, c->widths[i]);
    if (c->widths[i] % c->groups) return fail(ZDIT_EINVAL, "widths[%d] = %d not a multiple of groups %d", i, c->widths[i], c->groups);
  }
  if (c->resnets < 1 || c->resnets > 8) return fail(ZDIT_EUNSUPPORTED, "resnets %d (1..8)", c->resnets);
  if (!(c->eps >= 0.f) || !isfinite(c->eps)) return fail(ZDIT_EINVAL, "eps must be finite and >= 0");
  if (!(c->scale != 0.f) || !isfinite(c->scale) || !isfinite(c->shift)) return fail(ZDIT_EINVAL, "scale must be finite and nonzero, shift finite");
  if (c->flags & ~ZDIT_VAE_INPUT_UNSCALED) return fail(ZDIT_EINVAL, "unknown flags 0x%x", c->flags);
  return ZDIT_OK;
}

zdit_status check_shape(int batch, int lat_h, int lat_w) {
  if (batch < 1 || batch > ZDIT_MAX_BATCH) return fail(ZDIT_EINVAL, "batch %d (1..%d)", batch, ZDIT_MAX_BATCH);
  if (lat_h < 2 || lat_w < 2 || lat_h % 2 || lat_w % 2 || lat_h > kVaeMaxLat || lat_w > kVaeMaxLat)
    return fail(ZDIT_EUNSUPPORTED, "latent %d x %d (even, 2..%d)", lat_h, lat_w, kVaeMaxLat);
  return ZDIT_OK;
}

bool ok_ptr(const void* p) { return p && aligned16(p); }

// Workspace regions (byte offsets): the NHWC latent, three activation buffers of the largest
// stage, GroupNorm partials, the half-tile statistics the convolutions write, statistics and
// affines, and the attention's q/k/v, v^T and scores (gp_bytes 0: no half-tile statistics).
struct VaePlan {
  size_t lat, X, H, T, part, gp, gp_bytes, gc, stat, aff, qkv, vt, S, total;
};

int dec_width(const zdit_vae_cfg& c, int i) { return c.widths[3 - i]; }

VaePlan plan_vae(const zdit_vae_cfg& c, int B, int h, int w) {
  VaePlan p;
  const int64_t n0 = (int64_t)h * w;
  int64_t act = (int64_t)B * n0 * dec_width(c, 0);
  size_t part = vgn_part_floats(B, (int)n0, dec_width(c, 0));
  int64_t res = n0;
  int cin = dec_width(c, 0);
  for (int i = 0; i < 4; ++i) {
    const int co = dec_width(c, i);
    act = std::max(act, (int64_t)B * res * std::max(cin, co));
    part = std::max(part, vgn_part_floats(B, (int)res, cin));
    part = std::max(part, vgn_part_floats(B, (int)res, co));
    if (i < 3) {
      res *= 4;
      act = std::max(act, (int64_t)B * res * co);
    }
    cin = co;
  }
  part = std::max(part, vgn_part_floats(B, (int)res, cin));
  const int C = dec_width(c, 0);
  size_t off = 0;
  p.lat = off; off += al256((size_t)B * n0 * c.latent_ch * 4);
  p.X = off; off += al256((size_t)act * 4);
  p.H = off; off += al256((size_t)act * 4);
  p.T = off; off += al256((size_t)act * 4);
  p.part = off; off += al256(part * 4);
  // half tiles of 64 rows: at most act / 64 + one partial half per image, per channel
  p.gp_bytes = al256(((size_t)act / 64 + (size_t)B * 1024) * 8);
  p.gp = off; off += p.gp_bytes;
  // their first-level merges: per image, chunk of 16 half tiles (1024 rows) and group
  p.gc = off; off += al256(((size_t)act / 1024 + (size_t)B * c.groups) * 3 * 8);
  p.stat = off; off += al256((size_t)B * c.groups * 2 * 8);
  p.aff = off; off += al256((size_t)B * 1024 * 2 * 4);
  p.qkv = off; off += al256((size_t)B * n0 * 3 * C * 4);
  p.vt = off; off += al256((size_t)n0 * C * 4);
  p.S = off; off += al256((size_t)n0 * n0 * 4);
  p.total = off;
  return p;
}

// One launcher context: the workspace regions and the stream.  gp_valid: the half-tile
// statistics region holds those of the last output written by a convolution with stats on.
struct Ctx {
  const zdit_vae_cfg& c;
  char* ws;
  const VaePlan& pl;
  int B;
  hipStream_t st;
  mutable bool gp_valid = false;
  float* f(size_t off) const { return (float*)(ws + off); }
};

// stats: the output is GroupNorm's next input; the direct-to-LDS form then writes its half-tile
// statistics and gnorm uses them.  They are used only where H W is a multiple of 128, where every
// batch size runs the direct form: the choice then depends on the image size alone, so a batch
// item's statistics, and its image, are bit-identical to those of the same image decoded alone
// (the direct and staged forms give the same bits, the two GroupNorm paths do not).
hipError_t conv(const Ctx& x, const float* in, int H, int W, int cin, int cout, int ksize, int up, const float* aff,
                int silu, const zdit_vae_conv& cw, const float* res, float* out, int out_nchw = 0, bool stats = false) {
  VConvArgs a{};
  a.out_nchw = out_nchw;
  a.A = in; a.lda = cin;
  a.B = cw.w; a.ldb = (int64_t)ksize * ksize * cin;
  a.C = out; a.ldc = cout;
  a.res = res; a.bias = cw.b; a.affine = aff; a.silu = silu;
  a.M = x.B * H * W; a.N = cout; a.K = cin; a.H = H; a.W = W;
  a.ksize = ksize; a.upsample = up; a.alpha = 1.f;
  if (stats) {
    const size_t need = ((size_t)(a.M + 63) / 64 + x.B) * cout * 8;
    x.gp_valid = (int64_t)H * W % 128 == 0 && x.pl.gp_bytes >= need && vconv_direct_ok(a);
    if (x.gp_valid) a.gn_part = (float2*)(x.ws + x.pl.gp);
  }
  return launch_vconv(a, x.st);
}

hipError_t gnorm(const Ctx& x, const float* in, int hw, int C, const zdit_vae_norm& n) {
  VGnArgs a{};
  a.x = in; a.images = x.B; a.HW = hw; a.C = C; a.groups = x.c.groups;
  a.part = x.f(x.pl.part); a.stat = (double*)(x.ws + x.pl.stat);
  a.gamma = n.gamma; a.beta = n.beta; a.affine = x.f(x.pl.aff); a.eps = x.c.eps;
  if (x.gp_valid) {
    x.gp_valid = false;
    return launch_vgn_from_conv((const float2*)(x.ws + x.pl.gp), (double*)(x.ws + x.pl.gc), a, x.st);
  }
  return launch_vgn(a, x.st);
}

// x (in *X) -> *X, through H and (width change) T; swaps the buffers it leaves the result in.
// Each convolution's input SiLU(GroupNorm(.)) is written once (launch_vact) and read by the
// direct-to-LDS convolution: conv1's into T (free until the shortcut is written there), conv2's
// over H in place.
hipError_t resnet(const Ctx& x, float*& X, float*& Hb, float*& T, int H, int W, int cin, int cout,
                  const zdit_vae_resnet& r) {
  const int hw = H * W;
  float* aff = x.f(x.pl.aff);
  if (hipError_t e = gnorm(x, X, hw, cin, r.gn1)) return e;
  if (hipError_t e = launch_vact(X, aff, x.B, hw, cin, 1, T, x.st)) return e;
  if (hipError_t e = conv(x, T, H, W, cin, cout, 3, 0, nullptr, 0, r.conv1, nullptr, Hb, 0, true)) return e;
  if (hipError_t e = gnorm(x, Hb, hw, cout, r.gn2)) return e;
  if (hipError_t e = launch_vact(Hb, aff, x.B, hw, cout, 1, Hb, x.st)) return e;
  if (r.shortcut.w) {
    if (hipError_t e = conv(x, X, H, W, cin, cout, 1, 0, nullptr, 0, r.shortcut, nullptr, T)) return e;
    if (hipError_t e = conv(x, Hb, H, W, cout, cout, 3, 0, nullptr, 0, r.conv2, T, T, 0, true)) return e;
    std::swap(X, T);
    return hipSuccess;
  }
  return conv(x, Hb, H, W, cout, cout, 3, 0, nullptr, 0, r.conv2, X, X, 0, true);
}

hipError_t attention(const Ctx& x, float* X, float* Hb, int H, int W, int C, const zdit_vae_attn& at) {
  const int N = H * W;
  float* qkv = x.f(x.pl.qkv);
  float* vt = x.f(x.pl.vt);
  float* S = x.f(x.pl.S);
  // GroupNorm(x) into H (free until P v is written there), then the q/k/v map
  if (hipError_t e = gnorm(x, X, N, C, at.gn)) return e;
  if (hipError_t e = launch_vact(X, x.f(x.pl.aff), x.B, N, C, 0, Hb, x.st)) return e;
  if (hipError_t e = conv(x, Hb, H, W, C, 3 * C, 1, 0, nullptr, 0, at.qkv, nullptr, qkv)) return e;
  for (int b = 0; b < x.B; ++b) {
    const float* qb = qkv + (int64_t)b * N * 3 * C;
    VConvArgs s{};
    s.A = qb; s.lda = 3 * C;
    s.B = qb + C; s.ldb = 3 * C;
    s.C = S; s.ldc = N;
    s.M = N; s.N = N; s.K = C; s.H = 1; s.W = N; s.ksize = 1;
    s.alpha = 1.0f / sqrtf((float)C);
    if (hipError_t e = launch_vconv(s, x.st)) return e;
    if (hipError_t e = launch_vsoftmax(S, N, N, x.st)) return e;
    if (hipError_t e = launch_vtranspose(qb, 3 * C, 2 * C, vt, N, C, x.st)) return e;
    VConvArgs o{};
    o.A = S; o.lda = N;
    o.B = vt; o.ldb = N;
    o.C = Hb + (int64_t)b * N * C; o.ldc = C;
    o.M = N; o.N = C; o.K = N; o.H = 1; o.W = N; o.ksize = 1; o.alpha = 1.f;
    if (hipError_t e = launch_vconv(o, x.st)) return e;
  }
  return conv(x, Hb, H, W, C, C, 1, 0, nullptr, 0, at.out, X, X, 0, true);
}

zdit_status check_conv_w(const zdit_vae_conv& c, const char* what) {
  if (!ok_ptr(c.w) || !c.b) return fail(ZDIT_EINVAL, "%s: weight NULL or not 16-byte aligned, or bias NULL", what);
  return ZDIT_OK;
}

zdit_status check_norm(const zdit_vae_norm& n, const char* what) {
  if (!n.gamma || !n.beta) return fail(ZDIT_EINVAL, "%s: gamma or beta NULL", what);
  return ZDIT_OK;
}

zdit_status check_resnet(const zdit_vae_resnet& r, int cin, int cout, const char* what) {
  if (zdit_status s = check_norm(r.gn1, what)) return s;
  if (zdit_status s = check_norm(r.gn2, what)) return s;
  if (zdit_status s = check_conv_w(r.conv1, what)) return s;
  if (zdit_status s = check_conv_w(r.conv2, what)) return s;
  if ((cin != cout) != (r.shortcut.w != nullptr))
    return fail(ZDIT_EINVAL, "%s: the 1x1 shortcut is required exactly when the widths differ (%d -> %d)", what, cin, cout);
  if (r.shortcut.w) return check_conv_w(r.shortcut, what);
  return ZDIT_OK;
}

zdit_status check_vae_w(const zdit_vae_cfg& c, const zdit_vae_w* w) {
  if (!w) return fail(ZDIT_EINVAL, "weights NULL");
  const int c0 = dec_width(c, 0);
  if (zdit_status s = check_conv_w(w->conv_in, "conv_in")) return s;
  for (int i = 0; i < 2; ++i)
    if (zdit_status s = check_resnet(w->mid[i], c0, c0, "mid resnet")) return s;
  if (zdit_status s = check_norm(w->attn.gn, "attention norm")) return s;
  if (zdit_status s = check_conv_w(w->attn.qkv, "attention qkv")) return s;
  if (zdit_status s = check_conv_w(w->attn.out, "attention out")) return s;
  int cin = c0;
  for (int i = 0; i < 4; ++i) {
    if (!w->stages[i]) return fail(ZDIT_EINVAL, "stages[%d] NULL", i);
    const int co = dec_width(c, i);
    for (int j = 0; j < c.resnets; ++j)
      if (zdit_status s = check_resnet(w->stages[i][j], j ? co : cin, co, "stage resnet")) return s;
    if (i < 3)
      if (zdit_status s = check_conv_w(w->upconv[i], "upsample conv")) return s;
    cin = co;
  }
  if (zdit_status s = check_norm(w->norm_out, "norm_out")) return s;
  return check_conv_w(w->conv_out, "conv_out");
}

}  // namespace

extern "C" {

size_t zdit_vae_workspace(const zdit_vae_cfg* cfg, int32_t batch, int32_t lat_h, int32_t lat_w) {
  if (check_vae_cfg(cfg) || check_shape(batch, lat_h, lat_w)) return 0;
  return plan_vae(*cfg, batch, lat_h, lat_w).total;
}

zdit_status zdit_vae_decode(const zdit_vae_cfg* cfg, const zdit_vae_w* w, int32_t batch, int32_t lat_h, int32_t lat_w,
                            const float* latent, float* image, void* ws, size_t ws_bytes, void* hip_stream) {
  if (zdit_status s = check_vae_cfg(cfg)) return s;
  if (zdit_status s = check_shape(batch, lat_h, lat_w)) return s;
  if (zdit_status s = check_vae_w(*cfg, w)) return s;
  if (!latent || !image) return fail(ZDIT_EINVAL, "latent or image NULL");
  if (!ok_ptr(ws)) return fail(ZDIT_EINVAL, "workspace NULL or not 16-byte aligned");
  const zdit_vae_cfg& c = *cfg;
  const VaePlan pl = plan_vae(c, batch, lat_h, lat_w);
  if (ws_bytes < pl.total) return fail(ZDIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, pl.total);
  const int cl = c.widths[0];
  hipStream_t st = (hipStream_t)hip_stream;
  char* wsb = (char*)ws;
  Ctx x{c, wsb, pl, batch, st};
  float* X = x.f(pl.X);
  float* Hb = x.f(pl.H);
  float* T = x.f(pl.T);
  int H = lat_h, W = lat_w;
  const int c0 = dec_width(c, 0);
  HIP_TRY(launch_vlatent_in(latent, x.f(pl.lat), batch, c.latent_ch, H, W, !(c.flags & ZDIT_VAE_INPUT_UNSCALED),
                            c.scale, c.shift, st));
  HIP_TRY(conv(x, x.f(pl.lat), H, W, c.latent_ch, c0, 3, 0, nullptr, 0, w->conv_in, nullptr, X, 0, true));
  HIP_TRY(resnet(x, X, Hb, T, H, W, c0, c0, w->mid[0]));
  HIP_TRY(attention(x, X, Hb, H, W, c0, w->attn));
  HIP_TRY(resnet(x, X, Hb, T, H, W, c0, c0, w->mid[1]));
  int cin = c0;
  for (int i = 0; i < 4; ++i) {
    const int co = dec_width(c, i);
    for (int j = 0; j < c.resnets; ++j) HIP_TRY(resnet(x, X, Hb, T, H, W, j ? co : cin, co, w->stages[i][j]));
    if (i < 3) {
      H *= 2;
      W *= 2;
      HIP_TRY(conv(x, X, H, W, co, co, 3, 1, nullptr, 0, w->upconv[i], nullptr, T, 0, true));
      std::swap(X, T);
    }
    cin = co;
  }
  HIP_TRY(gnorm(x, X, H * W, cl, w->norm_out));
  HIP_TRY(launch_vact(X, x.f(pl.aff), batch, (int64_t)H * W, cl, 1, T, st));
  HIP_TRY(conv(x, T, H, W, cl, c.out_ch, 3, 0, nullptr, 0, w->conv_out, nullptr, image, 1));
  return ok();
}

// ------------------------------------------------------------------ single steps (tests)
size_t zdit_op_vae_groupnorm_workspace(int32_t batch, int32_t hw, int32_t C, int32_t groups) {
  if (batch < 1 || hw < 1 || !pow2_width(C) || groups < 1 || C % groups) return 0;
  return al256(vgn_part_floats(batch, hw, C) * 4) + al256((size_t)batch * groups * 16);
}

zdit_status zdit_op_vae_groupnorm(int32_t batch, int32_t hw, int32_t C, int32_t groups, float eps, const float* x,
                                  const float* gamma, const float* beta, float* affine, void* ws, size_t ws_bytes,
                                  void* hip_stream) {
  if (batch < 1 || batch > ZDIT_MAX_BATCH || hw < 1) return fail(ZDIT_EINVAL, "batch %d / hw %d", batch, hw);
  if (!pow2_width(C)) return fail(ZDIT_EUNSUPPORTED, "C %d (a power of two in 32..1024)", C);
  if (groups < 1 || C % groups) return fail(ZDIT_EINVAL, "groups %d must divide C %d", groups, C);
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(ZDIT_EINVAL, "eps must be finite and >= 0");
  if (!ok_ptr(x) || !gamma || !beta || !affine || !ok_ptr(ws)) return fail(ZDIT_EINVAL, "NULL or misaligned pointer");
  const size_t need = zdit_op_vae_groupnorm_workspace(batch, hw, C, groups);
  if (ws_bytes < need) return fail(ZDIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  VGnArgs a{};
  a.x = x; a.images = batch; a.HW = hw; a.C = C; a.groups = groups;
  a.part = (float*)ws;
  a.stat = (double*)((char*)ws + al256(vgn_part_floats(batch, hw, C) * 4));
  a.gamma = gamma; a.beta = beta; a.affine = affine; a.eps = eps;
  HIP_TRY(launch_vgn(a, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_vae_conv(int32_t batch, int32_t H, int32_t W, int32_t cin, int32_t cout, int32_t ksize,
                             int32_t upsample, const float* x, const float* affine, int32_t silu, const float* w,
                             const float* b, const float* res, float* out, void* hip_stream) {
  if (batch < 1 || H < 1 || W < 1) return fail(ZDIT_EINVAL, "batch %d, H %d, W %d", batch, H, W);
  if ((int64_t)batch * H * W > INT32_MAX / 2) return fail(ZDIT_EUNSUPPORTED, "too many pixels");
  if (ksize != 1 && ksize != 3) return fail(ZDIT_EUNSUPPORTED, "ksize %d (1 or 3)", ksize);
  if (upsample && (H % 2 || W % 2)) return fail(ZDIT_EINVAL, "upsample needs even output sides (%d x %d)", H, W);
  if (cin < 4 || cin % 4 || cout < 1) return fail(ZDIT_EUNSUPPORTED, "cin %d (a multiple of 4), cout %d", cin, cout);
  if (!ok_ptr(x) || !ok_ptr(w) || !out || (affine && !aligned16(affine)))
    return fail(ZDIT_EINVAL, "NULL or misaligned pointer");
  VConvArgs a{};
  a.A = x; a.lda = cin;
  a.B = w; a.ldb = (int64_t)ksize * ksize * cin;
  a.C = out; a.ldc = cout;
  a.res = res; a.bias = b; a.affine = affine; a.silu = silu ? 1 : 0;
  a.M = batch * H * W; a.N = cout; a.K = cin; a.H = H; a.W = W;
  a.ksize = ksize; a.upsample = upsample ? 1 : 0; a.alpha = 1.f;
  HIP_TRY(launch_vconv(a, (hipStream_t)hip_stream));
  return ok();
}

zdit_status zdit_op_vae_conv_out(int32_t batch, int32_t H, int32_t W, int32_t cin, int32_t cout, const float* x,
                                 const float* affine, const float* w, const float* b, float* image, void* hip_stream) {
  if (batch < 1 || batch > ZDIT_MAX_BATCH || H < 1 || W < 1) return fail(ZDIT_EINVAL, "batch %d, H %d, W %d", batch, H, W);
  if ((int64_t)batch * H * W > INT32_MAX / 2) return fail(ZDIT_EUNSUPPORTED, "too many pixels");
  if (cin < 4 || cin % 4 || cout < 1 || cout > 4) return fail(ZDIT_EUNSUPPORTED, "cin %d (a multiple of 4), cout %d (1..4)", cin, cout);
  if (!ok_ptr(x) || !ok_ptr(affine) || !ok_ptr(w) || !b || !image) return fail(ZDIT_EINVAL, "NULL or misaligned pointer");
  VConvArgs a{};
  a.A = x; a.lda = cin;
  a.B = w; a.ldb = (int64_t)9 * cin;
  a.C = image; a.out_nchw = 1;
  a.bias = b; a.affine = affine; a.silu = 1;
  a.M = batch * H * W; a.N = cout; a.K = cin; a.H = H; a.W = W;
  a.ksize = 3; a.alpha = 1.f;
  HIP_TRY(launch_vconv(a, (hipStream_t)hip_stream));
  return ok();
}

size_t zdit_op_vae_attention_workspace(int32_t batch, int32_t hw, int32_t C, int32_t groups) {
  if (batch < 1 || hw < 1 || hw % 4 || !pow2_width(C) || groups < 1 || C % groups) return 0;
  const size_t n = hw;
  return al256(vgn_part_floats(batch, hw, C) * 4) + al256((size_t)batch * groups * 16) +
         al256((size_t)batch * C * 8) + al256(batch * n * 3 * C * 4) + al256(n * C * 4) + al256(n * n * 4) +
         al256(batch * n * C * 4);
}

zdit_status zdit_op_vae_attention(int32_t batch, int32_t H, int32_t W, int32_t C, int32_t groups, float eps,
                                  const zdit_vae_attn* at, float* x, void* ws, size_t ws_bytes, void* hip_stream) {
  if (batch < 1 || batch > ZDIT_MAX_BATCH || H < 1 || W < 1 || (H * W) % 4)
    return fail(ZDIT_EINVAL, "batch %d, H %d, W %d (H * W a multiple of 4)", batch, H, W);
  if ((int64_t)H * W > 65536) return fail(ZDIT_EUNSUPPORTED, "more than 65536 positions");
  if (!pow2_width(C)) return fail(ZDIT_EUNSUPPORTED, "C %d (a power of two in 32..1024)", C);
  if (groups < 1 || C % groups) return fail(ZDIT_EINVAL, "groups %d must divide C %d", groups, C);
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(ZDIT_EINVAL, "eps must be finite and >= 0");
  if (!at) return fail(ZDIT_EINVAL, "weights NULL");
  if (zdit_status s = check_norm(at->gn, "attention norm")) return s;
  if (zdit_status s = check_conv_w(at->qkv, "attention qkv")) return s;
  if (zdit_status s = check_conv_w(at->out, "attention out")) return s;
  if (!ok_ptr(x) || !ok_ptr(ws)) return fail(ZDIT_EINVAL, "NULL or misaligned pointer");
  const size_t need = zdit_op_vae_attention_workspace(batch, H * W, C, groups);
  if (ws_bytes < need) return fail(ZDIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  // a plan over the caller's workspace with only the regions attention uses
  zdit_vae_cfg c{};
  c.groups = groups;
  c.eps = eps;
  const size_t n = (size_t)H * W;
  VaePlan pl{};
  size_t off = 0;
  pl.part = off; off += al256(vgn_part_floats(batch, H * W, C) * 4);
  pl.stat = off; off += al256((size_t)batch * groups * 16);
  pl.aff = off; off += al256((size_t)batch * C * 8);
  pl.qkv = off; off += al256(batch * n * 3 * C * 4);
  pl.vt = off; off += al256(n * C * 4);
  pl.S = off; off += al256(n * n * 4);
  pl.H = off;
  Ctx cx{c, (char*)ws, pl, batch, (hipStream_t)hip_stream};
  HIP_TRY(attention(cx, x, cx.f(pl.H), H, W, C, *at));
  return ok();
}

}  // extern "C"
