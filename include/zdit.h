/*
 * zdit.h - C ABI of the MI355X (gfx950) S3-DiT hot path: the Z-Image-Turbo single-stream
 * diffusion transformer block, its 2 + 2 + 30 block stack and the 8-step negated-CFG
 * FlowMatchEuler sampler.
 *
 * Also the text encoder that produces its caption features (a Qwen3-shaped causal decoder
 * read out at its penultimate hidden state), with random weights.
 *
 * Sources (web pages; cited by title and section):
 *   [CoreAI]  Core AI model zoo, "Z-Image-Turbo port - a 6B diffusion DiT on Core AI, and
 *             why it is Mac-only".
 *   [Status]  FastVideo, tests/local_tests/zimage "Z-Image Port Status".
 *   [Jobs]    1Cat-vLLM "Native creative jobs", section "Recipes and precision".
 *
 * Conventions for every call:
 *   - Device pointers are HIP device addresses; host pointers are ordinary memory.  The
 *     caller owns every buffer (weights, activations, workspace).  Pointers are borrowed for
 *     the call and must stay valid until the enqueued work completes.  The library allocates
 *     no device memory and keeps no pointer after returning (zdit_block_fwd_noalloc works in
 *     a fixed scratch array the library's code object holds on each device).
 *   - All device work is enqueued on `hip_stream` (a hipStream_t; NULL = default stream).
 *     Nothing synchronises; no host<->device copy is made, except that the text-encoder
 *     calls with more than 512 tokens (batch * max_len) copy the host token ids into their
 *     workspace (up to 512 they travel in the kernel arguments; either way the host array may
 *     be reused as soon as the call returns), and that calls with ZDIT_CHECK_FINITE set read
 *     their verdict back (see below).
 *   - Arguments are validated before anything is enqueued.  On error nothing runs, outputs
 *     are untouched, the return value is negative and zdit_last_error() says why.  Faults
 *     during execution surface at the caller's next synchronisation, as in any HIP library.
 *   - Matrices are row-major.  Linear weights are [out, in] (the `in` index contiguous).
 *     In ZDIT_BF16 precision, weight matrices are bf16 and activations between kernels are
 *     bf16 (GEMM operands) or fp32 (residual stream, norms, modulation, softmax).  In
 *     ZDIT_FP32_DEBUG precision every weight and activation is fp32.
 *   - Device pointers must be 16-byte aligned; leading dimensions are the dense ones implied
 *     by the shapes given.
 */
#ifndef ZDIT_H
#define ZDIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t zdit_status;
enum {
  ZDIT_OK = 0,
  ZDIT_EINVAL = -1,        /* bad argument (null/misaligned pointer, bad size, bad length) */
  ZDIT_EUNSUPPORTED = -2,  /* dimensions the kernels do not implement */
  ZDIT_EWORKSPACE = -3,    /* workspace smaller than the matching *_workspace() query */
  ZDIT_EHIP = -4,          /* a HIP launch failed */
  ZDIT_ENONFINITE = -5     /* ZDIT_CHECK_FINITE found a NaN or an infinity (see below) */
};

enum { ZDIT_BF16 = 0, ZDIT_FP32_DEBUG = 1 };

/* Token-sequence layouts for RoPE tables (ZDIT_SEQ_TEXT: the text encoder's tokens). */
enum { ZDIT_SEQ_IMAGE = 0, ZDIT_SEQ_CAPTION = 1, ZDIT_SEQ_JOINT = 2, ZDIT_SEQ_TEXT = 3 };

/* zdit_dims.flags.  ZDIT_CHECK_FINITE (debug): zdit_block_fwd, zdit_stack_fwd and zdit_sample
 * scan their inputs, the residual stream after every block and the velocity of every step for
 * NaN and infinity, and return ZDIT_ENONFINITE naming the first place one appeared (sampler step,
 * input or block) in zdit_last_error().  The activations of this model outgrow half precision,
 * and an fp16 run of the DiT turns to NaN by the second sampler step ([CoreAI] "fp16 does not
 * work. bf16 does.").  With the flag set these calls read the verdict back and synchronise the
 * stream before returning (so they cannot be captured into a graph); the numeric results are
 * the same as without it.  Unknown flag bits are ZDIT_EINVAL. */
#define ZDIT_CHECK_FINITE 1

#define ZDIT_MAX_BATCH 16
#define ZDIT_ABI_VERSION 2

/* Text of the last error on the calling thread; valid until the next zdit_* call on it. */
const char* zdit_last_error(void);
int32_t zdit_abi_version(void);

/* Block dimensions.  The kernels implement head_dim 128, rope axes summing to head_dim
 * (each even), dim = n_heads * head_dim with dim % 128 == 0, ffn_hidden % 128 == 0,
 * c_dim % 64 == 0 and c_dim <= 1024.  norm_eps is the RMSNorm epsilon.  flags: 0 or
 * ZDIT_CHECK_FINITE. */
typedef struct {
  int32_t dim, n_heads, head_dim, ffn_hidden;
  int32_t rope_axes[3];
  int32_t c_dim;
  int32_t precision; /* ZDIT_BF16 or ZDIT_FP32_DEBUG */
  float norm_eps;
  int32_t flags;
} zdit_dims;

/* One block's weights (device).  w_qkv [3*dim, dim]: rows 0..dim-1 produce q, dim..2dim-1
 * k, 2dim..3dim-1 v; heads are contiguous head_dim-wide slices.  w_out [dim, dim];
 * w1, w3 [ffn_hidden, dim]; w2 [dim, ffn_hidden]; norm1, norm2 fp32 [dim].  w_ada
 * [6*dim, c_dim] and b_ada fp32 [6*dim] give (shift1, scale1, gate1, shift2, scale2,
 * gate2); both NULL for a block without adaLN (shift = scale = 0, gate = 1). */
typedef struct {
  const void *w_qkv, *w_out, *w1, *w3, *w2;
  const float *norm1, *norm2;
  const void* w_ada;
  const float* b_ada;
} zdit_block_w;

/* ---------------------------------------------------------------------------------------
 * S3-DiT block forward ([CoreAI] table "Architecture -> export mapping", row DiT: adaLN,
 * 3-axis RoPE in the real interleaved cos/sin form, joint attention over one sequence):
 *   (shift1, scale1, gate1, shift2, scale2, gate2) = W_ada SiLU(c) + b_ada
 *   h  = RMSNorm(x; norm1) (1 + scale1) + shift1
 *   q, k, v = split(h W_qkv^T); q, k rotated by RoPE(cos, sin)
 *   x += gate1 * (softmax(q k^T / sqrt(head_dim)) v) W_out^T      (keys j < seq_len[b])
 *   h2 = RMSNorm(x; norm2) (1 + scale2) + shift2
 *   x += gate2 * ((SiLU(h2 W1^T) * (h2 W3^T)) W2^T)
 * Rows j >= seq_len[b] of x are padding: masked as keys and left untouched.
 *
 *   batch        1..ZDIT_MAX_BATCH rows (branches) of x
 *   s_max        rows per branch in x (>= every seq_len; s_max * 6 * dim <= 2^31 - 1)
 *   seq_len      host [batch], each in 1..s_max: valid rows of branch b
 *   x            device fp32 [batch, s_max, dim], in/out (the residual stream)
 *   c            device fp32 [batch, c_dim] conditioning vector; ignored when w_ada NULL
 *   rope_cos/sin device fp32 [batch, s_max, head_dim/2] (see zdit_rope_tables)
 *   ws           device workspace of at least zdit_block_workspace() bytes, 256-aligned
 * ------------------------------------------------------------------------------------- */
size_t zdit_block_workspace(const zdit_dims* dims, int32_t batch, int32_t s_max);
zdit_status zdit_block_fwd(const zdit_dims* dims, const zdit_block_w* w, int32_t batch,
                           int32_t s_max, const int32_t* seq_len, float* x, const float* c,
                           const float* rope_cos, const float* rope_sin, void* ws,
                           size_t ws_bytes, void* hip_stream);

/* zdit_block_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, hosts that forbid allocation): the same computation and results, with
 * the workspace replaced by a scratch array the library holds on each device (128 MiB, placed
 * when the library's code loads on that device and kept until the process ends).  Calls
 * zdit_block_fwd would accept whose zdit_block_workspace() exceeds 128 MiB return
 * ZDIT_EUNSUPPORTED (a 256 px branch, the 256 px pair and the 512 px pair fit; a pair of
 * 448-row branches, whose K-split GEMMs keep ~110 MB of partial products, and the 1024^2 pair
 * need a workspace).  All
 * calls on one device share its scratch: calls that overlap on one device (other streams,
 * other threads) race and must be ordered by the caller.  No allocation, no free, no host
 * copy (except the ZDIT_CHECK_FINITE read-back). */
zdit_status zdit_block_fwd_noalloc(const zdit_dims* dims, const zdit_block_w* w, int32_t batch,
                                   int32_t s_max, const int32_t* seq_len, float* x,
                                   const float* c, const float* rope_cos, const float* rope_sin,
                                   void* hip_stream);

/* Whole-model configuration.  n_noise_ref adaLN blocks on image tokens, n_ctx_ref blocks
 * without adaLN on caption tokens, n_main adaLN blocks on the joint sequence ([CoreAI]
 * "Architecture -> export mapping", row DiT: 2 + 2 + 30).  latent_ch 16, patch 2 (the
 * kernels implement exactly these), cap_dim the caption feature width, t_freq the
 * timestep-embedding width (== c_dim), seq_multiple the caption padding multiple (32),
 * max_cap_len the caption length limit (512), rope_theta the RoPE base, t_scale the
 * factor applied to model time before the sinusoid (1000). */
typedef struct {
  zdit_dims d;
  int32_t n_noise_ref, n_ctx_ref, n_main;
  int32_t latent_ch, patch, cap_dim, t_freq, seq_multiple, max_cap_len;
  float rope_theta, t_scale;
} zdit_model_cfg;

/* Whole-model weights (device pointers; the three block arrays are HOST arrays of
 * zdit_block_w).  x_emb_w [dim, patch*patch*latent_ch], cap_emb_w [dim, cap_dim] (bf16 or
 * fp32 by precision), biases fp32 [dim]; cap_pad fp32 [dim] (the learned caption pad);
 * t_w1 fp32 [c_dim, t_freq], t_b1 [c_dim], t_w2 fp32 [c_dim, c_dim], t_b2 [c_dim];
 * final_norm fp32 [dim]; final_ada_w [2*dim, c_dim] (shift then scale), final_ada_b fp32
 * [2*dim]; final_w [patch*patch*latent_ch, dim], final_b fp32 [patch*patch*latent_ch]. */
typedef struct {
  const void* x_emb_w;
  const float* x_emb_b;
  const void* cap_emb_w;
  const float* cap_emb_b;
  const float* cap_pad;
  const float *t_w1, *t_b1, *t_w2, *t_b2;
  const zdit_block_w *noise_ref, *ctx_ref, *main;
  const float* final_norm;
  const void* final_ada_w;
  const float* final_ada_b;
  const void* final_w;
  const float* final_b;
} zdit_model_w;

/* ---------------------------------------------------------------------------------------
 * DiT stack forward for `batch` branches ([CoreAI] "Architecture -> export mapping": x-embed
 * + cap-embed, noise refiners, context refiners, main blocks, final layer; host patchify,
 * RoPE, pad-mask and unpatchify done here on the device).  Each branch b:
 *   tokens  = patchify(latent_b) (feature f = (dy*2 + dx)*16 + ch, [CoreAI] "Three more
 *             things"); x_img = tokens W_x^T + b_x
 *   caption = cap_feats_b[0..L_b) W_cap^T + b_cap, then rows L_b..n_cap_b-1 set to cap_pad,
 *             n_cap_b = round_up(L_b, 32) ([CoreAI] "The three things that each cost a
 *             wrong image", item 3: pads are attention context, not masked)
 *   c       = W2 SiLU(W1 [cos(1000 t f_k), sin(1000 t f_k)] + b1) + b2
 *   noise refiners on x_img, context refiners on the caption, main blocks on the
 *   sequence (image tokens, then caption tokens), final layer, unpatchify.
 *
 *   latents       device fp32 [batch, latent_ch, lat_h, lat_w] with branch stride
 *                 latent_batch_stride floats (0: one latent shared by every branch)
 *   cap_feats     device fp32 [batch, max_cap_len, cap_dim]
 *   cap_len       host [batch], each in 1..min(max_cap_len, cfg->max_cap_len)
 *   t             host [batch] model time (1 - sigma for the sampler)
 *   velocity      device fp32 [batch, latent_ch, lat_h, lat_w], written
 *   lat_h, lat_w  even, >= 2
 * With latent_batch_stride 0 and the same t for every branch, the image tokens through the
 * noise refiners are the same in every branch: they are computed once and copied (the result
 * is bit-identical to computing each branch).
 * ------------------------------------------------------------------------------------- */
size_t zdit_stack_workspace(const zdit_model_cfg* cfg, int32_t batch, int32_t lat_h,
                            int32_t lat_w, int32_t max_cap_len);
zdit_status zdit_stack_fwd(const zdit_model_cfg* cfg, const zdit_model_w* w, int32_t batch,
                           int32_t lat_h, int32_t lat_w, const float* latents,
                           int64_t latent_batch_stride, const float* cap_feats,
                           int32_t max_cap_len, const int32_t* cap_len, const float* t,
                           float* velocity, void* ws, size_t ws_bytes, void* hip_stream);

/* Shifted FlowMatchEuler sigmas, host only: out[i] = shift (1 - i/n) / (shift (1 - i/n) +
 * i/n) for i = 0..num_steps, computed in double and stored fp32; out[0] = 1 and
 * out[num_steps] = 0 exactly ([CoreAI] "Three more things": closed form with t = i/(n-1)
 * over n = num_steps + 1 points; [Status] scheduler_contract: endpoint-preserving
 * num_steps + 1 schedule, sigma_min 0).  out: host [num_steps + 1]; num_steps 1..1000,
 * shift > 0. */
zdit_status zdit_sigmas(int32_t num_steps, float shift, float* out);

/* Padded caption length round_up(cap_len, multiple) ([CoreAI] "The three things...", item
 * 3).  cap_len 1..512, multiple 1..512.  Host only. */
zdit_status zdit_n_cap(int32_t cap_len, int32_t multiple, int32_t* out);

/* One negated-CFG Euler update, fp32, each product and sum rounded separately:
 *   d = v_cond - v_uncond; e = guidance * d; u = v_cond + e; np = -u   ([CoreAI] "The three
 *   things...", item 2: noise_pred = -(pos + g (pos - neg)))
 *   x = x + (sigma_next - sigma) * np
 *   decode_out = x / 0.3611 + 0.1159 when decode_out != NULL ([Status] decode_contract;
 *   x itself stays raw, so the unscale is applied exactly once)
 * v_uncond NULL means a single branch (np = -v_cond) and requires guidance == 0.
 * x, v_cond, v_uncond, decode_out: device fp32 [n]; n >= 0 (0 is a no-op). */
zdit_status zdit_euler_step(float* x, const float* v_cond, const float* v_uncond, int64_t n,
                            float guidance, float sigma, float sigma_next, float* decode_out,
                            void* hip_stream);

/* ---------------------------------------------------------------------------------------
 * The full sampler: num_steps negated-CFG FlowMatchEuler updates ([Status]
 * scheduler_contract: no DiT call at the final zero sigma; [CoreAI] "Architecture -> export
 * mapping", row Sampler: FlowMatchEuler, 8 steps, guidance 1.0, host loop).  Step i runs
 * the stack on the cond branch (and the uncond branch when guidance != 0) at model time
 * 1 - sigma_i on the shared latent x, then zdit_euler_step from sigma_i to sigma_{i+1}.
 *   x            device fp32 [latent_ch, lat_h, lat_w]: the initial noise in, the raw final
 *                latent out
 *   cap_feats    device fp32 [nb, max_cap_len, cap_dim], branch 0 cond, branch 1 uncond
 *                (nb = 2 when guidance != 0, else 1)
 *   cap_len      host [nb]
 *   decode_out   NULL or device fp32 [latent_ch, lat_h, lat_w]: final latent unscaled once
 * The caption rows after the context refiners depend on neither the latent nor t: they are
 * computed in the first step, kept in the workspace and reused in every later step (the
 * result is bit-identical to running the full stack each step).
 * ------------------------------------------------------------------------------------- */
size_t zdit_sample_workspace(const zdit_model_cfg* cfg, int32_t lat_h, int32_t lat_w,
                             int32_t max_cap_len, float guidance);
zdit_status zdit_sample(const zdit_model_cfg* cfg, const zdit_model_w* w, int32_t lat_h,
                        int32_t lat_w, float* x, const float* cap_feats, int32_t max_cap_len,
                        const int32_t* cap_len, float guidance, int32_t num_steps,
                        float shift, float* decode_out, void* ws, size_t ws_bytes,
                        void* hip_stream);

/* RoPE cos/sin tables for one of the three sequence layouts, fp32 [batch, s_max,
 * head_dim/2], computed on the device in double and rounded to fp32 ([CoreAI]
 * "Architecture -> export mapping", row DiT: precomputed cos/sin; [Status] issue I006:
 * RoPE buffers stay fp32).  Positions: image token (r, c) of a grid_h x grid_w grid ->
 * (0, r, c) in row-major order; caption token j -> (1 + j, 0, 0); ZDIT_SEQ_JOINT is the
 * image tokens followed by n_cap[b] caption tokens; ZDIT_SEQ_TEXT token j -> (j, 0, 0) for
 * j < n_cap[b] (the text encoder, with rope_axes {128, 0, 0}).  Column k enumerates rotation pairs:
 * axis 0's rope_axes[0]/2 pairs, then axis 1's, then axis 2's; pair p of axis a turns by
 * pos_a * theta^(-2p / rope_axes[a]).  Rows past a branch's length get cos 1, sin 0.
 * n_cap: host [batch] (ignored for ZDIT_SEQ_IMAGE).  cos_out, sin_out: device. */
zdit_status zdit_rope_tables(int32_t kind, const int32_t rope_axes[3], float theta,
                             int32_t batch, int32_t s_max, int32_t grid_h, int32_t grid_w,
                             const int32_t* n_cap, float* cos_out, float* sin_out,
                             void* hip_stream);

/* ---------------------------------------------------------------------------------------
 * Single-kernel entry points, for tests and measurement.  They run exactly the kernels the
 * block and stack use.
 * ------------------------------------------------------------------------------------- */

/* GEMM epilogues: C = A B^T with A [M, K], B [N, K] (K % 64 == 0 in ZDIT_BF16).
 *   ZDIT_EPI_STORE   C [M, N] activation type (bf16 / fp32) = A B^T
 *   ZDIT_EPI_BIAS    C [M, N] fp32 = A B^T + vec[n]
 *   ZDIT_EPI_RESID   C [M, N] fp32 += vec[n] * (A B^T)   (vec NULL: gate 1)
 *   ZDIT_EPI_SWIGLU  C [M, N] activation type = SiLU(A B^T) * (A B2^T), B and B2 [N, K] */
enum { ZDIT_EPI_STORE = 0, ZDIT_EPI_BIAS = 1, ZDIT_EPI_RESID = 2, ZDIT_EPI_SWIGLU = 3 };
zdit_status zdit_op_gemm(int32_t precision, int32_t epilogue, int32_t M, int32_t N, int32_t K,
                         const void* A, const void* B, const void* B2, const float* vec,
                         void* C, void* hip_stream);

/* The same contraction split over K, as the block runs its GEMMs for branches of at most 512
 * rows (bf16 only; epilogues ZDIT_EPI_STORE, ZDIT_EPI_RESID, ZDIT_EPI_SWIGLU): K is cut into
 * ranges chosen from N and K alone, the 256 x 256-tile kernel writes each range's fp32 partial
 * product to the workspace, and a second kernel sums the ranges in order and applies the
 * epilogue, so a row's result does not depend on M (a plan of one range runs the whole-K
 * kernel with the epilogue, as zdit_op_gemm).  K % 64 == 0, N % 8 == 0; ws:
 * zdit_op_gemm_ksplit_workspace() bytes (0 for a shape or epilogue this form rejects). */
size_t zdit_op_gemm_ksplit_workspace(int32_t epilogue, int32_t M, int32_t N, int32_t K);
zdit_status zdit_op_gemm_ksplit(int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A,
                                const void* B, const void* B2, const float* vec, void* C, void* ws,
                                size_t ws_bytes, void* hip_stream);

/* RMSNorm + modulation: out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * gain * (1 + scale) +
 * shift over `rows` rows of `dim`; x fp32, gain/shift/scale fp32 [dim] (shift/scale NULL:
 * 0); out activation type. */
zdit_status zdit_op_rmsnorm_mod(int32_t precision, int32_t rows, int32_t dim, const float* x,
                                const float* gain, const float* shift, const float* scale,
                                float eps, void* out, void* hip_stream);

/* RoPE on the q and k parts of a fused qkv buffer [batch, s_max, 3 * n_heads * 128]
 * (activation type), in place, with tables [batch, s_max, 64]; rows >= seq_len[b] are not
 * touched.  Bit-exact contract: y0 = x0 c - x1 s, y1 = x0 s + x1 c in fp32, each product
 * and sum rounded, then rounded to the activation type (bf16 ties-to-even). */
zdit_status zdit_op_rope(int32_t precision, int32_t batch, int32_t s_max, int32_t n_heads,
                         const int32_t* seq_len, void* qkv, const float* cos, const float* sin,
                         void* hip_stream);

/* Joint attention on a fused, already rotated qkv buffer [batch, s_max, 3 * n_heads * 128]
 * -> out [batch, s_max, n_heads * 128] (activation type); keys j >= seq_len[b] masked; rows
 * >= seq_len[b] of out are written as 0.  ws: zdit_op_attn_workspace() bytes.  n_heads
 * 1..32, s_max * 6 * n_heads * 128 <= 2^31 - 1 (else ZDIT_EUNSUPPORTED). */
size_t zdit_op_attn_workspace(int32_t precision, int32_t batch, int32_t s_max, int32_t n_heads);
zdit_status zdit_op_attn(int32_t precision, int32_t batch, int32_t s_max, int32_t n_heads,
                         const int32_t* seq_len, const void* qkv, void* out, void* ws,
                         size_t ws_bytes, void* hip_stream);

/* The block's attention half in its fused bf16 form: qkv = h W_qkv^T with q and k rotated by
 * RoPE (rows < seq_len[b]; tables [batch, s_max, 64]) in the projection's epilogue, V
 * transposed by that epilogue into the workspace, then joint attention into out [batch,
 * s_max, n_heads * 128] as zdit_op_attn.  h bf16 [batch * s_max, n_heads * 128], w_qkv bf16
 * [3 * n_heads * 128, n_heads * 128]; the v columns of qkv [batch, s_max, 3 * n_heads * 128]
 * are not written.  s_max % 32 == 0 (else ZDIT_EUNSUPPORTED); ws: zdit_op_attn_workspace(
 * ZDIT_BF16, ...) bytes, 16-byte aligned.  Bit-identical to zdit_op_gemm (ZDIT_EPI_STORE) +
 * zdit_op_rope + zdit_op_attn on the same inputs. */
zdit_status zdit_op_qkv_attn(int32_t batch, int32_t s_max, int32_t n_heads, const int32_t* seq_len,
                             const void* h, const void* w_qkv, const float* cos, const float* sin,
                             void* qkv, void* out, void* ws, size_t ws_bytes, void* hip_stream);

/* Patchify latents [batch, C, h, w] (branch stride lat_batch_stride floats) into fp32 tokens
 * [batch, (h/2)(w/2), 4C], token r*(w/2)+c, feature (dy*2 + dx)*C + ch. */
zdit_status zdit_op_patchify(int32_t batch, int32_t C, int32_t h, int32_t w, const float* lat,
                             int64_t lat_batch_stride, float* tokens, void* hip_stream);
/* Inverse: fp32 tokens [batch, (h/2)(w/2), 4C] -> latents [batch, C, h, w]. */
zdit_status zdit_op_unpatchify(int32_t batch, int32_t C, int32_t h, int32_t w,
                               const float* tokens, float* lat, void* hip_stream);

/* Learned caption pad: for branch b, rows row0 + j of x [batch, s_max, dim] (fp32) with
 * cap_len[b] <= j < round_up(cap_len[b], 32) are set to cap_pad [dim]; other rows untouched. */
zdit_status zdit_op_cap_pad(int32_t batch, int32_t s_max, int32_t dim, int32_t row0,
                            const int32_t* cap_len, const float* cap_pad, float* x,
                            void* hip_stream);

/* Timestep conditioning c [batch, c_dim] = W2 SiLU(W1 e + b1) + b2 with e = [cos(t_scale t
 * f_k), sin(t_scale t f_k)], f_k = 10000^(-k / (t_freq/2)); t host [batch]; fp32 weights. */
zdit_status zdit_op_temb(int32_t batch, const float* t, int32_t t_freq, int32_t c_dim,
                         float t_scale, const float* w1, const float* b1, const float* w2,
                         const float* b2, float* c_out, void* hip_stream);

/* adaLN projection out [batch, n_out] fp32 = W SiLU(c) + b, W [n_out, c_dim] (bf16 or fp32
 * by precision), b fp32 [n_out], c fp32 [batch, c_dim]. */
zdit_status zdit_op_adaln(int32_t precision, int32_t batch, int32_t c_dim, int32_t n_out,
                          const float* c, const void* w, const float* b, float* out,
                          void* hip_stream);

/* ---------------------------------------------------------------------------------------
 * Text encoder: the Qwen3-shaped causal decoder whose penultimate hidden state the DiT
 * reads as caption features ([Status] "Current Phase" summary: 36 decoder blocks, hidden
 * 2560, intermediate 9728, 32 attention heads, 8 KV heads, head dimension 128; component
 * matrix, row Production text encoder: hidden_states[-2]; [CoreAI] "Architecture -> export
 * mapping", row Text encoder: causal, additive causal and non-padding mask over right-padded
 * ids, embed_tokens inside the graph, bf16 weights with an fp32 boundary).  Block (the
 * published Qwen3 decoder; not spelled out on the pages):
 *   h = RMSNorm(x; in_norm); [q | k | v] = h W_qkv^T (n_heads query heads, n_kv_heads key
 *   and value heads of 128); q, k per head: RMSNorm over the 128 dims (q_norm / k_norm
 *   gains), then RoPE turning dims (i, i + 64) by pos * rope_theta^(-2i/128), pos = token
 *   index from 0; causal attention, query head h reading key/value head
 *   h / (n_heads / n_kv_heads), scale 1/sqrt(128); x += o W_o^T;
 *   h2 = RMSNorm(x; post_norm); x += (SiLU(h2 W_gate^T) * (h2 W_up^T)) W_down^T.
 * Residual stream fp32, GEMM operands bf16, accumulation fp32, norms in fp32.
 * ------------------------------------------------------------------------------------- */
typedef struct {
  int32_t n_layers;    /* blocks of the model (36); the output is taken after n_layers - 1 */
  int32_t hidden;      /* 2560; multiple of 128, <= 4096 */
  int32_t inter;       /* 9728; multiple of 128 */
  int32_t n_heads;     /* 32 query heads */
  int32_t n_kv_heads;  /* 8; divides n_heads */
  int32_t head_dim;    /* 128 (the only value implemented) */
  int32_t vocab;       /* embedding rows */
  float rope_theta;    /* 1e6 */
  float norm_eps;      /* 1e-6 */
  int32_t flags;       /* 0, or ZDIT_ENC_PACKED_WEIGHTS; any other bit: ZDIT_EINVAL */
} zdit_enc_cfg;

/* zdit_enc_cfg.flags.  ZDIT_ENC_PACKED_WEIGHTS: w_qkv, w_o, w_gate, w_up and w_down are in the
 * layout of zdit_op_pack_weights (same bytes, reordered), which the projections stream as 1 KB
 * runs instead of 64-byte pieces of 16 rows (the forward on two 64-id rows at the pinned widths:
 * 2.8 against 3.2 ms).  Only
 * the split-K path reads that layout: with the flag, batch * max_len must be <= 256
 * (ZDIT_EUNSUPPORTED otherwise).  The result is bit-identical to the row-major weights'. */
enum { ZDIT_ENC_PACKED_WEIGHTS = 1 };

typedef struct {
  const float* in_norm;    /* fp32 [hidden] */
  const void* w_qkv;       /* bf16 [(n_heads + 2 n_kv_heads) * 128, hidden]: q heads, k heads, v heads */
  const float* q_norm;     /* fp32 [128] */
  const float* k_norm;     /* fp32 [128] */
  const void* w_o;         /* bf16 [hidden, n_heads * 128] */
  const float* post_norm;  /* fp32 [hidden] */
  const void* w_gate;      /* bf16 [inter, hidden] */
  const void* w_up;        /* bf16 [inter, hidden] */
  const void* w_down;      /* bf16 [hidden, inter] */
} zdit_enc_layer_w;

typedef struct {
  const void* embed;               /* bf16 [vocab, hidden] */
  const zdit_enc_layer_w* layers;  /* host array of n_layers - 1 blocks (the last block does
                                      not enter hidden_states[-2] and is not read) */
} zdit_enc_w;

/* hidden_states[-2] of `batch` right-padded id rows: the residual stream after the first
 * n_layers - 1 blocks, fp32 [batch, max_len, hidden].  Row r of branch b is computed for
 * r < len[b] and is 0 for r >= len[b] (padding keys are masked, so valid rows do not depend
 * on max_len).
 *   ids        host int32 [batch, max_len]; ids[b][r] in [0, vocab) for r < len[b] (others
 *              not read)
 *   len        host [batch], each in 1..max_len
 *   hidden_out device fp32 [batch, max_len, hidden], written (it also holds the residual
 *              stream while the blocks run)
 *   batch 1..ZDIT_MAX_BATCH; max_len >= 1; ws: zdit_encoder_workspace() bytes. */
size_t zdit_encoder_workspace(const zdit_enc_cfg* cfg, int32_t batch, int32_t max_len);
zdit_status zdit_encoder_fwd(const zdit_enc_cfg* cfg, const zdit_enc_w* w, int32_t batch,
                             int32_t max_len, const int32_t* ids, const int32_t* len,
                             float* hidden_out, void* ws, size_t ws_bytes, void* hip_stream);

/* Encoder kernels alone (tests and measurement). */
/* Split-K GEMM for few rows, as the encoder's projections run when batch * max_len <= 256:
 * C = A B^T with A bf16 [M, K], B (and B2) bf16 [N, K]; epilogues ZDIT_EPI_STORE (C bf16),
 * ZDIT_EPI_RESID (C fp32 += vec[n] * (A B^T), vec NULL: gate 1) and ZDIT_EPI_SWIGLU (C bf16
 * = SiLU(A B^T) * (A B2^T)).  K is cut into ranges by N and K alone, each range's fp32
 * partial product goes to the workspace, and the partials are summed in range order, so a
 * row's result does not depend on M (SwiGLU over a single range applies SiLU and the product
 * in the GEMM itself, with the same arithmetic).  M 1..256, N % 8 == 0, K % 64 == 0 (else
 * ZDIT_EUNSUPPORTED); ws: zdit_op_gemm_splitk_workspace() bytes, which is 0 for a shape or
 * epilogue the GEMM rejects. */
size_t zdit_op_gemm_splitk_workspace(int32_t epilogue, int32_t M, int32_t N, int32_t K);
zdit_status zdit_op_gemm_splitk(int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A,
                                const void* B, const void* B2, const float* vec, void* C,
                                void* ws, size_t ws_bytes, void* hip_stream);
/* The same with B (and B2) packed by zdit_op_pack_weights; N % 16 == 0 as well.  Only the
 * weights' addresses differ: same sums in the same order, bit-identical results. */
zdit_status zdit_op_gemm_splitk_packed(int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A,
                                       const void* B, const void* B2, const float* vec, void* C,
                                       void* ws, size_t ws_bytes, void* hip_stream);

/* Packs a bf16 weight matrix src [N, K] (row-major, device) into dst (device, N K 2 bytes, not
 * overlapping src; both 16-byte aligned): bands of 16 rows, each a run of K / 32 slabs of 32
 * columns, each slab 64 chunks of 16 bytes, chunk l of slab t of band b holding columns
 * 32 t + 8 (l / 16) .. + 7 of row 16 b + l % 16 (the B operand of a 16 x 16 x 32 bf16 MFMA), so
 * a wavefront reads a slab of its band as 1 KB in a row.  N % 16 == 0, K % 32 == 0, at most
 * 2 GiB (else ZDIT_EUNSUPPORTED); enqueued on the stream. */
zdit_status zdit_op_pack_weights(int32_t N, int32_t K, const void* src, void* dst, void* hip_stream);

/* Embedding gather: out [batch, max_len, dim] fp32 = rows of table (bf16 [vocab, dim]) for
 * r < len[b], 0 after; ids / len host as in zdit_encoder_fwd; dim % 8 == 0; ws:
 * zdit_op_embed_workspace() bytes (the ids are copied there). */
size_t zdit_op_embed_workspace(int32_t batch, int32_t max_len);
zdit_status zdit_op_embed(int32_t batch, int32_t max_len, int32_t dim, int32_t vocab,
                          const int32_t* ids, const int32_t* len, const void* table, float* out,
                          void* ws, size_t ws_bytes, void* hip_stream);

/* Per-head RMSNorm + RoPE on the q and k heads of a bf16 qkv buffer [batch, s_max,
 * (n_heads + 2 n_kv_heads) * 128] in place, rows r < seq_len[b] (others untouched): each
 * 128-dim head y = x / sqrt(mean(x^2) + eps) * g (g = q_norm for query heads, k_norm for
 * key heads) in fp32, then y_i' = y_i c_i - y_{i+64} s_i, y_{i+64}' = y_{i+64} c_i + y_i s_i
 * with the row's fp32 tables cos/sin [batch, s_max, 64] (each product and sum rounded), then
 * rounded to bf16. */
zdit_status zdit_op_qknorm_rope(int32_t batch, int32_t s_max, int32_t n_heads, int32_t n_kv_heads,
                                const int32_t* seq_len, void* qkv, const float* q_norm,
                                const float* k_norm, const float* cos, const float* sin,
                                float eps, void* hip_stream);

/* Attention with grouped key/value heads and an optional causal mask on a rotated qkv buffer
 * [batch, s_max, (n_heads + 2 n_kv_heads) * 128] (q heads, k heads, v heads) -> out [batch,
 * s_max, n_heads * 128] (activation type).  Query head h reads key/value head
 * h / (n_heads / n_kv_heads); keys j >= seq_len[b] masked, and with causal != 0 keys j > i
 * for query i; rows >= seq_len[b] of out written as 0.  n_heads 1..64, n_kv_heads divides
 * n_heads, s_max * (n_heads + 2 n_kv_heads) * 256 <= 2^31 - 1 (else ZDIT_EUNSUPPORTED); ws:
 * zdit_op_attn_gqa_workspace() bytes.  With n_kv_heads == n_heads and causal == 0 this is
 * zdit_op_attn. */
size_t zdit_op_attn_gqa_workspace(int32_t precision, int32_t batch, int32_t s_max, int32_t n_kv_heads);
zdit_status zdit_op_attn_gqa(int32_t precision, int32_t batch, int32_t s_max, int32_t n_heads,
                             int32_t n_kv_heads, int32_t causal, const int32_t* seq_len,
                             const void* qkv, void* out, void* ws, size_t ws_bytes,
                             void* hip_stream);

/* ---------------------------------------------------------------------------------------
 * VAE decoder: the 16-channel AutoencoderKL decoder that turns the sampler's final latent
 * into the image ([CoreAI] "Architecture -> export mapping", row VAE: fp32, nearest-neighbour
 * upsampling, the unscale z / 0.3611 + 0.1159 built into the decoder, which is fed the raw
 * latent; [Status] component matrix, row VAE: the raw decode is the component boundary).
 * Architecture (the published 16-channel autoencoder with those constants; not spelled out
 * on the pages), widths in decoder order c0..c3 = widths[3], widths[2], widths[1], widths[0]:
 *   x = conv_in(z / scale + shift)                      3x3, latent_ch -> c0
 *   x = resnet(x); x = attention(x); x = resnet(x)      c0
 *   stage i = 0..3: `resnets` ResNet blocks to width ci (the first from c(i-1), c0 for
 *   stage 0); for i < 3 then x = conv(upsample2x_nearest(x)), 3x3, ci -> ci
 *   image = conv_out(SiLU(GroupNorm(x)))                3x3, c3 -> out_ch
 *   ResNet: h = conv1(SiLU(GN1(x))); h = conv2(SiLU(GN2(h))); out = s(x) + h with s the
 *     identity, or a 1x1 conv when the width changes.
 *   Attention: h = GN(x); [q | k | v] = per-position linear maps of h; out = x + (softmax(
 *     q k^T / sqrt(C)) v) W_o^T + b_o, one head over all positions of an image.
 *   GroupNorm: `groups` groups of consecutive channels, statistics over the group and all
 *     positions of one image, biased variance, eps; then a per-channel gain and shift.
 *   Convolutions: cross-correlation, zero padding (k - 1) / 2, stride 1, with biases.
 * All arithmetic fp32 (GroupNorm statistics accumulated in float64).  Activations inside
 * are NHWC; the latent is NCHW [batch, latent_ch, lat_h, lat_w], the image NCHW [batch,
 * out_ch, 8 lat_h, 8 lat_w].
 * ------------------------------------------------------------------------------------- */
#define ZDIT_VAE_INPUT_UNSCALED 1 /* cfg.flags: the latent is already unscaled (the sampler's
                                     decode_out); the decoder then skips z / scale + shift */

typedef struct {
  int32_t latent_ch; /* 16; a multiple of 4 */
  int32_t out_ch;    /* 3; 1..4 */
  int32_t widths[4]; /* encoder-order widths (128, 256, 512, 512): powers of two in 32..1024,
                        each a multiple of groups */
  int32_t resnets;   /* ResNet blocks per decoder stage (3); 1..8 */
  int32_t groups;    /* 32 */
  float eps;         /* 1e-6 */
  float scale;       /* 0.3611 */
  float shift;       /* 0.1159 */
  int32_t flags;     /* 0 or ZDIT_VAE_INPUT_UNSCALED */
} zdit_vae_cfg;

/* conv weights fp32 [cout][k][k][cin] (input channels innermost, 16-byte aligned), bias fp32
 * [cout]; norm gain and shift fp32 [C] */
typedef struct { const float* w; const float* b; } zdit_vae_conv;
typedef struct { const float* gamma; const float* beta; } zdit_vae_norm;
typedef struct {
  zdit_vae_norm gn1;
  zdit_vae_conv conv1;    /* 3x3, cin -> cout */
  zdit_vae_norm gn2;
  zdit_vae_conv conv2;    /* 3x3, cout -> cout */
  zdit_vae_conv shortcut; /* 1x1, cin -> cout; w NULL exactly when cin == cout */
} zdit_vae_resnet;
typedef struct {
  zdit_vae_norm gn;
  zdit_vae_conv qkv; /* w [3C][1][1][C]: the q rows, then k, then v; b [3C] */
  zdit_vae_conv out; /* w [C][1][1][C] */
} zdit_vae_attn;
typedef struct {
  zdit_vae_conv conv_in;
  zdit_vae_resnet mid[2];
  zdit_vae_attn attn;
  const zdit_vae_resnet* stages[4]; /* host arrays of cfg.resnets blocks each, decoder order */
  zdit_vae_conv upconv[3];
  zdit_vae_norm norm_out;
  zdit_vae_conv conv_out;
} zdit_vae_w;

/* Decode `batch` latents.  latent device fp32 [batch, latent_ch, lat_h, lat_w] (raw: the
 * sampler's final x, unless cfg.flags has ZDIT_VAE_INPUT_UNSCALED), image device fp32
 * [batch, out_ch, 8 lat_h, 8 lat_w], written.  batch 1..ZDIT_MAX_BATCH; lat_h, lat_w even,
 * 2..256; ws: zdit_vae_workspace() bytes (1024^2: ~4.3 GB for one image, the attention
 * scores of the 128 x 128 latent taking 1 GiB of it).  Images are independent. */
size_t zdit_vae_workspace(const zdit_vae_cfg* cfg, int32_t batch, int32_t lat_h, int32_t lat_w);
zdit_status zdit_vae_decode(const zdit_vae_cfg* cfg, const zdit_vae_w* w, int32_t batch,
                            int32_t lat_h, int32_t lat_w, const float* latent, float* image,
                            void* ws, size_t ws_bytes, void* hip_stream);

/* Decoder steps alone (tests and measurement); activations NHWC fp32 [batch, H, W, C]. */
/* GroupNorm of x [batch, hw, C] as a per-image, per-channel affine: affine [batch, C, 2] =
 * (gamma_c r, beta_c - mean gamma_c r), r = 1 / sqrt(var + eps) of the channel's group.
 * C a power of two in 32..1024, groups divides C; ws: zdit_op_vae_groupnorm_workspace(). */
size_t zdit_op_vae_groupnorm_workspace(int32_t batch, int32_t hw, int32_t C, int32_t groups);
zdit_status zdit_op_vae_groupnorm(int32_t batch, int32_t hw, int32_t C, int32_t groups, float eps,
                                  const float* x, const float* gamma, const float* beta,
                                  float* affine, void* ws, size_t ws_bytes, void* hip_stream);
/* out [batch, H, W, cout] = res + conv(t(x)) + b, ksize 1 or 3: x [batch, H, W, cin], or
 * [batch, H/2, W/2, cin] read at half the coordinates with upsample != 0 (2x nearest
 * upsampling before the conv); t(v) = a v + d with (a, d) = affine[img][c] if affine is
 * set (then SiLU if silu != 0), else v; zero padding after t.  res NULL or [batch, H, W,
 * cout] (may equal out).  w [cout][ksize][ksize][cin]; cin a multiple of 4. */
zdit_status zdit_op_vae_conv(int32_t batch, int32_t H, int32_t W, int32_t cin, int32_t cout,
                             int32_t ksize, int32_t upsample, const float* x, const float* affine,
                             int32_t silu, const float* w, const float* b, const float* res,
                             float* out, void* hip_stream);
/* image NCHW [batch, cout, H, W] = conv3x3(SiLU(a x + d)) + b with x NHWC [batch, H, W, cin],
 * (a, d) = affine[img][c] (16-byte aligned), w [cout][3][3][cin]; cout 1..4, cin a multiple
 * of 4. */
zdit_status zdit_op_vae_conv_out(int32_t batch, int32_t H, int32_t W, int32_t cin, int32_t cout,
                                 const float* x, const float* affine, const float* w,
                                 const float* b, float* image, void* hip_stream);
/* The middle attention block in place on x [batch, H, W, C]; H * W a multiple of 4 and at
 * most 65536; ws: zdit_op_vae_attention_workspace(batch, H * W, C, groups) bytes. */
size_t zdit_op_vae_attention_workspace(int32_t batch, int32_t hw, int32_t C, int32_t groups);
zdit_status zdit_op_vae_attention(int32_t batch, int32_t H, int32_t W, int32_t C, int32_t groups,
                                  float eps, const zdit_vae_attn* w, float* x, void* ws,
                                  size_t ws_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------------------
 * Measurement: the sustained bf16 MFMA rate, for roofline fractions against a measured
 * ceiling.  `workgroups` x 256 threads; every wavefront issues 4 x iters
 * v_mfma_f32_32x32x16_bf16 (32768 flops each) on register operands, with no memory traffic
 * in the loop; out: device fp32 [workgroups * 256] (one value per thread, keeps the work live).
 * ------------------------------------------------------------------------------------- */
zdit_status zdit_op_mfma_peak(int32_t workgroups, int32_t iters, float* out, void* hip_stream);
/* Compute units, peak engine clock (kHz) and L2 size (bytes) of HIP device `device`, as the
 * runtime reports them (host only; no device work). */
zdit_status zdit_device_info(int32_t device, int32_t* cu_count, int32_t* max_sclk_khz, int32_t* l2_bytes);

#ifdef __cplusplus
}
#endif
#endif /* ZDIT_H */
