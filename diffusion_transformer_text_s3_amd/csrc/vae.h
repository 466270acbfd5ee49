// Internal types and launchers of the fp32 VAE-decoder kernels (k_vae.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace zdit {

// Implicit-GEMM convolution / batched GEMM on fp32 MFMA:
//   C[z][m][n] = res[z][m][n] + alpha * sum_k A'[z][m][k] B[z][n][k] + bias[n]
// Convolution mode (ksize 3 or 1, batch folded into M): row m is output pixel (img, y, x) of
// an H x W image, k runs over (tap, channel) with channels innermost, A' is the input pixel
// at (y + ky - r, x + kx - r) (zero outside the image; with `upsample` the input has H/2 x W/2
// pixels and is read at half the coordinates), rows of `lda` floats; if `affine` is set each
// input value becomes a * x + d with (a, d) = affine[img][c] (then SiLU if `silu`) before the
// product, padding staying zero.  B holds weights [N][ksize * ksize * K] (ldb floats per row).
// GEMM mode (ksize 1, H = 1, W = M): plain row-major operands.  res may alias C (each element is read before it is written by the same thread).
// N <= 16 runs 256 x 16 tiles (the output conv), else 128 x 128.
struct VConvArgs {
  const float* A;
  int64_t lda;
  const float* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
  const float* res;
  const float* bias;
  const float* affine;  // [images][K][2]
  int silu;
  int M, N, K;          // K = channels per tap
  int H, W;             // output image size (conv mode)
  int ksize, upsample;
  int out_nchw;         // conv mode: C is [images][N][H][W] (ldc unused)
  float alpha;
  // direct-to-LDS form only (vconv_direct_ok): GroupNorm statistics of the output, per 64-row
  // half tile h (rows 64 h .. 64 h + 63) and channel n, at gn_part[h N + n]: the mean of the
  // half's valid rows and the sum of squared deviations from it (nullable)
  float2* gn_part;
};

// GroupNorm statistics over NHWC activations x [images][HW][C], groups of C / groups
// consecutive channels; partial sums per (image, chunk of pixels, channel), then per group.
struct VGnArgs {
  const float* x;
  int images, HW, C, groups;
  int chunk;            // pixels per workgroup
  float* part;          // [images][n_chunks][C]
  double* stat;         // [images][groups][2]: mean, then 1/sqrt(var + eps)
  const float* gamma;
  const float* beta;
  float* affine;        // [images][C][2]
  float eps;
};

int vgn_chunks(int HW, int C);
size_t vgn_part_floats(int images, int HW, int C);

hipError_t launch_vconv(const VConvArgs& a, hipStream_t s);
// whether launch_vconv runs the direct-to-LDS form (no input transform, channels a multiple of
// 16, a tile (128 or, for N <= 16, 256 rows) within one image, buffer offsets within 32 bits);
// otherwise the staged form
bool vconv_direct_ok(const VConvArgs& a);
// out = SiLU(a x + d) (silu != 0) or a x + d over NHWC x [images][hw][C], affine [images][C][2]
// (C a power of two, at least 4); bit-identical to the staged conv's input transform; out may
// alias x
hipError_t launch_vact(const float* x, const float* affine, int images, int64_t hw, int C, int silu, float* out,
                       hipStream_t s);
hipError_t launch_vgn(VGnArgs a, hipStream_t s);   // stats + affine (two passes over x)
// stats + affine from the half-tile statistics a convolution wrote (VConvArgs::gn_part) for
// x [images][HW][C] (C <= 1024): per (image, group) the halves' means and squared deviations
// combined in float64 with Chan et al.'s pairwise update, through chunk results in `chunk`
// (vgn_conv_chunk_doubles); the halves of an image are ceil(HW / 64) in a row (the direct
// form's tiles never straddle images)
size_t vgn_conv_chunk_doubles(int images, int HW, int groups);
hipError_t launch_vgn_from_conv(const float2* part, double* chunk, const VGnArgs& a, hipStream_t s);
// latent [images][ch][h][w] -> NHWC [images][h][w][ch], each value z / scale + shift (unscale
// != 0) or copied
hipError_t launch_vlatent_in(const float* z, float* out, int images, int ch, int h, int w, int unscale,
                             float scale, float shift, hipStream_t s);
// rows of S [rows][n] in place: exp(s - max) / sum
hipError_t launch_vsoftmax(float* S, int64_t rows, int n, hipStream_t s);
// out[c][j] = in[j][c0 + c] (in rows of ld floats), c < C, j < n
hipError_t launch_vtranspose(const float* in, int64_t ld, int c0, float* out, int n, int C, hipStream_t s);

}  // namespace zdit
