"""Oracle for the 16-channel AutoencoderKL decoder that turns the sampler's final latent into
the image: a plain, slow, obviously correct CPU implementation in NumPy.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg
may import this module.  It shares no code with the HIP library or its Python binding, and
imports neither.

What the pages fix (Core AI model zoo, "Z-Image-Turbo port", table "Architecture -> export
mapping", row VAE, and the warning below that table; FastVideo "Z-Image Port Status",
component matrix, row VAE): a 16-channel AutoencoderKL decoder run in fp32, the raw decode
as the component boundary, nearest-neighbour upsampling, and the unscale z / 0.3611 + 0.1159
built into the decoder and applied exactly once (the decoder is fed the raw latent).

Readings where the pages are silent (each is listed with its reason in the design notes):
  V1  architecture: the decoder of the published 16-channel autoencoder whose latent scale
      and shift are 0.3611 and 0.1159: a 3x3 input conv to 512 channels; a middle stage of
      ResNet block, single-head self-attention over all positions, ResNet block; four
      stages of widths 512, 512, 256, 128 with three ResNet blocks each, the first three
      ending in a 2x nearest-neighbour upsample followed by a 3x3 conv; then GroupNorm,
      SiLU and a 3x3 conv to 3 channels.  Convolutions are cross-correlations with zero
      padding 1 (3x3) or 0 (1x1), stride 1, with biases.
  V2  ResNet block: h = conv1(SiLU(GN1(x))), h = conv2(SiLU(GN2(h))), output = s(x) + h with
      s the identity when the widths agree and a 1x1 conv otherwise.
  V3  GroupNorm: 32 groups of consecutive channels, statistics over the group's channels
      and all positions of one image, biased variance, eps 1e-6, then a per-channel gain
      and shift.
  V4  attention: GroupNorm, then q, k, v = linear maps (with biases) of each position's
      channel vector, one head of the full width C, weights softmax(q k^T / sqrt(C)) over
      all positions of the image, output linear map (with bias), residual add.
  V5  the output is the raw decode [B, 3, 8h, 8w] in fp32: no clamp, no mapping to [0, 1].
Parity unpinned: the decoder against the real autoencoder weights (none are available);
the pins in tests/ fix each operation and the wiring.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def unscale(z: np.ndarray, scale: float = 0.3611, shift: float = 0.1159) -> np.ndarray:
    """The latent as the decoder's first layer sees it: z / scale + shift (Core AI page, row
    VAE of the export mapping)."""
    return z / z.dtype.type(scale) + z.dtype.type(shift)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1 + np.exp(-x))


def conv2d(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Cross-correlation of x [B, Cin, H, W] with w [Cout, Cin, k, k] (k odd), zero padding
    (k - 1) / 2, stride 1, plus the bias (reading V1):
    out[n, o, y, x] = b[o] + sum_{c, i, j} w[o, c, i, j] * xpad[n, c, y + i, x + j]."""
    B, C, H, Wd = x.shape
    O, C2, k, k2 = w.shape
    assert C == C2 and k == k2 and k % 2 == 1
    p = (k - 1) // 2
    xp = np.zeros((B, C, H + 2 * p, Wd + 2 * p), x.dtype)
    xp[:, :, p:p + H, p:p + Wd] = x
    out = np.zeros((B, O, H, Wd), x.dtype)
    for i in range(k):
        for j in range(k):
            tap = w[:, :, i, j].astype(x.dtype)                     # [O, C]
            win = xp[:, :, i:i + H, j:j + Wd]                       # [B, C, H, W]
            out += np.einsum("oc,bchw->bohw", tap, win, optimize=True)
    return out + b.astype(x.dtype)[None, :, None, None]


def group_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, groups: int = 32, eps: float = 1e-6) -> np.ndarray:
    """GroupNorm of x [B, C, H, W] (reading V3)."""
    B, C, H, Wd = x.shape
    xg = x.reshape(B, groups, C // groups, H, Wd)
    mean = xg.mean(axis=(2, 3, 4), keepdims=True)
    var = ((xg - mean) ** 2).mean(axis=(2, 3, 4), keepdims=True)
    y = ((xg - mean) / np.sqrt(var + x.dtype.type(eps))).reshape(B, C, H, Wd)
    return y * g.astype(x.dtype)[None, :, None, None] + b.astype(x.dtype)[None, :, None, None]


def upsample_nearest(x: np.ndarray) -> np.ndarray:
    """2x nearest-neighbour upsampling: out[..., y, x] = in[..., y // 2, x // 2]."""
    return np.repeat(np.repeat(x, 2, axis=2), 2, axis=3)


def resnet(x: np.ndarray, W: dict, p: str, groups: int, eps: float) -> np.ndarray:
    """ResNet block (reading V2)."""
    h = conv2d(silu(group_norm(x, W[p + ".gn1.g"], W[p + ".gn1.b"], groups, eps)), W[p + ".conv1.w"], W[p + ".conv1.b"])
    h = conv2d(silu(group_norm(h, W[p + ".gn2.g"], W[p + ".gn2.b"], groups, eps)), W[p + ".conv2.w"], W[p + ".conv2.b"])
    s = conv2d(x, W[p + ".short.w"], W[p + ".short.b"]) if (p + ".short.w") in W else x
    return s + h


def attention(x: np.ndarray, W: dict, p: str, groups: int, eps: float) -> np.ndarray:
    """Single-head self-attention over the positions of each image (reading V4)."""
    B, C, H, Wd = x.shape
    h = group_norm(x, W[p + ".gn.g"], W[p + ".gn.b"], groups, eps)
    t = h.reshape(B, C, H * Wd).transpose(0, 2, 1)                  # [B, N, C] positions x channels
    dt = x.dtype

    def lin(v, n):
        return v @ W[f"{p}.{n}.w"].astype(dt).T + W[f"{p}.{n}.b"].astype(dt)

    q, k, v = lin(t, "q"), lin(t, "k"), lin(t, "v")
    out = np.empty_like(t)
    for n in range(B):
        s = (q[n] @ k[n].T) / dt.type(math.sqrt(C))
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        out[n] = (e / e.sum(axis=1, keepdims=True)) @ v[n]
    o = lin(out, "o")
    return x + o.transpose(0, 2, 1).reshape(B, C, H, Wd)


def decoder(z: np.ndarray, W: dict, vd, dtype=F64, record: dict | None = None) -> np.ndarray:
    """Raw latent z [B, 16, h, w] -> image [B, 3, 8h, 8w] (the page's decode with the
    unscale built in; readings V1-V5).  record, if given, receives the activation after
    each named stage ("in", "mid", "up0".."up3")."""
    g, eps = vd.groups, vd.eps
    x = conv2d(unscale(np.asarray(z, dtype), vd.scale, vd.shift), W["conv_in.w"], W["conv_in.b"])
    if record is not None:
        record["in"] = x
    x = resnet(x, W, "mid.res0", g, eps)
    x = attention(x, W, "mid.attn", g, eps)
    x = resnet(x, W, "mid.res1", g, eps)
    if record is not None:
        record["mid"] = x
    for i, (_, _, up) in enumerate(vd.stages):
        for j in range(vd.resnets):
            x = resnet(x, W, f"up{i}.res{j}", g, eps)
        if up:
            x = conv2d(upsample_nearest(x), W[f"up{i}.upconv.w"], W[f"up{i}.upconv.b"])
        if record is not None:
            record[f"up{i}"] = x
    x = silu(group_norm(x, W["norm_out.g"], W["norm_out.b"], g, eps))
    return conv2d(x, W["conv_out.w"], W["conv_out.b"])
