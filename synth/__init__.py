"""Seeded synthetic inputs for the S3-DiT hot path (weights, latents, caption features,
residual-stream inputs), shared by the oracle tests, the GPU parity tests and the bench.

This module holds no arithmetic of the method: it only draws seeded random numbers and
lays them out.  Weights are drawn from N(0, 0.02) in fp32 and then truncated to the nearest
bf16-representable value toward zero (the low 16 bits of the fp32 pattern cleared), so the
oracle (which reads them as fp32) and the GPU (which reads the same values as bf16 bits)
see identical numbers.  Truncation is a choice of input distribution, not a rounding step
of the method.

Every tensor gets its own generator, seeded from ``SeedSequence([seed, tag, index])`` with
a fixed tag per tensor kind, so adding or removing one tensor never shifts another.

Workload shapes follow the pages: dim 3840, 30 heads of 128, a 34-block stack of
2 noise-refiner + 2 context-refiner + 30 main blocks (Core AI model zoo, "Z-Image-Turbo
port", table "Architecture -> export mapping", row DiT); caption width 2560 (FastVideo
"Z-Image Port Status", summary of the pinned text encoder); caption padding to a multiple
of 32 with a 45-token prompt and an empty negative (Core AI page, section "The three things
that each cost a wrong image", item 3); 16-channel latents and a 2x2 patch (Core AI page,
section "Three more things", patchify feature order); residual stream near 6.7e3 and w2 /
to_out outputs near 3.1e5 (Core AI page, section "fp16 does not work. bf16 does.").  The
SwiGLU hidden width 10240 and the 256-wide timestep embedding are not on the pages; they
are chosen.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

WEIGHT_STD = 0.02

# fixed tags, one per tensor kind
_T_BLOCK = 1
_T_EMBED = 2
_T_X = 3
_T_LAT = 4
_T_CAP = 5
_T_OUTLIER = 6


@dataclass(frozen=True)
class Dims:
    dim: int = 3840
    n_heads: int = 30
    head_dim: int = 128
    ffn_hidden: int = 10240
    rope_axes: tuple = (32, 48, 48)
    c_dim: int = 256
    t_freq: int = 256
    norm_eps: float = 1e-6
    rope_theta: float = 10000.0
    t_scale: float = 1000.0
    latent_ch: int = 16
    patch: int = 2
    cap_dim: int = 2560
    seq_multiple: int = 32
    max_cap_len: int = 512
    n_noise_ref: int = 2
    n_ctx_ref: int = 2
    n_main: int = 30

    def replace(self, **kw) -> "Dims":
        return dataclasses.replace(self, **kw)


FULL = Dims()
TINY = Dims(dim=384, n_heads=3, ffn_hidden=1024)


@dataclass(frozen=True)
class Workload:
    """One named workload: shapes and seeds only."""
    name: str
    dims: Dims
    batch: int
    lat_h: int              # latent height (pixels / 8)
    lat_w: int
    cap_len: tuple          # caption token counts per branch (before padding)
    t: float = 0.5
    seed: int = 0
    outlier_frac: float = 0.0
    outlier_mag: float = 6.7e3
    w2_outlier_channels: int = 0
    w2_outlier_alpha: float = 1.0
    guidance: float = 1.0
    num_steps: int = 8
    shift: float = 3.0
    extra: dict = field(default_factory=dict)


# The five workloads.  cfg1: tiny block/stack; cfg2: one full-width block at 256 px;
# cfg3: one full-width block at 1024^2 on a cond/uncond pair; cfg4: one full-stack step at
# 1024^2; cfg5: the 8-step negated-CFG loop at 1024^2 and 1536x1024.
CFG1 = Workload("tiny block d384 at 128px (64 image tokens + caption 20 -> 32)",
                TINY, batch=1, lat_h=16, lat_w=16, cap_len=(20,), t=0.5, seed=0)
CFG2 = Workload("full-width block at 256px (256 image tokens + caption 45 -> 64)",
                FULL, batch=1, lat_h=32, lat_w=32, cap_len=(45,), t=0.5, seed=2,
                outlier_frac=0.001)
# w2_outlier_alpha is fixed by tests/golden/calibrate_w2_alpha.py (oracle only) so that the
# largest |w2 output| on this input is about 3e5.
CFG3 = Workload("full-width block at 1024^2, cond/uncond pair (S = 4160 / 4128)",
                FULL, batch=2, lat_h=128, lat_w=128, cap_len=(45, 10), t=0.5, seed=3,
                outlier_frac=0.001, w2_outlier_channels=4, w2_outlier_alpha=41756.0)
CFG4 = Workload("full 34-block stack, one sampler step at 1024^2",
                FULL, batch=2, lat_h=128, lat_w=128, cap_len=(45, 10), t=0.5, seed=4)
CFG5 = Workload("8-step negated-CFG FlowMatchEuler pass at 1024x1024",
                FULL, batch=2, lat_h=128, lat_w=128, cap_len=(45, 10), seed=42,
                guidance=1.0, num_steps=8, shift=3.0)
CFG5_WIDE = Workload("8-step negated-CFG FlowMatchEuler pass at 1536x1024",
                     FULL, batch=2, lat_h=128, lat_w=192, cap_len=(45, 10), seed=42,
                     guidance=1.0, num_steps=8, shift=3.0)


def rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tag), int(index)]))


def bf16_truncate(a: np.ndarray) -> np.ndarray:
    """fp32 array -> fp32 array whose values are bf16-representable (low 16 bits cleared)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Bit pattern (uint16) of a bf16-representable fp32 array; exact, no rounding."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array is not bf16-representable")
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _weight(g, shape):
    return bf16_truncate(_normal(g, shape, WEIGHT_STD))


def block_weights(dims: Dims, seed: int, index: int = 0, adaln: bool = True,
                  w2_outlier_channels: int = 0, w2_outlier_alpha: float = 1.0) -> dict:
    """Weights of one transformer block, [out, in] row-major, as fp32 arrays.

    Matrices are bf16-representable; norm gains are 1 + 0.02 N(0,1) in fp32 (so a wrong
    gain index is visible); adaLN bias is N(0, 0.02) in fp32.  With adaln=False the block
    has no modulation weights (context-refiner blocks).
    """
    d, H = dims.dim, dims.ffn_hidden
    base = 16 * index
    w = {
        "w_qkv": _weight(rng(seed, _T_BLOCK, base + 0), (3 * d, d)),
        "w_out": _weight(rng(seed, _T_BLOCK, base + 1), (d, d)),
        "w1": _weight(rng(seed, _T_BLOCK, base + 2), (H, d)),
        "w3": _weight(rng(seed, _T_BLOCK, base + 3), (H, d)),
        "w2": _weight(rng(seed, _T_BLOCK, base + 4), (d, H)),
        "norm1": (1.0 + _normal(rng(seed, _T_BLOCK, base + 5), (d,), WEIGHT_STD)).astype(np.float32),
        "norm2": (1.0 + _normal(rng(seed, _T_BLOCK, base + 6), (d,), WEIGHT_STD)).astype(np.float32),
    }
    if adaln:
        w["w_ada"] = _weight(rng(seed, _T_BLOCK, base + 7), (6 * d, dims.c_dim))
        w["b_ada"] = _normal(rng(seed, _T_BLOCK, base + 8), (6 * d,), WEIGHT_STD)
    else:
        w["w_ada"] = None
        w["b_ada"] = None
    if w2_outlier_channels:
        # a few output channels of w2 scaled up, so the FFN output reaches the ~3e5 range
        g = rng(seed, _T_OUTLIER, index)
        ch = np.sort(g.choice(d, size=w2_outlier_channels, replace=False))
        w2 = w["w2"]
        w2[ch, :] = bf16_truncate(w2[ch, :] * np.float32(w2_outlier_alpha))
        w["w2_outlier_rows"] = ch
    return w


def embed_weights(dims: Dims, seed: int) -> dict:
    """x-embed, cap-embed, learned caption pad, timestep MLP and final-layer weights."""
    d, p, C = dims.dim, dims.patch, dims.latent_ch
    f = p * p * C
    cd, tf = dims.c_dim, dims.t_freq
    k = 0

    def nxt():
        nonlocal k
        k += 1
        return rng(seed, _T_EMBED, k)

    return {
        "x_emb_w": _weight(nxt(), (d, f)),
        "x_emb_b": _normal(nxt(), (d,), WEIGHT_STD),
        "cap_emb_w": _weight(nxt(), (d, dims.cap_dim)),
        "cap_emb_b": _normal(nxt(), (d,), WEIGHT_STD),
        "cap_pad": _normal(nxt(), (d,), 1.0),
        "t_w1": _normal(nxt(), (cd, tf), WEIGHT_STD),
        "t_b1": _normal(nxt(), (cd,), WEIGHT_STD),
        "t_w2": _normal(nxt(), (cd, cd), WEIGHT_STD),
        "t_b2": _normal(nxt(), (cd,), WEIGHT_STD),
        "final_norm": (1.0 + _normal(nxt(), (d,), WEIGHT_STD)).astype(np.float32),
        "final_ada_w": _weight(nxt(), (2 * d, cd)),
        "final_ada_b": _normal(nxt(), (2 * d,), WEIGHT_STD),
        "final_w": _weight(nxt(), (f, d)),
        "final_b": _normal(nxt(), (f,), WEIGHT_STD),
    }


def model_weights(dims: Dims, seed: int, threads: int | None = None) -> dict:
    """All weights of a stack: embeds plus noise-refiner, context-refiner and main blocks.

    Blocks are drawn on `threads` threads (default: the usable cores, at most 16); every tensor
    has its own generator, so the values do not depend on the thread count."""
    w = embed_weights(dims, seed)
    nr_, cr_ = dims.n_noise_ref, dims.n_ctx_ref
    jobs = [(i, i < nr_ or i >= nr_ + cr_) for i in range(nr_ + cr_ + dims.n_main)]
    if threads is None:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    make = lambda j: block_weights(dims, seed, j[0], adaln=j[1])
    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(min(threads, len(jobs))) as ex:
            blocks = list(ex.map(make, jobs))
    else:
        blocks = [make(j) for j in jobs]
    w["noise_ref"] = blocks[:nr_]
    w["ctx_ref"] = blocks[nr_:nr_ + cr_]
    w["main"] = blocks[nr_ + cr_:]
    return w


def residual_input(shape, seed: int, outlier_frac: float = 0.0, outlier_mag: float = 6.7e3,
                   index: int = 0) -> np.ndarray:
    """Residual-stream input: N(0,1) fp32 with a seeded fraction of entries set to +-mag."""
    g = rng(seed, _T_X, index)
    x = _normal(g, shape)
    if outlier_frac > 0:
        n = x.size
        k = int(round(outlier_frac * n))
        pos = g.choice(n, size=k, replace=False)
        sign = np.where(g.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
        x.reshape(-1)[pos] = sign * np.float32(outlier_mag)
    return x


def latents(shape, seed: int, index: int = 0) -> np.ndarray:
    """fp32 N(0,1) latents, shape [..., C, h, w]."""
    return _normal(rng(seed, _T_LAT, index), shape)


def caption_features(batch: int, max_len: int, cap_dim: int, seed: int) -> np.ndarray:
    """fp32 N(0,1) caption features [batch, max_len, cap_dim] (stand-in for the encoder's
    penultimate hidden state, which needs trained weights)."""
    return _normal(rng(seed, _T_CAP, 0), (batch, max_len, cap_dim))


# --------------------------------------------------------------------------------------
# text encoder that precedes the path (Qwen3-4B-shaped decoder stack, random weights)
# --------------------------------------------------------------------------------------
_T_ENC = 7
_T_IDS = 8


@dataclass(frozen=True)
class EncDims:
    """Shapes of the text encoder.  Depth, widths and head counts are the pinned encoder's
    (FastVideo "Z-Image Port Status": 36 decoder blocks, hidden 2560, intermediate 9728,
    32 attention heads, 8 KV heads, head dimension 128).  The vocabulary size, RoPE base and
    norm epsilon are not on the pages: the published Qwen3 values are used (151936, 1e6,
    1e-6); tests use a small vocabulary, which no arithmetic depends on."""
    hidden: int = 2560
    inter: int = 9728
    n_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    n_layers: int = 36
    vocab: int = 151936
    rope_theta: float = 1.0e6
    norm_eps: float = 1e-6

    def replace(self, **kw) -> "EncDims":
        return dataclasses.replace(self, **kw)


ENC_FULL = EncDims()
ENC_TINY = EncDims(hidden=256, inter=512, n_heads=4, n_kv_heads=2, n_layers=3, vocab=1000)


def encoder_layer_weights(ed: EncDims, seed: int, index: int) -> dict:
    """Weights of one encoder block, [out, in] row-major, fp32 arrays with bf16-representable
    matrices; norm gains 1 + 0.02 N(0,1) in fp32.  w_qkv rows: the n_heads query heads, then
    the n_kv_heads key heads, then the n_kv_heads value heads, 128 rows each."""
    D, I, hd = ed.hidden, ed.inter, ed.head_dim
    nq, nkv = ed.n_heads * hd, ed.n_kv_heads * hd
    base = 16 * index
    return {
        "in_norm": (1.0 + _normal(rng(seed, _T_ENC, base + 0), (D,), WEIGHT_STD)).astype(np.float32),
        "w_qkv": _weight(rng(seed, _T_ENC, base + 1), (nq + 2 * nkv, D)),
        "q_norm": (1.0 + _normal(rng(seed, _T_ENC, base + 2), (hd,), WEIGHT_STD)).astype(np.float32),
        "k_norm": (1.0 + _normal(rng(seed, _T_ENC, base + 3), (hd,), WEIGHT_STD)).astype(np.float32),
        "w_o": _weight(rng(seed, _T_ENC, base + 4), (D, nq)),
        "post_norm": (1.0 + _normal(rng(seed, _T_ENC, base + 5), (D,), WEIGHT_STD)).astype(np.float32),
        "w_gate": _weight(rng(seed, _T_ENC, base + 6), (I, D)),
        "w_up": _weight(rng(seed, _T_ENC, base + 7), (I, D)),
        "w_down": _weight(rng(seed, _T_ENC, base + 8), (D, I)),
    }


def encoder_weights(ed: EncDims, seed: int, n_layers: int | None = None, threads: int | None = None) -> dict:
    """Embedding table (bf16-representable N(0,1) rows) and the first n_layers blocks (drawn on
    `threads` threads; each block has its own generators, so the result does not depend on it)."""
    n = ed.n_layers if n_layers is None else n_layers
    embed = bf16_truncate(_normal(rng(seed, _T_ENC, 1 << 20), (ed.vocab, ed.hidden)))
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0))) if n > 4 else 1
    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            layers = list(ex.map(lambda i: encoder_layer_weights(ed, seed, i), range(n)))
    else:
        layers = [encoder_layer_weights(ed, seed, i) for i in range(n)]
    return {"embed": embed, "layers": layers}


def token_ids(batch: int, max_len: int, lengths, vocab: int, seed: int) -> np.ndarray:
    """int32 [batch, max_len]: uniform ids in [0, vocab) below each branch's length, the id
    0 after it (right padding, as the host tokenizer step produces)."""
    ids = rng(seed, _T_IDS, 0).integers(0, vocab, size=(batch, max_len), dtype=np.int64)
    for b, L in enumerate(lengths):
        ids[b, L:] = 0
    return ids.astype(np.int32)


# ----------------------------------------------------------------------------- VAE decoder
_T_VAE = 9


@dataclass(frozen=True)
class VaeDims:
    """The 16-channel AutoencoderKL decoder.  Core AI model zoo, "Z-Image-Turbo port", table
    "Architecture -> export mapping", row VAE, gives the latent width, fp32 and the unscale
    constants; the stage widths (given in encoder order, the decoder walks them reversed),
    three ResNet blocks per decoder stage and 32 norm groups are the published configuration
    of the 16-channel autoencoder with those constants (a reading, not on the pages)."""
    latent_ch: int = 16
    out_ch: int = 3
    widths: tuple = (128, 256, 512, 512)
    resnets: int = 3
    groups: int = 32
    eps: float = 1e-6
    scale: float = 0.3611
    shift: float = 0.1159

    def replace(self, **kw) -> "VaeDims":
        return dataclasses.replace(self, **kw)

    @property
    def stages(self):
        """Decoder stages in order: (input width, output width, upsample after)."""
        rev = list(reversed(self.widths))
        out, cin = [], rev[0]
        for i, c in enumerate(rev):
            out.append((cin, c, i < len(rev) - 1))
            cin = c
        return out


VAE_FULL = VaeDims()
VAE_TINY = VaeDims(widths=(32, 32, 64, 64))


def vae_weights(vd: VaeDims, seed: int) -> dict:
    """Weights of the decoder as fp32 arrays, convolutions [out, in, kh, kw], linear maps
    [out, in].  Convolutions draw N(0, 1/fan_in) (the second conv of each ResNet block
    N(0, 0.25/fan_in), so the residual stream grows slowly); norm gains 1 + 0.1 N(0,1),
    norm shifts and biases 0.05 N(0,1).  Keys: conv_in, mid.res0, mid.attn, mid.res1,
    up{i}.res{j}, up{i}.upconv (stages 0..2), norm_out, conv_out."""
    idx = [0]

    def nxt():
        idx[0] += 1
        return rng(seed, _T_VAE, idx[0])

    def conv(o, i, k, gain=1.0):
        return _normal(nxt(), (o, i, k, k), float(np.sqrt(gain / (i * k * k))))

    def vec(n, base=0.0, std=0.05):
        return (np.float32(base) + _normal(nxt(), (n,), std)).astype(np.float32)

    W = {}

    def resnet(p, cin, cout):
        W[p + ".gn1.g"], W[p + ".gn1.b"] = vec(cin, 1.0, 0.1), vec(cin)
        W[p + ".conv1.w"], W[p + ".conv1.b"] = conv(cout, cin, 3), vec(cout)
        W[p + ".gn2.g"], W[p + ".gn2.b"] = vec(cout, 1.0, 0.1), vec(cout)
        W[p + ".conv2.w"], W[p + ".conv2.b"] = conv(cout, cout, 3, 0.25), vec(cout)
        if cin != cout:
            W[p + ".short.w"], W[p + ".short.b"] = conv(cout, cin, 1), vec(cout)

    c0 = vd.widths[-1]
    W["conv_in.w"], W["conv_in.b"] = conv(c0, vd.latent_ch, 3), vec(c0)
    resnet("mid.res0", c0, c0)
    W["mid.attn.gn.g"], W["mid.attn.gn.b"] = vec(c0, 1.0, 0.1), vec(c0)
    for n in "qkvo":
        W[f"mid.attn.{n}.w"] = _normal(nxt(), (c0, c0), float(np.sqrt(1.0 / c0)))
        W[f"mid.attn.{n}.b"] = vec(c0)
    resnet("mid.res1", c0, c0)
    for i, (cin, c, up) in enumerate(vd.stages):
        for j in range(vd.resnets):
            resnet(f"up{i}.res{j}", cin if j == 0 else c, c)
        if up:
            W[f"up{i}.upconv.w"], W[f"up{i}.upconv.b"] = conv(c, c, 3), vec(c)
    cl = vd.widths[0]
    W["norm_out.g"], W["norm_out.b"] = vec(cl, 1.0, 0.1), vec(cl)
    W["conv_out.w"], W["conv_out.b"] = conv(vd.out_ch, cl, 3), vec(vd.out_ch)
    return W


def vae_activations(shape, seed: int, index: int = 0, std: float = 1.0) -> np.ndarray:
    """A seeded N(0, std^2) fp32 activation tensor (inputs of single-layer tests)."""
    return _normal(rng(seed, _T_VAE, 100000 + index), shape, std)
