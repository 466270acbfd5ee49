"""Pins of the VAE-decoder oracle (CPU only): each operation against brute force, a library
routine, a closed form or an invariant that the mathematics fixes, and the wiring of the
whole decoder against a reduction to a chain of already-pinned operations."""
import math

import numpy as np
import pytest
from scipy import signal

import synth
from oracle import vae_oracle as V


def _g(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------ convolution
def test_conv2d_matches_brute_force_loops():
    g = _g(1)
    x = g.standard_normal((2, 3, 5, 4))
    w = g.standard_normal((4, 3, 3, 3))
    b = g.standard_normal(4)
    got = V.conv2d(x, w, b)
    B, C, H, W = x.shape
    want = np.zeros((B, 4, H, W))
    for n in range(B):
        for o in range(4):
            for y in range(H):
                for xx in range(W):
                    acc = b[o]
                    for c in range(C):
                        for i in range(3):
                            for j in range(3):
                                yy, xs = y + i - 1, xx + j - 1
                                if 0 <= yy < H and 0 <= xs < W:
                                    acc += w[o, c, i, j] * x[n, c, yy, xs]
                    want[n, o, y, xx] = acc
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_conv2d_matches_scipy_correlate():
    g = _g(2)
    x = g.standard_normal((1, 4, 9, 7))
    w = g.standard_normal((2, 4, 3, 3))
    b = np.zeros(2)
    got = V.conv2d(x, w, b)
    for o in range(2):
        want = sum(signal.correlate2d(x[0, c], w[o, c], mode="same", boundary="fill") for c in range(4))
        np.testing.assert_allclose(got[0, o], want, rtol=1e-12, atol=1e-12)


def test_conv2d_zero_padding_closed_form():
    """All-ones input and kernel: a position sees as many taps as lie inside the image."""
    x = np.ones((1, 2, 4, 5))
    w = np.ones((1, 2, 3, 3))
    got = V.conv2d(x, w, np.array([0.5]))[0, 0]
    assert got[0, 0] == 2 * 4 + 0.5 and got[0, 2] == 2 * 6 + 0.5 and got[1, 1] == 2 * 9 + 0.5
    assert got[3, 4] == 2 * 4 + 0.5 and got[2, 0] == 2 * 6 + 0.5


def test_conv2d_is_correlation_not_convolution():
    """A kernel with a single 1 at (row 0, col 2) reads the input at (y - 1, x + 1)."""
    x = np.arange(20, dtype=np.float64).reshape(1, 1, 4, 5)
    w = np.zeros((1, 1, 3, 3))
    w[0, 0, 0, 2] = 1
    got = V.conv2d(x, w, np.zeros(1))[0, 0]
    assert got[2, 1] == x[0, 0, 1, 2] and got[0, 1] == 0 and got[1, 4] == 0


def test_conv1x1_is_a_per_position_matrix_product():
    g = _g(3)
    x = g.standard_normal((2, 6, 3, 4))
    w = g.standard_normal((5, 6, 1, 1))
    b = g.standard_normal(5)
    want = np.einsum("oc,bchw->bohw", w[:, :, 0, 0], x) + b[None, :, None, None]
    np.testing.assert_allclose(V.conv2d(x, w, b), want, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------------------ GroupNorm
def test_group_norm_hand_worked():
    """Two groups of two channels over a 1 x 2 image: group 0 holds 1, 2, 3, 4 (mean 2.5,
    variance 1.25), group 1 holds 10, 10, 10, 14 (mean 11, variance 3)."""
    x = np.array([1, 2, 3, 4, 10, 10, 10, 14], dtype=np.float64).reshape(1, 4, 1, 2)
    g = np.array([1.0, 2.0, 1.0, 1.0])
    b = np.array([0.0, 0.0, 0.5, 0.0])
    y = V.group_norm(x, g, b, groups=2, eps=0.0)
    s0, s1 = math.sqrt(1.25), math.sqrt(3.0)
    want = np.array([(1 - 2.5) / s0, (2 - 2.5) / s0, 2 * (3 - 2.5) / s0, 2 * (4 - 2.5) / s0,
                     (10 - 11) / s1 + 0.5, (10 - 11) / s1 + 0.5, (10 - 11) / s1, (14 - 11) / s1]).reshape(1, 4, 1, 2)
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-14)


def test_group_norm_eps_and_statistics():
    g = _g(4)
    x = 3.0 + 2.0 * g.standard_normal((2, 8, 5, 6))
    y = V.group_norm(x, np.ones(8), np.zeros(8), groups=4, eps=0.0)
    yg = y.reshape(2, 4, 2, 5, 6)
    np.testing.assert_allclose(yg.mean(axis=(2, 3, 4)), 0, atol=1e-12)
    np.testing.assert_allclose(yg.var(axis=(2, 3, 4)), 1, rtol=1e-12)
    # eps enters under the square root: a constant group normalises to zero, eps 1 gives x / sqrt(var + 1)
    c = np.zeros((1, 2, 1, 2))
    c[0, 0] = 5
    assert np.all(V.group_norm(c, np.ones(2), np.zeros(2), groups=2, eps=1e-6) == 0)
    z = np.array([-1.0, 1.0, -1.0, 1.0]).reshape(1, 2, 1, 2)
    np.testing.assert_allclose(V.group_norm(z, np.ones(2), np.zeros(2), groups=1, eps=1.0), z / math.sqrt(2), rtol=1e-15)


def test_group_norm_groups_are_consecutive_channels_per_image():
    """Scaling channels 2..3 (group 1 of 4 channels in 2 groups) or image 1 leaves the other
    group's and the other image's outputs unchanged."""
    g = _g(5)
    x = g.standard_normal((2, 4, 3, 3))
    base = V.group_norm(x, np.ones(4), np.zeros(4), groups=2, eps=1e-6)
    x2 = x.copy()
    x2[:, 2:4] *= 7.0
    x2[:, 2:4] += 3.0
    y2 = V.group_norm(x2, np.ones(4), np.zeros(4), groups=2, eps=1e-6)
    np.testing.assert_allclose(y2[:, 0:2], base[:, 0:2], rtol=1e-14)
    x3 = x.copy()
    x3[1] *= 9
    y3 = V.group_norm(x3, np.ones(4), np.zeros(4), groups=2, eps=1e-6)
    np.testing.assert_allclose(y3[0], base[0], rtol=1e-14)


# ------------------------------------------------------------------------------ small pieces
def test_silu_values():
    np.testing.assert_allclose(V.silu(np.array([0.0, 1.0, -1.0, 20.0])),
                               [0.0, 0.7310585786300049, -0.2689414213699951, 19.999999958776925], rtol=1e-15)


def test_upsample_nearest_is_a_kronecker_product():
    x = _g(6).standard_normal((2, 3, 4, 5))
    want = np.kron(x, np.ones((1, 1, 2, 2)))
    np.testing.assert_array_equal(V.upsample_nearest(x), want)
    assert V.upsample_nearest(x)[1, 2, 7, 3] == x[1, 2, 3, 1]


def test_unscale_constants():
    """The page's unscale: z / 0.3611 + 0.1159, so 0.3611 -> 1.1159 and 0 -> 0.1159."""
    np.testing.assert_allclose(V.unscale(np.array([0.3611, 0.0, -0.7222])), [1.1159, 0.1159, -1.8841], rtol=1e-14)


# ------------------------------------------------------------------------------ attention
def _attn_weights(C, seed, zero_q=False):
    g = _g(seed)
    W = {"a.gn.g": 1 + 0.1 * g.standard_normal(C), "a.gn.b": 0.1 * g.standard_normal(C)}
    for n in "qkvo":
        W[f"a.{n}.w"] = g.standard_normal((C, C)) / math.sqrt(C)
        W[f"a.{n}.b"] = 0.1 * g.standard_normal(C)
    if zero_q:
        W["a.q.w"] = np.zeros((C, C))
        W["a.q.b"] = np.zeros(C)
    return W


def test_attention_uniform_weights_when_queries_vanish():
    """q = 0: every position attends uniformly, so each output is x + W_o mean(v) + b_o."""
    C = 8
    W = _attn_weights(C, 7, zero_q=True)
    x = _g(8).standard_normal((1, C, 3, 4))
    h = V.group_norm(x, W["a.gn.g"], W["a.gn.b"], groups=4, eps=1e-6).reshape(C, 12).T
    v = h @ W["a.v.w"].T + W["a.v.b"]
    o = v.mean(axis=0) @ W["a.o.w"].T + W["a.o.b"]
    want = x + o[None, :, None, None]
    np.testing.assert_allclose(V.attention(x, W, "a", groups=4, eps=1e-6), want, rtol=1e-12, atol=1e-12)


def test_attention_against_softmax_definition_per_position():
    """Brute force: for one position, weights exp(q.k_j / sqrt(C)) / sum, output x + W_o sum_j w_j v_j + b_o."""
    C = 8
    W = _attn_weights(C, 9)
    x = _g(10).standard_normal((2, C, 2, 3))
    got = V.attention(x, W, "a", groups=2, eps=1e-6)
    for n in range(2):
        h = V.group_norm(x[n:n + 1], W["a.gn.g"], W["a.gn.b"], groups=2, eps=1e-6)[0].reshape(C, 6).T
        q = h @ W["a.q.w"].T + W["a.q.b"]
        k = h @ W["a.k.w"].T + W["a.k.b"]
        v = h @ W["a.v.w"].T + W["a.v.b"]
        for p in range(6):
            s = [float(q[p] @ k[j]) / math.sqrt(C) for j in range(6)]
            e = [math.exp(t) for t in s]
            a = sum(e[j] / sum(e) * v[j] for j in range(6))
            want = x[n, :, p // 3, p % 3] + a @ W["a.o.w"].T + W["a.o.b"]
            np.testing.assert_allclose(got[n, :, p // 3, p % 3], want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------ ResNet block
def test_resnet_reduces_to_shortcut_when_second_conv_is_zero():
    vd = synth.VAE_TINY
    W = synth.vae_weights(vd, 11)
    x = _g(12).standard_normal((1, 64, 4, 4))
    for p in ("mid.res0",):
        Wz = dict(W)
        Wz[p + ".conv2.w"] = np.zeros_like(W[p + ".conv2.w"])
        Wz[p + ".conv2.b"] = np.zeros_like(W[p + ".conv2.b"])
        np.testing.assert_allclose(V.resnet(x, Wz, p, 32, 1e-6), x, rtol=0, atol=0)
    # width change: 64 -> 32 in the last stage's first block; the shortcut is the 1x1 conv
    p = "up2.res0"
    assert W[p + ".short.w"].shape == (32, 64, 1, 1)
    Wz = dict(W)
    Wz[p + ".conv2.w"] = np.zeros_like(W[p + ".conv2.w"])
    Wz[p + ".conv2.b"] = np.zeros_like(W[p + ".conv2.b"])
    np.testing.assert_allclose(V.resnet(x, Wz, p, 32, 1e-6), V.conv2d(x, W[p + ".short.w"], W[p + ".short.b"]),
                               rtol=1e-14, atol=1e-14)


def test_resnet_residual_branch_by_hand():
    """The residual branch written out from the pinned pieces (norm, SiLU, conv) for one block."""
    vd = synth.VAE_TINY
    W = synth.vae_weights(vd, 13)
    x = _g(14).standard_normal((1, 64, 3, 5))
    p = "up0.res1"
    t = V.group_norm(x, W[p + ".gn1.g"], W[p + ".gn1.b"], 32, 1e-6)
    t = V.conv2d(t / (1 + np.exp(-t)), W[p + ".conv1.w"], W[p + ".conv1.b"])
    t = V.group_norm(t, W[p + ".gn2.g"], W[p + ".gn2.b"], 32, 1e-6)
    t = V.conv2d(t / (1 + np.exp(-t)), W[p + ".conv2.w"], W[p + ".conv2.b"])
    np.testing.assert_allclose(V.resnet(x, W, p, 32, 1e-6), x + t, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------------------ whole decoder
def _reduced(W, vd):
    """Weights where every ResNet block and the attention add nothing but their shortcut:
    second convs and the attention's output map zeroed."""
    Wz = dict(W)
    for k in list(W):
        if k.endswith(".conv2.w") or k.endswith(".conv2.b") or k in ("mid.attn.o.w", "mid.attn.o.b"):
            Wz[k] = np.zeros_like(W[k])
    return Wz


def test_decoder_wiring_reduced_to_a_chain():
    """With the residual branches zeroed the decoder is: unscale, conv_in, then per stage the
    1x1 shortcut where the width changes and the upsample + conv where the stage ends in
    one, then norm, SiLU, conv_out.  Written out from the pinned pieces."""
    vd = synth.VAE_TINY
    W = _reduced(synth.vae_weights(vd, 15), vd)
    z = _g(16).standard_normal((1, 16, 3, 2))
    x = V.conv2d(z / 0.3611 + 0.1159, W["conv_in.w"], W["conv_in.b"])
    assert x.shape == (1, 64, 3, 2)
    # stages 0, 1: 64 -> 64 with upsample; stage 2: 64 -> 32 (1x1 shortcut), upsample; stage 3: 32, none
    x = V.conv2d(V.upsample_nearest(x), W["up0.upconv.w"], W["up0.upconv.b"])
    x = V.conv2d(V.upsample_nearest(x), W["up1.upconv.w"], W["up1.upconv.b"])
    x = V.conv2d(x, W["up2.res0.short.w"], W["up2.res0.short.b"])
    x = V.conv2d(V.upsample_nearest(x), W["up2.upconv.w"], W["up2.upconv.b"])
    t = V.group_norm(x, W["norm_out.g"], W["norm_out.b"], 32, 1e-6)
    want = V.conv2d(t / (1 + np.exp(-t)), W["conv_out.w"], W["conv_out.b"])
    got = V.decoder(z, W, vd)
    assert got.shape == (1, 3, 24, 16)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_decoder_stage_shapes_and_widths():
    vd = synth.VAE_FULL
    assert vd.stages == [(512, 512, True), (512, 512, True), (512, 256, True), (256, 128, False)]
    W = synth.vae_weights(vd, 17)
    n_conv3 = sum(1 for k, v in W.items() if k.endswith(".w") and v.ndim == 4 and v.shape[-1] == 3)
    # conv_in + 2 x 2 (middle) + 4 stages x 3 blocks x 2 + 3 upsample convs + conv_out
    assert n_conv3 == 1 + 4 + 24 + 3 + 1
    assert sorted(k for k in W if k.endswith("short.w")) == ["up2.res0.short.w", "up3.res0.short.w"]
    assert W["conv_in.w"].shape == (512, 16, 3, 3) and W["conv_out.w"].shape == (3, 128, 3, 3)


def test_decoder_batch_items_are_independent():
    vd = synth.VAE_TINY
    W = synth.vae_weights(vd, 18)
    z = _g(19).standard_normal((2, 16, 2, 3))
    both = V.decoder(z, W, vd)
    one = V.decoder(z[1:2], W, vd)
    np.testing.assert_allclose(both[1:2], one, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", [np.float32])
def test_decoder_fp32_close_to_fp64(dtype):
    vd = synth.VAE_TINY
    W = synth.vae_weights(vd, 20)
    z = _g(21).standard_normal((1, 16, 4, 4))
    a = V.decoder(z, W, vd, dtype=np.float64)
    b = V.decoder(z, W, vd, dtype=dtype)
    assert b.dtype == dtype
    assert np.linalg.norm(b - a) / np.linalg.norm(a) < 1e-5
