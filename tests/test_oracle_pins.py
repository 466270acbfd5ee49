"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test names the fact it pins.  None re-types an oracle formula: they use values the
pages give, closed forms, invariants, brute force on tiny inputs, or a library routine.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth
from conftest import golden

F32 = np.float32


# ---------------------------------------------------------------- caption padding (n_cap)
def test_n_cap_worked_values():
    for L, want in golden("n_cap_cases.txt"):
        assert O.n_cap(int(L)) == int(want)


def test_n_cap_all_lengths_are_smallest_multiple():
    for L in range(1, 513):
        n = O.n_cap(L)
        assert n % 32 == 0 and n >= L and n - 32 < L


@pytest.mark.parametrize("bad", [0, -1, 513, 10_000])
def test_n_cap_rejects_out_of_range(bad):
    with pytest.raises(ValueError):
        O.n_cap(bad)


# ---------------------------------------------------------------- patchify / unpatchify
def _value_latent(C, h, w):
    ch, y, x = np.meshgrid(np.arange(C), np.arange(h), np.arange(w), indexing="ij")
    return (ch * 10000 + y * 100 + x).astype(np.float64)


def test_patchify_hand_checked_entries():
    lat = _value_latent(16, 6, 8)
    tok = O.patchify(lat)
    assert tok.shape == (12, 64)
    for n, f, v in golden("patchify_entries.txt"):
        assert tok[int(n), int(f)] == float(v), (n, f)


def test_patchify_vectorised_equals_loops_and_roundtrip():
    g = np.random.default_rng(1)
    lat = g.standard_normal((16, 10, 14)).astype(F32)
    tok = O.patchify(lat)
    np.testing.assert_array_equal(tok, O.patchify_loops(lat))
    np.testing.assert_array_equal(O.unpatchify(tok, 16, 10, 14), lat)


def test_patchify_is_a_permutation():
    lat = _value_latent(16, 4, 6)
    tok = O.patchify(lat)
    assert sorted(tok.ravel().tolist()) == sorted(lat.ravel().tolist())


# ---------------------------------------------------------------- position ids
def test_position_ids_image_then_caption():
    p = O.position_ids("joint", 2, 3, 32)
    assert p.shape == (6 + 32, 3)
    assert p[:6].tolist() == [[0, 0, 0], [0, 0, 1], [0, 0, 2], [0, 1, 0], [0, 1, 1], [0, 1, 2]]
    assert p[6].tolist() == [1, 0, 0] and p[6 + 31].tolist() == [32, 0, 0]
    # image ids do not depend on the caption length (each branch has its own caption part)
    np.testing.assert_array_equal(O.position_ids("image", 2, 3, 32), O.position_ids("image", 2, 3, 64))


# ---------------------------------------------------------------- RoPE
def _rand_qk(S, nh, hd, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal((S, nh, hd)).astype(F32)


def test_rope_real_form_equals_complex_rotation():
    """Real interleaved form == complex rotation (x0 + i x1) e^{i phi}."""
    pos = np.array([[0, 3, 5], [1, 0, 0], [7, 2, 9], [40, 0, 0], [0, 63, 63]])
    x = _rand_qk(len(pos), 2, 128, 3)
    cos, sin = O.rope_tables(pos)
    # in float64 (tables recomputed in float64 through the same definition) the forms agree
    y64 = O.rope_apply(x.astype(np.float64), cos.astype(np.float64), sin.astype(np.float64))
    yc = O.rope_apply_complex(x, pos)
    # tables are fp32-rounded, so the angle differs by <= 2^-24 relative
    np.testing.assert_allclose(y64, yc, rtol=0, atol=4e-7 * np.abs(x).max() * 2)
    # in fp32: within a few ulp of the exact complex product
    y32 = O.rope_apply(x, cos, sin)
    np.testing.assert_allclose(y32, yc, rtol=0, atol=2e-6 * np.abs(x).max())


def test_rope_matches_torch_complex64():
    """Library check: torch's view_as_complex rotation by cos + i sin (the form the real
    form replaced) agrees with the real form to within one rounding."""
    pos = O.position_ids("joint", 4, 4, 32)
    x = _rand_qk(len(pos), 3, 128, 4)
    cos, sin = O.rope_tables(pos)
    xc = torch.view_as_complex(torch.from_numpy(x).reshape(len(pos), 3, 64, 2).contiguous())
    fc = torch.complex(torch.from_numpy(cos), torch.from_numpy(sin))[:, None, :]
    yt = torch.view_as_real(xc * fc).reshape(len(pos), 3, 128).numpy()
    y = O.rope_apply(x, cos, sin)
    np.testing.assert_allclose(y, yt, rtol=0, atol=1e-6 * np.abs(x).max())


def test_rope_relative_position_identity():
    """<R_m q, R_n k> depends only on m - n on each axis (textbook RoPE property)."""
    g = np.random.default_rng(5)
    q = g.standard_normal((1, 1, 128))
    k = g.standard_normal((1, 1, 128))

    def dot(m, n):
        cm, sm = O.rope_tables(np.array([m]))
        cn, sn = O.rope_tables(np.array([n]))
        a = O.rope_apply(q, cm.astype(np.float64), sm.astype(np.float64))
        b = O.rope_apply(k, cn.astype(np.float64), sn.astype(np.float64))
        return float((a * b).sum())

    base = dot([3, 4, 5], [1, 1, 2])
    assert abs(dot([13, 14, 15], [11, 11, 12]) - base) < 1e-5 * (1 + abs(base))
    assert abs(dot([4, 4, 5], [1, 1, 2]) - base) > 1e-3  # a different offset changes it


def test_rope_axes_own_their_dims():
    """Axis 0 turns dims 0..31, axis 1 dims 32..79, axis 2 dims 80..127."""
    x = np.ones((1, 1, 128), dtype=np.float64)
    for axis, lo, hi in [(0, 0, 32), (1, 32, 80), (2, 80, 128)]:
        pos = np.zeros((1, 3), dtype=np.int64)
        pos[0, axis] = 7
        c, s = O.rope_tables(pos)
        y = O.rope_apply(x, c.astype(np.float64), s.astype(np.float64))[0, 0]
        moved = np.nonzero(np.abs(y - 1) > 1e-12)[0]
        assert moved.min() >= lo and moved.max() < hi
        # the fastest pair of each axis turns by exactly pos radians
        assert abs(y[lo] - (math.cos(7) - math.sin(7))) < 1e-6


def test_rope_frequencies_of_every_axis_hand_worked():
    """Frequencies of pairs k = 0..3 (and the last pair) of each axis against the hand-reduced
    powers of ten in tests/golden/rope_frequencies.txt: 10000^(-2k/32) = 10^(-k/4) on axis 0,
    10000^(-2k/48) = 10^(-k/6) on axes 1 and 2, at a position whose three coordinates differ."""
    pos = np.array([[5, 7, 11]])
    cos, sin = O.rope_tables(pos)
    assert cos.shape == (1, 64)
    for col, axis, k, num, den in golden("rope_frequencies.txt"):
        col, axis, num, den = int(col), int(axis), int(num), int(den)
        ang = float(pos[0, axis]) * 10.0 ** (-num / den)
        for got, want in ((cos[0, col], math.cos(ang)), (sin[0, col], math.sin(ang))):
            # the tables are fp32: within one fp32 ulp of the exact value
            assert abs(float(got) - want) <= np.spacing(np.float32(abs(want))), (col, axis, k)


def test_rope_zero_position_is_identity():
    x = _rand_qk(5, 2, 128, 6)
    c, s = O.rope_tables(np.zeros((5, 3), dtype=np.int64))
    np.testing.assert_array_equal(O.rope_apply(x, c, s), x)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_form_with_outliers():
    g = np.random.default_rng(7)
    x = g.standard_normal((6, 3840)).astype(F32)
    x[:, ::997] = 6.7e3
    x[2, 5] = -6.7e3
    gain = (1 + 0.02 * g.standard_normal(3840)).astype(F32)
    y = O.rmsnorm(x, gain, 1e-6)
    x64 = x.astype(np.float64)
    ref = np.empty_like(x64)
    for i in range(6):
        r = math.sqrt(math.fsum(v * v for v in x64[i]) / 3840 + 1e-6)
        ref[i] = x64[i] / r * gain
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-7)


def test_rmsnorm_scale_invariance_and_unit_rms():
    g = np.random.default_rng(8)
    x = g.standard_normal((4, 384))
    one = np.ones(384)
    y = O.rmsnorm(x, one, 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(axis=1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(O.rmsnorm(1000 * x, one, 0.0), y, rtol=1e-12)


# ---------------------------------------------------------------- attention
def test_attention_brute_force_float64():
    g = np.random.default_rng(9)
    q, k, v = (g.standard_normal((12, 2, 128)).astype(F32) for _ in range(3))
    ref = O.attention_brute(q, k, v)
    got = O.attention(q, k, v)
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-6)


def test_attention_identical_keys_average_values():
    g = np.random.default_rng(10)
    q = g.standard_normal((7, 2, 128))
    k = np.tile(g.standard_normal((1, 2, 128)), (7, 1, 1))
    v = g.standard_normal((7, 2, 128))
    np.testing.assert_allclose(O.attention(q, k, v), np.broadcast_to(v.mean(axis=0), (7, 2, 128)),
                               rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- timestep embedding
def test_timestep_embedding_closed_forms():
    e0 = O.timestep_embedding(np.array([0.0]), 256)
    np.testing.assert_array_equal(e0[0, :128], 1.0)
    np.testing.assert_array_equal(e0[0, 128:], 0.0)
    # frequency k = 0 is 1 rad per unit of 1000 t
    e = O.timestep_embedding(np.array([0.5]), 256, dtype=np.float64)
    assert abs(e[0, 0] - math.cos(500.0)) < 1e-12 and abs(e[0, 128] - math.sin(500.0)) < 1e-12
    # the last frequency is 10000^(-127/128)
    f = 10000 ** (-127 / 128)
    assert abs(e[0, 127] - math.cos(500 * f)) < 1e-12


def test_t_condition_closed_form_mlp():
    """Timestep MLP with coordinate weights: W1 = a I, W2 = g P for a non-symmetric permutation
    P (row j reads column pi(j)), so c_j = g SiLU(a e_pi(j) + b1_pi(j)) + b2_j on the already
    pinned sinusoid e.  Pins the SiLU between the two linears, which linear comes first, W2's
    orientation and both biases."""
    dims = synth.TINY
    n = dims.c_dim
    assert dims.t_freq == n
    g = np.random.default_rng(60)
    a, gm = 1.7, -0.6
    pi = np.roll(np.arange(n), 5)  # pi(j) = j - 5 mod n
    P = np.zeros((n, n))
    P[np.arange(n), pi] = 1.0
    ew = {"t_w1": a * np.eye(n), "t_b1": g.standard_normal(n), "t_w2": gm * P, "t_b2": g.standard_normal(n)}
    t = np.array([0.3, 0.85])
    c = O.t_condition(t, ew, dims, dtype=np.float64)
    e = O.timestep_embedding(t, dims.t_freq, dims.t_scale, dtype=np.float64)
    for b in range(2):
        for j in range(n):
            z = a * e[b, pi[j]] + ew["t_b1"][pi[j]]
            want = gm * (z / (1.0 + math.exp(-z))) + ew["t_b2"][j]
            assert abs(c[b, j] - want) < 1e-12 * (1 + abs(want)), (b, j)


# ---------------------------------------------------------------- block-level invariants
def _tiny_block(seed=11, S=40):
    dims = synth.TINY
    w = synth.block_weights(dims, seed, 0, adaln=True)
    g = np.random.default_rng(seed)
    x = g.standard_normal((S, dims.dim)).astype(F32)
    pos = O.position_ids("joint", 2, 4, S - 8)
    cos, sin = O.rope_tables(pos)
    c = g.standard_normal(dims.c_dim).astype(F32)
    return dims, w, x, cos, sin, c, pos


def test_block_zero_adaln_is_identity():
    dims, w, x, cos, sin, c, _ = _tiny_block()
    w = dict(w, w_ada=np.zeros_like(w["w_ada"]), b_ada=np.zeros_like(w["b_ada"]))
    mod = O.block_mod(c, w)
    assert np.all(mod == 0)
    np.testing.assert_array_equal(O.block(x, w, mod, cos, sin, dims), x)


def test_block_shift_scale_zero_gate_one_equals_context_refiner_block():
    dims, w, x, cos, sin, c, _ = _tiny_block()
    d = dims.dim
    mod = np.zeros((6, d), dtype=F32)
    mod[2] = 1
    mod[5] = 1
    np.testing.assert_array_equal(O.block(x, w, mod, cos, sin, dims), O.block(x, w, None, cos, sin, dims))


def test_block_mod_chunk_order():
    """W_ada = 0 makes the modulation the bias b_ada, read as six chunks (shift1, scale1, gate1,
    shift2, scale2, gate2).  One chunk at a time: only the gates move x (chunk 2 through the
    attention branch, chunk 5 through the FFN); a scale chunk of -1 with a zero shift zeroes its
    branch's normed input (so its update vanishes) while a shift chunk of -1 does not."""
    dims, w, x, cos, sin, c, _ = _tiny_block(S=24)
    d = dims.dim
    w = dict(w, w_ada=np.zeros_like(w["w_ada"]))

    def update(chunks, **wover):
        b = np.zeros(6 * d, dtype=F32)
        for i, v in chunks.items():
            b[i * d:(i + 1) * d] = v
        ww = dict(w, b_ada=b, **wover)
        return O.block(x, ww, O.block_mod(c, ww), cos, sin, dims) - x

    for i in (0, 1, 3, 4):  # shift / scale alone, both gates 0
        assert np.all(update({i: 0.5}) == 0), i
    # chunk 2 gates the attention branch: dead with W_out = 0, alive otherwise
    assert np.abs(update({2: 1.0})).max() > 1e-3
    assert np.all(update({2: 1.0}, w_out=np.zeros_like(w["w_out"])) == 0)
    # chunk 5 gates the FFN: dead with W3 = 0, alive otherwise
    assert np.abs(update({5: 1.0})).max() > 1e-3
    assert np.all(update({5: 1.0}, w3=np.zeros_like(w["w3"])) == 0)
    # scale chunks: -1 zeroes the modulated input (h = 0 -> q = k = v = 0, u = 0)
    assert np.all(update({2: 1.0, 1: -1.0}) == 0)
    assert np.abs(update({2: 1.0, 0: -1.0})).max() > 1e-3
    assert np.all(update({5: 1.0, 4: -1.0}) == 0)
    assert np.abs(update({5: 1.0, 3: -1.0})).max() > 1e-3


def test_block_w3_zero_kills_ffn():
    dims, w, x, cos, sin, c, _ = _tiny_block()
    w = dict(w, w3=np.zeros_like(w["w3"]))
    mod = O.block_mod(c, w)
    mod[2] = 0  # attention gate off too -> identity
    np.testing.assert_array_equal(O.block(x, w, mod, cos, sin, dims), x)


def test_block_permutation_equivariance():
    """Permuting tokens together with their position ids permutes the output."""
    dims, w, x, cos, sin, c, _ = _tiny_block(S=24)
    x = x.astype(np.float64)
    mod = O.block_mod(c, w, np.float64)
    perm = np.random.default_rng(12).permutation(24)
    y = O.block(x, w, mod, cos, sin, dims)
    yp = O.block(x[perm], w, mod, cos[perm], sin[perm], dims)
    np.testing.assert_allclose(yp, y[perm], rtol=1e-10, atol=1e-10)


def test_block_translation_invariance_of_positions():
    """Shifting every token's position on one axis changes nothing (relative RoPE) — fails
    if RoPE reaches v, or q and k see different tables."""
    dims, w, x, cos, sin, c, pos = _tiny_block(S=24)
    x = x.astype(np.float64)
    mod = O.block_mod(c, w, np.float64)
    c0, s0 = (a.astype(np.float64) for a in O.rope_tables(pos))
    for axis in range(3):
        sh = pos.copy()
        sh[:, axis] += 17
        c1, s1 = (a.astype(np.float64) for a in O.rope_tables(sh))
        np.testing.assert_allclose(O.block(x, w, mod, c1, s1, dims), O.block(x, w, mod, c0, s0, dims),
                                   rtol=1e-5, atol=1e-6)


def test_block_identical_tokens_stay_identical():
    """All tokens equal at one position -> attention returns v for every row, so every
    output row is the same."""
    dims, w, x, cos, sin, c, _ = _tiny_block(S=16)
    x = np.tile(x[:1].astype(np.float64), (16, 1))
    z = np.zeros((16, 3), dtype=np.int64)
    c0, s0 = O.rope_tables(z)
    y = O.block(x, w, O.block_mod(c, w, np.float64), c0.astype(np.float64), s0.astype(np.float64), dims)
    np.testing.assert_allclose(y, np.tile(y[:1], (16, 1)), rtol=1e-12, atol=1e-12)
    assert np.abs(y - x).max() > 1e-3


def _mod(d, shift1=0.0, scale1=0.0, gate1=1.0, shift2=0.0, scale2=0.0, gate2=1.0):
    m = np.zeros((6, d), dtype=np.float64)
    for i, v in enumerate((shift1, scale1, gate1, shift2, scale2, gate2)):
        m[i] = v
    return m


def _eye(rows, cols):
    e = np.zeros((rows, cols))
    n = min(rows, cols)
    e[np.arange(n), np.arange(n)] = 1
    return e


def test_block_ffn_reduces_to_coordinatewise_swiglu():
    """Attention off (gate1 = 0), shift2 = scale2 = 0, W1 = a E, W3 = b E, W2 = E^T with E the
    coordinate embedding: the update is SiLU(a h2) * (b h2) per coordinate, h2 = RMSNorm(x; g2).
    Pins SiLU on the W1 branch, the W3 product, W2's orientation, the second norm's gain and
    the FFN gate."""
    dims = synth.TINY
    d, H = dims.dim, dims.ffn_hidden
    g = np.random.default_rng(50)
    w = synth.block_weights(dims, 50, 0)
    E = _eye(H, d)
    w = dict(w, w1=1.5 * E, w3=-0.7 * E, w2=np.ascontiguousarray(E.T))
    x = g.standard_normal((5, d))
    pos = np.zeros((5, 3), dtype=np.int64)
    c, s = (a.astype(np.float64) for a in O.rope_tables(pos))
    y = O.block(x, w, _mod(d, gate1=0.0, gate2=0.8), c, s, dims)
    for i in range(5):
        r = math.sqrt(sum(v * v for v in x[i]) / d + dims.norm_eps)
        for j in range(0, d, 37):
            h2 = x[i, j] / r * w["norm2"][j]
            a = 1.5 * h2
            want = x[i, j] + 0.8 * (a / (1 + math.exp(-a))) * (-0.7 * h2)
            assert abs(y[i, j] - want) < 1e-9 * (1 + abs(want)), (i, j)


def test_block_scale_minus_one_makes_input_the_shift():
    """scale = -1 turns the normed input into the shift vector alone: every token then sees the
    same h, so the attention update is identical on every row."""
    dims, w, x, cos, sin, c, _ = _tiny_block(S=12)
    d = dims.dim
    g = np.random.default_rng(51)
    sh = g.standard_normal(d)
    y = O.block(x.astype(np.float64), w, _mod(d, shift1=sh, scale1=-1.0, gate2=0.0),
                np.ones_like(cos, dtype=np.float64), np.zeros_like(sin, dtype=np.float64), dims)
    upd = y - x
    np.testing.assert_allclose(upd, np.tile(upd[:1], (12, 1)), rtol=1e-10, atol=1e-12)
    assert np.abs(upd).max() > 1e-3


def _attn_only_block(dims, wq=None, wk=None, wv=None, seed=52):
    """Block with the FFN off, W_out = identity, gate1 = 1, no modulation: update = attention out."""
    d = dims.dim
    w = synth.block_weights(dims, seed, 0)
    qkv = w["w_qkv"].astype(np.float64).copy()
    for sl, m in ((slice(0, d), wq), (slice(d, 2 * d), wk), (slice(2 * d, 3 * d), wv)):
        if m is not None:
            qkv[sl] = m
    return dict(w, w_qkv=qkv, w_out=np.eye(d), norm1=np.ones(d))


def test_block_value_slice_is_the_third_block_of_rows():
    dims, _, x, cos, sin, c, _ = _tiny_block(S=12)
    d = dims.dim
    w = _attn_only_block(dims, wv=np.zeros((d, d)))
    y = O.block(x.astype(np.float64), w, _mod(d, gate2=0.0), cos.astype(np.float64), sin.astype(np.float64), dims)
    np.testing.assert_array_equal(y, x.astype(np.float64))


def test_block_zero_query_or_key_gives_mean_of_values():
    """W_q = 0 or W_k = 0 makes every score 0: each token's attention output is the mean of
    v = RMSNorm(x) W_v^T over the sequence, placed head by head in model dims."""
    dims, _, x, cos, sin, c, _ = _tiny_block(S=12)
    d = dims.dim
    x = x.astype(np.float64)
    for which in ("q", "k"):
        w = _attn_only_block(dims, **{"w" + which: np.zeros((d, d))})
        y = O.block(x, w, _mod(d, gate2=0.0), cos.astype(np.float64), sin.astype(np.float64), dims)
        hn = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + dims.norm_eps)
        v = hn @ w["w_qkv"][2 * d:3 * d].T
        np.testing.assert_allclose(y - x, np.tile(v.mean(axis=0), (12, 1)), rtol=1e-9, atol=1e-10)


def test_block_query_and_key_roles_are_not_swapped():
    """k constant over tokens, q varying: softmax over keys is uniform, so the update is the
    same on every row.  With the roles swapped the rows would differ."""
    dims = synth.TINY
    d = dims.dim
    g = np.random.default_rng(53)
    half = d // 2
    base = g.standard_normal(d - half)
    x = np.empty((10, d))
    for i in range(10):
        x[i, :half] = 0.5
        x[i, half:] = g.permutation(base)            # same norm, different content
    wq = np.zeros((d, d)); wq[:, half:] = g.standard_normal((d, d - half))
    wk = np.zeros((d, d)); wk[:, :half] = g.standard_normal((d, half))
    w = _attn_only_block(dims, wq=wq, wk=wk)
    z = np.zeros((10, 64))
    y = O.block(x, w, _mod(d, gate2=0.0), z + 1, z, dims)
    hn = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + dims.norm_eps)
    v = hn @ w["w_qkv"][2 * d:3 * d].T
    np.testing.assert_allclose(y - x, np.tile(v.mean(axis=0), (10, 1)), rtol=1e-9, atol=1e-10)


def test_block_query_heads_are_contiguous_slices():
    """Queries living only in head 1's rows of W_q: heads 0 and 2 score every key 0 and return
    the mean of v; head 1 does not."""
    dims, _, x, cos, sin, c, _ = _tiny_block(S=12)
    d = dims.dim
    g = np.random.default_rng(55)
    wq = np.zeros((d, d)); wq[128:256] = g.standard_normal((128, d))
    w = _attn_only_block(dims, wq=wq)
    x = x.astype(np.float64)
    y = O.block(x, w, _mod(d, gate2=0.0), cos.astype(np.float64), sin.astype(np.float64), dims)
    hn = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + dims.norm_eps)
    mv = np.tile((hn @ w["w_qkv"][2 * d:3 * d].T).mean(axis=0), (12, 1))
    upd = y - x
    np.testing.assert_allclose(upd[:, :128], mv[:, :128], rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(upd[:, 256:], mv[:, 256:], rtol=1e-9, atol=1e-10)
    assert np.abs(upd[:, 128:256] - mv[:, 128:256]).max() > 1e-4


def test_block_heads_are_contiguous_slices():
    """Values living only in head 1's rows of W_v (dims 128..255) come out only in dims
    128..255 of the attention output."""
    dims, _, x, cos, sin, c, _ = _tiny_block(S=12)
    d = dims.dim
    g = np.random.default_rng(54)
    wv = np.zeros((d, d)); wv[128:256] = g.standard_normal((128, d))
    w = _attn_only_block(dims, wv=wv)
    y = O.block(x.astype(np.float64), w, _mod(d, gate2=0.0), cos.astype(np.float64), sin.astype(np.float64), dims)
    upd = np.abs(y - x)
    assert upd[:, 128:256].min() > 0 and upd[:, :128].max() == 0 and upd[:, 256:].max() == 0


def test_silu_values():
    for v, want in ((0.0, 0.0), (1.0, 0.7310585786300049), (-1.0, -0.2689414213699951), (20.0, 19.999999958776925)):
        assert abs(O.silu(np.float64(v)) - want) < 1e-14


# ---------------------------------------------------------------- stack wiring
def _tiny_model(seed=20, n_main=2):
    dims = synth.TINY.replace(n_main=n_main)
    W = synth.model_weights(dims, seed)
    return dims, W


def _gate_off(bw):
    return dict(bw, w_ada=np.zeros_like(bw["w_ada"]), b_ada=np.zeros_like(bw["b_ada"]))


def test_stack_caption_reaches_image_only_through_main_blocks():
    dims, W = _tiny_model()
    g = np.random.default_rng(21)
    lat = g.standard_normal((16, 8, 8)).astype(F32)
    cap = g.standard_normal((40, dims.cap_dim)).astype(F32)
    v1 = O.stack(lat, cap, 20, 0.5, W, dims)
    v2 = O.stack(lat, cap * 2, 20, 0.5, W, dims)
    assert np.abs(v1 - v2).max() > 1e-4          # joint attention sees the caption
    W2 = dict(W, main=[_gate_off(b) for b in W["main"]])
    u1 = O.stack(lat, cap, 20, 0.5, W2, dims)
    u2 = O.stack(lat, cap * 2, 33, 0.5, W2, dims)
    np.testing.assert_array_equal(u1, u2)         # main blocks off: caption is invisible


def test_stack_learned_pad_is_attention_context():
    """Changing the learned pad vector changes the velocity (pads are not masked); a caption
    of exactly 32 tokens has no pads, so the pad vector is then invisible."""
    dims, W = _tiny_model()
    g = np.random.default_rng(22)
    lat = g.standard_normal((16, 8, 8)).astype(F32)
    cap = g.standard_normal((40, dims.cap_dim)).astype(F32)
    W2 = dict(W, cap_pad=W["cap_pad"] + 1)
    assert np.abs(O.stack(lat, cap, 20, 0.5, W, dims) - O.stack(lat, cap, 20, 0.5, W2, dims)).max() > 1e-5
    np.testing.assert_array_equal(O.stack(lat, cap, 32, 0.5, W, dims), O.stack(lat, cap, 32, 0.5, W2, dims))


def test_stack_with_all_blocks_off_is_embed_norm_project():
    """Every block off, the final modulation off, x-embed and the final projection chosen as
    coordinate maps: velocity = latent scaled per token by 1/sqrt(sum of its 64 features^2 / d + eps)."""
    dims, W = _tiny_model()
    d = dims.dim
    W = dict(W)
    W["noise_ref"] = [_gate_off(b) for b in W["noise_ref"]]
    W["main"] = [_gate_off(b) for b in W["main"]]
    W["ctx_ref"] = [dict(b, w_out=np.zeros_like(b["w_out"]), w2=np.zeros_like(b["w2"])) for b in W["ctx_ref"]]
    W["final_ada_w"] = np.zeros_like(W["final_ada_w"])
    W["final_ada_b"] = np.zeros_like(W["final_ada_b"])
    W["final_norm"] = np.ones(d, dtype=F32)
    ex = np.zeros((d, 64), dtype=F32)
    ex[np.arange(64) * 5, np.arange(64)] = 1      # feature f -> model dim 5f
    W["x_emb_w"], W["x_emb_b"] = ex, np.zeros(d, dtype=F32)
    W["final_w"], W["final_b"] = np.ascontiguousarray(ex.T), np.zeros(64, dtype=F32)
    g = np.random.default_rng(23)
    lat = g.standard_normal((16, 6, 10)).astype(np.float64)
    cap = g.standard_normal((20, dims.cap_dim))
    v = O.stack(lat, cap, 20, 0.5, W, dims, dtype=np.float64)
    want = np.empty_like(lat)
    for r in range(3):
        for cc in range(5):
            blk = lat[:, 2 * r:2 * r + 2, 2 * cc:2 * cc + 2]
            want[:, 2 * r:2 * r + 2, 2 * cc:2 * cc + 2] = blk / math.sqrt((blk * blk).sum() / d + dims.norm_eps)
    np.testing.assert_allclose(v, want, rtol=1e-9, atol=1e-12)
    # final modulation: first half of Linear(SiLU(c)) is the shift, second half the scale
    fb = np.zeros(2 * d)
    fb[:d] = 0.25
    fb[d:] = 0.5
    W["final_ada_b"] = fb
    v2 = O.stack(lat, cap, 20, 0.5, W, dims, dtype=np.float64)
    np.testing.assert_allclose(v2, want * 1.5 + 0.25, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- sampler
def test_sigmas_exact_rationals():
    sg = O.sigmas(8, 3.0)
    assert sg.dtype == np.float32 and len(sg) == 9
    for i, num, den in golden("sigmas_8_steps.txt"):
        assert sg[int(i)] == np.float32(float(Fraction(int(num), int(den)))), i
    assert sg[0] == 1.0 and sg[-1] == 0.0
    assert np.all(np.diff(sg) < 0)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 20, 50])
def test_sigmas_endpoints_any_step_count(n):
    sg = O.sigmas(n, 3.0)
    assert len(sg) == n + 1 and sg[0] == 1.0 and sg[-1] == 0.0 and np.all(np.diff(sg) < 0)
    # shift 1 gives the plain linear schedule 1 - i/n
    np.testing.assert_allclose(O.sigmas(n, 1.0), 1 - np.arange(n + 1) / n, rtol=0, atol=1e-7)


def test_cfg_worked_values():
    for row in golden("cfg_euler_unscale.txt"):
        if row[0] == "cfg":
            pos, neg, g, want = map(float, row[1:])
            assert O.cfg_noise_pred(np.array([pos]), np.array([neg]), g)[0] == np.float32(want)


def test_cfg_special_cases():
    g = np.random.default_rng(30)
    vc = g.standard_normal(100).astype(F32)
    vu = g.standard_normal(100).astype(F32)
    np.testing.assert_array_equal(O.cfg_noise_pred(vc, vu, 0.0), -vc)
    np.testing.assert_array_equal(O.cfg_noise_pred(vc, vc, 3.7), -vc)
    np.testing.assert_array_equal(O.cfg_noise_pred(vc, None, 0.0), -vc)
    # not the textbook neg + g (pos - neg)
    assert not np.allclose(O.cfg_noise_pred(vc, vu, 1.0), vu + (vc - vu))


def test_unscale_worked_values():
    for row in golden("cfg_euler_unscale.txt"):
        if row[0] == "unscale":
            z, want = float(row[1]), float(row[2])
            got = O.unscale(np.array([z], dtype=F32))[0]
            assert abs(float(got) - want) <= 2 * abs(np.spacing(np.float32(want)))


def test_euler_constant_velocity_telescopes():
    """DiT stubbed to a constant u: x_8 = x_0 + u (sigma_0 - sigma_8) = x_0 + u."""
    g = np.random.default_rng(31)
    x0 = g.standard_normal(1000).astype(F32)
    u = g.standard_normal(1000).astype(F32)
    calls = []

    def dit(x, branch, t):
        calls.append((branch, float(t)))
        return u

    xn, dec = O.sample(x0, dit, num_steps=8, shift=3.0, guidance=1.0)
    np.testing.assert_allclose(xn, x0 + u, rtol=0, atol=8e-7 * (1 + np.abs(x0).max() + np.abs(u).max()))
    # 8 calls per branch, 16 with CFG, none at sigma = 0 (t = 1)
    assert len(calls) == 16 and sum(1 for b, _ in calls if b == 1) == 8
    ts = sorted({t for _, t in calls})
    assert len(ts) == 8 and max(ts) < 1.0 and min(ts) == 0.0
    # the decode output is the raw latent unscaled once
    np.testing.assert_array_equal(dec, O.unscale(xn))


def test_guidance_zero_skips_uncond_branch():
    calls = []

    def dit(x, branch, t):
        calls.append(branch)
        return np.ones_like(x)

    O.sample(np.zeros(4, dtype=F32), dit, num_steps=8, guidance=0.0)
    assert calls == [0] * 8


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_round_matches_torch():
    g = np.random.default_rng(40)
    x = np.concatenate([g.standard_normal(100000).astype(F32) * 1e3,
                        np.array([0.0, -0.0, 1.0, 3e5, -6.7e3, 1e-40, np.inf, -np.inf], dtype=F32)])
    # exact ties: values whose low 16 bits are 0x8000
    ties = (g.integers(0, 2 ** 15, 1000, dtype=np.uint32) << 17 | 0x3F808000).view(F32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(O.bf16_round(x), want)
