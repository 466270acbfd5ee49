"""Pins of the text-encoder oracle against what the pages and the mathematics fix (CPU only).

Each test names the fact it pins: closed forms, invariants, brute force on tiny inputs, or
a library routine (torch's attention, RMSNorm and complex arithmetic on the CPU).  None
re-types an oracle formula.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import encoder_oracle as E

F32 = np.float32
ED = synth.ENC_TINY


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- RoPE (pairs i, i + 64)
def test_rope_rotate_half_equals_complex_rotation():
    g = _rng(1)
    x = g.standard_normal((37, 3, 128))
    pos = np.arange(37)
    cos, sin = E.rope_tables_1d(37, 128, 1e6)
    got = E.rope_rotate_half(x.astype(F32), cos, sin)
    want = E.rope_rotate_half_complex(x, pos, 1e6)
    np.testing.assert_allclose(got, want, rtol=0, atol=2e-5)


def test_rope_tables_match_torch_polar():
    """The fp32 tables are the float64 angles rounded once: compare with torch in float64."""
    n, hd, theta = 300, 128, 1e6
    cos, sin = E.rope_tables_1d(n, hd, theta)
    inv = torch.pow(torch.tensor(theta, dtype=torch.float64), -torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = torch.arange(n, dtype=torch.float64)[:, None] * inv[None, :]
    z = torch.polar(torch.ones_like(ang), ang)
    np.testing.assert_array_equal(cos, z.real.to(torch.float32).numpy())
    np.testing.assert_array_equal(sin, z.imag.to(torch.float32).numpy())


def test_rope_relative_position_identity():
    """<R_m q, R_n k> depends only on m - n (textbook RoPE), in float64."""
    g = _rng(2)
    q, k = g.standard_normal((1, 1, 128)), g.standard_normal((1, 1, 128))
    vals = []
    for m, n in [(5, 2), (13, 10), (403, 400)]:
        rq = E.rope_rotate_half_complex(q, np.array([m]))
        rk = E.rope_rotate_half_complex(k, np.array([n]))
        vals.append(float(np.sum(rq * rk)))
    assert max(vals) - min(vals) < 1e-9 * max(1.0, abs(vals[0]))


def test_rope_pairs_are_half_apart():
    """A vector with only dim i (< 64) set turns within the plane of dims i and i + 64."""
    cos, sin = E.rope_tables_1d(8, 128, 1e6)
    for i in (0, 5, 63):
        x = np.zeros((8, 1, 128), F32)
        x[:, 0, i] = 1.0
        y = E.rope_rotate_half(x, cos, sin)
        others = np.delete(y, [i, i + 64], axis=-1)
        assert np.all(others == 0)
        np.testing.assert_allclose(y[:, 0, i] ** 2 + y[:, 0, i + 64] ** 2, 1.0, atol=1e-6)
        assert y[3, 0, i + 64] != 0 or i == 63 and abs(sin[3, i]) < 1e-30


def test_rope_position_zero_is_identity():
    g = _rng(3)
    x = g.standard_normal((1, 4, 128)).astype(F32)
    cos, sin = E.rope_tables_1d(1)
    np.testing.assert_array_equal(E.rope_rotate_half(x, cos, sin), x)


# ---------------------------------------------------------------- norms
def test_head_norm_matches_torch_rms_norm():
    g = _rng(4)
    x = g.standard_normal((11, 4, 128)).astype(np.float64) * 3.0
    gain = 1.0 + 0.1 * g.standard_normal(128)
    got = E.head_norm(x, gain, 1e-6)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(gain), eps=1e-6).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_head_norm_heads_are_independent():
    g = _rng(5)
    x = g.standard_normal((3, 4, 128)).astype(F32)
    gain = np.ones(128, F32)
    y1 = E.head_norm(x, gain)
    x2 = x.copy()
    x2[:, 1, :] *= 50.0
    x2[:, 2, :] += 7.0
    y2 = E.head_norm(x2, gain)
    np.testing.assert_array_equal(y1[:, 0], y2[:, 0])
    np.testing.assert_array_equal(y1[:, 3], y2[:, 3])
    np.testing.assert_allclose(y2[:, 1], y1[:, 1], rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------- causal GQA attention
def _qkv(g, S, nq, nkv, scale=1.0):
    q = (g.standard_normal((S, nq, 128)) * scale).astype(F32)
    k = (g.standard_normal((S, nkv, 128)) * scale).astype(F32)
    v = g.standard_normal((S, nkv, 128)).astype(F32)
    return q, k, v


def test_causal_gqa_brute_force_float64():
    g = _rng(6)
    q, k, v = _qkv(g, 9, 4, 2)
    got = E.causal_gqa_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    np.testing.assert_allclose(got, E.causal_gqa_attention_brute(q, k, v), rtol=1e-10, atol=1e-12)
    got32 = E.causal_gqa_attention(q, k, v)
    np.testing.assert_allclose(got32, E.causal_gqa_attention_brute(q, k, v), rtol=2e-5, atol=2e-6)


def test_causal_gqa_matches_torch_sdpa():
    """torch's attention with is_causal and grouped heads (CPU, float64) as the library
    routine: its grouping repeats each key/value head over consecutive query heads."""
    g = _rng(7)
    q, k, v = _qkv(g, 40, 8, 2, scale=2.0)
    got = E.causal_gqa_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    t = lambda a: torch.from_numpy(a.astype(np.float64)).permute(1, 0, 2)[None]
    want = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(got, want[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_first_query_sees_only_first_key():
    g = _rng(8)
    q, k, v = _qkv(g, 6, 4, 2, scale=3.0)
    o = E.causal_gqa_attention(q, k, v)
    for h in range(4):
        np.testing.assert_array_equal(o[0, h], v[0, h // 2])


def test_zero_queries_average_the_visible_values():
    """q = 0 makes every visible key equally likely: o_i = mean(v_0..v_i)."""
    g = _rng(9)
    q, k, v = _qkv(g, 12, 4, 1)
    q[:] = 0
    o = E.causal_gqa_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    for i in range(12):
        np.testing.assert_allclose(o[i, 2], v[:i + 1, 0].astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-12)


def test_future_keys_change_nothing():
    g = _rng(10)
    q, k, v = _qkv(g, 10, 4, 2)
    o1 = E.causal_gqa_attention(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[6:] = 100.0
    v2[6:] = -50.0
    o2 = E.causal_gqa_attention(q, k2, v2)
    np.testing.assert_array_equal(o1[:6], o2[:6])
    assert not np.array_equal(o1[6:], o2[6:])


# ---------------------------------------------------------------- block and stack
def _weights(n_layers=3, seed=0, ed=ED):
    return synth.encoder_weights(ed, seed, n_layers)


def test_block_zero_output_projections_is_identity():
    W = _weights(1)
    w = dict(W["layers"][0])
    w["w_o"] = np.zeros_like(w["w_o"])
    w["w_down"] = np.zeros_like(w["w_down"])
    x = _rng(11).standard_normal((7, ED.hidden)).astype(F32)
    cos, sin = E.rope_tables_1d(7)
    np.testing.assert_array_equal(E.encoder_block(x, w, cos, sin, ED), x)


def test_block_is_causal_row_by_row():
    W = _weights(1)
    g = _rng(12)
    x = g.standard_normal((9, ED.hidden)).astype(F32)
    cos, sin = E.rope_tables_1d(9)
    y1 = E.encoder_block(x, W["layers"][0], cos, sin, ED)
    x2 = x.copy()
    x2[5:] = g.standard_normal((4, ED.hidden)).astype(F32) * 10
    y2 = E.encoder_block(x2, W["layers"][0], cos, sin, ED)
    np.testing.assert_array_equal(y1[:5], y2[:5])


def test_stack_depends_on_relative_positions_only():
    """Shifting every position by the same offset changes nothing (RoPE on q and k with the
    same tables), in float64 arithmetic on the fp32 tables (whose rounding bounds the
    agreement)."""
    ed = ED.replace(n_layers=2)
    W = _weights(2, seed=1)
    ids = synth.token_ids(1, 11, [11], ed.vocab, 3)[0]
    a = E.encoder_hidden_states(ids, W, ed, 2, dtype=np.float64)[-1]
    b = E.encoder_hidden_states(ids, W, ed, 2, dtype=np.float64, pos0=1000)[-1]
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6)


def test_stack_positions_matter():
    """Two tokens swapped change the output of the later rows (RoPE is present)."""
    W = _weights(1, seed=2)
    ids = synth.token_ids(1, 6, [6], ED.vocab, 4)[0]
    sw = ids.copy()
    sw[[1, 2]] = sw[[2, 1]]
    a = E.encoder_hidden_states(ids, W, ED, 1)[-1]
    b = E.encoder_hidden_states(sw, W, ED, 1)[-1]
    assert not np.allclose(a[3:], b[3:], rtol=1e-4, atol=1e-4)


def test_hidden_states_count_and_embedding_entry():
    W = _weights(3)
    ids = synth.token_ids(1, 8, [8], ED.vocab, 5)[0]
    hs = E.encoder_hidden_states(ids, W, ED, 3)
    assert len(hs) == 4
    np.testing.assert_array_equal(hs[0], W["embed"][ids])


def test_penultimate_ignores_last_block_and_padding():
    """hidden_states[-2] uses n_layers - 1 blocks: the last block's weights do not matter;
    rows past each length are zero; a branch does not depend on the other or on L_max."""
    W = _weights(3)
    lens = [7, 3]
    ids = synth.token_ids(2, 9, lens, ED.vocab, 6)
    a = E.encoder_penultimate(ids, lens, W, ED)
    W2 = {"embed": W["embed"], "layers": W["layers"][:2] + [_weights(1, seed=9)["layers"][0]]}
    np.testing.assert_array_equal(a, E.encoder_penultimate(ids, lens, W2, ED))
    assert np.all(a[0, 7:] == 0) and np.all(a[1, 3:] == 0)
    wider = np.zeros((2, 16), np.int32)
    wider[:, :9] = ids
    b = E.encoder_penultimate(wider, lens, W, ED)
    np.testing.assert_array_equal(a, b[:, :9])
    one = E.encoder_penultimate(ids[1:], lens[1:], W, ED)
    np.testing.assert_array_equal(one[0], a[1])
    hs = E.encoder_hidden_states(ids[0, :7], W, ED, 2)
    np.testing.assert_array_equal(a[0, :7], hs[-1])


def test_gqa_group_mapping_in_block():
    """Query heads 0 and 1 share key/value head 0 in the block: giving query head 1 the
    weights of query head 0 makes their attention outputs identical."""
    W = _weights(1, seed=3)
    w = dict(W["layers"][0])
    hd = ED.head_dim
    wq = w["w_qkv"].copy()
    wq[hd:2 * hd] = wq[:hd]
    w["w_qkv"] = wq
    x = _rng(13).standard_normal((6, ED.hidden)).astype(F32)
    cos, sin = E.rope_tables_1d(6)
    L = 6
    h = E.rmsnorm(x, w["in_norm"], ED.norm_eps)
    qkv = E.linear(h, w["w_qkv"])
    nq, nkv = ED.n_heads, ED.n_kv_heads
    q = E.rope_rotate_half(E.head_norm(qkv[:, :nq * hd].reshape(L, nq, hd), w["q_norm"]), cos, sin)
    k = E.rope_rotate_half(E.head_norm(qkv[:, nq * hd:(nq + nkv) * hd].reshape(L, nkv, hd), w["k_norm"]), cos, sin)
    v = qkv[:, (nq + nkv) * hd:].reshape(L, nkv, hd)
    o = E.causal_gqa_attention(q, k, v)
    np.testing.assert_array_equal(o[:, 0], o[:, 1])
    assert not np.allclose(o[:, 0], o[:, 2])


# ---------------------------------------------------------------- published implementation
def _hf_model(W, ed, n_layers):
    """transformers' Qwen3 decoder (CPU, float64) loaded with the same weights: the library
    routine that fixes readings E1-E3 (block structure, RoPE pairing and base, what
    hidden_states[-2] holds)."""
    from transformers import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import Qwen3Model
    cfg = Qwen3Config(vocab_size=ed.vocab, hidden_size=ed.hidden, intermediate_size=ed.inter,
                      num_hidden_layers=n_layers, num_attention_heads=ed.n_heads,
                      num_key_value_heads=ed.n_kv_heads, head_dim=ed.head_dim, rope_theta=ed.rope_theta,
                      rms_norm_eps=ed.norm_eps, attention_bias=False)
    m = Qwen3Model(cfg).double().eval()
    hd, nq, nkv = ed.head_dim, ed.n_heads * ed.head_dim, ed.n_kv_heads * ed.head_dim
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    sd = {"embed_tokens.weight": T(W["embed"]), "norm.weight": torch.ones(ed.hidden, dtype=torch.float64)}
    for i in range(n_layers):
        w, p = W["layers"][i], f"layers.{i}."
        sd[p + "self_attn.q_proj.weight"] = T(w["w_qkv"][:nq])
        sd[p + "self_attn.k_proj.weight"] = T(w["w_qkv"][nq:nq + nkv])
        sd[p + "self_attn.v_proj.weight"] = T(w["w_qkv"][nq + nkv:])
        sd[p + "self_attn.o_proj.weight"] = T(w["w_o"])
        sd[p + "self_attn.q_norm.weight"] = T(w["q_norm"])
        sd[p + "self_attn.k_norm.weight"] = T(w["k_norm"])
        sd[p + "mlp.gate_proj.weight"] = T(w["w_gate"])
        sd[p + "mlp.up_proj.weight"] = T(w["w_up"])
        sd[p + "mlp.down_proj.weight"] = T(w["w_down"])
        sd[p + "input_layernorm.weight"] = T(w["in_norm"])
        sd[p + "post_attention_layernorm.weight"] = T(w["post_norm"])
    m.load_state_dict(sd, strict=True)
    return m


def test_stack_matches_published_qwen3_hidden_states():
    n = 3
    W = _weights(n, seed=4)
    lens = [13, 6]
    ids = synth.token_ids(2, 16, lens, ED.vocab, 7)
    m = _hf_model(W, ED, n)
    mask = torch.tensor([[1] * L + [0] * (16 - L) for L in lens])
    with torch.no_grad():
        out = m(input_ids=torch.from_numpy(ids.astype(np.int64)), attention_mask=mask, output_hidden_states=True)
    hs_ref = [h.numpy() for h in out.hidden_states]
    assert len(hs_ref) == n + 1
    for b, L in enumerate(lens):
        hs = E.encoder_hidden_states(ids[b, :L], W, ED, n, dtype=np.float64)
        for i in range(n):  # the embedding and the un-normed block outputs
            np.testing.assert_allclose(hs[i], hs_ref[i][b, :L], rtol=2e-6, atol=2e-6)
    # the DiT's input: hidden_states[-2] of the valid tokens
    pen = E.encoder_penultimate(ids, lens, W, ED.replace(n_layers=n), dtype=np.float64)
    for b, L in enumerate(lens):
        np.testing.assert_allclose(pen[b, :L], hs_ref[-2][b, :L], rtol=2e-6, atol=2e-6)
