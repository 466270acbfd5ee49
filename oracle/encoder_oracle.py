"""Oracle for the text encoder that produces the S3-DiT caption features: a plain, slow,
obviously correct CPU implementation in NumPy of a Qwen3-shaped decoder stack read out at
its penultimate hidden state.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg
may import this module.  It shares no code with the HIP library or its Python binding, and
imports neither.

What the pages fix (FastVideo "Z-Image Port Status": the pinned encoder's summary and the
component matrix; Core AI model zoo "Z-Image-Turbo port", table "Architecture -> export
mapping", row Text encoder, and "The three things that each cost a wrong image", item 1):
a causal decoder of 36 blocks, hidden 2560, intermediate 9728, 32 query heads sharing 8
key/value heads (grouped-query attention), head dimension 128, fused q/k/v and gate/up
projections with SiLU gating, token embedding inside the graph, an additive causal and
non-padding mask over right-padded ids, and the DiT reading hidden_states[-2] of the valid
tokens (37 hidden states: the embedding, then one per block).

Readings where the pages are silent (each is listed with its reason in the design notes):
  E1  block structure of the published Qwen3 decoder: pre-norm RMSNorm (learned gain,
      eps 1e-6) before attention and before the MLP, an RMSNorm with a learned gain over
      each query head and each key head (before RoPE), no biases, attention scale
      1/sqrt(128), residual adds after attention and after the MLP.
  E2  RoPE pairs dimension i with dimension i + 64 of a head (the published Qwen3 layout),
      angle pos * theta^(-2i/128) with theta 1e6, position = token index from 0; tables
      computed in float64 and stored as fp32.
  E3  hidden_states[-2] is the residual stream after the first n_layers - 1 blocks, without
      the final norm (that norm only enters the last hidden state); the last block's
      weights do not affect it.
  E4  padding: each branch is computed on its valid tokens only; rows past a branch's length
      are zero in the output.
Parity unpinned: the output against the real encoder weights (none are available); only the
pins in tests/ fix this module.
"""
from __future__ import annotations

import math

import numpy as np

from .zdit_oracle import F32, linear, rmsnorm, silu


def embed(ids: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Rows of the embedding table selected by the token ids (the graph's embed_tokens)."""
    return table[np.asarray(ids, dtype=np.int64)].astype(table.dtype)


def rope_tables_1d(n_pos: int, head_dim: int = 128, theta: float = 1.0e6):
    """cos, sin [n_pos, head_dim/2] fp32 of the angles pos * theta^(-2i/head_dim), pos from 0
    (reading E2), computed in float64."""
    half = head_dim // 2
    inv = np.power(np.float64(theta), -2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def rope_rotate_half(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate dimension pairs (i, i + hd/2) of every head of x [S, nh, hd] by the row's
    angles (reading E2): y_i = x_i c - x_{i+hd/2} s, y_{i+hd/2} = x_{i+hd/2} c + x_i s.  Each
    product and each sum is rounded separately (NumPy does not fuse)."""
    half = x.shape[-1] // 2
    c = cos[:, None, :].astype(x.dtype)
    s = sin[:, None, :].astype(x.dtype)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_rotate_half_complex(x: np.ndarray, pos: np.ndarray, theta: float = 1.0e6) -> np.ndarray:
    """The same rotation written as complex multiplication, in float64: the pair
    (x_i, x_{i+hd/2}) is the complex number x_i + j x_{i+hd/2} turned by e^{j pos w_i}."""
    hd = x.shape[-1]
    half = hd // 2
    w = np.power(float(theta), -2.0 * np.arange(half) / hd)
    z = x[..., :half].astype(np.float64) + 1j * x[..., half:].astype(np.float64)
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[:, None, None] * w[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


def head_norm(x: np.ndarray, gain: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the head dimension of x [S, nh, hd] with one gain vector [hd] shared by
    the heads (reading E1)."""
    return rmsnorm(x, gain, eps)


def causal_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(hd) + causal mask) v with grouped key/value heads.

    q [S, nq, hd]; k, v [S, nkv, hd]; query head h reads key/value head h // (nq / nkv)
    (consecutive query heads share one key/value head).  Query i sees keys 0..i only (Core
    AI page, row Text encoder: additive causal and non-padding mask; the padding part never
    arises here because each branch is computed on its valid tokens).
    """
    S, nq, hd = q.shape
    nkv = k.shape[1]
    group = nq // nkv
    scale = q.dtype.type(1.0 / math.sqrt(hd))
    future = np.triu(np.ones((S, S), dtype=bool), 1)
    out = np.empty_like(q)
    for h in range(nq):
        hk = h // group
        s = (q[:, h, :] @ k[:, hk, :].T) * scale
        s = np.where(future, -np.inf, s)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, hk, :]
    return out


def causal_gqa_attention_brute(q, k, v):
    """Float64 loops over the definition (tiny inputs only)."""
    S, nq, hd = q.shape
    group = nq // k.shape[1]
    out = np.zeros((S, nq, hd), dtype=np.float64)
    for h in range(nq):
        hk = h // group
        for i in range(S):
            sc = [sum(float(q[i, h, e]) * float(k[j, hk, e]) for e in range(hd)) / math.sqrt(hd)
                  for j in range(i + 1)]
            mx = max(sc)
            ex = [math.exp(z - mx) for z in sc]
            tot = sum(ex)
            for e in range(hd):
                out[i, h, e] = sum(ex[j] * float(v[j, hk, e]) for j in range(i + 1)) / tot
    return out


def encoder_block(x: np.ndarray, w: dict, cos: np.ndarray, sin: np.ndarray, ed) -> np.ndarray:
    """One decoder block on one branch's valid rows x [L, hidden] (reading E1)."""
    L = x.shape[0]
    hd, nq, nkv = ed.head_dim, ed.n_heads, ed.n_kv_heads
    eps = ed.norm_eps
    h = rmsnorm(x, w["in_norm"], eps)
    qkv = linear(h, w["w_qkv"])
    q = qkv[:, :nq * hd].reshape(L, nq, hd)
    k = qkv[:, nq * hd:(nq + nkv) * hd].reshape(L, nkv, hd)
    v = qkv[:, (nq + nkv) * hd:].reshape(L, nkv, hd)
    q = rope_rotate_half(head_norm(q, w["q_norm"], eps), cos, sin)
    k = rope_rotate_half(head_norm(k, w["k_norm"], eps), cos, sin)
    o = causal_gqa_attention(q, k, v).reshape(L, nq * hd)
    x = x + linear(o, w["w_o"])
    h2 = rmsnorm(x, w["post_norm"], eps)
    u = silu(linear(h2, w["w_gate"])) * linear(h2, w["w_up"])
    return x + linear(u, w["w_down"])


def encoder_hidden_states(ids_row: np.ndarray, W: dict, ed, n_blocks: int, dtype=F32,
                          pos0: int = 0) -> list:
    """Hidden states of one branch's valid ids [L]: the embedding, then the residual stream
    after each of the first n_blocks blocks (n_blocks + 1 arrays [L, hidden]).  pos0 shifts
    every position (used only by the relative-position pin)."""
    L = len(ids_row)
    cos, sin = rope_tables_1d(pos0 + L, ed.head_dim, ed.rope_theta)
    cos, sin = cos[pos0:], sin[pos0:]
    x = embed(ids_row, W["embed"]).astype(dtype)
    hs = [x]
    for i in range(n_blocks):
        x = encoder_block(x, W["layers"][i], cos, sin, ed)
        hs.append(x)
    return hs


def encoder_penultimate(ids: np.ndarray, lengths, W: dict, ed, dtype=F32) -> np.ndarray:
    """hidden_states[-2] of every branch (reading E3): [B, L_max, hidden], rows at or past a
    branch's length zero (reading E4)."""
    B, L_max = ids.shape
    out = np.zeros((B, L_max, ed.hidden), dtype=dtype)
    for b in range(B):
        L = int(lengths[b])
        out[b, :L] = encoder_hidden_states(ids[b, :L], W, ed, ed.n_layers - 1, dtype)[-1]
    return out
