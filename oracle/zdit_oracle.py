"""Oracle for the Z-Image-Turbo S3-DiT hot path: a plain, slow, obviously correct CPU
implementation in NumPy.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg
may import this module.  It shares no code with the HIP library or its Python binding, and
imports neither.

Precision.  The pages measure every port against an fp32 reference run of the transformer
(Core AI model zoo, "Z-Image-Turbo port", sections "Numbers" and "Gates"), and the sampler
runs under an fp32 scalar contract (FastVideo "Z-Image Port Status", table "Parity Commands",
row Scheduler; and section "Pinned Official Pipeline Context", scheduler_contract).  So the
model math here runs in fp32 by default (``dtype=np.float64`` is accepted for self-checks),
and the sampler, RoPE and decode steps run in fp32 with every product and every sum rounded
separately (NumPy never fuses them).

Readings where the pages are silent (each is listed with its reason in the design notes):
  R1  one sequence per branch: image tokens (row-major grid) first, then caption tokens
      (pads included), then batch-alignment padding.
  R2  position ids: image token (r, c) -> (0, r, c); caption token j -> (1 + j, 0, 0).
  R3  RoPE axes of 32/48/48 dims at offsets 0/32/80 of the head; pair k of an axis is the
      adjacent dims (off + 2k, off + 2k + 1); frequency theta^(-2k / d_axis), theta 1e4;
      tables computed in float64 and stored as fp32.
  R4  the learned pad vector replaces caption rows L..n_cap-1 after cap-embed.
  R5  pre-norm block: RMSNorm (learned gain, eps 1e-6), adaLN (shift, scale, gate) x 2 from
      Linear(SiLU(c)), modulation h * (1 + scale) + shift, raw gates, no bias in the block
      linears, attention scale 1/sqrt(head_dim).
  R6  model time t = 1 - sigma; sinusoid [cos, sin] over 128 frequencies 1e4^(-k/128) of
      1000 t; MLP 256 -> 256 -> 256 with SiLU.
  R7  final layer: RMSNorm (gain) -> (1 + scale) / shift from Linear(SiLU(c)) -> Linear to
      the 64 patch features with bias.
  R9  learned caption pads are attention context; batch-alignment pad keys are masked and
      pad rows are left untouched.
Parity unpinned: the whole-model output against the real Z-Image weights (none are
available); only the pins in tests/ fix this module.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32


# --------------------------------------------------------------------------------------
# rounding helper (used only where a result is compared bit for bit with bf16 output)
# --------------------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value, ties to even; returns fp32.

    Definition of round-to-nearest-even on the fp32 bit pattern: add 0x7FFF plus the lowest
    kept bit, then clear the 16 low bits.  NaN stays NaN.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = r.view(F32).copy()
    nan = np.isnan(x)
    out[nan] = x[nan]
    return out


# --------------------------------------------------------------------------------------
# index work: caption padding, patchify, position ids
# --------------------------------------------------------------------------------------
def n_cap(L: int, multiple: int = 32) -> int:
    """Padded caption length: L rounded up to a multiple of 32.

    Core AI model zoo, "Z-Image-Turbo port", section "The three things that each cost a
    wrong image", item 3 (45 tokens -> 64; the empty negative -> 32).
    """
    if not (1 <= L <= 512):
        raise ValueError("caption length must be in 1..512")
    return multiple * math.ceil(L / multiple)


def patchify(lat: np.ndarray, p: int = 2) -> np.ndarray:
    """Latent [C, h, w] -> patch tokens [(h/p)(w/p), p*p*C].

    Token n = r * (w/p) + c covers latent pixels (p r + dy, p c + dx); its feature
    f = (dy * p + dx) * C + ch holds lat[ch, p r + dy, p c + dx].  Feature order from the
    Core AI page, section "Three more things" (host arithmetic re-implemented).
    """
    C, h, w = lat.shape
    assert h % p == 0 and w % p == 0
    t = lat.reshape(C, h // p, p, w // p, p)            # [ch, r, dy, c, dx]
    t = t.transpose(1, 3, 2, 4, 0)                       # [r, c, dy, dx, ch]
    return np.ascontiguousarray(t.reshape((h // p) * (w // p), p * p * C))


def patchify_loops(lat: np.ndarray, p: int = 2) -> np.ndarray:
    """Same as patchify, written as loops over the definition (small inputs only)."""
    C, h, w = lat.shape
    out = np.zeros(((h // p) * (w // p), p * p * C), dtype=lat.dtype)
    for r in range(h // p):
        for c in range(w // p):
            n = r * (w // p) + c
            for dy in range(p):
                for dx in range(p):
                    for ch in range(C):
                        out[n, (dy * p + dx) * C + ch] = lat[ch, p * r + dy, p * c + dx]
    return out


def unpatchify(tok: np.ndarray, C: int, h: int, w: int, p: int = 2) -> np.ndarray:
    """Inverse of patchify: tokens [(h/p)(w/p), p*p*C] -> [C, h, w]."""
    t = tok.reshape(h // p, w // p, p, p, C)              # [r, c, dy, dx, ch]
    t = t.transpose(4, 0, 2, 1, 3)                        # [ch, r, dy, c, dx]
    return np.ascontiguousarray(t.reshape(C, h, w))


def position_ids(kind: str, grid_h: int, grid_w: int, ncap: int) -> np.ndarray:
    """Integer 3-axis positions [S, 3] of one branch's tokens (reading R2).

    kind 'image': the grid_h x grid_w image tokens, row-major, token (r, c) -> (0, r, c).
    kind 'caption': ncap caption tokens, token j -> (1 + j, 0, 0).
    kind 'joint': image tokens then caption tokens (reading R1).
    """
    img = np.zeros((grid_h * grid_w, 3), dtype=np.int64)
    for r in range(grid_h):
        for c in range(grid_w):
            img[r * grid_w + c] = (0, r, c)
    cap = np.zeros((ncap, 3), dtype=np.int64)
    for j in range(ncap):
        cap[j] = (1 + j, 0, 0)
    if kind == "image":
        return img
    if kind == "caption":
        return cap
    if kind == "joint":
        return np.concatenate([img, cap], axis=0)
    raise ValueError(kind)


# --------------------------------------------------------------------------------------
# 3-axis rotary embedding
# --------------------------------------------------------------------------------------
def rope_tables(pos: np.ndarray, axes=(32, 48, 48), theta: float = 10000.0):
    """cos/sin tables [S, sum(axes)/2] for integer positions [S, 3] (reading R3).

    Column j enumerates the rotation pairs of the head in order: axis 0's pairs, then axis
    1's, then axis 2's.  Pair k of axis a turns by angle pos_a * theta^(-2k/d_a).  The
    angles and their cos/sin are computed in float64 and stored as fp32: the pages insist on
    fp32 RoPE buffers (FastVideo "Z-Image Port Status", issue I006) and on precomputed
    cos/sin (Core AI page, table "Architecture -> export mapping", row DiT).
    """
    cols = []
    for a, da in enumerate(axes):
        k = np.arange(da // 2, dtype=np.float64)
        omega = theta ** (-2.0 * k / da)
        cols.append(pos[:, a:a + 1].astype(np.float64) * omega[None, :])
    ang = np.concatenate(cols, axis=1)
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def rope_apply(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Real interleaved rotation of x [S, n_heads, hd] with tables [S, hd/2].

    For pair j (dims 2j, 2j+1): y0 = x0 c - x1 s, y1 = x0 s + x1 c, with every product and
    sum rounded in x's dtype (the "bit-exact real interleaved form" of the Core AI page,
    table "Architecture -> export mapping", row DiT).
    """
    dt = x.dtype
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    c = cos.astype(dt)[:, None, :]
    s = sin.astype(dt)[:, None, :]
    a = x0 * c
    b = x1 * s
    y0 = a - b
    e = x0 * s
    f = x1 * c
    y1 = e + f
    y = np.empty_like(x)
    y[..., 0::2] = y0
    y[..., 1::2] = y1
    return y


def rope_apply_complex(x: np.ndarray, pos: np.ndarray, axes=(32, 48, 48),
                       theta: float = 10000.0) -> np.ndarray:
    """The complex form the real form replaces: pair (x0, x1) as x0 + i x1 times e^{i phi},
    evaluated in complex128 (the definition; used only to check rope_apply)."""
    z = x[..., 0::2].astype(np.float64) + 1j * x[..., 1::2].astype(np.float64)
    cols = []
    for a, da in enumerate(axes):
        k = np.arange(da // 2, dtype=np.float64)
        cols.append(pos[:, a:a + 1].astype(np.float64) * (theta ** (-2.0 * k / da))[None, :])
    ang = np.concatenate(cols, axis=1)
    zr = z * np.exp(1j * ang)[:, None, :]
    y = np.empty(x.shape, dtype=np.float64)
    y[..., 0::2] = zr.real
    y[..., 1::2] = zr.imag
    return y


# --------------------------------------------------------------------------------------
# block pieces
# --------------------------------------------------------------------------------------
def silu(x):
    return x / (1 + np.exp(-x))


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis (reading R5)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + x.dtype.type(eps)) * gain.astype(x.dtype)


def modulate(h, shift, scale):
    """adaLN modulation h * (1 + scale) + shift (reading R5)."""
    return h * (1 + scale) + shift


def timestep_embedding(t: np.ndarray, dim: int = 256, t_scale: float = 1000.0,
                       max_period: float = 10000.0, dtype=F32) -> np.ndarray:
    """Sinusoidal embedding [B, dim] of model time t [B] (reading R6):
    [cos(tau f_k), sin(tau f_k)] for k < dim/2, f_k = max_period^(-k/(dim/2)), tau = 1000 t."""
    half = dim // 2
    k = np.arange(half, dtype=dtype)
    f = np.power(dtype(max_period), -k / dtype(half)).astype(dtype)
    tau = (np.asarray(t, dtype=dtype) * dtype(t_scale))[:, None]
    arg = tau * f[None, :]
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=1).astype(dtype)


def linear(x, w, b=None):
    """x @ w^T (+ b) with w stored [out, in]."""
    y = x @ w.T.astype(x.dtype)
    if b is not None:
        y = y + b.astype(x.dtype)
    return y


def t_condition(t, ew, dims, dtype=F32):
    """Conditioning vector c [B, c_dim] = W2 SiLU(W1 e + b1) + b2 of the timestep embed."""
    e = timestep_embedding(t, dims.t_freq, dims.t_scale, dtype=dtype)
    hdn = silu(linear(e, ew["t_w1"], ew["t_b1"]))
    return linear(hdn, ew["t_w2"], ew["t_b2"])


def final_mod(c_row, W, dtype=F32):
    """(shift_f, scale_f) [2, d] of the final layer = Linear(SiLU(c)) split in two (R7)."""
    m = linear(silu(c_row[None, :].astype(dtype)), W["final_ada_w"], W["final_ada_b"])[0]
    return m.reshape(2, -1)


def attention(q, k, v):
    """softmax(q k^T / sqrt(hd)) v per head, all keys visible.  q, k, v: [S, nh, hd].

    Joint attention over the whole single-stream sequence (Core AI page, table
    "Architecture -> export mapping", row DiT; gitdiagram "How tongyi-mai/z-image works",
    item 5).  The learned caption pads are ordinary keys here (Core AI page, "The three
    things...", item 3); batch-alignment padding never reaches this function because each
    branch is computed on its valid rows only.
    """
    S, nh, hd = q.shape
    out = np.empty_like(q)
    scale = q.dtype.type(1.0 / math.sqrt(hd))
    for h in range(nh):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
    return out


def attention_brute(q, k, v):
    """Float64 triple loop over the softmax definition (tiny inputs only)."""
    S, nh, hd = q.shape
    out = np.zeros((S, nh, hd), dtype=np.float64)
    for h in range(nh):
        for i in range(S):
            sc = [sum(float(q[i, h, e]) * float(k[j, h, e]) for e in range(hd)) / math.sqrt(hd)
                  for j in range(S)]
            mx = max(sc)
            ex = [math.exp(x - mx) for x in sc]
            z = sum(ex)
            for e in range(hd):
                out[i, h, e] = sum(ex[j] * float(v[j, h, e]) for j in range(S)) / z
    return out


def block(x, w, mod, cos, sin, dims, record=None):
    """One S3-DiT block on one branch's valid rows x [S, d] (reading R5).

    mod: [6, d] = (shift1, scale1, gate1, shift2, scale2, gate2), or None for a block without
    adaLN (context refiner): shift = scale = 0, gate = 1 (Core AI page, table "Architecture ->
    export mapping", row DiT: "2 context-refiner (no adaLN)").
    """
    dt = x.dtype
    S, d = x.shape
    nh, hd = dims.n_heads, dims.head_dim
    if mod is None:
        z = np.zeros(d, dtype=dt)
        o = np.ones(d, dtype=dt)
        shift1, scale1, gate1, shift2, scale2, gate2 = z, z, o, z, z, o
    else:
        shift1, scale1, gate1, shift2, scale2, gate2 = [m.astype(dt) for m in mod]
    h = modulate(rmsnorm(x, w["norm1"], dims.norm_eps), shift1, scale1)
    qkv = linear(h, w["w_qkv"])
    q = qkv[:, 0:d].reshape(S, nh, hd)
    k = qkv[:, d:2 * d].reshape(S, nh, hd)
    v = qkv[:, 2 * d:3 * d].reshape(S, nh, hd)
    q = rope_apply(q, cos, sin)
    k = rope_apply(k, cos, sin)
    a = attention(q, k, v).reshape(S, d)
    x = x + gate1 * linear(a, w["w_out"])
    h2 = modulate(rmsnorm(x, w["norm2"], dims.norm_eps), shift2, scale2)
    u = silu(linear(h2, w["w1"])) * linear(h2, w["w3"])
    ffn = linear(u, w["w2"])
    if record is not None:
        record["ffn_out"] = ffn
    x = x + gate2 * ffn
    return x


def block_mod(c_row, w, dtype=F32):
    """adaLN vectors [6, d] of one branch from its conditioning row c_row [c_dim]."""
    if w.get("w_ada") is None:
        return None
    m = linear(silu(c_row[None, :].astype(dtype)), w["w_ada"], w["b_ada"])[0]
    return m.reshape(6, -1)


# --------------------------------------------------------------------------------------
# full stack for one branch
# --------------------------------------------------------------------------------------
def stack(lat, cap, cap_len, t, W, dims, dtype=F32, record=None):
    """DiT forward of one branch: latent [C, h, w] fp32, caption features [>= L, cap_dim],
    caption length L, model time t -> velocity [C, h, w].

    x-embed + cap-embed, 2 noise-refiner blocks on the image tokens, 2 context-refiner
    blocks on the caption tokens, 30 main blocks on the concatenated sequence, final layer
    and unpatchify (Core AI page, table "Architecture -> export mapping", row DiT).
    """
    C, h, w_ = lat.shape
    p = dims.patch
    gh, gw = h // p, w_ // p
    nimg = gh * gw
    nc = n_cap(cap_len, dims.seq_multiple)
    lat = lat.astype(dtype)
    cap = cap.astype(dtype)

    c = t_condition(np.array([t], dtype=dtype), W, dims, dtype)[0]

    x_img = linear(patchify(lat, p), W["x_emb_w"], W["x_emb_b"])
    e = linear(cap[:cap_len], W["cap_emb_w"], W["cap_emb_b"])
    x_cap = np.concatenate([e, np.tile(W["cap_pad"].astype(dtype)[None, :], (nc - cap_len, 1))], axis=0)

    axes, th = dims.rope_axes, dims.rope_theta
    cos_i, sin_i = rope_tables(position_ids("image", gh, gw, nc), axes, th)
    cos_c, sin_c = rope_tables(position_ids("caption", gh, gw, nc), axes, th)
    cos_j, sin_j = rope_tables(position_ids("joint", gh, gw, nc), axes, th)

    for bw in W["noise_ref"]:
        x_img = block(x_img, bw, block_mod(c, bw, dtype), cos_i, sin_i, dims)
    for bw in W["ctx_ref"]:
        x_cap = block(x_cap, bw, None, cos_c, sin_c, dims)
    x = np.concatenate([x_img, x_cap], axis=0)
    if record is not None:
        record["c"] = c.copy()
        record["main_in"] = x.copy()
    for i, bw in enumerate(W["main"]):
        x = block(x, bw, block_mod(c, bw, dtype), cos_j, sin_j, dims)
        if record is not None:
            record.setdefault("main", []).append(x.copy())
    shift_f, scale_f = final_mod(c, W, dtype)
    hf = modulate(rmsnorm(x[:nimg], W["final_norm"], dims.norm_eps), shift_f, scale_f)
    out = linear(hf, W["final_w"], W["final_b"])
    return unpatchify(out, C, h, w_, p)


# --------------------------------------------------------------------------------------
# sampler
# --------------------------------------------------------------------------------------
def sigmas(num_steps: int, shift: float = 3.0) -> np.ndarray:
    """num_steps + 1 sigmas, sigma_i = s(1 - t)/(s(1 - t) + t) with t = i / num_steps.

    Closed form of the shifted FlowMatchEuler schedule (Core AI page, section "Three more
    things": t = i/(n-1) over the n = num_steps + 1 points); endpoint-preserving with a
    zero final sigma (FastVideo "Z-Image Port Status", scheduler_contract).  Float64, stored
    fp32.
    """
    out = np.empty(num_steps + 1, dtype=np.float64)
    for i in range(num_steps + 1):
        t = i / num_steps
        out[i] = shift * (1 - t) / (shift * (1 - t) + t)
    return out.astype(F32)


def cfg_noise_pred(v_c, v_u, g):
    """Negated classifier-free guidance, -(pos + g (pos - neg)), in fp32 with the order
    d = pos - neg; e = g d; u = pos + e; result -u (Core AI page, "The three things...",
    item 2).  v_u None means the single-branch case, -pos."""
    v_c = np.asarray(v_c, dtype=F32)
    if v_u is None:
        return -v_c
    dd = v_c - np.asarray(v_u, dtype=F32)
    e = F32(g) * dd
    u = v_c + e
    return -u


def euler_update(x, noise_pred, sigma, sigma_next):
    """x + (sigma_next - sigma) * noise_pred in fp32, product and sum rounded separately."""
    ds = F32(sigma_next) - F32(sigma)
    return np.asarray(x, dtype=F32) + ds * np.asarray(noise_pred, dtype=F32)


def unscale(z):
    """Decode un-scaling z / 0.3611 + 0.1159 in fp32 (FastVideo "Z-Image Port Status",
    decode_contract; Core AI page, section "Three more things": apply it once)."""
    return np.asarray(z, dtype=F32) / F32(0.3611) + F32(0.1159)


def sample(x0, dit, num_steps=8, shift=3.0, guidance=1.0, record=None):
    """The 8-step negated-CFG FlowMatchEuler loop.

    dit(x, branch, t) -> velocity; branch 0 = cond, 1 = uncond.  With guidance 0 the uncond
    branch is never evaluated.  No call is made at the final sigma = 0 (FastVideo "Z-Image
    Port Status", scheduler_contract).  Returns (raw final latent, unscaled latent).
    """
    sg = sigmas(num_steps, shift)
    x = np.asarray(x0, dtype=F32).copy()
    for i in range(num_steps):
        t = F32(1.0) - sg[i]
        v_c = dit(x, 0, t)
        v_u = dit(x, 1, t) if guidance != 0 else None
        npred = cfg_noise_pred(v_c, v_u, guidance)
        x = euler_update(x, npred, sg[i], sg[i + 1])
        if record is not None:
            record.setdefault("x", []).append(x.copy())
            record.setdefault("v_c", []).append(np.asarray(v_c, dtype=F32).copy())
            if v_u is not None:
                record.setdefault("v_u", []).append(np.asarray(v_u, dtype=F32).copy())
    return x, unscale(x)
