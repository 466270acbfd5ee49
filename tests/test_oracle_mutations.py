"""Plants plausible mistakes in a temporary copy of the oracle (CPU only) and checks that the
pin tests catch each one.  The repository's own oracle is never modified."""
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

MUTATIONS = {
    "modulation without the 1 +": ("return h * (1 + scale) + shift", "return h * scale + shift"),
    "q and k slices swapped": ("q = qkv[:, 0:d].reshape(S, nh, hd)\n    k = qkv[:, d:2 * d]",
                               "q = qkv[:, d:2 * d].reshape(S, nh, hd)\n    k = qkv[:, 0:d]"),
    "v taken from the q slice": ("v = qkv[:, 2 * d:3 * d]", "v = qkv[:, 0:d]"),
    "SwiGLU branches swapped": ('u = silu(linear(h2, w["w1"])) * linear(h2, w["w3"])',
                                'u = silu(linear(h2, w["w3"])) * linear(h2, w["w1"])'),
    "attention gate is the FFN gate": ('x = x + gate1 * linear(a, w["w_out"])', 'x = x + gate2 * linear(a, w["w_out"])'),
    "no 1/sqrt(hd) scale": ("s = (q[:, h, :] @ k[:, h, :].T) * scale", "s = (q[:, h, :] @ k[:, h, :].T)"),
    "heads strided, not contiguous": ("q = qkv[:, 0:d].reshape(S, nh, hd)",
                                      "q = qkv[:, 0:d].reshape(S, hd, nh).transpose(0, 2, 1)"),
    "RoPE applied to v": ("a = attention(q, k, v)", "a = attention(q, k, rope_apply(v, cos, sin))"),
    "FFN norm uses the attention gain": ('rmsnorm(x, w["norm2"]', 'rmsnorm(x, w["norm1"]'),
    "SiLU sign": ("return x / (1 + np.exp(-x))", "return x / (1 + np.exp(x))"),
    "learned pad dropped": ('np.tile(W["cap_pad"]', 'np.tile(0 * W["cap_pad"]'),
    "final shift/scale swapped": ("shift_f, scale_f = final_mod(c, W, dtype)", "scale_f, shift_f = final_mod(c, W, dtype)"),
    "timestep sin/cos swapped": ("[np.cos(arg), np.sin(arg)]", "[np.sin(arg), np.cos(arg)]"),
    "RoPE sign": ("y0 = a - b", "y0 = a + b"),
    "RoPE pairs not adjacent": ("x0 = x[..., 0::2]\n    x1 = x[..., 1::2]",
                                "x0 = x[..., :x.shape[-1] // 2]\n    x1 = x[..., x.shape[-1] // 2:]"),
    "RMSNorm without eps": ("np.sqrt(ms + x.dtype.type(eps))", "np.sqrt(ms)"),
    "patchify dy/dx swapped": ("t = t.transpose(1, 3, 2, 4, 0)", "t = t.transpose(1, 3, 4, 2, 0)"),
    "sigma schedule unshifted": ("out[i] = shift * (1 - t) / (shift * (1 - t) + t)", "out[i] = 1 - t"),
    "textbook CFG": ("u = v_c + e\n    return -u", "u = np.asarray(v_u, dtype=F32) + e\n    return -u"),
    "Euler step sign": ("ds = F32(sigma_next) - F32(sigma)", "ds = F32(sigma) - F32(sigma_next)"),
    "unscale inverted": ("/ F32(0.3611) + F32(0.1159)", "* F32(0.3611) + F32(0.1159)"),
    "caption position ids from 0": ("cap[j] = (1 + j, 0, 0)", "cap[j] = (j, 0, 0)"),
    "n_cap rounds down": ("return multiple * math.ceil(L / multiple)", "return multiple * max(1, L // multiple)"),
    "SiLU dropped in the timestep MLP": ('hdn = silu(linear(e, ew["t_w1"], ew["t_b1"]))', 'hdn = linear(e, ew["t_w1"], ew["t_b1"])'),
    "timestep MLP linears swapped": ('hdn = silu(linear(e, ew["t_w1"], ew["t_b1"]))\n    return linear(hdn, ew["t_w2"], ew["t_b2"])',
                                     'hdn = silu(linear(e, ew["t_w2"], ew["t_b1"]))\n    return linear(hdn, ew["t_w1"], ew["t_b2"])'),
    "adaLN chunks reordered (shift/scale)": ("    return m.reshape(6, -1)\n", "    return m.reshape(6, -1)[[1, 0, 2, 4, 3, 5]]\n"),
    "adaLN chunks interleaved": ("    return m.reshape(6, -1)\n", "    return m.reshape(-1, 6).T\n"),
    "RoPE frequency theta^(-k/d)": ("omega = theta ** (-2.0 * k / da)", "omega = theta ** (-1.0 * k / da)"),
}


# planted in oracle/encoder_oracle.py, caught by tests/test_encoder_oracle_pins.py
ENC_MUTATIONS = {
    "GQA heads strided, not grouped": ("hk = h // group\n        s = (q[:, h, :]", "hk = h % nkv\n        s = (q[:, h, :]"),
    "no causal mask": ("s = np.where(future, -np.inf, s)", "s = s + 0"),
    "causal mask off by one": ("np.triu(np.ones((S, S), dtype=bool), 1)", "np.triu(np.ones((S, S), dtype=bool), 2)"),
    "no attention scale": ("s = (q[:, h, :] @ k[:, hk, :].T) * scale", "s = (q[:, h, :] @ k[:, hk, :].T)"),
    "RoPE pairs adjacent": ("x1, x2 = x[..., :half], x[..., half:]", "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    "RoPE sign": ("x1 * c - x2 * s", "x1 * c + x2 * s"),
    "RoPE base 1e4": ("rope_tables_1d(pos0 + L, ed.head_dim, ed.rope_theta)", "rope_tables_1d(pos0 + L, ed.head_dim, 10000.0)"),
    "q and k norm gains swapped": ('head_norm(q, w["q_norm"], eps), cos, sin)\n    k = rope_rotate_half(head_norm(k, w["k_norm"], eps)',
                                   'head_norm(q, w["k_norm"], eps), cos, sin)\n    k = rope_rotate_half(head_norm(k, w["q_norm"], eps)'),
    "no key norm": ('k = rope_rotate_half(head_norm(k, w["k_norm"], eps), cos, sin)', "k = rope_rotate_half(k, cos, sin)"),
    "v from the k slice": ("v = qkv[:, (nq + nkv) * hd:]", "v = qkv[:, nq * hd:(nq + nkv) * hd]"),
    "gate and up swapped": ('silu(linear(h2, w["w_gate"])) * linear(h2, w["w_up"])',
                            'silu(linear(h2, w["w_up"])) * linear(h2, w["w_gate"])'),
    "MLP norm uses the attention gain": ('rmsnorm(x, w["post_norm"], eps)', 'rmsnorm(x, w["in_norm"], eps)'),
    "penultimate reads the last block": ("ed.n_layers - 1, dtype)[-1]", "ed.n_layers, dtype)[-1]"),
}


# planted in oracle/vae_oracle.py, caught by tests/test_vae_oracle_pins.py
VAE_MUTATIONS = {
    "convolution instead of correlation": ("tap = w[:, :, i, j].astype(x.dtype)", "tap = w[:, :, k - 1 - i, k - 1 - j].astype(x.dtype)"),
    "no zero padding (wrap around)": ("win = xp[:, :, i:i + H, j:j + Wd]",
                                      "win = np.roll(np.roll(x, p - i, axis=2), p - j, axis=3)"),
    "conv bias dropped": ("return out + b.astype(x.dtype)[None, :, None, None]", "return out"),
    "GroupNorm groups strided": ("xg = x.reshape(B, groups, C // groups, H, Wd)",
                                 "xg = x.reshape(B, C // groups, groups, H, Wd).transpose(0, 2, 1, 3, 4)"),
    "GroupNorm statistics over the batch": ("mean = xg.mean(axis=(2, 3, 4), keepdims=True)",
                                            "mean = xg.mean(axis=(0, 2, 3, 4), keepdims=True)"),
    "GroupNorm eps outside the root": ("np.sqrt(var + x.dtype.type(eps))", "(np.sqrt(var) + x.dtype.type(eps))"),
    "SiLU dropped before conv1": ('h = conv2d(silu(group_norm(x, W[p + ".gn1.g"]', 'h = conv2d((group_norm(x, W[p + ".gn1.g"]'),
    "ResNet norms swapped": ('group_norm(h, W[p + ".gn2.g"], W[p + ".gn2.b"]', 'group_norm(h, W[p + ".gn1.g"], W[p + ".gn1.b"]'),
    "no shortcut": ("    return s + h\n", "    return h\n"),
    "upsample by interleaving channels": ("return np.repeat(np.repeat(x, 2, axis=2), 2, axis=3)",
                                          "return np.tile(x, (1, 1, 2, 2))"),
    "upsample after the conv": ("x = conv2d(upsample_nearest(x), W[f\"up{i}.upconv.w\"], W[f\"up{i}.upconv.b\"])",
                                "x = upsample_nearest(conv2d(x, W[f\"up{i}.upconv.w\"], W[f\"up{i}.upconv.b\"]))"),
    "attention without 1/sqrt(C)": ("s = (q[n] @ k[n].T) / dt.type(math.sqrt(C))", "s = (q[n] @ k[n].T)"),
    "attention q and k swapped with v": ('q, k, v = lin(t, "q"), lin(t, "k"), lin(t, "v")',
                                         'q, k, v = lin(t, "q"), lin(t, "v"), lin(t, "k")'),
    "attention softmax over queries": ("out[n] = (e / e.sum(axis=1, keepdims=True)) @ v[n]",
                                       "out[n] = (e / e.sum(axis=0, keepdims=True)) @ v[n]"),
    "attention residual dropped": ("return x + o.transpose(0, 2, 1).reshape(B, C, H, Wd)",
                                   "return o.transpose(0, 2, 1).reshape(B, C, H, Wd)"),
    "unscale inverted": ("return z / z.dtype.type(scale) + z.dtype.type(shift)",
                         "return (z - z.dtype.type(shift)) * z.dtype.type(scale)"),
    "no SiLU before conv_out": ('x = silu(group_norm(x, W["norm_out.g"]', 'x = (group_norm(x, W["norm_out.g"]'),
}


@pytest.fixture(scope="module")
def sandbox(tmp_path_factory):
    d = tmp_path_factory.mktemp("oracle_mut")
    for sub in ("oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(d, sub),
                        ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(d, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    for f in ("conftest.py", "test_oracle_pins.py", "test_encoder_oracle_pins.py", "test_vae_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    return str(d)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(sandbox, name):
    src_path = os.path.join(ROOT, "oracle", "zdit_oracle.py")
    src = open(src_path).read()
    a, b = MUTATIONS[name]
    assert src.count(a) >= 1, f"mutation anchor not found: {name}"
    dst = os.path.join(sandbox, "oracle", "zdit_oracle.py")
    try:
        with open(dst, "w") as f:
            f.write(src.replace(a, b, 1))
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "tests/test_oracle_pins.py"], cwd=sandbox, capture_output=True, text=True,
                           timeout=300)
    finally:
        with open(dst, "w") as f:
            f.write(src)
    assert r.returncode != 0, f"pins did not catch: {name}"


def test_sandbox_copy_passes_unmutated(sandbox):
    """The unmutated sandbox passes both pin files, so a failure below is the mutation's."""
    for f in ("tests/test_oracle_pins.py", "tests/test_encoder_oracle_pins.py", "tests/test_vae_oracle_pins.py"):
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", f],
                           cwd=sandbox, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(ENC_MUTATIONS))
def test_encoder_pins_catch_planted_mistake(sandbox, name):
    src_path = os.path.join(ROOT, "oracle", "encoder_oracle.py")
    src = open(src_path).read()
    a, b = ENC_MUTATIONS[name]
    assert src.count(a) >= 1, f"mutation anchor not found: {name}"
    dst = os.path.join(sandbox, "oracle", "encoder_oracle.py")
    try:
        with open(dst, "w") as f:
            f.write(src.replace(a, b, 1))
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "tests/test_encoder_oracle_pins.py"], cwd=sandbox, capture_output=True,
                           text=True, timeout=300)
    finally:
        with open(dst, "w") as f:
            f.write(src)
    assert r.returncode != 0, f"pins did not catch: {name}"


@pytest.mark.parametrize("name", sorted(VAE_MUTATIONS))
def test_vae_pins_catch_planted_mistake(sandbox, name):
    src_path = os.path.join(ROOT, "oracle", "vae_oracle.py")
    src = open(src_path).read()
    a, b = VAE_MUTATIONS[name]
    assert src.count(a) >= 1, f"mutation anchor not found: {name}"
    dst = os.path.join(sandbox, "oracle", "vae_oracle.py")
    try:
        with open(dst, "w") as f:
            f.write(src.replace(a, b, 1))
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "tests/test_vae_oracle_pins.py"], cwd=sandbox, capture_output=True,
                           text=True, timeout=300)
    finally:
        with open(dst, "w") as f:
            f.write(src)
    assert r.returncode != 0, f"pins did not catch: {name}"
