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
}


@pytest.fixture(scope="module")
def sandbox(tmp_path_factory):
    d = tmp_path_factory.mktemp("oracle_mut")
    for sub in ("oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(d, sub),
                        ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(d, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    return str(d)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(sandbox, name):
    src_path = os.path.join(ROOT, "oracle", "zdit_oracle.py")
    src = open(src_path).read()
    a, b = MUTATIONS[name]
    assert src.count(a) >= 1, f"mutation anchor not found: {name}"
    with open(os.path.join(sandbox, "oracle", "zdit_oracle.py"), "w") as f:
        f.write(src.replace(a, b, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=sandbox, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0, f"pins did not catch: {name}"
