"""Expected values of the VAE decoder at the workloads' full sizes (calls only the oracle and
the seeded input generators).

The 16-channel AutoencoderKL decoder (Core AI model zoo, "Z-Image-Turbo port", table
"Architecture -> export mapping", row VAE: fp32, the raw latent fed in, the unscale inside) on
one seeded latent per resolution: 128 x 128 (the 1024x1024 image) and 192 x 128 (1536x1024),
with the full-width seeded decoder weights.  The oracle runs in fp32, the precision the page
fixes for this component.

Writes, per resolution, tests/golden/vae_<name>.npz with
  idx        65536 seeded flat indices into the image [3 * H * W]
  val        the image at those indices (fp32)
  ch_mean    per-channel mean of the whole image (float64)
  ch_rms     per-channel root-mean-square of the whole image (float64)
and the sha256 of each file into tests/golden/vae_expected.sha256.  The GPU test regenerates the
same weights and latent from the seeds and compares.  Run from the repository root (about 15
minutes of fp32 work on 8 cores, ~40 GB of memory at 1536x1024):
    python tests/golden/make_vae_expected.py
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import synth  # noqa: E402
from oracle import vae_oracle as V  # noqa: E402

N_IDX = 65536
SEED = 42


def cases():
    return {"1024x1024": (128, 128), "1536x1024": (192, 128)}


def inputs(lat_h, lat_w):
    vd = synth.VAE_FULL
    return vd, synth.vae_weights(vd, SEED), synth.latents((vd.latent_ch, lat_h, lat_w), SEED)[None]


def sample_idx(n):
    return np.sort(np.random.default_rng(np.random.SeedSequence([SEED, 77])).choice(n, N_IDX, replace=False))


def make(name, lat_h, lat_w):
    vd, W, z = inputs(lat_h, lat_w)
    t0 = time.perf_counter()
    img = V.decoder(z, W, vd, dtype=np.float32)[0]
    print(f"{name}: decoder {time.perf_counter() - t0:.1f} s, image {img.shape}", flush=True)
    idx = sample_idx(img.size)
    flat = img.reshape(-1)
    out = os.path.join(HERE, f"vae_{name}.npz")
    np.savez_compressed(out, idx=idx.astype(np.int64), val=flat[idx].astype(np.float32),
                        ch_mean=img.astype(np.float64).mean(axis=(1, 2)),
                        ch_rms=np.sqrt((img.astype(np.float64) ** 2).mean(axis=(1, 2))))
    return out


def main():
    lines = []
    for name, (h, w) in cases().items():
        p = make(name, h, w)
        lines.append(f"{hashlib.sha256(open(p, 'rb').read()).hexdigest()}  {os.path.basename(p)}")
    with open(os.path.join(HERE, "vae_expected.sha256"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
