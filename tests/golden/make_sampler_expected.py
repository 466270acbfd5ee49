"""Expected values of the full-width 8-step sampler at reduced depth (calls only the oracle and the
seeded input generators).

The 8-step negated-CFG FlowMatchEuler pass (Core AI model zoo, "Z-Image-Turbo port", table
"Architecture -> export mapping", row Sampler: 8 steps, guidance 1.0; FastVideo "Z-Image Port
Status", scheduler_contract) at 1024x1024 and at 1536x1024, with the full-width model (dim
3840, 30 heads) cut to 2 noise-refiner + 2 context-refiner + 2 main blocks: the full depth would
cost the fp32 oracle about 890 and 1420 TFLOP, which this CPU-side reference cannot afford.
The oracle's sampler runs the stack on both branches at every step (16 calls).

Writes, per resolution, tests/golden/sampler_<name>.npz with
  x_final   the raw final latent [16, h, w] (fp32)
  idx       16384 seeded flat indices into a velocity [16 * h * w]
  v_c, v_u  the cond / uncond velocities of every step at those indices [8, 16384] (fp32)
and the sha256 of each file into tests/golden/sampler_expected.sha256.  The GPU test regenerates
the same weights, latents and captions from the seeds and compares.  Run from the repository
root (about 10 minutes of fp32 work on 8 cores):
    python tests/golden/make_sampler_expected.py
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle as O  # noqa: E402
import synth  # noqa: E402

N_MAIN = 2
N_IDX = 16384


def cases():
    return {"1024x1024": synth.CFG5, "1536x1024": synth.CFG5_WIDE}


def make(name, wl):
    dims = wl.dims.replace(n_main=N_MAIN)
    W = synth.model_weights(dims, wl.seed)
    lat = synth.latents((dims.latent_ch, wl.lat_h, wl.lat_w), wl.seed)
    Lmax = max(wl.cap_len)
    cap = synth.caption_features(2, Lmax, dims.cap_dim, wl.seed)
    n = lat.size
    idx = np.sort(np.random.default_rng(np.random.SeedSequence([wl.seed, 99])).choice(n, N_IDX, replace=False))

    def dit(x, branch, t):
        t0 = time.perf_counter()
        v = O.stack(x, cap[branch], wl.cap_len[branch], t, W, dims)
        print(f"  {name} branch {branch} t={float(t):.4f}: {time.perf_counter() - t0:.1f} s", flush=True)
        return v

    rec = {}
    x, _ = O.sample(lat, dit, num_steps=wl.num_steps, shift=wl.shift, guidance=wl.guidance, record=rec)
    out = os.path.join(HERE, f"sampler_{name}.npz")
    np.savez(out, x_final=x.astype(np.float32), idx=idx.astype(np.int64),
             v_c=np.stack([v.reshape(-1)[idx] for v in rec["v_c"]]).astype(np.float32),
             v_u=np.stack([v.reshape(-1)[idx] for v in rec["v_u"]]).astype(np.float32))
    return out


def sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def main():
    lines = []
    for name, wl in cases().items():
        print(f"{name}: 8 steps x 2 branches", flush=True)
        path = make(name, wl)
        lines.append(f"{sha256(path)}  {os.path.basename(path)}")
    with open(os.path.join(HERE, "sampler_expected.sha256"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
