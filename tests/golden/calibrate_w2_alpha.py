"""Fix the w2 outlier-channel scale of the 1024^2 pair-block workload (calls only the oracle).

The pages report w2 / to_out outputs near 3.1e5 (Core AI model zoo, "Z-Image-Turbo port",
section "fp16 does not work. bf16 does.").  The workload scales 4 seeded output channels of
w2 by alpha; this script runs the oracle block on the workload's cond branch with alpha = 1,
takes the largest |w2 output| over those channels and prints alpha = 3e5 / that maximum
(the w2 output of those channels is linear in alpha).  Run from the repository root:
    python tests/golden/calibrate_w2_alpha.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle as O  # noqa: E402
import synth  # noqa: E402


def main():
    wl = synth.CFG3
    dims = wl.dims
    w = synth.block_weights(dims, wl.seed, 0, w2_outlier_channels=wl.w2_outlier_channels,
                            w2_outlier_alpha=1.0)
    ew = synth.embed_weights(dims, wl.seed)
    gh, gw = wl.lat_h // 2, wl.lat_w // 2
    L = wl.cap_len[0]
    S = gh * gw + O.n_cap(L)
    x = synth.residual_input((wl.batch, S, dims.dim), wl.seed, wl.outlier_frac)[0]
    c = O.t_condition(np.array([wl.t], dtype=np.float32), ew, dims)[0]
    cos, sin = O.rope_tables(O.position_ids("joint", gh, gw, O.n_cap(L)), dims.rope_axes, dims.rope_theta)
    rec = {}
    O.block(x, w, O.block_mod(c, w), cos, sin, dims, record=rec)
    m = float(np.abs(rec["ffn_out"][:, w["w2_outlier_rows"]]).max())
    print(f"max |w2 out| over outlier channels at alpha=1: {m:.6g}; alpha = {3e5 / m:.6g}")


if __name__ == "__main__":
    main()
