"""Text tokens to velocity on the GPU: the encoder's hidden_states[-2] feed the DiT stack as its
caption features, against the oracle chain (encoder oracle, then the DiT oracle on its output).
The encoder is full width (2560, the DiT's caption width) at reduced depth and head count; the
DiT is the tiny configuration at full depth."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from diffusion_transformer_text_s3_amd import binding as Z
from gpu_util import dev, drift, host, note, rel_l2
from oracle import encoder_oracle as E

pytestmark = pytest.mark.gpu


def test_tokens_to_velocity_pair():
    ed = synth.EncDims(hidden=2560, inter=512, n_heads=4, n_kv_heads=2, n_layers=3, vocab=1000)
    dims = synth.TINY
    assert ed.hidden == dims.cap_dim
    B, L, lens = 2, 64, [45, 10]
    note(f"pipeline: encoder {ed.n_layers - 1} blocks at width {ed.hidden} -> tiny DiT stack, lens={lens}")
    We = synth.encoder_weights(ed, 90, ed.n_layers - 1)
    ids = synth.token_ids(B, L, lens, ed.vocab, 91)
    cfg_e = Z.make_enc_cfg(ed)
    enc = Z.upload_encoder(We)
    cap = torch.empty((B, L, ed.hidden), device="cuda")
    ws_e = Z.workspace(Z.zdit_encoder_workspace(cfg_e, B, L))
    Z.zdit_encoder_fwd(cfg_e, enc, B, L, ids, lens, cap, ws_e)

    Wd = synth.model_weights(dims, 92)
    lat = synth.latents((dims.latent_ch, 16, 16), 92)
    cfg = Z.make_cfg(dims)
    model = Z.upload_model(Wd)
    vel = torch.empty((B, dims.latent_ch, 16, 16), device="cuda")
    ws = Z.workspace(Z.zdit_stack_workspace(cfg, B, 16, 16, L))
    Z.zdit_stack_fwd(cfg, model, B, 16, 16, dev(lat), 0, cap, L, lens, [0.5, 0.5], vel, ws)
    got = host(vel)

    ref_cap = E.encoder_penultimate(ids, lens, We, ed)
    for b in range(B):
        ref = O.stack(lat, ref_cap[b], lens[b], 0.5, Wd, dims)
        e, dr = rel_l2(got[b], ref), drift(got[b], ref)
        print(f"tokens -> velocity branch {b}: rel-L2 {e:.2e} drift {dr:.2e}", flush=True)
        assert e <= 1e-2 and dr <= 0.025
