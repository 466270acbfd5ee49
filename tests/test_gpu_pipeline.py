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


def test_tokens_to_image():
    """The whole chain: ids -> encoder -> 8-step negated-CFG sampler (tiny DiT, 2 + 2 + 2
    blocks) -> VAE decode (tiny widths) on a 16 x 16 latent, against the oracle chain.  The
    decoder is fed the sampler's raw final latent (the unscale is inside it, applied once);
    feeding the sampler's already unscaled decode output with ZDIT_VAE_INPUT_UNSCALED gives
    the same image bit for bit."""
    from oracle import vae_oracle as V
    ed = synth.EncDims(hidden=2560, inter=512, n_heads=4, n_kv_heads=2, n_layers=3, vocab=1000)
    dims = synth.TINY.replace(n_main=2)
    vd = synth.VAE_TINY
    B, L, lens = 2, 64, [45, 10]
    note("pipeline: ids -> encoder -> 8-step sampler -> VAE decode")
    We = synth.encoder_weights(ed, 93, ed.n_layers - 1)
    ids = synth.token_ids(B, L, lens, ed.vocab, 94)
    cfg_e = Z.make_enc_cfg(ed)
    cap = torch.empty((B, L, ed.hidden), device="cuda")
    ws_e = Z.workspace(Z.zdit_encoder_workspace(cfg_e, B, L))
    Z.zdit_encoder_fwd(cfg_e, Z.upload_encoder(We), B, L, ids, lens, cap, ws_e)

    Wd = synth.model_weights(dims, 95)
    lat = synth.latents((dims.latent_ch, 16, 16), 95)
    cfg = Z.make_cfg(dims)
    x = dev(lat)
    dec = torch.empty_like(x)
    ws = Z.workspace(Z.zdit_sample_workspace(cfg, 16, 16, L, 1.0))
    Z.zdit_sample(cfg, Z.upload_model(Wd), 16, 16, x, cap, L, lens, 1.0, 8, 3.0, dec, ws)

    Wv = synth.vae_weights(vd, 96)
    m = Z.upload_vae(Wv, vd)
    img = torch.empty((1, vd.out_ch, 128, 128), device="cuda")
    img2 = torch.empty_like(img)
    vws = Z.workspace(Z.zdit_vae_workspace(Z.make_vae_cfg(vd), 1, 16, 16))
    Z.zdit_vae_decode(Z.make_vae_cfg(vd), m, 1, 16, 16, x, img, vws)
    Z.zdit_vae_decode(Z.make_vae_cfg(vd, Z.ZDIT_VAE_INPUT_UNSCALED), m, 1, 16, 16, dec, img2, vws)
    np.testing.assert_array_equal(host(img2), host(img))

    ref_cap = E.encoder_penultimate(ids, lens, We, ed)
    calls = []

    def dit(xx, branch, t):
        calls.append(branch)
        return O.stack(xx, ref_cap[branch], lens[branch], t, Wd, dims)

    rx, _ = O.sample(lat, dit, num_steps=8, shift=3.0, guidance=1.0)
    ref_img = V.decoder(rx[None], Wv, vd)
    e_lat, e_img = rel_l2(host(x), rx), rel_l2(host(img), ref_img)
    print(f"tokens -> image: final latent rel-L2 {e_lat:.2e}, image rel-L2 {e_img:.2e}", flush=True)
    assert len(calls) == 16
    assert e_lat <= 1e-2 and e_img <= 1e-2
