"""The library's calls enqueue only kernels on the caller's stream (no allocation, no
synchronisation, no host copy at these shapes), so they can be captured into a HIP graph: the
block, the stack, the whole sampler and the text encoder captured once with torch's graph API
and replayed several times, with the program's own eager work between the replays, each replay
bit-identical to the eager call."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from diffusion_transformer_text_s3_amd import binding as Z
from gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


def _replays(run, reset, out, n=3):
    """Eager result, then the graph's replays with eager work (reset of the inputs and a
    poisoning of the output) between them."""
    reset()
    run()
    want = host(out).copy()
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(n):
        out.fill_(float("nan"))   # the block updates its input in place: poison first, then reset
        reset()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), want, err_msg=f"replay {i}")


def test_graph_block():
    note("graph capture: tiny block, cond/uncond pair")
    dims = synth.TINY
    ncs = [O.n_cap(45), O.n_cap(10)]
    S = [64 + nc for nc in ncs]
    s_max = max(S)
    x0 = dev(synth.residual_input((2, s_max, dims.dim), 80))
    x = x0.clone()
    c = dev(O.t_condition(np.full(2, 0.5, np.float32), synth.embed_weights(dims, 80), dims))
    cos = np.ones((2, s_max, 64), np.float32)
    sin = np.zeros((2, s_max, 64), np.float32)
    for b, nc in enumerate(ncs):
        cc, ss = O.rope_tables(O.position_ids("joint", 8, 8, nc), dims.rope_axes, dims.rope_theta)
        cos[b, :len(cc)], sin[b, :len(ss)] = cc, ss
    cos, sin = dev(cos), dev(sin)
    d = Z.make_dims(dims)
    w = Z.upload_block(synth.block_weights(dims, 80, 0))
    ws = Z.workspace(Z.zdit_block_workspace(d, 2, s_max))
    _replays(lambda: Z.zdit_block_fwd(d, w, 2, s_max, S, x, c, cos, sin, ws), lambda: x.copy_(x0), x)


def test_graph_stack_and_sampler():
    note("graph capture: tiny stack pair and a 3-step sampler")
    dims = synth.TINY.replace(n_main=3)
    model = Z.upload_model(synth.model_weights(dims, 81))
    lat = dev(synth.latents((dims.latent_ch, 16, 16), 81))
    cap = dev(synth.caption_features(2, 45, dims.cap_dim, 81))
    cfg = Z.make_cfg(dims)
    vel = torch.empty((2, dims.latent_ch, 16, 16), device="cuda")
    ws = Z.workspace(Z.zdit_stack_workspace(cfg, 2, 16, 16, 45))
    _replays(lambda: Z.zdit_stack_fwd(cfg, model, 2, 16, 16, lat, 0, cap, 45, [45, 10], [0.5, 0.5], vel, ws),
             lambda: None, vel)
    x = lat.clone()
    dec = torch.empty_like(x)
    sws = Z.workspace(Z.zdit_sample_workspace(cfg, 16, 16, 45, 1.0))
    _replays(lambda: Z.zdit_sample(cfg, model, 16, 16, x, cap, 45, [45, 10], 1.0, 3, 3.0, dec, sws),
             lambda: x.copy_(lat), dec)


def test_graph_text_encoder():
    note("graph capture: tiny text encoder, ids in the kernel arguments")
    ed = synth.ENC_TINY
    lens = [37, 12]
    W = synth.encoder_weights(ed, 82, ed.n_layers - 1)
    ids = synth.token_ids(2, 40, lens, ed.vocab, 83)
    m = Z.upload_encoder(W)
    cfg = Z.make_enc_cfg(ed)
    out = torch.empty((2, 40, ed.hidden), device="cuda")
    ws = Z.workspace(Z.zdit_encoder_workspace(cfg, 2, 40))
    _replays(lambda: Z.zdit_encoder_fwd(cfg, m, 2, 40, ids, lens, out, ws), lambda: None, out)


def test_graph_vae_decode():
    note("graph capture: tiny VAE decode")
    vd = synth.VAE_TINY
    m = Z.upload_vae(synth.vae_weights(vd, 84), vd)
    z = dev(synth.latents((2, vd.latent_ch, 6, 4), 84))
    cfg = Z.make_vae_cfg(vd)
    img = torch.empty((2, vd.out_ch, 48, 32), device="cuda")
    ws = Z.workspace(Z.zdit_vae_workspace(cfg, 2, 6, 4))
    _replays(lambda: Z.zdit_vae_decode(cfg, m, 2, 6, 4, z, img, ws), lambda: None, img)
