"""zdit_stack_fwd and zdit_sample against the oracle stack and sampler.

The full 2 + 2 + 30 depth is checked at the tiny width (dim 384); full width (dim 3840) is
checked at reduced depth at 256 px and at 1024^2 here, and at full depth in
tests/test_gpu_fullsize.py.  Also: two runs of the sampler are bit-identical, and the loop
resumes exactly from its state (x, step)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from diffusion_transformer_text_s3_amd import binding as Z
from gpu_util import dev, drift, host, note, rel_l2

pytestmark = pytest.mark.gpu
BF, F32P = Z.ZDIT_BF16, Z.ZDIT_FP32_DEBUG


def stack_case(dims, lat_h, lat_w, cap_len, seed, t=0.5):
    W = synth.model_weights(dims, seed)
    lat = synth.latents((dims.latent_ch, lat_h, lat_w), seed)
    Lmax = max(cap_len)
    cap = synth.caption_features(len(cap_len), Lmax, dims.cap_dim, seed)
    return dict(dims=dims, W=W, lat=lat, cap=cap, cap_len=list(cap_len), Lmax=Lmax, t=t, lat_h=lat_h, lat_w=lat_w)


def gpu_stack(case, prec=BF, model=None, batch=None, t=None, per_branch_latents=False):
    """per_branch_latents: pass B copies of the latent with a nonzero branch stride instead of
    one shared latent (stride 0); t: per-branch model times (default case["t"] for all)."""
    dims = case["dims"]
    B = batch or len(case["cap_len"])
    cfg = Z.make_cfg(dims, prec)
    model = model or Z.upload_model(case["W"], prec)
    vel = torch.empty((B, dims.latent_ch, case["lat_h"], case["lat_w"]), device="cuda")
    ws = Z.workspace(Z.zdit_stack_workspace(cfg, B, case["lat_h"], case["lat_w"], case["Lmax"]))
    lat, stride = dev(case["lat"]), 0
    if per_branch_latents:
        lat = dev(np.stack([case["lat"]] * B))
        stride = case["lat"].size
    Z.zdit_stack_fwd(cfg, model, B, case["lat_h"], case["lat_w"], lat, stride, dev(case["cap"][:B]),
                     case["Lmax"], case["cap_len"][:B], t or [case["t"]] * B, vel, ws)
    return host(vel), model


def oracle_stack(case, b, dtype=np.float32):
    return O.stack(case["lat"], case["cap"][b], case["cap_len"][b], case["t"], case["W"], case["dims"], dtype=dtype)


def test_stack_tiny_full_depth_bf16():
    """Tiny width, full 2 + 2 + 30 depth, cond/uncond pair with different n_cap."""
    note("stack tiny 2+2+30 bf16 pair")
    case = stack_case(synth.TINY, 16, 16, (20, 10), seed=70)
    got, _ = gpu_stack(case)
    for b in range(2):
        ref = oracle_stack(case, b)
        e, dr = rel_l2(got[b], ref), drift(got[b], ref)
        print(f"tiny stack branch {b}: rel-L2 {e:.2e} drift {dr:.2e}", flush=True)
        assert e <= 1e-2 and dr <= 0.025


def test_stack_tiny_41_main_blocks_two_adaln_launches():
    """The modulations of a stage are projected at most 40 blocks per launch: 41 main blocks
    take two launches, the 41st block's slice written by the second."""
    note("stack tiny 2+2+41 bf16 pair")
    case = stack_case(synth.TINY.replace(n_main=41), 16, 16, (32, 7), seed=78)
    got, _ = gpu_stack(case)
    for b in range(2):
        ref = oracle_stack(case, b)
        e, dr = rel_l2(got[b], ref), drift(got[b], ref)
        print(f"41-block stack branch {b}: rel-L2 {e:.2e} drift {dr:.2e}", flush=True)
        assert e <= 1e-2 and dr <= 0.025


def test_stack_tiny_fp32_debug_atol_1e4():
    note("stack tiny fp32 debug")
    case = stack_case(synth.TINY, 16, 16, (20,), seed=71)
    got, _ = gpu_stack(case, F32P)
    np.testing.assert_allclose(got[0], oracle_stack(case, 0), rtol=1e-4, atol=1e-4)


def test_stack_branch_alone_equals_branch_in_pair():
    note("stack branch alone vs pair")
    case = stack_case(synth.TINY.replace(n_main=3), 16, 16, (45, 10), seed=72)
    pair, model = gpu_stack(case)
    alone, _ = gpu_stack(case, model=model, batch=1)
    np.testing.assert_array_equal(alone[0], pair[0])


def test_stack_shared_latent_equals_per_branch_copies():
    """One shared latent at one model time lets the image path through the noise refiners run
    once for every branch; the result is bit-identical to giving each branch its own copy of
    the latent (which computes every branch), and to the oracle per branch."""
    note("stack shared latent vs per-branch copies")
    case = stack_case(synth.TINY.replace(n_main=3), 16, 16, (45, 10, 33), seed=76)
    shared, model = gpu_stack(case)
    copies, _ = gpu_stack(case, model=model, per_branch_latents=True)
    np.testing.assert_array_equal(shared, copies)
    for b in range(3):
        assert rel_l2(shared[b], oracle_stack(case, b)) <= 1e-2


def test_stack_shared_latent_different_times():
    """A shared latent at different model times per branch: each branch matches the oracle at
    its own time and equals that branch run alone."""
    note("stack shared latent, two model times")
    case = stack_case(synth.TINY.replace(n_main=2), 16, 16, (20, 20), seed=77)
    got, model = gpu_stack(case, t=[0.25, 0.75])
    for b, tb in enumerate((0.25, 0.75)):
        ref = O.stack(case["lat"], case["cap"][b], 20, tb, case["W"], case["dims"])
        assert rel_l2(got[b], ref) <= 1e-2
    alone, _ = gpu_stack(dict(case, cap=case["cap"][1:]), model=model, batch=1, t=[0.75])
    np.testing.assert_array_equal(alone[0], got[1])


def test_stack_full_width_reduced_depth_256px():
    note("stack full width 2+2+2 at 256px pair")
    case = stack_case(synth.FULL.replace(n_main=2), 32, 32, (45, 10), seed=73)
    got, _ = gpu_stack(case)
    for b in range(2):
        ref = oracle_stack(case, b)
        e, dr = rel_l2(got[b], ref), drift(got[b], ref)
        print(f"256px stack branch {b}: rel-L2 {e:.2e} drift {dr:.2e}", flush=True)
        assert e <= 1e-2 and dr <= 0.025


def test_stack_full_width_1024_one_block_each():
    note("stack full width 1+1+1 at 1024^2 cond")
    case = stack_case(synth.FULL.replace(n_noise_ref=1, n_ctx_ref=1, n_main=1), 128, 128, (45,), seed=74)
    got, _ = gpu_stack(case)
    ref = oracle_stack(case, 0)
    e, dr = rel_l2(got[0], ref), drift(got[0], ref)
    print(f"1024 stack: rel-L2 {e:.2e} drift {dr:.2e}", flush=True)
    assert e <= 1e-2 and dr <= 0.025


def _oracle_sample(case, guidance, num_steps=8):
    calls = []

    def dit(x, branch, t):
        calls.append(branch)
        return O.stack(x, case["cap"][branch], case["cap_len"][branch], t, case["W"], case["dims"])

    x, dec = O.sample(case["lat"], dit, num_steps=num_steps, shift=3.0, guidance=guidance)
    return x, dec, calls


@pytest.mark.parametrize("guidance", [1.0, 0.0])
def test_sample_tiny_full_depth(guidance):
    """8-step negated-CFG FlowMatchEuler loop (16 DiT calls with guidance, 8 without)."""
    note(f"sample tiny 8 steps g={guidance}")
    dims = synth.TINY
    case = stack_case(dims, 16, 16, (45, 10), seed=75)
    cfg = Z.make_cfg(dims)
    model = Z.upload_model(case["W"])
    nb = 2 if guidance != 0 else 1
    x = dev(case["lat"])
    dec = torch.empty_like(x)
    ws = Z.workspace(Z.zdit_sample_workspace(cfg, 16, 16, case["Lmax"], guidance))
    Z.zdit_sample(cfg, model, 16, 16, x, dev(case["cap"][:nb]), case["Lmax"], case["cap_len"][:nb], guidance, 8,
                  3.0, dec, ws)
    rx, rdec, calls = _oracle_sample(case, guidance)
    assert len(calls) == 8 * nb
    e = rel_l2(host(x), rx)
    print(f"sample g={guidance}: final latent rel-L2 {e:.2e}", flush=True)
    assert e <= 1e-2
    # the decode output is the GPU's own final latent unscaled exactly once
    np.testing.assert_array_equal(host(dec), O.unscale(host(x)))


def test_sample_equals_stack_and_euler_calls():
    """zdit_sample keeps the caption rows after the context refiners from its first step and
    reuses them in later steps; the final latent is bit-identical to calling zdit_stack_fwd
    (which runs the context refiners every time) and zdit_euler_step once per step."""
    note("sample vs per-step stack + euler calls")
    dims = synth.TINY.replace(n_main=4)
    case = stack_case(dims, 16, 16, (45, 10), seed=78)
    cfg = Z.make_cfg(dims)
    model = Z.upload_model(case["W"])
    steps, g = 4, 1.0
    x = dev(case["lat"])
    dec = torch.empty_like(x)
    ws = Z.workspace(Z.zdit_sample_workspace(cfg, 16, 16, case["Lmax"], g))
    Z.zdit_sample(cfg, model, 16, 16, x, dev(case["cap"]), case["Lmax"], case["cap_len"], g, steps, 3.0, dec, ws)
    sg = Z.zdit_sigmas(steps, 3.0)
    y = dev(case["lat"])
    vel = torch.empty((2,) + tuple(y.shape), device="cuda")
    sws = Z.workspace(Z.zdit_stack_workspace(cfg, 2, 16, 16, case["Lmax"]))
    n = y.numel()
    for i in range(steps):
        ti = float(np.float32(1.0) - np.float32(sg[i]))
        Z.zdit_stack_fwd(cfg, model, 2, 16, 16, y, 0, dev(case["cap"]), case["Lmax"], case["cap_len"], [ti, ti],
                         vel, sws)
        Z.zdit_euler_step(y, vel[0], vel[1], n, g, sg[i], sg[i + 1])
    np.testing.assert_array_equal(host(x), host(y))


def test_sample_base_recipe_50_steps_cfg4():
    """The Base recipe on the same path: 50 FlowMatchEuler updates with negated CFG at g = 4
    (shift 3), cond/uncond pair, against the oracle's sampler (100 DiT calls)."""
    note("sample 50 steps g=4")
    dims = synth.TINY.replace(n_main=4)
    case = stack_case(dims, 16, 16, (45, 10), seed=79)
    cfg = Z.make_cfg(dims)
    model = Z.upload_model(case["W"])
    x = dev(case["lat"])
    dec = torch.empty_like(x)
    ws = Z.workspace(Z.zdit_sample_workspace(cfg, 16, 16, case["Lmax"], 4.0))
    Z.zdit_sample(cfg, model, 16, 16, x, dev(case["cap"]), case["Lmax"], case["cap_len"], 4.0, 50, 3.0, dec, ws)
    rx, _, calls = _oracle_sample(case, 4.0, num_steps=50)
    assert len(calls) == 100
    e = rel_l2(host(x), rx)
    print(f"sample 50 steps g=4: final latent rel-L2 {e:.2e}", flush=True)
    assert e <= 1e-2
    np.testing.assert_array_equal(host(dec), O.unscale(host(x)))


def test_sampler_deterministic_and_resumable_from_its_state():
    """Two zdit_sample runs give the same bits; and the loop's state is (x, step): running
    steps 0-3 as per-step calls, taking x to the host and back, then steps 4-7 gives the
    uninterrupted run's final latent bit for bit."""
    note("sample determinism and resume")
    dims = synth.TINY
    case = stack_case(dims, 16, 16, (45, 10), seed=80)
    cfg = Z.make_cfg(dims)
    model = Z.upload_model(case["W"])
    ws = Z.workspace(Z.zdit_sample_workspace(cfg, 16, 16, case["Lmax"], 1.0))
    runs = []
    for _ in range(2):
        x = dev(case["lat"])
        dec = torch.empty_like(x)
        Z.zdit_sample(cfg, model, 16, 16, x, dev(case["cap"]), case["Lmax"], case["cap_len"], 1.0, 8, 3.0, dec, ws)
        runs.append((host(x), host(dec)))
    np.testing.assert_array_equal(runs[0][0], runs[1][0])
    np.testing.assert_array_equal(runs[0][1], runs[1][1])
    sg = Z.zdit_sigmas(8, 3.0)
    sws = Z.workspace(Z.zdit_stack_workspace(cfg, 2, 16, 16, case["Lmax"]))
    y = dev(case["lat"])
    vel = torch.empty((2,) + tuple(y.shape), device="cuda")
    for i in range(8):
        if i == 4:
            y = dev(host(y))   # the saved state: the fp32 latent and the step index
        ti = float(np.float32(1.0) - np.float32(sg[i]))
        Z.zdit_stack_fwd(cfg, model, 2, 16, 16, y, 0, dev(case["cap"]), case["Lmax"], case["cap_len"], [ti, ti],
                         vel, sws)
        Z.zdit_euler_step(y, vel[0], vel[1], y.numel(), 1.0, sg[i], sg[i + 1])
    np.testing.assert_array_equal(host(y), runs[0][0])
