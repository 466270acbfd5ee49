"""ZDIT_CHECK_FINITE on the GPU: a NaN or an infinity where the path reads or writes valid
values makes zdit_block_fwd / zdit_stack_fwd / zdit_sample return ZDIT_ENONFINITE naming the
first place it appeared (a flag the library reads back on the host); padding is not checked, and
a finite run is bit-identical to the same run without the flag."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from diffusion_transformer_text_s3_amd import binding as Z
from gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


def _block_case(S=96, s_max=128, seed=90):
    dims = synth.TINY
    w = synth.block_weights(dims, seed, 0)
    x = np.zeros((1, s_max, dims.dim), np.float32)
    x[0, :S] = synth.residual_input((S, dims.dim), seed)
    c = synth.residual_input((1, dims.c_dim), seed, index=1)
    cos = np.ones((1, s_max, 64), np.float32)
    sin = np.zeros((1, s_max, 64), np.float32)
    cc, ss = O.rope_tables(O.position_ids("joint", 8, 8, S - 64))
    cos[0, :S], sin[0, :S] = cc, ss
    return dims, w, x, c, cos, sin


def _run_block(dims, blk, x, c, cos, sin, S, flags):
    d = Z.make_dims(dims, flags=flags)
    s_max = x.shape[1]
    xs = dev(x)
    ws = Z.workspace(Z.zdit_block_workspace(d, 1, s_max))
    try:
        Z.zdit_block_fwd(d, blk, 1, s_max, [S], xs, dev(c), dev(cos), dev(sin), ws)
        return Z.ZDIT_OK, host(xs), ""
    except Z.ZditError as e:
        return e.code, host(xs), str(e)


def test_block_check_finite_clean_run_is_bit_identical():
    note("check finite: block, clean input")
    dims, w, x, c, cos, sin = _block_case()
    blk = Z.upload_block(w)
    rc0, y0, _ = _run_block(dims, blk, x, c, cos, sin, 96, 0)
    rc1, y1, _ = _run_block(dims, blk, x, c, cos, sin, 96, Z.ZDIT_CHECK_FINITE)
    assert rc0 == rc1 == Z.ZDIT_OK
    np.testing.assert_array_equal(y0, y1)


def test_block_check_finite_flags_nan_input_not_padding():
    note("check finite: block, NaN in a valid row and in a padding row")
    dims, w, x, c, cos, sin = _block_case()
    blk = Z.upload_block(w)
    bad = x.copy()
    bad[0, 40, 7] = np.nan
    rc, _, msg = _run_block(dims, blk, bad, c, cos, sin, 96, Z.ZDIT_CHECK_FINITE)
    assert rc == Z.ZDIT_ENONFINITE and "input x" in msg
    # without the flag the same call returns OK (and the NaN spreads through attention)
    rc, y, _ = _run_block(dims, blk, bad, c, cos, sin, 96, 0)
    assert rc == Z.ZDIT_OK and not np.isfinite(y[0, :96]).all()
    # a NaN in a padding row (row >= seq_len) is neither read as a key nor checked
    pad = x.copy()
    pad[0, 100, :] = np.nan
    rc, y, _ = _run_block(dims, blk, pad, c, cos, sin, 96, Z.ZDIT_CHECK_FINITE)
    assert rc == Z.ZDIT_OK and np.isfinite(y[0, :96]).all()


def test_block_check_finite_flags_infinite_output():
    """An infinite weight makes the block's output non-finite from a finite input."""
    note("check finite: block, infinite w2 entry")
    dims, w, x, c, cos, sin = _block_case()
    w = dict(w)
    w["w2"] = w["w2"].copy()
    w["w2"][3, 5] = np.inf
    rc, _, msg = _run_block(dims, Z.upload_block(w), x, c, cos, sin, 96, Z.ZDIT_CHECK_FINITE)
    assert rc == Z.ZDIT_ENONFINITE and "block output" in msg


def _stack_case(seed=91, n_main=4):
    dims = synth.TINY.replace(n_main=n_main)
    W = synth.model_weights(dims, seed)
    lat = synth.latents((16, 16, 16), seed)
    cap = synth.caption_features(2, 45, dims.cap_dim, seed)
    return dims, W, lat, cap


def _run_stack(dims, model, lat, cap, cap_len, flags):
    cfg = Z.make_cfg(dims, flags=flags)
    vel = torch.empty((2, 16, 16, 16), device="cuda")
    ws = Z.workspace(Z.zdit_stack_workspace(cfg, 2, 16, 16, 45))
    try:
        Z.zdit_stack_fwd(cfg, model, 2, 16, 16, dev(lat), 0, dev(cap), 45, cap_len, [0.5, 0.5], vel, ws)
        return Z.ZDIT_OK, host(vel), ""
    except Z.ZditError as e:
        return e.code, host(vel), str(e)


def test_stack_check_finite_names_the_first_place():
    note("check finite: stack, clean / NaN latent / NaN caption row / padding caption row / bad block")
    dims, W, lat, cap = _stack_case()
    model = Z.upload_model(W)
    rc0, v0, _ = _run_stack(dims, model, lat, cap, [45, 10], 0)
    rc1, v1, _ = _run_stack(dims, model, lat, cap, [45, 10], Z.ZDIT_CHECK_FINITE)
    assert rc0 == rc1 == Z.ZDIT_OK
    np.testing.assert_array_equal(v0, v1)
    bad = lat.copy()
    bad[3, 4, 5] = np.nan
    rc, _, msg = _run_stack(dims, model, bad, cap, [45, 10], Z.ZDIT_CHECK_FINITE)
    assert rc == Z.ZDIT_ENONFINITE and "latents" in msg
    badc = cap.copy()
    badc[1, 9, 100] = np.inf  # last valid row of the 10-token branch
    rc, _, msg = _run_stack(dims, model, lat, badc, [45, 10], Z.ZDIT_CHECK_FINITE)
    assert rc == Z.ZDIT_ENONFINITE and "caption features" in msg
    padc = cap.copy()
    padc[1, 10:, :] = np.nan  # rows past the 10-token branch's length are not read
    rc, v, _ = _run_stack(dims, model, lat, padc, [45, 10], Z.ZDIT_CHECK_FINITE)
    assert rc == Z.ZDIT_OK
    np.testing.assert_array_equal(v, v0)
    # an infinite weight in main block 2 first shows in the residual stream after that block
    W2 = dict(W, main=list(W["main"]))
    W2["main"][2] = dict(W["main"][2], w_out=W["main"][2]["w_out"].copy())
    W2["main"][2]["w_out"][0, 0] = np.inf
    rc, _, msg = _run_stack(dims, Z.upload_model(W2), lat, cap, [45, 10], Z.ZDIT_CHECK_FINITE)
    assert rc == Z.ZDIT_ENONFINITE and "after main block 2" in msg


def test_sample_check_finite_reports_step_and_place():
    note("check finite: sampler, clean run and a NaN caption row")
    dims, W, lat, cap = _stack_case(seed=92, n_main=2)
    model = Z.upload_model(W)

    def run(capv, flags):
        cfg = Z.make_cfg(dims, flags=flags)
        x = dev(lat)
        dec = torch.empty_like(x)
        ws = Z.workspace(Z.zdit_sample_workspace(cfg, 16, 16, 45, 1.0))
        try:
            Z.zdit_sample(cfg, model, 16, 16, x, dev(capv), 45, [45, 10], 1.0, 4, 3.0, dec, ws)
            return Z.ZDIT_OK, host(x), ""
        except Z.ZditError as e:
            return e.code, host(x), str(e)

    rc0, x0, _ = run(cap, 0)
    rc1, x1, _ = run(cap, Z.ZDIT_CHECK_FINITE)
    assert rc0 == rc1 == Z.ZDIT_OK
    np.testing.assert_array_equal(x0, x1)
    badc = cap.copy()
    badc[0, 0, 0] = np.nan
    rc, _, msg = run(badc, Z.ZDIT_CHECK_FINITE)
    assert rc == Z.ZDIT_ENONFINITE and "sampler step 0" in msg and "caption features" in msg
