"""zdit_block_fwd_noalloc (the block forward in the library's own per-device scratch, for callers
that cannot allocate) against zdit_block_fwd with a caller workspace: bit-identical outputs on
calls in a row, each on a smaller input than the one before, so stale scratch contents from the
previous call must not matter; a shape whose workspace exceeds the scratch is rejected before
anything runs."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from diffusion_transformer_text_s3_amd import binding as Z
from gpu_util import dev, host, note, rel_l2

pytestmark = pytest.mark.gpu


def _case(dims, B, gh, gw, cap_lens, seed, outliers=0.0):
    ncs = [O.n_cap(L) for L in cap_lens]
    S = [gh * gw + n for n in ncs]
    s_max = max(S)
    w = synth.block_weights(dims, seed, 0)
    ew = synth.embed_weights(dims, seed)
    x = synth.residual_input((B, s_max, dims.dim), seed, outliers)
    c = O.t_condition(np.full(B, 0.5, np.float32), ew, dims)
    cos = torch.empty((B, s_max, 64), device="cuda")
    sin = torch.empty_like(cos)
    Z.zdit_rope_tables(Z.ZDIT_SEQ_JOINT, list(dims.rope_axes), dims.rope_theta, B, s_max, gh, gw, ncs, cos, sin)
    return dict(dims=dims, B=B, S=S, s_max=s_max, w=w, x=x, c=c, cos=cos, sin=sin, gh=gh, gw=gw, ncs=ncs)


def _both(case, flags=0):
    dims, B, S, s_max = case["dims"], case["B"], case["S"], case["s_max"]
    d = Z.make_dims(dims, flags=flags)
    blk = Z.upload_block(case["w"])
    c = dev(case["c"])
    xa = dev(case["x"])
    ws = Z.workspace(Z.zdit_block_workspace(d, B, s_max))
    Z.zdit_block_fwd(d, blk, B, s_max, S, xa, c, case["cos"], case["sin"], ws)
    xb = dev(case["x"])
    Z.zdit_block_fwd_noalloc(d, blk, B, s_max, S, xb, c, case["cos"], case["sin"])
    return host(xa), host(xb)


def _oracle_update(case, br):
    n = case["S"][br]
    cs, sn = O.rope_tables(O.position_ids("joint", case["gh"], case["gw"], case["ncs"][br]))
    ref = O.block(case["x"][br, :n], case["w"], O.block_mod(case["c"][br], case["w"]), cs, sn, case["dims"])
    return ref - case["x"][br, :n]


def test_noalloc_matches_workspace_entry_calls_getting_smaller():
    """Three calls in a row, each smaller than the one before, on the scratch the previous one
    left behind: a full-width 512 px branch (S = 1088, whole-K GEMMs), a full-width 256 px branch
    (S = 320, K-split GEMMs) and a tiny block."""
    note("noalloc block: full-width 512 px, then 256 px, then a tiny block")
    for case in (_case(synth.FULL, 1, 32, 32, [45], 98, outliers=0.001),
                 _case(synth.FULL, 1, 16, 16, [45], 99, outliers=0.001)):
        a, b = _both(case)
        np.testing.assert_array_equal(b, a)
        n = case["S"][0]
        assert rel_l2(b[0, :n] - case["x"][0, :n], _oracle_update(case, 0)) <= 1e-2
        np.testing.assert_array_equal(b[0, n:], case["x"][0, n:])
    small = _case(synth.TINY, 1, 8, 8, [20], 97)
    a, b = _both(small)
    np.testing.assert_array_equal(b, a)
    # and with the non-finite check on
    a, b = _both(small, flags=Z.ZDIT_CHECK_FINITE)
    np.testing.assert_array_equal(b, a)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """The 1024^2 pair needs ~390 MB of workspace: rejected, x untouched (so is a pair of
    448-row branches, whose K-split GEMMs keep ~110 MB of fp32 partial products; the 256 px
    pair, 320 rows each, fits)."""
    note("noalloc block: 1024^2 pair rejected")
    dims = synth.FULL
    d = Z.make_dims(dims)
    assert Z.zdit_block_workspace(d, 2, 4160) > (128 << 20)
    blk = Z.upload_block(synth.block_weights(dims, 100, 0))
    x = torch.full((2, 4160, dims.dim), 3.0, device="cuda")
    c = torch.zeros((2, dims.c_dim), device="cuda")
    cos = torch.ones((2, 4160, 64), device="cuda")
    sin = torch.zeros((2, 4160, 64), device="cuda")
    with pytest.raises(Z.ZditError) as e:
        Z.zdit_block_fwd_noalloc(d, blk, 2, 4160, [4160, 4128], x, c, cos, sin)
    assert e.value.code == Z.ZDIT_EUNSUPPORTED and "scratch" in str(e.value)
    assert bool((x == 3.0).all())
    assert Z.zdit_block_workspace(d, 2, 320) <= (128 << 20) < Z.zdit_block_workspace(d, 2, 448)
