"""The C-ABI library loads, exports every symbol include/zdit.h declares, and its host-only
logic (sigmas, n_cap, workspace queries, argument validation) behaves; no device work."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
import synth
from conftest import ROOT, golden
from diffusion_transformer_text_s3_amd import binding as Z


def _header_functions():
    src = open(os.path.join(ROOT, "include", "zdit.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zdit_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = Z.lib()
    declared = _header_functions()
    assert len(declared) >= 20
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(Z.EXPORTS) == declared
    assert L.zdit_abi_version() == 2


def test_sigmas_match_oracle_bit_exact():
    for n in (1, 2, 4, 8, 20, 50, 1000):
        for shift in (1.0, 3.0, 7.5):
            got = np.array(Z.zdit_sigmas(n, shift), dtype=np.float32)
            np.testing.assert_array_equal(got, O.sigmas(n, shift))
    got = Z.zdit_sigmas(8, 3.0)
    assert got[0] == 1.0 and got[-1] == 0.0


def test_n_cap_matches_oracle_and_pages():
    for L, want in golden("n_cap_cases.txt"):
        assert Z.zdit_n_cap(int(L)) == int(want)
    for L in range(1, 513):
        assert Z.zdit_n_cap(L) == O.n_cap(L)


@pytest.mark.parametrize("bad", [0, -3, 513])
def test_n_cap_rejects(bad):
    with pytest.raises(Z.ZditError) as e:
        Z.zdit_n_cap(bad)
    assert e.value.code == Z.ZDIT_EINVAL


def test_sigmas_rejects():
    for n, s in ((0, 3.0), (1001, 3.0), (8, 0.0), (8, -1.0), (8, float("nan"))):
        with pytest.raises(Z.ZditError):
            Z.zdit_sigmas(n, s)


def test_block_workspace_and_dims_validation():
    d = Z.make_dims(synth.FULL)
    ws = Z.zdit_block_workspace(d, 2, 4160)
    # h + qkv + vt + o, plus the modulation vectors
    assert ws >= 2 * 4160 * 3840 * 2 * 5
    bad = Z.make_dims(synth.FULL)
    bad.head_dim = 64
    assert Z.zdit_block_workspace(bad, 2, 4160) == 0
    bad = Z.make_dims(synth.FULL)
    bad.rope_axes[:] = [32, 48, 40]
    assert Z.zdit_block_workspace(bad, 2, 4160) == 0
    assert Z.zdit_block_workspace(d, 0, 10) == 0 and Z.zdit_block_workspace(d, 17, 10) == 0


def _fake(addr=1 << 20):
    return C.c_void_p(addr)


def test_block_fwd_rejects_bad_arguments_before_launch():
    L = Z.lib()
    d = Z.make_dims(synth.TINY)
    w = Z.zdit_block_w()
    for k in ("w_qkv", "w_out", "w1", "w3", "w2", "norm1", "norm2"):
        setattr(w, k, 1 << 20)
    p = _fake()
    # seq_len outside 1..s_max
    for seq in ([0], [97]):
        rc = L.zdit_block_fwd(C.byref(d), C.byref(w), 1, 96, Z.i32_array(seq), p, None, p, p, p, 1 << 30, None)
        assert rc == Z.ZDIT_EINVAL and "seq_len" in Z.last_error()
    # misaligned x
    rc = L.zdit_block_fwd(C.byref(d), C.byref(w), 1, 96, Z.i32_array([96]), _fake((1 << 20) + 4), None, p, p, p,
                          1 << 30, None)
    assert rc == Z.ZDIT_EINVAL and "aligned" in Z.last_error()
    # workspace too small
    rc = L.zdit_block_fwd(C.byref(d), C.byref(w), 1, 96, Z.i32_array([96]), p, None, p, p, p, 1024, None)
    assert rc == Z.ZDIT_EWORKSPACE
    # adaLN weights without c
    w.w_ada, w.b_ada = 1 << 20, 1 << 20
    rc = L.zdit_block_fwd(C.byref(d), C.byref(w), 1, 96, Z.i32_array([96]), p, None, p, p, p, 1 << 30, None)
    assert rc == Z.ZDIT_EINVAL
    # unsupported head dim
    d.head_dim = 64
    rc = L.zdit_block_fwd(C.byref(d), C.byref(w), 1, 96, Z.i32_array([96]), p, p, p, p, p, 1 << 30, None)
    assert rc == Z.ZDIT_EUNSUPPORTED


def test_dims_flags_layout_and_validation():
    """zdit_dims ends with the flags word (ABI 2); ZDIT_CHECK_FINITE is accepted, any other bit
    is rejected before anything runs, and the checked workspaces are no larger."""
    assert C.sizeof(Z.zdit_dims) == 11 * 4 and Z.zdit_dims.flags.offset == 40
    L = Z.lib()
    d = Z.make_dims(synth.TINY)
    plain = Z.zdit_block_workspace(d, 1, 96)
    d.flags = Z.ZDIT_CHECK_FINITE
    assert Z.zdit_block_workspace(d, 1, 96) == plain > 0
    cfg_plain = Z.make_cfg(synth.TINY)
    cfg_chk = Z.make_cfg(synth.TINY, flags=Z.ZDIT_CHECK_FINITE)
    assert Z.zdit_stack_workspace(cfg_chk, 2, 16, 16, 45) == Z.zdit_stack_workspace(cfg_plain, 2, 16, 16, 45) > 0
    assert Z.zdit_sample_workspace(cfg_chk, 16, 16, 45, 1.0) == Z.zdit_sample_workspace(cfg_plain, 16, 16, 45, 1.0)
    for bad in (2, 4, 1 << 30, -1):
        d.flags = bad
        assert Z.zdit_block_workspace(d, 1, 96) == 0
        w = Z.zdit_block_w()
        for k in ("w_qkv", "w_out", "w1", "w3", "w2", "norm1", "norm2"):
            setattr(w, k, 1 << 20)
        p = _fake()
        rc = L.zdit_block_fwd(C.byref(d), C.byref(w), 1, 96, Z.i32_array([96]), p, None, p, p, p, 1 << 30, None)
        assert rc == Z.ZDIT_EINVAL and "flag" in Z.last_error()
        cfg = Z.make_cfg(synth.TINY, flags=bad)
        assert Z.zdit_stack_workspace(cfg, 2, 16, 16, 45) == 0
        assert Z.zdit_sample_workspace(cfg, 16, 16, 45, 1.0) == 0


def test_op_entry_points_reject_misaligned_pointers():
    """The RMSNorm, RoPE and adaLN op entry points make 16-byte accesses: misaligned pointers
    are rejected before launch."""
    L = Z.lib()
    p, q = _fake(), _fake((1 << 20) + 4)
    rc = L.zdit_op_rmsnorm_mod(Z.ZDIT_BF16, 4, 256, q, p, None, None, 1e-6, p, None)
    assert rc == Z.ZDIT_EINVAL and "aligned" in Z.last_error()
    rc = L.zdit_op_rmsnorm_mod(Z.ZDIT_BF16, 4, 256, p, p, q, p, 1e-6, p, None)
    assert rc == Z.ZDIT_EINVAL and "aligned" in Z.last_error()
    rc = L.zdit_op_rope(Z.ZDIT_BF16, 1, 8, 1, Z.i32_array([8]), q, p, p, None)
    assert rc == Z.ZDIT_EINVAL and "aligned" in Z.last_error()
    rc = L.zdit_op_adaln(Z.ZDIT_BF16, 1, 256, 64, p, q, p, p, None)
    assert rc == Z.ZDIT_EINVAL and "aligned" in Z.last_error()


def test_ksplit_gemm_validates_before_launch():
    L = Z.lib()
    p = _fake()
    assert Z.zdit_op_gemm_ksplit_workspace(Z.ZDIT_EPI_BIAS, 10, 64, 64) == 0
    assert Z.zdit_op_gemm_ksplit_workspace(Z.ZDIT_EPI_STORE, 10, 60, 64) == 0
    assert Z.zdit_op_gemm_ksplit_workspace(Z.ZDIT_EPI_STORE, 10, 64, 96) == 0
    w1 = Z.zdit_op_gemm_ksplit_workspace(Z.ZDIT_EPI_STORE, 10, 3840, 10240)
    w2 = Z.zdit_op_gemm_ksplit_workspace(Z.ZDIT_EPI_STORE, 20, 3840, 10240)
    assert w1 > 0 and w2 >= 2 * w1 - 256  # partial planes grow with M, the split does not
    assert Z.zdit_op_gemm_ksplit_workspace(Z.ZDIT_EPI_SWIGLU, 10, 3840, 10240) > 0
    rc = L.zdit_op_gemm_ksplit(Z.ZDIT_EPI_BIAS, 4, 64, 64, p, p, None, p, p, p, 1 << 20, None)
    assert rc == Z.ZDIT_EUNSUPPORTED
    rc = L.zdit_op_gemm_ksplit(Z.ZDIT_EPI_SWIGLU, 4, 64, 64, p, p, None, None, p, p, 1 << 20, None)
    assert rc == Z.ZDIT_EINVAL
    rc = L.zdit_op_gemm_ksplit(Z.ZDIT_EPI_STORE, 4, 64, 64, p, p, None, None, p, p, 16, None)
    assert rc == Z.ZDIT_EWORKSPACE


def test_ksplit_plan_fits_two_panels_in_one_round():
    """The K-split plan for branches of at most 512 rows, read back through the workspace query
    (ranges x M x Nv fp32 partials, 256 bytes of slack): at the block's four shapes a two-panel
    branch (257..512 rows) takes at most 256 workgroups of 256 x 256 tiles, i.e. one round on 256
    CUs, and a plan of one range needs no partial plane."""
    D, H, M = 3840, 10240, 320
    shapes = [(Z.ZDIT_EPI_STORE, 3 * D, D, 45, 2), (Z.ZDIT_EPI_RESID, D, D, 15, 7),
              (Z.ZDIT_EPI_SWIGLU, H, D, 80, 1), (Z.ZDIT_EPI_RESID, D, H, 15, 8)]
    for epi, N, K, n_tiles, want in shapes:
        nv = 2 * N if epi == Z.ZDIT_EPI_SWIGLU else N
        ws = Z.zdit_op_gemm_ksplit_workspace(epi, M, N, K) - 256
        plane = M * nv * 4
        splits = 1 if ws == 0 else ws // plane
        assert ws in (0, -(-splits * plane // 256) * 256), (epi, N, K, ws)
        assert splits == want, (epi, N, K, splits)
        assert 2 * n_tiles * splits <= 256


def test_fused_qkv_attn_validates_before_launch():
    L = Z.lib()
    p = _fake()
    seq = Z.i32_array([96])
    # s_max not a multiple of 32
    rc = L.zdit_op_qkv_attn(1, 100, 2, Z.i32_array([100]), p, p, p, p, p, p, p, 1 << 30, None)
    assert rc == Z.ZDIT_EUNSUPPORTED and "multiple of 32" in Z.last_error()
    # seq_len outside 1..s_max
    rc = L.zdit_op_qkv_attn(1, 96, 2, Z.i32_array([97]), p, p, p, p, p, p, p, 1 << 30, None)
    assert rc == Z.ZDIT_EINVAL and "seq_len" in Z.last_error()
    # misaligned operand, then a workspace too small
    rc = L.zdit_op_qkv_attn(1, 96, 2, seq, _fake((1 << 20) + 2), p, p, p, p, p, p, 1 << 30, None)
    assert rc == Z.ZDIT_EINVAL and "aligned" in Z.last_error()
    rc = L.zdit_op_qkv_attn(1, 96, 2, seq, p, p, p, p, p, p, p, 1024, None)
    assert rc == Z.ZDIT_EWORKSPACE


def test_euler_step_rejects_missing_uncond_with_guidance():
    L = Z.lib()
    p = _fake()
    rc = L.zdit_euler_step(p, p, None, 10, 1.0, 1.0, 0.5, None, None)
    assert rc == Z.ZDIT_EINVAL and "v_uncond" in Z.last_error()
    assert L.zdit_euler_step(p, p, None, -1, 0.0, 1.0, 0.5, None, None) == Z.ZDIT_EINVAL
    # n == 0 is a no-op that launches nothing
    assert L.zdit_euler_step(None, None, None, 0, 0.0, 1.0, 0.5, None, None) == Z.ZDIT_OK


def test_stack_fwd_rejects_bad_caption_lengths():
    L = Z.lib()
    dims = synth.TINY
    cfg = Z.make_cfg(dims)
    blk = Z.zdit_block_w()
    for k in ("w_qkv", "w_out", "w1", "w3", "w2", "norm1", "norm2", "w_ada", "b_ada"):
        setattr(blk, k, 1 << 20)
    arr = (Z.zdit_block_w * 40)(*([blk] * 40))
    ctx = Z.zdit_block_w()
    for k in ("w_qkv", "w_out", "w1", "w3", "w2", "norm1", "norm2"):
        setattr(ctx, k, 1 << 20)
    carr = (Z.zdit_block_w * 4)(*([ctx] * 4))
    mw = Z.zdit_model_w()
    for k, _ in Z.zdit_model_w._fields_:
        if k not in ("noise_ref", "ctx_ref", "main"):
            setattr(mw, k, 1 << 20)
    mw.noise_ref = C.cast(arr, C.POINTER(Z.zdit_block_w))
    mw.main = C.cast(arr, C.POINTER(Z.zdit_block_w))
    mw.ctx_ref = C.cast(carr, C.POINTER(Z.zdit_block_w))
    p = _fake()
    for cl, why in (([0, 10], "cap_len"), ([45, 600], "cap_len"), ([45, 30], None)):
        rc = L.zdit_stack_fwd(C.byref(cfg), C.byref(mw), 2, 16, 16, p, 0, p, 64, Z.i32_array(cl),
                              Z.f32_array([0.5, 0.5]), p, p, 16, None)
        if why:
            assert rc == Z.ZDIT_EINVAL and why in Z.last_error()
        else:
            assert rc == Z.ZDIT_EWORKSPACE  # valid arguments, workspace too small: still no launch
    # odd latent size
    rc = L.zdit_stack_fwd(C.byref(cfg), C.byref(mw), 2, 15, 16, p, 0, p, 64, Z.i32_array([4, 4]),
                          Z.f32_array([0.5, 0.5]), p, p, 1 << 40, None)
    assert rc == Z.ZDIT_EINVAL
    # a main block without adaLN weights
    bad = (Z.zdit_block_w * 40)(*([ctx] * 40))
    mw.main = C.cast(bad, C.POINTER(Z.zdit_block_w))
    rc = L.zdit_stack_fwd(C.byref(cfg), C.byref(mw), 2, 16, 16, p, 0, p, 64, Z.i32_array([4, 4]),
                          Z.f32_array([0.5, 0.5]), p, p, 1 << 40, None)
    assert rc == Z.ZDIT_EINVAL and "adaLN" in Z.last_error()


def test_gemm_op_rejects_unsupported_k():
    L = Z.lib()
    p = _fake()
    assert L.zdit_op_gemm(Z.ZDIT_BF16, Z.ZDIT_EPI_STORE, 16, 16, 40, p, p, None, None, p, None) == Z.ZDIT_EUNSUPPORTED
    assert L.zdit_op_gemm(Z.ZDIT_BF16, Z.ZDIT_EPI_SWIGLU, 16, 16, 64, p, p, None, None, p, None) == Z.ZDIT_EINVAL
    assert L.zdit_op_gemm(Z.ZDIT_BF16, 9, 16, 16, 64, p, p, None, None, p, None) == Z.ZDIT_EINVAL


# ---------------------------------------------------------------- text encoder entry points
def _enc_setup(**over):
    ed = synth.ENC_TINY.replace(**over)
    cfg = Z.make_enc_cfg(ed)
    lw = (Z.zdit_enc_layer_w * 4)()
    for i in range(4):
        for f, _ in Z.zdit_enc_layer_w._fields_:
            setattr(lw[i], f, 4096 * (i + 1))  # aligned, never dereferenced: validation fails first
    w = Z.zdit_enc_w()
    w.embed = 1 << 20
    w.layers = C.cast(lw, C.POINTER(Z.zdit_enc_layer_w))
    return ed, cfg, w, lw


def _enc_call(cfg, w, batch, max_len, ids, lens, out=1 << 16, ws_bytes=1 << 30):
    L = Z.lib()
    ids = np.ascontiguousarray(ids, np.int32)
    return L.zdit_encoder_fwd(C.byref(cfg), C.byref(w), batch, max_len,
                              ids.ctypes.data_as(C.POINTER(C.c_int32)), Z.i32_array(lens),
                              C.c_void_p(out), C.c_void_p(1 << 24), ws_bytes, None)


def test_encoder_workspace_query():
    ed, cfg, _, _ = _enc_setup()
    n = Z.zdit_encoder_workspace(cfg, 2, 64)
    # at least the fp32-free activations: h, qkv, attention output, tables and ids
    M = 2 * 64
    assert n >= M * ed.hidden * 2 + M * (ed.n_heads + 2 * ed.n_kv_heads) * 128 * 2
    assert Z.zdit_encoder_workspace(cfg, 0, 64) == 0
    bad = Z.make_enc_cfg(synth.ENC_TINY.replace(head_dim=64))
    assert Z.zdit_encoder_workspace(bad, 2, 64) == 0


def test_encoder_rejects_bad_arguments_before_launch():
    ed, cfg, w, _ = _enc_setup()
    ids = synth.token_ids(2, 16, [9, 4], ed.vocab, 0)
    assert _enc_call(cfg, w, 2, 16, ids, [0, 4]) == Z.ZDIT_EINVAL          # empty row
    assert _enc_call(cfg, w, 2, 16, ids, [17, 4]) == Z.ZDIT_EINVAL         # past max_len
    bad_ids = ids.copy(); bad_ids[1, 3] = ed.vocab
    assert _enc_call(cfg, w, 2, 16, bad_ids, [9, 4]) == Z.ZDIT_EINVAL      # id out of range
    assert "ids[1][3]" in Z.last_error()
    neg = ids.copy(); neg[0, 0] = -1
    assert _enc_call(cfg, w, 2, 16, neg, [9, 4]) == Z.ZDIT_EINVAL
    assert _enc_call(cfg, w, 2, 16, ids, [9, 4], ws_bytes=1024) == Z.ZDIT_EWORKSPACE
    assert _enc_call(cfg, w, 0, 16, ids, [9, 4]) == Z.ZDIT_EINVAL
    _, cfg2, w2, lw2 = _enc_setup()
    lw2[1].w_up = None
    assert _enc_call(cfg2, w2, 2, 16, ids, [9, 4]) == Z.ZDIT_EINVAL
    assert "layer 1" in Z.last_error() and "w_up" in Z.last_error()
    _, cfg3, w3, _ = _enc_setup(n_kv_heads=3)
    assert _enc_call(cfg3, w3, 2, 16, ids, [9, 4]) == Z.ZDIT_EINVAL
    _, cfg4, w4, _ = _enc_setup(head_dim=64)
    assert _enc_call(cfg4, w4, 2, 16, ids, [9, 4]) == Z.ZDIT_EUNSUPPORTED
    _, cfg5, w5, _ = _enc_setup(inter=500)
    assert _enc_call(cfg5, w5, 2, 16, ids, [9, 4]) == Z.ZDIT_EUNSUPPORTED


def test_encoder_packed_flag_checks_before_launch():
    ed, cfg, w, _ = _enc_setup()
    ids = synth.token_ids(2, 16, [9, 4], ed.vocab, 0)
    cfg.flags = 2
    assert _enc_call(cfg, w, 2, 16, ids, [9, 4]) == Z.ZDIT_EINVAL          # unknown flag
    cfg.flags = Z.ZDIT_ENC_PACKED_WEIGHTS
    wide = synth.token_ids(2, 200, [9, 4], ed.vocab, 0)
    assert _enc_call(cfg, w, 2, 200, wide, [9, 4]) == Z.ZDIT_EUNSUPPORTED  # 400 rows: not the split-K path
    assert "packed" in Z.last_error()


def test_pack_and_packed_gemm_reject_bad_arguments_before_launch():
    L = Z.lib()
    a, b = C.c_void_p(1 << 20), C.c_void_p(1 << 24)
    assert L.zdit_op_pack_weights(24, 64, a, b, None) == Z.ZDIT_EUNSUPPORTED            # N % 16
    assert L.zdit_op_pack_weights(32, 48, a, b, None) == Z.ZDIT_EUNSUPPORTED            # K % 32
    assert L.zdit_op_pack_weights(32, 64, None, b, None) == Z.ZDIT_EINVAL
    assert L.zdit_op_pack_weights(32, 64, C.c_void_p((1 << 20) + 8), b, None) == Z.ZDIT_EINVAL
    assert L.zdit_op_pack_weights(32, 64, a, C.c_void_p((1 << 20) + 1024), None) == Z.ZDIT_EINVAL  # overlap
    args = (C.c_void_p(1 << 20), C.c_void_p(1 << 24), None, None, C.c_void_p(1 << 26), C.c_void_p(1 << 27), 1 << 20,
            None)
    assert L.zdit_op_gemm_splitk_packed(Z.ZDIT_EPI_STORE, 8, 24, 64, *args) == Z.ZDIT_EUNSUPPORTED  # N % 16
    assert L.zdit_op_gemm_splitk(Z.ZDIT_EPI_STORE, 8, 24, 64, *args[:5], C.c_void_p(1 << 27), 16,
                                 None) == Z.ZDIT_EWORKSPACE  # the row-major form takes N % 8


def test_encoder_ops_reject_bad_arguments_before_launch():
    L = Z.lib()
    ids = np.zeros((1, 8), np.int32)
    pids = ids.ctypes.data_as(C.POINTER(C.c_int32))
    # id past the vocabulary; dim not a multiple of 8
    ids[0, 2] = 50
    assert L.zdit_op_embed(1, 8, 64, 50, pids, Z.i32_array([8]), C.c_void_p(4096), C.c_void_p(8192),
                           C.c_void_p(1 << 20), 1 << 20, None) == Z.ZDIT_EINVAL
    ids[0, 2] = 0
    assert L.zdit_op_embed(1, 8, 60, 50, pids, Z.i32_array([8]), C.c_void_p(4096), C.c_void_p(8192),
                           C.c_void_p(1 << 20), 1 << 20, None) == Z.ZDIT_EINVAL
    # n_kv_heads must divide n_heads; seq_len within s_max
    assert L.zdit_op_attn_gqa(0, 1, 64, 6, 4, 1, Z.i32_array([64]), C.c_void_p(4096), C.c_void_p(8192),
                              C.c_void_p(1 << 20), 1 << 22, None) == Z.ZDIT_EINVAL
    assert L.zdit_op_attn_gqa(0, 1, 64, 8, 2, 1, Z.i32_array([65]), C.c_void_p(4096), C.c_void_p(8192),
                              C.c_void_p(1 << 20), 1 << 22, None) == Z.ZDIT_EINVAL
    assert L.zdit_op_attn_gqa(0, 1, 64, 8, 2, 1, Z.i32_array([64]), C.c_void_p(4096), C.c_void_p(8192),
                              C.c_void_p(1 << 20), 16, None) == Z.ZDIT_EWORKSPACE
    assert L.zdit_op_qknorm_rope(1, 8, 4, 2, Z.i32_array([9]), C.c_void_p(4096), C.c_void_p(4096),
                                 C.c_void_p(4096), C.c_void_p(4096), C.c_void_p(4096), 1e-6, None) == Z.ZDIT_EINVAL
    assert L.zdit_rope_tables(4, Z.i32_array([128, 0, 0]), 1e6, 1, 8, 0, 0, Z.i32_array([8]),
                              C.c_void_p(4096), C.c_void_p(8192), None) == Z.ZDIT_EINVAL


def test_splitk_workspace_depends_on_rows_only_through_m():
    """The split-K GEMM cuts K into ranges chosen from N and K alone, so its partial-sum workspace
    is (ranges x M x row width x 4 bytes) + 256 for every M: a row's summation order cannot
    depend on how many rows are present.  The encoder's down projection (N 2560, K 9728) runs
    10 ranges of 1024 columns; the gate/up projection (SwiGLU, row width 2N) one range."""
    for epi, N, K, ranges, width in [(Z.ZDIT_EPI_RESID, 2560, 9728, 10, 2560),
                                     (Z.ZDIT_EPI_SWIGLU, 9728, 2560, 1, 2 * 9728),
                                     (Z.ZDIT_EPI_STORE, 6144, 2560, 5, 6144)]:
        for M in (1, 55, 64, 65, 128, 256):
            assert Z.zdit_op_gemm_splitk_workspace(epi, M, N, K) == ranges * M * width * 4 + 256, (epi, M)
    assert Z.zdit_op_gemm_splitk_workspace(Z.ZDIT_EPI_STORE, 257, 2560, 9728) == 0
    assert Z.zdit_op_gemm_splitk_workspace(Z.ZDIT_EPI_STORE, 64, 2560, 9700) == 0
    assert Z.zdit_op_gemm_splitk_workspace(Z.ZDIT_EPI_BIAS, 64, 2560, 9728) == 0


# ------------------------------------------------------------------------------ VAE decoder
_FAKE = 0x10000   # an aligned address; argument checks never dereference it


def _fake_vae_w(vd, drop_shortcut=False, extra_shortcut=False):
    """zdit_vae_w with every pointer set to a dummy aligned address (validation only)."""
    def conv(c):
        c.w, c.b = _FAKE, _FAKE

    def norm(n):
        n.gamma, n.beta = _FAKE, _FAKE

    def resnet(r, cin, cout):
        norm(r.gn1), conv(r.conv1), norm(r.gn2), conv(r.conv2)
        if cin != cout and not drop_shortcut:
            conv(r.shortcut)

    w = Z.zdit_vae_w()
    conv(w.conv_in)
    c0 = vd.widths[-1]
    resnet(w.mid[0], c0, c0)
    resnet(w.mid[1], c0, c0)
    norm(w.attn.gn), conv(w.attn.qkv), conv(w.attn.out)
    keep = []
    for i, (cin, c, up) in enumerate(vd.stages):
        arr = (Z.zdit_vae_resnet * vd.resnets)()
        for j in range(vd.resnets):
            resnet(arr[j], cin if j == 0 else c, c)
        if extra_shortcut and i == 0:
            conv(arr[1].shortcut)
        keep.append(arr)
        w.stages[i] = C.cast(arr, C.POINTER(Z.zdit_vae_resnet))
        if up:
            conv(w.upconv[i])
    norm(w.norm_out), conv(w.conv_out)
    return w, keep


def _vae_call(cfg, w, B, h, wd, ws_bytes=None, latent=_FAKE, image=_FAKE, ws=_FAKE):
    L = Z.lib()
    n = ws_bytes if ws_bytes is not None else max(L.zdit_vae_workspace(C.byref(cfg), B, h, wd), 1)
    return L.zdit_vae_decode(C.byref(cfg), C.byref(w), B, h, wd, latent, image, ws, n, None)


def test_vae_workspace_query():
    cfg = Z.make_vae_cfg(synth.VAE_FULL)
    n1 = Z.zdit_vae_workspace(cfg, 1, 128, 128)
    # three activation buffers of the largest stage (1024^2 x 256 channels) and the 1 GiB of scores
    assert n1 >= 3 * 1024 * 1024 * 256 * 4 + 16384 * 16384 * 4
    assert Z.zdit_vae_workspace(cfg, 2, 128, 128) > n1
    for bad in ((1, 7, 8), (1, 8, 0), (0, 8, 8), (17, 8, 8), (1, 258, 8)):
        assert Z.zdit_vae_workspace(cfg, *bad) == 0
    assert Z.zdit_vae_workspace(Z.make_vae_cfg(synth.VAE_FULL.replace(widths=(128, 256, 384, 512))), 1, 8, 8) == 0
    assert Z.zdit_vae_workspace(Z.make_vae_cfg(synth.VAE_FULL, flags=4), 1, 8, 8) == 0


def test_vae_decode_rejects_bad_arguments_before_launch():
    vd = synth.VAE_TINY
    cfg = Z.make_vae_cfg(vd)
    w, keep = _fake_vae_w(vd)
    L = Z.lib()
    assert L.zdit_vae_decode(None, C.byref(w), 1, 8, 8, _FAKE, _FAKE, _FAKE, 1 << 30, None) == Z.ZDIT_EINVAL
    assert _vae_call(cfg, w, 1, 8, 8, ws_bytes=1024) == Z.ZDIT_EWORKSPACE
    assert _vae_call(cfg, w, 1, 8, 8, ws=_FAKE + 4) == Z.ZDIT_EINVAL
    assert _vae_call(cfg, w, 1, 8, 8, latent=None) == Z.ZDIT_EINVAL
    assert _vae_call(cfg, w, 1, 9, 8, ws_bytes=1 << 30) == Z.ZDIT_EUNSUPPORTED
    w2, keep2 = _fake_vae_w(vd, drop_shortcut=True)
    assert _vae_call(cfg, w2, 1, 8, 8) == Z.ZDIT_EINVAL and "shortcut" in Z.last_error()
    w3, keep3 = _fake_vae_w(vd, extra_shortcut=True)
    assert _vae_call(cfg, w3, 1, 8, 8) == Z.ZDIT_EINVAL and "shortcut" in Z.last_error()
    w4, keep4 = _fake_vae_w(vd)
    w4.stages[2] = None
    assert _vae_call(cfg, w4, 1, 8, 8) == Z.ZDIT_EINVAL and "stages[2]" in Z.last_error()
    w5, keep5 = _fake_vae_w(vd)
    w5.conv_out.w = _FAKE + 4
    assert _vae_call(cfg, w5, 1, 8, 8) == Z.ZDIT_EINVAL and "conv_out" in Z.last_error()
    bad = Z.make_vae_cfg(vd.replace(groups=3))
    assert _vae_call(bad, w, 1, 8, 8, ws_bytes=1 << 30) == Z.ZDIT_EINVAL
    bad = Z.make_vae_cfg(vd.replace(out_ch=5))
    assert _vae_call(bad, w, 1, 8, 8, ws_bytes=1 << 30) == Z.ZDIT_EUNSUPPORTED


def test_vae_ops_reject_bad_arguments_before_launch():
    L = Z.lib()
    conv = lambda **k: L.zdit_op_vae_conv(k.get("B", 1), k.get("H", 8), k.get("W", 8), k.get("cin", 32),
                                          k.get("cout", 32), k.get("ks", 3), k.get("up", 0), k.get("x", _FAKE),
                                          None, 0, k.get("w", _FAKE), _FAKE, None, _FAKE, None)
    assert conv(ks=2) == Z.ZDIT_EUNSUPPORTED
    assert conv(cin=30) == Z.ZDIT_EUNSUPPORTED
    assert conv(up=1, H=7) == Z.ZDIT_EINVAL
    assert conv(x=_FAKE + 8) == Z.ZDIT_EINVAL
    assert conv(w=None) == Z.ZDIT_EINVAL
    assert conv(B=0) == Z.ZDIT_EINVAL
    out = lambda **k: L.zdit_op_vae_conv_out(k.get("B", 1), 8, 8, k.get("cin", 128), k.get("cout", 3), _FAKE, _FAKE,
                                             _FAKE, _FAKE, _FAKE, None)
    assert out(cout=5) == Z.ZDIT_EUNSUPPORTED
    assert out(cin=130) == Z.ZDIT_EUNSUPPORTED
    gn = lambda **k: L.zdit_op_vae_groupnorm(1, 64, k.get("C", 64), k.get("g", 32), k.get("eps", 1e-6), _FAKE, _FAKE,
                                             _FAKE, _FAKE, _FAKE, k.get("ws", 1 << 20), None)
    assert gn(C=48) == Z.ZDIT_EUNSUPPORTED
    assert gn(g=3) == Z.ZDIT_EINVAL
    assert gn(eps=float("nan")) == Z.ZDIT_EINVAL
    assert gn(ws=16) == Z.ZDIT_EWORKSPACE
    assert L.zdit_op_vae_groupnorm_workspace(1, 64, 48, 32) == 0
    at = Z.zdit_vae_attn()
    assert L.zdit_op_vae_attention(1, 3, 5, 64, 32, 1e-6, C.byref(at), _FAKE, _FAKE, 1 << 30, None) == Z.ZDIT_EINVAL
    assert L.zdit_op_vae_attention(1, 4, 4, 64, 32, 1e-6, C.byref(at), _FAKE, _FAKE, 1 << 30, None) == Z.ZDIT_EINVAL
    assert L.zdit_op_vae_attention_workspace(1, 15, 64, 32) == 0
    assert L.zdit_op_vae_attention_workspace(1, 16, 64, 32) >= 16 * 16 * 4 + 16 * 3 * 64 * 4
