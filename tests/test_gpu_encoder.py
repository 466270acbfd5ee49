"""Text-encoder parity on the GPU: the encoder's kernels (embedding gather, per-head q/k norm +
RoPE, causal grouped-query attention) and the whole forward to hidden_states[-2], against the
encoder oracle on the same seeded inputs.  Bit-exact where the contract is (gather, RoPE
tables, pad-length and causality invariances); elsewhere within the bf16 tolerance of the
DiT path (rel-L2 <= 1e-2 and mean |error| <= 0.025 RMS)."""
import numpy as np
import pytest
import torch

import synth
from diffusion_transformer_text_s3_amd import binding as Z
from gpu_util import assert_bf16_result, bf16_values, dev, drift, host, note, rel_l2
from oracle import encoder_oracle as E

pytestmark = pytest.mark.gpu
BF, F32P = Z.ZDIT_BF16, Z.ZDIT_FP32_DEBUG


def _rng(seed):
    return np.random.default_rng(seed)


def _text_tables(batch, s_max, lens, theta=1e6):
    cos = torch.empty((batch, s_max, 64), device="cuda")
    sin = torch.empty_like(cos)
    Z.zdit_rope_tables(Z.ZDIT_SEQ_TEXT, [128, 0, 0], theta, batch, s_max, 0, 0, lens, cos, sin)
    return cos, sin


# ------------------------------------------------------------------------------- split-K GEMM
def _sk_inputs(M, N, K, seed):
    g = _rng(seed)
    A = bf16_values(g.standard_normal((M, K)).astype(np.float32))
    B = bf16_values((0.05 * g.standard_normal((N, K))).astype(np.float32))
    B2 = bf16_values((0.05 * g.standard_normal((N, K))).astype(np.float32))
    return A, B, B2


def _sk_tol(K):
    """fp32 accumulation over K in ranges, then the ranges summed: relative to sum |a||b|."""
    return 2e-6 + 1e-9 * K


def _splitk(epi, M, N, K, A, B, B2, vec, C):
    ws = Z.workspace(Z.zdit_op_gemm_splitk_workspace(epi, M, N, K))
    Z.zdit_op_gemm_splitk(epi, M, N, K, dev(A, torch.bfloat16), dev(B, torch.bfloat16),
                          None if B2 is None else dev(B2, torch.bfloat16), None if vec is None else dev(vec), C, ws)


@pytest.mark.parametrize("M,N,K", [(128, 6144, 2560), (1, 64, 64), (77, 520, 192), (256, 2560, 9728)])
def test_gemm_splitk_store(M, N, K):
    note(f"gemm split-K STORE M={M} N={N} K={K}")
    A, B, _ = _sk_inputs(M, N, K, 60)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _splitk(Z.ZDIT_EPI_STORE, M, N, K, A, B, None, None, C)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    bound = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T
    assert_bf16_result(host(C), ref, _sk_tol(K) * bound)


@pytest.mark.parametrize("M,N,K", [(128, 2560, 4096), (200, 264, 9728)])
def test_gemm_splitk_resid_gate(M, N, K):
    note(f"gemm split-K RESID M={M} N={N} K={K}")
    A, B, _ = _sk_inputs(M, N, K, 61)
    g = _rng(62)
    C0 = (100 * g.standard_normal((M, N))).astype(np.float32)
    gate = g.standard_normal(N).astype(np.float32)
    for vec in (gate, None):
        C = dev(C0)
        _splitk(Z.ZDIT_EPI_RESID, M, N, K, A, B, None, vec, C)
        gv = np.ones(N) if vec is None else gate.astype(np.float64)
        ref = C0 + gv * (A.astype(np.float64) @ B.astype(np.float64).T)
        bound = np.abs(gv) * (np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T)
        assert np.all(np.abs(host(C) - ref) <= _sk_tol(K) * bound + 1e-6 * np.abs(C0) + 1e-6)


@pytest.mark.parametrize("M,N,K", [(128, 9728, 2560), (33, 136, 128), (70, 200, 256), (33, 136, 2560)])
def test_gemm_splitk_swiglu(M, N, K):
    note(f"gemm split-K SWIGLU M={M} N={N} K={K}")
    A, B, B2 = _sk_inputs(M, N, K, 63)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _splitk(Z.ZDIT_EPI_SWIGLU, M, N, K, A, B, B2, None, C)
    A64, B64, B264 = A.astype(np.float64), B.astype(np.float64), B2.astype(np.float64)
    a1, a3 = A64 @ B64.T, A64 @ B264.T
    e1 = _sk_tol(K) * (np.abs(A64) @ np.abs(B64).T)
    e3 = _sk_tol(K) * (np.abs(A64) @ np.abs(B264).T)
    silu = lambda z: z / (1 + np.exp(-z))
    u = silu(a1) * a3
    assert_bf16_result(host(C), u, 1.1 * e1 * np.abs(a3) + np.abs(silu(a1)) * e3 + 1e-6 * np.abs(u) + e1 * e3)


@pytest.mark.parametrize("epi", [Z.ZDIT_EPI_STORE, Z.ZDIT_EPI_RESID])
@pytest.mark.parametrize("K", [320, 384, 576])
def test_gemm_splitk_partial_last_chunk_ignores_memory_after_a(epi, K):
    """K not a multiple of 256: the last K range ends inside a 256-column A chunk.  A sits at the
    start of a NaN-filled allocation, so the bytes after its last row are NaN; the result must
    be finite and match the float64 reference (columns past K are neither read nor summed)."""
    M, N = 70, 264
    note(f"gemm split-K partial last chunk epi={epi} K={K}, NaN after A")
    A, B, _ = _sk_inputs(M, N, K, 65)
    buf = torch.full((M * K + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[:M * K] = dev(A, torch.bfloat16).reshape(-1)
    Ad = buf[:M * K].view(M, K)
    ws = Z.workspace(Z.zdit_op_gemm_splitk_workspace(epi, M, N, K))
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    bound = _sk_tol(K) * (np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T)
    if epi == Z.ZDIT_EPI_STORE:
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        Z.zdit_op_gemm_splitk(epi, M, N, K, Ad, dev(B, torch.bfloat16), None, None, C, ws)
        got = host(C)
        assert np.isfinite(got).all()
        assert_bf16_result(got, ref, bound)
    else:
        C0 = _rng(66).standard_normal((M, N)).astype(np.float32)
        C = dev(C0)
        Z.zdit_op_gemm_splitk(epi, M, N, K, Ad, dev(B, torch.bfloat16), None, None, C, ws)
        got = host(C)
        assert np.isfinite(got).all()
        assert np.all(np.abs(got - (C0 + ref)) <= bound + 1e-6 * np.abs(C0) + 1e-6)


def test_pack_weights_layout():
    """zdit_op_pack_weights against its definition: chunk l of slab t of band b holds columns
    32 t + 8 (l // 16) .. + 7 of row 16 b + l % 16."""
    note("pack weights layout 48 x 96")
    g = _rng(70)
    N, K = 48, 96
    W = bf16_values(g.standard_normal((N, K)).astype(np.float32))
    src = dev(W, torch.bfloat16)
    dst = torch.empty_like(src)
    Z.zdit_op_pack_weights(N, K, src, dst)
    got = host(dst).reshape(N // 16, K // 32, 64, 8)
    b, t, l, e = np.meshgrid(np.arange(N // 16), np.arange(K // 32), np.arange(64), np.arange(8), indexing="ij")
    want = W[16 * b + l % 16, 32 * t + 8 * (l // 16) + e]
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("epi,M,N,K", [(Z.ZDIT_EPI_STORE, 55, 6144, 2560), (Z.ZDIT_EPI_RESID, 55, 2560, 4096),
                                       (Z.ZDIT_EPI_RESID, 55, 2560, 9728), (Z.ZDIT_EPI_SWIGLU, 55, 9728, 2560),
                                       (Z.ZDIT_EPI_SWIGLU, 33, 208, 2560), (Z.ZDIT_EPI_STORE, 7, 64, 64)])
def test_gemm_splitk_packed_bit_identical(epi, M, N, K):
    """Weights packed by zdit_op_pack_weights give the row-major call's bits: same sums, same
    order, only the weights' addresses differ (ranges of two and four resident chunks, the
    double-buffered gate/up range, SwiGLU in the GEMM and through the reduction)."""
    note(f"gemm split-K packed vs row-major epi={epi} M={M} N={N} K={K}")
    A, B, B2 = _sk_inputs(M, N, K, 71)
    Ad, Bd = dev(A, torch.bfloat16), dev(B, torch.bfloat16)
    B2d = dev(B2, torch.bfloat16) if epi == Z.ZDIT_EPI_SWIGLU else None
    vec = dev((1.0 + 0.1 * _rng(72).standard_normal(N)).astype(np.float32)) if epi == Z.ZDIT_EPI_RESID else None
    if epi == Z.ZDIT_EPI_RESID:
        c0 = dev(_rng(73).standard_normal((M, N)).astype(np.float32))
        C1, C2 = c0.clone(), c0.clone()
    else:
        C1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        C2 = C1.clone()
    Bp = torch.empty_like(Bd)
    Z.zdit_op_pack_weights(N, K, Bd, Bp)
    B2p = None
    if B2d is not None:
        B2p = torch.empty_like(B2d)
        Z.zdit_op_pack_weights(N, K, B2d, B2p)
    ws = Z.workspace(Z.zdit_op_gemm_splitk_workspace(epi, M, N, K))
    Z.zdit_op_gemm_splitk(epi, M, N, K, Ad, Bd, B2d, vec, C1, ws)
    Z.zdit_op_gemm_splitk_packed(epi, M, N, K, Ad, Bp, B2p, vec, C2, ws)
    assert torch.equal(C1, C2)


def test_gemm_splitk_rows_do_not_depend_on_m():
    """The K ranges depend on N and K only: rows computed with 50 or 256 rows are identical."""
    N, K = 2560, 9728
    note("gemm split-K rows independent of M")
    A, B, _ = _sk_inputs(256, N, K, 64)
    C1 = torch.empty((256, N), dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty((50, N), dtype=torch.bfloat16, device="cuda")
    _splitk(Z.ZDIT_EPI_STORE, 256, N, K, A, B, None, None, C1)
    _splitk(Z.ZDIT_EPI_STORE, 50, N, K, A[:50], B, None, None, C2)
    np.testing.assert_array_equal(host(C1)[:50], host(C2))


# ------------------------------------------------------------------------------- tables
def test_text_rope_tables_match_oracle():
    lens = [300, 77]
    note(f"text rope tables lens={lens}")
    cos, sin = _text_tables(2, 300, lens)
    c, s = host(cos), host(sin)
    rc, rs = E.rope_tables_1d(300, 128, 1e6)
    for b, L in enumerate(lens):
        # float64 angles rounded once on both sides: at most one fp32 ulp apart
        np.testing.assert_allclose(c[b, :L], rc[:L], rtol=0, atol=1.2e-7)
        np.testing.assert_allclose(s[b, :L], rs[:L], rtol=0, atol=1.2e-7)
        assert np.all(c[b, L:] == 1) and np.all(s[b, L:] == 0)


# ------------------------------------------------------------------------------- embedding
def test_embed_gather_exact_and_padding_zero():
    vocab, dim, lens, L = 1000, 256, [37, 5, 64], 64
    note(f"embed vocab={vocab} dim={dim} lens={lens}")
    table = bf16_values(_rng(1).standard_normal((vocab, dim)).astype(np.float32))
    ids = synth.token_ids(3, L, lens, vocab, 2)
    ids[0, 0], ids[1, 4] = vocab - 1, 0
    out = torch.full((3, L, dim), 7.0, device="cuda")
    ws = Z.workspace(Z.zdit_op_embed_workspace(3, L))
    Z.zdit_op_embed(3, L, dim, vocab, ids, lens, dev(table, torch.bfloat16), out, ws)
    got = host(out)
    for b, n in enumerate(lens):
        np.testing.assert_array_equal(got[b, :n], table[ids[b, :n]])
        assert np.all(got[b, n:] == 0)


# ------------------------------------------------------------------------------- q/k norm + RoPE
def test_qknorm_rope_matches_oracle_within_one_bf16_ulp():
    B, S, nq, nkv = 2, 70, 8, 2
    lens = [70, 33]
    note(f"qknorm+rope B={B} S={S} nq={nq} nkv={nkv} lens={lens}")
    g = _rng(3)
    W = (nq + 2 * nkv) * 128
    x = bf16_values((g.standard_normal((B, S, W)) * 2.0).astype(np.float32))
    gq = (1 + 0.1 * g.standard_normal(128)).astype(np.float32)
    gk = (1 + 0.1 * g.standard_normal(128)).astype(np.float32)
    cos, sin = _text_tables(B, S, lens)
    t = dev(x, torch.bfloat16)
    Z.zdit_op_qknorm_rope(B, S, nq, nkv, lens, t, dev(gq), dev(gk), cos, sin, 1e-6)
    got = host(t)
    rc, rs = E.rope_tables_1d(S)
    for b, L in enumerate(lens):
        q = x[b, :L, :nq * 128].reshape(L, nq, 128)
        k = x[b, :L, nq * 128:(nq + nkv) * 128].reshape(L, nkv, 128)
        rq = E.rope_rotate_half(E.head_norm(q, gq, 1e-6), rc[:L], rs[:L]).reshape(L, -1)
        rk = E.rope_rotate_half(E.head_norm(k, gk, 1e-6), rc[:L], rs[:L]).reshape(L, -1)
        for part, ref in ((got[b, :L, :nq * 128], rq), (got[b, :L, nq * 128:(nq + nkv) * 128], rk)):
            # one rounding to bf16 of an fp32 value within a few fp32 ulps of the oracle's
            err = np.abs(part - ref)
            assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-6), err.max()
        np.testing.assert_array_equal(got[b, :L, (nq + nkv) * 128:], x[b, :L, (nq + nkv) * 128:])  # v untouched
        np.testing.assert_array_equal(got[b, L:], x[b, L:])  # rows past the length untouched


# ------------------------------------------------------------------------------- attention
def _gqa_qkv(B, S, nq, nkv, seed, scale=1.0):
    g = _rng(seed)
    W = (nq + 2 * nkv) * 128
    x = g.standard_normal((B, S, W)).astype(np.float32)
    x[:, :, :(nq + nkv) * 128] *= scale
    return bf16_values(x)


def _attn_ref(x, L, nq, nkv, causal):
    q = x[:L, :nq * 128].reshape(L, nq, 128)
    k = x[:L, nq * 128:(nq + nkv) * 128].reshape(L, nkv, 128)
    v = x[:L, (nq + nkv) * 128:].reshape(L, nkv, 128)
    if causal:
        return E.causal_gqa_attention(q, k, v).reshape(L, nq * 128)
    g = nq // nkv
    kk, vv = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    from oracle import attention
    return attention(q, kk, vv).reshape(L, nq * 128)


def _run_gqa(prec, x, B, S, nq, nkv, causal, lens):
    dt = torch.bfloat16 if prec == BF else torch.float32
    out = torch.full((B, S, nq * 128), 7.0, dtype=dt, device="cuda")
    ws = Z.workspace(Z.zdit_op_attn_gqa_workspace(prec, B, S, nkv))
    Z.zdit_op_attn_gqa(prec, B, S, nq, nkv, causal, lens, dev(x, dt), out, ws)
    return host(out)


@pytest.mark.parametrize("nq,nkv,causal", [(8, 2, 1), (8, 2, 0), (4, 4, 1), (32, 8, 1)])
def test_attn_gqa_matches_oracle(nq, nkv, causal):
    B, S, lens = 2, 200, [200, 131]
    note(f"attn gqa nq={nq} nkv={nkv} causal={causal} lens={lens}")
    x = _gqa_qkv(B, S, nq, nkv, 10 + nq + nkv + causal)
    got = _run_gqa(BF, x, B, S, nq, nkv, causal, lens)
    for b, L in enumerate(lens):
        ref = _attn_ref(x[b], L, nq, nkv, causal)
        assert rel_l2(got[b, :L], ref) < 1e-2
        assert np.abs(got[b, :L] - ref).max() < 0.05
        assert np.all(got[b, L:] == 0)


def test_attn_gqa_causal_key_block_counts():
    """Causal masking with tiles whose first query sits in every position of the key loop
    (1 .. 9 key blocks, ragged last blocks), large scores so the running max moves."""
    S, nq, nkv = 544, 4, 2
    lens = [1, 63, 64, 65, 200, 257, 300, 513, 544]
    note(f"attn gqa causal block counts lens={lens}")
    x = _gqa_qkv(len(lens), S, nq, nkv, 20, scale=2.0)
    got = _run_gqa(BF, x, len(lens), S, nq, nkv, 1, lens)
    for b, L in enumerate(lens):
        ref = _attn_ref(x[b], L, nq, nkv, True)
        assert rel_l2(got[b, :L], ref) < 1e-2, L
        assert np.abs(got[b, :L] - ref).max() < 0.05, L
        assert np.all(got[b, L:] == 0)


def test_attn_gqa_fp32_debug_path():
    B, S, nq, nkv, lens = 2, 90, 8, 2, [90, 41]
    note("attn gqa fp32 debug causal")
    x = _gqa_qkv(B, S, nq, nkv, 30)
    got = _run_gqa(F32P, x, B, S, nq, nkv, 1, lens)
    for b, L in enumerate(lens):
        np.testing.assert_allclose(got[b, :L], _attn_ref(x[b], L, nq, nkv, True), rtol=1e-5, atol=1e-5)


def test_attn_gqa_equals_dit_attention_when_heads_match():
    """n_kv_heads == n_heads and no causal mask is the DiT's joint attention, bit for bit."""
    B, S, nh, lens = 2, 160, 3, [160, 97]
    note("attn gqa == dit attention")
    x = _gqa_qkv(B, S, nh, nh, 40)
    got = _run_gqa(BF, x, B, S, nh, nh, 0, lens)
    out = torch.empty((B, S, nh * 128), dtype=torch.bfloat16, device="cuda")
    ws = Z.workspace(Z.zdit_op_attn_workspace(BF, B, S, nh))
    Z.zdit_op_attn(BF, B, S, nh, lens, dev(x, torch.bfloat16), out, ws)
    np.testing.assert_array_equal(got, host(out))


def test_attn_gqa_causal_ignores_later_tokens_bit_exact():
    B, S, nq, nkv, L = 1, 300, 8, 2, 300
    note("attn gqa causal: later tokens change nothing")
    x = _gqa_qkv(B, S, nq, nkv, 50)
    a = _run_gqa(BF, x, B, S, nq, nkv, 1, [L])
    y = x.copy()
    y[:, 150:, nq * 128:] = bf16_values(_rng(51).standard_normal(y[:, 150:, nq * 128:].shape).astype(np.float32) * 5)
    b = _run_gqa(BF, y, B, S, nq, nkv, 1, [L])
    np.testing.assert_array_equal(a[0, :150], b[0, :150])
    assert not np.array_equal(a[0, 150:], b[0, 150:])


# ------------------------------------------------------------------------------- whole encoder
def _encoder_run(ed, W, ids, lens, max_len=None):
    B = ids.shape[0]
    L = ids.shape[1] if max_len is None else max_len
    if L != ids.shape[1]:
        wide = np.zeros((B, L), np.int32)
        wide[:, :ids.shape[1]] = ids
        ids = wide
    m = Z.upload_encoder(W)
    cfg = Z.make_enc_cfg(ed)
    out = torch.full((B, L, ed.hidden), 3.0, device="cuda")
    ws = Z.workspace(Z.zdit_encoder_workspace(cfg, B, L))
    Z.zdit_encoder_fwd(cfg, m, B, L, ids, lens, out, ws)
    return host(out)


def _check_vs_oracle(got, ref, lens):
    for b, L in enumerate(lens):
        assert rel_l2(got[b, :L], ref[b, :L]) <= 1e-2
        assert drift(got[b, :L], ref[b, :L]) <= 0.025
        assert np.all(got[b, L:] == 0)


def test_encoder_tiny_matches_oracle():
    ed = synth.ENC_TINY
    lens = [37, 12]
    note(f"encoder tiny {ed} lens={lens}")
    W = synth.encoder_weights(ed, 5, ed.n_layers - 1)
    ids = synth.token_ids(2, 40, lens, ed.vocab, 6)
    got = _encoder_run(ed, W, ids, lens)
    _check_vs_oracle(got, E.encoder_penultimate(ids, lens, W, ed), lens)


def test_encoder_tiny_deep_matches_oracle():
    """A 12-block tiny encoder (11 computed): bf16 drift stays within the tolerance."""
    ed = synth.ENC_TINY.replace(n_layers=12)
    lens = [64, 29, 1]
    note(f"encoder tiny deep lens={lens}")
    W = synth.encoder_weights(ed, 7, ed.n_layers - 1)
    ids = synth.token_ids(3, 64, lens, ed.vocab, 8)
    got = _encoder_run(ed, W, ids, lens)
    _check_vs_oracle(got, E.encoder_penultimate(ids, lens, W, ed), lens)


def test_encoder_main_gemm_path_matches_oracle():
    """Over 256 rows in all (3 x 100) the projections run on the main GEMM instead of split-K."""
    ed = synth.ENC_TINY
    lens = [100, 61, 2]
    note(f"encoder main-GEMM path lens={lens}")
    W = synth.encoder_weights(ed, 15, ed.n_layers - 1)
    ids = synth.token_ids(3, 100, lens, ed.vocab, 16)
    got = _encoder_run(ed, W, ids, lens)
    _check_vs_oracle(got, E.encoder_penultimate(ids, lens, W, ed), lens)


def test_encoder_valid_rows_do_not_depend_on_padding_length():
    ed = synth.ENC_TINY
    lens = [33, 7]
    note("encoder pad-length independence")
    W = synth.encoder_weights(ed, 9, ed.n_layers - 1)
    ids = synth.token_ids(2, 33, lens, ed.vocab, 10)
    a = _encoder_run(ed, W, ids, lens)
    b = _encoder_run(ed, W, ids, lens, max_len=97)
    for i, L in enumerate(lens):
        np.testing.assert_array_equal(a[i, :L], b[i, :L])
    assert np.all(b[:, 33:] == 0)


def test_encoder_ids_inline_and_copied_paths_agree():
    """Up to 512 tokens (batch x max_len) the ids travel in the kernel arguments, beyond that they
    are copied into the workspace: the valid rows are bit-identical either way (both shapes run
    the main-GEMM projections) and match the oracle."""
    ed = synth.ENC_TINY
    lens = [250, 31]
    note("encoder ids inline (2 x 256) vs copied (2 x 300)")
    W = synth.encoder_weights(ed, 17, ed.n_layers - 1)
    ids = synth.token_ids(2, 256, lens, ed.vocab, 18)
    a = _encoder_run(ed, W, ids, lens)                # 512 tokens: inline
    b = _encoder_run(ed, W, ids, lens, max_len=300)   # 600 tokens: copied
    for i, L in enumerate(lens):
        np.testing.assert_array_equal(a[i, :L], b[i, :L])
    _check_vs_oracle(a, E.encoder_penultimate(ids, lens, W, ed), lens)


def test_encoder_is_causal_bit_exact():
    ed = synth.ENC_TINY
    note("encoder causality")
    W = synth.encoder_weights(ed, 11, ed.n_layers - 1)
    ids = synth.token_ids(1, 48, [48], ed.vocab, 12)
    a = _encoder_run(ed, W, ids, [48])
    ids2 = ids.copy()
    ids2[0, 20:] = (ids2[0, 20:] + 17) % ed.vocab
    b = _encoder_run(ed, W, ids2, [48])
    np.testing.assert_array_equal(a[0, :20], b[0, :20])
    assert not np.array_equal(a[0, 20:], b[0, 20:])


def test_encoder_full_width_two_blocks_matches_oracle():
    """The pinned encoder's widths (hidden 2560, 32 / 8 heads, intermediate 9728), two blocks,
    on the DiT's caption lengths (a 45-token prompt and a 10-token negative)."""
    ed = synth.ENC_FULL.replace(n_layers=3, vocab=4096)
    lens = [45, 10]
    note(f"encoder full width 2 blocks lens={lens}")
    W = synth.encoder_weights(ed, 13, ed.n_layers - 1)
    ids = synth.token_ids(2, 64, lens, ed.vocab, 14)
    got = _encoder_run(ed, W, ids, lens)
    _check_vs_oracle(got, E.encoder_penultimate(ids, lens, W, ed), lens)


def test_encoder_packed_weights_bit_identical():
    """The forward with ZDIT_ENC_PACKED_WEIGHTS and zdit_op_pack_weights'd projections equals the
    row-major forward bit for bit, at the pinned widths on the DiT's caption lengths."""
    ed = synth.ENC_FULL.replace(n_layers=3, vocab=4096)
    lens = [45, 10]
    note("encoder packed vs row-major weights, full width, 2 blocks")
    W = synth.encoder_weights(ed, 16, ed.n_layers - 1)
    ids = synth.token_ids(2, 64, lens, ed.vocab, 17)
    m = Z.upload_encoder(W)
    mp = Z.pack_encoder(m)
    outs = []
    for cfg, mm in ((Z.make_enc_cfg(ed), m), (Z.make_enc_cfg(ed, Z.ZDIT_ENC_PACKED_WEIGHTS), mp)):
        out = torch.full((2, 64, ed.hidden), 3.0, device="cuda")
        ws = Z.workspace(Z.zdit_encoder_workspace(cfg, 2, 64))
        Z.zdit_encoder_fwd(cfg, mm, 2, 64, ids, lens, out, ws)
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
