"""Single-kernel parity on the GPU: each zdit_op_* entry point against the oracle on the same
seeded inputs.  Bit-exact where the contract is bit-exact (RoPE, Euler/CFG/unscale, index
kernels, tables to 1 ulp); elsewhere within a stated tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from diffusion_transformer_text_s3_amd import binding as Z
from gpu_util import assert_attention_close, assert_bf16_result, bf16_values, dev, host, note, rel_l2, ulp_diff_bf16

pytestmark = pytest.mark.gpu
BF, F32P = Z.ZDIT_BF16, Z.ZDIT_FP32_DEBUG


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------- GEMM
def _gemm_inputs(M, N, K, seed, two_b=False):
    g = _rng(seed)
    A = bf16_values(g.standard_normal((M, K)).astype(np.float32))
    B = bf16_values((0.05 * g.standard_normal((N, K))).astype(np.float32))
    B2 = bf16_values((0.05 * g.standard_normal((N, K))).astype(np.float32)) if two_b else None
    return A, B, B2


@pytest.mark.parametrize("M,N,K", [(300, 520, 192), (64, 64, 64), (1, 3840, 128), (513, 257, 640)])
def test_gemm_bf16_bias_fp32_out(M, N, K):
    note(f"gemm bf16 EPI_BIAS M={M} N={N} K={K}")
    A, B, _ = _gemm_inputs(M, N, K, 1)
    bias = _rng(2).standard_normal(N).astype(np.float32)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Z.zdit_op_gemm(BF, Z.ZDIT_EPI_BIAS, M, N, K, dev(A, torch.bfloat16), dev(B, torch.bfloat16), None, dev(bias), C)
    got = host(C)
    ref = A.astype(np.float64) @ B.astype(np.float64).T + bias
    bound = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T
    assert np.all(np.abs(got - ref) <= 2e-6 * bound + 1e-6 * np.abs(bias) + 1e-7)


@pytest.mark.parametrize("M,N,K", [(300, 520, 192), (257, 1000, 256)])
def test_gemm_bf16_store_rounds_once(M, N, K):
    note(f"gemm bf16 EPI_STORE M={M} N={N} K={K}")
    A, B, _ = _gemm_inputs(M, N, K, 3)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Z.zdit_op_gemm(BF, Z.ZDIT_EPI_STORE, M, N, K, dev(A, torch.bfloat16), dev(B, torch.bfloat16), None, None, C)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    bound = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T
    assert_bf16_result(host(C), ref, 2e-6 * bound)


def test_gemm_bf16_resid_gate():
    M, N, K = 300, 520, 192
    note(f"gemm bf16 EPI_RESID M={M} N={N} K={K}")
    A, B, _ = _gemm_inputs(M, N, K, 4)
    g = _rng(5)
    C0 = (100 * g.standard_normal((M, N))).astype(np.float32)
    gate = g.standard_normal(N).astype(np.float32)
    C = dev(C0)
    Z.zdit_op_gemm(BF, Z.ZDIT_EPI_RESID, M, N, K, dev(A, torch.bfloat16), dev(B, torch.bfloat16), None, dev(gate), C)
    ref = C0 + gate * (A.astype(np.float64) @ B.astype(np.float64).T)
    bound = np.abs(gate) * (np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T)
    assert np.all(np.abs(host(C) - ref) <= 2e-6 * bound + 1e-6 * np.abs(C0) + 1e-6)
    # gate NULL means 1
    C = dev(C0)
    Z.zdit_op_gemm(BF, Z.ZDIT_EPI_RESID, M, N, K, dev(A, torch.bfloat16), dev(B, torch.bfloat16), None, None, C)
    ref1 = C0 + (A.astype(np.float64) @ B.astype(np.float64).T)
    assert np.abs(host(C) - ref1).max() < 1e-3


def test_gemm_bf16_swiglu():
    M, N, K = 300, 384, 256
    note(f"gemm bf16 EPI_SWIGLU M={M} N={N} K={K}")
    A, B, B2 = _gemm_inputs(M, N, K, 6, two_b=True)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Z.zdit_op_gemm(BF, Z.ZDIT_EPI_SWIGLU, M, N, K, dev(A, torch.bfloat16), dev(B, torch.bfloat16),
                   dev(B2, torch.bfloat16), None, C)
    _check_swiglu(host(C), A.astype(np.float64), B.astype(np.float64), B2.astype(np.float64))


def _check_swiglu(got, A, B, B2):
    """u = SiLU(a1) a3 from fp32 sums a1, a3 (each within 2e-6 sum|a||b| of exact), rounded
    once to bf16."""
    a1, a3 = A @ B.T, A @ B2.T
    e1 = 2e-6 * (np.abs(A) @ np.abs(B).T)
    e3 = 2e-6 * (np.abs(A) @ np.abs(B2).T)
    u = O.silu(a1) * a3
    err = 1.1 * e1 * np.abs(a3) + np.abs(O.silu(a1)) * e3 + 1e-6 * np.abs(u) + e1 * e3
    assert_bf16_result(got, u, err)


def _ksplit(epi, M, N, K, A, B, B2, vec, C):
    ws = Z.workspace(Z.zdit_op_gemm_ksplit_workspace(epi, M, N, K))
    Z.zdit_op_gemm_ksplit(epi, M, N, K, dev(A, torch.bfloat16), dev(B, torch.bfloat16),
                          None if B2 is None else dev(B2, torch.bfloat16), None if vec is None else dev(vec), C, ws)


@pytest.mark.parametrize("M,N,K", [(77, 520, 192), (320, 3840, 3840), (640, 1032, 1280), (300, 11520, 3840)])
def test_gemm_ksplit_store_and_resid(M, N, K):
    """The K-split form of the block GEMMs (branches of <= 512 rows): fp32 partial products over
    K ranges summed in order, then the epilogue; within the same fp32 accumulation bound."""
    note(f"gemm K-split STORE / RESID M={M} N={N} K={K}")
    A, B, _ = _gemm_inputs(M, N, K, 30)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    bound = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _ksplit(Z.ZDIT_EPI_STORE, M, N, K, A, B, None, None, C)
    assert_bf16_result(host(C), ref, 2e-6 * bound)
    g = _rng(31)
    C0 = (100 * g.standard_normal((M, N))).astype(np.float32)
    gate = g.standard_normal(N).astype(np.float32)
    C = dev(C0)
    _ksplit(Z.ZDIT_EPI_RESID, M, N, K, A, B, None, gate, C)
    r = C0 + gate * ref
    assert np.all(np.abs(host(C) - r) <= 2e-6 * np.abs(gate) * bound + 1e-6 * np.abs(C0) + 1e-6)


@pytest.mark.parametrize("M,N,K", [(77, 384, 256), (320, 10240, 3840)])
def test_gemm_ksplit_swiglu(M, N, K):
    note(f"gemm K-split SWIGLU M={M} N={N} K={K}")
    A, B, B2 = _gemm_inputs(M, N, K, 32, two_b=True)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _ksplit(Z.ZDIT_EPI_SWIGLU, M, N, K, A, B, B2, None, C)
    _check_swiglu(host(C), A.astype(np.float64), B.astype(np.float64), B2.astype(np.float64))


def test_gemm_ksplit_one_range_is_the_whole_k_gemm():
    """Where the K-split plan has one range (w1/w3 at 3840 wide) the K-split entry point runs the
    whole-K kernel with its epilogue: bit-identical to zdit_op_gemm at the 256 px block's rows."""
    M, N, K = 320, 10240, 3840
    note(f"gemm K-split one range == whole-K M={M} N={N} K={K}")
    assert Z.zdit_op_gemm_ksplit_workspace(Z.ZDIT_EPI_SWIGLU, M, N, K) == 256
    A, B, B2 = _gemm_inputs(M, N, K, 34, two_b=True)
    c1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    c2 = torch.empty_like(c1)
    _ksplit(Z.ZDIT_EPI_SWIGLU, M, N, K, A, B, B2, None, c1)
    Z.zdit_op_gemm(Z.ZDIT_BF16, Z.ZDIT_EPI_SWIGLU, M, N, K, dev(A, torch.bfloat16), dev(B, torch.bfloat16),
                   dev(B2, torch.bfloat16), None, c2)
    assert torch.equal(c1, c2)


def test_gemm_ksplit_rows_do_not_depend_on_m():
    """The K ranges depend on N and K only: rows computed among 40 or 600 rows are identical,
    rows past the first 256-row panel (whose last panel is mostly rows past M) too."""
    N, K = 3840, 10240
    note("gemm K-split rows independent of M")
    A, B, _ = _gemm_inputs(600, N, K, 33)
    outs = {}
    for M in (600, 40, 300):
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        _ksplit(Z.ZDIT_EPI_STORE, M, N, K, A[:M], B, None, None, C)
        outs[M] = host(C)
    np.testing.assert_array_equal(outs[600][:40], outs[40])
    np.testing.assert_array_equal(outs[600][:300], outs[300])


def test_gemm_whole_k_rows_do_not_depend_on_m():
    """The whole-K kernel: rows in a last panel whose lower row groups are empty (and skip their
    MFMAs) equal the same rows computed in a full panel."""
    N, K = 1024, 768
    note("gemm whole-K rows independent of M (empty row groups)")
    A, B, _ = _gemm_inputs(512, N, K, 34)
    outs = {}
    for M in (512, 300, 257, 100):
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        Z.zdit_op_gemm(BF, Z.ZDIT_EPI_STORE, M, N, K, dev(A[:M], torch.bfloat16), dev(B, torch.bfloat16), None,
                       None, C)
        outs[M] = host(C)
    for M in (300, 257, 100):
        np.testing.assert_array_equal(outs[512][:M], outs[M])


@pytest.mark.parametrize("epi", [Z.ZDIT_EPI_STORE, Z.ZDIT_EPI_BIAS, Z.ZDIT_EPI_RESID, Z.ZDIT_EPI_SWIGLU])
def test_gemm_fp32_debug(epi):
    M, N, K = 100, 130, 72
    note(f"gemm fp32 epi={epi}")
    g = _rng(7)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = (0.05 * g.standard_normal((N, K))).astype(np.float32)
    B2 = (0.05 * g.standard_normal((N, K))).astype(np.float32)
    vec = g.standard_normal(N).astype(np.float32)
    C0 = g.standard_normal((M, N)).astype(np.float32)
    C = dev(C0)
    Z.zdit_op_gemm(F32P, epi, M, N, K, dev(A), dev(B), dev(B2), dev(vec), C)
    a1 = A.astype(np.float64) @ B.astype(np.float64).T
    ref = {Z.ZDIT_EPI_STORE: a1, Z.ZDIT_EPI_BIAS: a1 + vec, Z.ZDIT_EPI_RESID: C0 + vec * a1,
           Z.ZDIT_EPI_SWIGLU: O.silu(a1) * (A.astype(np.float64) @ B2.astype(np.float64).T)}[epi]
    np.testing.assert_allclose(host(C), ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("name,M,N,K,epi", [
    ("qkv", 8320, 11520, 3840, Z.ZDIT_EPI_STORE),
    ("out", 8320, 3840, 3840, Z.ZDIT_EPI_RESID),
    ("w13", 8320, 10240, 3840, Z.ZDIT_EPI_SWIGLU),
    ("w2", 8320, 3840, 10240, Z.ZDIT_EPI_RESID),
])
def test_gemm_block_shapes_full_size_sampled(name, M, N, K, epi):
    """The four block GEMMs at the 1024^2 pair shape (M = 2 x 4160), checked on sampled rows."""
    note(f"gemm full-size {name} M={M} N={N} K={K}")
    g = _rng(11)
    A = torch.randn((M, K), generator=torch.Generator().manual_seed(12)).to(torch.bfloat16)
    B = (0.02 * torch.randn((N, K), generator=torch.Generator().manual_seed(13))).to(torch.bfloat16)
    B2 = (0.02 * torch.randn((N, K), generator=torch.Generator().manual_seed(14))).to(torch.bfloat16)
    gate = torch.from_numpy(g.standard_normal(N).astype(np.float32))
    C0 = torch.from_numpy(g.standard_normal((M, N)).astype(np.float32))
    if epi == Z.ZDIT_EPI_RESID:
        C = C0.cuda()
    else:
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Z.zdit_op_gemm(BF, epi, M, N, K, A.cuda(), B.cuda(), B2.cuda() if epi == Z.ZDIT_EPI_SWIGLU else None,
                   gate.cuda() if epi == Z.ZDIT_EPI_RESID else None, C)
    got = host(C)
    rows = np.unique(np.concatenate([g.choice(M, 40, replace=False), [0, 255, 256, 4159, 4160, M - 1]]))
    Ar = A[rows].double().numpy()
    a1 = Ar @ B.double().numpy().T
    if epi == Z.ZDIT_EPI_STORE:
        assert_bf16_result(got[rows], a1, 2e-6 * (np.abs(Ar) @ np.abs(B.double().numpy()).T))
    elif epi == Z.ZDIT_EPI_SWIGLU:
        _check_swiglu(got[rows], Ar, B.double().numpy(), B2.double().numpy())
    else:
        ref = C0.numpy()[rows] + gate.numpy() * a1
        bound = np.abs(gate.numpy()) * (np.abs(Ar) @ np.abs(B.double().numpy()).T)
        assert np.all(np.abs(got[rows] - ref) <= 2e-6 * bound + 1e-6 * np.abs(C0.numpy()[rows]) + 1e-6)


# ------------------------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("prec", [BF, F32P])
def test_rmsnorm_mod_with_outliers(prec):
    rows, d = 300, 3840
    note(f"rmsnorm_mod prec={prec} rows={rows}")
    x = synth.residual_input((rows, d), 8, outlier_frac=0.001)
    g = _rng(9)
    gain = (1 + 0.02 * g.standard_normal(d)).astype(np.float32)
    shift = (0.1 * g.standard_normal(d)).astype(np.float32)
    scale = (0.1 * g.standard_normal(d)).astype(np.float32)
    mod = dev(np.stack([shift, scale]))
    out = torch.empty((rows, d), dtype=torch.bfloat16 if prec == BF else torch.float32, device="cuda")
    Z.zdit_op_rmsnorm_mod(prec, rows, d, dev(x), dev(gain), mod[0], mod[1], 1e-6, out)
    ref = O.modulate(O.rmsnorm(x, gain, 1e-6), shift, scale)
    if prec == BF:
        assert ulp_diff_bf16(host(out), O.bf16_round(ref)).max() <= 1
    else:
        np.testing.assert_allclose(host(out), ref, rtol=2e-6, atol=2e-6)


# ------------------------------------------------------------------------------- RoPE
def _qkv(B, S, nh, seed):
    g = _rng(seed)
    return bf16_values(g.standard_normal((B, S, 3 * nh * 128)).astype(np.float32))


@pytest.mark.parametrize("prec", [BF, F32P])
def test_rope_bit_exact(prec):
    B, S, nh = 2, 100, 3
    seq = [100, 77]
    note(f"rope prec={prec}")
    qkv = _qkv(B, S, nh, 10)
    cos = np.zeros((B, S, 64), np.float32)
    sin = np.zeros((B, S, 64), np.float32)
    for b, nc in enumerate((36, 32)):
        c_, s_ = O.rope_tables(O.position_ids("joint", 8, 8, nc))
        cos[b, :len(c_)] = c_[:S]
        sin[b, :len(s_)] = s_[:S]
    t = dev(qkv, torch.bfloat16 if prec == BF else torch.float32)
    Z.zdit_op_rope(prec, B, S, nh, seq, t, dev(cos), dev(sin))
    want = qkv.copy()
    D = nh * 128
    for b in range(B):
        n = seq[b]
        for part in (0, 1):
            xs = qkv[b, :n, part * D:(part + 1) * D].reshape(n, nh, 128)
            y = O.rope_apply(xs, cos[b, :n], sin[b, :n]).reshape(n, D)
            want[b, :n, part * D:(part + 1) * D] = O.bf16_round(y) if prec == BF else y
    np.testing.assert_array_equal(host(t), want)


@pytest.mark.parametrize("kind", [Z.ZDIT_SEQ_IMAGE, Z.ZDIT_SEQ_CAPTION, Z.ZDIT_SEQ_JOINT])
def test_rope_tables_within_one_ulp(kind):
    gh, gw, ncap = 64, 64, [64, 32]
    S = {Z.ZDIT_SEQ_IMAGE: gh * gw, Z.ZDIT_SEQ_CAPTION: 64, Z.ZDIT_SEQ_JOINT: gh * gw + 64}[kind]
    note(f"rope tables kind={kind}")
    cos = torch.empty((2, S, 64), device="cuda")
    sin = torch.empty((2, S, 64), device="cuda")
    Z.zdit_rope_tables(kind, [32, 48, 48], 10000.0, 2, S, gh, gw, ncap, cos, sin)
    gc, gs = host(cos), host(sin)
    name = {Z.ZDIT_SEQ_IMAGE: "image", Z.ZDIT_SEQ_CAPTION: "caption", Z.ZDIT_SEQ_JOINT: "joint"}[kind]
    for b in range(2):
        rc, rs = O.rope_tables(O.position_ids(name, gh, gw, ncap[b]))
        n = len(rc)
        for got, ref in ((gc[b, :n], rc), (gs[b, :n], rs)):
            d = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
            assert d.max() <= 1 or np.abs(got - ref).max() < 1e-7
        assert np.all(gc[b, n:] == 1.0) and np.all(gs[b, n:] == 0.0)


# ------------------------------------------------------------------------------- attention
def _attn_ref(qkv, S, nh):
    D = nh * 128
    q = qkv[:S, :D].reshape(S, nh, 128)
    k = qkv[:S, D:2 * D].reshape(S, nh, 128)
    v = qkv[:S, 2 * D:].reshape(S, nh, 128)
    return O.attention(q, k, v).reshape(S, D)


@pytest.mark.parametrize("prec", [BF, F32P])
def test_attention_ragged(prec):
    B, S, nh = 2, 200, 2
    seq = [200, 137]
    note(f"attention prec={prec} seq={seq}")
    qkv = _qkv(B, S, nh, 20)
    dt = torch.bfloat16 if prec == BF else torch.float32
    out = torch.full((B, S, nh * 128), 7.0, dtype=dt, device="cuda")
    ws = Z.workspace(Z.zdit_op_attn_workspace(prec, B, S, nh))
    Z.zdit_op_attn(prec, B, S, nh, seq, dev(qkv, dt), out, ws)
    got = host(out)
    for b in range(B):
        ref = _attn_ref(qkv[b], seq[b], nh)
        if prec == BF:
            assert rel_l2(got[b, :seq[b]], ref) < 1e-2
            for h in range(nh):
                D_ = nh * 128
                assert_attention_close(got[b][:seq[b], h * 128:(h + 1) * 128], qkv[b][:seq[b], h * 128:(h + 1) * 128],
                                       qkv[b][:seq[b], D_ + h * 128:D_ + (h + 1) * 128],
                                       qkv[b][:seq[b], 2 * D_ + h * 128:2 * D_ + (h + 1) * 128])
        else:
            np.testing.assert_allclose(got[b, :seq[b]], ref, rtol=1e-5, atol=1e-5)
        assert np.all(got[b, seq[b]:] == 0)


def test_attention_key_block_counts():
    """Branches whose valid keys span 1, 2, 3, 4, 5 and 6 blocks of 64 (every first / last /
    next-to-last block arrangement of the key loop), with ragged final blocks."""
    S, nh = 384, 2
    seq = [1, 64, 65, 129, 200, 257, 300, 384]
    B = len(seq)
    note(f"attention key block counts seq={seq}")
    qkv = _qkv(B, S, nh, 23)
    out = torch.full((B, S, nh * 128), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = Z.workspace(Z.zdit_op_attn_workspace(BF, B, S, nh))
    Z.zdit_op_attn(BF, B, S, nh, seq, dev(qkv, torch.bfloat16), out, ws)
    got = host(out)
    for b in range(B):
        ref = _attn_ref(qkv[b], seq[b], nh)
        assert rel_l2(got[b, :seq[b]], ref) < 1e-2, seq[b]
        for h in range(nh):
            D_ = nh * 128
            assert_attention_close(got[b][:seq[b], h * 128:(h + 1) * 128], qkv[b][:seq[b], h * 128:(h + 1) * 128],
                                   qkv[b][:seq[b], D_ + h * 128:D_ + (h + 1) * 128],
                                   qkv[b][:seq[b], 2 * D_ + h * 128:2 * D_ + (h + 1) * 128])
        assert np.all(got[b, seq[b]:] == 0)


def test_attention_rising_scores_rescale():
    """Scores that grow along the keys (key norms ramp up, large query norms), so the running
    maximum keeps rising by more than the lazy-rescale threshold from block to block."""
    B, S, nh = 2, 448, 2
    seq = [448, 390]
    note(f"attention rising scores seq={seq}")
    g = _rng(24)
    x = g.standard_normal((B, S, 3 * nh * 128)).astype(np.float32)
    D = nh * 128
    x[:, :, :D] *= 3.0
    x[:, :, D:2 * D] *= (1.0 + 4.0 * np.arange(S, dtype=np.float32) / S)[None, :, None]
    qkv = bf16_values(x)
    out = torch.empty((B, S, D), dtype=torch.bfloat16, device="cuda")
    ws = Z.workspace(Z.zdit_op_attn_workspace(BF, B, S, nh))
    Z.zdit_op_attn(BF, B, S, nh, seq, dev(qkv, torch.bfloat16), out, ws)
    got = host(out)
    for b in range(B):
        ref = _attn_ref(qkv[b], seq[b], nh)
        assert rel_l2(got[b, :seq[b]], ref) < 1e-2
        for h in range(nh):
            D_ = nh * 128
            assert_attention_close(got[b][:seq[b], h * 128:(h + 1) * 128], qkv[b][:seq[b], h * 128:(h + 1) * 128],
                                   qkv[b][:seq[b], D_ + h * 128:D_ + (h + 1) * 128],
                                   qkv[b][:seq[b], 2 * D_ + h * 128:2 * D_ + (h + 1) * 128])
        assert np.all(got[b, seq[b]:] == 0)


def test_attention_padding_contents_are_invisible():
    """NaN in the batch-alignment padding rows changes no valid output bit."""
    B, S, nh = 2, 192, 2
    seq = [150, 101]
    note("attention NaN padding")
    qkv = _qkv(B, S, nh, 21)
    ws = Z.workspace(Z.zdit_op_attn_workspace(BF, B, S, nh))
    o1 = torch.empty((B, S, nh * 128), dtype=torch.bfloat16, device="cuda")
    Z.zdit_op_attn(BF, B, S, nh, seq, dev(qkv, torch.bfloat16), o1, ws)
    poisoned = qkv.copy()
    for b in range(B):
        poisoned[b, seq[b]:] = np.nan
    o2 = torch.empty_like(o1)
    Z.zdit_op_attn(BF, B, S, nh, seq, dev(poisoned, torch.bfloat16), o2, ws)
    a, b_ = host(o1), host(o2)
    for b in range(B):
        np.testing.assert_array_equal(a[b, :seq[b]], b_[b, :seq[b]])


def test_attention_full_size_sampled_queries():
    """1024^2 pair shape (S = 4160 / 4128, 30 heads): sampled queries of a few heads."""
    B, S, nh = 2, 4160, 30
    seq = [4160, 4128]
    note("attention full size 2 x 4160 x 30 heads")
    g = _rng(22)
    qkv = bf16_values(g.standard_normal((B, S, 3 * nh * 128)).astype(np.float32))
    out = torch.empty((B, S, nh * 128), dtype=torch.bfloat16, device="cuda")
    ws = Z.workspace(Z.zdit_op_attn_workspace(BF, B, S, nh))
    Z.zdit_op_attn(BF, B, S, nh, seq, dev(qkv, torch.bfloat16), out, ws)
    got = host(out)
    D = nh * 128
    for b in range(B):
        qs = np.unique(np.concatenate([g.choice(seq[b], 24, replace=False), [0, 127, 128, seq[b] - 1]]))
        for h in (0, 13, 29):
            k = qkv[b, :seq[b], D + h * 128:D + (h + 1) * 128].astype(np.float64)
            v = qkv[b, :seq[b], 2 * D + h * 128:2 * D + (h + 1) * 128].astype(np.float64)
            q = qkv[b, qs, h * 128:(h + 1) * 128].astype(np.float64)
            s = q @ k.T / np.sqrt(128)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            ref = (p / p.sum(axis=1, keepdims=True)) @ v
            assert rel_l2(got[b, qs, h * 128:(h + 1) * 128], ref) < 1e-2
            worst = assert_attention_close(got[b, qs, h * 128:(h + 1) * 128], q, k, v)
            print(f"branch {b} head {h}: worst error / element bound {worst:.3f}", flush=True)
        assert np.all(got[b, seq[b]:] == 0)


@pytest.mark.parametrize("B,S,nh,seq", [(2, 160, 3, [160, 131]), (1, 96, 2, [57]), (2, 4160, 30, [4160, 4128])])
def test_fused_qkv_rope_vt_bit_identical_to_separate_kernels(B, S, nh, seq):
    """The projection epilogue that rotates q, k and writes V^T reproduces GEMM + RoPE kernel +
    transpose kernel bit for bit: rotated q, k columns and the attention output."""
    note(f"fused qkv/rope/vt B={B} S={S} nh={nh} seq={seq}")
    D = nh * 128
    g = _rng(31 + S)
    h = bf16_values(g.standard_normal((B * S, D)).astype(np.float32))
    w = bf16_values((0.05 * g.standard_normal((3 * D, D))).astype(np.float32))
    cos = np.ones((B, S, 64), np.float32)
    sin = np.zeros((B, S, 64), np.float32)
    gh = 8 if S < 1000 else 64
    for b in range(B):
        c_, s_ = O.rope_tables(O.position_ids("joint", gh, gh, S - gh * gh))
        cos[b], sin[b] = c_[:S], s_[:S]
    ht, wt = dev(h, torch.bfloat16), dev(w, torch.bfloat16)
    ct, st = dev(cos), dev(sin)
    # separate kernels
    q1 = torch.empty((B * S, 3 * D), dtype=torch.bfloat16, device="cuda")
    Z.zdit_op_gemm(BF, Z.ZDIT_EPI_STORE, B * S, 3 * D, D, ht, wt, None, None, q1)
    Z.zdit_op_rope(BF, B, S, nh, seq, q1, ct, st)
    o1 = torch.empty((B, S, D), dtype=torch.bfloat16, device="cuda")
    ws1 = Z.workspace(Z.zdit_op_attn_workspace(BF, B, S, nh))
    Z.zdit_op_attn(BF, B, S, nh, seq, q1, o1, ws1)
    # fused; poison the workspace and the v columns first: neither may leak into the result
    q2 = torch.full((B * S, 3 * D), float("nan"), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty((B, S, D), dtype=torch.bfloat16, device="cuda")
    ws2 = Z.workspace(Z.zdit_op_attn_workspace(BF, B, S, nh))
    ws2.fill_(0xFF)
    Z.zdit_op_qkv_attn(B, S, nh, seq, ht, wt, ct, st, q2, o2, ws2)
    np.testing.assert_array_equal(host(q2)[:, :2 * D], host(q1)[:, :2 * D])
    np.testing.assert_array_equal(host(o2), host(o1))


# ------------------------------------------------------------------------------- index work
def test_patchify_unpatchify_bit_exact():
    B, C, h, w = 2, 16, 32, 48
    note("patchify/unpatchify")
    lat = synth.latents((B, C, h, w), 30)
    tok = torch.empty((B, (h // 2) * (w // 2), 4 * C), device="cuda")
    Z.zdit_op_patchify(B, C, h, w, dev(lat), C * h * w, tok)
    got = host(tok)
    for b in range(B):
        np.testing.assert_array_equal(got[b], O.patchify(lat[b]))
    # branch stride 0 broadcasts one latent
    Z.zdit_op_patchify(B, C, h, w, dev(lat[0]), 0, tok)
    got0 = host(tok)
    np.testing.assert_array_equal(got0[1], O.patchify(lat[0]))
    back = torch.empty((B, C, h, w), device="cuda")
    Z.zdit_op_unpatchify(B, C, h, w, dev(got), back)
    np.testing.assert_array_equal(host(back), lat)
    rnd = synth.latents((B, (h // 2) * (w // 2), 4 * C), 31)
    Z.zdit_op_unpatchify(B, C, h, w, dev(rnd), back)
    for b in range(B):
        np.testing.assert_array_equal(host(back)[b], O.unpatchify(rnd[b], C, h, w))


def test_cap_pad_bit_exact():
    B, S, d, row0 = 2, 160, 256, 64
    cap_len = [45, 10]
    note("cap_pad")
    x0 = synth.latents((B, S, d), 32)
    pad = synth.latents((d,), 33)
    x = dev(x0)
    Z.zdit_op_cap_pad(B, S, d, row0, cap_len, dev(pad), x)
    want = x0.copy()
    for b, L in enumerate(cap_len):
        want[b, row0 + L:row0 + O.n_cap(L)] = pad
    np.testing.assert_array_equal(host(x), want)


# ------------------------------------------------------------------------------- sampler math
@pytest.mark.parametrize("g", [1.0, 0.0, 3.7])
def test_euler_cfg_unscale_bit_exact(g):
    n = 16 * 128 * 128
    note(f"euler g={g}")
    x0 = synth.latents((n,), 40)
    vc = synth.latents((n,), 41)
    vu = synth.latents((n,), 42)
    sg = O.sigmas(8, 3.0)
    for i in (0, 3, 7):
        x = dev(x0)
        dec = torch.empty(n, device="cuda")
        Z.zdit_euler_step(x, dev(vc), dev(vu), n, g, float(sg[i]), float(sg[i + 1]), dec)
        want = O.euler_update(x0, O.cfg_noise_pred(vc, vu, g), sg[i], sg[i + 1])
        np.testing.assert_array_equal(host(x), want)
        np.testing.assert_array_equal(host(dec), O.unscale(want))
    # single branch
    x = dev(x0)
    Z.zdit_euler_step(x, dev(vc), None, n, 0.0, float(sg[0]), float(sg[1]), None)
    np.testing.assert_array_equal(host(x), O.euler_update(x0, O.cfg_noise_pred(vc, None, 0.0), sg[0], sg[1]))


# ------------------------------------------------------------------------------- conditioning
def test_timestep_mlp():
    dims = synth.FULL
    ew = synth.embed_weights(dims, 50)
    t = [0.5, 0.0, float(1 - O.sigmas(8)[1]), 0.7]
    note("temb")
    c = torch.empty((4, dims.c_dim), device="cuda")
    Z.zdit_op_temb(4, t, dims.t_freq, dims.c_dim, dims.t_scale, dev(ew["t_w1"]), dev(ew["t_b1"]),
                   dev(ew["t_w2"]), dev(ew["t_b2"]), c)
    ref = O.t_condition(np.array(t, np.float32), ew, dims)
    np.testing.assert_allclose(host(c), ref, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("prec", [BF, F32P])
def test_adaln_projection(prec):
    dims = synth.TINY
    w = synth.block_weights(dims, 51, 0)
    c = synth.latents((3, dims.c_dim), 52)
    note(f"adaln prec={prec}")
    out = torch.empty((3, 6 * dims.dim), device="cuda")
    Z.zdit_op_adaln(prec, 3, dims.c_dim, 6 * dims.dim, dev(c),
                    dev(w["w_ada"], torch.bfloat16 if prec == BF else torch.float32), dev(w["b_ada"]), out)
    ref = np.stack([O.block_mod(c[b], w).reshape(-1) for b in range(3)])
    np.testing.assert_allclose(host(out), ref, rtol=1e-5, atol=1e-5)
