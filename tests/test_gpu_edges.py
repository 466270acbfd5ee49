"""Edge cases of the hot path on the GPU against the oracle: empty inputs, one-token and
one-patch sequences, keys that make the softmax uniform, the largest batch the library
accepts, the largest configuration (1536 x 1024, 6144 image tokens) and the one-step sampler."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from diffusion_transformer_text_s3_amd import binding as Z
from gpu_util import assert_attention_close, assert_bf16_result, bf16_values, dev, drift, host, note, rel_l2

pytestmark = pytest.mark.gpu
BF, F32P = Z.ZDIT_BF16, Z.ZDIT_FP32_DEBUG


def _rng(seed):
    return np.random.default_rng(seed)


def _attn(prec, seq, S, nh, qkv):
    B = len(seq)
    dt = torch.bfloat16 if prec == BF else torch.float32
    out = torch.full((B, S, nh * 128), 7.0, dtype=dt, device="cuda")
    ws = Z.workspace(Z.zdit_op_attn_workspace(prec, B, S, nh))
    Z.zdit_op_attn(prec, B, S, nh, seq, dev(qkv, dt), out, ws)
    return host(out)


def _heads(qkv_b, rows, nh):
    D = nh * 128
    q = qkv_b[rows, :D].reshape(len(rows), nh, 128)
    k = qkv_b[:, D:2 * D].reshape(-1, nh, 128)
    v = qkv_b[:, 2 * D:].reshape(-1, nh, 128)
    return q, k, v


# ------------------------------------------------------------------------------- empty inputs
@pytest.mark.parametrize("prec", [BF, F32P])
@pytest.mark.parametrize("epi", [Z.ZDIT_EPI_STORE, Z.ZDIT_EPI_BIAS, Z.ZDIT_EPI_RESID, Z.ZDIT_EPI_SWIGLU])
def test_gemm_zero_rows_is_a_no_op(prec, epi):
    """M = 0: the call succeeds and writes nothing."""
    note(f"gemm M=0 prec={prec} epi={epi}")
    N, K = 256, 128
    dt = torch.bfloat16 if prec == BF else torch.float32
    A = torch.zeros((1, K), dtype=dt, device="cuda")
    B = torch.ones((N, K), dtype=dt, device="cuda")
    vec = torch.ones((N,), device="cuda")
    C = torch.full((4, N), 3.0, device="cuda")
    Z.zdit_op_gemm(prec, epi, 0, N, K, A, B, B if epi == Z.ZDIT_EPI_SWIGLU else None,
                   vec if epi in (Z.ZDIT_EPI_BIAS, Z.ZDIT_EPI_RESID) else None, C)
    assert np.all(host(C) == 3.0)


@pytest.mark.parametrize("prec", [BF, F32P])
def test_rmsnorm_zero_rows_is_a_no_op(prec):
    note(f"rmsnorm rows=0 prec={prec}")
    d = 256
    x = torch.ones((1, d), device="cuda")
    g = torch.ones((d,), device="cuda")
    out = torch.full((2, d), 5.0, dtype=torch.bfloat16 if prec == BF else torch.float32, device="cuda")
    Z.zdit_op_rmsnorm_mod(prec, 0, d, x, g, None, None, 1e-6, out)
    assert np.all(host(out) == 5.0)


# ------------------------------------------------------------------------------- attention
@pytest.mark.parametrize("prec", [BF, F32P])
def test_attention_one_token_branch_returns_its_value(prec):
    """A branch with one valid token attends to itself only: softmax weight 1, so the output
    is that token's value row (bit for bit on the bf16 path, where the weight rounds to 1
    before it meets V; the oracle gives the row exactly)."""
    S, nh = 96, 2
    seq = [1, 96, 1]
    note(f"attention one-token branches prec={prec}")
    qkv = bf16_values(_rng(40).standard_normal((len(seq), S, 3 * nh * 128)).astype(np.float32))
    got = _attn(prec, seq, S, nh, qkv)
    D = nh * 128
    for b in (0, 2):
        if prec == BF:
            np.testing.assert_array_equal(got[b, 0], qkv[b, 0, 2 * D:])
        else:  # fp32 debug path: o / l with o = p v and l = p for p within an ulp of 1
            np.testing.assert_allclose(got[b, 0], qkv[b, 0, 2 * D:], rtol=3e-7, atol=0)
        q, k, v = _heads(qkv[b, :1], [0], nh)
        np.testing.assert_allclose(O.attention(q, k, v).reshape(D), qkv[b, 0, 2 * D:], rtol=0, atol=0)
        assert np.all(got[b, 1:] == 0)
    q, k, v = _heads(qkv[1], np.arange(S), nh)
    assert rel_l2(got[1], O.attention(q, k, v).reshape(S, D)) < 1e-2


@pytest.mark.parametrize("prec", [BF, F32P])
def test_attention_equal_keys_average_the_values(prec):
    """Every key of a branch equal: the softmax is uniform and each output row is the mean of
    the value rows (within the fp32 sum's rounding and one rounding to the output type)."""
    S, nh = 200, 2
    seq = [200, 131]
    note(f"attention equal keys prec={prec}")
    g = _rng(41)
    qkv = bf16_values(g.standard_normal((2, S, 3 * nh * 128)).astype(np.float32))
    D = nh * 128
    qkv[:, :, D:2 * D] = qkv[:, :1, D:2 * D]
    got = _attn(prec, seq, S, nh, qkv)
    for b in range(2):
        n = seq[b]
        mean = qkv[b, :n, 2 * D:].astype(np.float64).mean(axis=0)
        q, k, v = _heads(qkv[b, :n], np.arange(n), nh)
        ref = O.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)).reshape(n, D)
        np.testing.assert_allclose(ref, np.broadcast_to(mean, ref.shape), rtol=1e-12, atol=1e-12)
        # fp32 sum of n values: error below 2^-24 n sum|v| / n per mean, with slack; then one
        # rounding to the output type
        acc = 2.0 ** -22 * np.abs(qkv[b, :n, 2 * D:]).astype(np.float64).sum(axis=0)
        rel = 2.0 ** -8 if prec == BF else 2.0 ** -22
        assert np.all(np.abs(got[b, :n] - mean) <= rel * np.abs(mean) + acc)
        assert np.all(got[b, n:] == 0)


def test_attention_largest_batch():
    """ZDIT_MAX_BATCH branches of ragged lengths in one call."""
    S, nh = 320, 2
    seq = [1, 7, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 257, 320]
    assert len(seq) == 16
    note("attention 16 branches")
    qkv = bf16_values(_rng(42).standard_normal((16, S, 3 * nh * 128)).astype(np.float32))
    got = _attn(BF, seq, S, nh, qkv)
    for b, n in enumerate(seq):
        q, k, v = _heads(qkv[b, :n], np.arange(n), nh)
        ref = O.attention(q, k, v).reshape(n, nh * 128)
        assert rel_l2(got[b, :n], ref) < 1e-2, n
        for h in range(nh):
            D_ = nh * 128
            assert_attention_close(got[b][:n, h * 128:(h + 1) * 128], qkv[b][:n, h * 128:(h + 1) * 128],
                                   qkv[b][:n, D_ + h * 128:D_ + (h + 1) * 128],
                                   qkv[b][:n, 2 * D_ + h * 128:2 * D_ + (h + 1) * 128])
        assert np.all(got[b, n:] == 0)


def test_attention_1536x1024_pair_sampled_queries():
    """The largest configuration: 6144 image tokens + n_cap 64 / 32 (S = 6208 / 6176), 30
    heads; sampled queries of a few heads against the oracle over every key."""
    B, S, nh = 2, 6208, 30
    seq = [6208, 6176]
    note("attention 1536x1024 pair 2 x 6208 x 30 heads")
    g = _rng(43)
    qkv = bf16_values(g.standard_normal((B, S, 3 * nh * 128)).astype(np.float32))
    got = _attn(BF, seq, S, nh, qkv)
    D = nh * 128
    for b in range(B):
        n = seq[b]
        qs = np.unique(np.concatenate([g.choice(n, 24, replace=False), [0, 255, 256, n - 1]]))
        q, k, v = _heads(qkv[b, :n], qs, nh)
        for h in (0, 17, 29):
            ref = O.attention(q[:, h:h + 1].astype(np.float64), k[:, h:h + 1].astype(np.float64),
                              v[:, h:h + 1].astype(np.float64))[:, 0]
            assert rel_l2(got[b, qs, h * 128:(h + 1) * 128], ref) < 1e-2
            worst = assert_attention_close(got[b, qs, h * 128:(h + 1) * 128], q[:, h], k[:, h], v[:, h])
            print(f"branch {b} head {h}: worst error / element bound {worst:.3f}", flush=True)
        assert np.all(got[b, n:] == 0)


# ------------------------------------------------------------------------------- GEMM at the largest shape
def test_gemm_swiglu_1536x1024_pair_sampled_rows():
    """w1/w3 + SwiGLU at M = 2 x 6208 rows (the largest configuration), sampled rows."""
    M, N, K = 2 * 6208, 10240, 3840
    note(f"gemm swiglu M={M}")
    g = _rng(44)
    A = torch.randn((M, K), generator=torch.Generator().manual_seed(45)).to(torch.bfloat16)
    B = (0.02 * torch.randn((N, K), generator=torch.Generator().manual_seed(46))).to(torch.bfloat16)
    B2 = (0.02 * torch.randn((N, K), generator=torch.Generator().manual_seed(47))).to(torch.bfloat16)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Z.zdit_op_gemm(BF, Z.ZDIT_EPI_SWIGLU, M, N, K, A.cuda(), B.cuda(), B2.cuda(), None, C)
    got = host(C)
    rows = np.unique(np.concatenate([g.choice(M, 32, replace=False), [0, 6207, 6208, 12287, 12288, M - 1]]))
    Ar, Bd, B2d = A[rows].double().numpy(), B.double().numpy(), B2.double().numpy()
    a1, a3 = Ar @ Bd.T, Ar @ B2d.T
    e1, e3 = 2e-6 * (np.abs(Ar) @ np.abs(Bd).T), 2e-6 * (np.abs(Ar) @ np.abs(B2d).T)
    u = O.silu(a1) * a3
    assert_bf16_result(got[rows], u, 1.1 * e1 * np.abs(a3) + np.abs(O.silu(a1)) * e3 + 1e-6 * np.abs(u) + e1 * e3)


# ------------------------------------------------------------------------------- smallest model inputs
def _stack_case(dims, lat_h, lat_w, cap_len, seed, t=0.5):
    W = synth.model_weights(dims, seed)
    lat = synth.latents((dims.latent_ch, lat_h, lat_w), seed)
    cap = synth.caption_features(len(cap_len), max(cap_len), dims.cap_dim, seed)
    return W, lat, cap


def test_stack_one_patch_one_caption_token():
    """The smallest sequence the model takes: a 2 x 2 latent (one image token) and a one-token
    caption padded to 32 with the learned pad, as a pair at full tiny depth."""
    note("stack tiny 1 patch + 1 caption token pair")
    dims = synth.TINY
    cap_len = [1, 1]
    W, lat, cap = _stack_case(dims, 2, 2, cap_len, seed=80)
    cfg = Z.make_cfg(dims)
    model = Z.upload_model(W)
    vel = torch.empty((2, dims.latent_ch, 2, 2), device="cuda")
    ws = Z.workspace(Z.zdit_stack_workspace(cfg, 2, 2, 2, 1))
    Z.zdit_stack_fwd(cfg, model, 2, 2, 2, dev(lat), 0, dev(cap), 1, cap_len, [0.5, 0.5], vel, ws)
    got = host(vel)
    for b in range(2):
        ref = O.stack(lat, cap[b], 1, 0.5, W, dims)
        e, dr = rel_l2(got[b], ref), drift(got[b], ref)
        print(f"one-patch stack branch {b}: rel-L2 {e:.2e} drift {dr:.2e}", flush=True)
        assert e <= 1e-2 and dr <= 0.025


def test_sample_one_step():
    """One FlowMatchEuler step: sigmas (1, 0), one DiT call per branch at model time 0, then
    the Euler update to sigma 0; against the oracle sampler."""
    note("sample tiny 1 step g=1")
    dims = synth.TINY.replace(n_main=4)
    cap_len = [45, 10]
    W, lat, cap = _stack_case(dims, 16, 16, cap_len, seed=81)
    cfg = Z.make_cfg(dims)
    model = Z.upload_model(W)
    x = dev(lat)
    dec = torch.empty_like(x)
    ws = Z.workspace(Z.zdit_sample_workspace(cfg, 16, 16, 45, 1.0))
    Z.zdit_sample(cfg, model, 16, 16, x, dev(cap), 45, cap_len, 1.0, 1, 3.0, dec, ws)
    calls = []

    def dit(xx, branch, t):
        calls.append((branch, t))
        return O.stack(xx, cap[branch], cap_len[branch], t, W, dims)

    rx, _ = O.sample(lat, dit, num_steps=1, shift=3.0, guidance=1.0)
    assert [c[0] for c in calls] == [0, 1]
    e = rel_l2(host(x), rx)
    print(f"one-step sample: rel-L2 {e:.2e}", flush=True)
    assert e <= 1e-2
    np.testing.assert_array_equal(host(dec), O.unscale(host(x)))
