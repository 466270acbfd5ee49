"""The FLOP counts behind bench.py's figures, against a second count written per token and per
stage from the method's shapes: one main block on the 1024^2 cond/uncond pair (caption
lengths 45 and 10, padded to 64 and 32 caption tokens beside 64 x 64 image tokens), the 8-step
pass at 1024^2 and 1536 x 1024, and the VAE decode of a 1024^2 image.  The block and pass totals
are the ones the hot-path scope table prints (3460.6 GFLOP per block pair, 885.8 and 1423.3
TFLOP per pass); the decode's 10.47 TFLOP is the figure the VAE bench line reports."""
import math

import bench
import synth

D, H = 3840, 10240


def n_cap(length):
    return 32 * math.ceil(length / 32)


def block_by_token(S):
    # per token: q, k, v and the output map (4 d^2 multiply-adds), w1, w3 and w2 (3 d H);
    # per query: S keys for q.k and S for p.v (2 S d); two flops per multiply-add
    return 2 * S * (4 * D * D + 3 * D * H) + 2 * (2 * S * D) * S


def test_block_pair_count():
    S = [64 * 64 + n_cap(45), 64 * 64 + n_cap(10)]
    assert S == [4160, 4128]
    gemm = sum(2 * s * (4 * D * D + 3 * D * H) for s in S)
    attn = sum(4 * s * s * D for s in S)
    assert round(gemm / 1e9, 1) == 2933.1 and round(attn / 1e9, 1) == 527.6
    assert sum(bench.block_flops(s, D, H) for s in S) == gemm + attn == sum(block_by_token(s) for s in S)
    assert round((gemm + attn) / 1e9, 1) == 3460.6


def pass_by_branch(nimg, lens, steps=8):
    # every step and branch: patch embed (64 -> d), 2 noise refiners on the image tokens,
    # caption embed (2560 -> d), 2 context refiners on the padded caption, 30 main blocks on the
    # joint sequence, the final layer (d -> 64)
    total = 0
    for _ in range(steps):
        for L in lens:
            total += 2 * nimg * 64 * D + 2 * block_by_token(nimg)
            total += 2 * L * 2560 * D + 2 * block_by_token(n_cap(L))
            total += 30 * block_by_token(nimg + n_cap(L)) + 2 * nimg * D * 64
    return total


def test_pass_counts():
    dims = synth.FULL
    for nimg, want in ((64 * 64, 885.8), (96 * 64, 1423.3)):
        got = bench.pass_flops(dims, nimg, [45, 10], 8, n_cap)
        assert got == pass_by_branch(nimg, [45, 10])
        assert round(got / 1e12, 1) == want
        # the executed count reuses the shared image path (once per step for both branches) and
        # the caption path (once per pass): strictly less, by exactly those parts
        ex = bench.pass_flops(dims, nimg, [45, 10], 8, n_cap, reuse=True)
        img_path = 2 * nimg * 64 * D + 2 * block_by_token(nimg)
        cap_path = sum(2 * L * 2560 * D + 2 * block_by_token(n_cap(L)) for L in (45, 10))
        assert got - ex == 8 * img_path + 7 * cap_path


def test_vae_decode_count():
    vd = synth.VAE_FULL
    hw = 128 * 128
    conv = lambda cin, cout, k, px: 2 * k * k * cin * cout * px
    c0 = vd.widths[-1]
    total = conv(vd.latent_ch, c0, 3, hw)
    resnet = lambda cin, cout, px: conv(cin, cout, 3, px) + conv(cout, cout, 3, px) + (
        conv(cin, cout, 1, px) if cin != cout else 0)
    total += 2 * resnet(c0, c0, hw)                       # middle ResNets
    total += 4 * 2 * c0 * c0 * hw + 2 * (2 * hw * hw * c0)  # attention: 4 maps, q.k^T and P v
    px = hw
    for cin, c, up in vd.stages:
        total += resnet(cin, c, px) + (vd.resnets - 1) * resnet(c, c, px)
        if up:
            px *= 4
            total += conv(c, c, 3, px)
    total += conv(vd.widths[0], vd.out_ch, 3, px)
    assert px == 1024 * 1024
    assert total == bench.vae_flops(vd, 1, 128, 128)
    assert round(total / 1e12, 3) == 10.472


def test_encoder_down_projection_bytes():
    """The encoder roofline's algorithmic bytes for the down projection on the 55 valid rows of
    the 45- and 10-token captions: the bf16 weights once, the bf16 activations once, the fp32
    residual rows read and written once (52.0 MB)."""
    ed = synth.ENC_FULL
    M, D, I = 45 + 10, ed.hidden, ed.inter
    weights = D * I * 2
    acts = M * I * 2
    resid = M * D * 4 * 2
    assert (D, I) == (2560, 9728)
    assert round((weights + acts + resid) / 1e6, 1) == 52.0
    # bench.py's formula for the same launch
    assert 2 * D * I + 2 * M * I + 2 * 4 * M * D == weights + acts + resid


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits non-zero with a message, before any GPU
    work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)

