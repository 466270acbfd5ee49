"""Helpers shared by the GPU parity tests: device upload, comparison metrics."""
import sys

import numpy as np
import torch

from diffusion_transformer_text_s3_amd import binding as Z

DEV = "cuda"


def note(msg):
    """Print what the next GPU step runs, flushed, so a failing run names its case."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, dtype=torch.float32):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == torch.bfloat16:
        t = t.to(torch.bfloat16)   # exact for bf16-representable values
    return t.to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy()


def bf16_values(a, seed=None):
    """fp32 array truncated to bf16-representable values (input preparation)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def drift(got, ref):
    """mean |got - ref| / RMS(ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).mean() / max(np.sqrt((ref * ref).mean()), 1e-300))


def ulp_diff_bf16(a, b):
    """Per-element distance, in bf16 units of the last place, between bf16-valued arrays."""
    def line(x):
        u = (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.int64)
        mag = u & 0x7FFF
        return np.where(u >> 15, -mag, mag)
    return np.abs(line(a) - line(b))


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (normal range)."""
    v = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(v)) - 7)


def assert_bf16_result(got, ref64, acc_err):
    """got = bf16(fp32 value within acc_err of ref64): |got - ref64| <= half a bf16 ulp of the
    fp32 value plus acc_err."""
    ref64 = np.asarray(ref64, dtype=np.float64)
    acc_err = np.asarray(acc_err, dtype=np.float64)
    allow = 0.5 * bf16_ulp(np.abs(ref64) + acc_err) + acc_err
    err = np.abs(np.asarray(got, dtype=np.float64) - ref64)
    bad = err > allow * (1 + 1e-9)
    assert not bad.any(), f"{bad.sum()} elements outside bound; worst excess {(err - allow).max():.3e}"


def attention_ref_bound(q, k, v):
    """Softmax attention of queries q [n, hd] over keys k and values v [m, hd] (all keys
    visible) in float64, and a per-element bound on a bf16 flash-attention result.

    The kernel rounds each probability to bf16 once and uses that number both in P V and in the
    row sum, so its output is the weighted mean of the values with every weight w_j scaled by
    (1 + d_j): o' - o = sum_j w_j (1 + d_j) (v_j - o) / (1 + sum_j w_j d_j), hence
    |o' - o| <= d / (1 - d) * sum_j w_j |v_j - o| with d = max |d_j|.  d collects the bf16
    rounding (2^-9), the fp32 score sum over hd products (hd 2^-24 |q| |k| / sqrt(hd)) and the
    exp2 argument rounding.  Added: the fp32 sums over m keys in P V and in the row sum
    (2 m 2^-24 sum_j w_j |v_j|); the caller adds half a bf16 ulp for the output rounding."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    hd = q.shape[1]
    m = k.shape[0]
    s = q @ k.T / np.sqrt(hd)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    o = w @ v
    ds = hd * 2.0 ** -24 * (np.abs(q) @ np.abs(k).T) / np.sqrt(hd)
    d = 2.0 ** -9 + ds.max(axis=1) + 2.0 ** -22 * (1 + np.abs(s).max(axis=1) * 1.4427)
    spread = np.stack([w[i] @ np.abs(v - o[i]) for i in range(q.shape[0])])
    bound = (d / (1 - d))[:, None] * spread + 2 * m * 2.0 ** -24 * (w @ np.abs(v))
    return o, bound


def assert_attention_close(got, q, k, v):
    """got [n, hd] (bf16 values) within attention_ref_bound's bound plus half a bf16 ulp of
    the output, element by element."""
    o, bound = attention_ref_bound(q, k, v)
    err = np.abs(np.asarray(got, np.float64) - o)
    allow = bound + 0.5 * bf16_ulp(np.abs(o) + bound)
    bad = err > allow * (1 + 1e-9) + 1e-30
    assert not bad.any(), (f"{bad.sum()} of {bad.size} elements outside the bound; worst err {err.max():.3e}, "
                           f"worst excess {(err - allow).max():.3e}")
    return float((err / np.maximum(allow, 1e-30)).max())
