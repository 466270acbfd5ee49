"""ctypes binding of libzdit.so (the gfx950 S3-DiT library).

Argument marshalling only: torch tensors supply device memory (``data_ptr()``) and streams
(``torch.cuda.current_stream().cuda_stream``); every step of the computation runs in the
library's HIP kernels.  The names mirror the C ABI in include/zdit.h.  If the library has
not been built, loading raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libzdit.so")

ZDIT_OK, ZDIT_EINVAL, ZDIT_EUNSUPPORTED, ZDIT_EWORKSPACE, ZDIT_EHIP, ZDIT_ENONFINITE = 0, -1, -2, -3, -4, -5
ZDIT_CHECK_FINITE = 1
ZDIT_BF16, ZDIT_FP32_DEBUG = 0, 1
ZDIT_SEQ_IMAGE, ZDIT_SEQ_CAPTION, ZDIT_SEQ_JOINT, ZDIT_SEQ_TEXT = 0, 1, 2, 3
ZDIT_EPI_STORE, ZDIT_EPI_BIAS, ZDIT_EPI_RESID, ZDIT_EPI_SWIGLU = 0, 1, 2, 3
MAX_BATCH = 16

# every exported symbol of include/zdit.h
EXPORTS = [
    "zdit_last_error", "zdit_abi_version", "zdit_block_workspace", "zdit_block_fwd", "zdit_block_fwd_noalloc",
    "zdit_stack_workspace", "zdit_stack_fwd", "zdit_sigmas", "zdit_n_cap", "zdit_euler_step",
    "zdit_sample_workspace", "zdit_sample", "zdit_rope_tables", "zdit_op_gemm",
    "zdit_op_gemm_ksplit_workspace", "zdit_op_gemm_ksplit",
    "zdit_op_rmsnorm_mod", "zdit_op_rope", "zdit_op_attn_workspace", "zdit_op_attn", "zdit_op_qkv_attn",
    "zdit_op_patchify", "zdit_op_unpatchify", "zdit_op_cap_pad", "zdit_op_temb", "zdit_op_adaln",
    "zdit_encoder_workspace", "zdit_encoder_fwd", "zdit_op_embed_workspace", "zdit_op_embed",
    "zdit_op_qknorm_rope", "zdit_op_attn_gqa_workspace", "zdit_op_attn_gqa",
    "zdit_op_gemm_splitk_workspace", "zdit_op_gemm_splitk", "zdit_op_gemm_splitk_packed", "zdit_op_pack_weights",
    "zdit_op_mfma_peak",
    "zdit_device_info",
    "zdit_vae_workspace", "zdit_vae_decode", "zdit_op_vae_groupnorm_workspace", "zdit_op_vae_groupnorm",
    "zdit_op_vae_conv", "zdit_op_vae_conv_out", "zdit_op_vae_attention_workspace", "zdit_op_vae_attention",
]
ZDIT_VAE_INPUT_UNSCALED = 1


class zdit_dims(C.Structure):
    _fields_ = [("dim", C.c_int32), ("n_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn_hidden", C.c_int32), ("rope_axes", C.c_int32 * 3), ("c_dim", C.c_int32),
                ("precision", C.c_int32), ("norm_eps", C.c_float), ("flags", C.c_int32)]


class zdit_block_w(C.Structure):
    _fields_ = [("w_qkv", C.c_void_p), ("w_out", C.c_void_p), ("w1", C.c_void_p),
                ("w3", C.c_void_p), ("w2", C.c_void_p), ("norm1", C.c_void_p),
                ("norm2", C.c_void_p), ("w_ada", C.c_void_p), ("b_ada", C.c_void_p)]


class zdit_model_cfg(C.Structure):
    _fields_ = [("d", zdit_dims), ("n_noise_ref", C.c_int32), ("n_ctx_ref", C.c_int32),
                ("n_main", C.c_int32), ("latent_ch", C.c_int32), ("patch", C.c_int32),
                ("cap_dim", C.c_int32), ("t_freq", C.c_int32), ("seq_multiple", C.c_int32),
                ("max_cap_len", C.c_int32), ("rope_theta", C.c_float), ("t_scale", C.c_float)]


class zdit_model_w(C.Structure):
    _fields_ = [("x_emb_w", C.c_void_p), ("x_emb_b", C.c_void_p), ("cap_emb_w", C.c_void_p),
                ("cap_emb_b", C.c_void_p), ("cap_pad", C.c_void_p), ("t_w1", C.c_void_p),
                ("t_b1", C.c_void_p), ("t_w2", C.c_void_p), ("t_b2", C.c_void_p),
                ("noise_ref", C.POINTER(zdit_block_w)), ("ctx_ref", C.POINTER(zdit_block_w)),
                ("main", C.POINTER(zdit_block_w)), ("final_norm", C.c_void_p),
                ("final_ada_w", C.c_void_p), ("final_ada_b", C.c_void_p),
                ("final_w", C.c_void_p), ("final_b", C.c_void_p)]


class zdit_enc_cfg(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("inter", C.c_int32),
                ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("vocab", C.c_int32), ("rope_theta", C.c_float), ("norm_eps", C.c_float), ("flags", C.c_int32)]


class zdit_enc_layer_w(C.Structure):
    _fields_ = [("in_norm", C.c_void_p), ("w_qkv", C.c_void_p), ("q_norm", C.c_void_p),
                ("k_norm", C.c_void_p), ("w_o", C.c_void_p), ("post_norm", C.c_void_p),
                ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p)]


class zdit_enc_w(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("layers", C.POINTER(zdit_enc_layer_w))]


class zdit_vae_cfg(C.Structure):
    _fields_ = [("latent_ch", C.c_int32), ("out_ch", C.c_int32), ("widths", C.c_int32 * 4), ("resnets", C.c_int32),
                ("groups", C.c_int32), ("eps", C.c_float), ("scale", C.c_float), ("shift", C.c_float),
                ("flags", C.c_int32)]


class zdit_vae_conv(C.Structure):
    _fields_ = [("w", C.c_void_p), ("b", C.c_void_p)]


class zdit_vae_norm(C.Structure):
    _fields_ = [("gamma", C.c_void_p), ("beta", C.c_void_p)]


class zdit_vae_resnet(C.Structure):
    _fields_ = [("gn1", zdit_vae_norm), ("conv1", zdit_vae_conv), ("gn2", zdit_vae_norm), ("conv2", zdit_vae_conv),
                ("shortcut", zdit_vae_conv)]


class zdit_vae_attn(C.Structure):
    _fields_ = [("gn", zdit_vae_norm), ("qkv", zdit_vae_conv), ("out", zdit_vae_conv)]


class zdit_vae_w(C.Structure):
    _fields_ = [("conv_in", zdit_vae_conv), ("mid", zdit_vae_resnet * 2), ("attn", zdit_vae_attn),
                ("stages", C.POINTER(zdit_vae_resnet) * 4), ("upconv", zdit_vae_conv * 3),
                ("norm_out", zdit_vae_norm), ("conv_out", zdit_vae_conv)]


class ZditError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"zdit error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m diffusion_transformer_text_s3_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
        pi32 = C.POINTER(C.c_int32)
        pf32 = C.POINTER(C.c_float)
        pd, pw = C.POINTER(zdit_dims), C.POINTER(zdit_block_w)
        pc, pm = C.POINTER(zdit_model_cfg), C.POINTER(zdit_model_w)
        pe, pew = C.POINTER(zdit_enc_cfg), C.POINTER(zdit_enc_w)
        pv, pvw, pva = C.POINTER(zdit_vae_cfg), C.POINTER(zdit_vae_w), C.POINTER(zdit_vae_attn)
        sig = {
            "zdit_last_error": (C.c_char_p, []),
            "zdit_abi_version": (i32, []),
            "zdit_block_workspace": (sz, [pd, i32, i32]),
            "zdit_block_fwd": (i32, [pd, pw, i32, i32, pi32, vp, vp, vp, vp, vp, sz, vp]),
            "zdit_block_fwd_noalloc": (i32, [pd, pw, i32, i32, pi32, vp, vp, vp, vp, vp]),
            "zdit_stack_workspace": (sz, [pc, i32, i32, i32, i32]),
            "zdit_stack_fwd": (i32, [pc, pm, i32, i32, i32, vp, i64, vp, i32, pi32, pf32, vp, vp, sz, vp]),
            "zdit_sigmas": (i32, [i32, f32, pf32]),
            "zdit_n_cap": (i32, [i32, i32, pi32]),
            "zdit_euler_step": (i32, [vp, vp, vp, i64, f32, f32, f32, vp, vp]),
            "zdit_sample_workspace": (sz, [pc, i32, i32, i32, f32]),
            "zdit_sample": (i32, [pc, pm, i32, i32, vp, vp, i32, pi32, f32, i32, f32, vp, vp, sz, vp]),
            "zdit_rope_tables": (i32, [i32, pi32, f32, i32, i32, i32, i32, pi32, vp, vp, vp]),
            "zdit_op_gemm": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
            "zdit_op_gemm_ksplit_workspace": (sz, [i32, i32, i32, i32]),
            "zdit_op_gemm_ksplit": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
            "zdit_op_rmsnorm_mod": (i32, [i32, i32, i32, vp, vp, vp, vp, f32, vp, vp]),
            "zdit_op_rope": (i32, [i32, i32, i32, i32, pi32, vp, vp, vp, vp]),
            "zdit_op_attn_workspace": (sz, [i32, i32, i32, i32]),
            "zdit_op_attn": (i32, [i32, i32, i32, i32, pi32, vp, vp, vp, sz, vp]),
            "zdit_op_qkv_attn": (i32, [i32, i32, i32, pi32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "zdit_op_patchify": (i32, [i32, i32, i32, i32, vp, i64, vp, vp]),
            "zdit_op_unpatchify": (i32, [i32, i32, i32, i32, vp, vp, vp]),
            "zdit_op_cap_pad": (i32, [i32, i32, i32, i32, pi32, vp, vp, vp]),
            "zdit_op_temb": (i32, [i32, pf32, i32, i32, f32, vp, vp, vp, vp, vp, vp]),
            "zdit_op_adaln": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp]),
            "zdit_encoder_workspace": (sz, [pe, i32, i32]),
            "zdit_encoder_fwd": (i32, [pe, pew, i32, i32, pi32, pi32, vp, vp, sz, vp]),
            "zdit_op_embed_workspace": (sz, [i32, i32]),
            "zdit_op_embed": (i32, [i32, i32, i32, i32, pi32, pi32, vp, vp, vp, sz, vp]),
            "zdit_op_qknorm_rope": (i32, [i32, i32, i32, i32, pi32, vp, vp, vp, vp, vp, f32, vp]),
            "zdit_op_attn_gqa_workspace": (sz, [i32, i32, i32, i32]),
            "zdit_op_attn_gqa": (i32, [i32, i32, i32, i32, i32, i32, pi32, vp, vp, vp, sz, vp]),
            "zdit_op_gemm_splitk_workspace": (sz, [i32, i32, i32, i32]),
            "zdit_op_gemm_splitk": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
            "zdit_op_gemm_splitk_packed": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
            "zdit_op_pack_weights": (i32, [i32, i32, vp, vp, vp]),
            "zdit_op_mfma_peak": (i32, [i32, i32, vp, vp]),
            "zdit_device_info": (i32, [i32, pi32, pi32, pi32]),
            "zdit_vae_workspace": (sz, [pv, i32, i32, i32]),
            "zdit_vae_decode": (i32, [pv, pvw, i32, i32, i32, vp, vp, vp, sz, vp]),
            "zdit_op_vae_groupnorm_workspace": (sz, [i32, i32, i32, i32]),
            "zdit_op_vae_groupnorm": (i32, [i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, sz, vp]),
            "zdit_op_vae_conv": (i32, [i32, i32, i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp]),
            "zdit_op_vae_conv_out": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
            "zdit_op_vae_attention_workspace": (sz, [i32, i32, i32, i32]),
            "zdit_op_vae_attention": (i32, [i32, i32, i32, i32, i32, f32, pva, vp, vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().zdit_last_error().decode()


def check(code: int):
    if code != ZDIT_OK:
        raise ZditError(code, last_error())
    return code


# ----------------------------------------------------------------------------- marshalling
def ptr(t):
    """Device (or host) address of a torch tensor, or None."""
    return None if t is None else C.c_void_p(t.data_ptr())


def i32_array(vals):
    vals = list(vals)
    return (C.c_int32 * max(1, len(vals)))(*vals)


def f32_array(vals):
    vals = list(vals)
    return (C.c_float * max(1, len(vals)))(*vals)


def stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def make_dims(d, precision=ZDIT_BF16, flags=0) -> zdit_dims:
    """zdit_dims from any object with dim / n_heads / head_dim / ffn_hidden / rope_axes /
    c_dim / norm_eps attributes; flags 0 or ZDIT_CHECK_FINITE."""
    out = zdit_dims()
    out.dim, out.n_heads, out.head_dim, out.ffn_hidden = d.dim, d.n_heads, d.head_dim, d.ffn_hidden
    out.rope_axes[:] = list(d.rope_axes)
    out.c_dim, out.precision, out.norm_eps, out.flags = d.c_dim, precision, d.norm_eps, flags
    return out


def make_cfg(d, precision=ZDIT_BF16, flags=0) -> zdit_model_cfg:
    c = zdit_model_cfg()
    c.d = make_dims(d, precision, flags)
    c.n_noise_ref, c.n_ctx_ref, c.n_main = d.n_noise_ref, d.n_ctx_ref, d.n_main
    c.latent_ch, c.patch, c.cap_dim, c.t_freq = d.latent_ch, d.patch, d.cap_dim, d.t_freq
    c.seq_multiple, c.max_cap_len = d.seq_multiple, d.max_cap_len
    c.rope_theta, c.t_scale = d.rope_theta, d.t_scale
    return c


class DeviceBlock:
    """Device copies of one block's weights (torch tensors) and its zdit_block_w view."""

    MATS = ("w_qkv", "w_out", "w1", "w3", "w2")

    def __init__(self, tensors: dict):
        self.t = tensors
        self.w = zdit_block_w()
        for k in self.MATS + ("norm1", "norm2", "w_ada", "b_ada"):
            v = tensors.get(k)
            setattr(self.w, k, None if v is None else v.data_ptr())


def _to_dev(a, precision, device, matrix):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a, dtype=np.float32)
    t = torch.from_numpy(a)
    if matrix and precision == ZDIT_BF16:
        # the values are bf16-representable: the conversion is exact
        t = t.to(torch.bfloat16)
    return t.to(device)


def upload_block(wdict: dict, precision=ZDIT_BF16, device="cuda") -> DeviceBlock:
    """Device tensors for a block weight dict (fp32 numpy arrays)."""
    out = {}
    for k in DeviceBlock.MATS + ("w_ada",):
        if wdict.get(k) is not None:
            out[k] = _to_dev(wdict[k], precision, device, True)
    for k in ("norm1", "norm2", "b_ada"):
        if wdict.get(k) is not None:
            out[k] = _to_dev(wdict[k], precision, device, False)
    return DeviceBlock(out)


class DeviceModel:
    """Device copies of all stack weights and the zdit_model_w view (keeps them alive)."""

    MATS = ("x_emb_w", "cap_emb_w", "final_ada_w", "final_w")
    VECS = ("x_emb_b", "cap_emb_b", "cap_pad", "t_w1", "t_b1", "t_w2", "t_b2", "final_norm",
            "final_ada_b", "final_b")

    def __init__(self, tensors: dict, noise_ref, ctx_ref, main):
        self.t = tensors
        self.blocks = (list(noise_ref), list(ctx_ref), list(main))
        self._arrs = []
        self.w = zdit_model_w()
        for k in self.MATS + self.VECS:
            setattr(self.w, k, tensors[k].data_ptr())
        for name, blocks in zip(("noise_ref", "ctx_ref", "main"), self.blocks):
            arr = (zdit_block_w * max(1, len(blocks)))(*[b.w for b in blocks])
            self._arrs.append(arr)
            setattr(self.w, name, C.cast(arr, C.POINTER(zdit_block_w)))


def upload_model(W: dict, precision=ZDIT_BF16, device="cuda") -> DeviceModel:
    t = {}
    for k in DeviceModel.MATS:
        t[k] = _to_dev(W[k], precision, device, True)
    for k in DeviceModel.VECS:
        t[k] = _to_dev(W[k], precision, device, False)
    nr = [upload_block(b, precision, device) for b in W["noise_ref"]]
    cr = [upload_block(b, precision, device) for b in W["ctx_ref"]]
    mb = [upload_block(b, precision, device) for b in W["main"]]
    return DeviceModel(t, nr, cr, mb)


ZDIT_ENC_PACKED_WEIGHTS = 1


def make_enc_cfg(ed, flags=0) -> zdit_enc_cfg:
    """zdit_enc_cfg from any object with the encoder shape attributes (n_layers, hidden,
    inter, n_heads, n_kv_heads, head_dim, vocab, rope_theta, norm_eps)."""
    c = zdit_enc_cfg()
    c.n_layers, c.hidden, c.inter = ed.n_layers, ed.hidden, ed.inter
    c.n_heads, c.n_kv_heads, c.head_dim, c.vocab = ed.n_heads, ed.n_kv_heads, ed.head_dim, ed.vocab
    c.rope_theta, c.norm_eps = ed.rope_theta, ed.norm_eps
    c.flags = flags
    return c


class DeviceEncoder:
    """Device copies of the encoder weights and the zdit_enc_w view (keeps them alive)."""

    MATS = ("w_qkv", "w_o", "w_gate", "w_up", "w_down")
    VECS = ("in_norm", "q_norm", "k_norm", "post_norm")

    def __init__(self, embed, layers: list):
        self.embed = embed
        self.layers = layers
        self.lw = (zdit_enc_layer_w * max(1, len(layers)))()
        for i, t in enumerate(layers):
            for k in self.MATS + self.VECS:
                setattr(self.lw[i], k, t[k].data_ptr())
        self.w = zdit_enc_w()
        self.w.embed = embed.data_ptr()
        self.w.layers = C.cast(self.lw, C.POINTER(zdit_enc_layer_w))


def pack_encoder(enc: DeviceEncoder, stream=None) -> DeviceEncoder:
    """A copy of a device encoder whose projection matrices are in the layout of
    zdit_op_pack_weights (for a zdit_enc_cfg with ZDIT_ENC_PACKED_WEIGHTS); gains and the
    embedding table are shared."""
    import torch
    layers = []
    for t in enc.layers:
        p = dict(t)
        for k in DeviceEncoder.MATS:
            src = t[k]
            dst = torch.empty_like(src)
            zdit_op_pack_weights(src.shape[0], src.shape[1], src, dst, stream)
            p[k] = dst
        layers.append(p)
    return DeviceEncoder(enc.embed, layers)


def upload_encoder(W: dict, device="cuda") -> DeviceEncoder:
    """Device tensors (bf16 matrices, fp32 gains) for an encoder weight dict of fp32 arrays."""
    emb = _to_dev(W["embed"], ZDIT_BF16, device, True)
    layers = []
    for lw in W["layers"]:
        t = {k: _to_dev(lw[k], ZDIT_BF16, device, True) for k in DeviceEncoder.MATS}
        t.update({k: _to_dev(lw[k], ZDIT_BF16, device, False) for k in DeviceEncoder.VECS})
        layers.append(t)
    return DeviceEncoder(emb, layers)


# ----------------------------------------------------------------------------- calls
def workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def zdit_block_workspace(dims: zdit_dims, batch: int, s_max: int) -> int:
    return lib().zdit_block_workspace(C.byref(dims), batch, s_max)


def zdit_block_fwd(dims, w: DeviceBlock, batch, s_max, seq_len, x, c, cos, sin, ws, stream=None):
    return check(lib().zdit_block_fwd(C.byref(dims), C.byref(w.w), batch, s_max, i32_array(seq_len),
                                      ptr(x), ptr(c), ptr(cos), ptr(sin), ptr(ws), ws.numel(),
                                      stream_handle(stream)))


def zdit_block_fwd_noalloc(dims, w: DeviceBlock, batch, s_max, seq_len, x, c, cos, sin, stream=None):
    return check(lib().zdit_block_fwd_noalloc(C.byref(dims), C.byref(w.w), batch, s_max, i32_array(seq_len),
                                              ptr(x), ptr(c), ptr(cos), ptr(sin), stream_handle(stream)))


def zdit_stack_workspace(cfg, batch, lat_h, lat_w, max_cap_len) -> int:
    return lib().zdit_stack_workspace(C.byref(cfg), batch, lat_h, lat_w, max_cap_len)


def zdit_stack_fwd(cfg, m: DeviceModel, batch, lat_h, lat_w, latents, latent_batch_stride, cap_feats,
                   max_cap_len, cap_len, t, velocity, ws, stream=None):
    return check(lib().zdit_stack_fwd(C.byref(cfg), C.byref(m.w), batch, lat_h, lat_w, ptr(latents),
                                      latent_batch_stride, ptr(cap_feats), max_cap_len, i32_array(cap_len),
                                      f32_array(t), ptr(velocity), ptr(ws), ws.numel(), stream_handle(stream)))


def zdit_sigmas(num_steps: int, shift: float):
    out = (C.c_float * (num_steps + 1))()
    check(lib().zdit_sigmas(num_steps, shift, out))
    return list(out)


def zdit_n_cap(cap_len: int, multiple: int = 32) -> int:
    out = C.c_int32()
    check(lib().zdit_n_cap(cap_len, multiple, C.byref(out)))
    return out.value


def zdit_euler_step(x, v_cond, v_uncond, n, guidance, sigma, sigma_next, decode_out=None, stream=None):
    return check(lib().zdit_euler_step(ptr(x), ptr(v_cond), ptr(v_uncond), n, guidance, sigma, sigma_next,
                                       ptr(decode_out), stream_handle(stream)))


def zdit_sample_workspace(cfg, lat_h, lat_w, max_cap_len, guidance) -> int:
    return lib().zdit_sample_workspace(C.byref(cfg), lat_h, lat_w, max_cap_len, guidance)


def zdit_sample(cfg, m: DeviceModel, lat_h, lat_w, x, cap_feats, max_cap_len, cap_len, guidance, num_steps,
                shift, decode_out, ws, stream=None):
    return check(lib().zdit_sample(C.byref(cfg), C.byref(m.w), lat_h, lat_w, ptr(x), ptr(cap_feats), max_cap_len,
                                   i32_array(cap_len), guidance, num_steps, shift, ptr(decode_out), ptr(ws),
                                   ws.numel(), stream_handle(stream)))


def zdit_rope_tables(kind, rope_axes, theta, batch, s_max, grid_h, grid_w, n_cap, cos_out, sin_out, stream=None):
    return check(lib().zdit_rope_tables(kind, i32_array(rope_axes), theta, batch, s_max, grid_h, grid_w,
                                        i32_array(n_cap if n_cap is not None else [0]), ptr(cos_out),
                                        ptr(sin_out), stream_handle(stream)))


def zdit_op_gemm(precision, epilogue, M, N, K, A, B, B2, vec, Cout, stream=None):
    return check(lib().zdit_op_gemm(precision, epilogue, M, N, K, ptr(A), ptr(B), ptr(B2), ptr(vec), ptr(Cout),
                                    stream_handle(stream)))


def zdit_op_gemm_ksplit_workspace(epilogue, M, N, K) -> int:
    return lib().zdit_op_gemm_ksplit_workspace(epilogue, M, N, K)


def zdit_op_gemm_ksplit(epilogue, M, N, K, A, B, B2, vec, Cout, ws, stream=None):
    return check(lib().zdit_op_gemm_ksplit(epilogue, M, N, K, ptr(A), ptr(B), ptr(B2), ptr(vec), ptr(Cout),
                                           ptr(ws), ws.numel() if ws is not None else 0, stream_handle(stream)))


def zdit_op_rmsnorm_mod(precision, rows, dim, x, gain, shift, scale, eps, out, stream=None):
    return check(lib().zdit_op_rmsnorm_mod(precision, rows, dim, ptr(x), ptr(gain), ptr(shift), ptr(scale), eps,
                                           ptr(out), stream_handle(stream)))


def zdit_op_rope(precision, batch, s_max, n_heads, seq_len, qkv, cos, sin, stream=None):
    return check(lib().zdit_op_rope(precision, batch, s_max, n_heads, i32_array(seq_len), ptr(qkv), ptr(cos),
                                    ptr(sin), stream_handle(stream)))


def zdit_op_attn_workspace(precision, batch, s_max, n_heads) -> int:
    return lib().zdit_op_attn_workspace(precision, batch, s_max, n_heads)


def zdit_op_attn(precision, batch, s_max, n_heads, seq_len, qkv, out, ws, stream=None):
    return check(lib().zdit_op_attn(precision, batch, s_max, n_heads, i32_array(seq_len), ptr(qkv), ptr(out),
                                    ptr(ws), ws.numel(), stream_handle(stream)))


def zdit_op_qkv_attn(batch, s_max, n_heads, seq_len, h, w_qkv, cos, sin, qkv, out, ws, stream=None):
    return check(lib().zdit_op_qkv_attn(batch, s_max, n_heads, i32_array(seq_len), ptr(h), ptr(w_qkv), ptr(cos),
                                        ptr(sin), ptr(qkv), ptr(out), ptr(ws), ws.numel(), stream_handle(stream)))


def zdit_op_patchify(batch, Cch, h, w, lat, lat_batch_stride, tokens, stream=None):
    return check(lib().zdit_op_patchify(batch, Cch, h, w, ptr(lat), lat_batch_stride, ptr(tokens),
                                        stream_handle(stream)))


def zdit_op_unpatchify(batch, Cch, h, w, tokens, lat, stream=None):
    return check(lib().zdit_op_unpatchify(batch, Cch, h, w, ptr(tokens), ptr(lat), stream_handle(stream)))


def zdit_op_cap_pad(batch, s_max, dim, row0, cap_len, cap_pad, x, stream=None):
    return check(lib().zdit_op_cap_pad(batch, s_max, dim, row0, i32_array(cap_len), ptr(cap_pad), ptr(x),
                                       stream_handle(stream)))


def zdit_op_temb(batch, t, t_freq, c_dim, t_scale, w1, b1, w2, b2, c_out, stream=None):
    return check(lib().zdit_op_temb(batch, f32_array(t), t_freq, c_dim, t_scale, ptr(w1), ptr(b1), ptr(w2),
                                    ptr(b2), ptr(c_out), stream_handle(stream)))


def zdit_op_adaln(precision, batch, c_dim, n_out, c, w, b, out, stream=None):
    return check(lib().zdit_op_adaln(precision, batch, c_dim, n_out, ptr(c), ptr(w), ptr(b), ptr(out),
                                     stream_handle(stream)))


def zdit_encoder_workspace(cfg, batch, max_len) -> int:
    return lib().zdit_encoder_workspace(C.byref(cfg), batch, max_len)


def _ids_array(ids):
    import numpy as np
    a = np.ascontiguousarray(ids, dtype=np.int32)
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def zdit_encoder_fwd(cfg, m: DeviceEncoder, batch, max_len, ids, lengths, hidden_out, ws, stream=None):
    a, p = _ids_array(ids)
    return check(lib().zdit_encoder_fwd(C.byref(cfg), C.byref(m.w), batch, max_len, p, i32_array(lengths),
                                        ptr(hidden_out), ptr(ws), ws.numel(), stream_handle(stream)))


def zdit_op_embed_workspace(batch, max_len) -> int:
    return lib().zdit_op_embed_workspace(batch, max_len)


def zdit_op_embed(batch, max_len, dim, vocab, ids, lengths, table, out, ws, stream=None):
    a, p = _ids_array(ids)
    return check(lib().zdit_op_embed(batch, max_len, dim, vocab, p, i32_array(lengths), ptr(table), ptr(out),
                                     ptr(ws), ws.numel(), stream_handle(stream)))


def zdit_op_qknorm_rope(batch, s_max, n_heads, n_kv_heads, seq_len, qkv, q_norm, k_norm, cos, sin, eps,
                        stream=None):
    return check(lib().zdit_op_qknorm_rope(batch, s_max, n_heads, n_kv_heads, i32_array(seq_len), ptr(qkv),
                                           ptr(q_norm), ptr(k_norm), ptr(cos), ptr(sin), eps,
                                           stream_handle(stream)))


def zdit_op_attn_gqa_workspace(precision, batch, s_max, n_kv_heads) -> int:
    return lib().zdit_op_attn_gqa_workspace(precision, batch, s_max, n_kv_heads)


def zdit_op_attn_gqa(precision, batch, s_max, n_heads, n_kv_heads, causal, seq_len, qkv, out, ws, stream=None):
    return check(lib().zdit_op_attn_gqa(precision, batch, s_max, n_heads, n_kv_heads, int(causal),
                                        i32_array(seq_len), ptr(qkv), ptr(out), ptr(ws), ws.numel(),
                                        stream_handle(stream)))


def zdit_op_gemm_splitk_workspace(epilogue, M, N, K) -> int:
    return lib().zdit_op_gemm_splitk_workspace(epilogue, M, N, K)


def zdit_op_gemm_splitk(epilogue, M, N, K, A, B, B2, vec, Cout, ws, stream=None):
    return check(lib().zdit_op_gemm_splitk(epilogue, M, N, K, ptr(A), ptr(B), ptr(B2), ptr(vec), ptr(Cout),
                                           ptr(ws), ws.numel(), stream_handle(stream)))


def zdit_op_gemm_splitk_packed(epilogue, M, N, K, A, B, B2, vec, Cout, ws, stream=None):
    return check(lib().zdit_op_gemm_splitk_packed(epilogue, M, N, K, ptr(A), ptr(B), ptr(B2), ptr(vec), ptr(Cout),
                                                  ptr(ws), ws.numel(), stream_handle(stream)))


def zdit_op_pack_weights(N, K, src, dst, stream=None):
    return check(lib().zdit_op_pack_weights(N, K, ptr(src), ptr(dst), stream_handle(stream)))


def zdit_op_mfma_peak(workgroups, iters, out, stream=None):
    return check(lib().zdit_op_mfma_peak(workgroups, iters, ptr(out), stream_handle(stream)))


def zdit_device_info(device=0) -> dict:
    cu, clk, l2 = C.c_int32(), C.c_int32(), C.c_int32()
    check(lib().zdit_device_info(device, C.byref(cu), C.byref(clk), C.byref(l2)))
    return {"cu_count": cu.value, "max_sclk_mhz": clk.value / 1000.0, "l2_bytes": l2.value}


# ----------------------------------------------------------------------------- VAE decoder
def make_vae_cfg(vd, flags=0) -> zdit_vae_cfg:
    """zdit_vae_cfg from any object with latent_ch / out_ch / widths / resnets / groups / eps /
    scale / shift attributes; flags 0 or ZDIT_VAE_INPUT_UNSCALED."""
    c = zdit_vae_cfg()
    c.latent_ch, c.out_ch, c.resnets, c.groups = vd.latent_ch, vd.out_ch, vd.resnets, vd.groups
    c.widths[:] = list(vd.widths)
    c.eps, c.scale, c.shift, c.flags = vd.eps, vd.scale, vd.shift, flags
    return c


def vae_conv_weight(w, device="cuda"):
    """A conv weight [out, in, k, k] (or a linear map [out, in]) as the library's
    [out][k][k][in] fp32 device tensor."""
    import numpy as np
    import torch
    w = np.asarray(w, dtype=np.float32)
    if w.ndim == 2:
        w = w[:, :, None, None]
    return torch.from_numpy(np.ascontiguousarray(w.transpose(0, 2, 3, 1))).to(device)


class DeviceVae:
    """Device copies of the decoder weights and the zdit_vae_w view (keeps them alive)."""

    def __init__(self, W: dict, vd, device="cuda"):
        import numpy as np
        import torch
        self.t = {}

        def vec(k):
            self.t[k] = torch.from_numpy(np.ascontiguousarray(W[k], dtype=np.float32)).to(device)
            return self.t[k].data_ptr()

        def conv(dst, p):
            self.t[p + ".w"] = vae_conv_weight(W[p + ".w"], device)
            dst.w, dst.b = self.t[p + ".w"].data_ptr(), vec(p + ".b")

        def norm(dst, p):
            dst.gamma, dst.beta = vec(p + ".g"), vec(p + ".b")

        def resnet(dst, p):
            norm(dst.gn1, p + ".gn1")
            conv(dst.conv1, p + ".conv1")
            norm(dst.gn2, p + ".gn2")
            conv(dst.conv2, p + ".conv2")
            if (p + ".short.w") in W:
                conv(dst.shortcut, p + ".short")

        w = zdit_vae_w()
        conv(w.conv_in, "conv_in")
        resnet(w.mid[0], "mid.res0")
        resnet(w.mid[1], "mid.res1")
        norm(w.attn.gn, "mid.attn.gn")
        qkv = np.concatenate([W["mid.attn.q.w"], W["mid.attn.k.w"], W["mid.attn.v.w"]], axis=0)
        self.t["qkv.w"] = vae_conv_weight(qkv, device)
        self.t["qkv.b"] = torch.from_numpy(np.concatenate(
            [W["mid.attn.q.b"], W["mid.attn.k.b"], W["mid.attn.v.b"]]).astype(np.float32)).to(device)
        w.attn.qkv.w, w.attn.qkv.b = self.t["qkv.w"].data_ptr(), self.t["qkv.b"].data_ptr()
        conv(w.attn.out, "mid.attn.o")
        self.stages = []
        for i in range(4):
            arr = (zdit_vae_resnet * vd.resnets)()
            for j in range(vd.resnets):
                resnet(arr[j], f"up{i}.res{j}")
            self.stages.append(arr)
            w.stages[i] = C.cast(arr, C.POINTER(zdit_vae_resnet))
            if i < 3:
                conv(w.upconv[i], f"up{i}.upconv")
        norm(w.norm_out, "norm_out")
        conv(w.conv_out, "conv_out")
        self.w = w
        self.attn = w.attn


def upload_vae(W: dict, vd, device="cuda") -> DeviceVae:
    return DeviceVae(W, vd, device)


def zdit_vae_workspace(cfg, batch, lat_h, lat_w) -> int:
    return lib().zdit_vae_workspace(C.byref(cfg), batch, lat_h, lat_w)


def zdit_vae_decode(cfg, m: DeviceVae, batch, lat_h, lat_w, latent, image, ws, stream=None):
    return check(lib().zdit_vae_decode(C.byref(cfg), C.byref(m.w), batch, lat_h, lat_w, ptr(latent), ptr(image),
                                       ptr(ws), ws.numel(), stream_handle(stream)))


def zdit_op_vae_groupnorm_workspace(batch, hw, C_, groups) -> int:
    return lib().zdit_op_vae_groupnorm_workspace(batch, hw, C_, groups)


def zdit_op_vae_groupnorm(batch, hw, C_, groups, eps, x, gamma, beta, affine, ws, stream=None):
    return check(lib().zdit_op_vae_groupnorm(batch, hw, C_, groups, eps, ptr(x), ptr(gamma), ptr(beta), ptr(affine),
                                             ptr(ws), ws.numel(), stream_handle(stream)))


def zdit_op_vae_conv(batch, H, W, cin, cout, ksize, upsample, x, affine, silu, w, b, res, out, stream=None):
    return check(lib().zdit_op_vae_conv(batch, H, W, cin, cout, ksize, upsample, ptr(x), ptr(affine), silu, ptr(w),
                                        ptr(b), ptr(res), ptr(out), stream_handle(stream)))


def zdit_op_vae_conv_out(batch, H, W, cin, cout, x, affine, w, b, image, stream=None):
    return check(lib().zdit_op_vae_conv_out(batch, H, W, cin, cout, ptr(x), ptr(affine), ptr(w), ptr(b), ptr(image),
                                            stream_handle(stream)))


def zdit_op_vae_attention_workspace(batch, hw, C_, groups) -> int:
    return lib().zdit_op_vae_attention_workspace(batch, hw, C_, groups)


def zdit_op_vae_attention(batch, H, W, C_, groups, eps, m: DeviceVae, x, ws, stream=None):
    return check(lib().zdit_op_vae_attention(batch, H, W, C_, groups, eps, C.byref(m.attn), ptr(x), ptr(ws),
                                             ws.numel(), stream_handle(stream)))
