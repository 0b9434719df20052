"""ctypes binding of ``libwhisper_enc.so``: the C ABI of ``include/whisper_enc.h`` under the same
names, with argument marshalling only (every step of the forward pass runs in the HIP kernels).

Pointer arguments accept a ``torch.Tensor`` (its ``data_ptr()``), a plain integer address or
``None``.  ``stream`` defaults to PyTorch's current stream on the current device.  A non-zero
status raises :class:`WencError`.

The library is loaded after ``import torch`` so that it binds to the HIP runtime PyTorch has
already loaded (both carry the soname ``libamdhip64.so.7``); a stream handle from PyTorch is then
valid inside the library.  There is no fallback: if the library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwhisper_enc.so")

WENC_OK = 0
WENC_ERR_ARG = 1
WENC_ERR_UNSUPPORTED = 2
WENC_ERR_WORKSPACE = 3
WENC_ERR_HIP = 4
WENC_ERR_SCRATCH = 5
WENC_NOALLOC_SCRATCH_BYTES = 64 << 20

WENC_PATH_BF16 = 0
WENC_PATH_FP32 = 1
WENC_PATH_FP16 = 2
WENC_PATH_Q8 = 3
WENC_PATH_Q4 = 4
WENC_PATH_BF16X2 = 5
WENC_PATH_BF16X3 = 6
WENC_PATH_MXFP8 = 7
PATHS = {"bf16": WENC_PATH_BF16, "fp32": WENC_PATH_FP32, "fp16": WENC_PATH_FP16,
         "q8": WENC_PATH_Q8, "q4": WENC_PATH_Q4, "bf16x2": WENC_PATH_BF16X2,
         "bf16x3": WENC_PATH_BF16X3, "mxfp8": WENC_PATH_MXFP8}

WENC_DTYPE_F32 = 0
WENC_DTYPE_BF16 = 1
WENC_DTYPE_F16 = 2
WENC_DTYPE_MXFP8 = 3

WENC_EPI_BIAS = 0
WENC_EPI_BIAS_GELU = 1
WENC_EPI_BIAS_RESIDUAL = 2
WENC_EPI_BIAS_GELU_RESIDUAL = 3

# Limits checked by every entry point.
WENC_HEAD_DIM = 64
WENC_MAX_D_MODEL = 4096
WENC_MAX_FFN_DIM = 65536
WENC_MAX_ROWS = 1 << 24
WENC_MAX_DEC_LAYERS = 64
WENC_MAX_MELS = 1024

HEAD_DIM = 64

EXPORTS = (
    "whisper_enc_strerror", "whisper_enc_layer_bytes", "whisper_enc_pack_layer",
    "whisper_enc_workspace_bytes", "whisper_enc_block_forward", "whisper_enc_stack_forward",
    "whisper_enc_layernorm", "whisper_enc_linear", "whisper_enc_attention",
    "whisper_enc_cross_kv_bytes", "whisper_enc_pack_cross_kv",
    "whisper_enc_cross_kv_workspace_bytes", "whisper_enc_cross_kv",
    "whisper_enc_stem_bytes", "whisper_enc_pack_stem", "whisper_enc_stem_workspace_bytes",
    "whisper_enc_stem_forward",
    "whisper_enc_varlen_workspace_bytes", "whisper_enc_stack_forward_varlen",
    "whisper_enc_attention_varlen", "whisper_enc_quantize_matrix", "whisper_enc_dequantize_matrix",
    "whisper_enc_stack_forward_noalloc", "whisper_enc_mx_bytes", "whisper_enc_mx_quantize",
)

_LIB: Optional[ctypes.CDLL] = None


class WencError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: status {code} ({strerror(code)})")


def load() -> ctypes.CDLL:
    """Load the library once (after torch's HIP runtime); raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  (binds the process to torch's libamdhip64 first)
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m speech_transformer_encoder_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "whisper_enc_strerror": (ctypes.c_char_p, [I]),
        "whisper_enc_layer_bytes": (Z, [I, I, I]),
        "whisper_enc_pack_layer": (I, [P] * 16 + [I, I, I, P, P]),
        "whisper_enc_workspace_bytes": (Z, [I, I, I, I, I, I]),
        "whisper_enc_block_forward": (I, [P, P, P, I, I, I, I, I, I, P, Z, P]),
        "whisper_enc_stack_forward": (I, [P, P, P, I, P, P, I, I, I, I, I, I, P, Z, P]),
        "whisper_enc_layernorm": (I, [P, P, P, P, I, I, I, P]),
        "whisper_enc_linear": (I, [P, P, P, P, P, I, I, I, I, I, P]),
        "whisper_enc_attention": (I, [P, P, P, P, I, I, I, I, I, I, P]),
        "whisper_enc_cross_kv_bytes": (Z, [I, I, I]),
        "whisper_enc_pack_cross_kv": (I, [P, P, P, I, I, I, P, P]),
        "whisper_enc_cross_kv_workspace_bytes": (Z, [I, I, I, I]),
        "whisper_enc_cross_kv": (I, [P, P, P, I, I, I, I, I, I, P, Z, P]),
        "whisper_enc_stem_bytes": (Z, [I, I, I, I]),
        "whisper_enc_pack_stem": (I, [P, P, P, P, P, I, I, I, I, P, P]),
        "whisper_enc_stem_workspace_bytes": (Z, [I, I, I, I, I]),
        "whisper_enc_stem_forward": (I, [P, P, P, I, I, I, I, I, I, P, Z, P]),
        "whisper_enc_varlen_workspace_bytes": (Z, [I, I, I, I, I, I, I]),
        "whisper_enc_stack_forward_varlen": (I, [P, P, P, I, P, P, P, I, I, I, I, I, I, I, P, Z, P]),
        "whisper_enc_attention_varlen": (I, [P, P, P, P, P, I, I, I, I, I, I, I, P]),
        "whisper_enc_quantize_matrix": (I, [P, P, P, I, I, I, P]),
        "whisper_enc_dequantize_matrix": (I, [P, P, P, I, I, I, P]),
        "whisper_enc_stack_forward_noalloc": (I, [P, P, P, I, P, P, I, I, I, I, I, I, P]),
        "whisper_enc_mx_bytes": (Z, [I, I]),
        "whisper_enc_mx_quantize": (I, [P, P, I, I, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(code: int, where: str) -> None:
    if code != WENC_OK:
        raise WencError(code, where)


def strerror(code: int) -> str:
    return load().whisper_enc_strerror(code).decode()


def whisper_enc_layer_bytes(d_model: int, ffn_dim: int, path: int) -> int:
    return load().whisper_enc_layer_bytes(d_model, ffn_dim, path)


def whisper_enc_workspace_bytes(batch: int, t: int, d_model: int, heads: int, ffn_dim: int,
                                path: int) -> int:
    return load().whisper_enc_workspace_bytes(batch, t, d_model, heads, ffn_dim, path)


def whisper_enc_pack_layer(ln1_g, ln1_b, wq, bq, wk, bk, wv, bv, wo, bo, ln2_g, ln2_b, w1, b1,
                           w2, b2, d_model, ffn_dim, path, dst_layer, stream=None) -> None:
    ptrs = [_ptr(a) for a in (ln1_g, ln1_b, wq, bq, wk, bk, wv, bv, wo, bo, ln2_g, ln2_b, w1, b1,
                              w2, b2)]
    _check(load().whisper_enc_pack_layer(*ptrs, d_model, ffn_dim, path, _ptr(dst_layer),
                                         _stream(stream)), "whisper_enc_pack_layer")


def whisper_enc_block_forward(x, y, layer, batch, t, d_model, heads, ffn_dim, path, workspace,
                              workspace_bytes, stream=None) -> None:
    _check(load().whisper_enc_block_forward(_ptr(x), _ptr(y), _ptr(layer), batch, t, d_model,
                                            heads, ffn_dim, path, _ptr(workspace),
                                            workspace_bytes, _stream(stream)),
           "whisper_enc_block_forward")


def whisper_enc_stack_forward(x, y, layers, n_layers, ln_post_g, ln_post_b, batch, t, d_model,
                              heads, ffn_dim, path, workspace, workspace_bytes,
                              stream=None) -> None:
    _check(load().whisper_enc_stack_forward(_ptr(x), _ptr(y), _ptr(layers), n_layers,
                                            _ptr(ln_post_g), _ptr(ln_post_b), batch, t, d_model,
                                            heads, ffn_dim, path, _ptr(workspace),
                                            workspace_bytes, _stream(stream)),
           "whisper_enc_stack_forward")


def whisper_enc_stack_forward_noalloc(x, y, layers, n_layers, ln_post_g, ln_post_b, batch, t,
                                      d_model, heads, ffn_dim, path, stream=None) -> None:
    _check(load().whisper_enc_stack_forward_noalloc(_ptr(x), _ptr(y), _ptr(layers), n_layers,
                                                    _ptr(ln_post_g), _ptr(ln_post_b), batch, t,
                                                    d_model, heads, ffn_dim, path,
                                                    _stream(stream)),
           "whisper_enc_stack_forward_noalloc")


def whisper_enc_layernorm(x, gamma, beta, y, rows, d, out_dtype, stream=None) -> None:
    _check(load().whisper_enc_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), rows, d,
                                        out_dtype, _stream(stream)), "whisper_enc_layernorm")


def whisper_enc_linear(a, w, bias, residual, c, m, n, k, path, epilogue, stream=None) -> None:
    _check(load().whisper_enc_linear(_ptr(a), _ptr(w), _ptr(bias), _ptr(residual), _ptr(c), m, n,
                                     k, path, epilogue, _stream(stream)), "whisper_enc_linear")


def whisper_enc_attention(q, k, v, o, batch, t, heads, ld_qkv, ld_o, path, stream=None) -> None:
    _check(load().whisper_enc_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o), batch, t, heads,
                                        ld_qkv, ld_o, path, _stream(stream)),
           "whisper_enc_attention")


def whisper_enc_cross_kv_bytes(d_model: int, n_dec_layers: int, path: int) -> int:
    return load().whisper_enc_cross_kv_bytes(d_model, n_dec_layers, path)


def whisper_enc_cross_kv_workspace_bytes(batch: int, t: int, d_model: int, path: int) -> int:
    return load().whisper_enc_cross_kv_workspace_bytes(batch, t, d_model, path)


def whisper_enc_pack_cross_kv(wk, wv, bv, n_dec_layers, d_model, path, dst, stream=None) -> None:
    """``wk``, ``wv``, ``bv``: sequences of ``n_dec_layers`` device tensors / addresses."""
    arr = ctypes.c_void_p * n_dec_layers
    pk = arr(*[_ptr(x) for x in wk])
    pv = arr(*[_ptr(x) for x in wv])
    pb = arr(*[_ptr(x) for x in bv])
    _check(load().whisper_enc_pack_cross_kv(ctypes.cast(pk, ctypes.c_void_p),
                                            ctypes.cast(pv, ctypes.c_void_p),
                                            ctypes.cast(pb, ctypes.c_void_p), n_dec_layers,
                                            d_model, path, _ptr(dst), _stream(stream)),
           "whisper_enc_pack_cross_kv")


def whisper_enc_cross_kv(y, kv, wkv, n_dec_layers, batch, t, d_model, heads, path, workspace,
                         workspace_bytes, stream=None) -> None:
    _check(load().whisper_enc_cross_kv(_ptr(y), _ptr(kv), _ptr(wkv), n_dec_layers, batch, t,
                                       d_model, heads, path, _ptr(workspace), workspace_bytes,
                                       _stream(stream)), "whisper_enc_cross_kv")


def whisper_enc_stem_bytes(n_mels: int, d_model: int, n_pos: int, path: int) -> int:
    return load().whisper_enc_stem_bytes(n_mels, d_model, n_pos, path)


def whisper_enc_stem_workspace_bytes(batch: int, t_mel: int, n_mels: int, d_model: int,
                                     path: int) -> int:
    return load().whisper_enc_stem_workspace_bytes(batch, t_mel, n_mels, d_model, path)


def whisper_enc_pack_stem(conv1_w, conv1_b, conv2_w, conv2_b, pos, n_mels, d_model, n_pos, path,
                          dst, stream=None) -> None:
    _check(load().whisper_enc_pack_stem(_ptr(conv1_w), _ptr(conv1_b), _ptr(conv2_w),
                                        _ptr(conv2_b), _ptr(pos), n_mels, d_model, n_pos, path,
                                        _ptr(dst), _stream(stream)), "whisper_enc_pack_stem")


def whisper_enc_stem_forward(mel, x, stem, batch, t_mel, n_mels, d_model, n_pos, path, workspace,
                             workspace_bytes, stream=None) -> None:
    _check(load().whisper_enc_stem_forward(_ptr(mel), _ptr(x), _ptr(stem), batch, t_mel, n_mels,
                                           d_model, n_pos, path, _ptr(workspace), workspace_bytes,
                                           _stream(stream)), "whisper_enc_stem_forward")


def whisper_enc_varlen_workspace_bytes(batch: int, total_rows: int, max_t: int, d_model: int,
                                       heads: int, ffn_dim: int, path: int) -> int:
    return load().whisper_enc_varlen_workspace_bytes(batch, total_rows, max_t, d_model, heads,
                                                     ffn_dim, path)


def whisper_enc_stack_forward_varlen(x, y, layers, n_layers, ln_post_g, ln_post_b, cu_seqlens,
                                     batch, total_rows, max_t, d_model, heads, ffn_dim, path,
                                     workspace, workspace_bytes, stream=None) -> None:
    """cu_seqlens: device int32 tensor [batch + 1] of window offsets."""
    _check(load().whisper_enc_stack_forward_varlen(
        _ptr(x), _ptr(y), _ptr(layers), n_layers, _ptr(ln_post_g), _ptr(ln_post_b),
        _ptr(cu_seqlens), batch, total_rows, max_t, d_model, heads, ffn_dim, path,
        _ptr(workspace), workspace_bytes, _stream(stream)), "whisper_enc_stack_forward_varlen")


def whisper_enc_attention_varlen(q, k, v, o, cu_seqlens, batch, total_rows, max_t, heads, ld_qkv,
                                 ld_o, path, stream=None) -> None:
    _check(load().whisper_enc_attention_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                               _ptr(cu_seqlens), batch, total_rows, max_t, heads,
                                               ld_qkv, ld_o, path, _stream(stream)),
           "whisper_enc_attention_varlen")


def whisper_enc_quantize_matrix(w, codes, scales, n, k, bits, stream=None) -> None:
    _check(load().whisper_enc_quantize_matrix(_ptr(w), _ptr(codes), _ptr(scales), n, k, bits,
                                              _stream(stream)), "whisper_enc_quantize_matrix")


def whisper_enc_mx_bytes(rows, k) -> int:
    return int(load().whisper_enc_mx_bytes(rows, k))


def whisper_enc_mx_quantize(src, dst, rows, k, stream=None) -> None:
    _check(load().whisper_enc_mx_quantize(_ptr(src), _ptr(dst), rows, k, _stream(stream)),
           "whisper_enc_mx_quantize")


def whisper_enc_dequantize_matrix(codes, scales, dst, n, k, bits, stream=None) -> None:
    _check(load().whisper_enc_dequantize_matrix(_ptr(codes), _ptr(scales), _ptr(dst), n, k, bits,
                                                _stream(stream)), "whisper_enc_dequantize_matrix")
