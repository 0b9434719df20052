"""CPU oracle for the Whisper-style pre-LN encoder block (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no code
with the HIP library: it reads plain numpy arrays in PyTorch layout (weights ``[n_out, n_in]``).

Every step is written the plain way, in float64 from fp32 inputs, with a library matmul or
``erf`` as the only primitives.  The steps and their sources (three Rust engines whose source
pages describe the same block):

  * LayerNorm - two passes: mean, then biased variance of the centred values, ``eps = 1e-5``
    inside the square root, then the affine (inferencelayer ``whisper_gpu.rs``, ``LN_SRC``
    shader; oxinfer ``whisper/model.rs``, ``LN_EPS``).
  * Q, K, V projections, K without a bias (turbospark-runtime ``whisper/metal.rs``,
    ``EncLayerGpu`` doc and ``encode_layer``; oxinfer ``encode``).
  * Bidirectional scaled-dot-product attention per head, ``score = q.k * hd^-0.5`` over every key,
    softmax, weighted sum of V, evaluated with the online (running max / running denominator)
    recurrence over tiles of 128 keys (inferencelayer ``VANILLA_ATTN`` doc and shader).
  * Output projection and residual add; second LayerNorm; fc1, erf-GELU, fc2 and residual add
    (inferencelayer ``WhisperEncoderGpu::forward``; turbospark-runtime ``encode_layer``;
    oxinfer ``encode``).
  * A stack repeats the block and ends in an optional final LayerNorm (inferencelayer
    ``forward``, ``ln_post``; oxinfer ``encode``, ``enc_ln``).

Readings taken where the pages leave a step open:
  * GELU is the exact-erf form ``0.5 z (1 + erf(z / sqrt 2))``; the pages name it ("GeluErf",
    ``gelu_erf``) without printing it.
  * A missing K bias is a zero bias; softmax is shift-invariant per query, so any K bias leaves the
    output unchanged (tested).
  * Windows of a batch never attend across each other (each page encodes one window at a time).
  * The ``exp`` is the exact one (oxinfer's decoder uses a fast approximation; the encoder
    attention the pages describe uses ``exp``).

Ragged batches (windows of different lengths packed back to back, no padding):
  * ``encoder_stack_varlen`` - each window through the stack on its own; the pages encode one
    window of t <= max_t rows per call (inferencelayer ``forward``) or pad to 30 s
    (turbospark-runtime module doc), and a window never attends outside itself.

The step before the encoder block (the convolutional front end):
  * ``conv_stem`` - ``h = gelu(conv1(mel))`` (kernel 3, stride 1, padding 1), then
    ``x = gelu(conv2(h)) + pos`` (kernel 3, stride 2, padding 1) over frames, with frames as rows
    (oxinfer ``WhisperModel::encode``, conv front end; turbospark-runtime ``encode_partial``,
    ``encode_whisper_conv1d3_gelu`` and ``encode_whisper_transpose_pos``).

The step after the encoder (cross-attention keys and values of the decoder):
  * ``cross_kv`` - for every decoder layer ``l``, ``K_l = y Wk_l^T`` (no bias) and
    ``V_l = y Wv_l^T + bv_l`` from the encoder output ``y``, stored head-major
    (turbospark-runtime ``build_cross_caches``; oxinfer ``cross_kv`` and ``Kv``).

Low-precision weights (oxinfer ``Precision``: q8 / q4 blocks of 32 quantised from bf16):
  * ``quantize_q8`` / ``quantize_q4`` and their inverses, ``quantized_layer``; the encodings are a
    reading (the pages name the formats without printing them), stated where they are defined.

Cross-check formulations (used only by the tests):
  * ``attention_two_pass`` - exact max pass, exponent/sum pass, weighted sum (inferencelayer
    ``DEC_QATTN`` shader; turbospark-runtime ``encode_layer`` score planes + ``softmax_rows``).
  * ``attention_split_kv`` - per-chunk (max, denominator, unnormalised sum) partials merged by
    rescaling with ``exp(m_chunk - m)`` (oxinfer ``CrossLayer::attend``).
"""

from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

LN_EPS = 1e-5
KEY_TILE = 128


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def layer_norm(x, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """Row-wise LayerNorm over the last axis: two-pass mean and biased variance.

    inferencelayer ``whisper_gpu.rs``, ``LN_SRC``: mean of the row, then the mean of squared
    deviations from it, ``inv = 1/sqrt(var + 1e-5)``, ``y = (x - mean) * inv * w + b``.
    """
    x = _f64(x)
    h = x.shape[-1]
    mean = x.sum(axis=-1, keepdims=True) / h
    dev = x - mean
    var = (dev * dev).sum(axis=-1, keepdims=True) / h
    inv = 1.0 / np.sqrt(var + eps)
    return dev * inv * _f64(gamma) + _f64(beta)


def gelu_erf(z) -> np.ndarray:
    """Exact-erf GELU, ``0.5 * z * (1 + erf(z / sqrt(2)))``."""
    z = _f64(z)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def linear(a, w, b=None) -> np.ndarray:
    """``a @ w.T + b`` with ``w`` in PyTorch ``[n_out, n_in]`` layout."""
    y = _f64(a) @ _f64(w).T
    if b is not None:
        y = y + _f64(b)
    return y


def _heads(x: np.ndarray, heads: int) -> np.ndarray:
    """``[t, d]`` -> ``[heads, t, hd]``: head ``h`` owns columns ``h*hd .. h*hd + hd - 1``."""
    t, d = x.shape
    return x.reshape(t, heads, d // heads).transpose(1, 0, 2)


def _merge_heads(o: np.ndarray) -> np.ndarray:
    h, t, hd = o.shape
    return o.transpose(1, 0, 2).reshape(t, h * hd)


def attention_online(q, k, v, heads: int, tile: int = KEY_TILE, return_probs: bool = False):
    """Bidirectional attention of one window via the online-softmax recurrence.

    inferencelayer ``VANILLA_ATTN``: for each (query row, head), keys are visited in tiles of
    128; for each tile the running max ``m`` becomes ``max(m, max_j s_j)``, the old state is
    scaled by ``corr = exp(m_old - m_new)``, ``p_j = exp(s_j - m_new)``, the denominator becomes
    ``l * corr + sum_j p_j`` and the accumulator ``acc * corr + sum_j p_j v_j``; the output is
    ``acc / l``.  ``s_j = (q . k_j) * hd^-0.5`` and there is no mask (bidirectional).  Here every
    query row of a head runs the same recurrence side by side (one row per numpy row).

    ``q``: ``[tq, d]`` (any subset of the window's query rows), ``k, v``: ``[t, d]``.  Returns
    ``[tq, d]`` (and, with ``return_probs``, the normalised probabilities ``[heads, tq, t]``
    rebuilt from the final ``m`` and ``l``, for invariant checks).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq, t = q.shape[0], k.shape[0]
    qh, kh, vh = _heads(q, heads), _heads(k, heads), _heads(v, heads)
    hd = qh.shape[-1]
    scale = hd ** -0.5
    out = np.empty_like(qh)
    probs = np.empty((heads, tq, t)) if return_probs else None
    for h in range(heads):
        m = np.full(tq, -np.inf)
        den = np.zeros(tq)
        acc = np.zeros((tq, hd))
        for j0 in range(0, t, tile):
            j1 = min(j0 + tile, t)
            s = (qh[h] @ kh[h, j0:j1].T) * scale
            m_new = np.maximum(m, s.max(axis=1))
            corr = np.exp(m - m_new)
            p = np.exp(s - m_new[:, None])
            den = den * corr + p.sum(axis=1)
            acc = acc * corr[:, None] + p @ vh[h, j0:j1]
            m = m_new
        out[h] = acc / den[:, None]
        if return_probs:
            s_all = (qh[h] @ kh[h].T) * scale
            probs[h] = np.exp(s_all - m[:, None]) / den[:, None]
    o = _merge_heads(out)
    return (o, probs) if return_probs else o


def attention_two_pass(q, k, v, heads: int) -> np.ndarray:
    """Same attention with the softmax taken in two explicit passes over a materialised score row.

    inferencelayer ``DEC_QATTN``: pass 1 finds the exact row max, pass 2 forms ``exp(s - max)``
    and its sum, then the output is ``sum_j p_j v_j / sum_j p_j``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    qh, kh, vh = _heads(q, heads), _heads(k, heads), _heads(v, heads)
    scale = qh.shape[-1] ** -0.5
    out = np.empty_like(qh)
    for h in range(heads):
        s = (qh[h] @ kh[h].T) * scale
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        out[h] = (e @ vh[h]) / e.sum(axis=1, keepdims=True)
    return _merge_heads(out)


def attention_split_kv(q, k, v, heads: int, chunks: int) -> np.ndarray:
    """Same attention over ``chunks`` key ranges, merged from per-chunk partial softmax states.

    oxinfer ``CrossLayer::attend``: each chunk keeps its own max ``m_c``, denominator ``l_c`` and
    unnormalised sum ``o_c``; the merge takes ``m = max_c m_c`` and sums ``exp(m_c - m) * l_c`` and
    ``exp(m_c - m) * o_c``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    qh, kh, vh = _heads(q, heads), _heads(k, heads), _heads(v, heads)
    t = qh.shape[1]
    scale = qh.shape[-1] ** -0.5
    bounds = np.linspace(0, t, chunks + 1).round().astype(int)
    out = np.empty_like(qh)
    for h in range(heads):
        parts = []
        for c in range(chunks):
            j0, j1 = bounds[c], bounds[c + 1]
            if j1 <= j0:
                continue
            s = (qh[h] @ kh[h, j0:j1].T) * scale
            mc = s.max(axis=1)
            e = np.exp(s - mc[:, None])
            parts.append((mc, e.sum(axis=1), e @ vh[h, j0:j1]))
        m = np.max(np.stack([p[0] for p in parts]), axis=0)
        den = np.zeros(t)
        acc = np.zeros_like(out[h])
        for mc, lc, oc in parts:
            w = np.exp(mc - m)
            den += w * lc
            acc += w[:, None] * oc
        out[h] = acc / den[:, None]
    return _merge_heads(out)


def _same(a):
    return a


def _window_block(x: np.ndarray, p: Dict[str, Optional[np.ndarray]], heads: int,
                  act=None) -> np.ndarray:
    """One pre-LN block on one window ``x [t, d]`` (float64 in, float64 out).  ``act``, when
    given, replaces the operands of the QKV, fc1 and fc2 products (the LayerNorm outputs and the
    GELU output) by ``act(operand)`` (``mx_values`` for the MXFP8 form)."""
    act = act or _same
    a = act(layer_norm(x, p["ln1_g"], p["ln1_b"]))
    q = linear(a, p["wq"], p["bq"])
    k = linear(a, p["wk"], p.get("bk"))
    v = linear(a, p["wv"], p["bv"])
    o = attention_online(q, k, v, heads)
    x1 = x + linear(o, p["wo"], p["bo"])
    a2 = act(layer_norm(x1, p["ln2_g"], p["ln2_b"]))
    hid = act(gelu_erf(linear(a2, p["w1"], p["b1"])))
    return x1 + linear(hid, p["w2"], p["b2"])


def encoder_block(x, p: Dict[str, Optional[np.ndarray]], heads: int, act=None) -> np.ndarray:
    """Pre-LN encoder block over ``x`` of shape ``[t, d]`` or ``[batch, t, d]``.

    ``x += out(attn(LN1 x))`` then ``x += fc2(gelu(fc1(LN2 x)))``; each window attends only
    within itself.  ``act`` as in ``_window_block``.
    """
    x = _f64(x)
    if x.ndim == 2:
        return _window_block(x, p, heads, act)
    return np.stack([_window_block(w, p, heads, act) for w in x])


def encoder_stack(x, layers: Sequence[Dict[str, Optional[np.ndarray]]], heads: int,
                  ln_post=None, act=None) -> np.ndarray:
    """``len(layers)`` blocks in order, then the final LayerNorm when ``ln_post = (g, b)``."""
    h = _f64(x)
    for p in layers:
        h = encoder_block(h, p, heads, act)
    if ln_post is not None:
        h = layer_norm(h, ln_post[0], ln_post[1])
    return h


def encoder_stack_varlen(x_rows, seqlens: Sequence[int],
                         layers: Sequence[Dict[str, Optional[np.ndarray]]], heads: int,
                         ln_post=None) -> np.ndarray:
    """The stack over a ragged batch: ``x_rows`` ``[sum(seqlens), d]`` holds the windows back to
    back, window ``b`` being the next ``seqlens[b]`` rows.  Each window runs through
    ``encoder_stack`` on its own (windows never attend across each other), and the outputs are
    packed the same way."""
    x = _f64(x_rows)
    starts = np.concatenate([[0], np.cumsum(np.asarray(seqlens, dtype=np.int64))])
    if starts[-1] != x.shape[0]:
        raise ValueError("window lengths do not add up to the number of rows")
    out = np.empty_like(x)
    for b in range(len(seqlens)):
        s0, s1 = int(starts[b]), int(starts[b + 1])
        if s1 > s0:
            out[s0:s1] = encoder_stack(x[s0:s1], layers, heads, ln_post)
    return out


def encoder_block_rows(x_window, p: Dict[str, Optional[np.ndarray]], heads: int,
                       rows: Sequence[int], act=None) -> np.ndarray:
    """Block output for the selected rows of one window ``[t, d]``.

    Same arithmetic as ``encoder_block`` applied to those rows only: every key and value of the
    window is still formed (attention reads all of them), but queries, the residual branch and the
    FFN run for the selected rows.  Lets a test check sampled outputs of a large batch.  ``act``
    as in ``_window_block`` (it acts on each row on its own, so taking rows first is the same).
    """
    act = act or _same
    x = _f64(x_window)
    rows = np.asarray(rows, dtype=np.int64)
    a = act(layer_norm(x, p["ln1_g"], p["ln1_b"]))
    k = linear(a, p["wk"], p.get("bk"))
    v = linear(a, p["wv"], p["bv"])
    q = linear(a[rows], p["wq"], p["bq"])
    o = attention_online(q, k, v, heads)
    x1 = x[rows] + linear(o, p["wo"], p["bo"])
    a2 = act(layer_norm(x1, p["ln2_g"], p["ln2_b"]))
    return x1 + linear(act(gelu_erf(linear(a2, p["w1"], p["b1"]))), p["w2"], p["b2"])


def max_rel_error(got, ref) -> float:
    """``max_i |g_i - o_i| / max(|o_i|, rms(o))``: each element's relative error, floored at the
    reference tensor's RMS so that entries near zero do not dominate."""
    g, o = _f64(got), _f64(ref)
    rms = math.sqrt(float(np.mean(o * o))) if o.size else 0.0
    floor = np.maximum(np.abs(o), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(g - o) / floor)) if o.size else 0.0


def mean_abs_error(got, ref) -> float:
    g, o = _f64(got), _f64(ref)
    return float(np.mean(np.abs(g - o))) if o.size else 0.0


def cross_kv(y, dec_layers: Sequence[Dict[str, np.ndarray]], heads: int) -> np.ndarray:
    """Cross-attention keys and values of every decoder layer for the encoder output ``y``.

    turbospark-runtime ``build_cross_caches`` / oxinfer ``cross_kv``: per decoder layer, the keys
    ``y Wk^T`` (the key projection has no bias) and the values ``y Wv^T + bv``; oxinfer's ``Kv``
    keeps each head's rows contiguous.  ``y``: ``[batch, t, d]`` (or ``[t, d]``);
    ``dec_layers``: dicts with ``wk``, ``wv`` ``[d, d]`` and ``bv`` ``[d]``.  Returns
    ``[batch, L, 2, heads, t, hd]`` (index 0 = K, 1 = V).
    """
    y = _f64(y)
    if y.ndim == 2:
        y = y[None]
    b, t, d = y.shape
    out = np.empty((b, len(dec_layers), 2, heads, t, d // heads))
    for w in range(b):
        for l, p in enumerate(dec_layers):
            out[w, l, 0] = _heads(linear(y[w], p["wk"]), heads)
            out[w, l, 1] = _heads(linear(y[w], p["wv"], p["bv"]), heads)
    return out


def conv1d_k3(x, w, b, stride: int) -> np.ndarray:
    """1-D convolution over rows with kernel 3 and zero padding 1: ``x`` ``[t, cin]`` (frames as
    rows), ``w`` ``[cout, cin, 3]`` (PyTorch layout), ``b`` ``[cout]``; output row ``i`` is
    ``b + sum_j w[:, :, j] x[stride i + j - 1]`` (terms outside ``[0, t)`` are zero), for
    ``i < floor((t - 1) / stride) + 1``."""
    x, w = _f64(x), _f64(w)
    t = x.shape[0]
    n = (t - 1) // stride + 1
    xp = np.zeros((t + 2, x.shape[1]))
    xp[1:t + 1] = x
    y = np.tile(_f64(b), (n, 1))
    for j in range(3):
        y += xp[j:j + stride * (n - 1) + 1:stride] @ w[:, :, j].T
    return y


def conv_stem(mel, conv1_w, conv1_b, conv2_w, conv2_b, pos) -> np.ndarray:
    """Whisper's convolutional front end on ``mel`` ``[t, n_mels]`` or ``[batch, t, n_mels]``
    (frames as rows): ``gelu(conv1)`` with stride 1, ``gelu(conv2)`` with stride 2, plus the
    positional rows ``pos[i]`` (oxinfer ``encode``: conv1 and conv2 as unfolded projections,
    ``gelu_erf(v) + p``).  Returns ``[ceil(t / 2), d]`` per window."""
    mel = _f64(mel)
    if mel.ndim == 2:
        mel = mel[None]
    outs = []
    for m in mel:
        h = gelu_erf(conv1d_k3(m, conv1_w, conv1_b, 1))
        x = gelu_erf(conv1d_k3(h, conv2_w, conv2_b, 2))
        outs.append(x + _f64(pos)[:x.shape[0]])
    return np.stack(outs)


# ---------------------------------------------------------------- low-precision weights
#
# oxinfer whisper/model.rs, Precision and make_lin: weight matrices may be stored as int8 (q8) or
# int4 (q4, also named q4_0) blocks of 32 consecutive input columns, quantised from the matrix
# rounded to bf16; norms, biases and positions stay f32.  The pages do not print the encodings.
# Reading: the q8_0 / q4_0 block formats the q4_0 name refers to, each block with one fp16 scale:
#   q8: d = amax / 127, codes q = round-half-away(x / d) in [-127, 127], value q d;
#   q4: m = the element of largest magnitude (the first on ties), d = m / -8, codes
#       q = min(15, floor(x / d + 8.5)) in [0, 15], value (q - 8) d.
# The codes are integers decided by floating point, so the steps below are the float32 steps an
# implementation takes (x times the float32 reciprocal of the float32 d; d rounded to fp16 only
# for storage), and the tests compare codes exactly.  Dequantised values are exact in float64.

QBLOCK = 32


def bf16_round(x) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def quantize_q8(w):
    """``w`` ``[n_out, n_in]`` (n_in a multiple of 32) -> (codes int8 ``[n_out, n_in]``, scales
    float16 ``[n_out, n_in / 32]``), from the bf16-rounded matrix."""
    x = bf16_round(w).reshape(w.shape[0], -1, QBLOCK)
    amax = np.max(np.abs(x), axis=2).astype(np.float32)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        idv = np.where(d != 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    v = (x * idv[:, :, None]).astype(np.float32)
    q = (np.sign(v) * np.floor(np.abs(v) + np.float32(0.5))).astype(np.int8)
    return q.reshape(w.shape), d.astype(np.float16)


def dequantize_q8(codes, scales) -> np.ndarray:
    n = codes.shape[0]
    q = codes.astype(np.float64).reshape(n, -1, QBLOCK)
    return (q * scales.astype(np.float64)[:, :, None]).reshape(codes.shape)


def quantize_q4(w):
    """``w`` ``[n_out, n_in]`` -> (codes uint8 in [0, 15] ``[n_out, n_in]``, scales float16
    ``[n_out, n_in / 32]``), from the bf16-rounded matrix."""
    x = bf16_round(w).reshape(w.shape[0], -1, QBLOCK)
    first = np.argmax(np.abs(x), axis=2)  # first index of the largest magnitude
    m = np.take_along_axis(x, first[:, :, None], axis=2)[:, :, 0].astype(np.float32)
    # m / -8 (an all-zero block takes the scale +0: the sign of a zero scale carries nothing)
    d = np.where(m != 0, m / np.float32(-8.0), np.float32(0.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        idv = np.where(d != 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    v = ((x * idv[:, :, None]).astype(np.float32) + np.float32(8.5)).astype(np.float32)
    q = np.minimum(np.floor(v), 15).astype(np.uint8)
    return q.reshape(w.shape), d.astype(np.float16)


def dequantize_q4(codes, scales) -> np.ndarray:
    n = codes.shape[0]
    q = codes.astype(np.float64).reshape(n, -1, QBLOCK) - 8.0
    return (q * scales.astype(np.float64)[:, :, None]).reshape(codes.shape)


QUANT_MATRICES = ("wq", "wk", "wv", "wo", "w1", "w2")


def quantized_layer(p: Dict[str, Optional[np.ndarray]], bits: int) -> Dict[str, Optional[np.ndarray]]:
    """The block's parameters with every weight matrix replaced by its q8 / q4 dequantised values
    (float64); norms and biases unchanged."""
    quant, deq = (quantize_q8, dequantize_q8) if bits == 8 else (quantize_q4, dequantize_q4)
    out = dict(p)
    for name in QUANT_MATRICES:
        out[name] = deq(*quant(p[name]))
    return out


# ---------------------------------------------------------------- MXFP8 operands
#
# The block-scaled fp8 format of gfx950's scaled MFMA (OCP Microscaling Formats (MX) v1.0,
# MXFP8 with E4M3 elements): blocks of 32 consecutive values along the contraction axis share one
# power-of-two scale 2^X (an E8M0 byte X + 127), and each value is stored as an E4M3 number
# (1 sign, 4 exponent bits with bias 7, 3 fraction bits; largest finite magnitude 448, smallest
# normal 2^-6, subnormal quantum 2^-9) rounded to nearest, ties to even.  The pages do not use fp8;
# this is the low-precision MFMA form of oxinfer's block-of-32 weights (Precision, make_lin), with
# the activations quantised the same way because the MFMA takes both operands in the format.
# Reading of the scale: X is the smallest integer with amax <= 448 2^X, so no element saturates
# (the MX specification's floor(log2 amax) - 8 differs only when amax's significand exceeds 1.75,
# where it clamps the block's largest elements to 448 2^X); an all-zero block takes X = -127.
# Every step below is exact in float64 (powers of two and a rounding to a 4-bit significand).

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_round(y) -> np.ndarray:
    """Nearest E4M3 value (ties to even) of each |y| <= 448."""
    y = _f64(y)
    a = np.abs(y)
    if np.any(a > E4M3_MAX):
        raise ValueError("magnitude beyond E4M3's largest finite value")
    _, ex = np.frexp(a)                       # a = f 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6).astype(np.float64)   # exponent of the leading bit; subnormals at -6
    quantum = np.exp2(e - 3)
    return np.copysign(np.round(a / quantum) * quantum, y)  # numpy rounds half to even


def e4m3_bits(v) -> np.ndarray:
    """Bit patterns (uint8) of E4M3 values ``v`` (as returned by ``e4m3_round``)."""
    v = _f64(v)
    a = np.abs(v)
    _, ex = np.frexp(a)
    normal = a >= 2.0 ** -6
    e = np.where(normal, ex - 1, -6)
    frac = np.where(normal, a / np.exp2(e) - 1.0, a / 2.0 ** -6) * 8.0
    field = np.where(normal, e + 7, 0)
    bits = (np.signbit(v).astype(np.int64) << 7) | (field.astype(np.int64) << 3) | frac.astype(np.int64)
    return bits.astype(np.uint8)


def mx_scale_exponent(amax) -> np.ndarray:
    """Smallest integer X with ``amax <= 448 2^X`` (X = -127 for amax = 0), clipped to the E8M0
    range [-127, 127]."""
    amax = _f64(amax)
    f, ex = np.frexp(amax)                    # amax = (2 f) 2^(ex - 1), 2 f in [1, 2)
    x = ex - 9 + (2.0 * f > 1.75)             # 448 = 1.75 2^8
    return np.clip(np.where(amax > 0, x, -127), -127, 127).astype(np.int64)


def mx_quantize(a):
    """MXFP8 blocks of 32 along the last axis (its length a multiple of 32).

    Returns ``(values, X)``: the dequantised values (float64, ``e4m3 * 2^X``, same shape as ``a``)
    and the scale exponents, shape ``a.shape[:-1] + (a.shape[-1] / 32,)``."""
    a = _f64(a)
    blocks = a.reshape(a.shape[:-1] + (-1, MX_BLOCK))
    x = mx_scale_exponent(np.max(np.abs(blocks), axis=-1))
    s = np.exp2(x.astype(np.float64))[..., None]
    vals = e4m3_round(blocks / s) * s
    return vals.reshape(a.shape), x


def mx_values(a) -> np.ndarray:
    """``a`` replaced by its MXFP8 values (blocks of 32 along the last axis)."""
    return mx_quantize(a)[0]


MX_MATRICES = ("wq", "wk", "wv", "w1", "w2")


def mxfp8_layer(p: Dict[str, Optional[np.ndarray]]) -> Dict[str, Optional[np.ndarray]]:
    """The block's parameters with the QKV, fc1 and fc2 matrices replaced by their MXFP8 values
    (blocks of 32 input columns per output row); the output projection, norms and biases
    unchanged."""
    out = dict(p)
    for name in MX_MATRICES:
        out[name] = mx_values(p[name])
    return out
