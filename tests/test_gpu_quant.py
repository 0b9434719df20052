"""Low-precision weights (q8 / q4 blocks of 32 with fp16 scales) on the GPU, against the CPU
oracle, through the C ABI.

* The quantiser's codes and scales are integers and fp16 bit patterns decided by floating point
  in the same fp32 steps on both sides: compared exactly.
* Dequantised fp16 weights: code * scale is exact in fp32 and rounded once to fp16 on the GPU;
  compared exactly with numpy's float16 rounding of the oracle's exact values.
* Blocks and stacks on the Q8 / Q4 paths against the oracle run on the dequantised weights
  (``oracle.quantized_layer``): the remaining error is the fp16 path's (weights rounded to fp16,
  16-bit activations), so the bar is the block's (max_rel 2e-2, MAE 1e-3).
* Each block call expands its layer's codes with the kernel behind
  ``whisper_enc_dequantize_matrix`` and runs the fp16 GEMMs: a Q8 / Q4 stack equals, bit for bit,
  the fp16 stack on the weights that entry point expands, at one window (split-k parts on the
  small kernel) and for three batched windows (the persistent kernel).
"""

import numpy as np
import pytest

import oracle
from speech_transformer_encoder_amd import binding as B
from speech_transformer_encoder_amd import synth
from speech_transformer_encoder_amd.encoder import build_from_workload, to_device_input
from tests.gpu_util import dev, errors, host, report, require_gpu

pytestmark = pytest.mark.gpu

QPATHS = {8: B.WENC_PATH_Q8, 4: B.WENC_PATH_Q4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _matrix(seed, n, k):
    r = np.random.default_rng([seed, 77])
    w = (r.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                              # an all-zero block
    w[1, :32] = (np.arange(32) - 16) * 2.0 ** -9  # exact levels and ties
    w[2, 32:64] = np.float32(1e-6)               # scales in the fp16 subnormal range
    if n > 3:
        w[3, :32] = r.standard_normal(32).astype(np.float32) * 50
    if n > 4:
        w[4, :32] = 0.01
        w[4, 5] = -0.01                           # equal magnitudes: the first one decides
    return w


def _gpu_quantize(w, bits):
    import torch
    n, k = w.shape
    codes = torch.empty(n * k * bits // 8, dtype=torch.uint8, device="cuda")
    scales = torch.empty(n * (k // 32), dtype=torch.int16, device="cuda")
    B.whisper_enc_quantize_matrix(dev(w), codes, scales, n, k, bits)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    s = scales.cpu().numpy().view(np.float16).reshape(n, k // 32)
    if bits == 8:
        return c.view(np.int8).reshape(n, k), s, codes, scales
    c = c.reshape(n, k // 2)
    unpacked = np.empty((n, k), np.uint8)
    unpacked[:, 0::2] = c & 15
    unpacked[:, 1::2] = c >> 4
    return unpacked, s, codes, scales


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("n,k", [(5, 32), (64, 1280), (1280, 5120), (3, 96)])
def test_quantize_matrix_exact(bits, n, k):
    w = _matrix(n + k, n, k)
    print(f"[case] quantize bits={bits} n={n} k={k}", flush=True)
    codes, scales, _, _ = _gpu_quantize(w, bits)
    ref_c, ref_s = (oracle.quantize_q8 if bits == 8 else oracle.quantize_q4)(w)
    np.testing.assert_array_equal(scales.view(np.uint16), ref_s.view(np.uint16))
    np.testing.assert_array_equal(codes, ref_c)


@pytest.mark.parametrize("bits", [8, 4])
def test_dequantize_matrix_exact(bits):
    import torch
    n, k = 384, 1536
    w = _matrix(3, n, k)
    _, _, codes, scales = _gpu_quantize(w, bits)
    out = torch.empty((n, k), dtype=torch.float16, device="cuda")
    B.whisper_enc_dequantize_matrix(codes, scales, out, n, k, bits)
    ref_c, ref_s = (oracle.quantize_q8 if bits == 8 else oracle.quantize_q4)(w)
    deq = (oracle.dequantize_q8 if bits == 8 else oracle.dequantize_q4)(ref_c, ref_s)
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got.view(np.uint16), deq.astype(np.float16).view(np.uint16))


def _check(e, tag):
    report(tag, e)
    assert e["finite"] and e["max_rel"] <= 2e-2 and e["mae"] <= 1e-3, (tag, e)


def _ref_stack(w, bits, n_layers=None, final_norm=True):
    layers = [oracle.quantized_layer(p, bits) for p in w.layers[:n_layers]]
    return oracle.encoder_stack(w.x, layers, w.cfg.heads, w.ln_post if final_norm else None)


@pytest.mark.parametrize("bits", [8, 4])
def test_block_quantized_small(bits):
    cfg = synth.CONFIGS["tiny_block"].with_(batch=2, t=200)
    w = synth.make_workload(cfg)
    print(f"[case] block q{bits} tiny 2 x 200", flush=True)
    enc = build_from_workload(w, QPATHS[bits])
    got = host(enc.forward(to_device_input(w.x)))
    _check(errors(got, _ref_stack(w, bits)), f"block q{bits} tiny")


@pytest.mark.parametrize("bits", [8, 4])
def test_stack_quantized_base(bits):
    cfg = synth.CONFIGS["base_stack"].with_(t=300, n_layers=3)
    w = synth.make_workload(cfg)
    print(f"[case] stack q{bits} base x3", flush=True)
    enc = build_from_workload(w, QPATHS[bits])
    got = host(enc.forward(to_device_input(w.x)))
    _check(errors(got, _ref_stack(w, bits)), f"stack q{bits} base")


def test_varlen_quantized():
    cfg = synth.CONFIGS["base_stack"].with_(batch=1, t=700, n_layers=2)
    w = synth.make_workload(cfg)
    lens = [300, 1, 399]
    enc = build_from_workload(w, B.WENC_PATH_Q8)
    got = host(enc.forward_varlen(to_device_input(w.x[0]), lens))
    layers = [oracle.quantized_layer(p, 8) for p in w.layers]
    ref = oracle.encoder_stack_varlen(w.x[0], lens, layers, cfg.heads, w.ln_post)
    _check(errors(got, ref), "varlen q8 base")


@pytest.mark.parametrize("bits", [8, 4])
def test_block_quantized_large_v3_batch16(bits):
    """The batched large-v3 block with q8 / q4 weights, sampled rows of every window."""
    cfg = synth.CONFIGS["large_v3_batch16_block"]
    w = synth.make_workload(cfg)
    print(f"[case] block q{bits} large-v3 16 x 1500", flush=True)
    enc = build_from_workload(w, QPATHS[bits])
    got = host(enc.forward(to_device_input(w.x), final_norm=False))
    p = oracle.quantized_layer(w.layers[0], bits)
    r = np.random.default_rng([9, 94])
    for b in range(cfg.batch):
        rows = np.unique(np.concatenate([[0, cfg.t - 1], r.choice(cfg.t, 6, replace=False)]))
        ref = oracle.encoder_block_rows(w.x[b], p, cfg.heads, rows)
        _check(errors(got[b, rows], ref), f"block q{bits} large window {b}")


def _expanded_layers(layers, bits):
    """Each matrix quantised and expanded back to fp16 by the library's codec (the values the
    Q8 / Q4 GEMMs multiply), as fp32 arrays in PyTorch layout."""
    import torch
    out = []
    for p in layers:
        q = dict(p)
        for name in ("wq", "wk", "wv", "wo", "w1", "w2"):
            n, k = p[name].shape
            _, _, codes, scales = _gpu_quantize(p[name], bits)
            e = torch.empty((n, k), dtype=torch.float16, device="cuda")
            B.whisper_enc_dequantize_matrix(codes, scales, e, n, k, bits)
            q[name] = host(e).astype(np.float32)
        out.append(q)
    return out


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("name,over", [("base_stack", {"n_layers": 2}),
                                       ("large_v3_stack", {"n_layers": 1}),
                                       ("large_v3_batch16_block", {"batch": 3})])
def test_quantized_equals_fp16_on_expanded_weights(bits, name, over):
    """Bit-identical to the fp16 path on the expanded weights.  base at one window: out-projection
    and fc2 as split-k parts with the fused LayerNorms; large-v3 at one window: QKV, fc1 on the
    128 x 256 tiles, fc2 in 4 parts; three large-v3 windows: 4500 rows on the persistent kernel."""
    from speech_transformer_encoder_amd.encoder import EncoderStack
    cfg = synth.CONFIGS[name].with_(**over)
    w = synth.make_workload(cfg)
    print(f"[case] q{bits} vs fp16 on expanded weights: {name} {over}", flush=True)
    x = to_device_input(w.x)
    got = host(build_from_workload(w, QPATHS[bits]).forward(x))
    enc16 = EncoderStack(_expanded_layers(w.layers, bits), cfg.d_model, cfg.heads, cfg.ffn_dim,
                         B.WENC_PATH_FP16, w.ln_post)
    ref = host(enc16.forward(x))
    assert np.isfinite(got).all()
    np.testing.assert_array_equal(got, ref)
