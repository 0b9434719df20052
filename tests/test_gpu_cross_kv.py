"""Cross-attention keys and values of the decoder layers (the step after the encoder) on the GPU,
against the CPU oracle, through the C ABI.

The projection's operands are rounded to the path's type first (the encoder output when the
library converts it, the weights when they are packed) and the oracle receives those exact values,
so the remaining error is the kernel's: fp32 accumulation and the rounding of the stored result
(one 16-bit ulp: 2^-8 bf16, 2^-11 fp16; fp32 accumulation noise on the fp32 path).
"""

import numpy as np
import pytest

import oracle
from speech_transformer_encoder_amd import binding as B
from speech_transformer_encoder_amd import synth
from tests.gpu_util import as_operand, dev, errors, host, report, require_gpu, torch_dtype

pytestmark = pytest.mark.gpu

PATHS = [B.WENC_PATH_BF16, B.WENC_PATH_FP16, B.WENC_PATH_FP32]
OUT_TOL = {B.WENC_PATH_BF16: 5e-3, B.WENC_PATH_FP16: 8e-4, B.WENC_PATH_FP32: 2e-5}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(y, layers, heads, path):
    import torch
    batch, t, d = y.shape
    L = len(layers)
    nbytes = B.whisper_enc_cross_kv_bytes(d, L, path)
    blob = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    wk = [dev(p["wk"]) for p in layers]
    wv = [dev(p["wv"]) for p in layers]
    bv = [dev(p["bv"]) for p in layers]
    B.whisper_enc_pack_cross_kv(wk, wv, bv, L, d, path, blob)
    ws_bytes = B.whisper_enc_cross_kv_workspace_bytes(batch, t, d, path)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    kv = torch.full((batch, L, 2, heads, t, 64), float("nan"), dtype=torch_dtype(path), device="cuda")
    yd = dev(y)
    B.whisper_enc_cross_kv(yd, kv, blob, L, batch, t, d, heads, path, ws, ws.numel())
    return kv


def _rounded(a, path):
    return as_operand(a, path)[1]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("batch,t,d,L", [(1, 1, 64, 1), (2, 150, 128, 3), (1, 333, 384, 2),
                                         (3, 1500, 256, 2)])
def test_cross_kv_small(path, batch, t, d, L):
    heads = d // 64
    r = np.random.default_rng([batch, t, d, L, 91])
    y = r.standard_normal((batch, t, d)).astype(np.float32) * 2
    layers = synth.make_cross_layers(batch + t, L, d, bf16=False)
    print(f"[case] cross_kv path={path} batch={batch} t={t} d={d} L={L}", flush=True)
    got = host(_run(y, layers, heads, path))
    yr = _rounded(y, path)
    lr = [{"wk": _rounded(p["wk"], path), "wv": _rounded(p["wv"], path), "bv": p["bv"]} for p in layers]
    e = errors(got, oracle.cross_kv(yr, lr, heads))
    report(f"cross_kv p{path} b{batch} t{t} d{d} L{L}", e)
    assert e["finite"] and e["max_rel"] <= OUT_TOL[path]


def test_cross_kv_large_v3_sampled():
    """The large-v3 decoder's 32 layers over 16 windows (3.9 GB of fp16 keys and values), checked
    on sampled (window, layer, head, position) rows against the oracle."""
    path = B.WENC_PATH_FP16
    batch, t, d, L, heads = 16, 1500, 1280, 32, 20
    cfg = synth.CONFIGS["large_v3_batch16_block"]
    y = synth.make_input(cfg)
    layers = synth.make_cross_layers(cfg.seed, L, d, bf16=True)
    print("[case] cross_kv large-v3 16 x 1500, 32 decoder layers", flush=True)
    kv = _run(y, layers, heads, path)
    r = np.random.default_rng([5, 92])
    yr = _rounded(y, path)
    for _ in range(6):
        b, l = int(r.integers(batch)), int(r.integers(L))
        rows = np.unique(np.concatenate([[0, t - 1], r.choice(t, 14, replace=False)]))
        ref = oracle.cross_kv(yr[b:b + 1, rows], [layers[l]], heads)[0, 0]  # [2, heads, rows, 64]
        got = host(kv[b, l][:, :, rows])
        e = errors(got, ref)
        report(f"cross_kv large b{b} l{l}", e)
        assert e["finite"] and e["max_rel"] <= OUT_TOL[path]
