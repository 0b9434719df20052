"""The convolutional front end (the step before the first block) on the GPU, against the CPU
oracle, through the C ABI.

The GPU path rounds the mel rows and the conv weights to the path's type, and stores the first
convolution's GELU output h in that type before the second convolution reads it.  Two references:

* staged: the oracle's conv1 + GELU on the rounded operands, h rounded to the path's type, then the
  oracle's conv2 + GELU + positions.  What remains is the kernels' fp32 accumulation and h values
  that land on the other side of a rounding boundary (one 16-bit ulp of one term), so the bound is
  tight: of the order of the path's unit roundoff;
* model: the oracle's conv_stem in float64 on the unrounded operands, at the block's output bar
  (max_rel 2e-2 and MAE 1e-3).
"""

import numpy as np
import pytest

import oracle
from speech_transformer_encoder_amd import binding as B
from speech_transformer_encoder_amd import synth
from tests.gpu_util import as_operand, dev, errors, host, report, require_gpu

pytestmark = pytest.mark.gpu

PATHS = [B.WENC_PATH_BF16, B.WENC_PATH_FP16, B.WENC_PATH_FP32]
STAGED_TOL = {B.WENC_PATH_BF16: 5e-3, B.WENC_PATH_FP16: 8e-4, B.WENC_PATH_FP32: 2e-5}
MODEL_MAX_REL, MODEL_MAE = 2e-2, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(mel, p, path):
    import torch
    batch, t, n_mels = mel.shape
    d = p["conv1_w"].shape[0]
    n_pos = p["pos"].shape[0]
    blob = torch.empty(B.whisper_enc_stem_bytes(n_mels, d, n_pos, path), dtype=torch.uint8,
                       device="cuda")
    src = {k: dev(v) for k, v in p.items()}
    B.whisper_enc_pack_stem(src["conv1_w"], src["conv1_b"], src["conv2_w"], src["conv2_b"],
                            src["pos"], n_mels, d, n_pos, path, blob)
    ws_bytes = B.whisper_enc_stem_workspace_bytes(batch, t, n_mels, d, path)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    t2 = (t + 1) // 2
    x = torch.full((batch, t2, d), float("nan"), dtype=torch.float32, device="cuda")
    B.whisper_enc_stem_forward(dev(mel), x, blob, batch, t, n_mels, d, n_pos, path, ws, ws.numel())
    return x


def _r(a, path):
    return as_operand(a, path)[1]


def _staged(mel, p, path):
    """conv1 + GELU, h rounded to the path's type, conv2 + GELU + positions (oracle steps)."""
    w1, w2 = _r(p["conv1_w"], path), _r(p["conv2_w"], path)
    out = []
    for m in _r(mel, path):
        h = _r(oracle.gelu_erf(oracle.conv1d_k3(m, w1, p["conv1_b"], 1)).astype(np.float32), path)
        x = oracle.gelu_erf(oracle.conv1d_k3(h, w2, p["conv2_b"], 2))
        out.append(x + p["pos"][:x.shape[0]])
    return np.stack(out)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("batch,t,n_mels,d", [(1, 1, 80, 64), (2, 2, 80, 64), (2, 7, 80, 128),
                                              (1, 301, 80, 384), (2, 3000, 80, 384),
                                              (1, 1001, 128, 256)])
def test_stem_small(path, batch, t, n_mels, d):
    p = synth.make_stem(batch * 7 + t, n_mels, d, bf16=False)
    mel = synth.make_mel(t + d, batch, t, n_mels)
    print(f"[case] stem path={path} batch={batch} t={t} n_mels={n_mels} d={d}", flush=True)
    got = host(_run(mel, p, path))
    assert got.shape == (batch, (t + 1) // 2, d)
    e = errors(got, _staged(mel, p, path))
    report(f"stem staged p{path} b{batch} t{t} m{n_mels} d{d}", e)
    assert e["finite"] and e["max_rel"] <= STAGED_TOL[path]
    e = errors(got, oracle.conv_stem(mel, **p))
    report(f"stem model p{path} b{batch} t{t} m{n_mels} d{d}", e)
    assert e["max_rel"] <= MODEL_MAX_REL and e["mae"] <= MODEL_MAE


def test_stem_more_positions_than_frames():
    """A short window reads only its first ceil(t / 2) positional rows."""
    path = B.WENC_PATH_FP32
    p = synth.make_stem(3, 80, 128, bf16=False, n_pos=1500)
    mel = synth.make_mel(4, 1, 40, 80)
    got = host(_run(mel, p, path))
    e = errors(got, oracle.conv_stem(mel, **p))
    assert e["max_rel"] <= STAGED_TOL[path]


@pytest.mark.parametrize("path", [B.WENC_PATH_FP16, B.WENC_PATH_BF16])
def test_stem_large_v3_batch16(path):
    """large-v3's front end (128 mel bins, width 1280) over 16 windows of 3000 frames, in the
    launch configuration the benchmark times; three whole windows checked against the oracle."""
    batch, t, n_mels, d = 16, 3000, 128, 1280
    p = synth.make_stem(11, n_mels, d, bf16=True)
    mel = synth.make_mel(12, batch, t, n_mels)
    print(f"[case] stem large-v3 16 x 3000 path={path}", flush=True)
    got = host(_run(mel, p, path))
    for b in (0, 7, batch - 1):
        e = errors(got[b:b + 1], _staged(mel[b:b + 1], p, path))
        report(f"stem large staged p{path} b{b}", e)
        assert e["finite"] and e["max_rel"] <= STAGED_TOL[path]
        e = errors(got[b:b + 1], oracle.conv_stem(mel[b:b + 1], **p))
        report(f"stem large model p{path} b{b}", e)
        assert e["max_rel"] <= MODEL_MAX_REL and e["mae"] <= MODEL_MAE
