"""The no-allocation stack entry point against the workspace entry point, through the C ABI.

``whisper_enc_stack_forward_noalloc`` runs the same kernels with the same split plans as
``whisper_enc_stack_forward``; only the workspace differs (a static device array instead of the
caller's buffer), so the outputs must be bit-identical.  Calls run back to back, the later ones on
smaller inputs, so a call that relied on what an earlier one left in the shared array would show.
"""

import numpy as np
import pytest

from speech_transformer_encoder_amd import binding as B
from speech_transformer_encoder_amd import synth
from speech_transformer_encoder_amd.encoder import build_from_workload, to_device_input
from tests.gpu_util import host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _both(cfg, path):
    import torch
    w = synth.make_workload(cfg)
    enc = build_from_workload(w, path)
    x = to_device_input(w.x)
    batch, t, d = x.shape
    g, b = enc.ln_post if enc.ln_post is not None else (None, None)
    print(f"[case] noalloc {cfg.name} batch={batch} t={t} d={d} layers={enc.n_layers} path={path}",
          flush=True)
    y = torch.full_like(x, float("nan"))
    B.whisper_enc_stack_forward_noalloc(x, y, enc.blob, enc.n_layers, g, b, batch, t, d,
                                        cfg.heads, cfg.ffn_dim, path)
    got = host(y)
    ref = host(enc.forward(x))  # the workspace entry point
    return got, ref


def test_noalloc_equals_workspace_call_on_shrinking_inputs():
    cases = [
        # one large-v3 window, 2 blocks + final norm: split-k parts (4 of fc2, 2 of the
        # out-projection) with the fused LayerNorms, 47.6 MiB of the 64 MiB scratch
        (synth.CONFIGS["large_v3_stack"].with_(n_layers=2), B.WENC_PATH_FP16),
        # smaller: 8 heads of an 1100-position window, attention key halves in the scratch
        (synth.CONFIGS["tiny_block"].with_(t=1100, d_model=512, heads=8, ffn_dim=1024),
         B.WENC_PATH_BF16),
        # smaller again: two short windows on the fp32 path
        (synth.CONFIGS["tiny_block"].with_(batch=2, t=130), B.WENC_PATH_FP32),
    ]
    for cfg, path in cases:
        got, ref = _both(cfg, path)
        assert np.isfinite(got).all()
        np.testing.assert_array_equal(got, ref)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    import torch
    d, h, f = 1280, 20, 5120
    need = B.whisper_enc_workspace_bytes(2, 1500, d, h, f, B.WENC_PATH_FP16)
    assert need > B.WENC_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(2, 1500, d, device="cuda")
    y = torch.empty_like(x)
    layer = torch.empty(B.whisper_enc_layer_bytes(d, f, B.WENC_PATH_FP16), dtype=torch.uint8,
                        device="cuda")
    with pytest.raises(B.WencError) as ei:
        B.whisper_enc_stack_forward_noalloc(x, y, layer, 1, None, None, 2, 1500, d, h, f,
                                            B.WENC_PATH_FP16)
    assert ei.value.code == B.WENC_ERR_SCRATCH
