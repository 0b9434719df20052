"""The C ABI under HIP graph capture: a whole stack call (every kernel of every block plus the
final LayerNorm) is recorded once on a capturing stream and replayed.  The library allocates,
synchronises and clears nothing, so the captured launches are the eager ones; every replay must
equal the eager result bit for bit.  Replays are interleaved with eager work and host
synchronisation, and each replay is checked."""

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


@pytest.mark.parametrize("path", [B.WENC_PATH_FP16, B.WENC_PATH_Q8])
def test_stack_graph_replays_match_eager(path):
    import torch
    cfg = synth.CONFIGS["base_stack"].with_(t=700, n_layers=3)
    w = synth.make_workload(cfg)
    enc = build_from_workload(w, path)
    x = to_device_input(w.x)
    y = torch.empty_like(x)
    enc.workspace(cfg.batch, cfg.t)  # allocated before capture
    print(f"[case] graph capture path={path}", flush=True)
    enc.forward(x, y)
    torch.cuda.synchronize()
    eager = host(y)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        y.zero_()
        with torch.cuda.graph(graph, stream=s):
            enc.forward(x, y, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), eager, err_msg=f"replay {rep}")
    # eager calls still agree after the replays
    enc.forward(x, y)
    np.testing.assert_array_equal(host(y), eager)
