"""The seeded generator: reproducible draws, the workload recipe, and bf16 rounding."""

import numpy as np
import torch

from speech_transformer_encoder_amd import synth


def test_round_to_bf16_matches_torch_rne():
    r = np.random.default_rng(0)
    a = np.concatenate([r.standard_normal(100000).astype(np.float32) * 0.02,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  3.0e38, 1e-40], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(synth.round_to_bf16(a), ref)


def test_workload_recipe_and_reproducibility():
    cfg = synth.CONFIGS["large_v3_batch16_block"].with_(batch=3, t=200)
    w1 = synth.make_workload(cfg)
    w2 = synth.make_workload(cfg)
    np.testing.assert_array_equal(w1.x, w2.x)
    p = w1.layers[0]
    assert p["bk"] is None and p["wq"].shape == (1280, 1280) and p["w1"].shape == (5120, 1280)
    # bf16 weights: the low 16 bits are zero
    assert (p["w2"].view(np.uint32) & 0xFFFF).max() == 0
    assert abs(p["wo"].std() - 0.02) < 1e-3 and abs(p["b1"].std() - 0.01) < 1e-3
    # exactly 5 % of the rows of each window are scaled by 20
    norms = np.linalg.norm(w1.x, axis=-1)
    assert ((norms > 200).sum(axis=1) == 10).all()
    tiny = synth.make_workload(synth.CONFIGS["tiny_block"])
    assert (tiny.layers[0]["wq"].view(np.uint32) & 0xFFFF).max() != 0  # fp32 weights


def test_flop_counts():
    c4 = synth.CONFIGS["large_v3_stack"]
    f = c4.flops()
    assert abs(f["gemm"] / 1e9 - 32 * 58.98) < 1.0
    assert abs(f["attention"] / 1e9 - 32 * 11.52) < 0.1
