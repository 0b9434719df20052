"""Write the stored expected outputs of the deep stack configs (oracle only).

The oracle takes tens of seconds per full-depth stack on a few CPU cores, so the GPU tests read
sampled output rows from here instead of recomputing them.  Inputs are regenerated from the
seeded recipe in ``speech_transformer_encoder_amd.synth`` on both sides.

    python tests/golden/make_golden.py [config ...]

Each ``<config>_rows.npz`` holds ``rows`` (row indices into the single window) and ``y`` (the
oracle's final output at those rows, float32), plus ``y_rms`` (RMS of the whole output) and
``pre_rows`` (the residual stream before the final LayerNorm at the same rows).
``<config>_mxfp8_rows.npz`` holds the same rows of the oracle's MXFP8 form of the stack
(``oracle.mxfp8_layer`` weights, ``act=oracle.mx_values`` on the QKV, fc1 and fc2 operands).

    python tests/golden/make_golden.py --mxfp8 [config ...]
"""

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from speech_transformer_encoder_amd import synth  # noqa: E402

N_ROWS = 96


def sample_rows(t: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 9000])
    mid = rng.choice(np.arange(8, t - 8), N_ROWS - 16, replace=False)
    return np.sort(np.concatenate([np.arange(8), mid, np.arange(t - 8, t)]))


def make(name: str) -> str:
    cfg = synth.CONFIGS[name]
    assert cfg.batch == 1
    w = synth.make_workload(cfg)
    t0 = time.time()
    pre = oracle.encoder_stack(w.x[0], w.layers, cfg.heads)
    y = oracle.layer_norm(pre, *w.ln_post) if w.ln_post is not None else pre
    rows = sample_rows(cfg.t, cfg.seed)
    out = os.path.join(HERE, f"{name}_rows.npz")
    np.savez_compressed(out, rows=rows, y=y[rows].astype(np.float32),
                        pre_rows=pre[rows].astype(np.float32),
                        y_rms=np.float64(np.sqrt(np.mean(y * y))))
    print(f"{name}: oracle {time.time() - t0:.1f} s -> {out}", flush=True)
    return out


def make_mx(name: str) -> str:
    cfg = synth.CONFIGS[name]
    assert cfg.batch == 1
    w = synth.make_workload(cfg)
    t0 = time.time()
    layers = [oracle.mxfp8_layer(p) for p in w.layers]
    y = oracle.encoder_stack(w.x[0], layers, cfg.heads, w.ln_post, act=oracle.mx_values)
    rows = sample_rows(cfg.t, cfg.seed)
    out = os.path.join(HERE, f"{name}_mxfp8_rows.npz")
    np.savez_compressed(out, rows=rows, y=y[rows].astype(np.float32))
    print(f"{name} (MXFP8): oracle {time.time() - t0:.1f} s -> {out}", flush=True)
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    mx = "--mxfp8" in args
    names = [a for a in args if a != "--mxfp8"] or ["small_stack", "large_v3_stack"]
    for n in names:
        (make_mx if mx else make)(n)
