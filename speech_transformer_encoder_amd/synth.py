"""Seeded synthetic inputs for the Whisper-style encoder block.

This module draws numbers and nothing else: it holds none of the block's arithmetic, so the
GPU path and the CPU oracle can both be fed from it without sharing any computation.

The shapes are those of the public Whisper encoders the pages discuss (tiny.en: 6 heads of width
384, large-v3: 20 heads of width 1280; turbospark-runtime ``whisper/metal.rs``, module doc on
the attention score store).  A 30 s window is zero-padded to ``max_source_positions`` = 1500 encoder
positions (same module doc, "Buffering"; oxinfer ``whisper/model.rs``, ``WhisperConfig`` defaults),
so every window here has t = 1500 unless a test asks for a smaller t.

Recipe (one ``numpy`` PCG64 stream per tensor, so any tensor can be regenerated alone):
  * ``rng = numpy.random.default_rng([seed, layer + 1, tensor_id])``,
    ``rng.standard_normal(shape, dtype=float32) * std``;
  * tensor ids: Wq 1, bq 2, Wk 3, Wv 4, bv 5, Wo 6, bo 7, W1 8, b1 9, W2 10, b2 11;
  * x uses ``[seed, 0, 0]`` and is N(0, 1); weights are N(0, 0.02^2), biases N(0, 0.01^2);
  * LayerNorm gamma = 1, beta = 0 (also for the final LayerNorm);
  * "bf16 weights": the fp32 draw rounded to the nearest bfloat16 (ties to even), stored back in
    fp32, so a consumer that reads the array in fp32 sees the exact bf16 values;
  * outlier rows: per window ``w``, ``default_rng([seed, 0, 1, w]).choice(t, round(frac*t))`` rows
    of x are multiplied by ``scale``.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

TENSOR_IDS = {"wq": 1, "bq": 2, "wk": 3, "wv": 4, "bv": 5, "wo": 6, "bo": 7,
              "w1": 8, "b1": 9, "w2": 10, "b2": 11}

W_STD = 0.02
B_STD = 0.01


@dataclass(frozen=True)
class EncoderConfig:
    """One workload: ``batch`` windows of ``t`` positions through ``n_layers`` blocks."""
    name: str
    seed: int
    batch: int
    t: int
    d_model: int
    heads: int
    ffn_dim: int
    n_layers: int
    bf16_weights: bool
    ln_post: bool
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0

    @property
    def head_dim(self) -> int:
        return self.d_model // self.heads

    @property
    def frames(self) -> int:
        return self.batch * self.t

    def flops(self) -> Dict[str, float]:
        """Algorithmic flops per call: GEMMs 2*M*(4d^2 + 2df) per layer, attention 4*B*t^2*d."""
        m = self.batch * self.t
        d, f = self.d_model, self.ffn_dim
        gemm = 2.0 * m * (4 * d * d + 2 * d * f) * self.n_layers
        attn = 4.0 * self.batch * self.t * self.t * d * self.n_layers
        return {"gemm": gemm, "attention": attn, "total": gemm + attn}

    def with_(self, **kw) -> "EncoderConfig":
        vals = dict(self.__dict__)
        vals.update(kw)
        return EncoderConfig(**vals)


# The five workloads: Whisper tiny, base, small and large-v3 encoder shapes at t = 1500.
CONFIGS: Dict[str, EncoderConfig] = {
    "tiny_block": EncoderConfig("tiny_block", 1, 1, 1500, 384, 6, 1536, 1, False, False),
    "base_stack": EncoderConfig("base_stack", 2, 1, 1500, 512, 8, 2048, 6, False, True),
    "small_stack": EncoderConfig("small_stack", 3, 1, 1500, 768, 12, 3072, 12, True, True),
    "large_v3_stack": EncoderConfig("large_v3_stack", 4, 1, 1500, 1280, 20, 5120, 32, True, True),
    "large_v3_batch16_block": EncoderConfig("large_v3_batch16_block", 5, 16, 1500, 1280, 20, 5120, 1,
                                            True, False, outlier_frac=0.05, outlier_scale=20.0),
}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each fp32 element, returned as fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32)
    # NaN/Inf never occur in these draws; keep them untouched anyway.
    bad = ~np.isfinite(a)
    if bad.any():
        out = out.copy()
        out[bad] = a[bad]
    return out


def _normal(seed: int, layer_plus_one: int, tensor_id: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng([seed, layer_plus_one, tensor_id])
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def make_layer(cfg: EncoderConfig, layer: int) -> Dict[str, Optional[np.ndarray]]:
    """One block's parameters in PyTorch layout: weights are ``[n_out, n_in]``; ``bk`` is None."""
    d, f, s = cfg.d_model, cfg.ffn_dim, cfg.seed
    L = layer + 1
    shapes = {"wq": (d, d), "wk": (d, d), "wv": (d, d), "wo": (d, d), "w1": (f, d), "w2": (d, f),
              "bq": (d,), "bv": (d,), "bo": (d,), "b1": (f,), "b2": (d,)}
    p: Dict[str, Optional[np.ndarray]] = {}
    for name, shp in shapes.items():
        std = W_STD if name.startswith("w") else B_STD
        arr = _normal(s, L, TENSOR_IDS[name], shp, std)
        if cfg.bf16_weights and name.startswith("w"):
            arr = round_to_bf16(arr)
        p[name] = arr
    p["bk"] = None
    p["ln1_g"] = np.ones(d, np.float32)
    p["ln1_b"] = np.zeros(d, np.float32)
    p["ln2_g"] = np.ones(d, np.float32)
    p["ln2_b"] = np.zeros(d, np.float32)
    return p


def make_input(cfg: EncoderConfig) -> np.ndarray:
    """x ``[batch, t, d]`` fp32, N(0, 1), with the configured outlier rows scaled per window."""
    x = _normal(cfg.seed, 0, 0, (cfg.batch, cfg.t, cfg.d_model), 1.0)
    if cfg.outlier_frac > 0.0:
        n = int(round(cfg.outlier_frac * cfg.t))
        for w in range(cfg.batch):
            rows = np.random.default_rng([cfg.seed, 0, 1, w]).choice(cfg.t, n, replace=False)
            x[w, rows, :] *= np.float32(cfg.outlier_scale)
    return x


def make_ln_post(cfg: EncoderConfig):
    if not cfg.ln_post:
        return None
    d = cfg.d_model
    return np.ones(d, np.float32), np.zeros(d, np.float32)


@dataclass
class Workload:
    cfg: EncoderConfig
    x: np.ndarray
    layers: List[Dict[str, Optional[np.ndarray]]] = field(default_factory=list)
    ln_post: Optional[tuple] = None


def make_workload(cfg: EncoderConfig, n_layers: Optional[int] = None) -> Workload:
    n = cfg.n_layers if n_layers is None else n_layers
    return Workload(cfg, make_input(cfg), [make_layer(cfg, i) for i in range(n)], make_ln_post(cfg))


def ragged_lengths(seed: int, batch: int, max_t: int = 1500, min_t: int = 150) -> np.ndarray:
    """Window lengths of a ragged batch: uniform integers in ``[min_t, max_t]`` (3 s to 30 s of
    audio at 50 encoder positions per second), int32."""
    rng = np.random.default_rng([seed, 300, 0])
    return rng.integers(min_t, max_t + 1, size=batch).astype(np.int32)


def random_qkv(seed: int, batch: int, t: int, heads: int, head_dim: int = 64,
               outlier_frac: float = 0.0, outlier_scale: float = 1.0):
    """Standalone attention operands ``q, k, v`` of shape ``[batch, t, heads*head_dim]``.

    Entries are N(0, 1) / head_dim^0.25 so that the scaled logits have unit variance; a fraction of
    query rows may be multiplied by ``outlier_scale`` (logit spreads of about +-100 at scale 20),
    which exercises the running-max bookkeeping of the online softmax.
    """
    d = heads * head_dim
    rng = np.random.default_rng([seed, 1000, 0])
    sc = np.float32(head_dim ** -0.25)
    q = rng.standard_normal((batch, t, d), dtype=np.float32) * sc
    k = rng.standard_normal((batch, t, d), dtype=np.float32) * sc
    v = rng.standard_normal((batch, t, d), dtype=np.float32)
    if outlier_frac > 0.0:
        n = max(1, int(round(outlier_frac * t)))
        for w in range(batch):
            rows = np.random.default_rng([seed, 1000, 1, w]).choice(t, n, replace=False)
            q[w, rows, :] *= np.float32(outlier_scale)
    return q, k, v


# Decoder cross-attention weights for the cross K/V step: tensor ids 21 (Wk), 22 (Wv), 23 (bv)
# of decoder layer l, drawn with ``default_rng([seed, 100 + l, id])`` like the encoder's.
CROSS_IDS = {"wk": 21, "wv": 22, "bv": 23}


def make_cross_layers(seed: int, n_layers: int, d: int, bf16: bool = True):
    layers = []
    for l in range(n_layers):
        p = {}
        for name, tid in CROSS_IDS.items():
            shape = (d,) if name == "bv" else (d, d)
            std = B_STD if name == "bv" else W_STD
            rng = np.random.default_rng([seed, 100 + l, tid])
            arr = (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
            if bf16 and name != "bv":
                arr = round_to_bf16(arr)
            p[name] = arr
        layers.append(p)
    return layers


# Conv front end inputs.  A 30 s window is 3000 mel frames (two per encoder position).  Whisper's
# log-mel features are clipped to 8 decades below the window's maximum and mapped by
# (log10 + 4) / 4, so they lie in about [-1, 1.5]; the synthetic frames are N(0.2, 0.4^2).
# Conv weights: tensor ids 31 (conv1_w), 32 (conv1_b), 33 (conv2_w), 34 (conv2_b), drawn like
# the block's (N(0, 0.02^2) weights, N(0, 0.01^2) biases).  Positions: the sinusoidal table of
# the Whisper encoder (sin of position / 10000^(k / (d/2 - 1)) in the first half of the row, cos
# in the second).
N_MELS = {384: 80, 512: 80, 768: 80, 1280: 128}
STEM_IDS = {"conv1_w": 31, "conv1_b": 32, "conv2_w": 33, "conv2_b": 34}


def make_mel(seed: int, batch: int, frames: int, n_mels: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 200, 0])
    return (rng.standard_normal((batch, frames, n_mels), dtype=np.float32) * np.float32(0.4)
            + np.float32(0.2)).astype(np.float32)


def sinusoid_positions(n: int, d: int) -> np.ndarray:
    half = d // 2
    inc = np.log(10000.0) / (half - 1)
    inv = np.exp(-inc * np.arange(half))
    ang = np.arange(n)[:, None] * inv[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1).astype(np.float32)


def make_stem(seed: int, n_mels: int, d: int, bf16: bool = True, n_pos: int = 1500):
    shapes = {"conv1_w": (d, n_mels, 3), "conv1_b": (d,), "conv2_w": (d, d, 3), "conv2_b": (d,)}
    p = {}
    for name, shp in shapes.items():
        rng = np.random.default_rng([seed, 200, STEM_IDS[name]])
        std = W_STD if name.endswith("_w") else B_STD
        arr = (rng.standard_normal(shp, dtype=np.float32) * np.float32(std)).astype(np.float32)
        if bf16 and name.endswith("_w"):
            arr = round_to_bf16(arr)
        p[name] = arr
    p["pos"] = sinusoid_positions(n_pos, d)
    return p
