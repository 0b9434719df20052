"""Helpers shared by the GPU parity tests: device transfers, 16-bit rounding of test operands and
the error metrics.  Nothing here computes the block; the oracle does that on the CPU."""

import math
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from speech_transformer_encoder_amd import binding as B  # noqa: E402

PATH_NAMES = {B.WENC_PATH_BF16: "bf16", B.WENC_PATH_FP16: "fp16", B.WENC_PATH_FP32: "fp32",
              B.WENC_PATH_BF16X2: "bf16x2", B.WENC_PATH_BF16X3: "bf16x3", B.WENC_PATH_Q8: "q8",
              B.WENC_PATH_Q4: "q4", B.WENC_PATH_MXFP8: "mxfp8"}


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B.load()  # raises if the library is missing: no silent fallback


def torch_dtype(path):
    import torch
    return {B.WENC_PATH_BF16: torch.bfloat16, B.WENC_PATH_FP16: torch.float16,
            B.WENC_PATH_FP32: torch.float32}[path]


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t if dtype is None else t.to(dtype)


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def as_operand(a, path):
    """The test operand rounded to the path's type: returns (device tensor, exact host values)."""
    t = dev(a, torch_dtype(path))
    return t, host(t)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    rms = math.sqrt(float(np.mean(ref * ref))) or 1.0
    return {
        "max_rel": float(np.max(diff / np.maximum(np.abs(ref), rms))),
        "mae": float(np.mean(diff)),
        "max_abs": float(np.max(diff)),
        "normwise": float(np.max(diff) / max(float(np.max(np.abs(ref))), 1e-300)),
        "finite": bool(np.isfinite(got).all()),
    }


def report(tag, e):
    print(f"[parity] {tag}: max_rel={e['max_rel']:.3e} mae={e['mae']:.3e} "
          f"max_abs={e['max_abs']:.3e}", flush=True)
