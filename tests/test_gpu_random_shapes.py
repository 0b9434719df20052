"""Seeded random shapes for the projection and attention steps, beside the hand-picked ones of
test_gpu_steps: every element against the oracle, with that file's bounds.  The draws are fixed
by the seed, so every run checks the same cases; they reach tiling, tail and dispatch
combinations a short list misses (odd row counts against every tile height, widths that are
multiples of 64 but not of 128 or 256, key counts around the 64-key tiles)."""

import numpy as np
import pytest

import oracle
from speech_transformer_encoder_amd import binding as B
from tests.gpu_util import as_operand, dev, errors, host, report, require_gpu, torch_dtype
from tests.test_gpu_steps import ATTN_CW, ATTN_TOL, OUT_TOL, _attention_case

pytestmark = pytest.mark.gpu

PATHS = [B.WENC_PATH_BF16, B.WENC_PATH_FP16, B.WENC_PATH_FP32]
EPIS = [B.WENC_EPI_BIAS, B.WENC_EPI_BIAS_GELU, B.WENC_EPI_BIAS_RESIDUAL,
        B.WENC_EPI_BIAS_GELU_RESIDUAL]


def _linear_cases(count=24, seed=2024):
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        m = int(r.integers(1, 6001))
        n = 64 * int(r.integers(1, 81))
        k = 64 * int(r.integers(1, 41))
        if m * n * k > 1.5e9:  # keeps the float64 reference to about a second
            continue
        cases.append((PATHS[len(cases) % 3], EPIS[int(r.integers(0, 4))], m, n, k))
    return cases


def _persistent_cases(count=12, seed=2029):
    """Shapes with at least 256 tiles of 256 x 256 (the persistent kernel, and its half-tile tail
    when the last round is short), k kept small for the reference."""
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        m = int(r.integers(3000, 24001))
        n = 64 * int(r.integers(8, 81))
        k = 64 * int(r.integers(1, 5))
        tiles = -(-m // 256) * -(-n // 256)
        if tiles < 256 or m * n * k > 5e9:
            continue
        cases.append((PATHS[len(cases) % 3], EPIS[int(r.integers(0, 4))], m, n, k))
    return cases


def _attention_cases(count=12, seed=2025):
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        batch, t, heads = int(r.integers(1, 4)), int(r.integers(1, 1601)), int(r.integers(1, 9))
        if batch * heads * t * t > 6e6:
            continue
        cases.append((PATHS[len(cases) % 3], batch, t, heads))
    return cases


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("path,epi,m,n,k", _linear_cases() + _persistent_cases())
def test_linear_random(path, epi, m, n, k):
    import torch
    r = np.random.default_rng([m, n, k, epi, 99])
    a = r.standard_normal((m, k)).astype(np.float32)
    w = (r.standard_normal((n, k)) * 0.02).astype(np.float32)
    bias = (r.standard_normal(n) * 0.1).astype(np.float32)
    ad, ah = as_operand(a, path)
    wd, wh = as_operand(w, path)
    ref = oracle.linear(ah, wh, bias)
    resid = None
    fp32_out = epi in (B.WENC_EPI_BIAS_RESIDUAL, B.WENC_EPI_BIAS_GELU_RESIDUAL)
    if epi in (B.WENC_EPI_BIAS_GELU, B.WENC_EPI_BIAS_GELU_RESIDUAL):
        ref = oracle.gelu_erf(ref)
    if fp32_out:
        res_np = r.standard_normal((m, n)).astype(np.float32) * 4
        resid = dev(res_np)
        ref = ref + res_np
        c = torch.empty((m, n), dtype=torch.float32, device="cuda")
    else:
        c = torch.empty((m, n), dtype=torch_dtype(path), device="cuda")
    print(f"[case] random linear path={path} epi={epi} m={m} n={n} k={k}", flush=True)
    B.whisper_enc_linear(ad, wd, dev(bias), resid, c, m, n, k, path, epi)
    e = errors(host(c), ref)
    report(f"random linear p{path} e{epi} {m}x{n}x{k}", e)
    assert e["finite"] and e["max_rel"] <= (2e-5 if fp32_out else OUT_TOL[path])


@pytest.mark.parametrize("path,batch,t,heads", _attention_cases())
def test_attention_random(path, batch, t, heads):
    e, cw = _attention_case(path, batch, t, heads, seed=t + 13 * heads + 101 * batch)
    report(f"random attn p{path} b{batch} t{t} h{heads} cw={cw:.3e}", e)
    assert e["finite"] and e["max_rel"] <= ATTN_TOL[path] and cw <= ATTN_CW[path]


def _block_cases(count=9, seed=2026):
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        heads = int(r.integers(1, 13))
        d = 64 * heads
        ffn = 64 * int(r.integers(1, 4 * heads + 9))
        batch, t = int(r.integers(1, 4)), int(r.integers(1, 700))
        if batch * t * (t * d + 4 * d * d + 2 * d * ffn) > 1.2e9:
            continue
        cases.append((PATHS[len(cases) % 3], batch, t, d, heads, ffn))
    return cases


@pytest.mark.parametrize("path,batch,t,d,heads,ffn", _block_cases())
def test_block_random(path, batch, t, d, heads, ffn):
    """A whole block at a random (windows, t, d, heads, ffn) with random fp32 weights, every
    element against the oracle under the block's bounds (the fp32 path: max-rel <= 1e-4; the
    16-bit paths: max-rel <= 2e-2 and MAE <= 1e-3 -- one block, so literal bf16 is held to the
    bar too)."""
    from speech_transformer_encoder_amd import synth
    from tests.test_gpu_block import check, run_gpu
    cfg = synth.CONFIGS["tiny_block"].with_(seed=97 + t, batch=batch, t=t, d_model=d, heads=heads,
                                            ffn_dim=ffn)
    w = synth.make_workload(cfg)
    print(f"[case] random block path={path} b{batch} t{t} d{d} h{heads} f{ffn}", flush=True)
    got = run_gpu(w, path)
    ref = oracle.encoder_block(w.x, w.layers[0], heads)
    check(errors(got, ref), path, f"random block b{batch} t{t} d{d} h{heads} f{ffn}")


@pytest.mark.parametrize("batch,t,d,heads,ffn", [c[1:] for c in _block_cases(count=6, seed=2027)])
def test_block_mxfp8_random(batch, t, d, heads, ffn):
    """The MXFP8 path at random block shapes, against the MXFP8 oracle (the block's bar on one
    block) and against the exact oracle (within the margins of the method's own error)."""
    from speech_transformer_encoder_amd import synth
    from speech_transformer_encoder_amd.encoder import build_from_workload, to_device_input
    from tests.test_gpu_mx import _check_mx
    cfg = synth.CONFIGS["tiny_block"].with_(seed=211 + t, batch=batch, t=t, d_model=d,
                                            heads=heads, ffn_dim=ffn)
    w = synth.make_workload(cfg)
    print(f"[case] random mxfp8 block b{batch} t{t} d{d} h{heads} f{ffn}", flush=True)
    enc = build_from_workload(w, B.WENC_PATH_MXFP8)
    got = host(enc.forward(to_device_input(w.x), final_norm=False))
    _check_mx(got, w, f"random block b{batch} t{t} d{d} h{heads} f{ffn}", ln_post=False,
              single_block=True)


def _ragged_cases(count=6, seed=2028):
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        heads = int(r.integers(1, 11))
        n = int(r.integers(1, 9))
        lens = [int(v) for v in r.integers(0, 900, n)]
        lens[int(r.integers(0, n))] = int(r.integers(0, 3))  # an empty or one- / two-row window
        if sum(lens) == 0 or sum(v * v for v in lens) * heads > 4e6:
            continue
        cases.append((PATHS[len(cases) % 3], heads, tuple(lens)))
    return cases


@pytest.mark.parametrize("path,heads,lens", _ragged_cases())
def test_stack_varlen_random(path, heads, lens):
    """Two blocks and the final norm over a ragged batch of random window lengths (empty and
    one-row windows included), every element against the oracle's per-window stack."""
    from speech_transformer_encoder_amd import synth
    from speech_transformer_encoder_amd.encoder import build_from_workload, to_device_input
    from tests.test_gpu_varlen import _check_block
    d = 64 * heads
    cfg = synth.CONFIGS["base_stack"].with_(seed=307 + sum(lens), batch=1, t=int(sum(lens)),
                                            d_model=d, heads=heads, ffn_dim=4 * d)
    w = synth.make_workload(cfg, n_layers=2)
    x = w.x[0]
    enc = build_from_workload(w, path)
    print(f"[case] random varlen path={path} heads={heads} lens={list(lens)}", flush=True)
    got = host(enc.forward_varlen(to_device_input(x), list(lens)))
    ref = oracle.encoder_stack_varlen(x, list(lens), w.layers, heads, w.ln_post)
    _check_block(errors(got, ref), path, f"random varlen h{heads} lens={list(lens)}")


def _mx_cases(count=12, seed=2030):
    r = np.random.default_rng(seed)
    cases = []
    epis = [B.WENC_EPI_BIAS, B.WENC_EPI_BIAS_RESIDUAL, B.WENC_EPI_BIAS_GELU]
    while len(cases) < count:
        persistent = len(cases) % 3 == 2
        m = int(r.integers(3000, 24001)) if persistent else int(r.integers(1, 4001))
        n = 64 * int(r.integers(8 if persistent else 1, 81))
        k = 64 * int(r.integers(1, 5 if persistent else 41))
        if m * n * k > (5e9 if persistent else 1.2e9):
            continue
        if persistent and -(-m // 256) * -(-n // 256) < 256:
            continue
        cases.append((epis[int(r.integers(0, 3))], m, n, k))
    return cases


@pytest.mark.parametrize("epi,m,n,k", _mx_cases())
def test_linear_mx_random(epi, m, n, k):
    """The MXFP8 product at random shapes (k tiles of 64 and 128 values, the small kernel, the
    persistent kernel and its tail), with the fixed-shape test's bounds."""
    from tests.test_gpu_mx import linear_mx_case
    linear_mx_case(m, n, k, epi)
