"""Block and stack parity on the GPU against the CPU oracle, through the C ABI.

Small shapes (several tiles and a ragged tail) are compared element by element.  The five full
workloads run in the launch configuration the benchmark times; their references are the full
oracle output (tiny block, base stack), stored sampled rows written by
``tests/golden/make_golden.py`` from the oracle (small and large-v3 stacks), or sampled rows of
every window recomputed by the oracle (batched large-v3 block).

Acceptance: fp32 path max relative error <= 1e-4; 16-bit paths max relative error <= 2e-2 and
mean absolute error <= 1e-3.  The max relative error is taken per element and floored at the
reference RMS (``oracle.max_rel_error``).

Paths that meet both 16-bit bounds: fp16 operands on every workload; BF16X3 (bf16 MFMA operands,
weights and the LayerNorm / GELU outputs carried as bf16 hi + lo pairs) on every workload; BF16X2
(only the activations split) on the workloads with bf16-valued weights (small, large-v3, batched),
where its weights are exact -- on the fp32-weight base stack the bf16 rounding of the weights
alone costs ~1e-3 (measured MAE 1.01e-3), which is what BF16X3 is for.  The literal bf16
path does NOT meet MAE <= 1e-3 on the base, small, large-v3 and batched workloads: rounding each
LayerNorm and GELU output to bf16 (2^-9 relative) before a projection leaves ~1e-3 of error per
block in the residual stream, growing with depth (measured 1.4e-3 after 6 blocks, 2.8e-3 after 32;
the fp32 weights of the tiny and base workloads lose 2^-9 more when stored as bf16).  Its tests
there assert the max relative bound, fail outright above BF16_MAE_CEILING (a regression of that
known miss), and otherwise report the MAE bar as an expected failure (xfail) with the measured
value; the 1e-3 bar itself is asserted on fp16, BF16X2 and BF16X3.
"""

import os

import numpy as np
import pytest

import oracle
from speech_transformer_encoder_amd import binding as B
from speech_transformer_encoder_amd import synth
from speech_transformer_encoder_amd.encoder import build_from_workload, to_device_input
from tests.gpu_util import PATH_NAMES, errors, host, report, require_gpu

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
PATHS = [B.WENC_PATH_BF16, B.WENC_PATH_FP16, B.WENC_PATH_FP32, B.WENC_PATH_BF16X2,
         B.WENC_PATH_BF16X3]
# BF16X2 is the path for bf16-valued weights: its full-workload checks run where they are.
FULL_CASES = [(name, path) for name in synth.CONFIGS for path in PATHS
              if not (path == B.WENC_PATH_BF16X2 and not synth.CONFIGS[name].bf16_weights)]
BF16_MAE_CEILING = 4e-3  # regression guard on literal bf16's measured MAE miss (not the bar)


def tolerance(path, name=None):
    if path == B.WENC_PATH_FP32:
        return {"max_rel": 1e-4, "mae": None}
    if path == B.WENC_PATH_BF16 and name not in (None, "tiny_block"):
        return {"max_rel": 2e-2, "mae": BF16_MAE_CEILING}
    return {"max_rel": 2e-2, "mae": 1e-3}


def check(e, path, tag, name=None):
    report(f"{tag} [{PATH_NAMES[path]}]", e)
    tol = tolerance(path, name)
    assert e["finite"], tag
    assert e["max_rel"] <= tol["max_rel"], (tag, e)
    if tol["mae"] is not None:
        assert e["mae"] <= tol["mae"], (tag, e)
    if path == B.WENC_PATH_BF16 and e["mae"] > 1e-3:
        # The bar is MAE <= 1e-3; literal bf16 operands miss it here (reported as an expected
        # failure, not passed under a wider bound; the ceiling above only catches a regression).
        pytest.xfail(f"{tag}: literal bf16 operands miss MAE <= 1e-3 (measured {e['mae']:.2e}); "
                     "fp16, BF16X2 and BF16X3 meet it")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_gpu(w, path, n_layers=None, final_norm=True, in_place=False):
    enc = build_from_workload(w, path)
    x = to_device_input(w.x)
    y = enc.forward(x, x if in_place else None, n_layers=n_layers, final_norm=final_norm)
    return host(y)


# ------------------------------------------------------------------ small shapes, every element


@pytest.mark.parametrize("path", PATHS)
def test_block_small_ragged(path):
    cfg = synth.CONFIGS["tiny_block"].with_(batch=2, t=200)
    w = synth.make_workload(cfg)
    print(f"[case] block small path={path}", flush=True)
    got = run_gpu(w, path)
    ref = oracle.encoder_block(w.x, w.layers[0], cfg.heads)
    check(errors(got, ref), path, "tiny block b2 t200")


@pytest.mark.parametrize("path", PATHS)
def test_stack_prefixes_and_final_norm(path):
    """Bisection: the first k blocks of a stack, with and without the final LayerNorm."""
    cfg = synth.CONFIGS["base_stack"].with_(t=130, n_layers=3)
    w = synth.make_workload(cfg)
    enc = build_from_workload(w, path)
    x = to_device_input(w.x)
    h = np.asarray(w.x, np.float64)
    for k in range(0, 4):
        if k > 0:
            h = oracle.encoder_block(h, w.layers[k - 1], cfg.heads)
        print(f"[case] stack prefix k={k} path={path}", flush=True)
        got = host(enc.forward(x, n_layers=k, final_norm=False))
        check(errors(got, h), path, f"base stack prefix {k}", name="base_stack")
        got = host(enc.forward(x, n_layers=k))
        check(errors(got, oracle.layer_norm(h, *w.ln_post)), path, f"base stack prefix {k} + ln",
              name="base_stack")


@pytest.mark.parametrize("path", PATHS)
def test_block_attention_key_halves(path):
    """8 heads of one 1100-position window give 72 query blocks of 128 rows: too few to fill
    the GPU, so on the 16-bit paths each block's keys are split over two workgroups (9 key tiles
    each) and, inside each, over its two wavefront groups (5 and 4 tiles, the last one ragged),
    and the four partial results merged; every element against the oracle."""
    cfg = synth.CONFIGS["tiny_block"].with_(t=1100, d_model=512, heads=8, ffn_dim=1024)
    w = synth.make_workload(cfg)
    print(f"[case] block key halves path={path}", flush=True)
    got = run_gpu(w, path)
    ref = oracle.encoder_block(w.x, w.layers[0], cfg.heads)
    check(errors(got, ref), path, "block d512 h8 t1100")


def test_block_key_halves_large_logits():
    """The key-split configuration of the last test (72 query blocks, each block's keys split
    over two workgroups and two wavefront groups in each, then merged) with Wq scaled by 100:
    logits then spread over about +-100 (standard deviation 20), so the running max is raised in
    the middle of the key loop of most rows, in every part, and the merges combine parts whose
    maxima differ widely.
    fp16 operands: rounding q, k and the probabilities to fp16 moves the block output by an MAE of
    3.4e-4 and a max relative error of 4.5e-3 at these logits (float64 emulation of those
    roundings), inside the block's bar; a wrong rescale would move it by the size of v.  (With
    bf16 operands the rounding of q alone moves logits of 100 by ~0.2, beyond the bar; the
    step-level outlier tests cover bf16 with a componentwise bound.)"""
    cfg = synth.CONFIGS["tiny_block"].with_(t=1100, d_model=512, heads=8, ffn_dim=1024)
    w = synth.make_workload(cfg)
    w.layers[0]["wq"] = (w.layers[0]["wq"] * 100.0).astype(np.float32)
    print("[case] block key halves, logits +-100, fp16", flush=True)
    got = run_gpu(w, B.WENC_PATH_FP16)
    ref = oracle.encoder_block(w.x, w.layers[0], cfg.heads)
    check(errors(got, ref), B.WENC_PATH_FP16, "block d512 h8 t1100 Wq x100")


def test_in_place_and_determinism():
    cfg = synth.CONFIGS["tiny_block"].with_(batch=3, t=150)
    w = synth.make_workload(cfg)
    a = run_gpu(w, B.WENC_PATH_BF16)
    b = run_gpu(w, B.WENC_PATH_BF16, in_place=True)
    c = run_gpu(w, B.WENC_PATH_BF16)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


def test_windows_are_independent():
    """At this shape a window's output is bit-identical whether it runs alone or inside a batch
    of four: 300 and 1200 rows get the same split-k plans (fc2 in 4 parts on 128-row tiles, the
    out-projection unsplit), and attention takes the same form for both (two wavefront groups
    per workgroup over the key halves, the keys split again over two workgroups), so each query
    row's sums run in the same order.  Where the plans differ, results differ in the last bits
    (test_window_alone_vs_batched_large_v3)."""
    cfg = synth.CONFIGS["tiny_block"].with_(batch=4, t=300)
    w = synth.make_workload(cfg)
    enc = build_from_workload(w, B.WENC_PATH_BF16)
    full = host(enc.forward(to_device_input(w.x)))
    alone = host(enc.forward(to_device_input(w.x[2:3])))
    np.testing.assert_array_equal(full[2:3], alone)


def test_window_alone_vs_batched_large_v3():
    """One large-v3 window alone runs its out-projection and fc2 as split-k products (2 and 4
    fp32 parts added in order, LN2 fused into the reduction), while inside the batch of 16 the
    same GEMMs run unsplit on the persistent kernel: the fp32 sums are formed in another order, so
    the two outputs may differ in the last bits.  Both must meet the block's bar against the
    oracle on sampled rows (the batch's other 15 windows do not matter)."""
    cfg = synth.CONFIGS["large_v3_batch16_block"]
    w = synth.make_workload(cfg)
    enc = build_from_workload(w, B.WENC_PATH_FP16)
    print("[case] large-v3 window 3 alone vs in the batch of 16", flush=True)
    batched = host(enc.forward(to_device_input(w.x)))[3]
    alone = host(enc.forward(to_device_input(w.x[3:4])))[0]
    big = np.where(np.abs(w.x[3]).max(axis=1) > 10)[0][:2]
    rows = np.unique(np.concatenate([[0, 1, 700, cfg.t - 1], big]))
    ref = oracle.encoder_block_rows(w.x[3], w.layers[0], cfg.heads, rows)
    check(errors(alone[rows], ref), B.WENC_PATH_FP16, "large-v3 window alone")
    check(errors(batched[rows], ref), B.WENC_PATH_FP16, "large-v3 window in the batch")
    report("large-v3 window alone vs batched (mutual)", errors(alone, batched))


@pytest.mark.parametrize("path", [B.WENC_PATH_BF16, B.WENC_PATH_FP16, B.WENC_PATH_Q8,
                                  B.WENC_PATH_BF16X2, B.WENC_PATH_BF16X3])
def test_stack_equals_chained_blocks(path):
    """A stack call is bit-identical to one block call per layer followed by the final LayerNorm.

    At one 1500-position window the residual GEMMs split k, and the stack call folds each
    following LayerNorm (the next block's LN1, then the final norm) into fc2's reduction pass;
    the chained calls run those norms as separate LayerNorm launches.  Both must round alike."""
    import torch
    cfg = synth.CONFIGS["base_stack"].with_(n_layers=3)
    w = synth.make_workload(cfg)
    enc = build_from_workload(w, path)
    x = to_device_input(w.x)
    print(f"[case] stack vs chained blocks path={path}", flush=True)
    stacked = host(enc.forward(x))
    batch, t, d = x.shape
    ws = enc.workspace(batch, t)
    cur, nxt = x.clone(), torch.empty_like(x)
    for l in range(cfg.n_layers):
        B.whisper_enc_block_forward(cur, nxt, enc.blob.data_ptr() + l * enc.layer_bytes, batch, t,
                                    d, cfg.heads, cfg.ffn_dim, path, ws, ws.numel())
        cur, nxt = nxt, cur
    g, b = enc.ln_post
    B.whisper_enc_layernorm(cur, g, b, nxt, batch * t, d, B.WENC_DTYPE_F32)
    np.testing.assert_array_equal(stacked, host(nxt))


@pytest.mark.parametrize("path", [B.WENC_PATH_BF16, B.WENC_PATH_FP16])
def test_pack_rounds_to_nearest_even(path):
    """Packing fp32 weights rounds them exactly as PyTorch's RNE conversion does: the block on
    fp32 weights equals, bit for bit, the block on weights pre-rounded to the operand type."""
    import torch
    from tests.gpu_util import torch_dtype
    cfg = synth.CONFIGS["tiny_block"].with_(t=128)
    w = synth.make_workload(cfg)
    a = run_gpu(w, path)
    for n in ("wq", "wk", "wv", "wo", "w1", "w2"):
        t = torch.from_numpy(w.layers[0][n]).to(torch_dtype(path)).to(torch.float32)
        w.layers[0][n] = t.numpy()
    b = run_gpu(w, path)
    np.testing.assert_array_equal(a, b)


def test_zero_weights_closed_form():
    cfg = synth.CONFIGS["tiny_block"].with_(t=100)
    w = synth.make_workload(cfg)
    p = w.layers[0]
    for n in ("wq", "wk", "wv", "wo", "w1", "w2"):
        p[n] = np.zeros_like(p[n])
    for path in PATHS:
        got = run_gpu(w, path)
        np.testing.assert_allclose(got, w.x + p["bo"] + p["b2"], rtol=0, atol=1e-6)


# ------------------------------------------------------------------ the five full workloads


def _sampled_block_rows(w, per_window=8):
    """Sampled rows of every window (outlier rows included) and the oracle's values there."""
    cfg = w.cfg
    refs, idx = [], []
    for b in range(cfg.batch):
        big = np.where(np.abs(w.x[b]).max(axis=1) > 10)[0][:2]
        rng = np.random.default_rng([cfg.seed, 7000, b])
        rows = np.unique(np.concatenate([[0, cfg.t - 1], big,
                                         rng.choice(cfg.t, per_window - 2 - len(big), replace=False)]))
        refs.append(oracle.encoder_block_rows(w.x[b], w.layers[0], cfg.heads, rows))
        idx.append((b, rows))
    return idx, np.concatenate(refs)


@pytest.mark.parametrize("name,path", FULL_CASES)
def test_full_config(name, path):
    cfg = synth.CONFIGS[name]
    w = synth.make_workload(cfg)
    print(f"[case] full config {name} path={PATH_NAMES[path]}", flush=True)
    got = run_gpu(w, path)
    if name in ("small_stack", "large_v3_stack"):
        g = np.load(os.path.join(GOLDEN, f"{name}_rows.npz"))
        e = errors(got[0][g["rows"]], g["y"])
        # Diagnostic only (parity is graded on the stack output): the residual stream before the
        # final LayerNorm, whose absolute scale grows with depth.
        pre = run_gpu(w, path, final_norm=False)
        report(f"{name} before the final norm, diagnostic [{PATH_NAMES[path]}]",
               errors(pre[0][g["rows"]], g["pre_rows"]))
    elif cfg.batch > 1:
        idx, ref = _sampled_block_rows(w)
        e = errors(np.concatenate([got[b][rows] for b, rows in idx]), ref)
    else:
        ref = oracle.encoder_stack(w.x, w.layers, cfg.heads, w.ln_post)
        e = errors(got, ref)
    check(e, path, name, name=name)
