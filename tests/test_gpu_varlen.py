"""Ragged batches on the GPU (windows of different lengths packed back to back, described by
device offsets cu_seqlens), against the CPU oracle, through the C ABI.

Each window must come out exactly as if it had been encoded alone: attention per window, the
row-wise steps over all rows.  References: the oracle per window (``attention_online``,
``encoder_stack_varlen``, ``encoder_block_rows``), and, bit for bit, the dense entry points when all
windows have one length.  Tolerances are the block's (fp32 max_rel 1e-4; 16-bit max_rel 2e-2 and
MAE 1e-3; literal bf16 as in the dense block tests: above 1e-3 an expected failure, above 4e-3 a
failure) and, for attention, the componentwise bound of the dense attention test.
"""

import numpy as np
import pytest

import oracle
from speech_transformer_encoder_amd import binding as B
from speech_transformer_encoder_amd import synth
from speech_transformer_encoder_amd.encoder import build_from_workload, to_device_input
from tests.gpu_util import PATH_NAMES, as_operand, errors, host, report, require_gpu, torch_dtype

pytestmark = pytest.mark.gpu

PATHS = [B.WENC_PATH_BF16, B.WENC_PATH_FP16, B.WENC_PATH_FP32]
ATTN_CW = {B.WENC_PATH_BF16: 2.0 ** -7, B.WENC_PATH_FP16: 2.0 ** -10, B.WENC_PATH_FP32: 2e-5}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _cu(lens):
    import torch
    return torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")


def _check_block(e, path, tag):
    """The dense block tests' bar.  Literal bf16 operands miss MAE <= 1e-3 beyond the tiny
    workload (rounding LayerNorm and GELU outputs to bf16 costs ~1e-3 per block at these
    magnitudes): that is reported as an expected failure, and only a regression past 4e-3 fails."""
    report(f"{tag} [{PATH_NAMES[path]}]", e)
    assert e["finite"], tag
    if path == B.WENC_PATH_FP32:
        assert e["max_rel"] <= 1e-4, (tag, e)
    else:
        mae = 4e-3 if path == B.WENC_PATH_BF16 else 1e-3
        assert e["max_rel"] <= 2e-2 and e["mae"] <= mae, (tag, e)
        if e["mae"] > 1e-3:
            pytest.xfail(f"{tag}: literal bf16 operands miss MAE <= 1e-3 (measured {e['mae']:.2e})")


def _attention_varlen(path, lens, heads, seed, cu=None, max_t=None):
    import torch
    total = int(sum(lens))
    q, k, v = synth.random_qkv(seed, 1, total, heads)
    d = heads * 64
    qd, qh = as_operand(q[0], path)
    kd, kh = as_operand(k[0], path)
    vd, vh = as_operand(v[0], path)
    qkv = torch.cat([qd, kd, vd], dim=1).contiguous()
    es = qkv.element_size()
    o = torch.full((total, d), float("nan"), dtype=torch_dtype(path), device="cuda")
    if cu is None:
        cu = _cu(lens)
    batch = cu.numel() - 1
    max_t = max(lens) if max_t is None else max_t
    print(f"[case] attention varlen path={path} cu={cu.tolist()} heads={heads}", flush=True)
    p = qkv.data_ptr()
    B.whisper_enc_attention_varlen(p, p + d * es, p + 2 * d * es, o, cu, batch, total, max_t,
                                   heads, 3 * d, d, path)
    return host(o), qh, kh, vh


@pytest.mark.parametrize("path", PATHS)
def test_attention_varlen(path):
    lens = [0, 1, 63, 64, 65, 255, 256, 257, 700, 1500, 0]
    heads = 2
    got, qh, kh, vh = _attention_varlen(path, lens, heads, seed=17)
    s = 0
    for n in lens:
        if n == 0:
            continue
        ref, pb = oracle.attention_online(qh[s:s + n], kh[s:s + n], vh[s:s + n], heads,
                                          return_probs=True)
        absv = np.abs(vh[s:s + n]).reshape(n, heads, 64).transpose(1, 0, 2)
        bound = np.einsum("hij,hjd->ihd", pb, absv).reshape(n, heads * 64)
        g = got[s:s + n]
        assert np.isfinite(g).all(), n
        cw = float(np.max(np.abs(g - ref) / bound))
        report(f"attn varlen p{path} len{n} cw={cw:.3e}", errors(g, ref))
        assert cw <= ATTN_CW[path], (n, cw)
        s += n


def test_attention_varlen_skips_invalid_windows():
    """Windows whose offsets break the rules are skipped (their rows keep what was there) and the
    valid windows are unaffected: a decreasing pair, a window longer than max_t and one that ends
    past total_rows."""
    import torch
    path = B.WENC_PATH_FP16
    heads, total, max_t = 1, 40, 16
    cu = torch.tensor([0, 10, 5, 40, 60], dtype=torch.int32, device="cuda")
    got, qh, kh, vh = _attention_varlen(path, [total], heads, seed=3, cu=cu, max_t=max_t)
    ref = oracle.attention_online(qh[:10], kh[:10], vh[:10], heads)
    assert errors(got[:10], ref)["max_rel"] <= 2e-3
    assert np.isnan(got[10:]).all()


def _ragged_workload(cfg, lens, n_layers):
    w = synth.make_workload(cfg.with_(batch=1, t=int(sum(lens))), n_layers=n_layers)
    return w, w.x[0]


@pytest.mark.parametrize("path", PATHS)
def test_stack_varlen(path):
    lens = [1500, 1, 700, 0, 257, 64, 1024]
    cfg = synth.CONFIGS["base_stack"]
    w, x = _ragged_workload(cfg, lens, n_layers=2)
    enc = build_from_workload(w, path)
    print(f"[case] stack varlen path={path} lens={lens}", flush=True)
    got = host(enc.forward_varlen(to_device_input(x), lens))
    ref = oracle.encoder_stack_varlen(x, lens, w.layers, cfg.heads, w.ln_post)
    _check_block(errors(got, ref), path, "stack varlen base x2")


@pytest.mark.parametrize("path", PATHS)
def test_stack_varlen_key_halves(path):
    """Four short windows (the longest 200 rows) x 8 heads = 64 blocks of 128 query rows: the
    keys of each block are split in two halves and merged, with windows of one key tile (the
    second half empty) and of one row."""
    lens = [50, 1, 64, 200]
    cfg = synth.CONFIGS["tiny_block"].with_(d_model=512, heads=8, ffn_dim=1024)
    w, x = _ragged_workload(cfg, lens, n_layers=1)
    enc = build_from_workload(w, path)
    print(f"[case] stack varlen key halves path={path} lens={lens}", flush=True)
    got = host(enc.forward_varlen(to_device_input(x), lens))
    ref = oracle.encoder_stack_varlen(x, lens, w.layers, cfg.heads, w.ln_post)
    _check_block(errors(got, ref), path, "stack varlen key halves")


@pytest.mark.parametrize("path", PATHS)
def test_varlen_equal_lengths_is_the_dense_call(path):
    """Equal window lengths: the ragged entry point reproduces the dense one bit for bit."""
    cfg = synth.CONFIGS["tiny_block"].with_(batch=3, t=333)
    w = synth.make_workload(cfg, n_layers=2)
    enc = build_from_workload(w, path)
    x = to_device_input(w.x)
    dense = host(enc.forward(x))
    rag = host(enc.forward_varlen(x.reshape(-1, cfg.d_model), [333] * 3))
    np.testing.assert_array_equal(rag.reshape(dense.shape), dense)


@pytest.mark.parametrize("path", [B.WENC_PATH_FP16, B.WENC_PATH_BF16])
def test_block_varlen_large_v3(path):
    """The large-v3 block over 16 windows of 150 .. 1500 rows (the ragged benchmark batch),
    sampled rows of every window against the oracle."""
    cfg = synth.CONFIGS["large_v3_batch16_block"]
    lens = synth.ragged_lengths(cfg.seed, cfg.batch)
    w, x = _ragged_workload(cfg, lens, n_layers=1)
    enc = build_from_workload(w, path)
    print(f"[case] block varlen large-v3 path={path} rows={int(sum(lens))}", flush=True)
    got = host(enc.forward_varlen(to_device_input(x), lens, final_norm=False))
    r = np.random.default_rng([8, 93])
    s = 0
    for n in lens:
        rows = np.unique(np.concatenate([[0, n - 1], r.choice(n, 6, replace=False)]))
        ref = oracle.encoder_block_rows(x[s:s + n], w.layers[0], cfg.heads, rows)
        _check_block(errors(got[s + rows], ref), path, f"block varlen large len{n}")
        s += n
