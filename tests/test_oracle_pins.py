"""Pins for the CPU oracle: each check ties it to something other than itself.

Independent library implementations (PyTorch's float64 CPU LayerNorm, GELU and scaled-dot-product
attention, and the Hugging Face ``WhisperEncoderLayer``), closed forms, invariants and brute force
on tiny inputs.  The mutation tests at the end plant plausible mistakes into the oracle and show
that the pins catch them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import oracle as orc
from speech_transformer_encoder_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rng(seed):
    return np.random.default_rng([seed, 4242])


def _rand_layer(seed, d, f, affine=True):
    r = _rng(seed)
    p = {
        "wq": r.standard_normal((d, d)) * 0.08, "bq": r.standard_normal(d) * 0.1,
        "wk": r.standard_normal((d, d)) * 0.08, "bk": None,
        "wv": r.standard_normal((d, d)) * 0.08, "bv": r.standard_normal(d) * 0.1,
        "wo": r.standard_normal((d, d)) * 0.08, "bo": r.standard_normal(d) * 0.1,
        "w1": r.standard_normal((f, d)) * 0.08, "b1": r.standard_normal(f) * 0.1,
        "w2": r.standard_normal((d, f)) * 0.08, "b2": r.standard_normal(d) * 0.1,
        "ln1_g": 1 + r.standard_normal(d) * 0.2 if affine else np.ones(d),
        "ln1_b": r.standard_normal(d) * 0.2 if affine else np.zeros(d),
        "ln2_g": 1 + r.standard_normal(d) * 0.2 if affine else np.ones(d),
        "ln2_b": r.standard_normal(d) * 0.2 if affine else np.zeros(d),
    }
    return p


def _hf_layer(p, d, heads, f):
    from transformers import WhisperConfig
    from transformers.models.whisper.modeling_whisper import WhisperEncoderLayer
    cfg = WhisperConfig(d_model=d, encoder_attention_heads=heads, encoder_ffn_dim=f,
                        activation_function="gelu", dropout=0.0, attention_dropout=0.0,
                        activation_dropout=0.0)
    cfg._attn_implementation = "eager"
    layer = WhisperEncoderLayer(cfg).double().eval()
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    sa = layer.self_attn
    with torch.no_grad():
        sa.q_proj.weight.copy_(t(p["wq"])); sa.q_proj.bias.copy_(t(p["bq"]))
        sa.k_proj.weight.copy_(t(p["wk"]))
        sa.v_proj.weight.copy_(t(p["wv"])); sa.v_proj.bias.copy_(t(p["bv"]))
        sa.out_proj.weight.copy_(t(p["wo"])); sa.out_proj.bias.copy_(t(p["bo"]))
        layer.self_attn_layer_norm.weight.copy_(t(p["ln1_g"]))
        layer.self_attn_layer_norm.bias.copy_(t(p["ln1_b"]))
        layer.final_layer_norm.weight.copy_(t(p["ln2_g"]))
        layer.final_layer_norm.bias.copy_(t(p["ln2_b"]))
        layer.fc1.weight.copy_(t(p["w1"])); layer.fc1.bias.copy_(t(p["b1"]))
        layer.fc2.weight.copy_(t(p["w2"])); layer.fc2.bias.copy_(t(p["b2"]))
    return layer


def _hf_block(p, x, heads):
    d = x.shape[-1]
    f = p["w1"].shape[0]
    layer = _hf_layer(p, d, heads, f)
    xt = torch.tensor(np.asarray(x, np.float64))
    if xt.ndim == 2:
        xt = xt[None]
    with torch.no_grad():
        y = layer(xt, attention_mask=None)
    if isinstance(y, tuple):
        y = y[0]
    return y.numpy().reshape(np.shape(x))


def _sdpa(q, k, v, heads):
    t, d = q.shape
    hd = d // heads
    f = lambda a: torch.tensor(a).reshape(-1, heads, hd).transpose(0, 1)[None]
    o = torch.nn.functional.scaled_dot_product_attention(f(q), f(k), f(v))
    return o[0].transpose(0, 1).reshape(-1, d).numpy()


# ---------------------------------------------------------------- attention


@pytest.mark.parametrize("t,heads,hd", [(300, 2, 64), (129, 3, 32), (1500, 1, 64), (1, 2, 64)])
def test_attention_matches_torch_sdpa(t, heads, hd):
    r = _rng(t)
    q, k, v = (r.standard_normal((t, heads * hd)) for _ in range(3))
    got = oracle.attention_online(q, k, v, heads)
    np.testing.assert_allclose(got, _sdpa(q, k, v, heads), rtol=0, atol=1e-12)


def test_attention_brute_force_loops():
    """Pure-Python definition on a tiny case: softmax over all keys, weighted sum of V."""
    r = _rng(7)
    t, heads, hd = 5, 2, 4
    q, k, v = (r.standard_normal((t, heads * hd)) for _ in range(3))
    ref = np.zeros((t, heads * hd))
    for h in range(heads):
        c = slice(h * hd, (h + 1) * hd)
        for i in range(t):
            s = [sum(q[i, c][u] * k[j, c][u] for u in range(hd)) / math.sqrt(hd) for j in range(t)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            for u in range(hd):
                ref[i, h * hd + u] = sum(e[j] * v[j, c][u] for j in range(t)) / z
    np.testing.assert_allclose(oracle.attention_online(q, k, v, heads, tile=2), ref, atol=1e-14)


@pytest.mark.parametrize("tile", [1, 7, 64, 128, 2000])
def test_online_two_pass_split_kv_agree(tile):
    r = _rng(11)
    t, heads = 1500, 2
    q, k, v = (r.standard_normal((t, heads * 64)) for _ in range(3))
    q[r.choice(t, 75, replace=False)] *= 20.0  # logit spreads of ~100: corr underflows to 0
    a = oracle.attention_online(q, k, v, heads, tile=tile)
    b = oracle.attention_two_pass(q, k, v, heads)
    c = oracle.attention_split_kv(q, k, v, heads, chunks=5)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)
    np.testing.assert_allclose(c, b, atol=1e-12, rtol=0)


def test_attention_single_key_returns_v():
    r = _rng(3)
    q, k, v = (r.standard_normal((1, 128)) for _ in range(3))
    np.testing.assert_array_equal(oracle.attention_online(q, k, v, 2), v)


def test_attention_identical_keys_give_mean_of_v():
    r = _rng(4)
    t, heads = 257, 2
    q, v = r.standard_normal((t, 128)), r.standard_normal((t, 128))
    k = np.tile(r.standard_normal((1, 128)), (t, 1))
    got = oracle.attention_online(q, k, v, heads)
    np.testing.assert_allclose(got, np.tile(v.mean(axis=0), (t, 1)), atol=1e-13)


def test_attention_probabilities_sum_to_one_and_k_bias_invariance():
    r = _rng(5)
    t, heads = 300, 2
    q, k, v = (r.standard_normal((t, 128)) for _ in range(3))
    o, p = oracle.attention_online(q, k, v, heads, return_probs=True)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-13)
    assert (p >= 0).all()
    # each output row is the probability-weighted mean of V
    np.testing.assert_allclose(o[:, :64], p[0] @ v[:, :64], atol=1e-12)
    # a K bias adds q_i.b to every score of row i: the softmax does not move
    kb = k + r.standard_normal(128)
    np.testing.assert_allclose(oracle.attention_online(q, kb, v, heads), o, atol=1e-12)


def test_attention_query_subset_matches_full():
    r = _rng(6)
    t, heads = 300, 2
    q, k, v = (r.standard_normal((t, 128)) for _ in range(3))
    rows = [0, 5, 128, 299]
    full = oracle.attention_online(q, k, v, heads)
    np.testing.assert_allclose(oracle.attention_online(q[rows], k, v, heads), full[rows], atol=1e-14)


# ---------------------------------------------------------------- LayerNorm and GELU


def test_layer_norm_matches_torch_and_invariants():
    r = _rng(8)
    x = r.standard_normal((50, 384)) * 3 + 1.5
    g, b = r.standard_normal(384), r.standard_normal(384)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (384,), torch.tensor(g), torch.tensor(b),
                                         eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.layer_norm(x, g, b), ref, atol=1e-12)
    y = oracle.layer_norm(x, np.ones(384), np.zeros(384))
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    # a constant row maps to beta
    np.testing.assert_allclose(oracle.layer_norm(np.full((2, 384), 7.0), g, b), np.tile(b, (2, 1)),
                               atol=1e-12)
    # scale and shift invariance up to the eps term
    y2 = oracle.layer_norm(20.0 * x - 3.0, np.ones(384), np.zeros(384))
    np.testing.assert_allclose(y2, y, atol=1e-5)


def test_gelu_erf_values_and_identities():
    z = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.tensor(z), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu_erf(z), ref, atol=1e-15)
    assert oracle.gelu_erf(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.gelu_erf(z) - oracle.gelu_erf(-z), z, atol=1e-14)
    # Phi(1) and Phi(-1) of the standard normal distribution
    np.testing.assert_allclose(oracle.gelu_erf(np.array([1.0, -1.0, 2.0])),
                               [0.8413447460685429, -0.15865525393145707, 2 * 0.9772498680518208],
                               rtol=1e-15)
    from scipy.special import erfc
    np.testing.assert_allclose(oracle.gelu_erf(z), 0.5 * z * erfc(-z / math.sqrt(2)), atol=1e-15)


def test_linear_loops():
    r = _rng(9)
    a, w, b = r.standard_normal((3, 5)), r.standard_normal((4, 5)), r.standard_normal(4)
    ref = [[sum(a[i, k] * w[n, k] for k in range(5)) + b[n] for n in range(4)] for i in range(3)]
    np.testing.assert_allclose(oracle.linear(a, w, b), ref, atol=1e-14)


# ---------------------------------------------------------------- block and stack


@pytest.mark.parametrize("t,d,heads,f,batch", [(150, 128, 2, 512, 1), (70, 192, 3, 256, 2)])
def test_block_matches_hf_whisper_encoder_layer(t, d, heads, f, batch):
    p = _rand_layer(t + d, d, f)
    x = _rng(t).standard_normal((batch, t, d)) * 2
    got = oracle.encoder_block(x, p, heads)
    np.testing.assert_allclose(got, _hf_block(p, x, heads), atol=1e-11, rtol=0)


def test_block_with_synth_layer_matches_hf():
    cfg = synth.CONFIGS["tiny_block"].with_(t=200)
    w = synth.make_workload(cfg)
    got = oracle.encoder_block(w.x, w.layers[0], cfg.heads)
    np.testing.assert_allclose(got, _hf_block(w.layers[0], w.x, cfg.heads), atol=1e-11)


def test_block_zero_weights_closed_form():
    d, f = 64, 128
    p = _rand_layer(1, d, f)
    for n in ("wq", "wk", "wv", "wo", "w1", "w2"):
        p[n] = np.zeros_like(p[n])
    x = _rng(2).standard_normal((33, d))
    np.testing.assert_allclose(oracle.encoder_block(x, p, 1), x + p["bo"] + p["b2"], atol=1e-14)


def test_block_zero_qk_gives_mean_of_values():
    d, f, t = 128, 256, 97
    p = _rand_layer(3, d, f)
    p["wq"][:] = 0
    p["wk"][:] = 0
    p["bq"][:] = 0
    x = _rng(3).standard_normal((t, d))
    a = oracle.layer_norm(x, p["ln1_g"], p["ln1_b"])
    v = oracle.linear(a, p["wv"], p["bv"])
    o = np.tile(v.mean(axis=0), (t, 1))
    x1 = x + oracle.linear(o, p["wo"], p["bo"])
    a2 = oracle.layer_norm(x1, p["ln2_g"], p["ln2_b"])
    ref = x1 + oracle.linear(oracle.gelu_erf(oracle.linear(a2, p["w1"], p["b1"])), p["w2"], p["b2"])
    np.testing.assert_allclose(oracle.encoder_block(x, p, 2), ref, atol=1e-12)


def test_block_row_permutation_and_window_independence():
    d, f, t = 128, 256, 90
    p = _rand_layer(4, d, f)
    r = _rng(4)
    x = r.standard_normal((3, t, d))
    y = oracle.encoder_block(x, p, 2)
    perm = r.permutation(t)
    np.testing.assert_allclose(oracle.encoder_block(x[:, perm], p, 2), y[:, perm], atol=1e-12)
    x2 = x.copy()
    x2[1] = r.standard_normal((t, d))
    y2 = oracle.encoder_block(x2, p, 2)
    np.testing.assert_array_equal(y2[0], y[0])
    np.testing.assert_array_equal(y2[2], y[2])
    wperm = [2, 0, 1]
    np.testing.assert_allclose(oracle.encoder_block(x[wperm], p, 2), y[wperm], atol=1e-13)


def test_block_rows_matches_block():
    cfg = synth.CONFIGS["tiny_block"].with_(t=260)
    w = synth.make_workload(cfg)
    full = oracle.encoder_block(w.x[0], w.layers[0], cfg.heads)
    rows = [0, 1, 127, 128, 259]
    np.testing.assert_allclose(oracle.encoder_block_rows(w.x[0], w.layers[0], cfg.heads, rows),
                               full[rows], atol=1e-13)


def test_stack_matches_hf_layers_and_final_norm():
    d, f, t, heads = 128, 256, 64, 2
    layers = [_rand_layer(10 + i, d, f) for i in range(3)]
    g, b = 1 + _rng(5).standard_normal(d) * 0.1, _rng(6).standard_normal(d) * 0.1
    x = _rng(7).standard_normal((t, d))
    got = oracle.encoder_stack(x, layers, heads, ln_post=(g, b))
    h = x
    for p in layers:
        h = _hf_block(p, h, heads)
    ref = torch.nn.functional.layer_norm(torch.tensor(h), (d,), torch.tensor(g), torch.tensor(b),
                                         eps=1e-5).numpy()
    np.testing.assert_allclose(got, ref, atol=1e-11)
    # no final norm: the last block's output is the stack output
    np.testing.assert_allclose(oracle.encoder_stack(x, layers, heads), h, atol=1e-11)


def test_stack_varlen_matches_hf_padded_batch_with_key_mask():
    """A ragged batch equals the Hugging Face layers run on the zero-padded batch with an additive
    key mask (padded keys get -inf before the softmax), on the rows that hold real frames."""
    d, f, heads = 128, 256, 2
    lens = [37, 1, 64, 0, 90]
    tmax = max(lens)
    layers = [_rand_layer(40 + i, d, f) for i in range(2)]
    g, b = 1 + _rng(41).standard_normal(d) * 0.1, _rng(42).standard_normal(d) * 0.1
    x = _rng(43).standard_normal((sum(lens), d))
    got = oracle.encoder_stack_varlen(x, lens, layers, heads, ln_post=(g, b))
    assert got.shape == x.shape
    pad = np.zeros((len(lens), tmax, d))
    mask = np.full((len(lens), 1, tmax, tmax), -np.inf)
    s = 0
    for i, n in enumerate(lens):
        pad[i, :n] = x[s:s + n]
        mask[i, :, :, :n] = 0.0
        s += n
    mask[np.isinf(mask).all(axis=-1)] = 0.0  # an empty window's rows: any finite mask
    h = torch.tensor(pad)
    with torch.no_grad():
        for p in layers:
            layer = _hf_layer(p, d, heads, f)
            h = layer(h, attention_mask=torch.tensor(mask))
            h = h[0] if isinstance(h, tuple) else h
    ref = torch.nn.functional.layer_norm(h, (d,), torch.tensor(g), torch.tensor(b), eps=1e-5).numpy()
    s = 0
    for i, n in enumerate(lens):
        np.testing.assert_allclose(got[s:s + n], ref[i, :n], atol=1e-11)
        s += n


def test_stack_varlen_rejects_bad_lengths_and_keeps_windows_apart():
    d, f, heads = 64, 128, 1
    layers = [_rand_layer(50, d, f)]
    x = _rng(51).standard_normal((10, d))
    with pytest.raises(ValueError):
        oracle.encoder_stack_varlen(x, [4, 5], layers, heads)
    a = oracle.encoder_stack_varlen(x, [4, 6], layers, heads)
    # changing the second window leaves the first one's output unchanged
    x2 = x.copy()
    x2[4:] += 3.0
    b = oracle.encoder_stack_varlen(x2, [4, 6], layers, heads)
    np.testing.assert_array_equal(a[:4], b[:4])
    assert np.abs(a[4:] - b[4:]).max() > 1e-3


# ---------------------------------------------------------------- metrics


def test_error_metrics():
    ref = np.array([1.0, -2.0, 0.0, 4.0])
    got = ref + np.array([0.01, 0.0, 0.05, -0.04])
    rms = math.sqrt(np.mean(ref ** 2))
    assert orc.max_rel_error(got, ref) == pytest.approx(max(0.01 / rms, 0.05 / rms, 0.04 / 4.0))
    assert orc.mean_abs_error(got, ref) == pytest.approx(0.025)


# ---------------------------------------------------------------- mutations: the pins bite


def _hf_check(monkeypatch_fn=None):
    p = _rand_layer(99, 128, 256)
    x = _rng(99).standard_normal((140, 128))
    return np.abs(oracle.encoder_block(x, p, 2) - _hf_block(p, x, 2)).max()


@pytest.mark.parametrize("mutation", ["transposed_weight", "no_corr", "scale_sqrt_d", "ln_unbiased",
                                      "gelu_tanh", "no_bias_v", "drop_residual"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    if mutation == "transposed_weight":
        monkeypatch.setattr(orc, "linear", lambda a, w, b=None: orc._f64(a) @ orc._f64(w)
                            + (0 if b is None else orc._f64(b)) if w.shape[0] == w.shape[1]
                            else orc._f64(a) @ orc._f64(w).T + (0 if b is None else orc._f64(b)))
    elif mutation == "no_corr":
        real = np.exp

        def bad_online(q, k, v, heads, tile=orc.KEY_TILE, return_probs=False):
            q, k, v = orc._f64(q), orc._f64(k), orc._f64(v)
            qh, kh, vh = orc._heads(q, heads), orc._heads(k, heads), orc._heads(v, heads)
            out = np.empty_like(qh)
            for h in range(heads):
                m = np.full(q.shape[0], -np.inf)
                den = np.zeros(q.shape[0])
                acc = np.zeros((q.shape[0], qh.shape[-1]))
                for j0 in range(0, k.shape[0], tile):
                    s = qh[h] @ kh[h, j0:j0 + tile].T * qh.shape[-1] ** -0.5
                    m = np.maximum(m, s.max(axis=1))
                    pr = real(s - m[:, None])
                    den = den + pr.sum(axis=1)          # corr dropped
                    acc = acc + pr @ vh[h, j0:j0 + tile]
                out[h] = acc / den[:, None]
            return orc._merge_heads(out)
        monkeypatch.setattr(orc, "attention_online", bad_online)
    elif mutation == "scale_sqrt_d":
        real = orc.attention_online
        monkeypatch.setattr(orc, "attention_online",
                            lambda q, k, v, heads, **kw: real(q * 0.5, k, v, heads, **kw))
    elif mutation == "ln_unbiased":
        def ln(x, g, b, eps=orc.LN_EPS):
            x = orc._f64(x)
            mu = x.mean(-1, keepdims=True)
            var = ((x - mu) ** 2).sum(-1, keepdims=True) / (x.shape[-1] - 1)
            return (x - mu) / np.sqrt(var + eps) * g + b
        monkeypatch.setattr(orc, "layer_norm", ln)
    elif mutation == "gelu_tanh":
        monkeypatch.setattr(orc, "gelu_erf", lambda z: 0.5 * z * (1 + np.tanh(
            math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3))))
    elif mutation == "no_bias_v":
        real_lin = orc.linear
        calls = {"n": 0}

        def lin(a, w, b=None):
            calls["n"] += 1
            return real_lin(a, w, None if calls["n"] == 3 else b)
        monkeypatch.setattr(orc, "linear", lin)
    elif mutation == "drop_residual":
        real_block = orc._window_block

        def blk(x, p, heads, act=None):
            return real_block(x, p, heads, act) - x
        monkeypatch.setattr(orc, "_window_block", blk)
    assert _hf_check() > 1e-6


# ---------------------------------------------------------------- cross-attention keys and values


def test_cross_kv_matches_hf_decoder_cross_attention_projections():
    """The oracle's cross K/V equal the key and value projections of the Hugging Face Whisper
    decoder layer's encoder attention (its k_proj has no bias, v_proj has one), split by head."""
    from transformers import WhisperConfig
    from transformers.models.whisper.modeling_whisper import WhisperDecoderLayer
    d, heads, t, L = 128, 2, 37, 3
    cfg = WhisperConfig(d_model=d, decoder_attention_heads=heads, decoder_ffn_dim=256,
                        dropout=0.0, attention_dropout=0.0, activation_dropout=0.0)
    r = _rng(77)
    y = r.standard_normal((2, t, d))
    dec = []
    ref = np.empty((2, L, 2, heads, t, d // heads))
    for l in range(L):
        layer = WhisperDecoderLayer(cfg).double().eval()
        ea = layer.encoder_attn
        assert ea.k_proj.bias is None and ea.v_proj.bias is not None
        p = {"wk": r.standard_normal((d, d)) * 0.1, "wv": r.standard_normal((d, d)) * 0.1,
             "bv": r.standard_normal(d) * 0.1}
        with torch.no_grad():
            ea.k_proj.weight.copy_(torch.tensor(p["wk"]))
            ea.v_proj.weight.copy_(torch.tensor(p["wv"]))
            ea.v_proj.bias.copy_(torch.tensor(p["bv"]))
            yt = torch.tensor(y)
            k = ea.k_proj(yt).reshape(2, t, heads, d // heads).transpose(1, 2)
            v = ea.v_proj(yt).reshape(2, t, heads, d // heads).transpose(1, 2)
        ref[:, l, 0], ref[:, l, 1] = k.numpy(), v.numpy()
        dec.append(p)
    np.testing.assert_allclose(oracle.cross_kv(y, dec, heads), ref, atol=1e-12, rtol=0)


def test_cross_kv_closed_forms():
    """Zero weights give K = 0 and V = bv on every row; a head's slab is the head's columns."""
    d, heads, t = 128, 2, 9
    r = _rng(78)
    y = r.standard_normal((t, d))
    p = {"wk": np.zeros((d, d)), "wv": np.zeros((d, d)), "bv": r.standard_normal(d)}
    out = oracle.cross_kv(y, [p], heads)
    assert out.shape == (1, 1, 2, heads, t, 64)
    assert np.all(out[0, 0, 0] == 0)
    for h in range(heads):
        np.testing.assert_array_equal(out[0, 0, 1, h], np.tile(p["bv"][64 * h:64 * h + 64], (t, 1)))
    # identity key weights: the key slab of head h is y's columns 64h .. 64h + 63
    p2 = {"wk": np.eye(d), "wv": np.zeros((d, d)), "bv": np.zeros(d)}
    out2 = oracle.cross_kv(y, [p2], heads)
    for h in range(heads):
        np.testing.assert_array_equal(out2[0, 0, 0, h], y[:, 64 * h:64 * h + 64])


# ---------------------------------------------------------------- conv front end


@pytest.mark.parametrize("t,cin,cout,stride", [(3000, 8, 16, 1), (3000, 16, 8, 2), (7, 3, 5, 2),
                                               (1, 4, 4, 2), (2, 4, 4, 2)])
def test_conv1d_k3_matches_torch(t, cin, cout, stride):
    r = _rng(t + cin + stride)
    x, w, b = r.standard_normal((t, cin)), r.standard_normal((cout, cin, 3)), r.standard_normal(cout)
    ref = torch.nn.functional.conv1d(torch.tensor(x.T[None]), torch.tensor(w), torch.tensor(b),
                                     stride=stride, padding=1)[0].numpy().T
    np.testing.assert_allclose(oracle.conv1d_k3(x, w, b, stride), ref, atol=1e-12, rtol=0)


def test_conv1d_k3_brute_force():
    r = _rng(81)
    x, w, b = r.standard_normal((5, 2)), r.standard_normal((3, 2, 3)), r.standard_normal(3)
    for stride in (1, 2):
        n = (5 - 1) // stride + 1
        ref = [[b[o] + sum(w[o, c, j] * x[stride * i + j - 1, c]
                           for c in range(2) for j in range(3) if 0 <= stride * i + j - 1 < 5)
                for o in range(3)] for i in range(n)]
        np.testing.assert_allclose(oracle.conv1d_k3(x, w, b, stride), ref, atol=1e-13)


def test_conv_stem_matches_hf_whisper_encoder_front_end():
    """Hugging Face's WhisperEncoder applies conv1 + GELU, conv2 + GELU and adds its positional
    embedding before the first layer; with no layers and no final norm its output is the stem's."""
    from transformers import WhisperConfig
    from transformers.models.whisper.modeling_whisper import WhisperEncoder
    d, n_mels, frames = 128, 16, 60
    cfg = WhisperConfig(d_model=d, num_mel_bins=n_mels, encoder_layers=0, encoder_attention_heads=2,
                        max_source_positions=frames // 2, dropout=0.0)
    enc = WhisperEncoder(cfg).double().eval()
    r = _rng(82)
    p = {"conv1_w": r.standard_normal((d, n_mels, 3)) * 0.1, "conv1_b": r.standard_normal(d) * 0.1,
         "conv2_w": r.standard_normal((d, d, 3)) * 0.05, "conv2_b": r.standard_normal(d) * 0.1,
         "pos": r.standard_normal((frames // 2, d))}
    with torch.no_grad():
        enc.conv1.weight.copy_(torch.tensor(p["conv1_w"])); enc.conv1.bias.copy_(torch.tensor(p["conv1_b"]))
        enc.conv2.weight.copy_(torch.tensor(p["conv2_w"])); enc.conv2.bias.copy_(torch.tensor(p["conv2_b"]))
        enc.embed_positions.weight.copy_(torch.tensor(p["pos"]))
        enc.layer_norm = torch.nn.Identity()
        mel = r.standard_normal((2, frames, n_mels))
        ref = enc(torch.tensor(mel.transpose(0, 2, 1))).last_hidden_state.numpy()
    got = oracle.conv_stem(mel, p["conv1_w"], p["conv1_b"], p["conv2_w"], p["conv2_b"], p["pos"])
    np.testing.assert_allclose(got, ref, atol=1e-11, rtol=0)


def test_sinusoid_positions_closed_form():
    pos = synth.sinusoid_positions(1500, 1280)
    assert pos.shape == (1500, 1280)
    np.testing.assert_array_equal(pos[0, :640], 0.0)
    np.testing.assert_array_equal(pos[0, 640:], 1.0)
    np.testing.assert_allclose(pos[1, 0], math.sin(1.0), rtol=1e-6)


# ---------------------------------------------------------------- low-precision weights


def test_bf16_rounding_matches_torch():
    x = np.concatenate([_rng(60).standard_normal(5000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, 1e-40], np.float32)])
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x), ref)


def _near_half(v, tol=1e-4):
    return np.abs(np.abs(v - np.floor(v)) - 0.5) < tol


def test_q8_codes_are_the_nearest_levels():
    w = (_rng(61).standard_normal((16, 128)) * 0.05).astype(np.float32)
    q, d = oracle.quantize_q8(w)
    x = oracle.bf16_round(w).astype(np.float64).reshape(16, -1, 32)
    d32 = (np.max(np.abs(x), axis=2) / 127.0)[:, :, None]
    ks = np.arange(-127, 128, dtype=np.float64)
    # brute force: the level k d nearest to x, ties away from zero
    dist = np.abs(x[..., None] - ks * d32[..., None])
    best = ks[np.argmin(dist - 1e-12 * np.abs(ks), axis=-1)]
    exact = x / d32
    ok = (q.reshape(best.shape) == best) | _near_half(exact)
    assert ok.all()
    # the block's largest magnitude maps to +-127; round trip within half a step
    qb = q.reshape(16, -1, 32).astype(np.int64)
    assert (np.max(np.abs(qb), axis=2) == 127).all()
    back = oracle.dequantize_q8(q, d).reshape(x.shape)
    d16 = d.astype(np.float64)[:, :, None]
    assert (np.abs(back - x) <= d32 / 2 + 127 * np.abs(d16 - d32) + 1e-12).all()


def test_q4_codes_are_the_nearest_levels():
    w = (_rng(62).standard_normal((16, 128)) * 0.05).astype(np.float32)
    v = np.float32(1.5 * np.abs(w[0, :32]).max())
    w[0, 2], w[0, 5] = v, -v  # the first largest magnitude, then its negation
    q, d = oracle.quantize_q4(w)
    assert q.dtype == np.uint8 and q.max() <= 15
    x = oracle.bf16_round(w).astype(np.float64).reshape(16, -1, 32)
    first = np.argmax(np.abs(x), axis=2)
    m = np.take_along_axis(x, first[:, :, None], axis=2)
    d32 = m / -8.0
    ks = np.arange(16, dtype=np.float64)
    dist = np.abs(x[..., None] - (ks - 8) * d32[..., None])
    best = ks[np.argmin(dist - 1e-12 * ks, axis=-1)]  # ties to the larger code
    exact = x / d32 + 8.0
    ok = (q.reshape(best.shape) == best) | _near_half(exact)
    assert ok.all()
    # the first largest magnitude maps to code 0; its negation clamps to 15
    qb = q.reshape(16, -1, 32)
    assert (np.take_along_axis(qb, first[:, :, None], axis=2) == 0).all()
    assert qb[0, 0, 5] == 15


def test_quantizers_zero_block_and_lossless_levels():
    z = np.zeros((2, 64), np.float32)
    q, d = oracle.quantize_q8(z)
    assert (q == 0).all() and (d == 0).all()
    q, d = oracle.quantize_q4(z)
    assert (q == 8).all() and (d.view(np.uint16) == 0).all()  # +0 scale
    assert (oracle.dequantize_q4(q, d) == 0).all()
    r = _rng(63)
    # q8: values k 2^-10 with +-127 in every block are stored exactly
    k = r.integers(-127, 128, size=(8, 96))
    k[:, ::32] = 127 * np.where(r.random((8, 3)) < 0.5, -1, 1)
    w = (k * 2.0 ** -10).astype(np.float32)
    q, d = oracle.quantize_q8(w)
    np.testing.assert_array_equal(q, k)
    np.testing.assert_array_equal(oracle.dequantize_q8(q, d), w.astype(np.float64))
    # q4: values (k - 8) 2^-8 with a unique -8 2^-8 in every block are stored exactly
    k = r.integers(1, 16, size=(8, 96))
    k[:, 7::32] = 0
    w = ((k - 8) * 2.0 ** -8).astype(np.float32)
    q, d = oracle.quantize_q4(w)
    np.testing.assert_array_equal(q, k)
    np.testing.assert_array_equal(oracle.dequantize_q4(q, d), w.astype(np.float64))


def test_quantized_layer_block_is_lossless_on_exact_levels():
    """A block whose matrices already sit on the q8 levels gives the same output as the unquantised
    block (catches a block or matrix applied to the wrong weights)."""
    d, f, heads = 64, 128, 1
    p = _rand_layer(64, d, f)
    r = _rng(65)
    for name in oracle.QUANT_MATRICES:
        k = r.integers(-127, 128, size=p[name].shape)
        k[:, ::32] = 127
        p[name] = (k * 2.0 ** -12).astype(np.float32)
    x = _rng(66).standard_normal((20, d))
    np.testing.assert_allclose(oracle.encoder_block(x, oracle.quantized_layer(p, 8), heads),
                               oracle.encoder_block(x, p, heads), atol=1e-12)
    q = oracle.quantized_layer(p, 4)
    assert np.abs(oracle.encoder_block(x, q, heads) - oracle.encoder_block(x, p, heads)).max() > 1e-4


def test_q8_ties_round_away_from_zero():
    """Exact half levels (d = 2^-10, so the reciprocal is exact) round away from zero."""
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 127 * 2.0 ** -10
    w[0, 1], w[0, 2], w[0, 3] = 2.5 * 2.0 ** -10, -2.5 * 2.0 ** -10, 0.5 * 2.0 ** -10
    q, d = oracle.quantize_q8(w)
    assert d[0, 0] == np.float16(2.0 ** -10)
    assert (q[0, :4] == [127, 3, -3, 1]).all()


def _quant_pins_hold():
    try:
        test_q8_codes_are_the_nearest_levels()
        test_q4_codes_are_the_nearest_levels()
        test_quantizers_zero_block_and_lossless_levels()
        test_q8_ties_round_away_from_zero()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutation", ["q8_scale_128", "q8_round_even", "q4_offset", "q4_last_max",
                                      "q4_dequant_offset"])
def test_planted_quantizer_mistakes_are_caught(monkeypatch, mutation):
    assert _quant_pins_hold()
    real_q8, real_q4, real_dq4 = orc.quantize_q8, orc.quantize_q4, orc.dequantize_q4

    def q8(w, scale=127.0, rnd=None):
        x = orc.bf16_round(w).reshape(w.shape[0], -1, 32)
        d = (np.max(np.abs(x), axis=2).astype(np.float32) / np.float32(scale)).astype(np.float32)
        idv = np.where(d != 0, 1 / np.where(d != 0, d, 1), 0).astype(np.float32)
        v = (x * idv[:, :, None]).astype(np.float32)
        q = rnd(v) if rnd else np.sign(v) * np.floor(np.abs(v) + np.float32(0.5))
        return np.clip(q, -128, 127).astype(np.int8).reshape(w.shape), d.astype(np.float16)

    def q4(w, off=8.5, last=False):
        x = orc.bf16_round(w).reshape(w.shape[0], -1, 32)
        a = np.abs(x)
        idx = (31 - np.argmax(a[:, :, ::-1], axis=2)) if last else np.argmax(a, axis=2)
        m = np.take_along_axis(x, idx[:, :, None], axis=2)[:, :, 0].astype(np.float32)
        d = (m / np.float32(-8.0)).astype(np.float32)
        idv = np.where(d != 0, 1 / np.where(d != 0, d, 1), 0).astype(np.float32)
        v = ((x * idv[:, :, None]).astype(np.float32) + np.float32(off)).astype(np.float32)
        return np.clip(np.floor(v), 0, 15).astype(np.uint8).reshape(w.shape), d.astype(np.float16)

    def plant(name, fn):  # in the module and in the package namespace the pins call
        monkeypatch.setattr(orc, name, fn)
        monkeypatch.setattr(oracle, name, fn)

    if mutation == "q8_scale_128":
        plant("quantize_q8", lambda w: q8(w, scale=128.0))
    elif mutation == "q8_round_even":
        plant("quantize_q8", lambda w: q8(w, rnd=np.rint))
    elif mutation == "q4_offset":
        plant("quantize_q4", lambda w: q4(w, off=8.0))
    elif mutation == "q4_last_max":
        plant("quantize_q4", lambda w: q4(w, last=True))
    elif mutation == "q4_dequant_offset":
        plant("dequantize_q4", lambda c, s: real_dq4(c, s) + s.astype(np.float64).repeat(32, axis=1))
    assert not _quant_pins_hold()
    del real_q8, real_q4


# ---------------------------------------------------------------- MXFP8 (E4M3 values, E8M0 scales)


def _e4m3_table():
    """Every finite E4M3 value, decoded by torch's float8_e4m3fn (an implementation independent of
    the oracle): codes 0 .. 126 and 128 .. 254 (0x7f and 0xff are NaN)."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return codes, vals


def test_e4m3_round_matches_torch_and_round_trips():
    """On float32 inputs of every magnitude up to 448, the oracle's rounding equals torch's
    float8_e4m3fn cast (value and bit pattern); every finite E4M3 value rounds to itself."""
    rng = np.random.default_rng(41)
    y = (rng.standard_normal(200_000) * np.exp2(rng.integers(-14, 9, 200_000))).astype(np.float32)
    y = y[np.abs(y) <= 448]
    t = torch.from_numpy(y.copy()).to(torch.float8_e4m3fn)
    r = orc.e4m3_round(y.astype(np.float64))
    np.testing.assert_array_equal(r, t.to(torch.float64).numpy())
    np.testing.assert_array_equal(orc.e4m3_bits(r), t.view(torch.uint8).numpy())
    codes, vals = _e4m3_table()
    np.testing.assert_array_equal(orc.e4m3_round(vals), vals)
    np.testing.assert_array_equal(orc.e4m3_bits(vals), codes)


def test_e4m3_codes_of_named_values():
    """Codes the E4M3 (fn) format fixes by its field layout (sign, 4 exponent bits with bias 7, 3
    mantissa bits, no infinities): the largest finite value 448 = 1.75 * 2^8 is S.1111.110 (0x7E),
    1 is 0.0111.000 (0x38), -2 is 1.1000.000 (0xC0), the smallest normal 2^-6 is 0.0001.000 (0x08),
    the smallest subnormal 2^-9 is 0.0000.001 (0x01), the largest subnormal 7 * 2^-9 is 0x07."""
    vals = np.array([448.0, 1.0, -2.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, 0.0, 1.5, 0.8125])
    want = np.array([0x7E, 0x38, 0xC0, 0x08, 0x01, 0x07, 0x00, 0x3C, 0x35])
    np.testing.assert_array_equal(orc.e4m3_round(vals), vals)
    np.testing.assert_array_equal(orc.e4m3_bits(vals), want)
    # halfway between 2^-9 and 2 * 2^-9 rounds to the even code (2 * 2^-9, 0x02); a quarter of
    # the smallest subnormal rounds to zero
    np.testing.assert_array_equal(orc.e4m3_bits(orc.e4m3_round(np.array([1.5 * 2.0 ** -9]))), [0x02])
    assert orc.e4m3_round(np.array([0.25 * 2.0 ** -9]))[0] == 0.0


def test_e4m3_ties_go_to_the_even_code():
    """The midpoint of two neighbouring non-negative values rounds to the one whose code is even."""
    codes, vals = _e4m3_table()
    pos = vals[codes < 0x80]
    pc = codes[codes < 0x80]
    order = np.argsort(pos)
    pos, pc = pos[order], pc[order]
    mid = (pos[:-1] + pos[1:]) / 2
    got = orc.e4m3_bits(orc.e4m3_round(mid))
    want = np.where(pc[:-1] % 2 == 0, pc[:-1], pc[1:])
    np.testing.assert_array_equal(got, want)
    with pytest.raises(ValueError):
        orc.e4m3_round(np.array([448.5]))


def test_mx_scale_exponent_closed_forms():
    """X is the smallest integer with amax <= 448 2^X: 448 2^j -> j, just above -> j + 1,
    2^j -> j - 8 (2^j <= 1.75 2^j), 1.75 2^j -> j - 8, zero -> -127, clipped to [-127, 127]."""
    j = np.arange(-100, 100)
    p = np.exp2(j.astype(np.float64))
    np.testing.assert_array_equal(orc.mx_scale_exponent(448 * p), j)
    np.testing.assert_array_equal(orc.mx_scale_exponent(np.nextafter(448 * p, np.inf)), j + 1)
    np.testing.assert_array_equal(orc.mx_scale_exponent(p), j - 8)
    np.testing.assert_array_equal(orc.mx_scale_exponent(1.75 * p), j - 8)
    np.testing.assert_array_equal(orc.mx_scale_exponent(np.nextafter(1.75 * p, np.inf)), j - 7)
    assert orc.mx_scale_exponent(np.array([0.0]))[0] == -127
    assert orc.mx_scale_exponent(np.array([1e-300]))[0] == -127
    assert orc.mx_scale_exponent(np.array([3e38]))[0] == 120


def test_mx_quantize_is_the_nearest_scaled_value():
    """Brute force over the 253 finite E4M3 values: each element becomes the nearest of
    {value 2^X} (ties to the even code) with X its block's exponent, which is the smallest that
    keeps the block's largest magnitude within 448 2^X; nothing saturates."""
    codes, vals = _e4m3_table()
    rng = np.random.default_rng(43)
    a = rng.standard_normal((6, 64)) * np.exp2(rng.integers(-20, 20, (6, 1)))
    a[0, :32] = 0.0
    a[1, :32] *= 1e-3
    a[2, 5] = 448.0 * 2.0 ** 3 * 1.0000001  # a largest magnitude just above a scale boundary
    got, x = orc.mx_quantize(a)
    assert x.shape == (6, 2)
    for r in range(6):
        for b in range(2):
            blk = a[r, 32 * b:32 * b + 32]
            amax = np.max(np.abs(blk))
            X = int(x[r, b])
            if amax == 0:
                assert X == -127 and np.all(got[r, 32 * b:32 * b + 32] == 0)
                continue
            assert amax <= 448 * 2.0 ** X and amax > 448 * 2.0 ** (X - 1)
            grid = vals * 2.0 ** X
            for i, v in enumerate(blk):
                dist = np.abs(grid - v)
                best = np.flatnonzero(dist == dist.min())
                cand = grid[best]
                if len(set(cand)) > 1:  # a tie: the even code
                    cand = grid[best[codes[best] % 2 == 0]]
                assert got[r, 32 * b + i] == cand[0] or (v == 0 and got[r, 32 * b + i] == 0)


def test_mxfp8_layer_and_block_operands():
    """mxfp8_layer quantises Wq, Wk, Wv, W1 and W2 along their input columns and leaves the
    out-projection, norms and biases alone; the block applies `act` to exactly three operands,
    LN1(x) and LN2(x1) ([t, d]) and the GELU output ([t, f]), and an identity act changes
    nothing."""
    cfg = synth.CONFIGS["tiny_block"].with_(t=40)
    w = synth.make_workload(cfg)
    p = w.layers[0]
    q = orc.mxfp8_layer(p)
    for n in ("wq", "wk", "wv", "w1", "w2"):
        np.testing.assert_array_equal(q[n], orc.mx_values(p[n]))
        assert not np.array_equal(q[n], p[n])
    for n in ("wo", "bo", "bq", "bv", "b1", "b2", "ln1_g", "ln2_b"):
        np.testing.assert_array_equal(q[n], p[n])
    seen = []

    def act(a):
        seen.append(a.shape)
        return a
    out = orc.encoder_block(w.x, p, cfg.heads, act=act)
    assert seen == [(40, 384), (40, 384), (40, 1536)]
    np.testing.assert_array_equal(out, orc.encoder_block(w.x, p, cfg.heads))
