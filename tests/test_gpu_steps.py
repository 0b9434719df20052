"""Step-level GPU parity: each kernel of the block against the CPU oracle, element by element,
through the C ABI.  Operands are first rounded to the path's type on the device and the oracle
receives those exact values, so the measured error is the kernel's own (accumulation order,
internal roundings, output rounding).

Tolerances (max relative error floored at the reference RMS) follow from the output type: one
ulp of the stored result (bf16 2^-8, fp16 2^-11) plus fp32 accumulation noise; the attention
kernel also rounds the probabilities to the operand type before P.V.
"""

import numpy as np
import pytest

import oracle
from speech_transformer_encoder_amd import binding as B
from speech_transformer_encoder_amd import synth
from tests.gpu_util import as_operand, dev, errors, host, report, require_gpu, torch_dtype

pytestmark = pytest.mark.gpu

PATHS = [B.WENC_PATH_BF16, B.WENC_PATH_FP16, B.WENC_PATH_FP32]
OUT_TOL = {B.WENC_PATH_BF16: 5e-3, B.WENC_PATH_FP16: 8e-4, B.WENC_PATH_FP32: 2e-5}
ATTN_TOL = {B.WENC_PATH_BF16: 1.2e-2, B.WENC_PATH_FP16: 2e-3, B.WENC_PATH_FP32: 2e-5}
LN_DT = {B.WENC_PATH_BF16: B.WENC_DTYPE_BF16, B.WENC_PATH_FP16: B.WENC_DTYPE_F16,
         B.WENC_PATH_FP32: B.WENC_DTYPE_F32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _rng(*s):
    return np.random.default_rng([*s, 777])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("rows,d", [(1, 384), (5, 512), (1500, 768), (333, 1280), (7, 4096)])
def test_layernorm(path, rows, d):
    import torch
    r = _rng(rows, d)
    x = r.standard_normal((rows, d)).astype(np.float32) * 3 + 0.5
    x[rows // 2] *= 20  # a scaled row normalises to the same values
    g = (1 + 0.1 * r.standard_normal(d)).astype(np.float32)
    b = (0.1 * r.standard_normal(d)).astype(np.float32)
    xd, gd, bd = dev(x), dev(g), dev(b)
    y = torch.empty((rows, d), dtype=torch_dtype(path), device="cuda")
    print(f"[case] layernorm path={path} rows={rows} d={d}", flush=True)
    B.whisper_enc_layernorm(xd, gd, bd, y, rows, d, LN_DT[path])
    e = errors(host(y), oracle.layer_norm(x, g, b))
    report(f"ln p{path} {rows}x{d}", e)
    assert e["finite"] and e["max_rel"] <= OUT_TOL[path] * 1.01


def test_layernorm_in_place_fp32():
    r = _rng(9)
    x = r.standard_normal((64, 512)).astype(np.float32)
    g, b = np.ones(512, np.float32), np.zeros(512, np.float32)
    xd = dev(x)
    B.whisper_enc_layernorm(xd, dev(g), dev(b), xd, 64, 512, B.WENC_DTYPE_F32)
    assert errors(host(xd), oracle.layer_norm(x, g, b))["max_rel"] < 2e-5


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("epi", [B.WENC_EPI_BIAS, B.WENC_EPI_BIAS_GELU, B.WENC_EPI_BIAS_RESIDUAL,
                                 B.WENC_EPI_BIAS_GELU_RESIDUAL])
@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (200, 384, 384), (257, 192, 512), (1500, 1152, 384),
                                   (129, 1280, 5120), (1300, 3840, 128), (6000, 4160, 128),
                                   (24000, 1280, 64), (4096, 4160, 256), (10240, 2048, 128),
                                   (11008, 1344, 64)])
def test_linear(path, epi, m, n, k):
    """Every element against the oracle.  The shapes reach every tiling of the 16-bit paths:
    below 128 tiles of 128 x 256, the small kernel's 128 x 128 tiles (e.g. (1500, 1152): 108 of
    them); (1300, 3840): 180 tiles of 128 x 256, the last row of tiles 20 rows high; from 256
    tiles of 256 x 256, the persistent kernel.  (4096, 4160): 272 tiles of 256 x 256 on 256 CUs,
    one whole round and 16 left over, which run as 128-column half tiles, 8 of them in the last
    64-column-wide tile (their second halves empty).  With at most eight n tiles the persistent
    order is n fastest: (24000, 1280) runs it in whole rounds and its own last round; (10240,
    2048): 320 tiles, one round and 64 left over as 128 half tiles; (11008, 1344): 258 tiles (the
    last n tile 64 columns wide), one round and 2 left over as 4 half tiles, one of them empty."""
    import torch
    r = _rng(m, n, k, epi)
    a = r.standard_normal((m, k)).astype(np.float32)
    w = (r.standard_normal((n, k)) * 0.02).astype(np.float32)
    bias = (r.standard_normal(n) * 0.1).astype(np.float32)
    ad, ah = as_operand(a, path)
    wd, wh = as_operand(w, path)
    ref = oracle.linear(ah, wh, bias)
    resid = None
    fp32_out = epi in (B.WENC_EPI_BIAS_RESIDUAL, B.WENC_EPI_BIAS_GELU_RESIDUAL)
    if fp32_out:
        res_np = r.standard_normal((m, n)).astype(np.float32) * 4
        resid = dev(res_np)
        c = torch.empty((m, n), dtype=torch.float32, device="cuda")
        if epi == B.WENC_EPI_BIAS_GELU_RESIDUAL:
            ref = oracle.gelu_erf(ref)
        ref = ref + res_np
    else:
        c = torch.empty((m, n), dtype=torch_dtype(path), device="cuda")
        if epi == B.WENC_EPI_BIAS_GELU:
            ref = oracle.gelu_erf(ref)
    print(f"[case] linear path={path} epi={epi} m={m} n={n} k={k}", flush=True)
    B.whisper_enc_linear(ad, wd, dev(bias), resid, c, m, n, k, path, epi)
    e = errors(host(c), ref)
    report(f"linear p{path} e{epi} {m}x{n}x{k}", e)
    tol = 2e-5 if fp32_out else OUT_TOL[path]
    assert e["finite"] and e["max_rel"] <= tol


def test_linear_residual_in_place():
    r = _rng(31)
    m, n, k = 300, 256, 128
    a = r.standard_normal((m, k)).astype(np.float32)
    w = (r.standard_normal((n, k)) * 0.05).astype(np.float32)
    bias = r.standard_normal(n).astype(np.float32)
    x = r.standard_normal((m, n)).astype(np.float32)
    xd = dev(x)
    B.whisper_enc_linear(dev(a), dev(w), dev(bias), xd, xd, m, n, k, B.WENC_PATH_FP32,
                         B.WENC_EPI_BIAS_RESIDUAL)
    assert errors(host(xd), x + oracle.linear(a, w, bias))["max_rel"] < 2e-5


def _attention_case(path, batch, t, heads, seed, outlier_frac=0.0, packed=True):
    """Run the kernel and return (errors, componentwise ratio).

    The componentwise ratio is ``max |g - o| / (P |V|)``: each output element's error over the
    probability-weighted sum of |v| that bounds the rounding error of P.V (P rounded to the
    operand type before the MFMA, the output rounded once).  It stays meaningful when large
    logits make the softmax nearly one-hot and the output itself cancels to small values.
    """
    import torch
    q, k, v = synth.random_qkv(seed, batch, t, heads, outlier_frac=outlier_frac,
                               outlier_scale=20.0)
    d = heads * 64
    qd, qh = as_operand(q, path)
    kd, kh = as_operand(k, path)
    vd, vh = as_operand(v, path)
    if packed:  # the block's layout: one [rows, 3d] buffer holding q | k | v
        qkv = torch.cat([qd.reshape(-1, d), kd.reshape(-1, d), vd.reshape(-1, d)], dim=1).contiguous()
        es = qkv.element_size()
        qp, kp, vp, ld = qkv.data_ptr(), qkv.data_ptr() + d * es, qkv.data_ptr() + 2 * d * es, 3 * d
    else:
        qp, kp, vp, ld = qd, kd, vd, d
    o = torch.full((batch * t, d), float("nan"), dtype=torch_dtype(path), device="cuda")
    print(f"[case] attention path={path} batch={batch} t={t} heads={heads} outliers={outlier_frac}",
          flush=True)
    B.whisper_enc_attention(qp, kp, vp, o, batch, t, heads, ld, d, path)
    got = host(o).reshape(batch, t, d)
    refs, bounds = [], []
    for b in range(batch):
        ob, pb = oracle.attention_online(qh[b], kh[b], vh[b], heads, return_probs=True)
        refs.append(ob)
        absv = np.abs(vh[b]).reshape(t, heads, 64).transpose(1, 0, 2)
        bounds.append(np.einsum("hij,hjd->ihd", pb, absv).reshape(t, d))
    ref, bound = np.stack(refs), np.stack(bounds)
    ratio = float(np.max(np.abs(got - ref) / bound)) if np.isfinite(got).all() else float("inf")
    return errors(got, ref), ratio


# Componentwise bound on |g - o| / (P|V|): bf16 2^-7 and fp16 2^-10 (twice the sum of the
# P and output roundings), fp32 2e-5 (exp2 and accumulation in fp32).
ATTN_CW = {B.WENC_PATH_BF16: 2.0 ** -7, B.WENC_PATH_FP16: 2.0 ** -10, B.WENC_PATH_FP32: 2e-5}


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("batch,t,heads", [(1, 1, 1), (1, 17, 2), (2, 63, 1), (1, 64, 1),
                                           (1, 65, 3), (1, 127, 1), (3, 129, 2), (1, 300, 2),
                                           (2, 1500, 2)])
def test_attention(path, batch, t, heads):
    e, cw = _attention_case(path, batch, t, heads, seed=t + 7 * heads)
    report(f"attn p{path} b{batch} t{t} h{heads} cw={cw:.3e}", e)
    assert e["finite"] and e["max_rel"] <= ATTN_TOL[path] and cw <= ATTN_CW[path]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("batch,heads,groups", [(2, 2, 2), (1, 12, 2), (2, 12, 1)])
def test_attention_outlier_queries(path, batch, heads, groups):
    """5 % of query rows scaled by 20: logit spreads of ~100 exercise the running max, including
    the raise of the max in the middle of the key loop (ballot, rescale, re-exponentiation).
    Both workgroup forms the 16-bit kernel has are reached at t = 1500: 48 and 144 blocks of 128
    query rows run workgroups of two wavefront groups over the two key halves (merged at the
    end, after raises in either half), 288 (at least 256) the one-group workgroups of 256 rows,
    the batched shape.  The softmax of the scaled rows is nearly one-hot, so the componentwise
    bound is the one that applies."""
    assert groups == (1 if 12 * heads * batch >= 256 else 2)
    e, cw = _attention_case(path, batch, 1500, heads, seed=5 + heads, outlier_frac=0.05)
    report(f"attn-outliers p{path} b{batch} h{heads} ({groups} key groups) cw={cw:.3e}", e)
    assert e["finite"] and cw <= ATTN_CW[path]


@pytest.mark.parametrize("path", [B.WENC_PATH_FP16, B.WENC_PATH_BF16])
@pytest.mark.parametrize("batch,t,heads", [(4, 1300, 6), (4, 257, 24), (16, 1, 16)])
def test_attention_batched_partial_query_blocks(path, batch, t, heads):
    """The one-group workgroups of 256 query rows (at least 256 blocks of 128 rows) when the last
    query block of each (window, head) is mostly past the window: t = 1300 leaves 20 rows in it
    (wavefronts 1-7 hold none), t = 257 one row, t = 1 one row in the only block.  Wavefronts
    without rows only copy their share of the key and value tiles; the rows that exist must
    still see every key."""
    assert ((t + 127) // 128) * heads * batch >= 256
    e, cw = _attention_case(path, batch, t, heads, seed=3 * t + heads)
    report(f"attn-partial p{path} b{batch} t{t} h{heads} cw={cw:.3e}", e)
    assert e["finite"] and e["max_rel"] <= ATTN_TOL[path] and cw <= ATTN_CW[path]


def test_attention_separate_buffers():
    e, cw = _attention_case(B.WENC_PATH_BF16, 2, 200, 3, seed=3, packed=False)
    assert e["max_rel"] <= ATTN_TOL[B.WENC_PATH_BF16] and cw <= ATTN_CW[B.WENC_PATH_BF16]


def test_attention_identical_keys_mean_of_v():
    import torch
    t, heads, d = 300, 2, 128
    r = _rng(44)
    q = r.standard_normal((t, d)).astype(np.float32)
    k = np.tile(r.standard_normal((1, d)).astype(np.float32), (t, 1))
    v = r.standard_normal((t, d)).astype(np.float32)
    o = torch.empty((t, d), dtype=torch.float32, device="cuda")
    B.whisper_enc_attention(dev(q), dev(k), dev(v), o, 1, t, heads, d, d, B.WENC_PATH_FP32)
    np.testing.assert_allclose(host(o), np.tile(v.mean(0), (t, 1)), atol=2e-5)
