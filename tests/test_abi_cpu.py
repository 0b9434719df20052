"""The C ABI without a GPU: the library loads, exports what the header declares, and rejects bad
arguments before it touches HIP (so every call below returns without a device)."""

import os
import re

import pytest

from speech_transformer_encoder_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "whisper_enc.h")

FAKE = 1 << 20  # aligned, non-null "device" address: validation must fail before any use


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libwhisper_enc.so is not built (run __graft_entry__.build())")
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(whisper_enc_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(B.EXPORTS)


def test_header_constants_match_binding():
    """Every #define WENC_* integer in the header has the same value in the Python binding."""
    text = open(HEADER).read()
    consts = dict(re.findall(r"^#define\s+(WENC_\w+)\s+(-?\d+)\b", text, re.M))
    assert len(consts) > 10
    for name, value in consts.items():
        assert getattr(B, name) == int(value), name


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_sizes():
    assert B.whisper_enc_layer_bytes(384, 1536, B.WENC_PATH_BF16) > 0
    bf = B.whisper_enc_layer_bytes(1280, 5120, B.WENC_PATH_BF16)
    f32 = B.whisper_enc_layer_bytes(1280, 5120, B.WENC_PATH_FP32)
    # matrices dominate: 12 d^2 elements of 2 or 4 bytes
    assert bf >= 12 * 1280 * 1280 * 2 and f32 >= 12 * 1280 * 1280 * 4
    assert bf % 256 == 0 and f32 % 256 == 0
    assert B.whisper_enc_layer_bytes(100, 5120, 0) == 0
    assert B.whisper_enc_layer_bytes(1280, 5120, 8) == 0
    ws = B.whisper_enc_workspace_bytes(16, 1500, 1280, 20, 5120, B.WENC_PATH_BF16)
    assert ws >= 16 * 1500 * (1280 + 5120) * 2
    assert B.whisper_enc_workspace_bytes(1, 1500, 1280, 16, 5120, 0) == 0  # head_dim 80


def test_workspace_follows_the_split_plans(lib):
    """One window: the workspace holds the 16-bit activations ([t, d] and [t, max(3d, f)]) and one
    scratch region sized for the larger of the residual GEMMs' fp32 k parts and the attention key
    halves' (O, m, l).  The sizes pin the largest part count (fc2's) against the key halves:
      d 1280, 20 heads: fc2 4 parts (the out-projection 2); 240 query blocks of 128 rows, no key
        halves -> 4 x 1500 x 1280 floats;
      d 512, 8 heads: fc2 4 parts (8 parts of 256 k halved); 96 blocks, key halves
        (2 x 1500 x 8 x 66 floats, smaller) -> 4 x 1500 x 512 floats;
      d 384, 6 heads: fc2 4 parts (the out-projection unsplit: k 384 has no two parts of 256);
        72 blocks, key halves -> 4 x 1500 x 384 floats."""
    P16 = B.WENC_PATH_FP16
    for d, h, f in [(1280, 20, 5120), (512, 8, 2048), (384, 6, 1536)]:
        act = 1500 * d * 2 + 1500 * max(3 * d, f) * 2
        assert B.whisper_enc_workspace_bytes(1, 1500, d, h, f, P16) == act + 4 * 1500 * d * 4, d


def test_bf16x2_path_sizes_and_validation(lib):
    """BF16X2 packs the same bf16 blob as BF16; its workspace holds the hi / lo activation pairs
    (LayerNorm outputs [M, 2d], FFN hidden [M, 2 ffn]); the step-level entry points reject it."""
    P2, P1 = B.WENC_PATH_BF16X2, B.WENC_PATH_BF16
    for d, f in [(384, 1536), (1280, 5120)]:
        assert B.whisper_enc_layer_bytes(d, f, P2) == B.whisper_enc_layer_bytes(d, f, P1)
    M, d, h, f = 16 * 1500, 1280, 20, 5120
    assert B.whisper_enc_workspace_bytes(16, 1500, d, h, f, P2) >= M * (2 * d + 2 * f) * 2
    assert B.whisper_enc_workspace_bytes(16, 1500, d, h, f, P2) > \
        B.whisper_enc_workspace_bytes(16, 1500, d, h, f, P1)
    assert lib.whisper_enc_linear(FAKE, FAKE, FAKE, None, FAKE, 64, 64, 64, P2,
                                  B.WENC_EPI_BIAS, None) == B.WENC_ERR_ARG
    assert lib.whisper_enc_attention(FAKE, FAKE, FAKE, FAKE, 1, 64, 1, 192, 64, P2,
                                     None) == B.WENC_ERR_ARG
    # BF16X3: the blob holds every weight as a hi / lo pair
    P3 = B.WENC_PATH_BF16X3
    weights = 4 * d * d + 2 * d * f
    assert B.whisper_enc_layer_bytes(d, f, P3) >= B.whisper_enc_layer_bytes(d, f, P1) + 2 * weights
    assert B.whisper_enc_workspace_bytes(1, 1500, 1280, 20, 5120, 8) == 0


def test_strerror(lib):
    for code in range(6):
        assert B.strerror(code)
    assert "unknown" in B.strerror(99)


def _block(lib, **kw):
    a = dict(x=FAKE, y=FAKE, layer=FAKE, batch=1, t=1500, d=384, heads=6, f=1536, path=0,
             ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.whisper_enc_block_forward(a["x"], a["y"], a["layer"], a["batch"], a["t"], a["d"],
                                         a["heads"], a["f"], a["path"], a["ws"], a["wsb"],
                                         a["stream"])


def test_block_validation(lib):
    assert _block(lib, heads=4) == B.WENC_ERR_UNSUPPORTED      # head_dim 96
    assert _block(lib, heads=5) == B.WENC_ERR_ARG              # d % heads != 0
    assert _block(lib, d=100, heads=1) == B.WENC_ERR_ARG
    assert _block(lib, f=100) == B.WENC_ERR_ARG
    assert _block(lib, path=8) == B.WENC_ERR_ARG
    assert _block(lib, batch=-1) == B.WENC_ERR_ARG
    assert _block(lib, x=None) == B.WENC_ERR_ARG
    assert _block(lib, layer=None) == B.WENC_ERR_ARG
    assert _block(lib, ws=None) == B.WENC_ERR_ARG
    assert _block(lib, x=FAKE + 4) == B.WENC_ERR_ARG           # misaligned
    assert _block(lib, layer=FAKE + 16) == B.WENC_ERR_ARG      # blob must be 256-aligned
    assert _block(lib, y=FAKE + 16) == B.WENC_ERR_ARG          # partial overlap with x
    assert _block(lib, wsb=1000) == B.WENC_ERR_WORKSPACE
    assert _block(lib, batch=1 << 20, t=1500) == B.WENC_ERR_ARG  # too many rows
    # empty input: nothing to do, pointers unused
    assert _block(lib, batch=0, x=None, y=None, layer=None, ws=None) == B.WENC_OK
    assert _block(lib, t=0, x=None, y=None, layer=None, ws=None) == B.WENC_OK


def test_stack_validation(lib):
    f = lib.whisper_enc_stack_forward
    args = [FAKE, FAKE + (1 << 24), FAKE, 4, None, None, 1, 1500, 512, 8, 2048, 0, FAKE, 1 << 40,
            None]
    ok = list(args)
    bad = list(args); bad[3] = -1
    assert f(*bad) == B.WENC_ERR_ARG
    bad = list(args); bad[4] = FAKE                            # gamma without beta
    assert f(*bad) == B.WENC_ERR_ARG
    bad = list(args); bad[13] = 10
    assert f(*bad) == B.WENC_ERR_WORKSPACE
    bad = list(args); bad[9] = 16
    assert f(*bad) == B.WENC_ERR_UNSUPPORTED
    assert ok  # the valid call itself needs a GPU


def test_noalloc_validation(lib):
    """The no-allocation entry point checks every argument, and the shape's workspace against its
    static scratch, before its first HIP call (the device's scratch address lookup)."""
    f = lib.whisper_enc_stack_forward_noalloc
    args = [FAKE, FAKE + (1 << 28), FAKE, 2, None, None, 1, 1500, 1280, 20, 5120,
            B.WENC_PATH_FP16, None]
    assert B.whisper_enc_workspace_bytes(1, 1500, 1280, 20, 5120, B.WENC_PATH_FP16) \
        <= B.WENC_NOALLOC_SCRATCH_BYTES
    bad = list(args); bad[6] = 2                               # two windows: 65.9 MiB
    assert f(*bad) == B.WENC_ERR_SCRATCH
    bad = list(args); bad[11] = B.WENC_PATH_Q8                 # + fp16 expansion: 85.1 MiB
    assert f(*bad) == B.WENC_ERR_SCRATCH
    bad = list(args); bad[3] = -1
    assert f(*bad) == B.WENC_ERR_ARG
    bad = list(args); bad[0] = FAKE + 4                        # misaligned x
    assert f(*bad) == B.WENC_ERR_ARG
    bad = list(args); bad[2] = None
    assert f(*bad) == B.WENC_ERR_ARG
    bad = list(args); bad[4] = FAKE                            # gamma without beta
    assert f(*bad) == B.WENC_ERR_ARG
    bad = list(args); bad[9] = 16                              # head_dim 80
    assert f(*bad) == B.WENC_ERR_UNSUPPORTED
    bad = list(args); bad[6] = 0                               # no rows: nothing to do
    assert f(*bad) == B.WENC_OK
    assert B.strerror(B.WENC_ERR_SCRATCH).startswith("shape needs more workspace")


def test_step_validation(lib):
    assert lib.whisper_enc_layernorm(FAKE, FAKE, FAKE, FAKE, 10, 100, 0, None) == B.WENC_ERR_ARG
    assert lib.whisper_enc_layernorm(FAKE, FAKE, FAKE, FAKE, 10, 384, 5, None) == B.WENC_ERR_ARG
    assert lib.whisper_enc_layernorm(FAKE, FAKE, FAKE, FAKE, 10, 384, 1, None) == B.WENC_ERR_ARG
    assert lib.whisper_enc_layernorm(None, None, None, None, 0, 384, 1, None) == B.WENC_OK
    lin = lib.whisper_enc_linear
    assert lin(FAKE, FAKE, FAKE, None, FAKE, 10, 100, 64, 0, 0, None) == B.WENC_ERR_ARG
    assert lin(FAKE, FAKE, FAKE, None, FAKE, 10, 128, 64, 0, 2, None) == B.WENC_ERR_ARG
    assert lin(FAKE, FAKE, None, None, FAKE, 10, 128, 64, 0, 0, None) == B.WENC_ERR_ARG
    assert lin(FAKE, FAKE, FAKE, None, FAKE, 10, 128, 64, 0, 9, None) == B.WENC_ERR_ARG
    att = lib.whisper_enc_attention
    assert att(FAKE, FAKE, FAKE, FAKE, 1, 100, 2, 64, 128, 0, None) == B.WENC_ERR_ARG
    assert att(FAKE, FAKE, FAKE, FAKE, 1, 100, 2, 130, 128, 0, None) == B.WENC_ERR_ARG
    assert att(None, None, None, None, 0, 100, 2, 128, 128, 0, None) == B.WENC_OK
    pk = lib.whisper_enc_pack_layer
    ptrs = [FAKE] * 16
    assert pk(*ptrs, 384, 1536, 0, FAKE + 8, None) == B.WENC_ERR_ARG
    ptrs2 = list(ptrs); ptrs2[2] = None
    assert pk(*ptrs2, 384, 1536, 0, FAKE, None) == B.WENC_ERR_ARG
    assert pk(*ptrs, 384, 1000, 0, FAKE, None) == B.WENC_ERR_ARG


def test_package_has_no_cpu_fallback():
    """The product package never imports the oracle."""
    pkg = os.path.join(ROOT, "speech_transformer_encoder_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn


def test_cross_kv_sizes_and_validation(lib):
    assert B.whisper_enc_cross_kv_bytes(1280, 32, B.WENC_PATH_FP16) > 2 * 32 * 1280 * 1280 * 2
    assert B.whisper_enc_cross_kv_bytes(1280, 0, B.WENC_PATH_FP16) == 0
    assert B.whisper_enc_cross_kv_bytes(100, 2, B.WENC_PATH_FP16) == 0
    assert B.whisper_enc_cross_kv_bytes(1280, 65, B.WENC_PATH_FP16) == 0
    assert B.whisper_enc_cross_kv_workspace_bytes(16, 1500, 1280, B.WENC_PATH_FP16) >= 16 * 1500 * 1280 * 2
    call = lambda *a: lib.whisper_enc_cross_kv(*a)  # noqa: E731
    # heads that do not give head_dim 64
    assert call(FAKE, FAKE, FAKE, 2, 1, 10, 1280, 10, B.WENC_PATH_FP16, FAKE, 1 << 30, None) == B.WENC_ERR_UNSUPPORTED
    # null output, misaligned weights, small workspace, bad layer count
    assert call(FAKE, None, FAKE, 2, 1, 10, 1280, 20, B.WENC_PATH_FP16, FAKE, 1 << 30, None) == B.WENC_ERR_ARG
    assert call(FAKE, FAKE, FAKE + 16, 2, 1, 10, 1280, 20, B.WENC_PATH_FP16, FAKE, 1 << 30, None) == B.WENC_ERR_ARG
    assert call(FAKE, FAKE, FAKE, 2, 1, 10, 1280, 20, B.WENC_PATH_FP16, FAKE, 16, None) == B.WENC_ERR_WORKSPACE
    assert call(FAKE, FAKE, FAKE, 0, 1, 10, 1280, 20, B.WENC_PATH_FP16, FAKE, 1 << 30, None) == B.WENC_ERR_ARG
    # zero rows enqueue nothing
    assert call(None, None, FAKE, 2, 0, 10, 1280, 20, B.WENC_PATH_FP16, None, 0, None) == B.WENC_OK


def test_stem_sizes_and_validation(lib):
    # large-v3 front end: 128 mel bins, width 1280, 1500 positions
    n = B.whisper_enc_stem_bytes(128, 1280, 1500, B.WENC_PATH_FP16)
    assert n >= (1280 * 384 + 1280 * 3 * 1280) * 2 + 1500 * 1280 * 4
    assert B.whisper_enc_stem_bytes(0, 1280, 1500, B.WENC_PATH_FP16) == 0
    assert B.whisper_enc_stem_bytes(128, 100, 1500, B.WENC_PATH_FP16) == 0
    assert B.whisper_enc_stem_bytes(128, 1280, 0, B.WENC_PATH_FP16) == 0
    ws = B.whisper_enc_stem_workspace_bytes(16, 3000, 128, 1280, B.WENC_PATH_FP16)
    assert ws >= 16 * 3000 * (384 + 1280) * 2 + 16 * 1500 * 3 * 1280 * 2
    call = lambda *a: lib.whisper_enc_stem_forward(*a)  # noqa: E731

    def go(mel=FAKE, x=1 << 40, stem=FAKE, batch=2, t=3000, mels=128, d=1280, npos=1500,
           path=B.WENC_PATH_FP16, ws=FAKE, wsb=1 << 34):
        return call(mel, x, stem, batch, t, mels, d, npos, path, ws, wsb, None)

    # more positions needed than packed, width not a multiple of 64, null output
    assert go(t=3002) == B.WENC_ERR_ARG
    assert go(d=1000) == B.WENC_ERR_ARG
    assert go(x=None) == B.WENC_ERR_ARG
    # misaligned stem, x overlapping mel, small workspace
    assert go(stem=FAKE + 16) == B.WENC_ERR_ARG
    assert go(x=FAKE) == B.WENC_ERR_ARG
    assert go(x=FAKE + 4096) == B.WENC_ERR_ARG
    assert go(wsb=16) == B.WENC_ERR_WORKSPACE
    # odd frame counts take ceil(t / 2) positions
    assert go(t=2999, npos=1500, wsb=16) == B.WENC_ERR_WORKSPACE
    # no frames enqueue nothing
    assert go(mel=None, x=None, stem=FAKE, t=0, ws=None, wsb=0) == B.WENC_OK


def test_varlen_sizes_and_validation(lib):
    P16 = B.WENC_PATH_FP16
    dense = B.whisper_enc_workspace_bytes(1, 9000, 1280, 20, 5120, P16)
    assert B.whisper_enc_varlen_workspace_bytes(16, 9000, 1500, 1280, 20, 5120, P16) == dense
    # more rows than batch * max_t, negative sizes, head_dim != 64
    assert B.whisper_enc_varlen_workspace_bytes(2, 3001, 1500, 1280, 20, 5120, P16) == 0
    assert B.whisper_enc_varlen_workspace_bytes(2, -1, 1500, 1280, 20, 5120, P16) == 0
    assert B.whisper_enc_varlen_workspace_bytes(2, 100, 1500, 1280, 10, 5120, P16) == 0

    def stack(x=FAKE, y=1 << 40, layers=FAKE, n_layers=2, cu=FAKE, batch=4, total=3000,
              max_t=1500, heads=20, ws=FAKE, wsb=1 << 34):
        return lib.whisper_enc_stack_forward_varlen(x, y, layers, n_layers, None, None, cu, batch,
                                                    total, max_t, 1280, heads, 5120, P16, ws,
                                                    wsb, None)

    assert stack(cu=None) == B.WENC_ERR_ARG
    assert stack(cu=FAKE + 2) == B.WENC_ERR_ARG
    assert stack(total=6001) == B.WENC_ERR_ARG
    assert stack(heads=10) == B.WENC_ERR_UNSUPPORTED
    assert stack(wsb=16) == B.WENC_ERR_WORKSPACE
    assert stack(y=FAKE + 4096) == B.WENC_ERR_ARG
    assert stack(x=None, y=None, cu=None, total=0, ws=None, wsb=0) == B.WENC_OK

    def attn(q=FAKE, cu=FAKE, batch=4, total=3000, max_t=1500, ld=3840, ldo=1280):
        return lib.whisper_enc_attention_varlen(q, q, q, q, cu, batch, total, max_t, 20, ld, ldo,
                                                P16, None)

    assert attn(cu=None) == B.WENC_ERR_ARG
    assert attn(total=6001) == B.WENC_ERR_ARG
    assert attn(ld=1000) == B.WENC_ERR_ARG
    assert attn(max_t=1 << 20) == B.WENC_ERR_UNSUPPORTED
    assert attn(q=None, cu=None, total=0) == B.WENC_OK


def test_quantized_paths_sizes_and_validation(lib):
    d, f = 1280, 5120
    fp16 = B.whisper_enc_layer_bytes(d, f, B.WENC_PATH_FP16)
    q8 = B.whisper_enc_layer_bytes(d, f, B.WENC_PATH_Q8)
    q4 = B.whisper_enc_layer_bytes(d, f, B.WENC_PATH_Q4)
    weights = 4 * d * d + 2 * d * f
    assert q8 >= weights * (1 + 1 / 16) and q8 < fp16 * 0.55
    assert q4 >= weights * (0.5 + 1 / 16) and q4 < fp16 * 0.3
    ws16 = B.whisper_enc_workspace_bytes(16, 1500, d, 20, f, B.WENC_PATH_FP16)
    assert B.whisper_enc_workspace_bytes(16, 1500, d, 20, f, B.WENC_PATH_Q8) >= ws16 + 2 * weights
    # the step-level entry points take operand types only
    assert lib.whisper_enc_linear(FAKE, FAKE, FAKE, None, FAKE, 64, 64, 64, B.WENC_PATH_Q8,
                                  B.WENC_EPI_BIAS, None) == B.WENC_ERR_ARG
    assert lib.whisper_enc_attention(FAKE, FAKE, FAKE, FAKE, 1, 64, 1, 192, 64, B.WENC_PATH_Q4,
                                     None) == B.WENC_ERR_ARG
    assert B.whisper_enc_stem_bytes(80, 384, 1500, B.WENC_PATH_Q8) == 0
    assert B.whisper_enc_cross_kv_bytes(384, 4, B.WENC_PATH_Q4) == 0
    q = lambda *a: lib.whisper_enc_quantize_matrix(*a)  # noqa: E731
    assert q(FAKE, FAKE, FAKE, 4, 64, 5, None) == B.WENC_ERR_ARG      # bits
    assert q(FAKE, FAKE, FAKE, 4, 48, 8, None) == B.WENC_ERR_ARG      # k % 32
    assert q(FAKE, FAKE, FAKE + 1, 4, 64, 8, None) == B.WENC_ERR_ARG  # scales alignment
    assert q(None, None, None, 0, 64, 4, None) == B.WENC_OK
    dq = lambda *a: lib.whisper_enc_dequantize_matrix(*a)  # noqa: E731
    assert dq(FAKE + 8, FAKE, FAKE, 4, 64, 8, None) == B.WENC_ERR_ARG
    assert dq(FAKE, FAKE, None, 4, 64, 4, None) == B.WENC_ERR_ARG


def test_mxfp8_sizes_and_validation(lib):
    """MXFP8 matrices: rows * k code bytes rounded up to 256, then k / 32 scale planes of rows
    rounded up to 16 bytes, the planes rounded up to 256.  An MXFP8 layer holds QKV, fc1 and fc2
    as MXFP8 matrices and the out-projection as fp16; its workspace is the fp16 path's (every
    MXFP8 activation fits the fp16 region it replaces).  The attention, front-end and cross K/V
    entry points do not take the MXFP8 path."""
    MX = B.WENC_PATH_MXFP8
    assert B.whisper_enc_mx_bytes(5, 32) == 256 + 256
    assert B.whisper_enc_mx_bytes(1500, 1280) == 1500 * 1280 + 40 * 1504  # both multiples of 256
    assert B.whisper_enc_mx_bytes(16, 64) == 1024 + 256
    for bad in [(-1, 64), (4, 48), (4, 0), (4, 1 << 17)]:
        assert B.whisper_enc_mx_bytes(*bad) == 0
    mxb = lambda r, k: B.whisper_enc_mx_bytes(r, k)  # noqa: E731
    rnd = lambda v: (v + 255) // 256 * 256  # noqa: E731
    for d, f in [(384, 1536), (1280, 5120), (512, 2048)]:
        fp32_sections = rnd(4 * d) * 6 + rnd(4 * 3 * d) + rnd(4 * f)  # LN, biases
        want = fp32_sections + mxb(3 * d, d) + rnd(2 * d * d) + mxb(f, d) + mxb(d, f)
        assert B.whisper_enc_layer_bytes(d, f, MX) == want, d
    for args in [(16, 1500, 1280, 20, 5120), (1, 1500, 384, 6, 1536), (3, 77, 512, 8, 2048)]:
        assert B.whisper_enc_workspace_bytes(*args, MX) == \
            B.whisper_enc_workspace_bytes(*args, B.WENC_PATH_FP16)
    assert lib.whisper_enc_attention(FAKE, FAKE, FAKE, FAKE, 1, 64, 1, 192, 64, MX, None) == \
        B.WENC_ERR_ARG
    assert B.whisper_enc_stem_bytes(80, 384, 1500, MX) == 0
    assert B.whisper_enc_cross_kv_bytes(384, 4, MX) == 0
    mq = lambda *a: lib.whisper_enc_mx_quantize(*a)  # noqa: E731
    assert mq(FAKE, FAKE + (1 << 24), 4, 48, None) == B.WENC_ERR_ARG      # k % 32
    assert mq(FAKE + 8, FAKE + (1 << 24), 4, 64, None) == B.WENC_ERR_ARG  # alignment
    assert mq(FAKE, FAKE + 256, 4, 64, None) == B.WENC_ERR_ARG            # dst overlaps src
    assert mq(None, FAKE, 4, 64, None) == B.WENC_ERR_ARG
    assert mq(None, None, 0, 64, None) == B.WENC_OK
    ln = lambda *a: lib.whisper_enc_layernorm(*a)  # noqa: E731
    assert ln(FAKE, FAKE, FAKE, FAKE + 512, 4, 64, B.WENC_DTYPE_MXFP8, None) == B.WENC_ERR_ARG
    assert ln(FAKE, FAKE, FAKE, FAKE, 4, 64, 4, None) == B.WENC_ERR_ARG  # no such dtype
    lin = lambda *a: lib.whisper_enc_linear(*a)  # noqa: E731
    assert lin(FAKE, FAKE, FAKE, None, FAKE, 64, 64, 48, MX, B.WENC_EPI_BIAS, None) == B.WENC_ERR_ARG
    assert lin(FAKE, FAKE, FAKE, None, FAKE, 1 << 24, 64, 256, MX, B.WENC_EPI_BIAS, None) == \
        B.WENC_ERR_UNSUPPORTED  # m * k >= 2^31
