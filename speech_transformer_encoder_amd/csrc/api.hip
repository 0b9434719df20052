// C ABI of the encoder-block library: argument validation, packed-layer and workspace layout,
// and the launch sequence of one block (inferencelayer whisper_gpu.rs,
// WhisperEncoderGpu::forward: LN, QKV, attention, out + add, LN, fc1 + GELU, fc2 + add, and
// the optional ln_post).  Everything is checked before the first launch so that a rejected
// call enqueues nothing and never touches HIP.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/whisper_enc.h"
#include "wenc_internal.h"

using namespace wenc;

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int path_dtype(int path) {
  switch (path) {
    case WENC_PATH_BF16: return DT_BF16;
    case WENC_PATH_FP16: return DT_F16;
    case WENC_PATH_FP32: return DT_F32;
    case WENC_PATH_MXFP8: return DT_MX8;
  }
  return -1;
}
// Operand type of the steps that have no MXFP8 form (attention, the conv front end, cross K/V).
int plain_dtype(int path) { return path == WENC_PATH_MXFP8 ? -1 : path_dtype(path); }

// MXFP8: the QKV, fc1 and fc2 projections on MXFP8 operands (weights quantised at pack time, the
// LayerNorm and GELU outputs by the kernels that produce them); attention and the
// out-projection, whose input is the attention output, stay fp16.
bool mx_path(int path) { return path == WENC_PATH_MXFP8; }

// BF16X2 / BF16X3: bf16 MFMA operands; the LayerNorm and GELU outputs that feed the QKV, fc1 and
// fc2 projections are bf16 hi / lo pairs, and on BF16X3 so are the weights.  Each projection then
// runs over k segments (KMap): x_hi w + x_lo w (X2); x_hi w_hi + x_lo w_hi + x_hi w_lo (X3; the
// out-projection, whose input is single bf16, x w_hi + x w_lo).
bool split_acts(int path) { return path == WENC_PATH_BF16X2 || path == WENC_PATH_BF16X3; }
bool split_weights(int path) { return path == WENC_PATH_BF16X3; }
int kmul(int path) { return split_acts(path) ? 2 : 1; }
// k segments of a projection whose activation is a LayerNorm or GELU output (QKV, fc1, fc2) ...
KMap kmap_split(int path, int kb) {
  if (split_weights(path)) return KMap{kb, 3, 0b010, 0b100, 2 * kb};
  if (split_acts(path)) return KMap{kb, 2, 0b10, 0, kb};
  return KMap{kb, 1, 0, 0, kb};
}
// ... and of the out-projection, whose activation (the attention output) is single.
KMap kmap_single(int path, int kb) {
  if (split_weights(path)) return KMap{kb, 2, 0, 0b10, 2 * kb};
  return KMap{kb, 1, 0, 0, kb};
}

size_t elem_bytes(int path) { return path == WENC_PATH_FP32 ? 4 : 2; }

// Weight storage of the q8 / q4 paths (0 for the others); their activations are fp16.
int quant_bits(int path) { return path == WENC_PATH_Q8 ? 8 : path == WENC_PATH_Q4 ? 4 : 0; }

// Operand type of a block or stack: the step-level entry points take path_dtype (no q8 / q4).
int layer_dtype(int path) {
  return quant_bits(path) ? DT_F16 : split_acts(path) ? DT_BF16 : path_dtype(path);
}
// Type of the LayerNorm outputs (the QKV and fc1 operands) of a block.
int ln_dtype(int path) { return split_acts(path) ? DT_BF16X2 : layer_dtype(path); }
// Operand type of attention and of the out-projection.
int attn_dtype(int path) { return mx_path(path) ? DT_F16 : layer_dtype(path); }

// Bytes of one stored [n][k] matrix: codes (int8 or nibbles) for q8 / q4, codes and scale planes
// for MXFP8, else operand values.
size_t matrix_bytes(size_t n, size_t k, int path) {
  const int bits = quant_bits(path);
  if (mx_path(path)) return mx_matrix_bytes(n, k);
  return bits ? n * k * bits / 8 : n * k * elem_bytes(path) * (split_weights(path) ? 2 : 1);
}
size_t scale_bytes(size_t n, size_t k, int path) { return quant_bits(path) ? n * (k / 32) * 2 : 0; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct LayerLayout {
  size_t ln1_g, ln1_b, bqkv, bo, ln2_g, ln2_b, b1, b2;  // fp32 sections
  size_t wqkv, wo, w1, w2;  // operand-type values, or q8 / q4 codes
  size_t sqkv, so, s1, s2;  // q8 / q4: fp16 scales [n][k / 32] (empty otherwise)
  size_t total;
};

LayerLayout layer_layout(int d, int f, int path) {
  LayerLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += round_up(bytes);
    return o;
  };
  L.ln1_g = take(4 * (size_t)d);
  L.ln1_b = take(4 * (size_t)d);
  L.bqkv = take(4 * 3 * (size_t)d);
  L.bo = take(4 * (size_t)d);
  L.ln2_g = take(4 * (size_t)d);
  L.ln2_b = take(4 * (size_t)d);
  L.b1 = take(4 * (size_t)f);
  L.b2 = take(4 * (size_t)d);
  L.wqkv = take(matrix_bytes(3 * (size_t)d, d, path));
  L.wo = take(mx_path(path) ? 2 * (size_t)d * d : matrix_bytes(d, d, path));  // MXFP8: fp16
  L.w1 = take(matrix_bytes(f, d, path));
  L.w2 = take(matrix_bytes(d, f, path));
  L.sqkv = take(scale_bytes(3 * (size_t)d, d, path));
  L.so = take(scale_bytes(d, d, path));
  L.s1 = take(scale_bytes(f, d, path));
  L.s2 = take(scale_bytes(d, f, path));
  L.total = off;
  return L;
}

bool valid_dims(int d, int f) {
  return d >= 64 && d <= WENC_MAX_D_MODEL && d % 64 == 0 && f >= 64 && f <= WENC_MAX_FFN_DIM &&
         f % 64 == 0;
}

// Shape check shared by workspace/block/stack: returns WENC_OK, ARG or UNSUPPORTED.
int check_shape(int batch, int t, int d, int heads, int f, int path) {
  if (layer_dtype(path) < 0) return WENC_ERR_ARG;
  if (batch < 0 || t < 0 || heads <= 0) return WENC_ERR_ARG;
  if ((long long)batch * t > WENC_MAX_ROWS) return WENC_ERR_ARG;
  if (!valid_dims(d, f)) return WENC_ERR_ARG;
  if (d % heads != 0) return WENC_ERR_ARG;
  if (d / heads != WENC_HEAD_DIM) return WENC_ERR_UNSUPPORTED;
  // One window's QKV rows must span less than 2 GiB: the attention kernel addresses them with
  // 32-bit buffer offsets.
  if ((size_t)t * 3 * d * elem_bytes(path) > (size_t)INT32_MAX) return WENC_ERR_UNSUPPORTED;
  return WENC_OK;
}

struct Workspace {
  void* a;  // [M, d]: LN outputs and the attention output
  void* b;  // [M, max(3d, f)]: QKV, then the FFN hidden activations
  float* part = nullptr;  // split-k parts of the residual GEMMs when M is small (else empty)
  uint16_t* wqkv = nullptr;  // q8 / q4: the block's weights expanded to fp16
  uint16_t* wo = nullptr;
  uint16_t* w1 = nullptr;
  uint16_t* w2 = nullptr;
};

// Bytes of the fp16 weights of one layer (q8 / q4 paths): [3d][d], [d][d], [f][d], [d][f].
size_t dequant_bytes(int d, int f, int path) {
  if (!quant_bits(path)) return 0;
  return round_up(2 * 3 * (size_t)d * d) + round_up(2 * (size_t)d * d) +
         2 * round_up(2 * (size_t)f * d);
}

// fp32 parts of the split-k residual GEMMs of a block (out-projection and fc2, both [M, d]).
size_t split_bytes(size_t rows, int d, int f, int path) {
  const KMap ko = kmap_single(path, d), k2 = kmap_split(path, f);
  const int s = std::max(
      linear_split((int)rows, d, ko.nseg * d, attn_dtype(path), EPI_BIAS_RESIDUAL),
      linear_split((int)rows, d, k2.nseg * f, layer_dtype(path), EPI_BIAS_RESIDUAL));
  return s > 1 ? round_up((size_t)s * rows * d * sizeof(float)) : 0;
}

// fp32 (O, m, l) of both key halves when attention splits its keys (few query blocks).
size_t attn_split_bytes(int batch, int t, int heads, size_t rows, int path) {
  if (attention_split(batch, t, heads, attn_dtype(path)) < 2) return 0;
  return round_up(2 * rows * (size_t)heads * 66 * sizeof(float));
}

// One scratch region serves both: attention's halves are merged before the out-projection runs.
size_t scratch_bytes(int batch, int t, int heads, size_t rows, int d, int f, int path) {
  return std::max(split_bytes(rows, d, f, path), attn_split_bytes(batch, t, heads, rows, path));
}

// rows: batch * t, or the packed rows of a ragged batch (t = its longest window).
// Widths (elements per row) of the two activation regions: a holds the LayerNorm outputs (hi /
// lo pairs on BF16X2) and the attention output; b the QKV projection and the FFN hidden layer.
size_t width_a(int d, int path) { return (size_t)kmul(path) * d; }
size_t width_b(int d, int f, int path) {
  const size_t fh = (size_t)kmul(path) * f;
  return 3 * (size_t)d > fh ? 3 * (size_t)d : fh;
}

// Bytes of the two activation regions (MXFP8: also room for the MXFP8 LayerNorm output in a and
// the MXFP8 hidden layer in b, which are at most a few scale planes larger than the fp16 ones).
size_t region_a_bytes(size_t rows, int d, int path) {
  const size_t b = round_up(rows * width_a(d, path) * elem_bytes(path));
  return mx_path(path) ? std::max(b, mx_matrix_bytes(rows, d)) : b;
}
size_t region_b_bytes(size_t rows, int d, int f, int path) {
  const size_t b = round_up(rows * width_b(d, f, path) * elem_bytes(path));
  return mx_path(path) ? std::max(b, mx_matrix_bytes(rows, f)) : b;
}

size_t workspace_size(int batch, int t, int heads, size_t rows, int d, int f, int path) {
  return region_a_bytes(rows, d, path) + region_b_bytes(rows, d, f, path) +
         dequant_bytes(d, f, path) + scratch_bytes(batch, t, heads, rows, d, f, path);
}

Workspace carve(void* ws, int batch, int t, int heads, size_t rows, int d, int f, int path) {
  Workspace w;
  const size_t ra = region_a_bytes(rows, d, path), rb = region_b_bytes(rows, d, f, path);
  char* p = static_cast<char*>(ws);
  w.a = p;
  w.b = p + ra;
  if (quant_bits(path)) {
    char* q = p + ra + rb;
    w.wqkv = reinterpret_cast<uint16_t*>(q);
    q += round_up(2 * 3 * (size_t)d * d);
    w.wo = reinterpret_cast<uint16_t*>(q);
    q += round_up(2 * (size_t)d * d);
    w.w1 = reinterpret_cast<uint16_t*>(q);
    q += round_up(2 * (size_t)f * d);
    w.w2 = reinterpret_cast<uint16_t*>(q);
  }
  if (scratch_bytes(batch, t, heads, rows, d, f, path))
    w.part = reinterpret_cast<float*>(p + ra + rb + dequant_bytes(d, f, path));
  return w;
}

#define WENC_TRY(expr)                       \
  do {                                       \
    if ((expr) != hipSuccess) return WENC_ERR_HIP; \
  } while (0)

// Enqueue one block; all arguments already validated.  cu: ragged-batch offsets or nullptr.
// ln1_ready: ws.a already holds LN1(x) (fused into the previous block's last pass).  next: the
// LayerNorm that reads this block's output (the next block's LN1, or the stack's final norm);
// when fc2 splits k it is fused into fc2's second pass and *next_done is set.  Where the
// out-projection splits k, LN2 is fused into its second pass the same way.
int run_block(const float* x, float* y, const char* blob, int rows, int t, int batch, int d,
              int heads, int f, int path, const Workspace& ws, hipStream_t st, const int* cu,
              bool ln1_ready, const LnFuse* next, bool* next_done) {
  *next_done = false;
  const LayerLayout L = layer_layout(d, f, path);
  const int dt = layer_dtype(path), da = attn_dtype(path);  // projections fed by LN / GELU; the rest
  const size_t es = elem_bytes(path);
  auto fp = [&](size_t off) { return reinterpret_cast<const float*>(blob + off); };
  const void* wqkv = blob + L.wqkv;
  const void* wo = blob + L.wo;
  const void* w1 = blob + L.w1;
  const void* w2 = blob + L.w2;
  char* qkv = static_cast<char*>(ws.b);
  if (const int bits = quant_bits(path)) {
    // Expand this layer's q8 / q4 matrices to fp16 in the workspace; the GEMMs read those.
    auto sc = [&](size_t off) { return reinterpret_cast<const uint16_t*>(blob + off); };
    DequantSegments seg{{blob + L.wqkv, blob + L.wo, blob + L.w1, blob + L.w2},
                        {sc(L.sqkv), sc(L.so), sc(L.s1), sc(L.s2)},
                        {ws.wqkv, ws.wo, ws.w1, ws.w2},
                        {3 * d, d, f, d},
                        {d, d, d, f},
                        4};
    WENC_TRY(launch_dequant(seg, bits, st));
    wqkv = ws.wqkv;
    wo = ws.wo;
    w1 = ws.w1;
    w2 = ws.w2;
  }

  // BF16X2 / X3: the LayerNorm and GELU outputs are hi / lo pairs (rows of 2 d / 2 f), and each
  // projection runs over its k segments (kmap_split / kmap_single).
  const int lt = ln_dtype(path), km = kmul(path);
  const KMap kq = kmap_split(path, d), ko = kmap_single(path, d), k1 = kmap_split(path, d),
             k2 = kmap_split(path, f);
  if (!ln1_ready)
    WENC_TRY(launch_layernorm(x, fp(L.ln1_g), fp(L.ln1_b), ws.a, rows, d, lt, st));
  WENC_TRY(launch_linear(ws.a, km * d, wqkv, fp(L.bqkv), nullptr, qkv, 3 * d, rows, 3 * d,
                         kq.nseg * d, dt, EPI_BIAS, st, nullptr, nullptr, &kq));
  WENC_TRY(launch_attention(qkv, qkv + es * d, qkv + es * 2 * d, 3 * d, ws.a, d, batch, t, heads,
                            0.125f, da, st, cu, rows, ws.part));
  if (ws.part && linear_split(rows, d, ko.nseg * d, da, EPI_BIAS_RESIDUAL) > 1) {
    const LnFuse ln2{fp(L.ln2_g), fp(L.ln2_b), ws.a, lt, true};
    WENC_TRY(launch_linear(ws.a, d, wo, fp(L.bo), x, y, d, rows, d, ko.nseg * d, da,
                           EPI_BIAS_RESIDUAL, st, ws.part, &ln2, &ko));
  } else {
    WENC_TRY(launch_linear(ws.a, d, wo, fp(L.bo), x, y, d, rows, d, ko.nseg * d, da,
                           EPI_BIAS_RESIDUAL, st, ws.part, nullptr, &ko));
    WENC_TRY(launch_layernorm(y, fp(L.ln2_g), fp(L.ln2_b), ws.a, rows, d, lt, st));
  }
  WENC_TRY(launch_linear(ws.a, km * d, w1, fp(L.b1), nullptr, ws.b, km * f, rows, f, k1.nseg * d,
                         dt, km > 1 ? EPI_BIAS_GELU_X2 : EPI_BIAS_GELU, st, nullptr, nullptr,
                         &k1));
  const bool fuse_next =
      next && ws.part && linear_split(rows, d, k2.nseg * f, dt, EPI_BIAS_RESIDUAL) > 1;
  WENC_TRY(launch_linear(ws.b, km * f, w2, fp(L.b2), y, y, d, rows, d, k2.nseg * f, dt,
                         EPI_BIAS_RESIDUAL, st, ws.part, fuse_next ? next : nullptr, &k2));
  *next_done = fuse_next;
  return WENC_OK;
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + bbytes && pb < pa + abytes;
}

bool overlaps_partially(const void* a, const void* b, size_t bytes) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  if (pa == pb) return false;
  return pa < pb + bytes && pb < pa + bytes;
}

}  // namespace

extern "C" {

const char* whisper_enc_strerror(int code) {
  switch (code) {
    case WENC_OK: return "ok";
    case WENC_ERR_ARG: return "invalid argument (null or misaligned pointer, bad size or enum)";
    case WENC_ERR_UNSUPPORTED: return "unsupported shape (head_dim must be 64)";
    case WENC_ERR_WORKSPACE: return "workspace too small";
    case WENC_ERR_HIP: return "HIP launch error";
    case WENC_ERR_SCRATCH:
      return "shape needs more workspace than the no-alloc entry point's static scratch "
             "(WENC_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status code";
}

size_t whisper_enc_layer_bytes(int d_model, int ffn_dim, int path) {
  if (layer_dtype(path) < 0 || !valid_dims(d_model, ffn_dim)) return 0;
  return layer_layout(d_model, ffn_dim, path).total;
}

int whisper_enc_pack_layer(const float* ln1_g, const float* ln1_b, const float* wq,
                           const float* bq, const float* wk, const float* bk, const float* wv,
                           const float* bv, const float* wo, const float* bo,
                           const float* ln2_g, const float* ln2_b, const float* w1,
                           const float* b1, const float* w2, const float* b2, int d_model,
                           int ffn_dim, int path, void* dst_layer, void* stream) {
  if (layer_dtype(path) < 0 || !valid_dims(d_model, ffn_dim)) return WENC_ERR_ARG;
  const float* req[] = {ln1_g, ln1_b, wq, bq, wk, wv, bv, wo, bo, ln2_g, ln2_b, w1, b1, w2, b2};
  for (const float* p : req)
    if (!p) return WENC_ERR_ARG;
  if (!dst_layer || !aligned(dst_layer, kAlign)) return WENC_ERR_ARG;

  const int d = d_model, f = ffn_dim, dt = layer_dtype(path);
  const size_t dd = (size_t)d * d;
  const LayerLayout L = layer_layout(d, f, path);
  const size_t es = elem_bytes(path);
  const int bits = quant_bits(path);
  char* blob = static_cast<char*>(dst_layer);
  auto fo = [&](size_t off) { return reinterpret_cast<float*>(blob + off); };
  hipStream_t st = static_cast<hipStream_t>(stream);

  WENC_TRY(launch_copy_or_zero(ln1_g, fo(L.ln1_g), d, st));
  WENC_TRY(launch_copy_or_zero(ln1_b, fo(L.ln1_b), d, st));
  WENC_TRY(launch_copy_or_zero(bq, fo(L.bqkv), d, st));
  WENC_TRY(launch_copy_or_zero(bk, fo(L.bqkv) + d, d, st));
  WENC_TRY(launch_copy_or_zero(bv, fo(L.bqkv) + 2 * d, d, st));
  WENC_TRY(launch_copy_or_zero(bo, fo(L.bo), d, st));
  WENC_TRY(launch_copy_or_zero(ln2_g, fo(L.ln2_g), d, st));
  WENC_TRY(launch_copy_or_zero(ln2_b, fo(L.ln2_b), d, st));
  WENC_TRY(launch_copy_or_zero(b1, fo(L.b1), f, st));
  WENC_TRY(launch_copy_or_zero(b2, fo(L.b2), d, st));
  if (bits) {
    // q8 / q4: codes and fp16 scales; Q, K and V fill rows 0, d and 2d of the fused [3d][d].
    const size_t crow = (size_t)d * bits / 8, srow = (size_t)(d / 32) * 2;  // bytes per row
    for (int i = 0; i < 3; ++i)
      WENC_TRY(launch_quantize(i == 0 ? wq : i == 1 ? wk : wv, blob + L.wqkv + i * d * crow,
                               blob + L.sqkv + i * d * srow, d, d, bits, st));
    WENC_TRY(launch_quantize(wo, blob + L.wo, blob + L.so, d, d, bits, st));
    WENC_TRY(launch_quantize(w1, blob + L.w1, blob + L.s1, f, d, bits, st));
    WENC_TRY(launch_quantize(w2, blob + L.w2, blob + L.s2, d, f, bits, st));
    return WENC_OK;
  }
  if (mx_path(path)) {
    // MXFP8 codes and scale planes; Q, K and V fill rows 0, d and 2d of the fused [3d][d]; the
    // out-projection in fp16.
    for (int i = 0; i < 3; ++i)
      WENC_TRY(launch_mx_quantize(i == 0 ? wq : i == 1 ? wk : wv, blob + L.wqkv, d, d, i * d, 3 * d,
                                  st));
    WENC_TRY(launch_convert(wo, blob + L.wo, dd, DT_F16, st));
    WENC_TRY(launch_mx_quantize(w1, blob + L.w1, f, d, 0, f, st));
    WENC_TRY(launch_mx_quantize(w2, blob + L.w2, d, f, 0, d, st));
    return WENC_OK;
  }
  if (split_weights(path)) {
    // BF16X3: every row as a bf16 [hi | lo] pair (rows of 2 n_in)
    WENC_TRY(launch_convert_split(wq, blob + L.wqkv, d, d, st));
    WENC_TRY(launch_convert_split(wk, blob + L.wqkv + 2 * es * dd, d, d, st));
    WENC_TRY(launch_convert_split(wv, blob + L.wqkv + 4 * es * dd, d, d, st));
    WENC_TRY(launch_convert_split(wo, blob + L.wo, d, d, st));
    WENC_TRY(launch_convert_split(w1, blob + L.w1, f, d, st));
    WENC_TRY(launch_convert_split(w2, blob + L.w2, d, f, st));
    return WENC_OK;
  }
  WENC_TRY(launch_convert(wq, blob + L.wqkv, dd, dt, st));
  WENC_TRY(launch_convert(wk, blob + L.wqkv + es * dd, dd, dt, st));
  WENC_TRY(launch_convert(wv, blob + L.wqkv + es * 2 * dd, dd, dt, st));
  WENC_TRY(launch_convert(wo, blob + L.wo, dd, dt, st));
  WENC_TRY(launch_convert(w1, blob + L.w1, (size_t)f * d, dt, st));
  WENC_TRY(launch_convert(w2, blob + L.w2, (size_t)d * f, dt, st));
  return WENC_OK;
}

size_t whisper_enc_workspace_bytes(int batch, int t, int d_model, int heads, int ffn_dim,
                                   int path) {
  if (check_shape(batch, t, d_model, heads, ffn_dim, path) != WENC_OK) return 0;
  return workspace_size(batch, t, heads, (size_t)batch * t, d_model, ffn_dim, path);
}

}  // extern "C"

namespace {

// Pointer and count checks of a stack call (shapes already checked).
int check_stack_args(const float* x, const float* y, const void* layers, int n_layers,
                     const float* ln_post_g, const float* ln_post_b, size_t rows, int d_model) {
  if (n_layers < 0) return WENC_ERR_ARG;
  if ((ln_post_g == nullptr) != (ln_post_b == nullptr)) return WENC_ERR_ARG;
  if (rows == 0) return WENC_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return WENC_ERR_ARG;
  if (overlaps_partially(x, y, rows * d_model * sizeof(float))) return WENC_ERR_ARG;
  if (ln_post_g && (!aligned(ln_post_g, 16) || !aligned(ln_post_b, 16))) return WENC_ERR_ARG;
  if (n_layers > 0 && (!layers || !aligned(layers, kAlign))) return WENC_ERR_ARG;
  return WENC_OK;
}

// Stack over `rows` rows: equal windows of t (cu == nullptr) or a ragged batch (t = longest
// window); shapes already checked.
int stack_impl(const float* x, float* y, const void* layers, int n_layers, const float* ln_post_g,
               const float* ln_post_b, const int* cu, int batch, size_t rows, int t, int d_model,
               int heads, int ffn_dim, int path, void* workspace, size_t workspace_bytes,
               void* stream) {
  int rc = check_stack_args(x, y, layers, n_layers, ln_post_g, ln_post_b, rows, d_model);
  if (rc != WENC_OK || rows == 0) return rc;
  const size_t xbytes = rows * d_model * sizeof(float);
  if (n_layers > 0) {
    if (!workspace || !aligned(workspace, kAlign)) return WENC_ERR_ARG;
    if (workspace_bytes < workspace_size(batch, t, heads, rows, d_model, ffn_dim, path))
      return WENC_ERR_WORKSPACE;
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t lb = layer_layout(d_model, ffn_dim, path).total;
  const Workspace ws = carve(workspace, batch, t, heads, rows, d_model, ffn_dim, path);
  const float* src = x;
  const LayerLayout L = layer_layout(d_model, ffn_dim, path);
  const int dt = layer_dtype(path);
  bool ln1_ready = false, post_done = false;
  for (int l = 0; l < n_layers; ++l) {
    // The LayerNorm that reads this block's output: the next block's LN1 (into the workspace's
    // operand buffer) or the final norm (into y, the block output itself not kept).
    const char* blob = static_cast<const char*>(layers) + (size_t)l * lb;
    LnFuse next{nullptr, nullptr, nullptr, 0, true};
    if (l + 1 < n_layers) {
      const char* nb = blob + lb;
      next = {reinterpret_cast<const float*>(nb + L.ln1_g),
              reinterpret_cast<const float*>(nb + L.ln1_b), ws.a, ln_dtype(path), true};
    } else if (ln_post_g) {
      next = {ln_post_g, ln_post_b, y, DT_F32, false};
    }
    bool done = false;
    rc = run_block(src, y, blob, (int)rows, t, batch, d_model, heads, ffn_dim, path, ws, st, cu,
                   ln1_ready, next.gamma ? &next : nullptr, &done);
    if (rc != WENC_OK) return rc;
    ln1_ready = done && l + 1 < n_layers;
    post_done = done && l + 1 == n_layers;
    src = y;
  }
  if (ln_post_g && !post_done) {
    WENC_TRY(launch_layernorm(src, ln_post_g, ln_post_b, y, (int)rows, d_model, DT_F32, st));
  } else if (!ln_post_g && src != y) {
    WENC_TRY(hipMemcpyAsync(y, src, xbytes, hipMemcpyDeviceToDevice, st));
  }
  return WENC_OK;
}

// Shape check of a ragged batch: `batch` windows packed into total_rows rows, none longer than
// max_t (same per-window limits as check_shape with t = max_t).
int check_varlen(int batch, int total_rows, int max_t, int d, int heads, int f, int path) {
  if (batch < 0 || total_rows < 0 || max_t < 0 || total_rows > WENC_MAX_ROWS) return WENC_ERR_ARG;
  if ((long long)batch * max_t < total_rows) return WENC_ERR_ARG;
  return check_shape(1, max_t, d, heads, f, path);
}

}  // namespace

extern "C" {

int whisper_enc_stack_forward(const float* x, float* y, const void* layers, int n_layers,
                              const float* ln_post_g, const float* ln_post_b, int batch, int t,
                              int d_model, int heads, int ffn_dim, int path, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const int rc = check_shape(batch, t, d_model, heads, ffn_dim, path);
  if (rc != WENC_OK) return rc;
  return stack_impl(x, y, layers, n_layers, ln_post_g, ln_post_b, nullptr, batch,
                    (size_t)batch * t, t, d_model, heads, ffn_dim, path, workspace,
                    workspace_bytes, stream);
}

size_t whisper_enc_varlen_workspace_bytes(int batch, int total_rows, int max_t, int d_model,
                                          int heads, int ffn_dim, int path) {
  if (check_varlen(batch, total_rows, max_t, d_model, heads, ffn_dim, path) != WENC_OK) return 0;
  return workspace_size(batch, max_t, heads, (size_t)total_rows, d_model, ffn_dim, path);
}

int whisper_enc_stack_forward_varlen(const float* x, float* y, const void* layers, int n_layers,
                                     const float* ln_post_g, const float* ln_post_b,
                                     const int* cu_seqlens, int batch, int total_rows, int max_t,
                                     int d_model, int heads, int ffn_dim, int path,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_varlen(batch, total_rows, max_t, d_model, heads, ffn_dim, path);
  if (rc != WENC_OK) return rc;
  if (total_rows > 0 && n_layers > 0 && (!cu_seqlens || !aligned(cu_seqlens, 4)))
    return WENC_ERR_ARG;
  return stack_impl(x, y, layers, n_layers, ln_post_g, ln_post_b, cu_seqlens, batch,
                    (size_t)total_rows, max_t, d_model, heads, ffn_dim, path, workspace,
                    workspace_bytes, stream);
}

int whisper_enc_block_forward(const float* x, float* y, const void* layer, int batch, int t,
                              int d_model, int heads, int ffn_dim, int path, void* workspace,
                              size_t workspace_bytes, void* stream) {
  int rc = check_shape(batch, t, d_model, heads, ffn_dim, path);
  if (rc != WENC_OK) return rc;
  if ((size_t)batch * t == 0) return WENC_OK;
  if (!layer) return WENC_ERR_ARG;
  return whisper_enc_stack_forward(x, y, layer, 1, nullptr, nullptr, batch, t, d_model, heads,
                                   ffn_dim, path, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- The stack without a caller workspace, for callers that cannot allocate. ----
//
// The workspace lives in a static device array of WENC_NOALLOC_SCRATCH_BYTES (one copy per GPU,
// held until the process ends).  In host code the array's name stands for a host-side shadow,
// not a device address, so the address every kernel receives is the one hipGetSymbolAddress
// returns for the current device, looked up once per device and kept.  No kernel of the block
// reads workspace memory it has not written in the same call, so nothing needs clearing
// between calls; calls that overlap on one GPU share the array and race.

namespace {

constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[WENC_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on first use).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return WENC_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return WENC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return WENC_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WENC_OK;
}

}  // namespace

extern "C" {

int whisper_enc_stack_forward_noalloc(const float* x, float* y, const void* layers, int n_layers,
                                      const float* ln_post_g, const float* ln_post_b, int batch,
                                      int t, int d_model, int heads, int ffn_dim, int path,
                                      void* stream) {
  int rc = check_shape(batch, t, d_model, heads, ffn_dim, path);
  if (rc != WENC_OK) return rc;
  const size_t rows = (size_t)batch * t;
  rc = check_stack_args(x, y, layers, n_layers, ln_post_g, ln_post_b, rows, d_model);
  if (rc != WENC_OK || rows == 0) return rc;
  if (n_layers > 0 && workspace_size(batch, t, heads, rows, d_model, ffn_dim, path) >
                          (size_t)WENC_NOALLOC_SCRATCH_BYTES)
    return WENC_ERR_SCRATCH;
  void* ws = nullptr;
  if (n_layers > 0) {  // every argument is valid: now look up the device's scratch
    rc = scratch_of_current_device(&ws);
    if (rc != WENC_OK) return rc;
  }
  return stack_impl(x, y, layers, n_layers, ln_post_g, ln_post_b, nullptr, batch, rows, t,
                    d_model, heads, ffn_dim, path, ws, ws ? (size_t)WENC_NOALLOC_SCRATCH_BYTES : 0,
                    stream);
}

int whisper_enc_layernorm(const float* x, const float* gamma, const float* beta, void* y,
                          int rows, int d, int out_dtype, void* stream) {
  if (rows < 0 || rows > WENC_MAX_ROWS) return WENC_ERR_ARG;
  if (d < 64 || d > WENC_MAX_D_MODEL || d % 64 != 0) return WENC_ERR_ARG;
  if (out_dtype != WENC_DTYPE_F32 && out_dtype != WENC_DTYPE_BF16 && out_dtype != WENC_DTYPE_F16 &&
      out_dtype != WENC_DTYPE_MXFP8)
    return WENC_ERR_ARG;
  if (rows == 0) return WENC_OK;
  if (!x || !gamma || !beta || !y) return WENC_ERR_ARG;
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(beta, 16) || !aligned(y, 16))
    return WENC_ERR_ARG;
  const size_t xbytes = (size_t)rows * d * sizeof(float);
  if (out_dtype == WENC_DTYPE_F32) {
    if (overlaps_partially(x, y, xbytes)) return WENC_ERR_ARG;  // in place (y == x) is allowed
  } else {
    // A 16-bit or MXFP8 y must not overlap x at all.
    const size_t ybytes = out_dtype == WENC_DTYPE_MXFP8 ? mx_matrix_bytes(rows, d)
                                                         : (size_t)rows * d * 2;
    if (overlaps(x, xbytes, y, ybytes)) return WENC_ERR_ARG;
  }
  const int dt = out_dtype == WENC_DTYPE_F32    ? DT_F32
                 : out_dtype == WENC_DTYPE_BF16 ? DT_BF16
                 : out_dtype == WENC_DTYPE_F16  ? DT_F16
                                                : DT_MX8;
  WENC_TRY(launch_layernorm(x, gamma, beta, y, rows, d, dt, static_cast<hipStream_t>(stream)));
  return WENC_OK;
}

int whisper_enc_linear(const void* a, const void* w, const float* bias, const float* residual,
                       void* c, int m, int n, int k, int path, int epilogue, void* stream) {
  const int dt = path_dtype(path);
  if (dt < 0) return WENC_ERR_ARG;
  if (epilogue != WENC_EPI_BIAS && epilogue != WENC_EPI_BIAS_GELU &&
      epilogue != WENC_EPI_BIAS_RESIDUAL && epilogue != WENC_EPI_BIAS_GELU_RESIDUAL)
    return WENC_ERR_ARG;
  const bool fp32_out = epilogue == WENC_EPI_BIAS_RESIDUAL || epilogue == WENC_EPI_BIAS_GELU_RESIDUAL;
  if (m < 0 || m > WENC_MAX_ROWS || n < 64 || k < 64 || n % 64 || k % 64 || n > WENC_MAX_FFN_DIM ||
      k > WENC_MAX_FFN_DIM)
    return WENC_ERR_ARG;
  if (m == 0) return WENC_OK;
  if (!a || !w || !bias || !c) return WENC_ERR_ARG;
  if (fp32_out && !residual) return WENC_ERR_ARG;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(bias, 16) || !aligned(c, 16) ||
      (residual && !aligned(residual, 16)))
    return WENC_ERR_ARG;
  if (fp32_out && overlaps_partially(residual, c, (size_t)m * n * sizeof(float)))
    return WENC_ERR_ARG;
  if (dt == DT_MX8 && ((size_t)m * k > (size_t)INT32_MAX || (size_t)n * k > (size_t)INT32_MAX))
    return WENC_ERR_UNSUPPORTED;  // 32-bit buffer offsets of the operand rows
  const int epi = epilogue == WENC_EPI_BIAS        ? EPI_BIAS
                  : epilogue == WENC_EPI_BIAS_GELU ? EPI_BIAS_GELU
                  : epilogue == WENC_EPI_BIAS_RESIDUAL ? EPI_BIAS_RESIDUAL
                                                       : EPI_BIAS_GELU_RESIDUAL;
  WENC_TRY(launch_linear(a, k, w, bias, residual, c, n, m, n, k, dt, epi,
                         static_cast<hipStream_t>(stream)));
  return WENC_OK;
}

int whisper_enc_attention(const void* q, const void* k, const void* v, void* o, int batch, int t,
                          int heads, int ld_qkv, int ld_o, int path, void* stream) {
  const int dt = plain_dtype(path);
  if (dt < 0) return WENC_ERR_ARG;
  if (batch < 0 || t < 0 || heads <= 0 || (long long)batch * t > WENC_MAX_ROWS) return WENC_ERR_ARG;
  if (heads * WENC_HEAD_DIM > WENC_MAX_FFN_DIM) return WENC_ERR_ARG;
  if (ld_qkv < heads * WENC_HEAD_DIM || ld_o < heads * WENC_HEAD_DIM || ld_qkv % 8 || ld_o % 8)
    return WENC_ERR_ARG;
  if ((size_t)t * ld_qkv * elem_bytes(path) > (size_t)INT32_MAX) return WENC_ERR_UNSUPPORTED;
  if ((size_t)batch * t == 0) return WENC_OK;
  if (!q || !k || !v || !o) return WENC_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return WENC_ERR_ARG;
  WENC_TRY(launch_attention(q, k, v, ld_qkv, o, ld_o, batch, t, heads, 0.125f, dt,
                            static_cast<hipStream_t>(stream)));
  return WENC_OK;
}

int whisper_enc_attention_varlen(const void* q, const void* k, const void* v, void* o,
                                 const int* cu_seqlens, int batch, int total_rows, int max_t,
                                 int heads, int ld_qkv, int ld_o, int path, void* stream) {
  const int dt = plain_dtype(path);
  if (dt < 0) return WENC_ERR_ARG;
  if (batch < 0 || total_rows < 0 || max_t < 0 || heads <= 0 || total_rows > WENC_MAX_ROWS)
    return WENC_ERR_ARG;
  if ((long long)batch * max_t < total_rows) return WENC_ERR_ARG;
  if (heads * WENC_HEAD_DIM > WENC_MAX_FFN_DIM) return WENC_ERR_ARG;
  if (ld_qkv < heads * WENC_HEAD_DIM || ld_o < heads * WENC_HEAD_DIM || ld_qkv % 8 || ld_o % 8)
    return WENC_ERR_ARG;
  if ((size_t)max_t * ld_qkv * elem_bytes(path) > (size_t)INT32_MAX) return WENC_ERR_UNSUPPORTED;
  if (total_rows == 0) return WENC_OK;
  if (!q || !k || !v || !o || !cu_seqlens) return WENC_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(cu_seqlens, 4))
    return WENC_ERR_ARG;
  WENC_TRY(launch_attention(q, k, v, ld_qkv, o, ld_o, batch, max_t, heads, 0.125f, dt,
                            static_cast<hipStream_t>(stream), cu_seqlens, total_rows));
  return WENC_OK;
}

}  // extern "C"

// ---- Cross-attention keys and values of the decoder layers (turbospark-runtime
// build_cross_caches; oxinfer cross_kv): one projection of the encoder output through the packed
// [2 L d, d] weights, written head-major. ----

namespace {

struct CrossLayout {
  size_t bias, w, total;
};

CrossLayout cross_layout(int d, int n_layers, int path) {
  CrossLayout L;
  const size_t rows = 2 * (size_t)n_layers * d;
  L.bias = 0;
  L.w = round_up(rows * sizeof(float));
  L.total = L.w + round_up(rows * d * elem_bytes(path));
  return L;
}

bool valid_cross(int d, int n_layers, int path) {
  return plain_dtype(path) >= 0 && d >= 64 && d <= WENC_MAX_D_MODEL && d % 64 == 0 &&
         n_layers >= 1 && n_layers <= WENC_MAX_DEC_LAYERS;
}

}  // namespace

extern "C" {

size_t whisper_enc_cross_kv_bytes(int d_model, int n_dec_layers, int path) {
  if (!valid_cross(d_model, n_dec_layers, path)) return 0;
  return cross_layout(d_model, n_dec_layers, path).total;
}

int whisper_enc_pack_cross_kv(const float* const* wk, const float* const* wv,
                              const float* const* bv, int n_dec_layers, int d_model, int path,
                              void* dst, void* stream) {
  if (!valid_cross(d_model, n_dec_layers, path)) return WENC_ERR_ARG;
  if (!wk || !wv || !bv || !dst || !aligned(dst, kAlign)) return WENC_ERR_ARG;
  for (int l = 0; l < n_dec_layers; ++l)
    if (!wk[l] || !wv[l] || !bv[l]) return WENC_ERR_ARG;
  const int d = d_model, dt = plain_dtype(path);
  const size_t dd = (size_t)d * d, es = elem_bytes(path);
  const CrossLayout L = cross_layout(d, n_dec_layers, path);
  char* blob = static_cast<char*>(dst);
  float* bias = reinterpret_cast<float*>(blob + L.bias);
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int l = 0; l < n_dec_layers; ++l) {
    WENC_TRY(launch_copy_or_zero(nullptr, bias + (size_t)(2 * l) * d, d, st));  // K: no bias
    WENC_TRY(launch_copy_or_zero(bv[l], bias + (size_t)(2 * l + 1) * d, d, st));
    WENC_TRY(launch_convert(wk[l], blob + L.w + es * (size_t)(2 * l) * dd, dd, dt, st));
    WENC_TRY(launch_convert(wv[l], blob + L.w + es * (size_t)(2 * l + 1) * dd, dd, dt, st));
  }
  return WENC_OK;
}

size_t whisper_enc_cross_kv_workspace_bytes(int batch, int t, int d_model, int path) {
  if (plain_dtype(path) < 0 || batch < 0 || t < 0 || (long long)batch * t > WENC_MAX_ROWS ||
      d_model < 64 || d_model > WENC_MAX_D_MODEL || d_model % 64)
    return 0;
  if (path == WENC_PATH_FP32) return kAlign;  // the fp32 path reads y directly
  return round_up((size_t)batch * t * d_model * elem_bytes(path));
}

int whisper_enc_cross_kv(const float* y, void* kv, const void* wkv, int n_dec_layers, int batch,
                         int t, int d_model, int heads, int path, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!valid_cross(d_model, n_dec_layers, path)) return WENC_ERR_ARG;
  if (batch < 0 || t < 0 || heads <= 0 || (long long)batch * t > WENC_MAX_ROWS) return WENC_ERR_ARG;
  if (d_model % heads != 0) return WENC_ERR_ARG;
  if (d_model / heads != WENC_HEAD_DIM) return WENC_ERR_UNSUPPORTED;
  const size_t rows = (size_t)batch * t;
  if (rows == 0) return WENC_OK;
  if (!y || !kv || !wkv || !workspace) return WENC_ERR_ARG;
  if (!aligned(y, 16) || !aligned(kv, 16) || !aligned(wkv, kAlign) || !aligned(workspace, kAlign))
    return WENC_ERR_ARG;
  if (workspace_bytes < whisper_enc_cross_kv_workspace_bytes(batch, t, d_model, path))
    return WENC_ERR_WORKSPACE;
  const int d = d_model, dt = plain_dtype(path);
  const int n = 2 * n_dec_layers * d;
  const CrossLayout L = cross_layout(d, n_dec_layers, path);
  const char* blob = static_cast<const char*>(wkv);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const void* a = y;
  if (path != WENC_PATH_FP32) {
    WENC_TRY(launch_convert(y, workspace, rows * d, dt, st));
    a = workspace;
  }
  WENC_TRY(launch_linear(a, d, blob + L.w, reinterpret_cast<const float*>(blob + L.bias), nullptr,
                         kv, t, (int)rows, n, d, dt, EPI_BIAS_HEADMAJOR, st));
  return WENC_OK;
}

}  // extern "C"

// ---- Conv front end (oxinfer WhisperModel::encode, conv1 / conv2 / positions; turbospark-runtime
// encode_partial): unfold, GEMM + GELU, unfold with stride 2, GEMM + GELU + positions. ----

namespace {

int stem_k1(int n_mels) { return (3 * n_mels + 63) / 64 * 64; }

struct StemLayout {
  size_t b1, b2, pos, w1, w2, total;
};

StemLayout stem_layout(int n_mels, int d, int n_pos, int path) {
  StemLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += round_up(bytes);
    return o;
  };
  const size_t es = elem_bytes(path);
  L.b1 = take(4 * (size_t)d);
  L.b2 = take(4 * (size_t)d);
  L.pos = take(4 * (size_t)n_pos * d);
  L.w1 = take(es * (size_t)d * stem_k1(n_mels));
  L.w2 = take(es * (size_t)d * 3 * d);
  L.total = off;
  return L;
}

bool valid_stem(int n_mels, int d, int n_pos, int path) {
  return plain_dtype(path) >= 0 && n_mels >= 1 && n_mels <= WENC_MAX_MELS && d >= 64 &&
         d <= WENC_MAX_D_MODEL && d % 64 == 0 && n_pos >= 1 && n_pos <= WENC_MAX_ROWS;
}

struct StemWorkspace {
  void* cols1;  // [B t, k1]
  void* h;      // [B t, d]
  void* cols2;  // [B t2, 3 d]
  size_t total;
};

StemWorkspace stem_workspace(void* base, size_t batch, int t, int n_mels, int d, int path) {
  const size_t es = elem_bytes(path);
  const size_t t2 = (size_t)(t + 1) / 2;
  StemWorkspace w;
  char* p = static_cast<char*>(base);
  const size_t a = round_up(batch * t * stem_k1(n_mels) * es);
  const size_t b = round_up(batch * t * d * es);
  const size_t c = round_up(batch * t2 * 3 * d * es);
  w.cols1 = p;
  w.h = p ? p + a : nullptr;
  w.cols2 = p ? p + a + b : nullptr;
  w.total = a + b + c;
  return w;
}

}  // namespace

extern "C" {

size_t whisper_enc_stem_bytes(int n_mels, int d_model, int n_pos, int path) {
  if (!valid_stem(n_mels, d_model, n_pos, path)) return 0;
  return stem_layout(n_mels, d_model, n_pos, path).total;
}

int whisper_enc_pack_stem(const float* conv1_w, const float* conv1_b, const float* conv2_w,
                          const float* conv2_b, const float* pos, int n_mels, int d_model,
                          int n_pos, int path, void* dst, void* stream) {
  if (!valid_stem(n_mels, d_model, n_pos, path)) return WENC_ERR_ARG;
  if (!conv1_w || !conv1_b || !conv2_w || !conv2_b || !pos) return WENC_ERR_ARG;
  if (!dst || !aligned(dst, kAlign)) return WENC_ERR_ARG;
  const int d = d_model, dt = plain_dtype(path);
  const StemLayout L = stem_layout(n_mels, d, n_pos, path);
  char* blob = static_cast<char*>(dst);
  hipStream_t st = static_cast<hipStream_t>(stream);
  WENC_TRY(launch_copy_or_zero(conv1_b, reinterpret_cast<float*>(blob + L.b1), d, st));
  WENC_TRY(launch_copy_or_zero(conv2_b, reinterpret_cast<float*>(blob + L.b2), d, st));
  WENC_TRY(launch_copy_or_zero(pos, reinterpret_cast<float*>(blob + L.pos), (size_t)n_pos * d, st));
  WENC_TRY(launch_pack_conv(conv1_w, blob + L.w1, d, n_mels, stem_k1(n_mels), dt, st));
  WENC_TRY(launch_pack_conv(conv2_w, blob + L.w2, d, d, 3 * d, dt, st));
  return WENC_OK;
}

size_t whisper_enc_stem_workspace_bytes(int batch, int t_mel, int n_mels, int d_model, int path) {
  if (!valid_stem(n_mels, d_model, 1, path) || batch < 0 || t_mel < 0 ||
      (long long)batch * t_mel > WENC_MAX_ROWS)
    return 0;
  return stem_workspace(nullptr, (size_t)batch, t_mel, n_mels, d_model, path).total;
}

int whisper_enc_stem_forward(const float* mel, float* x, const void* stem, int batch, int t_mel,
                             int n_mels, int d_model, int n_pos, int path, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!valid_stem(n_mels, d_model, n_pos, path)) return WENC_ERR_ARG;
  if (batch < 0 || t_mel < 0 || (long long)batch * t_mel > WENC_MAX_ROWS) return WENC_ERR_ARG;
  const int t2 = (t_mel + 1) / 2;
  if (t2 > n_pos) return WENC_ERR_ARG;
  if ((size_t)batch * t_mel == 0) return WENC_OK;
  if (!mel || !x || !stem || !workspace) return WENC_ERR_ARG;
  if (!aligned(mel, 16) || !aligned(x, 16) || !aligned(stem, kAlign) || !aligned(workspace, kAlign))
    return WENC_ERR_ARG;
  {
    const uintptr_t pm = (uintptr_t)mel, px = (uintptr_t)x;
    const size_t mel_bytes = (size_t)batch * t_mel * n_mels * sizeof(float);
    const size_t x_bytes = (size_t)batch * t2 * d_model * sizeof(float);
    if (pm < px + x_bytes && px < pm + mel_bytes) return WENC_ERR_ARG;  // x must not alias mel
  }
  const StemWorkspace w = stem_workspace(workspace, (size_t)batch, t_mel, n_mels, d_model, path);
  if (workspace_bytes < w.total) return WENC_ERR_WORKSPACE;
  const int d = d_model, dt = plain_dtype(path), k1 = stem_k1(n_mels);
  const StemLayout L = stem_layout(n_mels, d, n_pos, path);
  const char* blob = static_cast<const char*>(stem);
  auto fp = [&](size_t off) { return reinterpret_cast<const float*>(blob + off); };
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int m1 = batch * t_mel, m2 = batch * t2;
  WENC_TRY(launch_unfold_s1(mel, w.cols1, batch, t_mel, n_mels, k1, dt, st));
  WENC_TRY(launch_linear(w.cols1, k1, blob + L.w1, fp(L.b1), nullptr, w.h, d, m1, d, k1, dt,
                         EPI_BIAS_GELU, st));
  WENC_TRY(launch_unfold_s2(w.h, w.cols2, fp(L.pos), x, batch, t_mel, t2, d, dt, st));
  WENC_TRY(launch_linear(w.cols2, 3 * d, blob + L.w2, fp(L.b2), x, x, d, m2, d, 3 * d, dt,
                         EPI_BIAS_GELU_RESIDUAL, st));
  return WENC_OK;
}

}  // extern "C"

// ---- Low-precision weights, one matrix at a time (the quantiser and dequantiser the q8 / q4
// layer paths use). ----

extern "C" {

int whisper_enc_quantize_matrix(const float* w, void* codes, void* scales, int n, int k, int bits,
                                void* stream) {
  if ((bits != 8 && bits != 4) || n < 0 || k < 0 || k % 32 != 0 || n > WENC_MAX_ROWS ||
      k > WENC_MAX_FFN_DIM)
    return WENC_ERR_ARG;
  if ((size_t)n * k == 0) return WENC_OK;
  if (!w || !codes || !scales || !aligned(scales, 2)) return WENC_ERR_ARG;
  WENC_TRY(launch_quantize(w, codes, scales, n, k, bits, static_cast<hipStream_t>(stream)));
  return WENC_OK;
}

size_t whisper_enc_mx_bytes(int rows, int k) {
  if (rows < 0 || rows > WENC_MAX_ROWS || k < 32 || k % 32 != 0 || k > WENC_MAX_FFN_DIM) return 0;
  return mx_matrix_bytes((size_t)rows, (size_t)k);
}

int whisper_enc_mx_quantize(const float* src, void* dst, int rows, int k, void* stream) {
  if (rows < 0 || rows > WENC_MAX_ROWS || k < 32 || k % 32 != 0 || k > WENC_MAX_FFN_DIM)
    return WENC_ERR_ARG;
  if (rows == 0) return WENC_OK;
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16)) return WENC_ERR_ARG;
  if (overlaps(src, (size_t)rows * k * sizeof(float), dst, mx_matrix_bytes(rows, k)))
    return WENC_ERR_ARG;
  WENC_TRY(launch_mx_quantize(src, dst, rows, k, 0, rows, static_cast<hipStream_t>(stream)));
  return WENC_OK;
}

int whisper_enc_dequantize_matrix(const void* codes, const void* scales, void* dst, int n, int k,
                                  int bits, void* stream) {
  if ((bits != 8 && bits != 4) || n < 0 || k < 0 || k % 32 != 0 || n > WENC_MAX_ROWS ||
      k > WENC_MAX_FFN_DIM)
    return WENC_ERR_ARG;
  if ((size_t)n * k == 0) return WENC_OK;
  if ((size_t)n * (k / 8) > (size_t)INT32_MAX) return WENC_ERR_UNSUPPORTED;
  if (!codes || !scales || !dst || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(dst, 16))
    return WENC_ERR_ARG;
  DequantSegments seg{{codes, nullptr, nullptr, nullptr},
                      {static_cast<const uint16_t*>(scales), nullptr, nullptr, nullptr},
                      {static_cast<uint16_t*>(dst), nullptr, nullptr, nullptr},
                      {n, 0, 0, 0},
                      {k, 0, 0, 0},
                      1};
  WENC_TRY(launch_dequant(seg, bits, static_cast<hipStream_t>(stream)));
  return WENC_OK;
}

}  // extern "C"
