// Host-side launchers of the gfx950 kernels.  Each returns the launch's hipError_t; none of
// them allocates, synchronises or validates shapes (the C ABI in api.hip does that first).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wenc {

// DT_BF16X2: a value v carried as two bfloat16 numbers hi = bf16(v), lo = bf16(v - hi), a row of
// d values stored as [hi_0 .. hi_{d-1} | lo_0 .. lo_{d-1}] (2 d elements); a GEMM whose k runs over
// both halves while the weight row repeats computes w . hi + w . lo = w . v to ~2^-17.
// MXFP8 matrix (OCP Microscaling Formats v1.0, MXFP8: E4M3 values with one E8M0 scale per block
// of 32 consecutive values of a row): `rows` rows of k values are stored as codes [rows][k] (one
// E4M3 byte each) followed, at byte offset mx_planes_offset(rows, k), by k / 32 scale planes of
// mx_plane_stride(rows) bytes: the byte X + 127 of block j of row r at plane j, position r.
// Value = code * 2^X.
__host__ __device__ inline size_t mx_planes_offset(size_t rows, size_t k) {
  return (rows * k + 255) / 256 * 256;
}
__host__ __device__ inline size_t mx_plane_stride(size_t rows) { return (rows + 15) / 16 * 16; }
__host__ __device__ inline size_t mx_matrix_bytes(size_t rows, size_t k) {
  return mx_planes_offset(rows, k) + ((k / 32) * mx_plane_stride(rows) + 255) / 256 * 256;
}

// DT_MX8: an MXFP8 matrix (above).
enum DType { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_BF16X2 = 3, DT_MX8 = 4 };
enum Epilogue {
  EPI_BIAS = 0,
  EPI_BIAS_GELU = 1,
  EPI_BIAS_RESIDUAL = 2,
  EPI_BIAS_HEADMAJOR = 3,
  EPI_BIAS_GELU_RESIDUAL = 4,
  EPI_PARTIAL = 5,  // split-k part: raw fp32 sums (no bias) to partial[split][m][n]
  EPI_BIAS_GELU_X2 = 6  // gelu_erf(. + bias) as a bf16 hi / lo pair: row m = [hi (n) | lo (n)]
};

// y[rows, d] = LayerNorm(x[rows, d]) * gamma + beta, stored as out_dtype (DT_BF16X2: rows of
// 2 d, hi then lo; DT_MX8: an MXFP8 matrix of rows x d, d % 64 == 0).  d % 4 == 0, d <= 4096.
hipError_t launch_layernorm(const float* x, const float* gamma, const float* beta, void* y,
                            int rows, int d, int out_dtype, hipStream_t st);

// Second pass of a split-k residual GEMM with the LayerNorm that follows it: per row of [rows, d],
// x = residual + (part[0] + ... + part[ksplit - 1] + bias) (parts of rows * d floats, added in
// order), stored to x_out unless it is null, and y = LayerNorm(x) * gamma + beta as y_dtype.
// Rounds exactly as the plain reduction followed by launch_layernorm.  x_out / y may alias residual.
hipError_t launch_splitk_reduce_ln(const float* part, int ksplit, const float* bias,
                                   const float* residual, float* x_out, const float* gamma,
                                   const float* beta, void* y, int y_dtype, int rows, int d,
                                   hipStream_t st);

// A LayerNorm to fuse into the second pass of a split-k residual GEMM (launch_linear).
struct LnFuse {
  const float* gamma;
  const float* beta;
  void* y;       // [m, n] in y_dtype
  int y_dtype;
  bool keep_x;   // also store the GEMM's own output c
};

// c[m, n] = epilogue(a[m, k] . w[n, k]^T + bias[n]) with 16-bit (dtype) or fp32 operands.
//   EPI_BIAS          -> c in the operand dtype (fp32 for DT_F32)
//   EPI_BIAS_GELU     -> c = gelu_erf(.) in the operand dtype
//   EPI_BIAS_RESIDUAL -> c fp32 = residual + (.)   (c may alias residual)
//   EPI_BIAS_GELU_RESIDUAL -> c fp32 = residual + gelu_erf(.)   (c may alias residual)
//   EPI_BIAS_HEADMAJOR-> c in the operand dtype, head-major: row m = b * T + i of window b and
//                        column n = 64 j + e go to c[((b * (n / 64 count) + j) * T + i) * 64 + e],
//                        with the window length T passed in ldc.
// lda / ldc are row strides in elements.  k % 64 == 0, n % 64 == 0.
// partial: optional fp32 scratch of linear_split(m, n, k, dtype, epilogue) * m * n floats; given,
// a residual GEMM too small to fill the GPU splits k over that many workgroups and a second
// kernel adds the parts in a fixed order (deterministic), then bias and residual.
// ln: with a split EPI_BIAS_RESIDUAL GEMM (ldc == n), the second kernel also applies this
// LayerNorm to the rows it forms (launch_splitk_reduce_ln); anything else with ln is an error.
// How a GEMM's k range maps onto its operand rows when values are carried as bf16 hi / lo pairs:
// k runs over nseg segments of kb elements; segment s reads the activation row's half
// (xmask >> s) & 1 and the weight row's half (wmask >> s) & 1 (half 0: elements 0 .. kb - 1, half
// 1: kb .. 2 kb - 1); a weight row holds wrow elements (kb, or 2 kb when it is a hi / lo pair).
// E.g. x = hi + lo against one weight row: {kb, 2, 0b10, 0, kb}; both split, dropping lo . lo:
// {kb, 3, 0b010, 0b100, 2 kb} (hi.hi + lo.hi + hi.lo).
struct KMap {
  int kb, nseg, xmask, wmask, wrow;
};
// Scale planes of the MXFP8 operands of one GEMM (x: the activation rows, w: the weight rows,
// c: the MXFP8 output of EPI_BIAS_GELU), each plane's stride in bytes.
struct MxPlanes {
  const uint8_t* x;
  int x_stride;
  const uint8_t* w;
  int w_stride;
  uint8_t* c;
  int c_stride;
};
// kmap: nullptr for the plain contraction over k; else k == kmap->nseg * kmap->kb.
// DT_MX8: a and w are MXFP8 matrices ([m][k] and [n][k] codes, lda == k, followed by their scale
// planes); EPI_BIAS writes fp16, EPI_BIAS_GELU an MXFP8 [m][n] matrix (ldc == n), the residual
// epilogues fp32; no kmap, no EPI_BIAS_HEADMAJOR.
hipError_t launch_linear(const void* a, int lda, const void* w, const float* bias,
                         const float* residual, void* c, int ldc, int m, int n, int k, int dtype,
                         int epilogue, hipStream_t st, float* partial = nullptr,
                         const LnFuse* ln = nullptr, const KMap* kmap = nullptr);
// Number of k parts launch_linear uses with a partial buffer (1: none).  Fixed for a shape,
// whatever the device, so that workspace sizes are too.
int linear_split(int m, int n, int k, int dtype, int epilogue);

// Bidirectional attention per (window, head), head_dim 64.  q/k/v/o rows of the window b at
// ptr + (b * t + i) * ld, head h at column offset 64 * h.  scale multiplies q.k.
// Equal windows of t rows (cu == nullptr), or a packed ragged batch: window b is rows
// cu[b] .. cu[b + 1] - 1 (device int32 [batch + 1]) of `total`, each at most t rows long.
// part: optional fp32 scratch of attention_split(batch, t, heads, dtype) == 2 ?
// 2 * rows * heads * 66 floats (rows = batch * t, or total for a ragged batch); given, a problem
// with too few query blocks to fill the GPU splits each block's keys in two halves over two
// workgroups and a second kernel merges the halves' (O, m, l).
hipError_t launch_attention(const void* q, const void* k, const void* v, int ld_qkv, void* o,
                            int ld_o, int batch, int t, int heads, float scale, int dtype,
                            hipStream_t st, const int* cu = nullptr, int total = 0,
                            float* part = nullptr);
// Key halves launch_attention uses with a part buffer (1: none).  Fixed for a shape.
int attention_split(int batch, int t, int heads, int dtype);

// dst[i] = round(src[i]) in dtype (or a copy for DT_F32); n elements.
hipError_t launch_convert(const float* src, void* dst, size_t n, int dtype, hipStream_t st);
// Rows of src [n][k] fp32 as bf16 hi / lo pairs: dst [n][2 k], row r = [bf16(v) | bf16(v - hi)].
hipError_t launch_convert_split(const float* src, void* dst, size_t n, int k, hipStream_t st);
// dst[i] = src ? src[i] : 0 for i < n (fp32).
hipError_t launch_copy_or_zero(const float* src, float* dst, size_t n, hipStream_t st);

// Low-precision weights (quant.hip).  quantize: w [n][k] fp32 -> codes (int8 [n][k] for bits 8;
// nibbles [n][k / 2] for bits 4, column 2i low, 2i + 1 high) and fp16 scales [n][k / 32].
// dequant: up to four matrices of codes + scales -> fp16 [n][k].
struct DequantSegments {
  const void* codes[4];
  const uint16_t* scales[4];
  uint16_t* dst[4];
  int n[4], k[4];
  int count;
};
hipError_t launch_quantize(const float* w, void* codes, void* scales, int n, int k, int bits,
                           hipStream_t st);
hipError_t launch_dequant(const DequantSegments& seg, int bits, hipStream_t st);
// MXFP8: src [n][k] fp32 (16-byte aligned rows, k % 32 == 0) -> rows r0 .. r0 + n - 1 of the
// MXFP8 matrix of `total` rows at dst (codes and scale planes; mx_planes_offset).
hipError_t launch_mx_quantize(const float* src, void* dst, int n, int k, int r0, int total,
                              hipStream_t st);

// Conv front end rearrangements (stem.hip).  dst[o][j * cin + i] = w[o][i][j] (zero past 3 cin,
// kp columns); unfold_s1: out[b t + i][j c + q] = src[b][i + j - 1][q] (fp32 src, kp columns);
// unfold_s2: out[b t2 + i][j d + q] = src[b t + 2 i + j - 1][q] (src in dtype) and
// pos_out[b t2 + i] = pos[i].  Zeros outside each window.
hipError_t launch_pack_conv(const float* w, void* dst, int cout, int cin, int kp, int dtype,
                            hipStream_t st);
hipError_t launch_unfold_s1(const float* src, void* out, int batch, int t, int c, int kp,
                            int dtype, hipStream_t st);
hipError_t launch_unfold_s2(const void* src, void* out, const float* pos, float* pos_out,
                            int batch, int t, int t2, int d, int dtype, hipStream_t st);

}  // namespace wenc
