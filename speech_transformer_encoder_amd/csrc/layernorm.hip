// LayerNorm over rows of an fp32 matrix, one wavefront per row.
//
// Whisper's pre-LN block normalises each position before attention and before the FFN, and a
// stack ends in one more LayerNorm (inferencelayer whisper_gpu.rs, LN_SRC and
// WhisperEncoderGpu::forward; oxinfer whisper/model.rs, encode).  Two passes as there: the row
// mean, then the biased variance of the centred values, inv = 1/sqrt(var + 1e-5), and the affine.
//
// The pages' shader runs one 256-thread workgroup per row with shared-memory tree reductions.
// Here a 64-lane wavefront owns a row: it loads the whole row into registers with 16-byte
// loads (d <= 4096), reduces with cross-lane shuffles, and writes the normalised row in the
// GEMM operand type (bf16 / fp16, or MXFP8 codes with their scale planes) or fp32.  Four rows
// per 256-thread workgroup.  The pass is HBM-bound: 4 bytes read and 1, 2 or 4 bytes written per
// element.
//
// When the residual GEMM before a LayerNorm splits k (one window), the GEMM's second pass and the
// LayerNorm are one kernel here (splitk_reduce_ln_rows): the row is formed from the parts in
// registers, stored, and normalised by the same row routine, so x is not read back.
#include "wenc_device.h"
#include "wenc_internal.h"

namespace wenc {

template <int NV, typename OutT>
struct LnStore;

template <int NV>
struct LnStore<NV, float> {
  static __device__ __forceinline__ void put(void* y, size_t row, int d, int c, float4 v, int) {
    *reinterpret_cast<float4*>(static_cast<float*>(y) + row * d + c) = v;
  }
};
template <int NV>
struct LnStore<NV, bf16_t> {
  static __device__ __forceinline__ void put(void* y, size_t row, int d, int c, float4 v, int) {
    u32x2 w = {pack2<bf16_t>(v.x, v.y), pack2<bf16_t>(v.z, v.w)};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + row * d + c) = w;
  }
};
template <int NV>
struct LnStore<NV, f16_t> {
  static __device__ __forceinline__ void put(void* y, size_t row, int d, int c, float4 v, int) {
    u32x2 w = {pack2<f16_t>(v.x, v.y), pack2<f16_t>(v.z, v.w)};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + row * d + c) = w;
  }
};

// bf16 hi / lo pair: row stride 2 d, hi in columns 0 .. d - 1, lo = bf16(v - hi) in d .. 2 d - 1.
struct bf16x2_t {};
template <int NV>
struct LnStore<NV, bf16x2_t> {
  static __device__ __forceinline__ void put(void* y, size_t row, int d, int c, float4 v, int) {
    const float h0 = (float)(__bf16)v.x, h1 = (float)(__bf16)v.y, h2 = (float)(__bf16)v.z,
                h3 = (float)(__bf16)v.w;
    uint16_t* base = static_cast<uint16_t*>(y) + row * 2 * d + c;
    *reinterpret_cast<u32x2*>(base) = u32x2{pack2<bf16_t>(h0, h1), pack2<bf16_t>(h2, h3)};
    *reinterpret_cast<u32x2*>(base + d) =
        u32x2{pack2<bf16_t>(v.x - h0, v.y - h1), pack2<bf16_t>(v.z - h2, v.w - h3)};
  }
};

// MXFP8 rows (codes [rows][d], then the scale planes): the 32 columns of a block are held by
// eight consecutive lanes (four each), which share the block's largest magnitude; the first of
// them stores the scale byte.  Called by every lane of those eight (d is a multiple of 64).
template <int NV>
struct LnStore<NV, mx8_t> {
  static __device__ __forceinline__ void put(void* y, size_t row, int d, int c, float4 v, int rows) {
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    const int xe = mx_exponent(amax);
    uint8_t* base = static_cast<uint8_t*>(y);
    *reinterpret_cast<uint32_t*>(base + row * d + c) = mx_pack4(v, mx_inv_scale(xe));
    if ((c & 31) == 0)
      base[mx_planes_offset(rows, d) + (size_t)(c >> 5) * mx_plane_stride(rows) + row] =
          (uint8_t)(xe + 127);
  }
};

// Normalises one row held in a wavefront's registers (lane l has columns 4 (l + 64 j) .. + 3 in
// v[j]; entries past d are ignored) and stores it as OutT.  Both the plain LayerNorm and the fused
// split-k reduction below end in this routine, so they round identically.
template <int NV, typename OutT>
__device__ __forceinline__ void ln_row(float4 (&v)[NV], int lane, const float* __restrict__ gamma,
                                       const float* __restrict__ beta, void* y, size_t row, int d,
                                       float eps, int rows) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (lane + 64 * j) * 4;
    if (c < d) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  }
  const float inv_d = 1.0f / (float)d;
  const float mean = wave_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (lane + 64 * j) * 4;
    if (c < d) {
      v[j].x -= mean; v[j].y -= mean; v[j].z -= mean; v[j].w -= mean;
      q += (v[j].x * v[j].x + v[j].y * v[j].y) + (v[j].z * v[j].z + v[j].w * v[j].w);
    }
  }
  const float var = wave_sum(q) * inv_d;
  const float inv = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (lane + 64 * j) * 4;
    if (c < d) {
      const float4 g = *reinterpret_cast<const float4*>(gamma + c);
      const float4 b = *reinterpret_cast<const float4*>(beta + c);
      float4 o;
      o.x = v[j].x * inv * g.x + b.x;
      o.y = v[j].y * inv * g.y + b.y;
      o.z = v[j].z * inv * g.z + b.z;
      o.w = v[j].w * inv * g.w + b.w;
      LnStore<NV, OutT>::put(y, row, d, c, o, rows);
    }
  }
}

// NV = float4 vectors per lane (d <= 256 * NV).
template <int NV, typename OutT>
__global__ __launch_bounds__(256) void layernorm_rows(const float* __restrict__ x,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ beta,
                                                      void* y, int rows, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (size_t)rows) return;
  const float* xr = x + row * d;
  float4 v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (lane + 64 * j) * 4;
    v[j] = c < d ? *reinterpret_cast<const float4*>(xr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  ln_row<NV, OutT>(v, lane, gamma, beta, y, row, d, eps, rows);
}

// Second pass of a split-k residual GEMM fused with the LayerNorm that reads its output: per row,
// x = residual + (sum of the k parts, added in order, + bias) -- the same sums as the plain
// reduction kernel -- stored to x_out when given, then y = LayerNorm(x) * gamma + beta.  One
// wavefront per row reads the whole row before it writes, so x_out and y may alias residual.
template <int NV, typename OutT>
__global__ __launch_bounds__(256) void splitk_reduce_ln_rows(
    const float* __restrict__ part, int ksplit, const float* __restrict__ bias,
    const float* residual, float* x_out, const float* __restrict__ gamma,
    const float* __restrict__ beta, void* y, int rows, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (size_t)rows) return;
  const size_t plane = (size_t)rows * d;
  const float* pr = part + row * d;
  // Parts outermost, the row's columns innermost, with no branches around the loads (columns
  // past d read column d - 4 and are ignored by ln_row): each step keeps NV independent loads in
  // flight, which a row owned by one wavefront needs to move enough bytes.  Per element the
  // parts are still added in order 0, 1, ...
  int cl[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) cl[j] = min((lane + 64 * j) * 4, d - 4);
  float4 v[NV], r[NV], b[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    r[j] = *reinterpret_cast<const float4*>(residual + row * d + cl[j]);
    b[j] = *reinterpret_cast<const float4*>(bias + cl[j]);
    v[j] = *reinterpret_cast<const float4*>(pr + cl[j]);
  }
#pragma unroll 4
  for (int p = 1; p < ksplit; ++p) {
    float4 q[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) q[j] = *reinterpret_cast<const float4*>(pr + p * plane + cl[j]);
#pragma unroll
    for (int j = 0; j < NV; ++j)
      v[j] = make_float4(v[j].x + q[j].x, v[j].y + q[j].y, v[j].z + q[j].z, v[j].w + q[j].w);
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const float4 u = make_float4(v[j].x + b[j].x, v[j].y + b[j].y, v[j].z + b[j].z, v[j].w + b[j].w);
    v[j] = make_float4(r[j].x + u.x, r[j].y + u.y, r[j].z + u.z, r[j].w + u.w);
  }
  if (x_out) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c = (lane + 64 * j) * 4;
      if (c < d) *reinterpret_cast<float4*>(x_out + row * d + c) = v[j];
    }
  }
  ln_row<NV, OutT>(v, lane, gamma, beta, y, row, d, eps, rows);
}

template <typename OutT>
static hipError_t launch_ln_t(const float* x, const float* g, const float* b, void* y, int rows,
                              int d, hipStream_t st) {
  dim3 grid((rows + 3) / 4), block(256);
  const float eps = 1e-5f;
  const int nv = (d + 255) / 256;
  switch (nv) {
#define WENC_LN_CASE(N) \
  case N: layernorm_rows<N, OutT><<<grid, block, 0, st>>>(x, g, b, y, rows, d, eps); break;
    WENC_LN_CASE(1) WENC_LN_CASE(2) WENC_LN_CASE(3) WENC_LN_CASE(4) WENC_LN_CASE(5)
    WENC_LN_CASE(6) WENC_LN_CASE(7) WENC_LN_CASE(8) WENC_LN_CASE(9) WENC_LN_CASE(10)
    WENC_LN_CASE(11) WENC_LN_CASE(12) WENC_LN_CASE(13) WENC_LN_CASE(14) WENC_LN_CASE(15)
    WENC_LN_CASE(16)
#undef WENC_LN_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename OutT>
static hipError_t launch_reduce_ln_t(const float* part, int ksplit, const float* bias,
                                     const float* residual, float* x_out, const float* g,
                                     const float* b, void* y, int rows, int d, hipStream_t st) {
  dim3 grid((rows + 3) / 4), block(256);
  const float eps = 1e-5f;
  const int nv = (d + 255) / 256;
  switch (nv) {
#define WENC_RLN_CASE(N)                                                                       \
  case N:                                                                                      \
    splitk_reduce_ln_rows<N, OutT><<<grid, block, 0, st>>>(part, ksplit, bias, residual, x_out, \
                                                           g, b, y, rows, d, eps);             \
    break;
    WENC_RLN_CASE(1) WENC_RLN_CASE(2) WENC_RLN_CASE(3) WENC_RLN_CASE(4) WENC_RLN_CASE(5)
    WENC_RLN_CASE(6) WENC_RLN_CASE(7) WENC_RLN_CASE(8) WENC_RLN_CASE(9) WENC_RLN_CASE(10)
    WENC_RLN_CASE(11) WENC_RLN_CASE(12) WENC_RLN_CASE(13) WENC_RLN_CASE(14) WENC_RLN_CASE(15)
    WENC_RLN_CASE(16)
#undef WENC_RLN_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce_ln(const float* part, int ksplit, const float* bias,
                                   const float* residual, float* x_out, const float* gamma,
                                   const float* beta, void* y, int y_dtype, int rows, int d,
                                   hipStream_t st) {
  if (rows == 0) return hipSuccess;
  switch (y_dtype) {
    case DT_F32:
      return launch_reduce_ln_t<float>(part, ksplit, bias, residual, x_out, gamma, beta, y, rows,
                                       d, st);
    case DT_BF16:
      return launch_reduce_ln_t<bf16_t>(part, ksplit, bias, residual, x_out, gamma, beta, y,
                                        rows, d, st);
    case DT_F16:
      return launch_reduce_ln_t<f16_t>(part, ksplit, bias, residual, x_out, gamma, beta, y, rows,
                                       d, st);
    case DT_BF16X2:
      return launch_reduce_ln_t<bf16x2_t>(part, ksplit, bias, residual, x_out, gamma, beta, y,
                                          rows, d, st);
    case DT_MX8:
      return launch_reduce_ln_t<mx8_t>(part, ksplit, bias, residual, x_out, gamma, beta, y, rows,
                                       d, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* y, int rows,
                            int d, int out_dtype, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  switch (out_dtype) {
    case DT_F32: return launch_ln_t<float>(x, g, b, y, rows, d, st);
    case DT_BF16: return launch_ln_t<bf16_t>(x, g, b, y, rows, d, st);
    case DT_F16: return launch_ln_t<f16_t>(x, g, b, y, rows, d, st);
    case DT_BF16X2: return launch_ln_t<bf16x2_t>(x, g, b, y, rows, d, st);
    case DT_MX8: return launch_ln_t<mx8_t>(x, g, b, y, rows, d, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace wenc
