// The convolutional front end of the encoder, the step before the first block: two kernel-3
// convolutions over mel frames (stride 1, then stride 2, padding 1), each followed by erf-GELU,
// plus the positional rows (oxinfer whisper/model.rs, WhisperModel::encode: conv1 and conv2 as
// projections of unfolded rows, conv_weight; turbospark-runtime whisper/metal.rs,
// encode_partial: encode_whisper_conv1d3_gelu and encode_whisper_transpose_pos).
//
// Each convolution runs as one MFMA GEMM (the same kernels as the block's projections) over
// unfolded rows: row i of the unfolded input holds the three input rows s * i - 1, s * i,
// s * i + 1 side by side (zeros outside the window), and the weight [cout, cin, 3] is rearranged
// to [cout][k][cin] to match.  The kernels here are the HBM-bound rearrangements: the weight pack,
// the two unfoldings (16-bit rows, widths padded with zeros to a multiple of 64) and the
// positional rows the second GEMM adds to in place.
#include "wenc_device.h"
#include "wenc_internal.h"

namespace wenc {

template <typename T> struct Store16;
template <> struct Store16<float> {
  static __device__ __forceinline__ void put(void* p, size_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <> struct Store16<bf16_t> {
  static __device__ __forceinline__ void put(void* p, size_t i, float v) {
    static_cast<uint16_t*>(p)[i] = (uint16_t)Cvt<bf16_t>::bits(v);
  }
};
template <> struct Store16<f16_t> {
  static __device__ __forceinline__ void put(void* p, size_t i, float v) {
    static_cast<uint16_t*>(p)[i] = (uint16_t)Cvt<f16_t>::bits(v);
  }
};

// dst[o][j * cin + i] = w[o][i][j] for j < 3, zero for columns 3 cin .. kp - 1.
template <typename T>
__global__ void pack_conv_kernel(const float* __restrict__ w, void* __restrict__ dst, int cout,
                                 int cin, int kp) {
  const size_t n = (size_t)cout * kp;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
       e += (size_t)gridDim.x * blockDim.x) {
    const int o = (int)(e / kp), col = (int)(e % kp);
    float v = 0.f;
    if (col < 3 * cin) {
      const int j = col / cin, i = col % cin;
      v = w[((size_t)o * cin + i) * 3 + j];
    }
    Store16<T>::put(dst, e, v);
  }
}

// Unfolded rows of the stride-1 convolution: out[b * t + i][j * c + q] = src[b][i + j - 1][q]
// (fp32 source, zero outside [0, t) and for columns 3 c .. kp - 1).
template <typename T>
__global__ void unfold_s1_kernel(const float* __restrict__ src, void* __restrict__ out, int batch,
                                 int t, int c, int kp) {
  const size_t n = (size_t)batch * t * kp;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t row = e / kp;
    const int col = (int)(e % kp);
    const int b = (int)(row / t), i = (int)(row % t);
    float v = 0.f;
    if (col < 3 * c) {
      const int j = col / c, q = col % c, s = i + j - 1;
      if (s >= 0 && s < t) v = src[((size_t)b * t + s) * c + q];
    }
    Store16<T>::put(out, e, v);
  }
}

// Unfolded rows of the stride-2 convolution over 16-bit (or fp32) rows of width d:
// out[b * t2 + i][j * d + q] = src[b * t + 2 i + j - 1][q] (zero outside [0, t)), 16 bytes per
// thread, and pos_out[b * t2 + i][q] = pos[i][q] (the rows the GEMM adds to).
template <int ES>
__global__ void unfold_s2_kernel(const void* __restrict__ src, void* __restrict__ out,
                                 const float* __restrict__ pos, float* __restrict__ pos_out,
                                 int batch, int t, int t2, int d) {
  constexpr int V = 16 / ES;  // elements per 16-byte vector
  const int dv = d / V;       // vectors per source row
  const size_t n = (size_t)batch * t2 * 3 * dv;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t row = e / (3 * dv);
    const int col = (int)(e % (3 * dv));
    const int b = (int)(row / t2), i = (int)(row % t2);
    const int j = col / dv, q = col % dv, s = 2 * i + j - 1;
    u32x4 v = {0, 0, 0, 0};
    if (s >= 0 && s < t)
      v = reinterpret_cast<const u32x4*>(src)[((size_t)b * t + s) * dv + q];
    reinterpret_cast<u32x4*>(out)[e] = v;
  }
  const size_t np = (size_t)batch * t2 * (d / 4);
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < np;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t row = e / (d / 4);
    const int q = (int)(e % (d / 4));
    const int i = (int)(row % t2);
    reinterpret_cast<float4*>(pos_out)[e] = reinterpret_cast<const float4*>(pos)[(size_t)i * (d / 4) + q];
  }
}

static dim3 grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  if (b == 0) b = 1;
  return dim3((unsigned)b);
}

hipError_t launch_pack_conv(const float* w, void* dst, int cout, int cin, int kp, int dtype,
                            hipStream_t st) {
  const dim3 g = grid_for((size_t)cout * kp);
  switch (dtype) {
    case DT_F32: pack_conv_kernel<float><<<g, 256, 0, st>>>(w, dst, cout, cin, kp); break;
    case DT_BF16: pack_conv_kernel<bf16_t><<<g, 256, 0, st>>>(w, dst, cout, cin, kp); break;
    case DT_F16: pack_conv_kernel<f16_t><<<g, 256, 0, st>>>(w, dst, cout, cin, kp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_unfold_s1(const float* src, void* out, int batch, int t, int c, int kp,
                            int dtype, hipStream_t st) {
  const dim3 g = grid_for((size_t)batch * t * kp);
  switch (dtype) {
    case DT_F32: unfold_s1_kernel<float><<<g, 256, 0, st>>>(src, out, batch, t, c, kp); break;
    case DT_BF16: unfold_s1_kernel<bf16_t><<<g, 256, 0, st>>>(src, out, batch, t, c, kp); break;
    case DT_F16: unfold_s1_kernel<f16_t><<<g, 256, 0, st>>>(src, out, batch, t, c, kp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_unfold_s2(const void* src, void* out, const float* pos, float* pos_out,
                            int batch, int t, int t2, int d, int dtype, hipStream_t st) {
  const dim3 g = grid_for((size_t)batch * t2 * 3 * d / 8);
  if (dtype == DT_F32)
    unfold_s2_kernel<4><<<g, 256, 0, st>>>(src, out, pos, pos_out, batch, t, t2, d);
  else
    unfold_s2_kernel<2><<<g, 256, 0, st>>>(src, out, pos, pos_out, batch, t, t2, d);
  return hipGetLastError();
}

}  // namespace wenc
