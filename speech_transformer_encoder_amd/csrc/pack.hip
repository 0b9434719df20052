// Element-wise conversion kernels used when a layer's weights are packed into the library's blob:
// fp32 -> bf16 / fp16 with round-to-nearest-even (oxinfer whisper/model.rs, make_lin: bf16
// storage of [n_out, n_in] matrices; norms and biases stay fp32), fp32 copies, and zero fill for
// the absent K bias (turbospark-runtime whisper/metal.rs, DecLayerGpu: packed QKV with a zero K
// bias slot).
#include "wenc_device.h"
#include "wenc_internal.h"

namespace wenc {

template <typename T>
__global__ void convert16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                 size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = (uint16_t)Cvt<T>::bits(src[i]);
}

// src [n][k] fp32 -> dst [n][2 k] bf16 rows [hi | lo], hi = bf16(v), lo = bf16(v - hi).
__global__ void convert_split_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                     size_t n, int k) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n * k; i += stride) {
    const size_t r = i / k, c = i - r * k;
    const float v = src[i];
    const float hi = (float)(__bf16)v;
    dst[r * 2 * k + c] = (uint16_t)Cvt<bf16_t>::bits(hi);
    dst[r * 2 * k + k + c] = (uint16_t)Cvt<bf16_t>::bits(v - hi);
  }
}

__global__ void copy_or_zero_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                    size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : 0.0f;
}

static dim3 grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  if (b > 8192) b = 8192;
  if (b == 0) b = 1;
  return dim3((unsigned)b);
}

hipError_t launch_convert(const float* src, void* dst, size_t n, int dtype, hipStream_t st) {
  if (n == 0) return hipSuccess;
  switch (dtype) {
    case DT_BF16:
      convert16_kernel<bf16_t><<<grid_for(n), 256, 0, st>>>(src, static_cast<uint16_t*>(dst), n);
      break;
    case DT_F16:
      convert16_kernel<f16_t><<<grid_for(n), 256, 0, st>>>(src, static_cast<uint16_t*>(dst), n);
      break;
    case DT_F32:
      copy_or_zero_kernel<<<grid_for(n), 256, 0, st>>>(src, static_cast<float*>(dst), n);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_convert_split(const float* src, void* dst, size_t n, int k, hipStream_t st) {
  if (n * k == 0) return hipSuccess;
  convert_split_kernel<<<grid_for(n * k), 256, 0, st>>>(src, static_cast<uint16_t*>(dst), n, k);
  return hipGetLastError();
}

hipError_t launch_copy_or_zero(const float* src, float* dst, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  copy_or_zero_kernel<<<grid_for(n), 256, 0, st>>>(src, dst, n);
  return hipGetLastError();
}

}  // namespace wenc
