// Measurement probe (not part of the encoder path): the dense 16-bit (and MXFP8) MFMA rate this
// GPU sustains on register operands, and the shader clock while it does.  The rated peak assumes the 2.4 GHz
// peak engine clock; under a full matrix-core load the clock settles lower, and this probe gives
// the rate the GEMM and attention kernels can actually approach.
//
// Every wavefront issues `iters` rounds of four independent v_mfma_f32_32x32x16 (f16 or bf16) on
// operands drawn from a lane hash in [-1, 1), so the data toggles like real operands, or of
// v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 operands from the same hash (exponent fields 0 .. 14,
// no NaN codes; unit scales) for the MXFP8 rate.  Wavefront 0 of workgroup 0 reads the
// shader-clock counter and the constant 100 MHz counter around its loop.
#include "../wenc_device.h"
#include "../../../include/wenc_probe.h"

namespace wenc {

template <typename T>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, unsigned long long* clocks,
                                                        float sentinel, float* sink) {
  const int lane = threadIdx.x & 63;
  u32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h1 = (lane + 64u * i + 1u) * 0x9E3779B1u ^ (threadIdx.x >> 6) * 0x85EBCA77u;
    const uint32_t h2 = h1 * 0xC2B2AE3Du + 0x27D4EB2Fu;
    auto u = [](uint32_t h) { return (float)(h & 0xFFFFu) * (2.0f / 65536.0f) - 1.0f; };
    a[i] = pack2<T>(u(h1), u(h1 >> 16));
    b[i] = pack2<T>(u(h2), u(h2 >> 16));
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
  unsigned long long c0 = 0, r0 = 0;
  if (timer) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma32x32x16<T>(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (timer) {
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      clocks[0] = c1 - c0;
      clocks[1] = r1 - r0;
    }
  }
  if (s == sentinel) sink[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the MFMAs live
}

__global__ __launch_bounds__(256) void mfma_peak_mx8_kernel(int iters, unsigned long long* clocks,
                                                            float sentinel, float* sink) {
  const int lane = threadIdx.x & 63;
  u32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h1 = (lane + 64u * i + 1u) * 0x9E3779B1u ^ (threadIdx.x >> 6) * 0x85EBCA77u;
    const uint32_t h2 = h1 * 0xC2B2AE3Du + 0x27D4EB2Fu;
    a[i] = h1 & 0xF7F7F7F7u;  // bit 3 of each byte clear: exponent fields <= 14, no NaN code
    b[i] = h2 & 0xF7F7F7F7u;
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
  unsigned long long c0 = 0, r0 = 0;
  if (timer) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma_mx8(a, b, 127, 127, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (timer) {
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      clocks[0] = c1 - c0;
      clocks[1] = r1 - r0;
    }
  }
  if (s == sentinel) sink[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the MFMAs live
}

}  // namespace wenc

extern "C" int wenc_probe_mfma(int dtype, int blocks, int iters, unsigned long long* clocks,
                               float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || !clocks || !sink) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float sentinel = __builtin_nanf("");  // never equal: the sink is never written
  if (dtype == WENC_PROBE_F16)
    wenc::mfma_peak_kernel<wenc::f16_t><<<blocks, 256, 0, st>>>(iters, clocks, sentinel, sink);
  else if (dtype == WENC_PROBE_BF16)
    wenc::mfma_peak_kernel<wenc::bf16_t><<<blocks, 256, 0, st>>>(iters, clocks, sentinel, sink);
  else if (dtype == WENC_PROBE_MXFP8)
    wenc::mfma_peak_mx8_kernel<<<blocks, 256, 0, st>>>(iters, clocks, sentinel, sink);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" long long wenc_probe_mfma_flops(int dtype, int blocks, int iters) {
  const long long k = dtype == WENC_PROBE_MXFP8 ? 64 : 16;  // k of one MFMA
  return (long long)blocks * 4 /* wavefronts */ * iters * 4 /* chains */ * (2LL * 32 * 32 * k);
}
