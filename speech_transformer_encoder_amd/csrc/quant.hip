// Low-precision weights: q8 / q4 blocks of 32 consecutive input columns with one fp16 scale each,
// quantised from the matrix rounded to bf16 (oxinfer whisper/model.rs, Precision and make_lin:
// int8 / int4 blocks of 32, from bf16; norms and biases stay f32).  The pages name the formats
// without printing them; the encodings are the q8_0 / q4_0 block formats the q4_0 name refers to:
//   q8: d = amax / 127, code round-half-away(x / d) in [-127, 127], value code * d;
//   q4: m = first element of largest magnitude, d = m / -8, code min(15, floor(x / d + 8.5)),
//       value (code - 8) * d.
// The code is an integer decided by floating point, so each step is an explicitly rounded fp32
// operation (x times the correctly rounded reciprocal of d; no contraction into an FMA).
//
// At rest a layer's matrices stay quantised (1 + 1/16 or 1/2 + 1/16 bytes per weight); before a
// block runs, one HBM-bound kernel expands them to fp16 in the workspace and the fp16 GEMMs read
// those.  Dequantised values are code * d16 rounded once to fp16.
#include <algorithm>

#include "wenc_device.h"
#include "wenc_internal.h"

namespace wenc {

__device__ __forceinline__ float bf16_value(float x) { return (float)(__bf16)x; }

// One thread per (row, block of 32): codes (int8 [n][k], or nibbles [n][k / 2] with column 2i in
// the low and 2i + 1 in the high nibble of byte i) and scales (fp16 [n][k / 32]).
template <int BITS>
__global__ void quantize_kernel(const float* __restrict__ w, uint8_t* __restrict__ codes,
                                uint16_t* __restrict__ scales, int n, int k) {
#pragma clang fp contract(off)
  const int nb = k / 32;
  const size_t total = (size_t)n * nb;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(e / nb), blk = (int)(e % nb);
    const float* src = w + (size_t)row * k + blk * 32;
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = bf16_value(src[i]);
    float d;
    if constexpr (BITS == 8) {
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
      d = __fdiv_rn(amax, 127.0f);
      const float id = d != 0.f ? __fdiv_rn(1.0f, d) : 0.f;
      int8_t* out = reinterpret_cast<int8_t*>(codes) + (size_t)row * k + blk * 32;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float v = __fmul_rn(x[i], id);
        out[i] = (int8_t)(int)copysignf(floorf(__fadd_rn(fabsf(v), 0.5f)), v);
      }
    } else {
      float amax = 0.f, m = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (fabsf(x[i]) > amax) {
          amax = fabsf(x[i]);
          m = x[i];
        }
      d = m != 0.f ? __fdiv_rn(m, -8.0f) : 0.f;  // an all-zero block: scale +0
      const float id = d != 0.f ? __fdiv_rn(1.0f, d) : 0.f;
      uint8_t* out = codes + (size_t)row * (k / 2) + blk * 16;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p0 = __fmul_rn(x[2 * i], id), p1 = __fmul_rn(x[2 * i + 1], id);
        asm volatile("" : "+v"(p0), "+v"(p1));  // the products are rounded before the add
        const int lo = min(15, (int)floorf(__fadd_rn(p0, 8.5f)));
        const int hi = min(15, (int)floorf(__fadd_rn(p1, 8.5f)));
        out[i] = (uint8_t)(lo | (hi << 4));
      }
    }
    scales[(size_t)row * nb + blk] = __builtin_bit_cast(uint16_t, (_Float16)d);
  }
}

// Eight consecutive outputs per thread; grid row blockIdx.y is matrix s (rows n[s], columns
// k[s]); fp16 results, 16-byte stores.  Each matrix has fewer than 2^31 eight-column vectors.
template <int BITS>
__global__ void dequant_kernel(DequantSegments seg) {
  const int s = blockIdx.y;
  if (s >= seg.count) return;
  const uint32_t k = (uint32_t)seg.k[s], kv = k / 8, nb = k / 32;
  const uint32_t total = (uint32_t)seg.n[s] * kv;
  const uint8_t* codes = static_cast<const uint8_t*>(seg.codes[s]);
  const uint16_t* scales = seg.scales[s];
  uint16_t* dst = seg.dst[s];
  for (uint32_t e = blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += gridDim.x * blockDim.x) {
    const uint32_t row = e / kv, c0 = (e - row * kv) * 8;
    const float d = (float)__builtin_bit_cast(_Float16, scales[(size_t)row * nb + c0 / 32]);
    float v[8];
    if constexpr (BITS == 8) {
      const uint2 c = *reinterpret_cast<const uint2*>(codes + (size_t)row * k + c0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t word = i < 4 ? c.x : c.y;
        v[i] = (float)(int8_t)(word >> (8 * (i & 3))) * d;
      }
    } else {
      const uint32_t c = *reinterpret_cast<const uint32_t*>(codes + (size_t)row * (k / 2) + c0 / 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)((int)((c >> (4 * i)) & 15u) - 8) * d;
    }
    const u32x4 o = {Cvt<f16_t>::pack(v[0], v[1]), Cvt<f16_t>::pack(v[2], v[3]),
                     Cvt<f16_t>::pack(v[4], v[5]), Cvt<f16_t>::pack(v[6], v[7])};
    *reinterpret_cast<u32x4*>(dst + (size_t)row * k + c0) = o;
  }
}

static dim3 grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  if (b == 0) b = 1;
  return dim3((unsigned)b);
}

hipError_t launch_quantize(const float* w, void* codes, void* scales, int n, int k, int bits,
                           hipStream_t st) {
  const dim3 g = grid_for((size_t)n * (k / 32));
  auto c = static_cast<uint8_t*>(codes);
  auto s = static_cast<uint16_t*>(scales);
  if (bits == 8)
    quantize_kernel<8><<<g, 256, 0, st>>>(w, c, s, n, k);
  else if (bits == 4)
    quantize_kernel<4><<<g, 256, 0, st>>>(w, c, s, n, k);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantSegments& seg, int bits, hipStream_t st) {
  size_t most = 0;
  for (int s = 0; s < seg.count; ++s) most = std::max(most, (size_t)seg.n[s] * (seg.k[s] / 8));
  if (most == 0) return hipSuccess;
  const dim3 g(grid_for(most).x, (unsigned)seg.count);
  if (bits == 8)
    dequant_kernel<8><<<g, 256, 0, st>>>(seg);
  else if (bits == 4)
    dequant_kernel<4><<<g, 256, 0, st>>>(seg);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// MXFP8 weights (the operands of the scaled-MFMA GEMMs): rows r0 .. r0 + n - 1 of an MXFP8 matrix
// of `total` rows and k columns at dst (codes, then the scale planes), from fp32 src [n][k].  One
// thread per (row, block of 32): the block's largest magnitude fixes X (mx_exponent), the codes
// are the E4M3 roundings of v 2^-X (exact scaling by a power of two, then round to nearest even).
__global__ void mx_quantize_kernel(const float* __restrict__ src, uint8_t* __restrict__ dst,
                                   int n, int k, int r0, int total) {
  const int nb = k / 32;
  const size_t blocks = (size_t)n * nb;
  uint8_t* planes = dst + mx_planes_offset(total, k);
  const size_t pstride = mx_plane_stride(total);
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < blocks;
       e += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(e / nb), blk = (int)(e % nb);
    const float4* s4 = reinterpret_cast<const float4*>(src + (size_t)row * k + blk * 32);
    float4 v[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = s4[i];
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    const int xe = mx_exponent(amax);
    const float sc = mx_inv_scale(xe);
    u32x4* out = reinterpret_cast<u32x4*>(dst + (size_t)(r0 + row) * k + blk * 32);
    out[0] = u32x4{mx_pack4(v[0], sc), mx_pack4(v[1], sc), mx_pack4(v[2], sc), mx_pack4(v[3], sc)};
    out[1] = u32x4{mx_pack4(v[4], sc), mx_pack4(v[5], sc), mx_pack4(v[6], sc), mx_pack4(v[7], sc)};
    planes[(size_t)blk * pstride + r0 + row] = (uint8_t)(xe + 127);
  }
}

hipError_t launch_mx_quantize(const float* src, void* dst, int n, int k, int r0, int total,
                              hipStream_t st) {
  const size_t blocks = (size_t)n * (k / 32);
  if (blocks == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((blocks + 255) / 256, 8192);
  mx_quantize_kernel<<<grid, 256, 0, st>>>(src, static_cast<uint8_t*>(dst), n, k, r0, total);
  return hipGetLastError();
}

}  // namespace wenc
