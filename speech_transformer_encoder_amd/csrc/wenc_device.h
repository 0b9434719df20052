// Device-side helpers shared by the gfx950 kernels: operand vector types, fp32 -> 16-bit
// rounding, MFMA wrappers and wavefront reductions.  CDNA4 only (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wenc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-bit storage tags.  Both are held as raw uint16_t bit patterns in memory.
struct bf16_t {};
struct f16_t {};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// fp32 -> 16-bit conversions, round to nearest even.  gfx950 converts to bf16 in hardware
// (v_cvt_pk_bf16_f32), and to fp16 with v_cvt_f16_f32.
template <typename T> struct Cvt;
template <> struct Cvt<bf16_t> {
  static __device__ __forceinline__ uint32_t bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
};
template <> struct Cvt<f16_t> {
  static __device__ __forceinline__ uint32_t bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
};

// Two fp32 -> one packed 32-bit word (lo in bits 0..15).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return Cvt<T>::pack(lo, hi);
}

// D(32x32) += A(32x16) * B(16x32), 16-bit operands held as 4 packed dwords per lane.
// Lane l supplies A[row l%32][k 8*(l/32) .. +7] and B[k 8*(l/32) .. +7][col l%32];
// D lane l holds column l%32, rows 8*j + 4*(l/32) + i at register 4*j + i.
template <typename T>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32x32x16<bf16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32x32x16<f16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// MXFP8 operand tag (E4M3 codes with E8M0 scale planes; layout: mx_planes_offset).
struct mx8_t {};

// D(32x32) += A(32x64) * B(64x32) with E4M3 operands and E8M0 block scales
// (v_mfma_scale_f32_32x32x64_f8f6f4).  Lane l supplies 32 bytes of row l % 32 of A (and of
// column l % 32 of B): bytes 0 .. 15 hold 16 k values of 32-k block 0 and bytes 16 .. 31 16 of
// block 1, the two halves of the wavefront covering each block together; block b of row r is
// scaled by 2^(s - 127) with s the low byte of the scale register of lane r + 32 b (measured with
// exact small-integer products on gfx950).  D has the layout of the 16-bit form.
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma_mx8(u32x8 a, u32x8 b, int sa, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                         __builtin_bit_cast(i32x8, b), c, 0, 0, 0,
                                                         sa, 0, sb);
}
// An MXFP8 fragment from LDS: bytes 0 .. 15 at lo, 16 .. 31 at hi, read straight into the eight
// consecutive registers the MFMA takes.
__device__ __forceinline__ u32x8 lds_frag8(const char* lo, const char* hi) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(lo), b = *reinterpret_cast<const u32x4*>(hi);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// D(32x32) += A(32x2) * B(2x32) in fp32.  Lane l supplies A[row l%32][k l/32] and
// B[k l/32][col l%32]; D has the same layout as the 16-bit form.
__device__ __forceinline__ f32x16 mfma32x32x2_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Combine a value with the one held by lane l^32 (the other half of the wavefront).
// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes 0..31 of its
// second; with the same value in both, every lane ends up with {own, partner} across the two
// results, so a symmetric operation of the pair needs no lane-dependent select.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- MXFP8 (OCP Microscaling Formats v1.0, E4M3 elements, E8M0 scale per 32 values) ----
// (matrix layout: mx_planes_offset in wenc_internal.h)

// Scale exponent of a block whose largest magnitude is amax: the smallest X with
// amax <= 448 * 2^X (448 = 1.75 * 2^8, E4M3's largest finite value), so no element saturates;
// -127 for amax = 0 (or below the normal range), which the E8M0 range also bounds.
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int x = (int)(b >> 23) - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return x < -127 ? -127 : x;
}
// 2^-X as a float (X in [-127, 120]: a normal number).
__device__ __forceinline__ float mx_inv_scale(int x) { return __uint_as_float((uint32_t)(127 - x) << 23); }
// Four values times s -> four E4M3 codes (round to nearest even; every |v s| <= 448) in one word,
// value i in byte i.
__device__ __forceinline__ uint32_t mx_pack4(float4 v, float s) {
  uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(v.x * s, v.y * s, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(v.z * s, v.w * s, r, true);
}

// erf-GELU for outputs rounded to 16 bits or fewer: the complementary error function from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26 (Hastings' rational
// approximation, absolute error <= 1.5e-7):
//   erfc(a) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-a^2),  t = 1 / (1 + p a),  a >= 0.
// With a = |z| / sqrt 2 and w = 1 - erfc(a) = erf(a):  gelu(z) = z/2 (1 + erf(z/sqrt 2))
// = (z + |z| w) / 2 for both signs of z.  13 VALU operations (two of them transcendental).
__device__ __forceinline__ float gelu_erf_as(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.7071067811865476f, az, 1.0f));
  float q = fmaf(t, 1.061405429f, -1.453152027f);
  q = fmaf(t, q, 1.421413741f);
  q = fmaf(t, q, -0.284496736f);
  q = fmaf(t, q, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(z * (z * (-0.5f * 1.4426950408889634f)));  // exp(-a^2)
  const float w = fmaf(-(q * t), e, 1.0f);
  return 0.5f * fmaf(az, w, z);
}

// Workgroups of a 1-D grid are dispatched round-robin over the eight XCDs (id % 8).  This
// bijective renumbering gives each XCD a contiguous range of virtual ids, so workgroups that
// share operands can be placed on one XCD and share its L2.
__device__ __forceinline__ int xcd_virtual_id(int id, int nb) {
  const int q = nb >> 3, r = nb & 7;
  const int xcd = id & 7, pos = id >> 3;
  return (xcd < r) ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
}


// Global -> LDS copy of 16 bytes per lane (lane i to lds_base + 16 i) from a range-checked buffer,
// as inline assembly so that the compiler does not treat the copies in flight as possible writers
// of every later LDS read (it would wait for all of them).  M0 is listed as clobbered for the
// reader; the compiler reserves M0 (and says so in a warning, silenced here) and nothing else in
// these kernels reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(u32x4 rsrc, uint32_t lds_base, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer resource over `bytes` bytes at `base` (loads past the end return zeros).
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

}  // namespace wenc
