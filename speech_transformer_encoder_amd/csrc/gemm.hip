// Projection GEMMs of the encoder block on MFMA, with the block's element-wise steps fused into
// the epilogue.
//
// Every projection of the block is y = x . W^T + b with W in [n_out, n_in] layout: the packed
// QKV projection (K rows carry a zero bias), the output projection followed by the residual
// add, fc1 followed by erf-GELU, and fc2 followed by the residual add (inferencelayer
// whisper_gpu.rs, WhisperEncoderGpu::forward and the gemm flags "bias | act << 8";
// turbospark-runtime whisper/metal.rs, encode_layer and the fused-residual GEMV;
// oxinfer whisper/model.rs, encode).  The pages' GEMM shaders are not shown; this is a gfx950
// design of the same contraction.
//
// Both operands are K-contiguous (x rows, W rows), so the tile is computed as
// D[n][m] = W[n][:] . X[m][:]: W feeds the MFMA's A operand and X its B operand, and each lane
// of the 32x32 accumulator then owns four consecutive output columns n for one row m, which
// the epilogue reads and writes as one 8- or 16-byte vector.
//
// Tile: 128 (n) x 128 (m) x 64 (k) per 256-thread workgroup, four wavefronts in a 2 x 2 grid,
// each owning 64 x 64 outputs as 2 x 2 blocks of v_mfma_f32_32x32x16 (16-bit operands) or
// v_mfma_f32_32x32x2_f32 (fp32 operands, 32-wide k tile).  Operand tiles are staged through
// LDS, double buffered with one barrier per k tile; the next tile's global loads are issued
// before the current tile's MFMAs.  Rows are padded by 16 bytes so that the 16-byte fragment
// reads of 8 consecutive lanes hit 32 distinct banks.
#include "wenc_device.h"
#include "wenc_internal.h"

namespace wenc {

constexpr int GB_N = 128;  // W rows (output columns) per tile
constexpr int GB_M = 128;  // X rows per tile
constexpr int GB_K = 64;   // 16-bit elements of k per tile
constexpr int GLDS = GB_K + 8;  // LDS row stride in 16-bit elements (144 bytes)

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.7071067811865476f));
}

template <typename T, int EPI>
__device__ __forceinline__ void store4(void* c, const float* residual, size_t off, float4 v) {
  if constexpr (EPI == EPI_BIAS_RESIDUAL) {
    const float4 r = *reinterpret_cast<const float4*>(residual + off);
    float4 o = make_float4(r.x + v.x, r.y + v.y, r.z + v.z, r.w + v.w);
    *reinterpret_cast<float4*>(static_cast<float*>(c) + off) = o;
  } else {
    if constexpr (EPI == EPI_BIAS_GELU) {
      v.x = gelu_erf(v.x); v.y = gelu_erf(v.y); v.z = gelu_erf(v.z); v.w = gelu_erf(v.w);
    }
    u32x2 w = {pack2<T>(v.x, v.y), pack2<T>(v.z, v.w)};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(c) + off) = w;
  }
}

template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm16_kernel(const uint16_t* __restrict__ X, int lda,
                                                     const uint16_t* __restrict__ W,
                                                     const float* __restrict__ bias,
                                                     const float* residual, void* C, int ldc,
                                                     int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][(GB_N + GB_M) * GLDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int n0 = blockIdx.x * GB_N;
  const int m0 = blockIdx.y * GB_M;

  // Global -> register staging: 4 chunks of 16 bytes for each operand per thread.
  u32x4 rw[4], rx[4];
  auto gload = [&](int kt) {
    const int kbase = kt * GB_K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, col = (c & 7) * 8;
      const int n = n0 + row, m = m0 + row;
      rw[i] = (n < N) ? *reinterpret_cast<const u32x4*>(W + (size_t)n * K + kbase + col)
                      : u32x4{0, 0, 0, 0};
      rx[i] = (m < M) ? *reinterpret_cast<const u32x4*>(X + (size_t)m * lda + kbase + col)
                      : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* ws = lds[buf];
    uint16_t* xs = lds[buf] + GB_N * GLDS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(ws + row * GLDS + col) = rw[i];
      *reinterpret_cast<u32x4*>(xs + row * GLDS + col) = rx[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = K / GB_K;
  gload(0);
  lstore(0);
  __syncthreads();

  const int frow = lane & 31;
  const int fcol = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* ws = lds[buf] + (wn * 64 + frow) * GLDS + fcol;
    const uint16_t* xs = lds[buf] + GB_N * GLDS + (wm * 64 + frow) * GLDS + fcol;
#pragma unroll
    for (int s = 0; s < GB_K / 16; ++s) {
      u32x4 fa[2], fb[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        fa[b] = *reinterpret_cast<const u32x4*>(ws + b * 32 * GLDS + s * 16);
        fb[b] = *reinterpret_cast<const u32x4*>(xs + b * 32 * GLDS + s * 16);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32x32x16<T>(fa[a], fb[b], acc[a][b]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane owns column m, rows n = base + 8j + 4*(lane/32) + i (i = 0..3).
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = m0 + wm * 64 + b * 32 + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + a * 32 + j * 8 + (lane >> 5) * 4;
        if (n >= N) continue;
        const float4 bb = *reinterpret_cast<const float4*>(bias + n);
        float4 v = make_float4(acc[a][b][4 * j + 0] + bb.x, acc[a][b][4 * j + 1] + bb.y,
                               acc[a][b][4 * j + 2] + bb.z, acc[a][b][4 * j + 3] + bb.w);
        store4<T, EPI>(C, residual, (size_t)m * ldc + n, v);
      }
    }
  }
}

// Large-problem variant: 256 (n) x 256 (m) x 64 (k) tiles, four wavefronts each owning a
// 128 x 128 block of outputs (4 x 4 MFMA blocks, 256 fp32 accumulators per lane).  At this
// wave tile each 32x32x16 MFMA needs 64 bytes of fragments from LDS, a quarter of what a
// 64 x 64 wave tile needs, which keeps LDS bandwidth well below the MFMA rate.  LDS rows are
// 128 bytes with the eight 16-byte chunks of row r stored at slot (chunk ^ (r & 7)): every
// 8-lane phase of a 16-byte fragment read or write then covers all banks without padding.
// Workgroups are renumbered so that each XCD (eight of them, dispatched round-robin) gets a
// contiguous range of tiles, grouped 8 m-tiles deep, so concurrently running tiles share
// operand rows in that XCD's L2.
constexpr int BG_N = 256;
constexpr int BG_M = 256;
constexpr int BG_K = 64;
constexpr int BG_GROUP_M = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BG_K + ((chunk ^ (row & 7)) << 3); }

// Bijective renumbering of a 1-D grid so consecutive virtual ids run on the same XCD.
__device__ __forceinline__ int xcd_virtual_id(int id, int nb) {
  const int q = nb >> 3, r = nb & 7;
  const int xcd = id & 7, pos = id >> 3;
  return (xcd < r) ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
}

template <typename T, int EPI>
__global__ __launch_bounds__(256, 1) void gemm16_big_kernel(const uint16_t* __restrict__ X,
                                                            int lda,
                                                            const uint16_t* __restrict__ W,
                                                            const float* __restrict__ bias,
                                                            const float* residual, void* C,
                                                            int ldc, int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) uint16_t glds[];  // [2][(BG_N + BG_M) * BG_K]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;

  const int tiles_m = (M + BG_M - 1) / BG_M;
  const int tiles_n = (N + BG_N - 1) / BG_N;
  const int v = xcd_virtual_id(blockIdx.x, gridDim.x);
  const int group = BG_GROUP_M * tiles_n;
  const int first_m = (v / group) * BG_GROUP_M;
  const int gm = min(tiles_m - first_m, BG_GROUP_M);
  const int tm = first_m + (v % group) % gm;
  const int tn = (v % group) / gm;
  const int n0 = tn * BG_N, m0 = tm * BG_M;

  // Global -> register staging: 8 chunks of 16 bytes of each operand per thread and k tile.
  u32x4 rw[8], rx[8];
  auto gload = [&](int kt) {
    const int kbase = kt * BG_K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, col = (c & 7) * 8;
      const int n = n0 + row, m = m0 + row;
      rw[i] = (n < N) ? *reinterpret_cast<const u32x4*>(W + (size_t)n * K + kbase + col)
                      : u32x4{0, 0, 0, 0};
      rx[i] = (m < M) ? *reinterpret_cast<const u32x4*>(X + (size_t)m * lda + kbase + col)
                      : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* ws = glds + buf * (BG_N + BG_M) * BG_K;
    uint16_t* xs = ws + BG_N * BG_K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(ws + swz(row, ch)) = rw[i];
      *reinterpret_cast<u32x4*>(xs + swz(row, ch)) = rx[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = K / BG_K;
  gload(0);
  lstore(0);
  __syncthreads();

  const int frow = lane & 31;
  const int g = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* ws = glds + buf * (BG_N + BG_M) * BG_K;
    const uint16_t* xs = ws + BG_N * BG_K;
#pragma unroll
    for (int s = 0; s < BG_K / 16; ++s) {
      u32x4 fa[4], fb[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int rn = wn * 128 + b * 32 + frow;
        const int rm = wm * 128 + b * 32 + frow;
        fa[b] = *reinterpret_cast<const u32x4*>(ws + swz(rn, 2 * s + g));
        fb[b] = *reinterpret_cast<const u32x4*>(xs + swz(rm, 2 * s + g));
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma32x32x16<T>(fa[a], fb[b], acc[a][b]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int m = m0 + wm * 128 + b * 32 + frow;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 128 + a * 32 + j * 8 + g * 4;
        if (n >= N) continue;
        const float4 bb = *reinterpret_cast<const float4*>(bias + n);
        float4 v4 = make_float4(acc[a][b][4 * j + 0] + bb.x, acc[a][b][4 * j + 1] + bb.y,
                                acc[a][b][4 * j + 2] + bb.z, acc[a][b][4 * j + 3] + bb.w);
        store4<T, EPI>(C, residual, (size_t)m * ldc + n, v4);
      }
    }
  }
}

// fp32-operand fallback: same tiling with a 32-wide k tile of fp32 (128 bytes per row) and
// v_mfma_f32_32x32x2_f32.  Two consecutive k of a lane feed two MFMAs, so each fragment read
// is one 8-byte LDS load; the LDS row stride of 34 floats keeps 16 lanes on distinct banks.
constexpr int GF_K = 32;
constexpr int GFLDS = GF_K + 2;

template <int EPI>
__global__ __launch_bounds__(256) void gemm32_kernel(const float* __restrict__ X, int lda,
                                                     const float* __restrict__ W,
                                                     const float* __restrict__ bias,
                                                     const float* residual, float* C, int ldc,
                                                     int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) float lds[2][(GB_N + GB_M) * GFLDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int n0 = blockIdx.x * GB_N;
  const int m0 = blockIdx.y * GB_M;

  float4 rw[4], rx[4];
  auto gload = [&](int kt) {
    const int kbase = kt * GF_K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, col = (c & 7) * 4;
      const int n = n0 + row, m = m0 + row;
      rw[i] = (n < N) ? *reinterpret_cast<const float4*>(W + (size_t)n * K + kbase + col)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      rx[i] = (m < M) ? *reinterpret_cast<const float4*>(X + (size_t)m * lda + kbase + col)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto lstore = [&](int buf) {
    float* ws = lds[buf];
    float* xs = lds[buf] + GB_N * GFLDS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, col = (c & 7) * 4;
      *reinterpret_cast<float2*>(ws + row * GFLDS + col) = make_float2(rw[i].x, rw[i].y);
      *reinterpret_cast<float2*>(ws + row * GFLDS + col + 2) = make_float2(rw[i].z, rw[i].w);
      *reinterpret_cast<float2*>(xs + row * GFLDS + col) = make_float2(rx[i].x, rx[i].y);
      *reinterpret_cast<float2*>(xs + row * GFLDS + col + 2) = make_float2(rx[i].z, rx[i].w);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = K / GF_K;
  gload(0);
  lstore(0);
  __syncthreads();

  const int frow = lane & 31;
  const int fcol = (lane >> 5) * 2;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const float* ws = lds[buf] + (wn * 64 + frow) * GFLDS + fcol;
    const float* xs = lds[buf] + GB_N * GFLDS + (wm * 64 + frow) * GFLDS + fcol;
#pragma unroll
    for (int s = 0; s < GF_K / 4; ++s) {
      float2 fa[2], fb[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        fa[b] = *reinterpret_cast<const float2*>(ws + b * 32 * GFLDS + s * 4);
        fb[b] = *reinterpret_cast<const float2*>(xs + b * 32 * GFLDS + s * 4);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          acc[a][b] = mfma32x32x2_f32(fa[a].x, fb[b].x, acc[a][b]);
          acc[a][b] = mfma32x32x2_f32(fa[a].y, fb[b].y, acc[a][b]);
        }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = m0 + wm * 64 + b * 32 + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + a * 32 + j * 8 + (lane >> 5) * 4;
        if (n >= N) continue;
        const float4 bb = *reinterpret_cast<const float4*>(bias + n);
        float4 v = make_float4(acc[a][b][4 * j + 0] + bb.x, acc[a][b][4 * j + 1] + bb.y,
                               acc[a][b][4 * j + 2] + bb.z, acc[a][b][4 * j + 3] + bb.w);
        const size_t off = (size_t)m * ldc + n;
        if constexpr (EPI == EPI_BIAS_RESIDUAL) {
          const float4 r = *reinterpret_cast<const float4*>(residual + off);
          v = make_float4(r.x + v.x, r.y + v.y, r.z + v.z, r.w + v.w);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
          v = make_float4(gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w));
        }
        *reinterpret_cast<float4*>(C + off) = v;
      }
    }
  }
}

constexpr size_t BG_LDS_BYTES = 2 * (BG_N + BG_M) * BG_K * sizeof(uint16_t);

template <typename T, int EPI>
static void launch16_epi(const uint16_t* X, int lda, const uint16_t* W, const float* bias,
                         const float* residual, void* c, int ldc, int m, int n, int k,
                         hipStream_t st) {
  const long big_tiles = (long)((m + BG_M - 1) / BG_M) * ((n + BG_N - 1) / BG_N);
  if (big_tiles >= 384) {
    gemm16_big_kernel<T, EPI><<<dim3((unsigned)big_tiles), dim3(256), BG_LDS_BYTES, st>>>(
        X, lda, W, bias, residual, c, ldc, m, n, k);
  } else {
    dim3 grid((n + GB_N - 1) / GB_N, (m + GB_M - 1) / GB_M), block(256);
    gemm16_kernel<T, EPI><<<grid, block, 0, st>>>(X, lda, W, bias, residual, c, ldc, m, n, k);
  }
}

template <typename T>
static hipError_t launch16(const void* a, int lda, const void* w, const float* bias,
                           const float* residual, void* c, int ldc, int m, int n, int k, int epi,
                           hipStream_t st) {
  // Dynamic LDS beyond 64 KiB needs an explicit opt-in, once per kernel instantiation.
  static const hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute((const void*)gemm16_big_kernel<T, EPI_BIAS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)BG_LDS_BYTES);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gemm16_big_kernel<T, EPI_BIAS_GELU>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)BG_LDS_BYTES);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gemm16_big_kernel<T, EPI_BIAS_RESIDUAL>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)BG_LDS_BYTES);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  auto X = static_cast<const uint16_t*>(a);
  auto W = static_cast<const uint16_t*>(w);
  switch (epi) {
    case EPI_BIAS: launch16_epi<T, EPI_BIAS>(X, lda, W, bias, residual, c, ldc, m, n, k, st); break;
    case EPI_BIAS_GELU:
      launch16_epi<T, EPI_BIAS_GELU>(X, lda, W, bias, residual, c, ldc, m, n, k, st);
      break;
    case EPI_BIAS_RESIDUAL:
      launch16_epi<T, EPI_BIAS_RESIDUAL>(X, lda, W, bias, residual, c, ldc, m, n, k, st);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static hipError_t launch32(const void* a, int lda, const void* w, const float* bias,
                           const float* residual, void* c, int ldc, int m, int n, int k, int epi,
                           hipStream_t st) {
  dim3 grid((n + GB_N - 1) / GB_N, (m + GB_M - 1) / GB_M), block(256);
  auto X = static_cast<const float*>(a);
  auto W = static_cast<const float*>(w);
  auto C = static_cast<float*>(c);
  switch (epi) {
    case EPI_BIAS:
      gemm32_kernel<EPI_BIAS><<<grid, block, 0, st>>>(X, lda, W, bias, residual, C, ldc, m, n, k);
      break;
    case EPI_BIAS_GELU:
      gemm32_kernel<EPI_BIAS_GELU><<<grid, block, 0, st>>>(X, lda, W, bias, residual, C, ldc, m, n, k);
      break;
    case EPI_BIAS_RESIDUAL:
      gemm32_kernel<EPI_BIAS_RESIDUAL><<<grid, block, 0, st>>>(X, lda, W, bias, residual, C, ldc, m,
                                                               n, k);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_linear(const void* a, int lda, const void* w, const float* bias,
                         const float* residual, void* c, int ldc, int m, int n, int k, int dtype,
                         int epilogue, hipStream_t st) {
  if (m == 0) return hipSuccess;
  switch (dtype) {
    case DT_BF16: return launch16<bf16_t>(a, lda, w, bias, residual, c, ldc, m, n, k, epilogue, st);
    case DT_F16: return launch16<f16_t>(a, lda, w, bias, residual, c, ldc, m, n, k, epilogue, st);
    case DT_F32: return launch32(a, lda, w, bias, residual, c, ldc, m, n, k, epilogue, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace wenc
