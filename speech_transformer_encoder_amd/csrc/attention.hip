// Bidirectional multi-head attention of the encoder block with an online softmax, head_dim 64.
//
// For each window and head: s_ij = (q_i . k_j) * hd^-0.5 over every key j of the window (no mask,
// no positional term), softmax over j, o_i = sum_j p_ij v_j (inferencelayer whisper_gpu.rs,
// VANILLA_ATTN; turbospark-runtime whisper/metal.rs, encode_layer).  As in the pages' online
// form, keys are visited tile by tile with a running max m and running denominator l: each tile
// rescales the previous state by exp(m_old - m_new).  The t x t scores never reach memory.
//
// gfx950 mapping.  One 256-thread workgroup per (128 query rows, head, window); wavefront w owns
// 32 query rows.  Keys go in tiles of 64, double-buffered in LDS.  The scores are computed
// transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16: lane l then holds 32 scores of one query
// (l % 32), so the row max and sum are 31 in-register operations plus one exchange with lane
// l ^ 32 (v_permlane32_swap), and the running (m, l) of a query live in one lane's registers.
// The probabilities stay in registers and feed O^T = V^T . P^T directly as the MFMA's B
// operand: the 8 keys a lane contributes per MFMA step are exactly the 8 score registers it
// already holds, provided V^T is laid out with the same key order.  The V tile is therefore
// transposed into LDS as [dim][key] with keys permuted inside each group of 16
// (0-3, 8-11, 4-7, 12-15), which makes every A-operand fragment one 16-byte LDS read.
// Scores are scaled by hd^-0.5 * log2(e) so the exponentials are v_exp_f32 (exp2).
//
// The fp32 variant keeps the same structure with v_mfma_f32_32x32x2_f32; with one k per lane
// it reads V in its natural [key][dim] layout.
#include "wenc_device.h"
#include "wenc_internal.h"

namespace wenc {

constexpr int AQ = 128;   // query rows per workgroup
constexpr int AK = 64;    // keys per tile
constexpr int ALDS = 72;  // LDS row stride (16-bit elements) for K [key][dim] and V^T [dim][key]

__device__ __forceinline__ int vt_pos(int r) {  // key r (0..15) -> position inside its 16-group
  return (r & 3) | (((r >> 2) & 1) << 3) | (((r >> 3) & 1) << 2);
}

template <typename T>
__global__ __launch_bounds__(256) void attn16_kernel(const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ Kp,
                                                     const uint16_t* __restrict__ Vp, int ld,
                                                     uint16_t* __restrict__ O, int ldo, int t,
                                                     float c) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][AK * ALDS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][64 * ALDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int wave = tid >> 6;
  const int h = blockIdx.y;
  const size_t win = (size_t)blockIdx.z * t;  // first row of this window
  const int col0 = h * 64;

  // Query fragments: B operand of S^T, lane holds q = lane%32, dims 16s + 8g .. +7.
  const int qi = blockIdx.x * AQ + wave * 32 + (lane & 31);
  u32x4 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qf[s] = (qi < t) ? *reinterpret_cast<const u32x4*>(Q + (win + qi) * ld + col0 + s * 16 + g * 8)
                     : u32x4{0, 0, 0, 0};

  // Tile loaders.  K: 2 chunks of 16 bytes per thread.  V: keys (2kp, 2kp+1), dims 8dc..8dc+7.
  u32x4 rk[2], rv[2];
  const int kp = tid >> 3, dc = tid & 7;
  auto gload = [&](int j0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cidx = tid + 256 * i;
      const int key = j0 + (cidx >> 3);
      rk[i] = (key < t) ? *reinterpret_cast<const u32x4*>(Kp + (win + key) * ld + col0 + (cidx & 7) * 8)
                        : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = j0 + 2 * kp + i;
      rv[i] = (key < t) ? *reinterpret_cast<const u32x4*>(Vp + (win + key) * ld + col0 + dc * 8)
                        : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cidx = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&ks[buf][(cidx >> 3) * ALDS + (cidx & 7) * 8]) = rk[i];
    }
    const int kk = 2 * kp;
    const int pos = (kk & ~15) + vt_pos(kk & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // dims 8dc + 2e and 8dc + 2e + 1: pair the two keys' values of each dim.
      const uint32_t a = rv[0][e], b = rv[1][e];
      const uint32_t lo = (a & 0xffffu) | (b << 16);
      const uint32_t hi = (a >> 16) | (b & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(&vt[buf][(dc * 8 + 2 * e) * ALDS + pos]) = lo;
      *reinterpret_cast<uint32_t*>(&vt[buf][(dc * 8 + 2 * e + 1) * ALDS + pos]) = hi;
    }
  };

  f32x16 oacc[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[a][r] = 0.f;
  float m_run = -INFINITY;  // running max of s * c
  float l_part = 0.f;       // this lane's share of the running denominator

  const int ntiles = (t + AK - 1) / AK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int frow = lane & 31;
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int j0 = it * AK;
    if (it + 1 < ntiles) gload(j0 + AK);

    // S^T = K . Q^T for 64 keys x 32 queries.
    f32x16 sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[mb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4 ka =
            *reinterpret_cast<const u32x4*>(&ks[buf][(mb * 32 + frow) * ALDS + s * 16 + g * 8]);
        sacc[mb] = mfma32x32x16<T>(ka, qf[s], sacc[mb]);
      }
    }
    if (j0 + AK > t) {  // last tile: keys past the window get no weight
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + mb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          if (key >= t) sacc[mb][r] = -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mb][r]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float corr = fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[mb][r], c, -m_new));
        sacc[mb][r] = p;
        psum += p;
      }
    l_part = l_part * corr + psum;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[a][r] *= corr;

    // O^T += V^T . P^T, 4 steps of 16 keys.
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const int mb = kstep >> 1, js = kstep & 1;
      u32x4 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pb[e] = pack2<T>(sacc[mb][8 * js + 2 * e], sacc[mb][8 * js + 2 * e + 1]);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const u32x4 va =
            *reinterpret_cast<const u32x4*>(&vt[buf][(db * 32 + frow) * ALDS + kstep * 16 + g * 8]);
        oacc[db] = mfma32x32x16<T>(va, pb, oacc[db]);
      }
    }

    if (it + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  const float inv = 1.0f / halves_sum(l_part);
  if (qi < t) {
    uint16_t* orow = O + (win + qi) * ldo + col0;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dim = db * 32 + j * 8 + g * 4;
        u32x2 w = {pack2<T>(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv),
                   pack2<T>(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + dim) = w;
      }
  }
}

constexpr int AFLDS = 66;  // fp32 LDS row stride

__global__ __launch_bounds__(256) void attn32_kernel(const float* __restrict__ Q,
                                                     const float* __restrict__ Kp,
                                                     const float* __restrict__ Vp, int ld,
                                                     float* __restrict__ O, int ldo, int t,
                                                     float c) {
  __shared__ __attribute__((aligned(16))) float ks[2][AK * AFLDS];
  __shared__ __attribute__((aligned(16))) float vs[2][AK * AFLDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int wave = tid >> 6;
  const int h = blockIdx.y;
  const size_t win = (size_t)blockIdx.z * t;
  const int col0 = h * 64;

  // B operand of S^T: lane holds q = lane%32 and dims 4s + 2g, 4s + 2g + 1 for s = 0..15.
  const int qi = blockIdx.x * AQ + wave * 32 + (lane & 31);
  float2 qf[16];
#pragma unroll
  for (int s = 0; s < 16; ++s)
    qf[s] = (qi < t) ? *reinterpret_cast<const float2*>(Q + (win + qi) * ld + col0 + 4 * s + 2 * g)
                     : make_float2(0.f, 0.f);

  // 64 rows x 16 float4 per tile and operand: 4 per thread.
  float4 rk[4], rv[4];
  auto gload = [&](int j0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = tid + 256 * i;
      const int key = j0 + (cidx >> 4);
      const size_t off = (win + key) * ld + col0 + (cidx & 15) * 4;
      rk[i] = (key < t) ? *reinterpret_cast<const float4*>(Kp + off) : make_float4(0, 0, 0, 0);
      rv[i] = (key < t) ? *reinterpret_cast<const float4*>(Vp + off) : make_float4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = tid + 256 * i;
      const int o = (cidx >> 4) * AFLDS + (cidx & 15) * 4;
      *reinterpret_cast<float2*>(&ks[buf][o]) = make_float2(rk[i].x, rk[i].y);
      *reinterpret_cast<float2*>(&ks[buf][o + 2]) = make_float2(rk[i].z, rk[i].w);
      *reinterpret_cast<float2*>(&vs[buf][o]) = make_float2(rv[i].x, rv[i].y);
      *reinterpret_cast<float2*>(&vs[buf][o + 2]) = make_float2(rv[i].z, rv[i].w);
    }
  };

  f32x16 oacc[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[a][r] = 0.f;
  float m_run = -INFINITY;
  float l_part = 0.f;

  const int ntiles = (t + AK - 1) / AK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int frow = lane & 31;
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int j0 = it * AK;
    if (it + 1 < ntiles) gload(j0 + AK);

    f32x16 sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[mb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const float2 ka =
            *reinterpret_cast<const float2*>(&ks[buf][(mb * 32 + frow) * AFLDS + 4 * s + 2 * g]);
        sacc[mb] = mfma32x32x2_f32(ka.x, qf[s].x, sacc[mb]);
        sacc[mb] = mfma32x32x2_f32(ka.y, qf[s].y, sacc[mb]);
      }
    }
    if (j0 + AK > t) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + mb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          if (key >= t) sacc[mb][r] = -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mb][r]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float corr = fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[mb][r], c, -m_new));
        sacc[mb][r] = p;
        psum += p;
      }
    l_part = l_part * corr + psum;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[a][r] *= corr;

    // O^T += V^T . P^T: one key per lane per step; lane half g contributes key
    // mb*32 + 8j + 4g + i, which is the score it holds in register 4j + i.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = mb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const float va = vs[buf][key * AFLDS + db * 32 + frow];
          oacc[db] = mfma32x32x2_f32(va, sacc[mb][r], oacc[db]);
        }
      }

    if (it + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  const float inv = 1.0f / halves_sum(l_part);
  if (qi < t) {
    float* orow = O + (win + qi) * ldo + col0;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dim = db * 32 + j * 8 + g * 4;
        *reinterpret_cast<float4*>(orow + dim) =
            make_float4(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                        oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
      }
  }
}

hipError_t launch_attention(const void* q, const void* k, const void* v, int ld_qkv, void* o,
                            int ld_o, int batch, int t, int heads, float scale, int dtype,
                            hipStream_t st) {
  if (batch == 0 || t == 0) return hipSuccess;
  const float c = scale * 1.4426950408889634f;  // fold log2(e): exp(x) = exp2(x * log2 e)
  dim3 grid((t + AQ - 1) / AQ, heads, batch), block(256);
  switch (dtype) {
    case DT_BF16:
      attn16_kernel<bf16_t><<<grid, block, 0, st>>>(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
          static_cast<const uint16_t*>(v), ld_qkv, static_cast<uint16_t*>(o), ld_o, t, c);
      break;
    case DT_F16:
      attn16_kernel<f16_t><<<grid, block, 0, st>>>(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
          static_cast<const uint16_t*>(v), ld_qkv, static_cast<uint16_t*>(o), ld_o, t, c);
      break;
    case DT_F32:
      attn32_kernel<<<grid, block, 0, st>>>(static_cast<const float*>(q),
                                            static_cast<const float*>(k),
                                            static_cast<const float*>(v), ld_qkv,
                                            static_cast<float*>(o), ld_o, t, c);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace wenc
