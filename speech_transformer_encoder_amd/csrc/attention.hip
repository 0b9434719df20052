// Bidirectional multi-head attention of the encoder block with an online softmax, head_dim 64.
//
// For each window and head: s_ij = (q_i . k_j) * hd^-0.5 over every key j of the window (no mask,
// no positional term), softmax over j, o_i = sum_j p_ij v_j (inferencelayer whisper_gpu.rs,
// VANILLA_ATTN; turbospark-runtime whisper/metal.rs, encode_layer).  As in the pages' online
// form, keys are visited tile by tile with a running max m and running denominator l, and the
// accumulated state is rescaled by exp(m_old - m_new) when m moves.  The t x t scores never reach
// memory.
//
// gfx950 mapping.  One 512-thread workgroup per (256 query rows, head, window); wavefront w owns
// 32 queries.  (Problems with fewer than 256 blocks of 128 query rows, e.g. one window, run
// workgroups of 128 query rows whose eight wavefronts form two groups over the two halves of the
// keys, and split the keys again over two workgroups when there are fewer than 128 blocks.)
// Keys go in tiles of 64 through three LDS stages, each a K tile and a V tile of 64 rows x 128
// bytes, loaded global -> LDS directly (buffer_load_dwordx4 ... lds, range-checked
// so that keys past t read as zeros) two tiles ahead of their use.  Chunk c (16 bytes) of row r
// sits at slot c ^ f(r), f chosen per tile so that the 16-lane phases of its reads hit distinct
// banks.  The scores are computed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16: lane l
// then holds 32 scores of one query (l % 32), and (m, l) of a query live in one lane's
// registers.  The probabilities stay in registers and feed O^T = V^T . P^T as the MFMA's B
// operand; the V^T fragments come straight from the row-major V tile with ds_read_b64_tr_b16
// (within each group of 16 lanes, lane i receives element i & 3 of the 8-byte rows addressed by
// lanes 4s + (i >> 2), s = 0..3), so V is never transposed in memory.  The row sums are taken
// from the rounded probabilities the MFMA consumes (v_dot2 against (1, 1)), so the numerator and
// denominator see the same values.
//
// Scores are scaled by hd^-0.5 * log2(e) so the exponentials are v_exp_f32 (exp2).  A tile is
// first exponentiated against the running max m as it stands: when every probability of a lane
// stays below 2^15 (checked through the lane's sum of them, which bounds each term), m is kept
// and no per-tile max is needed.  Otherwise (the first tile, or a score more than ~10 log2 units
// above m) the tile's true max is taken, m is raised, the running state is rescaled by
// exp2(m_old - m_new) and the tile is exponentiated again.  Both cases compute the same softmax up
// to rounding; the rescale and the max run only on the few tiles that need them.
//
// The fp32 variant keeps the score layout with v_mfma_f32_32x32x2_f32; with one k per lane it
// reads V in its natural [key][dim] layout.
#include "wenc_device.h"
#include "wenc_internal.h"

namespace wenc {

// Query rows per workgroup: 32 per wavefront, NW = 8 wavefronts (fewer when a problem has too
// few query blocks to fill the GPU, e.g. one 1500-position window).
constexpr int AK = 64;    // keys per tile
constexpr int ATILE = AK * 64;  // 16-bit elements of one K or V tile
constexpr float P_BOUND = 32768.0f;  // largest probability kept without raising the max (2^15)

typedef __attribute__((address_space(3))) void lds_void_a;
typedef short short4_t __attribute__((ext_vector_type(4)));

// Rows of window wi: equal windows of tmax rows (cu == nullptr), or rows cu[wi] .. cu[wi + 1] - 1
// of a packed ragged batch of `total` rows.  False (the workgroup has nothing to do) when the
// workgroup's first query row q0 lies past the window, or when the offsets break
// 0 <= cu[wi] <= cu[wi + 1] <= total, cu[wi + 1] - cu[wi] <= tmax: then the window is skipped and
// nothing outside [0, total) is ever addressed.  Uniform over the workgroup, taken before any
// LDS use or barrier.
__device__ __forceinline__ bool window_rows(const int* cu, int total, int wi, int tmax, int q0,
                                            size_t& win, int& t) {
  if (cu == nullptr) {
    win = (size_t)wi * tmax;
    t = tmax;
    return true;
  }
  const int s0 = cu[wi], s1 = cu[wi + 1];
  if (s0 < 0 || s1 < s0 || s1 > total || s1 - s0 > tmax) return false;
  win = (size_t)s0;
  t = s1 - s0;
  return q0 < t;
}

template <typename T> struct RowSum;
template <> struct RowSum<f16_t> {
  static __device__ __forceinline__ float add(uint32_t p2, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p2), one, acc, false);
  }
};
template <> struct RowSum<bf16_t> {
  static __device__ __forceinline__ float add(uint32_t p2, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p2), one, acc, false);
  }
};

// kvs = 1: O = softmax(.) V, normalised, in T.  kvs = 2 (too few query blocks to fill the GPU):
// each query block's keys are split in two halves handled by two workgroups, which write the
// unnormalised partial O (fp32) and their (m, l) to `part`; attn_merge_kernel combines them.
// total: rows of the packed batch (batch * tmax for equal windows).
// KS = 2: the NW wavefronts form two groups of NW / 2 over the same query rows, each running
// the recurrence over its own half of the workgroup's key tiles through its own LDS stages; at
// the end the second group hands its (O, m, l) to the first through LDS, which merges them as
// attn_merge_kernel does.  This doubles the wavefronts a small grid runs (one window) without
// the partial results going through memory.  Its 96 KB of stages keep one workgroup per CU.
// Eight-wavefront workgroups of one group run two per CU (four wavefronts per SIMD, 128 VGPRs
// each); the two-group form (grids smaller than the GPU) keeps two wavefronts per SIMD.
template <typename T, int NW, int KS = 1>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 8 && KS == 1 ? 4 : 2, NW == 8 && KS == 1 ? 4 : 2))) void attn16_kernel(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ Kp,
                                                        const uint16_t* __restrict__ Vp, int ld,
                                                        uint16_t* __restrict__ O, int ldo, int tmax,
                                                        int heads, float c,
                                                        const int* __restrict__ cu, int total,
                                                        int kvs, float* __restrict__ part) {
  static_assert(KS == 1 || KS == 2, "one or two key groups");
  constexpr int NQ = NW / KS;  // wavefronts of one key group (one per 32 query rows)
  // Three stages of 2 * ATILE elements (a K and a V tile) per key group.
  __shared__ __attribute__((aligned(1024))) uint16_t st0_all[KS * 3 * 2 * ATILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int frow = lane & 31;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = KS == 1 ? 0 : wave_all / NQ;  // key group
  const int wave = KS == 1 ? wave_all : wave_all % NQ;  // wavefront within its group
  // The group's stages.
  const uint16_t* st0 = st0_all + kg * 6 * ATILE;
  const uint16_t* st1 = st0 + 2 * ATILE;
  const uint16_t* st2 = st0 + 4 * ATILE;
  // 1-D grid over (query block, head, window), renumbered so that the query blocks of one
  // (window, head) run on the same XCD and read its K and V through one L2.
  constexpr int AQ = 32 * NQ;  // query rows of the workgroup
  constexpr int CPW = 8 / NQ;   // 8-row blocks of each K and V tile a wavefront copies
  const int nqb = (tmax + AQ - 1) / AQ;
  const int vk = xcd_virtual_id(blockIdx.x, gridDim.x);
  const int half = vk % kvs, v = vk / kvs;  // the two halves of a query block are neighbours
  const int qb = v % nqb;
  const int h = (v / nqb) % heads;
  const int wi = v / (nqb * heads);
  size_t win;  // first row of this window
  int t;       // its length
  if (!window_rows(cu, total, wi, tmax, qb * AQ, win, t)) return;
  const int col0 = h * 64;

  // Query fragments: B operand of S^T, lane holds q = lane%32, dims 16s + 8g .. +7.
  const int qi = qb * AQ + wave * 32 + frow;
  u32x4 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qf[s] = (qi < t) ? *reinterpret_cast<const u32x4*>(Q + (win + qi) * ld + col0 + s * 16 + g * 8)
                     : u32x4{0, 0, 0, 0};
  // Wait for the query fragments here, once, and hand them to the loop as plain register values
  // (otherwise the wait for them lands inside the key loop and stalls on the tile copies).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
  for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(qf[s]));

  // K and V: the window's rows of this head; rows at or past t read as zeros.  The whole offset
  // (key row included) is in the range-checked VGPR offset.  Wavefront w copies rows
  // 8w .. 8w + 7 of each tile: lane l row r = 8w + (l >> 3), slot (l & 7), which holds chunk
  // (l & 7) ^ f(r):
  //   K: f(r) = (r >> 1) & 7           (32-row x 16-byte fragment reads)
  //   V: f(r) = ((r >> 1) & 1) << 2    (8-byte transposing reads of 4 rows x 4 chunks)
  const uint32_t nrec = (uint32_t)((t - 1) * ld * 2 + 128);
  const u32x4 rK = buffer_rsrc(Kp + win * ld + col0, nrec);
  const u32x4 rV = buffer_rsrc(Vp + win * ld + col0, nrec);
  const int lr = 8 * wave + (lane >> 3);
  const int kvo = lr * ld * 2 + (((lane & 7) ^ ((lr >> 1) & 7)) << 4);
  const int vvo = lr * ld * 2 + (((lane & 7) ^ (((lr >> 1) & 1) << 2)) << 4);
  // With NQ < 8 wavefront w also copies rows 8 (w + NQ i) .. + 7, i < CPW: a shift by a multiple
  // of 16 rows leaves both swizzles unchanged.
  const uint32_t blk = (uint32_t)wave * 1024u;
  // This workgroup's key tiles: all of the window's, or one half of them (kvs = 2); with KS = 2
  // the first ceil(n / 2) of those n go to group 0, the rest to group 1.  Both groups run
  // nloop iterations (one barrier each); a group with fewer tiles idles through its last one.
  const int ntile_all = (t + AK - 1) / AK;
  const int per = (ntile_all + kvs - 1) / kvs;
  const int kt0w = min(ntile_all, half * per);
  const int ntiles_w = min(ntile_all, kt0w + per) - kt0w;
  const int nloop = (ntiles_w + KS - 1) / KS;
  const int kt0 = kt0w + kg * nloop;
  const int ntiles = KS == 1 ? ntiles_w : max(0, min(nloop, ntiles_w - kg * nloop));
  const int kbase = kt0 * AK;  // first key
  auto load_tile = [&](int j0, const uint16_t* st) {
    const uint32_t base = lds_addr(st) + blk;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int ro = (j0 + 8 * NQ * i) * ld * 2;
      lds_copy16(rK, base + (uint32_t)(NQ * i) * 1024u, kvo + ro);
      lds_copy16(rV, base + ATILE * 2 + (uint32_t)(NQ * i) * 1024u, vvo + ro);
    }
  };

  const int xk = (lane >> 1) & 7;  // K fragment-read swizzle of row (lane & 31)
  // V^T fragment source address for (kstep, db, jj): this lane's 8-byte row piece is key
  // 16 kstep + 8 jj + 4 g + s, dims db * 32 + 16 (q & 1) + 4 u  (q = lane >> 4, s, u from lane).
  const int vq = (lane >> 4) & 1, vs = (lane >> 2) & 3, vu = lane & 3;
  int vro[2][2];  // byte offset inside the V tile for kstep 0, [jj][db]
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int key = 8 * jj + 4 * g + vs;  // + 16 kstep: does not change ((key >> 1) & 1)
    const int fbit = (key >> 1) & 1;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      // chunk 2 vq + (vu >> 1) + 4 db, at slot chunk ^ (fbit << 2)
      const int slot = 2 * vq + (vu >> 1) + 4 * (db ^ fbit);
      vro[jj][db] = key * 128 + slot * 16 + (vu & 1) * 8;
    }
  }

  f32x16 oacc[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[a][r] = 0.f;
  float m_run = -INFINITY;  // max used in the exponents (scaled units), per query
  float l_part = 0.f;       // this lane's share of the running denominator

  // Tile it's copies have landed (this wavefront's: only tile it + 1's may still be in flight)
  // and, after the barrier, every wavefront's; the tile two ahead is then loaded into `ahead`,
  // whose previous tile every wavefront of the group is done with.
  auto sync_tile = [&](int it, const uint16_t* ahead) {
    if (it + 1 < ntiles)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * CPW));  // the copies of tile it + 1 may be in flight
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (it + 2 < ntiles) load_tile(kbase + (it + 2) * AK, ahead);
  };

  // S^T = K . Q^T for the 64 keys of tile it x 32 queries.
  f32x16 sacc[2];
  auto scores = [&](int it, const uint16_t* cur) {
    const int j0 = kbase + it * AK;
    const char* kb = reinterpret_cast<const char*>(cur);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(kb + (mb * 32 + frow) * 128 +
                                                         (((2 * s + g) ^ xk) << 4));
        sacc[mb] = mfma32x32x16<T>(ka, qf[s], s == 0 ? f32x16{} : sacc[mb]);
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
  };

  // Probabilities of sacc against the running max, packed for the MFMA (pb), and the running
  // state updated; the max is raised first when the probabilities would pass the bound.
  u32x4 pb[4];
  auto softmax = [&]() {
    float tsum;
    auto exponentiate = [&]() {
      float ts[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial sums (shorter chains)
#pragma unroll
      for (int kstep = 0; kstep < 4; ++kstep) {
        const int mb = kstep >> 1, js = kstep & 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(sacc[mb][8 * js + 2 * e], c, -m_run));
          const float p1 = fast_exp2(fmaf(sacc[mb][8 * js + 2 * e + 1], c, -m_run));
          pb[kstep][e] = pack2<T>(p0, p1);
          ts[e] = RowSum<T>::add(pb[kstep][e], ts[e]);
        }
      }
      tsum = (ts[0] + ts[1]) + (ts[2] + ts[3]);
    };
    exponentiate();
    if (__builtin_amdgcn_ballot_w64(!(tsum <= P_BOUND))) {
      // Raise the max to the tile's (only for the queries whose probabilities ran past the
      // bound), rescale the running state and exponentiate again.
      float mx = sacc[0][0];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = (mb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, sacc[mb][r]);
      mx = halves_max(mx) * c;
      const bool raise = !(halves_max(tsum) <= P_BOUND);
      const float m_new = raise ? fmaxf(m_run, mx) : m_run;
      const float corr = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_part *= corr;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[a][r] *= corr;
      exponentiate();
    }
    l_part += tsum;
  };

  // O^T += V^T . P^T, 4 steps of 16 keys; V^T fragments by transposing reads.
  auto pv = [&](const uint16_t* cur) {
    const uint16_t* vtile = cur + ATILE;
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int off = kstep * 16 * 128;  // 16 keys per step
        const short4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(vtile + (vro[0][db] + off) / 2));
        const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(vtile + (vro[1][db] + off) / 2));
        const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
        const u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
        oacc[db] = mfma32x32x16<T>(va, pb[kstep], oacc[db]);
      }
    }
  };

  // One key tile per iteration from stage `cur`: scores, softmax, P.V.
  if (ntiles > 0) load_tile(kbase, st0);
  if (ntiles > 1) load_tile(kbase + AK, st1);
  // A wavefront whose 32 query rows all lie past the window (the last query block's) only
  // copies and keeps the barriers.
  const bool no_rows = qb * AQ + wave * 32 >= t;
  auto tile = [&](int it, const uint16_t* cur, const uint16_t* ahead) {
    sync_tile(it, ahead);
    if (KS > 1 && it >= ntiles) return;  // this group's tiles are done; the other's are not
    if (no_rows) return;
    scores(it, cur);
    softmax();
    pv(cur);
  };
  int it = 0;
  for (; it + 3 <= nloop; it += 3) {
    tile(it, st0, st2);
    tile(it + 1, st1, st0);
    tile(it + 2, st2, st1);
  }
  if (it < nloop) tile(it, st0, st2);
  if (it + 1 < nloop) tile(it + 1, st1, st0);

  if constexpr (KS == 2) {
    // Group 1 hands (O, m, l) to group 0 through group 0's stages, which every wavefront is done
    // with after the barrier: O as 32 values per lane (8 KB per wavefront), then m and l per
    // lane.  Group 0 rescales both to the larger max, exp2(m_g - m) (zero for a group without
    // keys).
    __syncthreads();
    float* xo = reinterpret_cast<float*>(st0_all) + wave * (32 * 64) + lane;
    float* xml = reinterpret_cast<float*>(st0_all + 4 * ATILE) + wave * 128 + lane;
    if (kg == 1) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(a * 16 + r) * 64] = oacc[a][r];
      xml[0] = m_run;
      xml[64] = l_part;
    }
    __syncthreads();
    if (kg == 1) return;
    const float m1 = xml[0], l1 = xml[64];
    const float m = fmaxf(m_run, m1);
    const float c0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m);
    const float c1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - m);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[a][r] = oacc[a][r] * c0 + xo[(a * 16 + r) * 64] * c1;
    l_part = l_part * c0 + l1 * c1;
    m_run = m;
  }

  if (kvs > 1) {
    // Partial state of this half: unnormalised O (fp32) [half][row][head][64], then (m, l)
    // [half][row][head][2], rows numbered as in the packed batch.
    const float l_all = halves_sum(l_part);
    if (qi < t) {
      const size_t slot = ((size_t)half * total + win + qi) * heads + h;
      float* po = part + slot * 64;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dim = db * 32 + j * 8 + g * 4;
          *reinterpret_cast<float4*>(po + dim) = make_float4(oacc[db][4 * j], oacc[db][4 * j + 1],
                                                            oacc[db][4 * j + 2], oacc[db][4 * j + 3]);
        }
      if (g == 0) {
        float* pml = part + (size_t)kvs * total * heads * 64 + slot * 2;
        *reinterpret_cast<float2*>(pml) = make_float2(m_run, l_all);
      }
    }
    return;
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

constexpr int AQ32 = 128;  // query rows per workgroup of the fp32 kernel
constexpr int AFLDS = 66;  // fp32 LDS row stride

__global__ __launch_bounds__(256) void attn32_kernel(const float* __restrict__ Q,
                                                     const float* __restrict__ Kp,
                                                     const float* __restrict__ Vp, int ld,
                                                     float* __restrict__ O, int ldo, int tmax,
                                                     float c, const int* __restrict__ cu,
                                                     int total) {
  __shared__ __attribute__((aligned(16))) float ks[2][AK * AFLDS];
  __shared__ __attribute__((aligned(16))) float vs[2][AK * AFLDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int wave = tid >> 6;
  const int h = blockIdx.y;
  size_t win;
  int t;
  if (!window_rows(cu, total, blockIdx.z, tmax, blockIdx.x * AQ32, win, t)) return;
  const int col0 = h * 64;

  // B operand of S^T: lane holds q = lane%32 and dims 4s + 2g, 4s + 2g + 1 for s = 0..15.
  const int qi = blockIdx.x * AQ32 + wave * 32 + (lane & 31);
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

// Combines the two key halves of a split attention: per (row, head), with a_h = exp2(m_h - m),
// m = max(m_0, m_1), O = (a_0 O_0 + a_1 O_1) / (a_0 l_0 + a_1 l_1), which is the softmax over
// all keys (the same recurrence the online form runs tile by tile, applied once more).  One
// 64-lane wavefront per (window, head, 4 rows): 16 lanes per row, 4 dims each.  Windows whose
// offsets are invalid are skipped, as in the attention kernel.
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part,
                                                         uint16_t* __restrict__ O, int ldo,
                                                         int tmax, int heads,
                                                         const int* __restrict__ cu, int total) {
  const int wi = blockIdx.z, h = blockIdx.y;
  const int i = (blockIdx.x * 256 + threadIdx.x) >> 4;  // row within the window
  const int dim = (threadIdx.x & 15) * 4;
  size_t win;
  int t;
  if (!window_rows(cu, total, wi, tmax, blockIdx.x * 16, win, t) || i >= t) return;
  const size_t s0 = (win + i) * heads + h, s1 = ((size_t)total + win + i) * heads + h;
  const float* ml = part + (size_t)2 * total * heads * 64;
  const float2 a = *reinterpret_cast<const float2*>(ml + s0 * 2);
  const float2 b = *reinterpret_cast<const float2*>(ml + s1 * 2);
  const float m = fmaxf(a.x, b.x);
  const float ca = fast_exp2(a.x - m), cb = fast_exp2(b.x - m);
  const float inv = 1.0f / (ca * a.y + cb * b.y);
  const float4 oa = *reinterpret_cast<const float4*>(part + s0 * 64 + dim);
  const float4 ob = *reinterpret_cast<const float4*>(part + s1 * 64 + dim);
  u32x2 w = {pack2<T>((ca * oa.x + cb * ob.x) * inv, (ca * oa.y + cb * ob.y) * inv),
             pack2<T>((ca * oa.z + cb * ob.z) * inv, (ca * oa.w + cb * ob.w) * inv)};
  *reinterpret_cast<u32x2*>(O + (win + i) * ldo + h * 64 + dim) = w;
}

// Query blocks of 128 rows (four-wavefront workgroups) per (window, head) over the batch.
static long query_blocks128(int batch, int t, int heads) {
  return (long)((t + 127) / 128) * heads * batch;
}

int attention_split(int batch, int t, int heads, int dtype) {
  // Fewer than 128 blocks of 128 query rows (one 1500-position window with 6 or 8 heads) leave
  // most of a 256-CU GPU idle: the keys of each block are then split in two halves.  Measured
  // on one window: 6 heads 20.4 -> 18.2 us, 8 heads 20.7 -> 19.3 us (merge included); at 12 and
  // 20 heads (144, 240 blocks) the split costs more than it gains.
  if (dtype == DT_F32) return 1;
  return query_blocks128(batch, t, heads) < 128 ? 2 : 1;
}

hipError_t launch_attention(const void* q, const void* k, const void* v, int ld_qkv, void* o,
                            int ld_o, int batch, int t, int heads, float scale, int dtype,
                            hipStream_t st, const int* cu, int total, float* part) {
  if (batch == 0 || t == 0) return hipSuccess;
  if (!cu) total = batch * t;
  const int kvs = part ? attention_split(batch, t, heads, dtype) : 1;
  const float c = scale * 1.4426950408889634f;  // fold log2(e): exp(x) = exp2(x * log2 e)
  // Eight wavefronts per workgroup: over 256 query rows (two workgroups per CU) once there are
  // at least 256 blocks of 128 rows; below that, over 128 query rows in two key groups (KS = 2,
  // one workgroup per CU), which runs twice the wavefronts on the same rows.  Measured on one
  // window against the four-wavefront workgroups of one group used before (which themselves
  // beat eight-wavefront ones of 256 rows there: 23.1 against 31.4 us at 20 heads): 6 heads
  // 20.0 -> 18.2 us, 8 heads 19.8 -> 18.2, 12 heads 20.4 -> 18.4, 20 heads 21.6 -> 19.7.
  const bool ks2 = query_blocks128(batch, t, heads) < 256;
  const long nblk = (long)((t + (ks2 ? 127 : 255)) / (ks2 ? 128 : 256)) * heads * batch * kvs;
  dim3 grid((t + AQ32 - 1) / AQ32, heads, batch), block(256);
  auto run16 = [&](auto tag) {
    using T = decltype(tag);
    const auto Qp = static_cast<const uint16_t*>(q);
    const auto Kp = static_cast<const uint16_t*>(k);
    const auto Vp = static_cast<const uint16_t*>(v);
    auto Op = static_cast<uint16_t*>(o);
    const dim3 g((unsigned)nblk);
    float* pp = kvs > 1 ? part : nullptr;
    if (ks2)
      attn16_kernel<T, 8, 2><<<g, 512, 0, st>>>(Qp, Kp, Vp, ld_qkv, Op, ld_o, t, heads, c, cu,
                                                total, kvs, pp);
    else
      attn16_kernel<T, 8><<<g, 512, 0, st>>>(Qp, Kp, Vp, ld_qkv, Op, ld_o, t, heads, c, cu, total,
                                             kvs, pp);
    if (kvs > 1)
      attn_merge_kernel<T><<<dim3((unsigned)((t + 15) / 16), (unsigned)heads, (unsigned)batch), 256,
                             0, st>>>(part, Op, ld_o, t, heads, cu, total);
  };
  switch (dtype) {
    case DT_BF16: run16(bf16_t{}); break;
    case DT_F16: run16(f16_t{}); break;
    case DT_F32:
      attn32_kernel<<<grid, block, 0, st>>>(static_cast<const float*>(q),
                                            static_cast<const float*>(k),
                                            static_cast<const float*>(v), ld_qkv,
                                            static_cast<float*>(o), ld_o, t, c, cu, total);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace wenc
