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
// D[n][m] = W[n][:] . X[m][:]: W feeds the MFMA's A operand and X its B operand.
//
// 16-bit operands (bf16 or fp16).  One 512-thread workgroup (8 wavefronts, two per SIMD) owns a
// 256 (n) x 256 (m) output tile; wavefront w owns 64 (n) x 128 (m) of it as 2 x 4 blocks of
// v_mfma_f32_32x32x16 with 128 fp32 accumulators per lane.  k advances in tiles of 64:
//   * operand tiles go global -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging), into one
//     of two 64 KB stages; buffer range checks return zeros for rows past M or N;
//   * an LDS row is 128 bytes (64 k values) held as eight 16-byte chunks, chunk c of row r at
//     slot c ^ ((r >> 1) & 7): each 16-lane phase of a fragment read then covers the 64 banks once;
//   * the fragments of the next 16-k step are read while the MFMAs of the current one run;
//   * one barrier per k tile; the loads of tile kt + 2 are issued right after it.
// The epilogue stages each wavefront's 32 x 64 block through LDS so that global stores (and the
// residual loads) are whole 128- or 256-byte row segments.  The kernel is persistent, one
// workgroup per CU: each XCD (eight, dispatched round-robin) runs a contiguous range of tiles
// grouped 8 m-tiles deep (n fastest when there are at most 8 n tiles), so tiles running together
// share operand rows in that XCD's L2, and
// the next tile's first operand loads overlap the current tile's epilogue.  A short last round
// (at most half the CUs' worth of tiles) runs as half tiles on the small kernel instead.
//
// Problems with fewer 256 x 256 tiles than CUs (the 1500-row GEMMs of one window) run on the
// small kernel: 128 x 256 tiles of eight wavefronts, or 128 x 128 tiles where those would leave
// more than half the CUs idle, with the residual GEMMs split over k (fp32 parts added in a fixed
// order by a second kernel, which can also apply the LayerNorm that follows).
#include <algorithm>
#include <type_traits>

#include "wenc_device.h"
#include "wenc_internal.h"

namespace wenc {

// erf-GELU, gelu(z) = z/2 (1 + erf(z / sqrt 2)), with the device library's erff (fp32 path).
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.7071067811865476f));
}

typedef __attribute__((address_space(3))) void lds_void;

// Element offset of (row m, column n) in the head-major layout of EPI_BIAS_HEADMAJOR: rows are
// windows of T positions, columns blocks of 64; block j of window b is a [T][64] slab.
__device__ __forceinline__ size_t headmajor_offset(int m, int n, int N, int T) {
  const int b = m / T, i = m - b * T;
  return ((size_t)((size_t)b * (N >> 6) + (n >> 6)) * T + i) * 64 + (n & 63);
}

// The low halves of eight values whose bf16 roundings (hi) are packed in w4: lo = bf16(v - hi),
// v - hi exact in fp32.
__device__ __forceinline__ u32x4 split_lo8(float4 v0, float4 v1, u32x4 w4) {
  auto lo2 = [](float a, float b, uint32_t hw) {
    return pack2<bf16_t>(a - __uint_as_float(hw << 16), b - __uint_as_float(hw & 0xffff0000u));
  };
  return u32x4{lo2(v0.x, v0.y, w4[0]), lo2(v0.z, v0.w, w4[1]), lo2(v1.x, v1.y, w4[2]),
               lo2(v1.z, v1.w, w4[3])};
}

constexpr int G_N = 256, G_M = 256, G_K = 64;  // workgroup tile

// m tiles per group of the persistent kernel's tile order (m fastest within a group).  Eight
// keep the 32 tiles an XCD runs together at 8 m x 4 n, which share 12 operand panels in its L2.
// With at most eight n tiles (N <= 2048: the out-projection and fc2) the groups are single m
// tiles, i.e. n fastest: the tiles of one round then take every n tile of about 32 / tiles_n
// m panels, so an activation panel is fetched in one round instead of again for the n tiles a
// deeper group leaves to the next round.
__device__ __forceinline__ int persistent_group_depth(int tiles_n) { return tiles_n <= 8 ? 1 : 8; }
constexpr int G_WN = 4, G_WM = 2;              // wavefront grid: n x m
constexpr int G_TN = G_N / G_WN, G_TM = G_M / G_WM;  // 64 x 128 per wavefront
constexpr int G_NA = G_TN / 32, G_NB = G_TM / 32;     // 2 x 4 MFMA blocks
constexpr int G_WAVES = G_WN * G_WM;
constexpr int G_THREADS = 64 * G_WAVES;
constexpr int G_LPO = 32 / G_WAVES;  // 1 KB loads per operand per wavefront and k tile
constexpr int G_STAGE = (G_N + G_M) * G_K;  // 16-bit elements per stage

// Persistent: one workgroup per CU (the grid is the CU count, a multiple of 8; workgroup b runs
// on XCD b % 8, which dispatches round-robin).  XCD x owns the contiguous range
// [x T / 8, (x + 1) T / 8) of the T tiles in grouped order, and its workgroup j takes tiles
// j, j + P / 8, ... of that range, so the tiles running together on one XCD are neighbours that
// share operand rows in its L2.  Between two tiles the epilogue overlaps memory traffic with
// compute: the next tile's first k tile is loaded into stage 0 before the epilogue, which stages
// through stage 1, and the epilogue's loads and stores are range-checked buffer operations issued
// unconditionally (rows past M and columns past N are dropped by the range check), so the number
// of vector-memory operations behind that load is fixed and the next tile waits for the load
// alone, not for the stores.
// tiles_lim: the first tiles_lim tiles of the grouped order (the rest, when the tiles do not
// divide into whole rounds, go to gemm16_small_kernel as half tiles).
//
// T = mx8_t: MXFP8 operands on v_mfma_scale_f32_32x32x64_f8f6f4.  A 128-byte LDS row then holds
// 128 k values, two MFMA steps of 64 (the 16-bit steps 0, 1 and 2, 3 by their chunks); per k tile
// wavefront 0 copies the tile's four 32-k scale blocks of the 256 W rows and wavefront 1 those of
// the X rows into a 2 KB window after the stage.  EPI_BIAS writes fp16, EPI_BIAS_GELU MXFP8.
template <typename T, int EPI>
__global__ __launch_bounds__(G_THREADS, 1) void gemm16_kernel(const uint16_t* __restrict__ X,
                                                             int lda,
                                                             const uint16_t* __restrict__ W,
                                                             const float* __restrict__ bias,
                                                             const float* residual, void* C,
                                                             int ldc, int M, int N, int K,
                                                             int tiles_lim, KMap km, MxPlanes mx) {
  constexpr bool MX = std::is_same<T, mx8_t>::value;
  using OutT = typename std::conditional<MX, f16_t, T>::type;  // type of 16-bit outputs
  constexpr int EB = MX ? 1 : 2;                                // operand bytes per k value
  constexpr bool kMxOut = MX && EPI == EPI_BIAS_GELU;
  static_assert(!MX || (EPI != EPI_BIAS_HEADMAJOR && EPI != EPI_BIAS_GELU_X2), "MXFP8 epilogues");
  constexpr bool kResidual = EPI == EPI_BIAS_RESIDUAL || EPI == EPI_BIAS_GELU_RESIDUAL;
  // Head-major rows scatter over windows (64-bit addresses): those stores stay plain, predicated
  // global stores, and the next tile waits for them.
  constexpr bool kBufferOut = EPI != EPI_BIAS_HEADMAJOR;
  // Vector-memory operations of one wavefront's epilogue: 4 row blocks x (8 residual loads + 8
  // stores), or 4 x 4 stores (MXFP8 output: 4 x (4 code + 4 scale stores)).
  constexpr int kEpiOps = kResidual ? 64 : (EPI == EPI_BIAS_GELU_X2 || kMxOut) ? 32 : 16;
  constexpr int kStage = G_STAGE + (MX ? 1024 : 0);  // + the MXFP8 scale window (2 KB)
  __shared__ __attribute__((aligned(1024))) uint16_t s0[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[kStage];

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / G_WM, wm = wave % G_WM;
  const int tiles_m = (M + G_M - 1) / G_M, tiles_n = (N + G_N - 1) / G_N;
  const int tiles = min(tiles_m * tiles_n, tiles_lim);
  const int nk = K / (G_K * 2 / EB);  // k tiles of 128 bytes per row
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int t_begin = (int)((long)tiles * xcd / 8), t_end = (int)((long)tiles * (xcd + 1) / 8);
  const int ntile = t_end - t_begin > j ? (t_end - t_begin - j + per_xcd - 1) / per_xcd : 0;
  if (ntile <= 0) return;
  // km: k segments of km.kb (the bf16 hi / lo pairs of the BF16X2 / X3 paths; one segment
  // otherwise); weight rows of km.wrow elements.
  const int nkb = km.kb / G_K, kw = km.wrow;
  const int stepW = 64 * kw * EB, stepX = 64 * lda * EB;
  // Copies per wavefront and k tile (MXFP8: one more on wavefronts 0 and 1, the scale blocks).
  const int LT = 2 * G_LPO + ((MX && wave < 2) ? 1 : 0);
  const u32x4 rWs = buffer_rsrc(mx.w, MX ? (uint32_t)((K / 32) * mx.w_stride) : 0u);
  const u32x4 rXs = buffer_rsrc(mx.x, MX ? (uint32_t)((K / 32) * mx.x_stride) : 0u);

  int n0 = 0, m0 = 0;
  u32x4 rW, rX;
  // Tile tt of the grouped order (8 m tiles deep, m fastest); buffer resources cover exactly the
  // tile's valid rows, so operand loads past M or N return zeros.
  auto setup = [&](int tt) {
    const int gd = persistent_group_depth(tiles_n);
    const int group = gd * tiles_n;
    const int first_m = (tt / group) * gd;
    const int gm = min(tiles_m - first_m, gd);
    const int tm = first_m + (tt % group) % gm, tn = (tt % group) / gm;
    n0 = tn * G_N;
    m0 = tm * G_M;
    const int wrows = min(N - n0, G_N), xrows = min(M - m0, G_M);
    rW = buffer_rsrc(reinterpret_cast<const char*>(W) + (size_t)n0 * kw * EB,
                     (uint32_t)(wrows * kw * EB));
    rX = buffer_rsrc(reinterpret_cast<const char*>(X) + (size_t)m0 * lda * EB,
                     (uint32_t)(xrows * lda * EB));
  };

  f32x16 acc[G_NA][G_NB];
  for (int it = 0; it < ntile; ++it) {
    // Lane-dependent offsets are formed per tile from an opaque copy of the lane index, so that
    // they are not all kept live across the tile loop.
    int lane = tid & 63;
    asm volatile("" : "+v"(lane));
    const int g = lane >> 5, frow = lane & 31;

    // Copy i of wavefront w fills the 1 KB LDS block (i * 8 + w): rows 8 * block .. + 7, lane l
    // writing row (l >> 3), slot (l & 7), which holds chunk slot ^ ((row >> 1) & 7).
    const int lrow = 8 * wave + (lane >> 3);
    const int lchunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
    const int voW = lrow * kw * EB + lchunk * 16, voX = lrow * lda * EB + lchunk * 16;
    auto load_tile = [&](int kt, const uint16_t* st) {
      int ko, kow;
      const uint32_t base = lds_addr(st);
      if constexpr (MX) {
        ko = kow = kt * 128;
        // Scale window: lane l copies plane 4 kt + (l >> 4), rows 16 (l & 15) .. of the tile
        // (byte [plane][row] at plane * 256 + row).
        const int pl = 4 * kt + (lane >> 4), r16 = (lane & 15) * 16;
        if (wave == 0)
          lds_copy16(rWs, base + G_STAGE * 2, pl * mx.w_stride + n0 + r16);
        else if (wave == 1)
          lds_copy16(rXs, base + G_STAGE * 2 + 1024u, pl * mx.x_stride + m0 + r16);
      } else {
        const int seg = (kt >= nkb) + (kt >= 2 * nkb), kk = kt - seg * nkb;
        ko = (((km.xmask >> seg) & 1) * nkb + kk) * (G_K * 2);
        kow = (((km.wmask >> seg) & 1) * nkb + kk) * (G_K * 2);
      }
#pragma unroll
      for (int i = 0; i < G_LPO; ++i)
        lds_copy16(rW, base + (uint32_t)(i * G_WAVES + wave) * 1024u, voW + i * stepW + kow);
#pragma unroll
      for (int i = 0; i < G_LPO; ++i)
        lds_copy16(rX, base + (uint32_t)(G_N * G_K * 2) + (uint32_t)(i * G_WAVES + wave) * 1024u,
                   voX + i * stepX + ko);
    };

    // Fragment of step s (16 k): lane l reads row (l & 31) of a 32-row block, chunk 2s + (l >> 5).
    const int rowA = (wn * G_TN + frow) * 128;
    const int rowB = (G_N + wm * G_TM + frow) * 128;
    int xo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xo[s] = ((2 * s + g) ^ ((lane >> 1) & 7)) << 4;
    auto read_frags = [&](const uint16_t* st, int s, u32x4 (&fa)[G_NA], u32x4 (&fb)[G_NB]) {
      const char* base = reinterpret_cast<const char*>(st);
      // in the order the MFMAs consume them
      fa[0] = *reinterpret_cast<const u32x4*>(base + rowA + xo[s]);
#pragma unroll
      for (int b = 0; b < G_NB; ++b)
        fb[b] = *reinterpret_cast<const u32x4*>(base + rowB + b * 4096 + xo[s]);
#pragma unroll
      for (int a = 1; a < G_NA; ++a)
        fa[a] = *reinterpret_cast<const u32x4*>(base + rowA + a * 4096 + xo[s]);
    };
    auto mm = [&](const u32x4 (&fa)[G_NA], const u32x4 (&fb)[G_NB]) {
#pragma unroll
      for (int a = 0; a < G_NA; ++a)
#pragma unroll
        for (int b = 0; b < G_NB; ++b) acc[a][b] = mfma32x32x16<OutT>(fa[a], fb[b], acc[a][b]);
    };
    // MXFP8 step s of a tile (k 64 s .. 64 s + 63): the fragments of the 16-bit steps 2 s and
    // 2 s + 1 (lo, hi) and each lane's scale byte of 32-k block 2 s + g.
    auto read_scales = [&](const uint16_t* st, int s, int (&sa)[G_NA], int (&sb)[G_NB]) {
      const uint8_t* w = reinterpret_cast<const uint8_t*>(st) + G_STAGE * 2 + (2 * s + g) * 256;
#pragma unroll
      for (int a = 0; a < G_NA; ++a) sa[a] = w[wn * G_TN + a * 32 + frow];
#pragma unroll
      for (int b = 0; b < G_NB; ++b) sb[b] = w[1024 + wm * G_TM + b * 32 + frow];
    };
    auto frag_a = [&](const uint16_t* st, int s, int a) {
      const char* base = reinterpret_cast<const char*>(st) + rowA + a * 4096;
      return lds_frag8(base + xo[2 * s], base + xo[2 * s + 1]);
    };
    auto frag_b = [&](const uint16_t* st, int s, int b) {
      const char* base = reinterpret_cast<const char*>(st) + rowB + b * 4096;
      return lds_frag8(base + xo[2 * s], base + xo[2 * s + 1]);
    };
    // MXFP8 step s of a k tile: its fragments and scale bytes, then its MFMAs.  The scheduling
    // barriers keep each step's reads after the previous step's MFMAs, so that one set of
    // fragment registers serves (the accumulators take half the register file).
    auto step_mx = [&](const uint16_t* st, int s) {
      u32x8 fa[G_NA], fb[G_NB];
      int sa[G_NA], sb[G_NB];
#pragma unroll
      for (int a = 0; a < G_NA; ++a) fa[a] = frag_a(st, s, a);
#pragma unroll
      for (int b = 0; b < G_NB; ++b) fb[b] = frag_b(st, s, b);
      read_scales(st, s, sa, sb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < G_NB; ++b)
#pragma unroll
        for (int a = 0; a < G_NA; ++a) acc[a][b] = mfma_mx8(fa[a], fb[b], sa[a], sb[b], acc[a][b]);
      __builtin_amdgcn_sched_barrier(0);
    };
    // Interleave the next step's fragment reads with the current step's MFMAs.
    auto sched = [&]() {
#pragma unroll
      for (int q = 0; q < G_NA + G_NB; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, G_NA * G_NB - G_NA - G_NB, 0);
    };

    if (it == 0) setup(t_begin + j);  // later tiles are set up where their prefetch is issued
#pragma unroll
    for (int a = 0; a < G_NA; ++a)
#pragma unroll
      for (int b = 0; b < G_NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    u32x4 fa0[G_NA], fb0[G_NB], fa1[G_NA], fb1[G_NB];
    __syncthreads();  // the previous tile's staging reads of stage 1 are done
    if (it == 0) load_tile(0, s0);
    if (nk > 1) {
      load_tile(1, s1);
      // k tile 0 has landed.  Still allowed in flight: k tile 1 and, after the first tile, the
      // previous epilogue's operations, which were issued after k tile 0.
      if (it == 0 || !kBufferOut) {
        if (LT > 2 * G_LPO) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * G_LPO + 1));  // vmcnt(9)
        else __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * G_LPO));  // vmcnt(8)
      } else if constexpr (kEpiOps + 2 * G_LPO + (MX ? 1 : 0) >= 63) {
        __builtin_amdgcn_s_waitcnt(0xCF7F);  // vmcnt(63): waits a little more than needed
      } else {
        constexpr int n = kEpiOps + 2 * G_LPO, n1 = n + 1;
        if (LT > 2 * G_LPO) __builtin_amdgcn_s_waitcnt(0x0F70 | (n1 & 15) | ((n1 >> 4) << 14));
        else __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
      }
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    __syncthreads();
    if constexpr (!MX) read_frags(s0, 0, fa0, fb0);

    // One k tile.  `loads` / `next` are compile-time flags so that the loop body has no branch
    // (the scheduling barriers only act inside one basic block).
    auto body = [&](int kt, auto loads, auto next) {
      const uint16_t* cur = (kt & 1) ? s1 : s0;
      const uint16_t* nxt = (kt & 1) ? s0 : s1;
      read_frags(cur, 1, fa1, fb1); mm(fa0, fb0); sched();
      read_frags(cur, 2, fa0, fb0); mm(fa1, fb1); sched();
      read_frags(cur, 3, fa1, fb1); mm(fa0, fb0); sched();
      if constexpr (decltype(next)::value) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // this wavefront's loads of tile kt + 1 have landed
        __syncthreads();                     // ... everyone's, and tile kt is no longer read
        if constexpr (decltype(loads)::value) load_tile(kt + 2, cur);
        read_frags(nxt, 0, fa0, fb0);
      }
      mm(fa1, fb1);
      if constexpr (decltype(next)::value) sched();
    };
    if constexpr (MX) {
      // One k tile = two MXFP8 steps.  One set of fragment registers (the accumulators take half
      // the register file): each step's reads follow the previous step's MFMAs, and the other
      // wavefront of the SIMD covers their latency.  A plain loop (one copy of the body) keeps
      // the register assignment simple.
      for (int kt = 0; kt < nk; ++kt) {
        const uint16_t* cur = (kt & 1) ? s1 : s0;
        step_mx(cur, 0);
        step_mx(cur, 1);
        if (kt + 1 < nk) {
          __builtin_amdgcn_s_waitcnt(0x0F70);  // this wavefront's loads of tile kt + 1 have landed
          __syncthreads();                     // ... everyone's, and tile kt is no longer read
          if (kt + 2 < nk) load_tile(kt + 2, cur);
        }
      }
    } else {
      int kt = 0;
      for (; kt + 2 < nk; ++kt) body(kt, std::true_type{}, std::true_type{});
      if (kt + 1 < nk) {
        body(kt, std::false_type{}, std::true_type{});
        ++kt;
      }
      body(kt, std::false_type{}, std::false_type{});
    }

    // Epilogue, one 32-row block of the wavefront at a time: (acc + bias) as fp32 into the
    // wavefront's 8 KB of stage 1 (row r, 16-byte chunk c at slot c ^ (r & 15)), then read back
    // by rows (LDS operations of one wavefront complete in order).
    const int em0 = m0;
    const int nw = n0 + wn * G_TN;  // first output column of the wavefront
    const bool cols_ok = nw < N;    // N % 64 == 0: the wavefront's 64 columns are all in or out
    float* ep = reinterpret_cast<float*>(s1) + wave * (32 * 64);
    float4 bias4[G_NA][4];  // loaded before the prefetch, so that nothing waits for it
#pragma unroll
    for (int a = 0; a < G_NA; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = a * 8 + 2 * q + g;  // columns 4c .. 4c + 3 of the wavefront
        bias4[a][q] = cols_ok ? *reinterpret_cast<const float4*>(bias + nw + 4 * c)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    __syncthreads();  // every wavefront is done reading both stages
    if (it + 1 < ntile) {
      setup(t_begin + j + (it + 1) * per_xcd);
      load_tile(0, s0);
    }
    // Output (and residual) rows of the tile from the wavefront's first column; the range covers
    // the tile's rows below M, or nothing when the wavefront's columns are past N.
    const size_t row0 = (size_t)em0 * ldc + nw;
    constexpr int esz = kResidual ? 4 : kMxOut ? 1 : 2;
    const int nrec = cols_ok ? min(M - em0, G_M) * ldc * esz : 0;
    const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(C) + row0 * esz, (short)0, nrec, 0x00020000);
    // MXFP8 output: the scale planes (N / 32 planes of mx.c_stride bytes).
    const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
        mx.c, (short)0, kMxOut ? (N / 32) * mx.c_stride : 0, 0x00020000);
#pragma unroll
    for (int b = 0; b < G_NB; ++b) {
#pragma unroll
      for (int a = 0; a < G_NA; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = a * 8 + 2 * q + g;
          const float4 bb = bias4[a][q];
          *reinterpret_cast<float4*>(ep + frow * 64 + ((c ^ (frow & 15)) << 2)) =
              make_float4(acc[a][b][4 * q] + bb.x, acc[a][b][4 * q + 1] + bb.y,
                          acc[a][b][4 * q + 2] + bb.z, acc[a][b][4 * q + 3] + bb.w);
        }
      const int rb = wm * G_TM + b * 32;  // first row of the block within the tile
      if constexpr (kResidual) {
        // fp32 rows of 64 columns: 16 lanes per row, 4 rows per instruction.  All residual loads
        // are issued before the first store; the stores are non-temporal (the residual stream
        // is next read by a different kernel).
        const __amdgpu_buffer_rsrc_t rR = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(residual) + row0, (short)0, nrec, 0x00020000);
        float4 res[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = rb + (lane >> 4) + 4 * q;
          res[q] = __builtin_bit_cast(
              float4, __builtin_amdgcn_raw_buffer_load_b128(rR, (r * ldc + 4 * (lane & 15)) * 4, 0, 0));
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = (lane >> 4) + 4 * q, c = lane & 15;
          float4 v4 = *reinterpret_cast<const float4*>(ep + r * 64 + ((c ^ (r & 15)) << 2));
          if constexpr (EPI == EPI_BIAS_GELU_RESIDUAL)
            v4 = make_float4(gelu_erf_as(v4.x), gelu_erf_as(v4.y), gelu_erf_as(v4.z),
                             gelu_erf_as(v4.w));
          const float4 o = make_float4(res[q].x + v4.x, res[q].y + v4.y, res[q].z + v4.z,
                                       res[q].w + v4.w);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rC,
                                                 ((rb + r) * ldc + 4 * c) * 4, 0, 2 /* nt */);
        }
      } else {
        // 16-bit rows of 64 columns (128 bytes): 8 lanes per row, 8 rows per instruction.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = (lane >> 3) + 8 * q, c0 = 2 * (lane & 7);
          float4 v0 = *reinterpret_cast<const float4*>(ep + r * 64 + ((c0 ^ (r & 15)) << 2));
          float4 v1 = *reinterpret_cast<const float4*>(ep + r * 64 + (((c0 + 1) ^ (r & 15)) << 2));
          if constexpr (EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_X2) {
            v0 = make_float4(gelu_erf_as(v0.x), gelu_erf_as(v0.y), gelu_erf_as(v0.z), gelu_erf_as(v0.w));
            v1 = make_float4(gelu_erf_as(v1.x), gelu_erf_as(v1.y), gelu_erf_as(v1.z), gelu_erf_as(v1.w));
          }
          if constexpr (kMxOut) {
            // MXFP8 output: the four lanes 4 j .. 4 j + 3 hold a row's 32-column block (eight
            // columns each); its scale byte goes to plane (column / 32), position m.  Both stores
            // are issued by every lane (the range checks drop rows past M and non-writers), so
            // the epilogue's operation count stays fixed.
            float amax = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                               fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            const int xe = mx_exponent(amax);
            const float sc = mx_inv_scale(xe);
            const u32x2 w2 = {mx_pack4(v0, sc), mx_pack4(v1, sc)};
            __builtin_amdgcn_raw_buffer_store_b64(w2, rC, (rb + r) * ldc + 4 * c0, 0, 0);
            const int m = em0 + rb + r;
            const bool writer = (lane & 3) == 0 && cols_ok && m < M;
            const int soff = writer ? ((nw + 4 * c0) >> 5) * mx.c_stride + m : 0x7ffffff0;
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(xe + 127), rS, soff, 0, 0);
            continue;
          }
          const u32x4 w4 = {pack2<OutT>(v0.x, v0.y), pack2<OutT>(v0.z, v0.w),
                            pack2<OutT>(v1.x, v1.y), pack2<OutT>(v1.z, v1.w)};
          if constexpr (EPI == EPI_BIAS_GELU_X2) {
            // lo = bf16(v - hi) N columns to the right (ldc = 2 N)
            const u32x4 l4 = split_lo8(v0, v1, w4);
            __builtin_amdgcn_raw_buffer_store_b128(w4, rC, ((rb + r) * ldc + 4 * c0) * 2, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(l4, rC, ((rb + r) * ldc + N + 4 * c0) * 2, 0, 0);
          } else if constexpr (kBufferOut) {
            __builtin_amdgcn_raw_buffer_store_b128(w4, rC, ((rb + r) * ldc + 4 * c0) * 2, 0, 0);
          } else {
            const int m = em0 + rb + r;
            if (cols_ok && m < M)
              *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(C) +
                                        headmajor_offset(m, nw + 4 * c0, N, ldc)) = w4;
          }
        }
      }
    }
  }
}
// Smaller-problem variant (fewer 256 x 256 tiles than CUs, e.g. the 1500-row GEMMs of a single
// window): 128 (n) x 256 (m) tiles for a 512-thread workgroup (eight wavefronts, 64 x 64 outputs
// each, two per SIMD so that one's waits overlap the other's MFMAs even when each CU holds a
// single workgroup, as at one window), three LDS stages of KB-byte rows: 128 bytes (a 64-wide k
// tile of 16-bit values, the persistent kernel's row layout, chunk c of row r at slot
// c ^ ((r >> 1) & 7)) for the launches, or 64 bytes (chunk c at slot c ^ ((r >> 2) & 3)) for
// MXFP8 k not a multiple of 128; either way conflict-free for the 16-lane fragment phases.
// The tile copies are inline assembly (lds_copy16), so the kernel's own s_waitcnt vmcnt is the
// only wait on them.  (Four wavefronts of 64 x 128 read a third fewer fragments per MFMA but
// leave one wavefront per SIMD at one workgroup per CU: 12-14 % slower on the one-window QKV and
// fc1 shapes, measured with 64-byte rows.)
constexpr int H_N = 128, H_M = 256, H_K = 32;
constexpr int H_WN = 2, H_WM = 4;
constexpr int H_TN = H_N / H_WN, H_TM = H_M / H_WM;  // 64 x 64 per wavefront
constexpr int H_NA = H_TN / 32;                       // 2 MFMA blocks along n
constexpr int H_WAVES = H_WN * H_WM;
constexpr int H_THREADS = 64 * H_WAVES;

// WM wavefronts along m, HM rows per tile: (4, 256) for 128 x 256 tiles of eight wavefronts of
// 64 x 64; for problems whose 128 x 256 grid would leave most CUs idle (e.g. the 1500-row GEMMs of
// a tiny-, base- or small-shaped window), (4, 128): 128 x 128 tiles of eight wavefronts of 64 x 32.
// (2, 128), four wavefronts of 64 x 64, is kept as a shape the kernel supports.  Every output is
// the same k-ordered MFMA chain whatever the tile, so all shapes give identical results.
//
// T = mx8_t: MXFP8 operands (codes and E8M0 scale planes, see mx_planes_offset) on
// v_mfma_scale_f32_32x32x64_f8f6f4.  A 64-byte LDS row then holds 64 k values (one MFMA deep),
// in the same layout and with the same copies; per k tile, wavefront 0 also copies the tile's two
// 32-k scale blocks of its 128 W rows and wavefront 1 those of its X rows into a 2 KB window after
// the stage's operand rows.  EPI_BIAS writes fp16; EPI_BIAS_GELU writes MXFP8 (mx.c).
template <typename T, int EPI, int WM = H_WM, int HM = H_M, int KB = 64>
__global__ __launch_bounds__(128 * WM) __attribute__((amdgpu_waves_per_eu(2, 4))) void gemm16_small_kernel(
    const uint16_t* __restrict__ X, int lda, const uint16_t* __restrict__ W,
    const float* __restrict__ bias, const float* residual, void* C, int ldc, int M, int N, int K,
    int ksplit, int big0, KMap km, MxPlanes mx) {
  constexpr bool MX = std::is_same<T, mx8_t>::value;
  using OutT = typename std::conditional<MX, f16_t, T>::type;  // type of 16-bit outputs
  constexpr int EB = MX ? 1 : 2;                           // operand bytes per k value
  static_assert(KB == 64 || KB == 128, "LDS row bytes");
  constexpr int KT = KB / EB;                              // k values per LDS row (one k tile)
  constexpr int NSTEP = KB / 32;                           // 16-bit k16 steps per k tile
  constexpr int RPC = 1024 / KB;                           // rows per 1 KB copy
  constexpr int BLK = 32 * KB;                             // LDS bytes of 32 rows
  constexpr int HW = H_WN * WM;                            // wavefronts
  constexpr int TM = HM / WM, NB = TM / 32;                // rows per wavefront, 32-row blocks
  constexpr int HLW = H_N * KB / 1024 / HW, HLX = HM * KB / 1024 / HW;  // 1 KB copies per operand
  // 16-bit elements per stage: the operand rows (+ the MXFP8 scale window, 2 KB).
  constexpr int HSTAGE = (H_N + HM) * KB / 2 + (MX ? 1024 : 0);
  constexpr int SCALE_OFF = (H_N + HM) * KB;              // byte offset of the scale window
  // Three stages, or the epilogue's 8 KB (4096 16-bit elements) per wavefront if that is more.
  constexpr int LDS_ELEMS = 3 * HSTAGE > HW * 4096 ? 3 * HSTAGE : HW * 4096;
  static_assert((WM == 4 && (HM == 256 || HM == 128)) || (WM == 2 && HM == 128), "tile shapes");
  static_assert(!MX || (EPI != EPI_BIAS_HEADMAJOR && EPI != EPI_BIAS_GELU_X2), "MXFP8 epilogues");
  // One array for the three stages: the copies are inline assembly, invisible to the compiler's
  // wait insertion, so separate arrays buy nothing; the epilogue reuses it (8 KB per wavefront).
  __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
  uint16_t* const s0 = lds;
  uint16_t* const s1 = lds + HSTAGE;
  uint16_t* const s2 = lds + 2 * HSTAGE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / WM, wm = wave % WM;
  const int g = lane >> 5, frow = lane & 31;

  const int tiles_m = (M + HM - 1) / HM, tiles_n = (N + H_N - 1) / H_N;
  // Workgroup (tile, part): with ksplit > 1 (EPI_PARTIAL) part p covers k in
  // [p K / ksplit, (p + 1) K / ksplit).
  const int vv = xcd_virtual_id(blockIdx.x, gridDim.x);
  const int v = vv / ksplit, part = vv % ksplit;
  int n0, m0;
  if (HM != G_M || big0 < 0) {  // the half tiles below are 256 rows high
    const int group = 8 * tiles_n;
    const int first_m = (v / group) * 8;
    const int gm = min(tiles_m - first_m, 8);
    const int tm = first_m + (v % group) % gm, tn = (v % group) / gm;
    n0 = tn * H_N;
    m0 = tm * HM;
  } else {
    // Half (128 columns) v % 2 of the 256 x 256 tile big0 + v / 2 in the persistent kernel's
    // grouped order: the tiles left over after its whole rounds.
    const int gtn = (N + G_N - 1) / G_N;
    const int gd = persistent_group_depth(gtn);
    const int tb = big0 + v / 2, group = gd * gtn;
    const int first_m = (tb / group) * gd;
    const int gm = min(tiles_m - first_m, gd);
    n0 = ((tb % group) / gm) * G_N + (v & 1) * H_N;
    m0 = (first_m + (tb % group) % gm) * G_M;
    if (n0 >= N) return;  // the second half of a last tile only 64 columns wide
  }
  const int kc = K / ksplit, kbyte0 = part * kc * EB;  // this part's first k, in bytes

  const int wrows = min(N - n0, H_N), xrows = min(M - m0, HM);
  const int kw = km.wrow;  // weight row length (k segments: the BF16X2 / X3 hi / lo pairs)
  const char* const Wb = reinterpret_cast<const char*>(W);
  const char* const Xb = reinterpret_cast<const char*>(X);
  const u32x4 rW = buffer_rsrc(Wb + (size_t)n0 * kw * EB, (uint32_t)(wrows * kw * EB));
  const u32x4 rX = buffer_rsrc(Xb + (size_t)m0 * lda * EB, (uint32_t)(xrows * lda * EB));
  // MXFP8 scale planes (K / 32 planes each); reads past the last plane return zeros.
  const u32x4 rWs = buffer_rsrc(mx.w, MX ? (uint32_t)((K / 32) * mx.w_stride) : 0u);
  const u32x4 rXs = buffer_rsrc(mx.x, MX ? (uint32_t)((K / 32) * mx.x_stride) : 0u);

  // Copy i of wavefront w fills 1 KB block (i * HW + w) of its operand.  64-byte rows: 16 rows,
  // lane l row (l >> 2), slot (l & 3) holding chunk slot ^ ((row >> 2) & 3); 128-byte rows: 8
  // rows, lane l row (l >> 3), slot (l & 7) holding chunk slot ^ ((row >> 1) & 7) (the persistent
  // kernel's layout).  Either way each 16-lane phase of a fragment read covers the banks once.
  const int lrow = RPC * wave + lane / (KB / 16);
  const int lchunk = KB == 64 ? ((lane & 3) ^ ((lane >> 4) & 3))
                              : ((lane & 7) ^ ((4 * wave + (lane >> 4)) & 7));
  const int voW = lrow * kw * EB + lchunk * 16, voX = lrow * lda * EB + lchunk * 16;
  // Scale copies: lane l of wavefront 0 (1) copies 16 scale bytes of the tile's W (X) rows, block
  // l / L of the tile's KB / 32, rows 16 (l % L) ..; the other lanes read out of range (zeros)
  // into the rest of the 1 KB window.  The window holds byte [block][row] at block * rows + row.
  constexpr int XL = HM / 16, NBLK = KB / 32;
  const int sc_off =
      wave == 0 ? (lane < 8 * NBLK ? (lane >> 3) * mx.w_stride + n0 + (lane & 7) * 16 : -1)
                : (lane < XL * NBLK ? (lane / XL) * mx.x_stride + m0 + (lane % XL) * 16 : -1);
  auto load_tile = [&](int kt, const uint16_t* st) {
    const uint32_t base = lds_addr(st);
    int ko, kow;
    if constexpr (MX) {
      ko = kow = kbyte0 + kt * KB;
      const int blk = ko >> 5;  // first 32-k block of the tile
      if (wave == 0)
        lds_copy16(rWs, base + SCALE_OFF, sc_off < 0 ? 0x7ffffff0 : sc_off + blk * mx.w_stride);
      else if (wave == 1)
        lds_copy16(rXs, base + SCALE_OFF + 1024u, sc_off < 0 ? 0x7ffffff0 : sc_off + blk * mx.x_stride);
    } else {
      const int ke = kbyte0 / 2 + kt * KT;  // first k of the tile
      const int seg = (ke >= km.kb) + (ke >= 2 * km.kb), kk = ke - seg * km.kb;
      ko = (((km.xmask >> seg) & 1) * km.kb + kk) * 2;
      kow = (((km.wmask >> seg) & 1) * km.kb + kk) * 2;
    }
#pragma unroll
    for (int i = 0; i < HLW; ++i)
      lds_copy16(rW, base + (uint32_t)(i * HW + wave) * 1024u, voW + i * RPC * HW * kw * EB + kow);
#pragma unroll
    for (int i = 0; i < HLX; ++i)
      lds_copy16(rX, base + H_N * KB + (uint32_t)(i * HW + wave) * 1024u,
                 voX + i * RPC * HW * lda * EB + ko);
  };

  const int rowA = (wn * H_TN + frow) * KB;
  const int rowB = (H_N + wm * TM + frow) * KB;
  int xo[NSTEP];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s)
    xo[s] = (KB == 64 ? ((2 * s + g) ^ ((lane >> 2) & 3)) : ((2 * s + g) ^ ((lane >> 1) & 7))) << 4;
  auto read_frags = [&](const uint16_t* st, int s, u32x4 (&fa)[H_NA], u32x4 (&fb)[NB]) {
    const char* base = reinterpret_cast<const char*>(st);
    fa[0] = *reinterpret_cast<const u32x4*>(base + rowA + xo[s]);
#pragma unroll
    for (int b = 0; b < NB; ++b)
      fb[b] = *reinterpret_cast<const u32x4*>(base + rowB + b * BLK + xo[s]);
#pragma unroll
    for (int a = 1; a < H_NA; ++a)
      fa[a] = *reinterpret_cast<const u32x4*>(base + rowA + a * BLK + xo[s]);
  };

  f32x16 acc[H_NA][NB];
#pragma unroll
  for (int a = 0; a < H_NA; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  auto mm = [&](const u32x4 (&fa)[H_NA], const u32x4 (&fb)[NB]) {
#pragma unroll
    for (int a = 0; a < H_NA; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] = mfma32x32x16<OutT>(fa[a], fb[b], acc[a][b]);
  };
  auto sched = [&]() {
    constexpr int R = H_NA + NB, MF = H_NA * NB, P = R < MF ? R : MF;  // reads, MFMAs, pairs
#pragma unroll
    for (int q = 0; q < P; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MF - P, 0);
    if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
  };

  constexpr int LT = HLW + HLX;  // copies per wavefront and tile (MXFP8: +1 on wavefronts 0, 1)
  // Wait until this wavefront's copies of the next tile have landed, with those of the tile after
  // it (`ahead`) still allowed in flight.
  auto wait_copies = [&](bool ahead) {
    if (!ahead) __builtin_amdgcn_s_waitcnt(0x0F70);
    else if (MX && wave < 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (LT + 1));
    else __builtin_amdgcn_s_waitcnt(0x0F70 | LT);
  };
  const int nk = kc / KT;
  if constexpr (MX) {
    // Per k tile each fragment is chunks g and g + 2 of its LDS row (k 16 g .. and 32 + 16 g ..:
    // the MFMA's 32 bytes per lane, bytes 0 .. 15 in 32-k block 0 and 16 .. 31 in block 1, block
    // b scaled by the register of lane row + 32 b), and the lane's scale byte is that of block g.
    // The fragments of tile kt + 1 are read after the barrier that follows tile kt's MFMAs
    // (the compiler gives alternate tiles their own registers, so those reads overlap the MFMAs
    // still running; an explicit second register set measured no faster and cost 27 VGPRs).
    // MXFP8 step s of a k tile: chunks of the 16-bit steps 2 s and 2 s + 1, scale block 2 s + g.
    auto read_scales = [&](const uint16_t* st, int (&sa)[H_NA], int (&sb)[NB], int s = 0) {
      const uint8_t* w = reinterpret_cast<const uint8_t*>(st) + SCALE_OFF;
#pragma unroll
      for (int a = 0; a < H_NA; ++a) sa[a] = w[(2 * s + g) * H_N + wn * H_TN + a * 32 + frow];
#pragma unroll
      for (int b = 0; b < NB; ++b) sb[b] = w[1024 + (2 * s + g) * HM + wm * TM + b * 32 + frow];
    };
    u32x8 A[H_NA], Bf[NB];
    int SA[H_NA], SB[NB];
    auto read_mx = [&](const uint16_t* st, int s = 0) {
      const char* base = reinterpret_cast<const char*>(st);
      const int lo = xo[2 * s], hi = xo[2 * s + 1];
      A[0] = lds_frag8(base + rowA + lo, base + rowA + hi);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        Bf[b] = lds_frag8(base + rowB + b * BLK + lo, base + rowB + b * BLK + hi);
#pragma unroll
      for (int a = 1; a < H_NA; ++a)
        A[a] = lds_frag8(base + rowA + a * BLK + lo, base + rowA + a * BLK + hi);
    };
    auto mm_row = [&](int a) {
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] = mfma_mx8(A[a], Bf[b], SA[a], SB[b], acc[a][b]);
    };
    load_tile(0, s0);
    if (nk > 1) load_tile(1, s1);
    wait_copies(nk > 1);
    __syncthreads();
    if constexpr (KB == 128) {
      // Two MXFP8 steps per k tile: each step's fragments are read after the previous step's
      // MFMAs (one register set), and one barrier per tile.
      auto body2 = [&](int kt, const uint16_t* cur, const uint16_t* ahead) {
        const bool loads = kt + 2 < nk, next = kt + 1 < nk;
        if (loads) load_tile(kt + 2, ahead);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          read_mx(cur, s);
          read_scales(cur, SA, SB, s);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int a = 0; a < H_NA; ++a) mm_row(a);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (next) {
          wait_copies(loads);
          __syncthreads();  // tile kt + 1 landed everywhere; every read of tile kt is complete
        }
      };
      for (int kt = 0; kt < nk; kt += 3) {
        body2(kt, s0, s2);
        if (kt + 1 < nk) body2(kt + 1, s1, s0);
        if (kt + 2 < nk) body2(kt + 2, s2, s1);
      }
    } else {
    read_mx(s0);
    read_scales(s0, SA, SB);
    auto body = [&](int kt, const uint16_t* nxt, const uint16_t* ahead) {
      const bool loads = kt + 2 < nk, next = kt + 1 < nk;
      if (loads) load_tile(kt + 2, ahead);
#pragma unroll
      for (int a = 0; a < H_NA; ++a) mm_row(a);
      if (next) {
        wait_copies(loads);
        // Tile kt + 1 landed everywhere, and every wavefront's reads of tile kt are complete (the
        // barrier waits for them), so tile kt's stage may take tile kt + 3 in body(kt + 1).
        __syncthreads();
        read_mx(nxt);
        read_scales(nxt, SA, SB);
      }
    };
    for (int kt = 0; kt < nk; kt += 3) {
      body(kt, s1, s2);
      if (kt + 1 < nk) body(kt + 1, s2, s0);
      if (kt + 2 < nk) body(kt + 2, s0, s1);
    }
    }
  } else {
    u32x4 fa0[H_NA], fb0[NB], fa1[H_NA], fb1[NB];
    load_tile(0, s0);
    if (nk > 1) load_tile(1, s1);
    if (nk > 1) __builtin_amdgcn_s_waitcnt(0x0F70 | LT); else __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    read_frags(s0, 0, fa0, fb0);

    // k tile kt from `cur`; tile kt + 2 goes to `ahead` (the stage of tile kt - 1, which every
    // wavefront finished reading before the barrier of body(kt - 1)).
    auto body = [&](int kt, const uint16_t* cur, const uint16_t* nxt, const uint16_t* ahead) {
      const bool loads = kt + 2 < nk, next = kt + 1 < nk;
      if (loads) load_tile(kt + 2, ahead);
      read_frags(cur, 1, fa1, fb1); mm(fa0, fb0); sched();
      if constexpr (NSTEP == 4) {
        read_frags(cur, 2, fa0, fb0); mm(fa1, fb1); sched();
        read_frags(cur, 3, fa1, fb1); mm(fa0, fb0); sched();
      }
      if (next) {
        if (loads) __builtin_amdgcn_s_waitcnt(0x0F70 | LT);
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();  // tile kt + 1 landed everywhere; tile kt no longer read after this step
        read_frags(nxt, 0, fa0, fb0);
      }
      mm(fa1, fb1);
    };
    for (int kt = 0; kt < nk; kt += 3) {
      body(kt, s0, s1, s2);
      if (kt + 1 < nk) body(kt + 1, s1, s2, s0);
      if (kt + 2 < nk) body(kt + 2, s2, s0, s1);
    }
  }

  // Epilogue as in the persistent kernel: 32-row blocks staged through the wavefront's own 8 KB of
  // LDS (wavefront-private, so only the first reuse of the stage memory needs a barrier).
  __syncthreads();
  float* ep = reinterpret_cast<float*>(lds) + wave * (32 * 64);
  const int nw = n0 + wn * H_TN;
  const bool cols_ok = nw < N;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int a = 0; a < H_NA; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = a * 8 + 2 * j + g;
        const float4 bb = (cols_ok && EPI != EPI_PARTIAL)
                              ? *reinterpret_cast<const float4*>(bias + nw + 4 * c)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(ep + frow * 64 + ((c ^ (frow & 15)) << 2)) =
            make_float4(acc[a][b][4 * j] + bb.x, acc[a][b][4 * j + 1] + bb.y,
                        acc[a][b][4 * j + 2] + bb.z, acc[a][b][4 * j + 3] + bb.w);
      }
    if (!cols_ok) continue;
    const int mb = m0 + wm * TM + b * 32;
    if constexpr (EPI == EPI_PARTIAL) {
      // fp32 rows of 64 columns of this part's sums: partial[part][m][n], row stride N.
      float* P = static_cast<float*>(C) + (size_t)part * M * N;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = (lane >> 4) + 4 * q, c = lane & 15;
        const int m = mb + r;
        const float4 v4 = *reinterpret_cast<const float4*>(ep + r * 64 + ((c ^ (r & 15)) << 2));
        if (m < M) *reinterpret_cast<float4*>(P + (size_t)m * N + nw + 4 * c) = v4;
      }
    } else if constexpr (EPI == EPI_BIAS_RESIDUAL || EPI == EPI_BIAS_GELU_RESIDUAL) {
      float4 res[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int m = mb + (lane >> 4) + 4 * q;
        res[q] = m < M ? *reinterpret_cast<const float4*>(residual + (size_t)m * ldc + nw + 4 * (lane & 15))
                       : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = (lane >> 4) + 4 * q, c = lane & 15;
        const int m = mb + r;
        float4 v4 = *reinterpret_cast<const float4*>(ep + r * 64 + ((c ^ (r & 15)) << 2));
        if constexpr (EPI == EPI_BIAS_GELU_RESIDUAL)
          v4 = make_float4(gelu_erf_as(v4.x), gelu_erf_as(v4.y), gelu_erf_as(v4.z), gelu_erf_as(v4.w));
        if (m < M)
          *reinterpret_cast<float4*>(static_cast<float*>(C) + (size_t)m * ldc + nw + 4 * c) =
              make_float4(res[q].x + v4.x, res[q].y + v4.y, res[q].z + v4.z, res[q].w + v4.w);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = (lane >> 3) + 8 * q, c0 = 2 * (lane & 7);
        const int m = mb + r;
        float4 v0 = *reinterpret_cast<const float4*>(ep + r * 64 + ((c0 ^ (r & 15)) << 2));
        float4 v1 = *reinterpret_cast<const float4*>(ep + r * 64 + (((c0 + 1) ^ (r & 15)) << 2));
        if constexpr (EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_X2) {
          v0 = make_float4(gelu_erf_as(v0.x), gelu_erf_as(v0.y), gelu_erf_as(v0.z), gelu_erf_as(v0.w));
          v1 = make_float4(gelu_erf_as(v1.x), gelu_erf_as(v1.y), gelu_erf_as(v1.z), gelu_erf_as(v1.w));
        }
        if constexpr (MX && EPI == EPI_BIAS_GELU) {
          // MXFP8 output: a 32-column block of row m is held by the four lanes 4 j .. 4 j + 3 (eight
          // columns each); its scale byte goes to plane (column / 32), position m.
          float amax = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                             fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
          amax = fmaxf(amax, __shfl_xor(amax, 1));
          amax = fmaxf(amax, __shfl_xor(amax, 2));
          const int xe = mx_exponent(amax);
          const float sc = mx_inv_scale(xe);
          const u32x2 w2 = {mx_pack4(v0, sc), mx_pack4(v1, sc)};
          if (m < M) {
            *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(C) + (size_t)m * ldc + nw + 4 * c0) = w2;
            if ((lane & 3) == 0)
              mx.c[(size_t)((nw + 4 * c0) >> 5) * mx.c_stride + m] = (uint8_t)(xe + 127);
          }
          continue;
        }
        const u32x4 w4 = {pack2<OutT>(v0.x, v0.y), pack2<OutT>(v0.z, v0.w), pack2<OutT>(v1.x, v1.y),
                          pack2<OutT>(v1.z, v1.w)};
        if (m < M) {
          const size_t off = EPI == EPI_BIAS_HEADMAJOR ? headmajor_offset(m, nw + 4 * c0, N, ldc)
                                                       : (size_t)m * ldc + nw + 4 * c0;
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(C) + off) = w4;
          if constexpr (EPI == EPI_BIAS_GELU_X2)
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(C) + off + N) = split_lo8(v0, v1, w4);
        }
      }
    }
  }
}


constexpr int GB_N = 128;  // W rows (output columns) per tile
constexpr int GB_M = 128;  // X rows per tile

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
        const size_t off = EPI == EPI_BIAS_HEADMAJOR ? headmajor_offset(m, n, N, ldc)
                                                     : (size_t)m * ldc + n;
        if constexpr (EPI == EPI_BIAS_GELU_RESIDUAL)
          v = make_float4(gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w));
        if constexpr (EPI == EPI_BIAS_RESIDUAL || EPI == EPI_BIAS_GELU_RESIDUAL) {
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

// Second pass of a split-k residual GEMM: c = residual + epi(sum of the parts + bias), the parts
// added in order (deterministic).  A workgroup per row (grid-stride over rows), four columns per
// thread.  (When a LayerNorm reads the result, launch_splitk_reduce_ln does this pass instead.)
template <bool GELU>
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int ksplit,
                                     const float* __restrict__ bias, const float* residual,
                                     float* c, int ldc, int M, int N) {
  const size_t plane = (size_t)M * N;
  for (int m = blockIdx.x; m < M; m += gridDim.x) {
    for (int n = 4 * threadIdx.x; n < N; n += 4 * blockDim.x) {
      const size_t e = (size_t)m * N + n;
      float4 s = *reinterpret_cast<const float4*>(part + e);
#pragma unroll 4
      for (int p = 1; p < ksplit; ++p) {
        const float4 q = *reinterpret_cast<const float4*>(part + p * plane + e);
        s = make_float4(s.x + q.x, s.y + q.y, s.z + q.z, s.w + q.w);
      }
      const float4 b = *reinterpret_cast<const float4*>(bias + n);
      float4 v = make_float4(s.x + b.x, s.y + b.y, s.z + b.z, s.w + b.w);
      if constexpr (GELU)
        v = make_float4(gelu_erf_as(v.x), gelu_erf_as(v.y), gelu_erf_as(v.z), gelu_erf_as(v.w));
      const float4 r = *reinterpret_cast<const float4*>(residual + (size_t)m * ldc + n);
      *reinterpret_cast<float4*>(c + (size_t)m * ldc + n) =
          make_float4(r.x + v.x, r.y + v.y, r.z + v.z, r.w + v.w);
    }
  }
}

// LDS row bytes of the small kernel's launches: 128, one k tile of 64 16-bit or 128 fp8 values,
// four 16-bit MFMA steps (two fp8 ones) per barrier.  Measured against 64-byte rows (two steps per
// barrier, two workgroups per CU where the LDS allowed it), one window: large-v3 stack 5.09 ->
// 4.60 ms (fp16) and 4.13 -> 3.73 ms (MXFP8), small 1.17 -> 1.07, base 0.441 -> 0.415, tiny
// 0.073 -> 0.068 ms.  Three 48 KB stages (+ the MXFP8 scale windows) hold one workgroup per CU.
constexpr int kSmallKB = 128;

// Split-k plan of a residual GEMM: the number of k parts, and the rows (256 or 128) of the small
// kernel's tiles for them.  Reference device: 256 CUs (the plan fixes the results and the
// workspace size, so it must not depend on the device).  Split only problems the persistent
// kernel would not take, into parts of at least 256 k, while the parts still fit one workgroup per
// CU.  Where the parts are shorter than 512 k, there are at least four, and their tiles would be
// 128 x 256, half as many parts on 128 x 128 tiles instead (the same workgroup count, half the
// partial sums to write and add).
// Measured at M = 1500, GEMM + reduction + LayerNorm: d 1280 out-projection 24.3 -> 22.0 us
// (4 parts of 320 -> 2 of 640), d 512 fc2 19.9 -> 17.2 us (8 of 256 -> 4 of 512); with parts of
// 768 k or more (d 768 and d 1280 fc2) the 128 x 256 tiles stay faster.  Fewer 128 x 256 tiles
// than half the CUs also take 128 x 128 tiles.
// kt: the k values per k tile (32 for 16-bit operands, 64 for MXFP8); every part is whole tiles.
static int split_plan(int m, int n, int k, int* tile_rows, int kt = H_K) {
  *tile_rows = H_M;
  const long big = (long)((m + G_M - 1) / G_M) * ((n + G_N - 1) / G_N);
  if (big >= 256) return 1;
  const long small = (long)((m + H_M - 1) / H_M) * ((n + H_N - 1) / H_N);
  int s = 1;
  while (s < 8 && small * s * 2 <= 256 && k % (s * 2 * kt) == 0 && k / (s * 2) >= 256) s *= 2;
  if (2 * small * s < 256) {
    *tile_rows = 128;
  } else if (s >= 4 && k / s < 512) {
    s /= 2;
    *tile_rows = 128;
  }
  return s;
}

int linear_split(int m, int n, int k, int dtype, int epilogue) {
  if (dtype == DT_F32 || (epilogue != EPI_BIAS_RESIDUAL && epilogue != EPI_BIAS_GELU_RESIDUAL))
    return 1;
  int rows;
  return split_plan(m, n, k, &rows, dtype == DT_MX8 ? kSmallKB : kSmallKB / 2);
}

// Workgroups of the persistent kernel: the current device's CU count, rounded down to a multiple
// of the eight XCDs.
static int persistent_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 8)
    return 256;
  return cus & ~7;
}

template <typename T, int EPI>
static hipError_t launch16_epi(const uint16_t* X, int lda, const uint16_t* W, const float* bias,
                               const float* residual, void* c, int ldc, int m, int n, int k,
                               hipStream_t st, float* partial, const LnFuse* ln, KMap kw) {
  const long tiles = (long)((m + G_M - 1) / G_M) * ((n + G_N - 1) / G_N);
  const long small = (long)((m + H_M - 1) / H_M) * ((n + H_N - 1) / H_N);
  int split_rows = H_M;
  const int split = partial ? linear_split(m, n, k, DT_F16, EPI) : 1;
  if (split > 1) split_plan(m, n, k, &split_rows, kSmallKB / 2);
  if (ln && (EPI != EPI_BIAS_RESIDUAL || split < 2 || ldc != n)) return hipErrorInvalidValue;
  const int grid = persistent_grid();
  const long small2 = (long)((m + 127) / 128) * ((n + H_N - 1) / H_N);  // 128 x 128 tiles
  if constexpr (EPI == EPI_BIAS_RESIDUAL || EPI == EPI_BIAS_GELU_RESIDUAL) {
    if (split > 1) {
      // Each part's sums do not depend on the tile shape (split_plan picks it).
      if (split_rows == 128)
        gemm16_small_kernel<T, EPI_PARTIAL, 4, 128, kSmallKB><<<dim3((unsigned)(small2 * split)),
                                                       dim3(H_THREADS), 0, st>>>(
            X, lda, W, bias, nullptr, partial, n, m, n, k, split, -1, kw, MxPlanes{});
      else
        gemm16_small_kernel<T, EPI_PARTIAL, H_WM, H_M, kSmallKB><<<dim3((unsigned)(small * split)), dim3(H_THREADS),
                                              0, st>>>(X, lda, W, bias, nullptr, partial, n, m, n,
                                                       k, split, -1, kw, MxPlanes{});
      if (ln)
        return launch_splitk_reduce_ln(partial, split, bias, residual,
                                       ln->keep_x ? static_cast<float*>(c) : nullptr, ln->gamma,
                                       ln->beta, ln->y, ln->y_dtype, m, n, st);
      const unsigned g = (unsigned)std::min(m, 16384);
      splitk_reduce_kernel<EPI == EPI_BIAS_GELU_RESIDUAL><<<g, 256, 0, st>>>(
          partial, split, bias, residual, static_cast<float*>(c), ldc, m, n);
      return hipGetLastError();
    }
  }
  if (tiles >= grid) {
    // Whole rounds on the persistent kernel.  A last partial round that would leave most CUs
    // idle for a whole tile runs instead as half tiles (128 columns) on the small kernel, at most
    // one per CU, in about half the time; each output is still one wavefront's k-ordered sum, so
    // the results do not change.
    const long whole = tiles / grid * grid, tail = tiles - whole;
    const bool halves = tail > 0 && 2 * tail <= grid;
    gemm16_kernel<T, EPI><<<dim3((unsigned)grid), dim3(G_THREADS), 0, st>>>(
        X, lda, W, bias, residual, c, ldc, m, n, k, (int)(halves ? whole : tiles), kw, MxPlanes{});
    if (halves)
      gemm16_small_kernel<T, EPI, H_WM, H_M, kSmallKB><<<dim3((unsigned)(2 * tail)), dim3(H_THREADS), 0, st>>>(
          X, lda, W, bias, residual, c, ldc, m, n, k, 1, (int)whole, kw, MxPlanes{});
  } else if (2 * small < grid) {
    // Fewer 128 x 256 tiles than half the CUs: 128 x 128 tiles, eight wavefronts of 64 x 32, twice
    // as many workgroups.  Measured at M = 1500 (us, 128 x 256 -> 128 x 128 with four wavefronts
    // of 64 x 64 -> with eight of 64 x 32): d 384 QKV 9.2 -> 7.6 -> 6.4, fc1 12.2 -> 9.6 -> 8.3;
    // d 512 QKV 10.7 -> 8.8 -> 7.5, fc1 14.0 -> 11.0 -> 9.7; d 768 QKV 14.4 -> 12.0 -> 11.0.  With
    // 144 tiles or more (d 768 fc1, d 1280) the 128 x 256 tiles stay as fast or faster.
    gemm16_small_kernel<T, EPI, 4, 128, kSmallKB><<<dim3((unsigned)small2), dim3(H_THREADS), 0, st>>>(
        X, lda, W, bias, residual, c, ldc, m, n, k, 1, -1, kw, MxPlanes{});
  } else {
    gemm16_small_kernel<T, EPI, H_WM, H_M, kSmallKB><<<dim3((unsigned)small), dim3(H_THREADS), 0, st>>>(
        X, lda, W, bias, residual, c, ldc, m, n, k, 1, -1, kw, MxPlanes{});
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch16(const void* a, int lda, const void* w, const float* bias,
                           const float* residual, void* c, int ldc, int m, int n, int k, int epi,
                           hipStream_t st, float* partial, const LnFuse* ln, KMap kw) {
  auto X = static_cast<const uint16_t*>(a);
  auto W = static_cast<const uint16_t*>(w);
  switch (epi) {
    case EPI_BIAS:
      return launch16_epi<T, EPI_BIAS>(X, lda, W, bias, residual, c, ldc, m, n, k, st, partial, ln,
                                       kw);
    case EPI_BIAS_GELU:
      return launch16_epi<T, EPI_BIAS_GELU>(X, lda, W, bias, residual, c, ldc, m, n, k, st,
                                            partial, ln, kw);
    case EPI_BIAS_RESIDUAL:
      return launch16_epi<T, EPI_BIAS_RESIDUAL>(X, lda, W, bias, residual, c, ldc, m, n, k, st,
                                                partial, ln, kw);
    case EPI_BIAS_HEADMAJOR:
      return launch16_epi<T, EPI_BIAS_HEADMAJOR>(X, lda, W, bias, residual, c, ldc, m, n, k, st,
                                                 partial, ln, kw);
    case EPI_BIAS_GELU_RESIDUAL:
      return launch16_epi<T, EPI_BIAS_GELU_RESIDUAL>(X, lda, W, bias, residual, c, ldc, m, n, k,
                                                     st, partial, ln, kw);
  }
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (epi == EPI_BIAS_GELU_X2)
      return launch16_epi<T, EPI_BIAS_GELU_X2>(X, lda, W, bias, residual, c, ldc, m, n, k, st,
                                               partial, ln, kw);
  }
  return hipErrorInvalidValue;
}

// MXFP8 operands, with the same choices as 16-bit ones: whole rounds of 256 x 256 tiles on the
// persistent kernel (k % 128 == 0), else the small kernel (128 x 256 tiles, or 128 x 128 where
// those would leave more than half the CUs idle), and the same split-k rule.  KB: the small
// kernel's LDS row bytes, 128 (two MXFP8 steps per k tile) where k allows, else 64.
template <int EPI, int KB = kSmallKB>
static hipError_t launch_mx_epi(const uint16_t* X, const uint16_t* W, const float* bias,
                                const float* residual, void* c, int ldc, int m, int n, int k,
                                hipStream_t st, float* partial, const LnFuse* ln,
                                const MxPlanes& mx) {
  const KMap kw{k, 1, 0, 0, k};
  const long small = (long)((m + H_M - 1) / H_M) * ((n + H_N - 1) / H_N);
  const long small2 = (long)((m + 127) / 128) * ((n + H_N - 1) / H_N);
  int split_rows = H_M;
  const int split = partial ? linear_split(m, n, k, DT_MX8, EPI) : 1;
  if (split > 1) split_plan(m, n, k, &split_rows, KB);
  if (ln && (EPI != EPI_BIAS_RESIDUAL || split < 2 || ldc != n)) return hipErrorInvalidValue;
  if constexpr (EPI == EPI_BIAS_RESIDUAL || EPI == EPI_BIAS_GELU_RESIDUAL) {
    if (split > 1) {
      if (split_rows == 128)
        gemm16_small_kernel<mx8_t, EPI_PARTIAL, 4, 128, KB><<<dim3((unsigned)(small2 * split)),
                                                           dim3(H_THREADS), 0, st>>>(
            X, k, W, bias, nullptr, partial, n, m, n, k, split, -1, kw, mx);
      else
        gemm16_small_kernel<mx8_t, EPI_PARTIAL, H_WM, H_M, KB><<<dim3((unsigned)(small * split)),
                                                  dim3(H_THREADS), 0, st>>>(
            X, k, W, bias, nullptr, partial, n, m, n, k, split, -1, kw, mx);
      if (ln)
        return launch_splitk_reduce_ln(partial, split, bias, residual,
                                       ln->keep_x ? static_cast<float*>(c) : nullptr, ln->gamma,
                                       ln->beta, ln->y, ln->y_dtype, m, n, st);
      const unsigned g = (unsigned)std::min(m, 16384);
      splitk_reduce_kernel<EPI == EPI_BIAS_GELU_RESIDUAL><<<g, 256, 0, st>>>(
          partial, split, bias, residual, static_cast<float*>(c), ldc, m, n);
      return hipGetLastError();
    }
  }
  const int grid = persistent_grid();
  const long tiles = (long)((m + G_M - 1) / G_M) * ((n + G_N - 1) / G_N);
  if (tiles >= grid && k % 128 == 0) {
    // As for 16-bit operands: whole rounds of 256 x 256 tiles on the persistent kernel, a short
    // last round as 128-column half tiles on the small kernel.
    const long whole = tiles / grid * grid, tail = tiles - whole;
    const bool halves = tail > 0 && 2 * tail <= grid;
    gemm16_kernel<mx8_t, EPI><<<dim3((unsigned)grid), dim3(G_THREADS), 0, st>>>(
        X, k, W, bias, residual, c, ldc, m, n, k, (int)(halves ? whole : tiles), kw, mx);
    if (halves)
      gemm16_small_kernel<mx8_t, EPI, H_WM, H_M, KB><<<dim3((unsigned)(2 * tail)), dim3(H_THREADS), 0, st>>>(
          X, k, W, bias, residual, c, ldc, m, n, k, 1, (int)whole, kw, mx);
  } else if (2 * small < grid) {
    gemm16_small_kernel<mx8_t, EPI, 4, 128, KB><<<dim3((unsigned)small2), dim3(H_THREADS), 0, st>>>(
        X, k, W, bias, residual, c, ldc, m, n, k, 1, -1, kw, mx);
  } else {
    gemm16_small_kernel<mx8_t, EPI, H_WM, H_M, KB><<<dim3((unsigned)small), dim3(H_THREADS), 0, st>>>(
        X, k, W, bias, residual, c, ldc, m, n, k, 1, -1, kw, mx);
  }
  return hipGetLastError();
}

static hipError_t launch_mx(const void* a, int lda, const void* w, const float* bias,
                            const float* residual, void* c, int ldc, int m, int n, int k, int epi,
                            hipStream_t st, float* partial, const LnFuse* ln) {
  if (lda != k || k % 64 != 0) return hipErrorInvalidValue;
  MxPlanes mx{static_cast<const uint8_t*>(a) + mx_planes_offset(m, k), (int)mx_plane_stride(m),
              static_cast<const uint8_t*>(w) + mx_planes_offset(n, k), (int)mx_plane_stride(n),
              nullptr, 0};
  auto X = static_cast<const uint16_t*>(a);
  auto W = static_cast<const uint16_t*>(w);
  if (k % kSmallKB != 0) {  // k tiles of 64: only the unsplit small kernel (no split plan fits)
    if (partial && linear_split(m, n, k, DT_MX8, epi) > 1) return hipErrorInvalidValue;
    switch (epi) {
      case EPI_BIAS: return launch_mx_epi<EPI_BIAS, 64>(X, W, bias, residual, c, ldc, m, n, k, st, nullptr, ln, mx);
      case EPI_BIAS_GELU:
        if (ldc != n) return hipErrorInvalidValue;
        mx.c = static_cast<uint8_t*>(c) + mx_planes_offset(m, n);
        mx.c_stride = (int)mx_plane_stride(m);
        return launch_mx_epi<EPI_BIAS_GELU, 64>(X, W, bias, residual, c, ldc, m, n, k, st, nullptr, ln, mx);
      case EPI_BIAS_RESIDUAL:
        return launch_mx_epi<EPI_BIAS_RESIDUAL, 64>(X, W, bias, residual, c, ldc, m, n, k, st, nullptr, ln, mx);
      case EPI_BIAS_GELU_RESIDUAL:
        return launch_mx_epi<EPI_BIAS_GELU_RESIDUAL, 64>(X, W, bias, residual, c, ldc, m, n, k, st, nullptr, ln, mx);
    }
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case EPI_BIAS:
      return launch_mx_epi<EPI_BIAS>(X, W, bias, residual, c, ldc, m, n, k, st, partial, ln, mx);
    case EPI_BIAS_GELU:
      if (ldc != n) return hipErrorInvalidValue;
      mx.c = static_cast<uint8_t*>(c) + mx_planes_offset(m, n);
      mx.c_stride = (int)mx_plane_stride(m);
      return launch_mx_epi<EPI_BIAS_GELU>(X, W, bias, residual, c, ldc, m, n, k, st, partial, ln,
                                          mx);
    case EPI_BIAS_RESIDUAL:
      return launch_mx_epi<EPI_BIAS_RESIDUAL>(X, W, bias, residual, c, ldc, m, n, k, st, partial,
                                              ln, mx);
    case EPI_BIAS_GELU_RESIDUAL:
      return launch_mx_epi<EPI_BIAS_GELU_RESIDUAL>(X, W, bias, residual, c, ldc, m, n, k, st,
                                                   partial, ln, mx);
  }
  return hipErrorInvalidValue;
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
    case EPI_BIAS_HEADMAJOR:
      gemm32_kernel<EPI_BIAS_HEADMAJOR><<<grid, block, 0, st>>>(X, lda, W, bias, residual, C, ldc,
                                                                m, n, k);
      break;
    case EPI_BIAS_GELU_RESIDUAL:
      gemm32_kernel<EPI_BIAS_GELU_RESIDUAL><<<grid, block, 0, st>>>(X, lda, W, bias, residual, C,
                                                                    ldc, m, n, k);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_linear(const void* a, int lda, const void* w, const float* bias,
                         const float* residual, void* c, int ldc, int m, int n, int k, int dtype,
                         int epilogue, hipStream_t st, float* partial, const LnFuse* ln,
                         const KMap* kmap) {
  if (m == 0) return hipSuccess;
  const KMap kw = kmap ? *kmap : KMap{k, 1, 0, 0, k};
  const bool plain = kw.nseg == 1 && kw.wrow == kw.kb && kw.xmask == 0 && kw.wmask == 0;
  if (kmap && (kw.nseg < 1 || kw.nseg > 3 || k != kw.nseg * kw.kb || kw.kb % G_K != 0 ||
               (kw.wrow != kw.kb && kw.wrow != 2 * kw.kb) || (dtype == DT_F32 && !plain)))
    return hipErrorInvalidValue;
  switch (dtype) {
    case DT_BF16:
      return launch16<bf16_t>(a, lda, w, bias, residual, c, ldc, m, n, k, epilogue, st, partial,
                              ln, kw);
    case DT_F16:
      return launch16<f16_t>(a, lda, w, bias, residual, c, ldc, m, n, k, epilogue, st, partial,
                             ln, kw);
    case DT_F32:
      if (ln) return hipErrorInvalidValue;
      return launch32(a, lda, w, bias, residual, c, ldc, m, n, k, epilogue, st);
    case DT_MX8:
      if (!plain) return hipErrorInvalidValue;
      return launch_mx(a, lda, w, bias, residual, c, ldc, m, n, k, epilogue, st, partial, ln);
  }
  return hipErrorInvalidValue;
}

}  // namespace wenc
