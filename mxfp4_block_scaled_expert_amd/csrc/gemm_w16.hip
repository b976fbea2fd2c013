// bf16-activation GEMMs with FP8 or MXFP4 weights on the gfx950 bf16 matrix cores.
//
// * W8A16 per-tensor ("SGLang PR 32618 review", implementation items 1-2):
//   out = bf16((A @ dec(W)^T) * s + bias).  The scale is applied once after the
//   K loop, which equals applying it per K block (every block scale is the
//   same constant).
// * W8A16 block-scaled experts ("vLLM PR 50949 review", moe_fp8.cpp listing):
//   each 128-wide K block's partial sum is multiplied by its weight-block scale
//   before it is added to the accumulator.
// * W4A16 MXFP4 experts (same listing, MXFP4 weights): the e8m0 scale of each
//   32-element group is a power of two, so it is folded into the exact
//   e2m1 -> bf16 decode and no promotion step is needed.
//
// Weights are decoded to bf16 in registers right after their LDS fragment read
// (e4m3 and scaled e2m1 values are exact in bf16); V_MFMA_F32_16X16X32_BF16
// accumulates in fp32.  A is staged through LDS; K may end on any multiple of
// 32 (the tail of the last 128-wide step is zero-filled on both operands).
// Routed weights and MX scales may come in the tiled layout of prepack.hip
// (TILED): each weight chunk is then read from one contiguous 2 KB tile, and
// the K tail is already zero in memory.
#include <algorithm>

#include "tile_rows.hpp"

namespace mxq {

template <int WFMT>
struct W16Layout {
  // bytes of one weight row per 128-wide K step, and the padded LDS row
  static constexpr int row_bytes = (WFMT == W_E2M1_MX) ? 64 : 128;
  static constexpr int lds_row = row_bytes + 16;
  static constexpr int chunks = row_bytes / 16;  // 16-byte chunks per row
};

// LDS of one tile: A [BM][A_LROW] | W [BN][lds_row] | MX scales [BN]; after the K loop the
// same memory stages the output tile (bf16 or fp32 rows) for row-contiguous stores.
template <int BM, int BN, int WFMT, bool OUT_F32>
__host__ __device__ constexpr size_t w16_lds_bytes() {
  const size_t ops = size_t(BM) * (256 + 16) + size_t(BN) * W16Layout<WFMT>::lds_row + (WFMT == W_E2M1_MX ? 4 * BN : 16);
  const size_t out = OUT_F32 ? size_t(BM) * (BN + 4) * 4 : size_t(BM) * (BN + 8) * 2;
  return ops > out ? ops : out;
}

// One BM x BN output tile computed by NT threads (NT / 64 waves, WAVES_M of them along M);
// `bid` is the tile's index in its launch, `lds` its share of LDS.
//
// Per 128-wide K step: the weight chunks of the step are requested first (they depend only on
// the expert and the column tile), the activation rows once the row table is in LDS; operands
// are staged through registers into LDS one step ahead of the products.  Activation rows past
// the block's row count are neither loaded nor multiplied: a wave skips the 16-row MFMA tiles
// that lie wholly past it.
template <int NT, int BM, int BN, int WAVES_M, int MODE, int WFMT, bool OUT_F32, bool HAS_BIAS, bool TILED>
__device__ __forceinline__ void w16_tile(const GemmArgs& a, int64_t grid_blocks, int64_t bid, uint8_t* lds) {
  constexpr int WAVES = NT / 64;
  constexpr int WAVES_N = WAVES / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  static_assert(WAVES_M * WAVES_N == WAVES && TM >= 1 && TN >= 1, "wave tile smaller than one MFMA tile");
  static_assert(BN <= NT, "one thread per weight row for the MX scales");
  using L = W16Layout<WFMT>;
  constexpr int A_LROW = 256 + 16;  // 128 bf16 + pad
  constexpr int A_IT = (BM * 16 + NT - 1) / NT;
  constexpr int B_IT = (BN * L::chunks + NT - 1) / NT;
  constexpr bool MX = WFMT == W_E2M1_MX;

  uint8_t* sA = lds;
  uint8_t* sB = lds + BM * A_LROW;
  uint32_t* sBs = reinterpret_cast<uint32_t*>(sB + BN * L::lds_row);
  __shared__ int64_t sArow[BM];
  __shared__ int64_t sOrow[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // K split: chunk `split` of the tile's K range (fastest-varying), then row tile, then column tile
  const int nsplit = a.k_split > 1 ? a.k_split : 1;
  const int split = int(bid % nsplit);
  const int64_t rest = bid / nsplit;
  const int64_t tile = rest % grid_blocks;
  const int64_t nt = rest / grid_blocks;
  const int64_t n0 = nt * BN;
  if (n0 >= a.N) return;

  TileInfo t;
  if (!tile_info<BM, MODE>(a, tile, t)) return;
  const int64_t expert = t.expert;
  const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A);
  const uint8_t* Wb = a.W + expert * a.w_estride;
  const int KS = int(cdiv(a.K, 128));
  // this workgroup's 128-wide K steps; an empty range (a chunk past K) stores zeros
  int ks_b = 0, ks_e = KS;
  if (nsplit > 1) {
    const int cs = int(a.k_chunk >> 7);
    ks_b = min(KS, split * cs);
    ks_e = min(KS, ks_b + cs);
  }

  // weight chunk addresses (independent of the rows)
  const uint8_t* pb[B_IT];
  int kbo[B_IT];
  int sbo[B_IT];  // LDS byte offset of the chunk
  // tiled layout: 128-byte row steps per 16-row tile; an MXFP4 K step uses half a row step
  const int64_t tsteps = (a.K * (MX ? 1 : 2) / 2 + 127) / 128;
#pragma unroll
  for (int i = 0; i < B_IT; ++i) {
    const int c = min(tid + NT * i, BN * L::chunks - 1);
    if (TILED) {
      // FP8: chunk c = bytes 16 (c % 128) of tile c / 128.  MXFP4: the K step is one half
      // (512 bytes per 1 KB half-tile) of a tile step, chunk c = 16 (c % 32) of half c / 32 % 2.
      constexpr int CPT = MX ? 64 : 128;  // chunks per tile per K step
      const int tt = c / CPT, p = c % CPT;
      const int64_t grp16 = min<int64_t>(n0 / 16 + tt, a.N / 16 - 1);
      const int h = MX ? (p >> 5) : (p >> 6);
      const int L16 = p & 15, qq = MX ? ((p >> 4) & 1) : ((p >> 4) & 3);
      pb[i] = Wb + grp16 * tsteps * 2048 + h * 1024 + (qq * 16 + L16) * 16;
      sbo[i] = (16 * tt + L16) * L::lds_row + qq * 32 + h * 16;
      kbo[i] = 0;  // the K tail is zero-padded in memory
    } else {
      const int64_t n = min<int64_t>(n0 + c / L::chunks, a.N - 1);
      kbo[i] = (c % L::chunks) * (MX ? 32 : 16);  // first K element of the chunk
      pb[i] = Wb + n * a.ldw + (c % L::chunks) * 16;
      sbo[i] = (c / L::chunks) * L::lds_row + (c % L::chunks) * 16;
    }
  }
  const uint8_t* pbs = nullptr;
  if (MX) {
    if (TILED) {
      const int r = min(tid, BN - 1);
      const int64_t grp16 = min<int64_t>(n0 / 16 + r / 16, a.N / 16 - 1);
      pbs = reinterpret_cast<const uint8_t*>(a.ws) + expert * a.ws_estride + grp16 * tsteps * 128 + (r & 15) * 2;
    } else {
      const int64_t n = min<int64_t>(n0 + min(tid, BN - 1), a.N - 1);
      pbs = reinterpret_cast<const uint8_t*>(a.ws) + expert * a.ws_estride + n * a.ws_s0;
    }
  }
  const float* swb = reinterpret_cast<const float*>(a.ws) + expert * a.ws_estride;
  const int64_t nb_scale = n0 / 128;

  uint4 ra[A_IT], rb[B_IT];
  uint32_t rbs = 0;
  float sw_next = 0.f;
  auto gload_w = [&](int ks) __attribute__((always_inline)) {
    const int64_t kbase = int64_t(ks) * 128;
    // byte offset of this K step inside a chunk's row (plain) or tile sequence (tiled)
    const int64_t bstep = TILED ? (MX ? int64_t(ks >> 1) * 2048 + (ks & 1) * 512 : int64_t(ks) * 2048)
                                : kbase * L::row_bytes / 128;
#pragma unroll
    for (int i = 0; i < B_IT; ++i)
      rb[i] = (kbase + kbo[i] < a.K) ? *reinterpret_cast<const uint4*>(pb[i] + bstep) : make_uint4(0, 0, 0, 0);
    if (MX && TILED && tid < BN) {
      // groups 4 ks .. 4 ks + 3: two byte pairs of the row's scale tile
      const uint8_t* sp = pbs + int64_t(ks >> 1) * 128 + (ks & 1) * 64;
      rbs = uint32_t(*reinterpret_cast<const uint16_t*>(sp)) |
            (uint32_t(*reinterpret_cast<const uint16_t*>(sp + 32)) << 16);
    } else if (MX && tid < BN) {
      const int g0 = ks * 4;  // first 32-group of this step
      uint32_t v = 0;
      const int ngrp = int(a.K >> 5);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (g0 + g < ngrp) v |= uint32_t(pbs[g0 + g]) << (8 * g);
      rbs = v;
    }
    // the weight-block scale of the step is read with its operands, one step ahead of its use
    if (WFMT == W_E4M3_BLOCK) sw_next = swb[nb_scale * a.ws_s0 + ks * a.ws_s1];
  };

  for (int m_base = 0; m_base < t.m_total; m_base += BM) {
  const int m_size = min(BM, t.m_total - m_base);
  __syncthreads();
  if (ks_b < ks_e) gload_w(ks_b);
  fill_rows<BM, MODE>(a, t, m_base, sArow, sOrow);
  __syncthreads();

  const uint16_t* pa[A_IT];
  int ka[A_IT];
  bool la[A_IT];  // the chunk's row holds data (rows past m_size are zero-filled)
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int c = min(tid + NT * i, BM * 16 - 1);
    ka[i] = (c & 15) * 8;
    la[i] = (c >> 4) < m_size;
    pa[i] = A + sArow[c >> 4] * a.lda + ka[i];
  }
  auto gload_a = [&](int ks) __attribute__((always_inline)) {
    const int64_t kbase = int64_t(ks) * 128;
#pragma unroll
    for (int i = 0; i < A_IT; ++i)
      ra[i] = (la[i] && kbase + ka[i] < a.K) ? *reinterpret_cast<const uint4*>(pa[i] + kbase) : make_uint4(0, 0, 0, 0);
  };
  auto lstore = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const int c = tid + NT * i;
      if (A_IT * NT == BM * 16 || c < BM * 16)
        *reinterpret_cast<uint4*>(sA + (c >> 4) * A_LROW + (c & 15) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      const int c = tid + NT * i;
      if (B_IT * NT == BN * L::chunks || c < BN * L::chunks) *reinterpret_cast<uint4*>(sB + sbo[i]) = rb[i];
    }
    if (MX && tid < BN) sBs[tid] = rbs;
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fq = lane >> 4;  // which 8-element K slice of a 32-wide MFMA step
  // 16-row MFMA tiles of this wave that hold rows of the block
  const int tm_live = min(TM, max(0, (m_size - wm * WM + 15) >> 4));

  if (ks_b < ks_e) gload_a(ks_b);
  for (int ks = ks_b; ks < ks_e; ++ks) {
    const float sw = sw_next;
    __syncthreads();
    lstore();
    __syncthreads();
    if (ks + 1 < ks_e) {
      gload_w(ks + 1);
      gload_a(ks + 1);
    }

    const int nsub = int(min<int64_t>(4, (a.K - int64_t(ks) * 128) >> 5));
    f32x4 part[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s >= nsub) break;
      i32x4 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        if (i < tm_live)
          af[i] = *reinterpret_cast<const i32x4*>(sA + (wm * WM + 16 * i + frow) * A_LROW + (s * 32 + fq * 8) * 2);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int brow = wn * WN + 16 * j + frow;
        if (MX) {
          const uint32_t v = *reinterpret_cast<const uint32_t*>(sB + brow * L::lds_row + s * 16 + fq * 4);
          const float sc = e8m0_to_f32((sBs[brow] >> (8 * s)) & 0xffu);
          uint32_t o[4];
          e2m1x8_to_bf16(v, sc, o);
          bfr[j] = i32x4{int(o[0]), int(o[1]), int(o[2]), int(o[3])};
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(sB + brow * L::lds_row + s * 32 + fq * 8);
          uint32_t o0, o1, o2, o3;
          e4m3x4_to_bf16(v.x, o0, o1);
          e4m3x4_to_bf16(v.y, o2, o3);
          bfr[j] = i32x4{int(o0), int(o1), int(o2), int(o3)};
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i >= tm_live) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if (WFMT == W_E4M3_BLOCK)
            part[i][j] = mfma_16x16x32_bf16(af[i], bfr[j], part[i][j]);
          else
            acc[i][j] = mfma_16x16x32_bf16(af[i], bfr[j], acc[i][j]);
        }
      }
    }
    if (WFMT == W_E4M3_BLOCK) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(part[i][j][r], sw, acc[i][j][r]);
    }
  }

  const float tscale = (WFMT == W_E4M3_TENSOR) ? reinterpret_cast<const float*>(a.ws)[0] : 1.f;
  // Outputs with 16-byte aligned rows go through LDS (the operand buffers are free after the K
  // loop) and leave as 16-byte row chunks instead of 2- or 4-byte column stores.  K-split
  // chunks write their fp32 partial sums to their own slice; the bias rides on chunk 0.
  constexpr int OE = OUT_F32 ? 4 : 2;          // output element bytes
  constexpr int OROW = BN + (OUT_F32 ? 4 : 8); // staged row, elements (padding against bank conflicts)
  constexpr int CH = 16 / OE;                  // elements per 16-byte chunk
  static_assert(size_t(BM) * OROW * OE <= w16_lds_bytes<BM, BN, WFMT, OUT_F32>(), "staged output fits the tile's LDS");
  uint8_t* const obase = static_cast<uint8_t*>(a.out) + (nsplit > 1 ? split * a.split_stride * OE : 0);
  const bool staged = (reinterpret_cast<uintptr_t>(obase) & 15) == 0 && (a.ldo % CH) == 0;
  if (staged) {
    __syncthreads();  // every wave is done with the operand buffers
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int cl = wn * WN + 16 * j + frow;
      const int64_t col = n0 + cl;
      const float b = HAS_BIAS && split == 0 && col < a.N ? load_bias(a, expert, col) : 0.f;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = acc[i][j][r];
          if (WFMT == W_E4M3_TENSOR) v = v * tscale;
          const int rl = wm * WM + 16 * i + 4 * (lane >> 4) + r;
          if (OUT_F32)
            reinterpret_cast<float*>(lds)[rl * OROW + cl] = v + b;
          else
            reinterpret_cast<uint16_t*>(lds)[rl * OROW + cl] = f2bf(v + b);
        }
    }
    __syncthreads();
    const int64_t ncols = min<int64_t>(BN, a.N - n0);
    for (int c = tid; c < m_size * (BN / CH); c += NT) {
      const int rl = c / (BN / CH), ch = c % (BN / CH);
      const int64_t col = n0 + ch * CH;
      uint8_t* dst = obase + (sOrow[rl] * a.ldo + col) * OE;
      const uint8_t* src = lds + (rl * OROW + ch * CH) * OE;
      if (ch * CH + CH <= ncols) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int e = 0; e < CH && ch * CH + e < ncols; ++e)
          for (int k = 0; k < OE; ++k) dst[e * OE + k] = src[e * OE + k];
      }
    }
    continue;  // next row pass (its first barrier orders these LDS reads before new writes)
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t col = n0 + wn * WN + 16 * j + frow;
    if (col >= a.N) continue;
    const float b = HAS_BIAS && split == 0 ? load_bias(a, expert, col) : 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * WM + 16 * i + 4 * (lane >> 4) + r;
        if (rl >= m_size) continue;
        float v = acc[i][j][r];
        if (WFMT == W_E4M3_TENSOR) v = v * tscale;
        v = v + b;
        const int64_t o = sOrow[rl] * a.ldo + col;
        if (OUT_F32)
          reinterpret_cast<float*>(obase)[o] = v;
        else
          reinterpret_cast<uint16_t*>(obase)[o] = f2bf(v);
      }
  }
  }  // m sub-tiles
}

template <int BM, int BN, int WAVES_M, int MODE, int WFMT, bool OUT_F32, bool HAS_BIAS, bool TILED>
__global__ __launch_bounds__(256) void gemm_w16_kernel(GemmArgs a, int64_t grid_blocks) {
  extern __shared__ __align__(16) uint8_t w16_lds[];
  if constexpr (MODE == ROWS_DENSE && WFMT == W_E4M3_TENSOR) {
    // batch entry z = blockIdx.y of a batched product (z = 0 otherwise)
    const int64_t z = blockIdx.y;
    a.A = static_cast<const uint16_t*>(a.A) + z * a.a_bstride;
    a.W += z * a.w_estride;
    a.ws = static_cast<const float*>(a.ws) + z * a.ws_estride;
    if (HAS_BIAS)
      a.bias = static_cast<const uint8_t*>(a.bias) + z * a.bias_estride * (a.bias_bf16 ? 2 : 4);
    a.out = static_cast<uint8_t*>(a.out) + z * a.o_bstride * (OUT_F32 ? 4 : 2);
  }
  w16_tile<256, BM, BN, WAVES_M, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(a, grid_blocks, blockIdx.x, w16_lds);
}

// Routed tile classes 16 / 32 / 64 / 128 rows in one launch of 512-thread workgroups (two
// waves per SIMD, so one wave's LDS reads overlap the other's products): workgroups
// [off[c], off[c + 1]) run tiles of class c over its own work list, so the classes of a stage
// run side by side instead of one launch after another (small batches leave most of the GPU
// idle in each).  The 128-row class comes first in the grid, then 64, 32, 16: the longest
// tiles start first instead of queueing behind the other classes' workgroups.
constexpr int kW16GroupThreads = 512;
struct W16Group {
  GemmArgs a[4];    // per class (16, 32, 64, 128 rows): the stage's arguments with its work list
  int64_t gb[4];    // per class: work-list capacity
  int64_t off[5];   // launch order 128, 64, 32, 16 rows: off[0] = 0, off[4] = grid size
};

template <int MODE, int WFMT, bool OUT_F32, bool HAS_BIAS, bool TILED>
__global__ __launch_bounds__(kW16GroupThreads) void gemm_w16_grouped_kernel(W16Group g) {
  extern __shared__ __align__(16) uint8_t w16_lds[];
  constexpr int NT = kW16GroupThreads;
  const int64_t b = blockIdx.x;
  if (b < g.off[1])
    w16_tile<NT, 128, 128, 4, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(g.a[3], g.gb[3], b - g.off[0], w16_lds);
  else if (b < g.off[2])
    w16_tile<NT, 64, 128, 2, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(g.a[2], g.gb[2], b - g.off[1], w16_lds);
  else if (b < g.off[3])
    w16_tile<NT, 32, 128, 2, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(g.a[1], g.gb[1], b - g.off[2], w16_lds);
  else
    w16_tile<NT, 16, 128, 1, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(g.a[0], g.gb[0], b - g.off[3], w16_lds);
}

template <int BM, int BN, int WAVES_M, int MODE, int WFMT, bool TL>
static void launch_w16_tl(const GemmArgs& a, bool out_f32, int64_t grid_blocks, hipStream_t st, unsigned batch = 1) {
  const int64_t n_tiles = cdiv(a.N, BN);
  const int64_t nsplit = a.k_split > 1 ? a.k_split : 1;
  const dim3 grid(unsigned(grid_blocks * n_tiles * nsplit), batch), block(256);
  const bool bias = a.bias != nullptr;
  const size_t lds = out_f32 ? w16_lds_bytes<BM, BN, WFMT, true>() : w16_lds_bytes<BM, BN, WFMT, false>();
#define MXQ_W16_GO(OF, HB) \
  hipLaunchKernelGGL((gemm_w16_kernel<BM, BN, WAVES_M, MODE, WFMT, OF, HB, TL>), grid, block, lds, st, a, grid_blocks)
  if (out_f32) { if (bias) MXQ_W16_GO(true, true); else MXQ_W16_GO(true, false); }
  else { if (bias) MXQ_W16_GO(false, true); else MXQ_W16_GO(false, false); }
#undef MXQ_W16_GO
}

template <int BM, int BN, int WAVES_M, int MODE, int WFMT>
static void launch_w16_t(const GemmArgs& a, bool out_f32, int64_t grid_blocks, hipStream_t st, unsigned batch = 1) {
  if constexpr (MODE != ROWS_DENSE && WFMT != W_E4M3_TENSOR) {
    if (a.w_tiled) {
      launch_w16_tl<BM, BN, WAVES_M, MODE, WFMT, true>(a, out_f32, grid_blocks, st);
      return;
    }
  }
  launch_w16_tl<BM, BN, WAVES_M, MODE, WFMT, false>(a, out_f32, grid_blocks, st, batch);
}

template <int MODE, int WFMT>
static void launch_w16_mode(const GemmArgs& a, int tile, bool out_f32, int64_t gb, hipStream_t st,
                            unsigned batch = 1) {
  switch (tile) {
    case 0: launch_w16_t<128, 128, 2, MODE, WFMT>(a, out_f32, gb, st, batch); break;
    case 1: launch_w16_t<64, 128, 2, MODE, WFMT>(a, out_f32, gb, st, batch); break;
    case 2: launch_w16_t<32, 128, 1, MODE, WFMT>(a, out_f32, gb, st, batch); break;
    default: launch_w16_t<16, 128, 1, MODE, WFMT>(a, out_f32, gb, st, batch); break;
  }
}

template <int MODE>
static void launch_w16_fmt(const GemmArgs& a, int wfmt, int tile, bool out_f32, int64_t gb, hipStream_t st) {
  switch (wfmt) {
    case W_E4M3_BLOCK: launch_w16_mode<MODE, W_E4M3_BLOCK>(a, tile, out_f32, gb, st); break;
    case W_E4M3_TENSOR: launch_w16_mode<MODE, W_E4M3_TENSOR>(a, tile, out_f32, gb, st); break;
    default: launch_w16_mode<MODE, W_E2M1_MX>(a, tile, out_f32, gb, st); break;
  }
}

template <int MODE, int WFMT, bool TL>
static void launch_w16_grouped_t(const W16Group& g, bool out_f32, size_t lds, hipStream_t st) {
  const dim3 grid(unsigned(g.off[4])), block(kW16GroupThreads);
  const bool bias = g.a[0].bias != nullptr;
#define MXQ_W16G_GO(OF, HB) \
  hipLaunchKernelGGL((gemm_w16_grouped_kernel<MODE, WFMT, OF, HB, TL>), grid, block, lds, st, g)
  if (out_f32) { if (bias) MXQ_W16G_GO(true, true); else MXQ_W16G_GO(true, false); }
  else { if (bias) MXQ_W16G_GO(false, true); else MXQ_W16G_GO(false, false); }
#undef MXQ_W16G_GO
}

template <int MODE, int WFMT>
static void launch_w16_grouped_m(const W16Group& g, bool out_f32, hipStream_t st) {
  // LDS of the largest class that holds workgroups (launch order 128, 64, 32, 16 rows)
  size_t lds = 0;
  const size_t per_f32[4] = {w16_lds_bytes<128, 128, WFMT, true>(), w16_lds_bytes<64, 128, WFMT, true>(),
                             w16_lds_bytes<32, 128, WFMT, true>(), w16_lds_bytes<16, 128, WFMT, true>()};
  const size_t per_bf16[4] = {w16_lds_bytes<128, 128, WFMT, false>(), w16_lds_bytes<64, 128, WFMT, false>(),
                              w16_lds_bytes<32, 128, WFMT, false>(), w16_lds_bytes<16, 128, WFMT, false>()};
  for (int i = 0; i < 4; ++i)
    if (g.off[i + 1] > g.off[i]) lds = std::max(lds, out_f32 ? per_f32[i] : per_bf16[i]);
  if (g.a[0].w_tiled)
    launch_w16_grouped_t<MODE, WFMT, true>(g, out_f32, lds, st);
  else
    launch_w16_grouped_t<MODE, WFMT, false>(g, out_f32, lds, st);
}

void launch_gemm_w16_batched(const GemmArgs& a, int tile, int64_t batch, hipStream_t stream) {
  const int64_t gb = cdiv(a.M, int64_t(tile == 0 ? 128 : tile == 1 ? 64 : tile == 2 ? 32 : 16));
  if (batch <= 0 || gb <= 0 || a.N <= 0) return;
  launch_w16_mode<ROWS_DENSE, W_E4M3_TENSOR>(a, tile, false, gb, stream, unsigned(batch));
}

void launch_gemm_w16_grouped(const GemmArgs cls[4], const int64_t grid_blocks[4], int wfmt, int row_mode,
                             bool out_f32, hipStream_t stream) {
  W16Group g{};
  g.off[0] = 0;
  for (int c = 0; c < 4; ++c) {
    g.a[c] = cls[c];
    g.gb[c] = std::max<int64_t>(grid_blocks[c], 0);
  }
  for (int i = 0; i < 4; ++i) {  // launch order: 128-, 64-, 32-, 16-row class
    const int c = 3 - i;
    g.off[i + 1] = g.off[i] + g.gb[c] * cdiv(cls[c].N, 128) * std::max<int64_t>(cls[c].k_split, 1);
  }
  if (g.off[4] <= 0) return;
  const bool mx = wfmt == W_E2M1_MX;
  if (row_mode == ROWS_GATHER_TOK) {
    if (mx) launch_w16_grouped_m<ROWS_GATHER_TOK, W_E2M1_MX>(g, out_f32, stream);
    else launch_w16_grouped_m<ROWS_GATHER_TOK, W_E4M3_BLOCK>(g, out_f32, stream);
  } else {
    if (mx) launch_w16_grouped_m<ROWS_COMPACT_IN, W_E2M1_MX>(g, out_f32, stream);
    else launch_w16_grouped_m<ROWS_COMPACT_IN, W_E4M3_BLOCK>(g, out_f32, stream);
  }
}

void launch_gemm_w16(const GemmArgs& a, int wfmt, int row_mode, int tile, bool out_f32, int64_t grid_blocks,
                     hipStream_t stream) {
  if (grid_blocks <= 0 || a.N <= 0) return;
  switch (row_mode) {
    case ROWS_DENSE: launch_w16_fmt<ROWS_DENSE>(a, wfmt, tile, out_f32, grid_blocks, stream); break;
    case ROWS_GATHER_TOK: launch_w16_fmt<ROWS_GATHER_TOK>(a, wfmt, tile, out_f32, grid_blocks, stream); break;
    default: launch_w16_fmt<ROWS_COMPACT_IN>(a, wfmt, tile, out_f32, grid_blocks, stream); break;
  }
}

}  // namespace mxq
