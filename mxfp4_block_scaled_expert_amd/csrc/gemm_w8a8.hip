// Block-scaled W8A8 GEMM on the gfx950 FP8 matrix cores.
//
// "SGLang PR 35605 review" (implementation item 1, fp8_utils.py listing):
// out[m, n] = sum_kb sa[m, kb] * sw[n / block_n, kb] * sum_{k in kb} qa[m, k] * w[n, k]
// (+ bias), activations scaled per token per 128 columns, weights per 128x128
// (or 1x128) block, bf16 output.  The same kernel runs the W8A8 stages of the
// routed MoE ("vLLM PR 50949 review", moe_fp8.cpp listing), reading and
// writing rows through the expert-block tables.
//
// One V_MFMA_F32_16X16X128_F8F6F4 covers exactly one 128-wide K block, so each
// K block's 16x16 partial product is formed on the matrix core from zero and
// promoted into the fp32 accumulator with its combined scale sa * sw on the
// vector ALU (one FMA per accumulator element per K block).
//
// Tiles: BM x BN per 256-thread workgroup (4 waves, WAVES_M x WAVES_N), K step 128.
// Routed weights may come in the tiled layout of prepack.hip (TILED): then each
// 16-row x 128-byte piece of the weight tile is one contiguous 2 KB tile.
// Operand tiles are staged through LDS with a 16-byte row pad (no bank
// conflicts on the 32-byte fragment reads); the next K block's tiles are
// fetched into registers while the current one is multiplied.
#include "tile_rows.hpp"

namespace mxq {

constexpr int kLdsRow = 144;  // 128 data bytes + 16 pad

template <int BM, int BN, int WAVES_M, int MODE, bool SW_COL, bool OUT_F32, bool HAS_BIAS, bool TILED>
__global__ __launch_bounds__(256, 2) void gemm_w8a8_kernel(GemmArgs a, int64_t grid_blocks) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  static_assert(TM >= 1 && TN >= 1, "wave tile smaller than one MFMA tile");
  static_assert(SW_COL || BN <= 128, "a 128-wide weight scale block must cover the whole N tile");
  constexpr int A_IT = (BM * 8 + 255) / 256;
  constexpr int B_IT = (BN * 8 + 255) / 256;

  __shared__ __align__(16) uint8_t sA[BM * kLdsRow];
  __shared__ __align__(16) uint8_t sB[BN * kLdsRow];
  __shared__ float sSa[BM];
  __shared__ int64_t sArow[BM];
  __shared__ int64_t sOrow[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int64_t tile = blockIdx.x % grid_blocks;
  const int64_t nt = blockIdx.x / grid_blocks;
  const int64_t n0 = nt * BN;
  if (n0 >= a.N) return;

  TileInfo t;
  if (!tile_info<BM, MODE>(a, tile, t)) return;
  const int64_t expert = t.expert;
  for (int m_base = 0; m_base < t.m_total; m_base += BM) {
  const int m_size = min(BM, t.m_total - m_base);
  __syncthreads();
  fill_rows<BM, MODE>(a, t, m_base, sArow, sOrow);
  __syncthreads();

  const uint8_t* A = reinterpret_cast<const uint8_t*>(a.A);
  const uint8_t* Wb = a.W + expert * a.w_estride;
  const float* swb = reinterpret_cast<const float*>(a.ws) + expert * a.ws_estride;
  const int KB = int(a.K >> 7);

  // per-thread global chunk coordinates (16-byte chunks, 8 per 128-byte row)
  const uint8_t* pa[A_IT];
  const uint8_t* pb[B_IT];
  int sbo[B_IT];  // LDS byte offset of the chunk
  constexpr int B_KSTRIDE = TILED ? 2048 : 128;  // bytes between consecutive K blocks of one chunk
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int c = min(tid + 256 * i, BM * 8 - 1);
    pa[i] = A + sArow[c >> 3] * a.lda + (c & 7) * 16;
  }
#pragma unroll
  for (int i = 0; i < B_IT; ++i) {
    const int c = min(tid + 256 * i, BN * 8 - 1);
    if (TILED) {
      // chunk c = 16 contiguous bytes of tile c / 128 (consecutive threads read one 2 KB tile)
      const int t = c >> 7, p = c & 127, L = p & 63;
      const int64_t grp16 = min<int64_t>(n0 / 16 + t, a.N / 16 - 1);
      pb[i] = Wb + grp16 * KB * 2048 + p * 16;
      sbo[i] = (16 * t + (L & 15)) * kLdsRow + (L >> 4) * 32 + (p >> 6) * 16;
    } else {
      const int64_t n = min<int64_t>(n0 + (c >> 3), a.N - 1);
      pb[i] = Wb + n * a.ldw + (c & 7) * 16;
      sbo[i] = (c >> 3) * kLdsRow + (c & 7) * 16;
    }
  }
  const float* psa = a.sa + sArow[min(tid, BM - 1)] * a.lds;

  i32x4 ra[A_IT], rb[B_IT];
  float rsa = 0.f;
#define MXQ_W8A8_GLOAD(KB)                                                                     \
  do {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < A_IT; ++i) ra[i] =                                   \
        *reinterpret_cast<const i32x4*>(pa[i] + (KB) * 128);                                   \
    _Pragma("unroll") for (int i = 0; i < B_IT; ++i) rb[i] =                                   \
        *reinterpret_cast<const i32x4*>(pb[i] + (KB) * B_KSTRIDE);                             \
    rsa = psa[KB];                                                                             \
  } while (0)

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane fragment coordinates
  const int frow = lane & 15;
  const int fk = (lane >> 4) * 32;
  const int64_t nb_scale = n0 / 128;  // weight-scale grid row for 128-wide blocks

  MXQ_W8A8_GLOAD(0);
  for (int kb = 0; kb < KB; ++kb) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const int c = tid + 256 * i;
      if (A_IT * 256 == BM * 8 || c < BM * 8)
        *reinterpret_cast<i32x4*>(sA + (c >> 3) * kLdsRow + (c & 7) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      const int c = tid + 256 * i;
      if (B_IT * 256 == BN * 8 || c < BN * 8) *reinterpret_cast<i32x4*>(sB + sbo[i]) = rb[i];
    }
    if (tid < BM) sSa[tid] = rsa;
    __syncthreads();
    // this block's weight scales are loaded before the next block's operands: loads retire
    // in order, so waiting for the scales does not wait for the prefetch
    float sw_tile = 1.f;
    float swc[TN];
    if (!SW_COL) sw_tile = swb[nb_scale * a.ws_s0 + kb * a.ws_s1];
    if (SW_COL) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = min<int64_t>(n0 + wn * WN + 16 * j + frow, a.N - 1);
        swc[j] = swb[n * a.ws_s0 + kb * a.ws_s1];
      }
    }
    if (kb + 1 < KB) MXQ_W8A8_GLOAD(kb + 1);

    i32x8 af[TM], bfr[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint8_t* p = sA + (wm * WM + 16 * i + frow) * kLdsRow + fk;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
      af[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint8_t* p = sB + (wn * WN + 16 * j + frow) * kLdsRow + fk;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
      bfr[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    float cs[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) cs[i][r] = sSa[wm * WM + 16 * i + 4 * (lane >> 4) + r] * sw_tile;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // Products t = TN * i + j run as a software pipeline: step t issues the MFMA of product
    // t + 2 and promotes product t, whose MFMA went out two MFMAs earlier, from a ring of
    // three partial-sum registers; the fence after each step keeps that order.
    constexpr int NT = TM * TN, DIST = NT < 2 ? NT : 2, NB = DIST + 1;
    f32x4 pb[NB];
#pragma unroll
    for (int t = 0; t < DIST; ++t) pb[t] = mfma_16x16x128_e4m3(af[t / TN], bfr[t % TN], zero);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tm = t + DIST;
      if (tm < NT) pb[tm % NB] = mfma_16x16x128_e4m3(af[tm / TN], bfr[tm % TN], zero);
      const int i = t / TN, j = t % TN;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float c = SW_COL ? cs[i][r] * swc[j] : cs[i][r];
        acc[i][j][r] = fmaf(pb[t % NB][r], c, acc[i][j][r]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+r of each 16x16 tile, column lane%16
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t col = n0 + wn * WN + 16 * j + frow;
    if (col >= a.N) continue;
    const float b = HAS_BIAS ? load_bias(a, expert, col) : 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * WM + 16 * i + 4 * (lane >> 4) + r;
        if (rl >= m_size) continue;
        const float v = acc[i][j][r] + b;
        const int64_t orow = sOrow[rl];
        if (OUT_F32)
          reinterpret_cast<float*>(a.out)[orow * a.ldo + col] = v;
        else
          reinterpret_cast<uint16_t*>(a.out)[orow * a.ldo + col] = f2bf(v);
      }
  }
  }  // m sub-tiles
#undef MXQ_W8A8_GLOAD
}

template <int BM, int BN, int WAVES_M, int MODE, bool TL>
static void launch_w8a8_tl(const GemmArgs& a, bool sw_col, bool out_f32, int64_t grid_blocks, hipStream_t st) {
  const int64_t n_tiles = cdiv(a.N, BN);
  const dim3 grid(unsigned(grid_blocks * n_tiles)), block(256);
  const bool bias = a.bias != nullptr;
#define MXQ_W8A8_GO(SWC, OF, HB) \
  hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, WAVES_M, MODE, SWC, OF, HB, TL>), grid, block, 0, st, a, grid_blocks)
  if (sw_col) {
    if (out_f32) { if (bias) MXQ_W8A8_GO(true, true, true); else MXQ_W8A8_GO(true, true, false); }
    else { if (bias) MXQ_W8A8_GO(true, false, true); else MXQ_W8A8_GO(true, false, false); }
  } else {
    if (out_f32) { if (bias) MXQ_W8A8_GO(false, true, true); else MXQ_W8A8_GO(false, true, false); }
    else { if (bias) MXQ_W8A8_GO(false, false, true); else MXQ_W8A8_GO(false, false, false); }
  }
#undef MXQ_W8A8_GO
}

template <int BM, int BN, int WAVES_M, int MODE>
static void launch_w8a8_t(const GemmArgs& a, bool sw_col, bool out_f32, int64_t grid_blocks, hipStream_t st) {
  if constexpr (MODE != ROWS_DENSE) {
    if (a.w_tiled) {
      launch_w8a8_tl<BM, BN, WAVES_M, MODE, true>(a, sw_col, out_f32, grid_blocks, st);
      return;
    }
  }
  launch_w8a8_tl<BM, BN, WAVES_M, MODE, false>(a, sw_col, out_f32, grid_blocks, st);
}

template <int MODE>
static void launch_w8a8_mode(const GemmArgs& a, int tile, bool out_f32, int64_t gb, hipStream_t st) {
  const bool sw_col = a.block_n == 1;
  switch (tile) {
    case 0: launch_w8a8_t<128, 128, 2, MODE>(a, sw_col, out_f32, gb, st); break;
    case 1: launch_w8a8_t<64, 128, 2, MODE>(a, sw_col, out_f32, gb, st); break;
    case 2: launch_w8a8_t<32, 128, 1, MODE>(a, sw_col, out_f32, gb, st); break;
    default: launch_w8a8_t<16, 128, 1, MODE>(a, sw_col, out_f32, gb, st); break;
  }
}

void launch_gemm_w8a8(const GemmArgs& a, int row_mode, int tile, bool out_f32, int64_t grid_blocks,
                      hipStream_t stream) {
  if (grid_blocks <= 0 || a.N <= 0) return;
  switch (row_mode) {
    case ROWS_DENSE: launch_w8a8_mode<ROWS_DENSE>(a, tile, out_f32, grid_blocks, stream); break;
    case ROWS_GATHER_TOK: launch_w8a8_mode<ROWS_GATHER_TOK>(a, tile, out_f32, grid_blocks, stream); break;
    default: launch_w8a8_mode<ROWS_COMPACT_IN>(a, tile, out_f32, grid_blocks, stream); break;
  }
}

}  // namespace mxq
