// Wavefront-reduction GEMV for tiny routed expert blocks.
//
// "vLLM PR 50949 review" (implementation item 2 and the gemm.h listing): a
// block with few rows is better served by a fixed-row micro-kernel than by a
// large-tile GEMM.  On gfx950 that micro-kernel is this one: each wave owns
// four weight rows and streams them with coalesced 16-byte loads along K (64
// lanes cover 1024 e4m3 or 2048 e2m1 values per step), decodes each chunk to
// bf16 pairs, and forms the dot products against up to four activation rows
// with V_DOT2_F32_BF16; the 64 lane partials of each (row, column) are summed
// with a butterfly at the end.  Block scales are applied per 128-wide K block
// (e4m3 weights; times the per-token activation scale for W8A8) or folded into
// the exact e2m1 decode (MXFP4).  Blocks taller than four rows are processed
// four rows at a time.
#include "tile_rows.hpp"

namespace mxq {

constexpr int kGemvRows = 4;     // activation rows per pass
constexpr int kGemvRowsPerWave = 4;
constexpr int kGemvTileN = 4 * kGemvRowsPerWave;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int WFMT, bool A_E4M3, int MODE, bool OUT_F32, bool HAS_BIAS>
__global__ __launch_bounds__(256) void gemv_kernel(GemmArgs a, int64_t grid_blocks) {
  constexpr bool MX = WFMT == W_E2M1_MX;
  constexpr int CHUNK = MX ? 32 : 16;  // K elements per 16-byte weight load
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tile = blockIdx.x % grid_blocks;
  const int64_t nt = blockIdx.x / grid_blocks;
  const int64_t nw0 = nt * kGemvTileN + wave * kGemvRowsPerWave;  // first weight row of this wave
  if (nt * kGemvTileN >= a.N) return;

  TileInfo t;
  if (!tile_info<1, MODE>(a, tile, t)) return;
  const int64_t expert = t.expert;
  const uint8_t* Wb = a.W + expert * a.w_estride;
  const int64_t nchunks = a.K / CHUNK;

  int64_t nrow[kGemvRowsPerWave];
#pragma unroll
  for (int r = 0; r < kGemvRowsPerWave; ++r) nrow[r] = min<int64_t>(nw0 + r, a.N - 1);

  for (int m_base = 0; m_base < t.m_total; m_base += kGemvRows) {
    const int m_size = min(kGemvRows, t.m_total - m_base);
    int64_t arow[kGemvRows], orow[kGemvRows];
#pragma unroll
    for (int m = 0; m < kGemvRows; ++m) row_of<MODE>(a, t, m_base + min(m, m_size - 1), arow[m], orow[m]);

    float acc[kGemvRows][kGemvRowsPerWave];
#pragma unroll
    for (int m = 0; m < kGemvRows; ++m)
#pragma unroll
      for (int r = 0; r < kGemvRowsPerWave; ++r) acc[m][r] = 0.f;

    for (int64_t c = lane; c < nchunks; c += 64) {
      const int64_t k0 = c * CHUNK;
      // activations for this chunk as bf16 pairs (CHUNK / 2 dwords per row)
      uint32_t av[kGemvRows][CHUNK / 2];
      float asc[kGemvRows];
#pragma unroll
      for (int m = 0; m < kGemvRows; ++m) {
        if (A_E4M3) {
          const uint8_t* ap = reinterpret_cast<const uint8_t*>(a.A) + arow[m] * a.lda + k0;
          const uint4 q = *reinterpret_cast<const uint4*>(ap);
          e4m3x4_to_bf16(q.x, av[m][0], av[m][1]);
          e4m3x4_to_bf16(q.y, av[m][2], av[m][3]);
          e4m3x4_to_bf16(q.z, av[m][4], av[m][5]);
          e4m3x4_to_bf16(q.w, av[m][6], av[m][7]);
          asc[m] = a.sa[arow[m] * a.lds + (k0 >> 7)];
        } else {
          const uint16_t* ap = reinterpret_cast<const uint16_t*>(a.A) + arow[m] * a.lda + k0;
#pragma unroll
          for (int v = 0; v < CHUNK / 8; ++v) {
            const uint4 q = *reinterpret_cast<const uint4*>(ap + 8 * v);
            av[m][4 * v + 0] = q.x;
            av[m][4 * v + 1] = q.y;
            av[m][4 * v + 2] = q.z;
            av[m][4 * v + 3] = q.w;
          }
          asc[m] = 1.f;
        }
      }
#pragma unroll
      for (int r = 0; r < kGemvRowsPerWave; ++r) {
        const uint4 wq = *reinterpret_cast<const uint4*>(Wb + nrow[r] * a.ldw + (MX ? (k0 >> 1) : k0));
        uint32_t wv[CHUNK / 2];
        float wscale = 1.f;
        if (MX) {
          const uint8_t e = reinterpret_cast<const uint8_t*>(a.ws)[expert * a.ws_estride + nrow[r] * a.ws_s0 + c];
          const float sc = e8m0_to_f32(e);
          e2m1x8_to_bf16(wq.x, sc, wv + 0);
          e2m1x8_to_bf16(wq.y, sc, wv + 4);
          e2m1x8_to_bf16(wq.z, sc, wv + 8);
          e2m1x8_to_bf16(wq.w, sc, wv + 12);
        } else {
          e4m3x4_to_bf16(wq.x, wv[0], wv[1]);
          e4m3x4_to_bf16(wq.y, wv[2], wv[3]);
          e4m3x4_to_bf16(wq.z, wv[4], wv[5]);
          e4m3x4_to_bf16(wq.w, wv[6], wv[7]);
          const int64_t nb = (a.block_n == 1) ? nrow[r] : (nrow[r] >> 7);
          wscale = reinterpret_cast<const float*>(a.ws)[expert * a.ws_estride + nb * a.ws_s0 + (k0 >> 7) * a.ws_s1];
        }
#pragma unroll
        for (int m = 0; m < kGemvRows; ++m) {
          float p = 0.f;
#pragma unroll
          for (int v = 0; v < CHUNK / 2; ++v) p = dot2(av[m][v], wv[v], p);
          if (MX)
            acc[m][r] += p;
          else
            acc[m][r] = fmaf(p, asc[m] * wscale, acc[m][r]);
        }
      }
    }

#pragma unroll
    for (int m = 0; m < kGemvRows; ++m)
#pragma unroll
      for (int r = 0; r < kGemvRowsPerWave; ++r) acc[m][r] = wave_sum(acc[m][r]);

    // lane (m * 4 + r) stores output (m, r)
    if (lane < kGemvRows * kGemvRowsPerWave) {
      const int m = lane / kGemvRowsPerWave, r = lane % kGemvRowsPerWave;
      float v = 0.f;
#pragma unroll
      for (int mm = 0; mm < kGemvRows; ++mm)
#pragma unroll
        for (int rr = 0; rr < kGemvRowsPerWave; ++rr)
          if (mm == m && rr == r) v = acc[mm][rr];
      const int64_t col = nw0 + r;
      if (m < m_size && col < a.N) {
        int64_t o = 0;
#pragma unroll
        for (int mm = 0; mm < kGemvRows; ++mm)
          if (mm == m) o = orow[mm];
        if (HAS_BIAS) v += load_bias(a, expert, col);
        if (OUT_F32)
          reinterpret_cast<float*>(a.out)[o * a.ldo + col] = v;
        else
          reinterpret_cast<uint16_t*>(a.out)[o * a.ldo + col] = f2bf(v);
      }
    }
  }
}

template <int WFMT, bool AE, int MODE>
static void launch_gemv_t(const GemmArgs& a, bool out_f32, int64_t gb, hipStream_t st) {
  const int64_t n_tiles = cdiv(a.N, kGemvTileN);
  const dim3 grid(unsigned(gb * n_tiles)), block(256);
  const bool bias = a.bias != nullptr;
#define MXQ_GEMV_GO(OF, HB) hipLaunchKernelGGL((gemv_kernel<WFMT, AE, MODE, OF, HB>), grid, block, 0, st, a, gb)
  if (out_f32) { if (bias) MXQ_GEMV_GO(true, true); else MXQ_GEMV_GO(true, false); }
  else { if (bias) MXQ_GEMV_GO(false, true); else MXQ_GEMV_GO(false, false); }
#undef MXQ_GEMV_GO
}

template <int MODE>
static void launch_gemv_mode(const GemmArgs& a, int wfmt, bool a_e4m3, bool out_f32, int64_t gb, hipStream_t st) {
  if (wfmt == W_E2M1_MX)
    launch_gemv_t<W_E2M1_MX, false, MODE>(a, out_f32, gb, st);
  else if (a_e4m3)
    launch_gemv_t<W_E4M3_BLOCK, true, MODE>(a, out_f32, gb, st);
  else
    launch_gemv_t<W_E4M3_BLOCK, false, MODE>(a, out_f32, gb, st);
}

void launch_gemv(const GemmArgs& a, int wfmt, bool a_e4m3, int row_mode, bool out_f32, int64_t grid_blocks,
                 hipStream_t stream) {
  if (grid_blocks <= 0 || a.N <= 0) return;
  switch (row_mode) {
    case ROWS_DENSE: launch_gemv_mode<ROWS_DENSE>(a, wfmt, a_e4m3, out_f32, grid_blocks, stream); break;
    case ROWS_GATHER_TOK: launch_gemv_mode<ROWS_GATHER_TOK>(a, wfmt, a_e4m3, out_f32, grid_blocks, stream); break;
    default: launch_gemv_mode<ROWS_COMPACT_IN>(a, wfmt, a_e4m3, out_f32, grid_blocks, stream); break;
  }
}

}  // namespace mxq
