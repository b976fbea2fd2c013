// Row bookkeeping shared by the GEMM kernels: which operand rows a tile reads
// and which output rows it writes, for dense tiles and for routed expert
// blocks ("vLLM PR 50949 review", moe_fp8.cpp listing: a block's expert comes
// from expert_ids[mb], its row count is offsets[mb+1] - offsets[mb] and empty
// blocks are skipped, its input rows are sorted_ids[mb * BLOCK_M + m] / topk,
// and its outputs land in the compact intermediate at row offsets[mb] + m).
#pragma once

#include "kernels.hpp"

namespace mxq {

struct TileInfo {
  int64_t expert;
  int64_t m0;     // dense: first row of the tile
  int m_total;    // rows to process (a routed block may be taller than one tile)
  int mb;         // routed: block id
  int off;        // routed: compact row of the block's first row
};

// Uniform over the workgroup.  Returns false when the tile has no rows.
template <int BM, int MODE>
__device__ __forceinline__ bool tile_info(const GemmArgs& a, int64_t tile, TileInfo& t) {
  t.expert = 0;
  t.m0 = 0;
  t.mb = 0;
  t.off = 0;
  if (MODE == ROWS_DENSE) {
    t.m0 = tile * BM;
    if (t.m0 >= a.M) return false;
    t.m_total = int(min<int64_t>(BM, a.M - t.m0));
    return true;
  }
  // the count and the descriptor are read together (one memory round trip); a launch holds
  // at most the list's capacity of tiles, so the descriptor read stays in bounds
  const int4 d = *reinterpret_cast<const int4*>(a.rt.work_desc + tile * 4);
  const int32_t count = *a.rt.work_count;
  // one combined test over every field (no short-circuit), so that no part of either read
  // is deferred behind the other
  const bool live = (tile < int64_t(count)) & (d.x >= 0) & (d.y >= 0) & (d.w > 0);
  t.mb = d.x;
  t.expert = d.y;
  t.off = d.z;
  t.m_total = d.w;
  return live;
}

// Input row / output row of local row i (0 <= i < m_total).
template <int MODE>
__device__ __forceinline__ void row_of(const GemmArgs& a, const TileInfo& t, int i, int64_t& arow, int64_t& orow) {
  if (MODE == ROWS_DENSE) {
    arow = t.m0 + i;
    orow = t.m0 + i;
  } else {
    const int32_t id = a.rt.sorted_ids[int64_t(t.mb) * a.rt.block_m + i];
    if (MODE == ROWS_GATHER_TOK) {
      arow = id / a.rt.topk;
      orow = t.off + i;
    } else {
      arow = t.off + i;
      orow = id;
    }
  }
}

// Fills the LDS row tables for local rows m_base .. m_base + BM - 1; rows past
// m_total repeat the last valid input row and are never stored.
template <int BM, int MODE>
__device__ __forceinline__ void fill_rows(const GemmArgs& a, const TileInfo& t, int m_base, int64_t* s_arow,
                                          int64_t* s_orow) {
  for (int i = threadIdx.x; i < BM; i += blockDim.x) {
    const int ii = min(m_base + i, t.m_total - 1);
    int64_t ar, orw;
    row_of<MODE>(a, t, ii, ar, orw);
    s_arow[i] = ar;
    s_orow[i] = orw;
  }
}

__device__ __forceinline__ float load_bias(const GemmArgs& a, int64_t expert, int64_t col) {
  const int64_t idx = expert * a.bias_estride + col;
  return a.bias_bf16 ? bf16f(reinterpret_cast<const uint16_t*>(a.bias)[idx])
                     : reinterpret_cast<const float*>(a.bias)[idx];
}

}  // namespace mxq
