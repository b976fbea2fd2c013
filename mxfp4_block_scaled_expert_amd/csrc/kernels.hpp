// Internal interface between the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include "common.hpp"

namespace mxq {

// Which rows a GEMM tile reads and writes.
enum RowMode : int {
  ROWS_DENSE = 0,      // tile rows m0 .. m0+BM of a plain [M, K] operand
  ROWS_GATHER_TOK = 1, // routed block: A row = sorted_ids[..] / topk, out row = offsets[mb] + i
  ROWS_COMPACT_IN = 2, // routed block: A row = offsets[mb] + i, out row = sorted_ids[..]
};

// Weight formats.
enum WFmt : int {
  W_E4M3_BLOCK = 0,   // e4m3 + fp32 scale per (block_n x 128) block
  W_E4M3_TENSOR = 1,  // e4m3 + one fp32 scale (device scalar)
  W_E2M1_MX = 2,      // packed e2m1 + e8m0 scale per row per 32 columns
};

// Per-block tile-class policy: the class of a block of m_size rows.
struct ClassPolicy {
  int32_t n_classes;      // 0: no class lists
  int32_t bound[8];       // class c takes blocks with bound[c-1] < m_size <= bound[c]
  int32_t forced;         // >= 0: every non-empty block goes to this class
  int32_t n_live;         // classes >= n_live are not launched; their blocks go to class n_live - 1
};

// The smallest launched class whose bound holds the block; the largest launched class takes
// every block past the bounds (the tile kernels loop over row sub-tiles, so any block fits).
// Unrolled over the eight slots so that every bound is read at a constant offset (a loop
// indexing the argument struct at run time reads it from memory on every step).
__device__ __forceinline__ int pick_class(const ClassPolicy& pol, int m_size) {
  if (pol.forced >= 0) return pol.forced;
  int c = pol.n_live - 1;
#pragma unroll
  for (int k = 7; k >= 0; --k)
    if (k < pol.n_live - 1 && m_size <= pol.bound[k]) c = k;
  return c;
}

// Routed-block description shared by every MoE stage kernel.
struct BlockRouting {
  const int32_t* sorted_ids;  // [max_blocks * block_m]
  const int32_t* expert_ids;  // [max_blocks]
  const int32_t* offsets;     // [max_blocks + 1]
  const int32_t* work_desc;   // this tile class's blocks, 4 ints each: block id, expert, first
                              // compact row, row count (entries past work_count are stale)
  const int32_t* work_count;  // device scalar: number of valid entries
  int32_t block_m;
  int32_t topk;
  // Self-routed small routings (ring-fed tiles only): with route_ids set, each workgroup finds
  // its block from the routing itself -- the sort's expert order, each expert's rows cut into
  // blocks of block_m, each block's class from route_pol -- and no sort kernel runs.
  const int32_t* route_ids;   // [route_R] expert of each flat routed row (ids outside [0, E) drop)
  int32_t route_R, route_E;
  ClassPolicy route_pol;
};

struct GemmArgs {
  // activations
  const void* A;        // bf16 or e4m3 rows
  int64_t lda;          // elements (bf16) or bytes (e4m3)
  int32_t a_silu;       // tiny-block kernel: A rows are [gate | up] pairs of width K; the kernel
                        // stages bf16(silu(gate) * up) (the SiLU-and-mul fused into stage 2)
  const float* sa;      // e4m3 activations: [rows, K/128] fp32
  int64_t lds;          // row stride of sa (elements)
  // weights (per expert: base + e * w_estride)
  const uint8_t* W;
  int64_t ldw;          // bytes per weight row
  int64_t w_estride;    // bytes per expert
  int32_t w_tiled;      // routed weights (and MX scales) in the tiled layout of prepack.hip
  const void* ws;       // fp32 block grid | fp32 scalar | e8m0 [N, K/32] bytes
  int64_t ws_s0, ws_s1; // grid strides (elements); for e8m0: row stride (bytes)
  int64_t ws_estride;   // per expert (elements or bytes)
  int32_t block_n;      // 1 or 128 for W_E4M3_BLOCK
  // bias (optional)
  const void* bias;
  int32_t bias_bf16;    // 1: bf16 bias, 0: fp32 bias
  int64_t bias_estride; // elements per expert
  // output
  void* out;
  int64_t ldo;          // elements
  int64_t M, N, K;
  BlockRouting rt;
  // batched dense products (launch_gemm_w16_batched): entry z reads A + z * a_bstride
  // (elements), W + z * w_estride, ws + z * ws_estride, bias + z * bias_estride and writes
  // out + z * o_bstride (elements)
  int64_t a_bstride, o_bstride;
  // K split (routed bf16-activation stages): k_split > 1 runs every tile over K chunks of
  // k_chunk elements (a multiple of 256), chunk c writing its fp32 partial sums to
  // out + c * split_stride (the bias rides on chunk 0); 0 or 1: whole K, one output
  int32_t k_split;
  int64_t k_chunk;
  int64_t split_stride;
  // Stage 1 on the ring-fed tiles with the SiLU-and-mul in the epilogue (N = 2 I, I % 64 == 0,
  // whole K): column tile nt pairs gate rows [64 nt, +64) with up rows [I + 64 nt, +64) and
  // writes bf16(silu(gate) * up) of the bf16-rounded stage-1 values to out [rows, ldo = I]
  int32_t silu_pair;
  // Self-routed stage 2 with top-1 routing and whole K ranges: the top-k combine folds into the
  // epilogue -- out (bf16 [M, ldo]) row t = bf16(top1_w[t] * y[t]), and the rows of tokens
  // whose id lies outside [0, E) are written as zeros
  const float* top1_w;
};

// MX-scaled dense GEMM (gemm_mx.hip): MXFP8 activations x MXFP8 / MXFP4 weights.
enum MxWFmt : int { MX_W_E4M3 = 0, MX_W_E2M1 = 1 };
struct MxArgs {
  const void* A;       // e4m3 [M, K], row stride lda bytes
  int64_t lda;
  const void* sa;      // e8m0 [M, K/32], row stride lds_bytes
  int64_t lds_bytes;
  const void* W;       // e4m3 [N, K] or packed e2m1 [N, K/2], row stride ldw bytes
  int64_t ldw;
  const void* sw;      // e8m0 [N, K/32], row stride ldws_bytes
  int64_t ldws_bytes;
  int32_t w_fmt;       // MxWFmt
  const void* bias;    // NULL or [N] fp32 / bf16
  int32_t bias_bf16;
  void* out;           // bf16 [M, N], row stride ldo elements
  int64_t ldo;
  int64_t M, N, K;     // K % 128 == 0
  // K split: k_split > 1 chunks of k_chunk elements (a multiple of 128), chunk c (blockIdx.y)
  // writing fp32 partial sums to out + c * split_stride floats (row stride ldo); the bias rides
  // on chunk 0
  int32_t k_split;
  int64_t k_chunk, split_stride;
};
void launch_gemm_mx(const MxArgs& a, hipStream_t stream);
// bf16 [M, K] (row stride ldx) -> e4m3 [M, K] (contiguous) + e8m0 [M, K/32] (contiguous)
void launch_quant_mx(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, uint8_t* s,
                     hipStream_t stream);

// ---------------------------------------------------------------- launchers

void launch_quant_1x128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                        float* s, hipStream_t stream);

// W8A8: e4m3 activations with 1x128 scales x e4m3 block-scaled weights (MFMA 16x16x128).
// tile: 0 = 128x128, 1 = 64x128, 2 = 32x128, 3 = 16x128.  `grid_blocks` is the number of
// row tiles (dense) or the work-list capacity (routed); out_f32 selects an fp32 output.
void launch_gemm_w8a8(const GemmArgs& a, int row_mode, int tile, bool out_f32, int64_t grid_blocks,
                      hipStream_t stream);

// W8A8 with large direct-to-LDS tiles; 128x128 weight blocks (1x128 too for the dense GEMM); K <= 16384; operand offsets
// below 4 GiB.  Dense shape: 0 = 256x256, 1 = 128x256, 2 = 128x128 tiles; routed modes use
// 128x256 and read plain or tiled weights.  `grid_blocks` = row tiles (dense) or work-list capacity.
void launch_gemm_w8a8_big(const GemmArgs& a, int row_mode, int shape, bool out_f32, int64_t grid_blocks,
                          hipStream_t stream);
int big_tile_rows(int shape);

// W8A16 / W4A16: bf16 activations x decoded e4m3 / e2m1 weights (MFMA 16x16x32 bf16).
void launch_gemm_w16(const GemmArgs& a, int wfmt, int row_mode, int tile, bool out_f32, int64_t grid_blocks,
                     hipStream_t stream);

// Routed W8A16 / W4A16 tile classes of 16, 32, 64 and 128 rows (cls[c]: the stage's arguments
// with class c + 1's work list; grid_blocks[c]: its capacity, 0 for none) in one launch.
// Batched dense W8A16 products with per-tensor e4m3 weights: `batch` independent entries
// (grid.y), each exactly the product launch_gemm_w16 computes for W_E4M3_TENSOR / ROWS_DENSE.
void launch_gemm_w16_batched(const GemmArgs& a, int tile, int64_t batch, hipStream_t stream);

void launch_gemm_w16_grouped(const GemmArgs cls[4], const int64_t grid_blocks[4], int wfmt, int row_mode,
                             bool out_f32, hipStream_t stream);
// The same classes on tiles fed by a ring of LDS stages (direct global-to-LDS copies); usable
// when w16_ring_supported(stage arguments, wfmt): block-FP8 (128 x 128 blocks) or MXFP4 weights,
// K % 32 == 0, K <= 16384, 16-byte aligned operand rows (plain MXFP4: K % 128 == 0).
bool w16_ring_supported(const GemmArgs& a, int wfmt);
// The part of that test that does not depend on the weight layout (the class policy uses it, so
// that both layouts run the same classes and give the same bits).
bool w16_ring_shape_ok(const GemmArgs& a, int wfmt);
void launch_gemm_w16_ring(const GemmArgs cls[4], const int64_t grid_blocks[4], int wfmt, int row_mode,
                          bool out_f32, hipStream_t stream);
// The same tiles on dense per-tensor W8A16 products (bf16 out, batch entries on grid.y as in
// launch_gemm_w16_batched; tile 0..3 = 128, 64, 32, 16 rows).  Supported: K % 32 == 0,
// 16-byte aligned A / W / out rows (and batch strides), plain weights.
bool w16_ring_dense_supported(const GemmArgs& a, int64_t batch);
void launch_gemm_w16_ring_dense(const GemmArgs& a, int tile, int64_t batch, hipStream_t stream);
// The same tiles self-routed (g.rt.route_ids set): one workgroup per (block, column tile, K
// chunk) over max_blocks blocks; live[i]: tile class i (16, 32, 64, 128 rows) can occur.
void launch_gemm_w16_ring_routed(const GemmArgs& g, int64_t max_blocks, const bool live[4], int wfmt, int row_mode,
                                 bool out_f32, hipStream_t stream);

// Wavefront-reduction GEMV for routed blocks of at most 4 rows.
// a_e4m3: activations are e4m3 + 1x128 scales (W8A8), else bf16.
void launch_gemv(const GemmArgs& a, int wfmt, bool a_e4m3, int row_mode, bool out_f32, int64_t grid_blocks,
                 hipStream_t stream);

// Weight-streaming MFMA kernel for routed blocks of at most 4 rows (more rows are processed
// 4 at a time); routed row modes only.
// Dense rows on the weight-streaming kernel (e4m3 activations with 1x128 scales, or bf16
// activations; plain e4m3 weights with 128 x 128 block scales -- a per-tensor scale is the grid
// with strides 0 -- K a multiple of 128, N * K < 2^32): tiles of `ar` (4 or 8) rows, 64 or 128
// columns (skinny_dense_col_tiles per row tile), K split by a.k_split / a.k_chunk (fp32 partial
// slices when split, out_f32 then true), each workgroup staging only its K range in LDS
// (skinny_dense_lds bytes for kstage staged elements, 0 = all of K); launch_dense_split_sum adds
// the slices in chunk order into bf16.
// swcol: per-column (1 x 128) weight scales, e4m3 activations only.
size_t skinny_dense_lds(int64_t N, int64_t K, int ar, int64_t kstage, bool a_e4m3, bool swcol = false);
int64_t skinny_dense_col_tiles(int64_t N);
void launch_skinny_dense(const GemmArgs& a, int ar, bool a_e4m3, bool out_f32, hipStream_t stream,
                         bool swcol = false);
void launch_dense_split_sum(const float* part, int32_t S, int64_t M, int64_t N, uint16_t* out, int64_t ldo,
                            hipStream_t stream);
void launch_skinny(const GemmArgs& a, int wfmt, bool a_e4m3, int row_mode, bool out_f32, int64_t grid_blocks,
                   hipStream_t stream);
// Dynamic LDS the weight-streaming kernel takes for reduction length K.
size_t skinny_lds_bytes(int wfmt, bool a_e4m3, int64_t K);

// Persistent expert-streaming kernel for routings made only of tiny expert blocks (bf16
// activations, e2m1 or e4m3 weights): each workgroup groups the routed rows by expert itself
// (no sorted block tables) and rows are indexed by flat routed id.  Stage 1 reads x rows
// (flat id / topk), takes N = 2 I weight rows (gate then up, I % 16 == 0) and writes
// h = bf16(silu(gate + b) * (up + b)) as [R, I] bf16 (b: fp32 bias, optional); stage 2 reads h
// rows and writes [R, N] fp32.
struct EsRoute {
  const int32_t* ids;  // [R] expert of each flat routed row; ids outside [0, E) are dropped
  int32_t R, E, topk;
};
void launch_expert_stream(const GemmArgs& a, int wfmt, int stage, const EsRoute& rt, hipStream_t stream);
// Dynamic LDS of one workgroup of that kernel (N: weight rows of the stage, K: reduction length).
size_t expert_stream_lds_bytes(int wfmt, int stage, int64_t N, int64_t K, int64_t E, int64_t R);

// Load-time relayout into the tiled layout (see prepack.hip).
int64_t tiled_steps(int64_t row_bytes);
int64_t tiled_scale_steps(int64_t groups);
void launch_prepack_w(const uint8_t* w, int64_t E, int64_t N, int64_t row_bytes, uint8_t* out, hipStream_t stream);
void launch_prepack_s(const uint8_t* s, int64_t E, int64_t N, int64_t groups, uint8_t* out, hipStream_t stream);

// Expert sort / block alignment.  Optionally also fills per-class work lists using the
// per-block selector: class c's i-th block descriptor is the int4 at
// class_lists + (c * list_stride + i) * 4 (block id, expert, first compact row, row
// count), and class_counts[c] holds the number of entries.
// `scratch` (NULL, or align_multi_scratch_ints(R, E) ints): with more than kAlignMultiMinRows
// routed rows and no pad slots to write, the sort runs over many workgroups (a histogram pass,
// the tables in one workgroup, a scatter pass) and keeps its per-chunk counts there.
constexpr int64_t kAlignMultiMinRows = 4096;
int64_t align_multi_scratch_ints(int64_t R, int32_t E);
void launch_moe_align(const int32_t* topk_ids, int64_t M, int32_t topk, int32_t E, int32_t block_m,
                      int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets, int32_t* num_blocks,
                      int64_t max_blocks, const ClassPolicy& pol, int32_t* class_lists, int64_t list_stride,
                      int32_t* class_counts, bool write_pads, int32_t* scratch, hipStream_t stream);

// ic1 = bf16(silu(gate) * up) over compact rows; optionally re-quantised 1x128 to e4m3.
// ic0 rows are `ld_in` elements apart; ic1 / q / s are contiguous.
void launch_silu_mul(const uint16_t* ic0, int64_t rows, int64_t inter, int64_t ld_in, uint16_t* ic1_bf16,
                     uint8_t* ic1_q, float* ic1_s, hipStream_t stream);

// Split stage 1: ic0 = bf16(sum over the n_split fp32 partial slices [rows, 2I], slice c at
// part + c * slice), then ic1 = bf16(silu(gate) * up) as launch_silu_mul.
void launch_split_silu_mul(const float* part, int32_t n_split, int64_t slice, int64_t rows, int64_t inter,
                           uint16_t* ic1_bf16, hipStream_t stream);

// out[t] = bf16(sum_k w[t,k] * y[t*topk+k]), y[r] = sum over the n_split slices y + c * slice
// (n_split 1: y itself).  Rows whose expert id lies outside [0, E) are skipped.
void launch_combine(const float* y, int32_t n_split, int64_t slice, const float* topk_weights,
                    const int32_t* topk_ids, int32_t E, int64_t M, int32_t topk, int64_t H, uint16_t* out,
                    hipStream_t stream);

}  // namespace mxq
