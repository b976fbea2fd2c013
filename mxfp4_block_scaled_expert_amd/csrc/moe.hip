// Routed-MoE support kernels: expert sort / block alignment with the per-block
// tile-class selector, SiLU-and-mul (with the W8A8 1x128 re-quantisation) and
// the top-k weighted combine.
//
// Alignment ("vLLM PR 50949 review", moe_fp8.cpp listing, and implementation
// items 2-3): the fused expert kernels walk blocks of at most BLOCK_M rows of
// one expert; expert_ids[mb], offsets[mb] (compact row prefix; the block holds
// offsets[mb+1] - offsets[mb] rows and an empty block is skipped) and
// sorted_ids[mb * BLOCK_M + m] (flat routed id t * topk + k) describe them.
// The layout produced here: experts in ascending id, rows of one expert in
// ascending flat id (a stable counting sort), pad value R in unused slots,
// trailing blocks with expert -1 and offset R.  The whole sort runs in one
// workgroup (256 or 1024 threads) with no host synchronisation.  Wave w owns a contiguous
// chunk of the routed rows and walks it 64 rows at a time, twice: first counting its rows per
// expert, then (after a prefix over the waves) placing them; ranks inside a 64-row step come
// from ballots over the bits of the expert id.  No barrier is needed inside a walk and the
// order is deterministic.
//
// The per-block selector (implementation items 1-2: the decision is taken per
// expert block from its real row count, not once per layer from an average)
// assigns every non-empty block to the smallest tile class whose row bound
// holds it and appends the block's descriptor (block id, expert, first compact
// row, row count) to that class's work list, so that a tile kernel learns all of
// it in one read.  Classes the host did not launch (their lower bound reaches the
// token count, which caps an expert's rows when a token's experts are distinct)
// receive nothing: a block past every launched bound goes to the largest
// launched class.
#include <algorithm>

#include "kernels.hpp"
#include "quant_common.hpp"

namespace mxq {

// Lanes of the wave holding the same valid expert id as this lane (ballots over the id's bits).
__device__ __forceinline__ uint64_t same_expert(int e, bool valid, int nbits) {
  uint64_t mask = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool set = valid && ((e >> bit) & 1);
    const uint64_t bm = __ballot(set);
    mask &= set ? bm : ~bm;
  }
  return mask;
}

// Routed rows per workgroup of the multi-workgroup sort (the histogram and scatter kernels).
constexpr int kAlignChunk = 256;

// One workgroup of T threads (1024 for large routings; 256 when the routing is small, where
// the kernel is a chain of barriers and fewer waves make each one cheaper).  MULTI: the middle
// of the multi-workgroup sort -- the per-expert counts come from the per-chunk histograms
// `hist` [G][E] (each chunk's first position within every expert goes to `base` [G][E]), the
// block tables and class lists are built as in the one-workgroup sort, the block starts go to
// `blk_out` [E + 1], and the scatter is left to align_scatter_kernel.
template <int T, bool MULTI>
__global__ __launch_bounds__(T) void moe_align_kernel(
    const int32_t* __restrict__ ids, int64_t R, int32_t E, int32_t block_m, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ offsets, int32_t* __restrict__ num_blocks,
    int64_t max_blocks, ClassPolicy pol, int32_t* __restrict__ class_lists, int64_t list_stride,
    int32_t* __restrict__ class_counts, int write_pads, int cache_ids, const int32_t* __restrict__ hist,
    int32_t G, int32_t* __restrict__ base, int32_t* __restrict__ blk_out) {
  constexpr int kAlignThreads = T;
  constexpr int kAlignWaves = T / 64;
  extern __shared__ int32_t smem[];
  int32_t* cnt = smem;                     // [E]
  int32_t* blk_start = cnt + E;            // [E + 1]
  int32_t* row_start = blk_start + E + 1;  // [E + 1]
  int32_t* wave_cnt = row_start + E + 1;   // [T / 64][E]: a wave's rows per expert, then its base
  int32_t* s_ids = wave_cnt + (T / 64) * E; // [R] when cache_ids: the ids, read once from memory
  __shared__ int32_t cls_cnt[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* my_cnt = wave_cnt + wave * E;
  for (int e = lane; e < E; e += 64) my_cnt[e] = 0;
  if (tid < 8) cls_cnt[tid] = 0;

  // rows of wave w: [w * chunk, min(R, (w + 1) * chunk)), chunk a multiple of 64
  const int64_t chunk = ((R + kAlignWaves - 1) / kAlignWaves + 63) / 64 * 64;
  const int64_t r_lo = min<int64_t>(R, int64_t(wave) * chunk), r_hi = min<int64_t>(R, r_lo + chunk);
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  if (MULTI) {
    // 1'. per expert: total rows, and each chunk's first position among them
    for (int e = tid; e < E; e += kAlignThreads) {
      // the chunk counts are read 32 at a time (one memory round trip per batch)
      constexpr int kBatch = 32;
      int acc = 0;
      for (int g0 = 0; g0 < G; g0 += kBatch) {
        int h[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) h[j] = g0 + j < G ? hist[int64_t(g0 + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (g0 + j < G) base[int64_t(g0 + j) * E + e] = acc;
          acc += h[j];
        }
      }
      cnt[e] = acc;
    }
    __syncthreads();
  } else {
  // 1. per-wave histogram of the chunk (expert ids outside [0, E) are ignored); the ids are read
  // 8 steps at a time and, when they fit, kept in LDS for the second walk
  constexpr int kIdBatch = 8;
  for (int64_t r0 = r_lo; r0 < r_hi; r0 += 64 * kIdBatch) {
    int eb[kIdBatch];
#pragma unroll
    for (int j = 0; j < kIdBatch; ++j) eb[j] = ids[min<int64_t>(r0 + 64 * j + lane, R - 1)];
#pragma unroll
    for (int j = 0; j < kIdBatch; ++j) {
      const int64_t r = r0 + 64 * j + lane;
      if (r0 + 64 * j >= r_hi) break;  // wave-uniform
      const int e = r < r_hi ? eb[j] : -1;
      if (cache_ids && r < r_hi) s_ids[r] = e;
      const bool valid = e >= 0 && e < E;
      const uint64_t mask = same_expert(e, valid, nbits);
      if (valid && __popcll(mask & lt) == 0) my_cnt[e] += __popcll(mask);
    }
  }
  __syncthreads();
  // per expert: total rows, and each wave's first position among them
  for (int e = tid; e < E; e += kAlignThreads) {
    int acc = 0;
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = wave_cnt[w * E + e];
      wave_cnt[w * E + e] = acc;
      acc += c;
    }
    cnt[e] = acc;
  }
  __syncthreads();
  }  // MULTI

  // 2. exclusive scans of blocks and rows per expert (each thread owns a run of experts)
  const int per = int(cdiv(E, kAlignThreads));
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  {
    int nb = 0, nr = 0;
    for (int e = e0; e < e1; ++e) {
      nb += (cnt[e] + block_m - 1) / block_m;
      nr += cnt[e];
    }
    // wave-level inclusive scan of (nb, nr)
    int sb = nb, sr = nr;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int tb = __shfl_up(sb, o, 64), tr = __shfl_up(sr, o, 64);
      if (lane >= o) {
        sb += tb;
        sr += tr;
      }
    }
    __shared__ int32_t wsum_b[kAlignWaves], wsum_r[kAlignWaves];
    if (lane == 63) {
      wsum_b[wave] = sb;
      wsum_r[wave] = sr;
    }
    __syncthreads();
    int pb = 0, pr = 0;
    for (int w = 0; w < wave; ++w) {
      pb += wsum_b[w];
      pr += wsum_r[w];
    }
    int b = pb + sb - nb, rr = pr + sr - nr;  // exclusive prefix at e0
    for (int e = e0; e < e1; ++e) {
      blk_start[e] = b;
      row_start[e] = rr;
      b += (cnt[e] + block_m - 1) / block_m;
      rr += cnt[e];
    }
    if (tid == kAlignThreads - 1) {
      blk_start[E] = pb + sb;
      row_start[E] = pr + sr;
    }
  }
  __syncthreads();
  const int nblocks = blk_start[E];
  const int rows_total = row_start[E];
  if (tid == 0) *num_blocks = nblocks;

  // 3. block table and class lists.  A class list holds its blocks in expert order (a scan of
  // each thread's per-class block counts gives its run's first position in every list), so the
  // blocks of one expert sit side by side for the tile kernels.
  int pos[8];
  if (pol.n_classes > 0) {
    int my[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) my[c] = 0;
    for (int e = e0; e < e1; ++e)
      for (int b = 0; b * block_m < cnt[e]; ++b) {
        const int c = pick_class(pol, min(block_m, cnt[e] - b * block_m));
#pragma unroll
        for (int k = 0; k < 8; ++k) my[k] += (k == c) ? 1 : 0;
      }
    __shared__ int32_t wsum_c[kAlignWaves][8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      int sc = my[c];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(sc, o, 64);
        if (lane >= o) sc += t;
      }
      pos[c] = sc - my[c];  // exclusive, within the wave
      if (lane == 63) wsum_c[wave][c] = sc;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      int base = 0, total = 0;
      for (int w = 0; w < kAlignWaves; ++w) {
        base += w < wave ? wsum_c[w][c] : 0;
        total += wsum_c[w][c];
      }
      pos[c] += base;
      if (tid == 0) cls_cnt[c] = total;
    }
  }
  for (int e = e0; e < e1; ++e) {
    const int c_e = cnt[e];
    for (int b = 0; b * block_m < c_e; ++b) {
      const int mb = blk_start[e] + b;
      const int m_size = min(block_m, c_e - b * block_m);
      expert_ids[mb] = e;
      offsets[mb] = row_start[e] + b * block_m;
      if (pol.n_classes > 0) {
        const int c = pick_class(pol, m_size);
        int p = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k == c) p = pos[k]++;
        *reinterpret_cast<int4*>(class_lists + (int64_t(c) * list_stride + p) * 4) =
            make_int4(mb, e, row_start[e] + b * block_m, m_size);
      }
    }
  }
  for (int64_t mb = nblocks + tid; mb < max_blocks; mb += kAlignThreads) {
    expert_ids[mb] = -1;
    offsets[mb] = rows_total;
  }
  if (tid == 0) offsets[max_blocks] = rows_total;
  // pad slots (slots past a block's rows, and every slot of a trailing block) hold R; the
  // fused path never reads them and skips this
  if (write_pads) {
    for (int64_t idx = tid; idx < max_blocks * block_m; idx += kAlignThreads) {
      const int64_t mb = idx / block_m;
      const int i = int(idx - mb * block_m);
      bool pad = mb >= nblocks;
      if (!pad) {
        int lo = 0, hi = E;  // the expert e with blk_start[e] <= mb < blk_start[e + 1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (blk_start[mid] <= mb) lo = mid; else hi = mid;
        }
        pad = i >= cnt[lo] - int(mb - blk_start[lo]) * block_m;
      }
      if (pad) sorted_ids[idx] = int32_t(R);
    }
  }
  __syncthreads();
  if (pol.n_classes > 0 && tid < pol.n_classes) class_counts[tid] = cls_cnt[tid];
  if (MULTI) {
    for (int e = tid; e <= E; e += kAlignThreads) blk_out[e] = blk_start[e];
    return;
  }

  // 4. stable scatter: each wave walks its chunk again; a row's position within its expert is
  // the wave's base for that expert plus its rank among the wave's earlier rows of the expert
  for (int64_t r0 = r_lo; r0 < r_hi; r0 += 64) {
    const int64_t r = r0 + lane;
    const int e = r < r_hi ? (cache_ids ? s_ids[r] : ids[r]) : -1;
    const bool valid = e >= 0 && e < E;
    const uint64_t mask = same_expert(e, valid, nbits);
    const int rank = __popcll(mask & lt);
    int pos = 0;
    if (valid) pos = my_cnt[e] + rank;
    if (valid && rank == 0) my_cnt[e] += __popcll(mask);
    if (valid) {
      const int b = pos / block_m, slot = pos - b * block_m;
      sorted_ids[int64_t(blk_start[e] + b) * block_m + slot] = int32_t(r);
    }
  }
}

// Multi-workgroup sort, first pass: workgroup g counts the rows of chunk g per expert.
__global__ __launch_bounds__(256) void align_hist_kernel(const int32_t* __restrict__ ids, int64_t R, int32_t E,
                                                         int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];  // [E]
  const int64_t g = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int64_t r = g * kAlignChunk + threadIdx.x;
  if (r < R) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[g * E + e] = cnt[e];
}

// Multi-workgroup sort, last pass: workgroup g places the rows of chunk g.  A row's position
// within its expert is the chunk's base, plus the rows of that expert in the chunk's earlier
// waves, plus its rank among the wave's earlier rows of the expert (ballots): the same stable
// order as the one-workgroup sort.
__global__ __launch_bounds__(256) void align_scatter_kernel(const int32_t* __restrict__ ids, int64_t R, int32_t E,
                                                            int32_t block_m, const int32_t* __restrict__ base,
                                                            const int32_t* __restrict__ blk_start,
                                                            int32_t* __restrict__ sorted_ids) {
  extern __shared__ int32_t wcnt[];  // [4][E]: rows per expert of each wave, then their prefix
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t g = blockIdx.x;
  for (int i = tid; i < 4 * E; i += 256) wcnt[i] = 0;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t r = g * kAlignChunk + tid;
  const int e = r < R ? ids[r] : -1;
  const bool valid = e >= 0 && e < E;
  const uint64_t mask = same_expert(e, valid, nbits);
  const int rank = __popcll(mask & lt);
  __syncthreads();
  if (valid && rank == 0) wcnt[wave * E + e] = __popcll(mask);
  __syncthreads();
  if (valid) {
    int pos = base[g * E + e] + rank;
    for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
    const int b = pos / block_m, slot = pos - b * block_m;
    sorted_ids[int64_t(blk_start[e] + b) * block_m + slot] = int32_t(r);
  }
}

int64_t align_multi_scratch_ints(int64_t R, int32_t E) {
  if (R <= kAlignMultiMinRows) return 0;
  return 2 * cdiv(R, int64_t(kAlignChunk)) * E + E + 1;
}

void launch_moe_align(const int32_t* topk_ids, int64_t M, int32_t topk, int32_t E, int32_t block_m,
                      int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets, int32_t* num_blocks,
                      int64_t max_blocks, const ClassPolicy& pol, int32_t* class_lists, int64_t list_stride,
                      int32_t* class_counts, bool write_pads, int32_t* scratch, hipStream_t stream) {
  // cnt[E] + blk_start[E+1] + row_start[E+1] + wave_cnt[waves][E] (+ ids[R])
  const int64_t R = M * topk;
  const bool small = R <= 2048;  // one 64-row step per wave or a few
  const int waves = small ? 4 : 16;
  size_t smem = sizeof(int32_t) * (size_t(E) * 3 + 2 + size_t(waves) * E);
  // keep the ids in LDS for the scatter when they fit beside the tables (gfx950: 160 KB)
  const bool cache = smem + sizeof(int32_t) * size_t(R) <= size_t(152) * 1024;
  if (cache) smem += sizeof(int32_t) * size_t(R);
  if (scratch && !write_pads && R > kAlignMultiMinRows) {
    // many rows: count and place them over many workgroups (one workgroup walking every row
    // is bound by its own instruction issue); the tables in between stay in one workgroup
    const int32_t G = int32_t(cdiv(R, int64_t(kAlignChunk)));
    int32_t* hist = scratch;
    int32_t* base = hist + int64_t(G) * E;
    int32_t* blk = base + int64_t(G) * E;
    hipLaunchKernelGGL(align_hist_kernel, dim3(G), dim3(256), sizeof(int32_t) * E, stream, topk_ids, R, E, hist);
    // 256 threads: the tables are a chain of scans and barriers over E experts, which more
    // waves only make longer
    const size_t tsmem = sizeof(int32_t) * (size_t(E) * 3 + 2 + size_t(4) * E);
    hipLaunchKernelGGL((moe_align_kernel<256, true>), dim3(1), dim3(256), tsmem, stream, topk_ids, R, E, block_m,
                       sorted_ids, expert_ids, offsets, num_blocks, max_blocks, pol, class_lists, list_stride,
                       class_counts, 0, 0, hist, G, base, blk);
    hipLaunchKernelGGL(align_scatter_kernel, dim3(G), dim3(256), sizeof(int32_t) * 4 * E, stream, topk_ids, R, E,
                       block_m, base, blk, sorted_ids);
    return;
  }
  if (small)
    hipLaunchKernelGGL((moe_align_kernel<256, false>), dim3(1), dim3(256), smem, stream, topk_ids, R, E, block_m,
                       sorted_ids, expert_ids, offsets, num_blocks, max_blocks, pol, class_lists, list_stride,
                       class_counts, write_pads ? 1 : 0, cache ? 1 : 0, nullptr, 0, nullptr, nullptr);
  else
    hipLaunchKernelGGL((moe_align_kernel<1024, false>), dim3(1), dim3(1024), smem, stream, topk_ids, R, E, block_m,
                       sorted_ids, expert_ids, offsets, num_blocks, max_blocks, pol, class_lists, list_stride,
                       class_counts, write_pads ? 1 : 0, cache ? 1 : 0, nullptr, 0, nullptr, nullptr);
}

// ---------------------------------------------------------------- SiLU-and-mul

// ic0 [rows, 2I] bf16 (gate = columns [0, I), up = [I, 2I)).  16 lanes cover
// 128 output columns (8 each).  bf16 output: ic1 [rows, I]; W8A8: the bf16
// products are re-quantised per 128 columns into q [rows, I] + s [rows, I/128].
template <bool QUANT>
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ ic0, int64_t rows, int64_t inter,
                                                       int64_t ld_in, uint16_t* __restrict__ ic1,
                                                       uint8_t* __restrict__ q, float* __restrict__ s) {
  const int64_t per_row = inter / 8;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool valid = idx < rows * per_row;
  const int64_t ii = valid ? idx : 0;
  const int64_t row = ii / per_row;
  const int64_t col = (ii - row * per_row) * 8;
  uint4 g = make_uint4(0, 0, 0, 0), u = make_uint4(0, 0, 0, 0);
  if (valid) {
    g = *reinterpret_cast<const uint4*>(ic0 + row * ld_in + col);
    u = *reinterpret_cast<const uint4*>(ic0 + row * ld_in + inter + col);
  }
  const uint4 h = silu_mul8(g, u);
  if (!QUANT) {
    if (valid) *reinterpret_cast<uint4*>(ic1 + row * inter + col) = h;
  } else {
    const float amax = group16_max(amax8_bf16(h));
    if (valid) {
      uint2 qv;
      const float sc = quant8_e4m3(h, amax, qv);
      *reinterpret_cast<uint2*>(q + row * inter + col) = qv;
      if ((threadIdx.x & 15) == 0) s[row * (inter >> 7) + (col >> 7)] = sc;
    }
  }
}

// Split stage 1: the n_split fp32 partial slices of ic0 are summed (slice order), rounded to
// bf16 (the ic0 value) and passed through the same SiLU-and-mul as silu_mul_kernel.
__global__ __launch_bounds__(256) void split_silu_mul_kernel(const float* __restrict__ part, int32_t n_split,
                                                             int64_t slice, int64_t rows, int64_t inter,
                                                             uint16_t* __restrict__ ic1) {
  const int64_t per_row = inter / 8;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= rows * per_row) return;
  const int64_t row = idx / per_row;
  const int64_t col = (idx - row * per_row) * 8;
  const float* pg = part + row * 2 * inter + col;
  float g[8], u[8];
  {
    const float4 g0 = *reinterpret_cast<const float4*>(pg), g1 = *reinterpret_cast<const float4*>(pg + 4);
    const float4 u0 = *reinterpret_cast<const float4*>(pg + inter), u1 = *reinterpret_cast<const float4*>(pg + inter + 4);
    g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    u[0] = u0.x; u[1] = u0.y; u[2] = u0.z; u[3] = u0.w; u[4] = u1.x; u[5] = u1.y; u[6] = u1.z; u[7] = u1.w;
  }
  for (int c = 1; c < n_split; ++c) {
    const float* p = pg + c * slice;
    const float4 g0 = *reinterpret_cast<const float4*>(p), g1 = *reinterpret_cast<const float4*>(p + 4);
    const float4 u0 = *reinterpret_cast<const float4*>(p + inter), u1 = *reinterpret_cast<const float4*>(p + inter + 4);
    g[0] += g0.x; g[1] += g0.y; g[2] += g0.z; g[3] += g0.w; g[4] += g1.x; g[5] += g1.y; g[6] += g1.z; g[7] += g1.w;
    u[0] += u0.x; u[1] += u0.y; u[2] += u0.z; u[3] += u0.w; u[4] += u1.x; u[5] += u1.y; u[6] += u1.z; u[7] += u1.w;
  }
  const uint4 gb = make_uint4(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                              pack_bf16x2(g[6], g[7]));
  const uint4 ub = make_uint4(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]), pack_bf16x2(u[4], u[5]),
                              pack_bf16x2(u[6], u[7]));
  *reinterpret_cast<uint4*>(ic1 + row * inter + col) = silu_mul8(gb, ub);
}

void launch_split_silu_mul(const float* part, int32_t n_split, int64_t slice, int64_t rows, int64_t inter,
                           uint16_t* ic1_bf16, hipStream_t stream) {
  const int64_t threads = rows * (inter / 8);
  if (threads == 0) return;
  hipLaunchKernelGGL(split_silu_mul_kernel, dim3(unsigned(cdiv(threads, 256))), dim3(256), 0, stream, part, n_split,
                     slice, rows, inter, ic1_bf16);
}

void launch_silu_mul(const uint16_t* ic0, int64_t rows, int64_t inter, int64_t ld_in, uint16_t* ic1_bf16,
                     uint8_t* ic1_q, float* ic1_s, hipStream_t stream) {
  const int64_t threads = rows * (inter / 8);
  if (threads == 0) return;
  const unsigned grid = unsigned(cdiv(threads, 256));
  if (ic1_q)
    hipLaunchKernelGGL(silu_mul_kernel<true>, dim3(grid), dim3(256), 0, stream, ic0, rows, inter, ld_in, ic1_bf16,
                       ic1_q, ic1_s);
  else
    hipLaunchKernelGGL(silu_mul_kernel<false>, dim3(grid), dim3(256), 0, stream, ic0, rows, inter, ld_in, ic1_bf16,
                       ic1_q, ic1_s);
}

// ---------------------------------------------------------------- combine

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int32_t n_split, int64_t slice,
                                                      const float* __restrict__ w, const int32_t* __restrict__ ids,
                                                      int32_t E, int64_t M, int32_t topk, int64_t H,
                                                      uint16_t* __restrict__ out) {
  constexpr int kBatch = 8;  // routed rows whose loads go out together
  const int64_t per_row = H / 4;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= M * per_row) return;
  const int64_t t = idx / per_row;
  const int64_t col = (idx - t * per_row) * 4;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int k0 = 0; k0 < topk; k0 += kBatch) {
    // routing ids and weights of the batch first, then every y read, then the sums (k ascending):
    // two memory round trips per batch instead of two per routed row
    float wk[kBatch];
    int64_t rk[kBatch];
    bool ok[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int k = min(k0 + j, topk - 1);
      const int64_t r = t * topk + k;
      const int e = ids[r];
      ok[j] = k0 + j < topk && e >= 0 && e < E;
      wk[j] = w[r];
      rk[j] = r;
    }
    // non-temporal: y is read once (4096 tokens top-8 over 256 experts, H = 7168: 3.41 -> 3.39 ms)
    float4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + rk[j] * H + col));
      v[j] = make_float4(t[0], t[1], t[2], t[3]);
    }
    // K-split partial slices of y, summed in slice order
    for (int c = 1; c < n_split; ++c) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float4 p = *reinterpret_cast<const float4*>(y + c * slice + rk[j] * H + col);
        v[j].x += p.x;
        v[j].y += p.y;
        v[j].z += p.z;
        v[j].w += p.w;
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (!ok[j]) continue;  // past top-k, or an id outside [0, E) (its y row is never written)
      a0 = fmaf(wk[j], v[j].x, a0);
      a1 = fmaf(wk[j], v[j].y, a1);
      a2 = fmaf(wk[j], v[j].z, a2);
      a3 = fmaf(wk[j], v[j].w, a3);
    }
  }
  uint2 o;
  o.x = pack_bf16x2(a0, a1);
  o.y = pack_bf16x2(a2, a3);
  *reinterpret_cast<uint2*>(out + t * H + col) = o;
}

void launch_combine(const float* y, int32_t n_split, int64_t slice, const float* topk_weights,
                    const int32_t* topk_ids, int32_t E, int64_t M, int32_t topk, int64_t H, uint16_t* out,
                    hipStream_t stream) {
  const int64_t threads = M * (H / 4);
  if (threads == 0) return;
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned(cdiv(threads, 256))), dim3(256), 0, stream, y,
                     std::max<int32_t>(n_split, 1), slice, topk_weights, topk_ids, E, M, topk, H, out);
}

}  // namespace mxq
