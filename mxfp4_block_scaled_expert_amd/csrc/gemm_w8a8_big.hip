// Large-tile block-scaled W8A8 GEMM for gfx950: 256 x 256 output tile per
// 512-thread workgroup (8 waves, 2 per SIMD), K step 128 = one weight-scale
// block = one V_MFMA_F32_16X16X128_F8F6F4 per 16 x 16 sub-tile.
//
// Arithmetic ("SGLang PR 35605 review", implementation item 1 and the
// fp8_utils.py listing): out[m, n] = sum_kb sa[m, kb] * sw[n/128, kb] *
// sum_{k in kb} qa[m, k] * w[n, k] (+ bias), fp32 accumulation, bf16 (or fp32)
// output.  Each K block's partial product is formed on the matrix core from
// zero and promoted into the fp32 accumulator with one FMA by sa * sw.
//
// gfx950 specifics:
//  * operands go global -> LDS with GLOBAL_LOAD_LDS_DWORDX4 (no VGPR staging):
//    one instruction moves 64 x 16 bytes = 8 rows of a 128-byte K slice; the
//    16-byte chunk c of row r is stored at chunk position c ^ swz(r), which
//    keeps the 32-byte fragment reads free of bank conflicts;
//  * two LDS stages (2 x 64 KB of the 160 KB) and one barrier per K block: the
//    loads of block kb+1 are in flight while block kb is multiplied;
//  * the MFMA A operand is the weight tile and the B operand the activation
//    tile, so each lane ends up owning four consecutive output columns of one
//    row: one activation scale per lane per sub-tile and 8-byte (bf16) or
//    16-byte (fp32) stores;
//  * waves are laid out 2 (rows) x 4 (columns); a wave owns 128 x 64 outputs,
//    so its 64 weight rows sit inside one 128-wide scale block (one scalar
//    weight scale per wave per K block);
//  * dense tiles are rastered so that the tiles resident on one XCD (the
//    dispatcher deals workgroups round-robin over the 8 XCDs) share operands in
//    that XCD's L2.
#include "tile_rows.hpp"

namespace mxq {

namespace {

constexpr int kBM = 256, kBN = 256, kKS = 128;
constexpr int kThreads = 512;
constexpr int kMaxKB = 128;  // K <= 16384 on this kernel

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)(const_cast<void*>(p))));
}

// GLOBAL_LOAD_LDS (each lane's `size` bytes land at M0 + lane * size).  Issued
// as inline asm so the compiler does not treat the loads of the next K block
// as a hazard for the LDS reads of the current one (it cannot tell the two
// stages apart and would wait for the DMA before every fragment read); the
// kernel waits on vmcnt itself before each barrier.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}

// 32-byte fragment of row `row` (K chunks 2q, 2q+1) from a swizzled tile.
__device__ __forceinline__ i32x8 read_frag(const uint8_t* tile, int row, int q) {
  const int s = swz(row);
  const uint8_t* base = tile + row * kKS;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + (((2 * q) ^ s) << 4));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + (((2 * q + 1) ^ s) << 4));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

}  // namespace

template <int MODE, bool OUT_F32, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads) void gemm_w8a8_big_kernel(GemmArgs a, int64_t grid_blocks, int64_t n_tiles) {
  __shared__ __align__(1024) uint8_t sA0[kBM * kKS];
  __shared__ __align__(1024) uint8_t sA1[kBM * kKS];
  __shared__ __align__(1024) uint8_t sB0[kBN * kKS];
  __shared__ __align__(1024) uint8_t sB1[kBN * kKS];
  __shared__ __align__(16) float sS0[kBM];
  __shared__ __align__(16) float sS1[kBM];
  __shared__ int64_t sArow[kBM];
  __shared__ int64_t sOrow[kBM];
  __shared__ float sSW[2][kMaxKB];
  __shared__ __align__(256) float sPF[kThreads];  // landing area of the L2 prefetch (never read)  // weight scales of the tile's two 128-wide column blocks, all K blocks

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int l16 = lane & 15, q = lane >> 4;

  // ---- which tile
  int64_t tile, nt;
  if (MODE == ROWS_DENSE) {
    // XCD-aware raster: workgroup b runs on XCD b % 8; consecutive tile ids go to one XCD,
    // and tile ids walk 4 row tiles for each column tile.
    const int64_t total = grid_blocks * n_tiles;
    const int64_t per_xcd = cdiv(total, 8);
    const int64_t t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= total) return;
    const int64_t gm = min<int64_t>(4, grid_blocks);
    const int64_t band = t / (gm * n_tiles);
    const int64_t band_rows = min<int64_t>(gm, grid_blocks - band * gm);
    const int64_t in_band = t - band * gm * n_tiles;
    tile = band * gm + in_band % band_rows;
    nt = in_band / band_rows;
  } else {
    tile = blockIdx.x % grid_blocks;
    nt = blockIdx.x / grid_blocks;
  }
  const int64_t n0 = nt * kBN;
  if (n0 >= a.N) return;

  TileInfo t;
  if (!tile_info<kBM, MODE>(a, tile, t)) return;
  const int64_t expert = t.expert;
  const uint8_t* A = reinterpret_cast<const uint8_t*>(a.A);
  const uint8_t* Wb = a.W + expert * a.w_estride;
  const float* swb = reinterpret_cast<const float*>(a.ws) + expert * a.ws_estride;
  const int KB = int(a.K >> 7);
  // The weight scales the tile needs are staged in LDS once: every K block then reads
  // its scale with a DS load, so no vector-memory load (and no vmcnt wait) sits in
  // the K loop besides the operand DMA.
  for (int i = tid; i < 2 * KB; i += kThreads) {
    const int blk = i / KB, kb = i - blk * KB;
    const int64_t nb = min<int64_t>((n0 >> 7) + blk, cdiv(a.N, 128) - 1);
    sSW[blk][kb] = swb[nb * a.ws_s0 + kb * a.ws_s1];
  }
  const int sw_blk = wn >> 1;  // waves 0-1 cover the first 128 columns, 2-3 the second
  const bool vec_store = (a.ldo & 3) == 0;   // 16-byte fp32 stores
  const bool vec8_store = (a.ldo & 7) == 0;  // 16-byte bf16 stores

  for (int m_base = 0; m_base < t.m_total; m_base += kBM) {
    const int m_size = min(kBM, t.m_total - m_base);
    __syncthreads();
    fill_rows<kBM, MODE>(a, t, m_base, sArow, sOrow);
    __syncthreads();

    // ---- per-lane DMA sources: 4 x 1 KB blocks of A and of W per wave per K block
    // (32-bit byte offsets: the host only routes operands below 4 GiB here)
    uint32_t oa[4], ob[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = (wave * 4 + b) * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ swz(row);
      oa[b] = uint32_t(sArow[row] * a.lda + chunk * 16);
      const int64_t n = min<int64_t>(n0 + row, a.N - 1);
      ob[b] = uint32_t(n * a.ldw + chunk * 16);
    }
    const float* gs = a.sa + sArow[(wave & 3) * 64 + lane] * a.lds;

    auto issue = [&](int kb, uint8_t* dA, uint8_t* dB, float* dS) __attribute__((always_inline)) {
      const uint8_t* Ak = A + kb * kKS;
      const uint8_t* Wk = Wb + kb * kKS;
      const uint32_t la = __builtin_amdgcn_readfirstlane(lds_addr(dA) + wave * 4096);
      const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(dB) + wave * 4096);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        lds_dma16(Ak + oa[b], la + b * 1024);
        lds_dma16(Wk + ob[b], lb + b * 1024);
      }
      if (wave < 4) lds_dma4(gs + kb, __builtin_amdgcn_readfirstlane(lds_addr(dS) + wave * 256));
    };
    // Warm L2 with the K block after the one being DMA'd: one dword of every 128-byte
    // operand line (threads 0-255 the activation rows, 256-511 the weight rows).  With
    // only two LDS stages this is what lets the next DMA find its lines in L2.
    const uint8_t* pf_base = (tid < 256) ? A + sArow[tid] * a.lda
                                         : Wb + min<int64_t>(n0 + (tid - 256), a.N - 1) * a.ldw;
    const uint32_t pf_lds = __builtin_amdgcn_readfirstlane(lds_addr(sPF) + wave * 256);
    auto prefetch = [&](int kb) __attribute__((always_inline)) {
      lds_dma4(pf_base + kb * kKS, pf_lds);
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One K block: hold the wave's 4 weight fragments and stream the 8 activation
    // fragments.  Software-pipelined: the MFMAs of sub-tile row i+1 are interleaved with
    // the promotion FMAs of row i (whose partials finished during row i+1's issue), so a
    // single wave keeps its matrix core busy instead of waiting on its own results.
    auto compute = [&](int kb, const uint8_t* cA, const uint8_t* cB, const float* cS) __attribute__((always_inline)) {
      i32x8 wf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wf[j] = read_frag(cB, wn * 64 + 16 * j + l16, q);
      const float sw = sSW[sw_blk][kb];
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      i32x8 af_n = read_frag(cA, wm * 128 + 16 + l16, q);
      float sa_n = cS[wm * 128 + 16 + l16];
      f32x4 pc[4];
      {
        const i32x8 af0 = read_frag(cA, wm * 128 + l16, q);
#pragma unroll
        for (int j = 0; j < 4; ++j) pc[j] = mfma_16x16x128_e4m3(wf[j], af0, zero);
      }
      float c_cur = cS[wm * 128 + l16] * sw;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // for each j: promote row i's partial j, then reuse its registers for row i+1
        const i32x8 af = af_n;
        const float c_next = sa_n * sw;
        if (i < 6) {
          af_n = read_frag(cA, wm * 128 + 16 * (i + 2) + l16, q);
          sa_n = cS[wm * 128 + 16 * (i + 2) + l16];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(pc[j][r], c_cur, acc[i][j][r]);
          if (i < 7) pc[j] = mfma_16x16x128_e4m3(wf[j], af, zero);
        }
        if (i < 7) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
        }
        // pin row i's promotion here (otherwise it sinks below every later MFMA)
        asm volatile("" : "+v"(acc[i][0]), "+v"(acc[i][1]), "+v"(acc[i][2]), "+v"(acc[i][3]));
        c_cur = c_next;
      }
    };

    // vmcnt bookkeeping: every iteration issues the operand DMA of block kb+1 and then one
    // prefetch of block kb+2; waiting for vmcnt <= 1 at the top of the next iteration
    // retires the DMA (loads retire in issue order) while the prefetch stays in flight.
    issue(0, sA0, sB0, sS0);
    prefetch(KB > 1 ? 1 : 0);
    for (int kb = 0; kb < KB; kb += 2) {
      asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
      __syncthreads();
      if (kb + 1 < KB) issue(kb + 1, sA1, sB1, sS1);
      prefetch(min(kb + 2, KB - 1));
      compute(kb, sA0, sB0, sS0);
      if (kb + 1 < KB) {
        asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
        __syncthreads();
        if (kb + 2 < KB) issue(kb + 2, sA0, sB0, sS0);
        prefetch(min(kb + 3, KB - 1));
        compute(kb + 1, sA1, sB1, sS1);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: lane owns rows m = wm*128 + 16i + l16, columns n = wn*64 + 16j + 4q .. +3
    if (!OUT_F32) {
      // bf16: stage each wave's 128 x 64 block through LDS (the operand buffers are free
      // now) and write whole 128-byte row segments; 16-byte chunk c of row r sits at
      // chunk position c ^ (r & 7).
      __syncthreads();
      uint8_t* region = (wave < 2 ? sA0 : wave < 4 ? sA1 : wave < 6 ? sB0 : sB1) + (wave & 1) * 16384;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + 16 * j + 4 * q;
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if (HAS_BIAS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) b[r] = (n + r < a.N) ? load_bias(a, expert, n + r) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 16 * i + l16;
          const int pc = (2 * j + (q >> 1)) ^ (row & 7);
          uint2 pk;
          pk.x = pack_bf16x2(acc[i][j][0] + b[0], acc[i][j][1] + b[1]);
          pk.y = pack_bf16x2(acc[i][j][2] + b[2], acc[i][j][3] + b[3]);
          *reinterpret_cast<uint2*>(region + row * 128 + pc * 16 + (q & 1) * 8) = pk;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      // all 16 chunk reads first (the accumulators are dead, registers are free), then
      // all 16 stores, so each wave keeps 16 KB of writes in flight
      i32x4 v[16];
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int id = it * 64 + lane;
        v[it] = *reinterpret_cast<const i32x4*>(region + (id >> 3) * 128 + (id & 7) * 16);
      }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int id = it * 64 + lane;
        const int row = id >> 3, pc = id & 7;
        const int c = pc ^ (row & 7);
        const int ml = wm * 128 + row;
        if (ml >= m_size) continue;
        const int64_t n = n0 + wn * 64 + c * 8;
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + sOrow[ml] * a.ldo + n;
        if (vec8_store && n + 8 <= a.N) {
          *reinterpret_cast<i32x4*>(o) = v[it];
        } else {
          const uint16_t* e = reinterpret_cast<const uint16_t*>(&v[it]);
          for (int r = 0; r < 8 && n + r < a.N; ++r) o[r] = e[r];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + 16 * j + 4 * q;
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if (HAS_BIAS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) b[r] = (n + r < a.N) ? load_bias(a, expert, n + r) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int ml = wm * 128 + 16 * i + l16;
          if (ml >= m_size) continue;
          const int64_t o = sOrow[ml] * a.ldo + n;
          const float v[4] = {acc[i][j][0] + b[0], acc[i][j][1] + b[1], acc[i][j][2] + b[2], acc[i][j][3] + b[3]};
          if (vec_store && n + 3 < a.N) {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < a.N) reinterpret_cast<float*>(a.out)[o + r] = v[r];
          }
        }
      }
    }
  }
}

void launch_gemm_w8a8_big(const GemmArgs& a, int row_mode, bool out_f32, int64_t grid_blocks, hipStream_t st) {
  if (grid_blocks <= 0 || a.N <= 0) return;
  const int64_t n_tiles = cdiv(a.N, kBN);
  int64_t nwg = grid_blocks * n_tiles;
  if (row_mode == ROWS_DENSE) nwg = cdiv(nwg, 8) * 8;
  const dim3 grid(static_cast<unsigned>(nwg)), block(kThreads);
  const bool bias = a.bias != nullptr;
#define MXQ_BIG_GO(MODE, OF, HB) \
  hipLaunchKernelGGL((gemm_w8a8_big_kernel<MODE, OF, HB>), grid, block, 0, st, a, grid_blocks, n_tiles)
#define MXQ_BIG_MODE(MODE)                                   \
  do {                                                       \
    if (out_f32) {                                           \
      if (bias) MXQ_BIG_GO(MODE, true, true);                \
      else MXQ_BIG_GO(MODE, true, false);                    \
    } else {                                                 \
      if (bias) MXQ_BIG_GO(MODE, false, true);               \
      else MXQ_BIG_GO(MODE, false, false);                   \
    }                                                        \
  } while (0)
  switch (row_mode) {
    case ROWS_DENSE: MXQ_BIG_MODE(ROWS_DENSE); break;
    case ROWS_GATHER_TOK: MXQ_BIG_MODE(ROWS_GATHER_TOK); break;
    default: MXQ_BIG_MODE(ROWS_COMPACT_IN); break;
  }
#undef MXQ_BIG_MODE
#undef MXQ_BIG_GO
}

}  // namespace mxq
