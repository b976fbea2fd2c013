// Large-tile block-scaled W8A8 GEMM for gfx950: BM x 256 output tile per
// 512-thread workgroup (8 waves, 2 per SIMD), K step 128 = one weight-scale
// block = one V_MFMA_F32_16X16X128_F8F6F4 per 16 x 16 sub-tile.  BM = 256 (two
// LDS stages) or 128 (three stages: one more K block in flight).
//
// Arithmetic ("SGLang PR 35605 review", implementation item 1 and the
// fp8_utils.py listing): out[m, n] = sum_kb sa[m, kb] * sw[n/128, kb] *
// sum_{k in kb} qa[m, k] * w[n, k] (+ bias), fp32 accumulation, bf16 (or fp32)
// output.  Each K block's partial product is formed on the matrix core from
// zero and promoted into the fp32 accumulator with one FMA by sa * sw.  The
// routed-expert stages ("vLLM PR 50949 review", moe_fp8.cpp listing) run the
// same tile over an expert block's rows.
//
// gfx950 specifics:
//  * operands go global -> LDS with GLOBAL_LOAD_LDS_DWORDX4 (no VGPR staging):
//    one instruction moves 64 x 16 bytes.  Plain-layout rows: 8 rows of a
//    128-byte K slice, 16-byte chunk c of row r stored at chunk c ^ swz(r) so the
//    32-byte fragment reads are free of bank conflicts.  Tiled weights (the
//    load-time layout of prepack.hip): half of one 2 KB tile, stored as is, which
//    is already the fragment order (lane L reads 16 bytes at 16 L and 1024 + 16 L);
//  * the MFMA A operand is the weight tile and the B operand the activation
//    tile, so each lane ends up owning four consecutive output columns of one
//    row: one activation scale per lane per sub-tile and 8-byte (bf16) or
//    16-byte (fp32) stores;
//  * waves are laid out 2 (rows) x 4 (columns); a wave owns BM/2 x 64 outputs,
//    so its 64 weight rows sit inside one 128-wide scale block (one weight scale
//    per wave per K block, staged in LDS for all K blocks up front);
//  * the products of a K block run as a software pipeline (the MFMA of product
//    t + 2 is issued before product t is promoted);
//  * tiles are rastered so that the tiles resident on one XCD (the dispatcher
//    deals workgroups round-robin over the 8 XCDs) share operands in that XCD's
//    L2: bands of 4 row tiles (dense) or of 3 work-list entries (routed, where an
//    expert's blocks are adjacent; bands dealt round-robin over the XCDs) run all
//    their column tiles together.
#include <type_traits>

#include "lds_dma.hpp"
#include "tile_rows.hpp"

namespace mxq {

namespace {

constexpr int kKS = 128;
constexpr int kMaxKB = 128;  // K <= 16384 on this kernel

// BM x BN tile, NW waves laid out WM (rows) x WN (columns) with 64 columns per wave, NS stages.
template <int BM, int BN, int NW, int NS>
struct BigCfg {
  static constexpr int THREADS = NW * 64;
  static constexpr int WN = BN / 64, WM = NW / WN;
  static constexpr int WROWS = BM / WM;  // rows per wave
  static constexpr int TI = WROWS / 16;  // 16-row sub-tiles per wave
  static constexpr int STAGE_BYTES = (BM + BN) * kKS;
  static constexpr int STAGES = NS;  // LDS stages (2 or 3)
  static constexpr int SA_WAVES = BM / 64;   // waves fetching 64 activation scales each
  // Copying waves: only the upper half of the waves copies (twice the pieces each).  Issuing
  // copies holds a wave until the copy engine has queued them (it moves ~64 B per clock per
  // CU, ~1000 clocks per 256x256 block); this way the lower wave of each SIMD starts its
  // products right after the barrier instead of waiting there too.
  static constexpr int COPY_WAVES = NW / 2;
  static constexpr int A_PIECES = BM / 8 / COPY_WAVES;  // 1 KB activation DMAs per copying wave
  static constexpr int B_PIECES = BN / 8 / COPY_WAVES;  // 1 KB weight DMAs per copying wave
  static_assert(WM * WN == NW && TI >= 2 && A_PIECES >= 1 && B_PIECES >= 1 && SA_WAVES <= COPY_WAVES, "tile shape");
  static_assert(BN / 64 <= COPY_WAVES, "per-column scale fetch");
  static_assert(BN % 128 == 0 || BN == 64, "a wave's 64 columns sit inside one 128-wide weight-scale block");
};

// Work-list entries per band of the routed raster (1, 2, 3, 4 and 8 measured on the DeepSeek
// prefill shapes, 512 and 4096 tokens, uniform and Zipf routing: 3 fastest at 4096 tokens by
// ~10 % over block-fastest order without XCD bands, within a few % of the best elsewhere).
constexpr int64_t kRoutedBand = 3;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// 32-byte fragment of row `row` (K chunks 2q, 2q+1) from a swizzled row-major tile.
__device__ __forceinline__ i32x8 read_frag(const uint8_t* tile, int row, int q) {
  const int s = swz(row);
  const uint8_t* base = tile + row * kKS;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + (((2 * q) ^ s) << 4));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + (((2 * q + 1) ^ s) << 4));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Fragment of 16-row group g of a tile stored in the tiled (lane) order.
__device__ __forceinline__ i32x8 read_frag_tiled(const uint8_t* tile, int g, int lane) {
  const uint8_t* base = tile + g * 2048 + lane * 16;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + 1024);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}


}  // namespace

// SWCOL (dense, block_n = 1: one weight scale per output column and 128-wide K block): each K
// block's column scales travel with its operands into LDS, and each product is promoted with
// sa[row] * sw[col] -- the promotion of the smaller tiles, element for element.
template <int BM, int BN, int NW, int NS, int MODE, bool OUT_F32, bool HAS_BIAS, bool TILED, bool SWCOL = false>
__global__ __launch_bounds__((BigCfg<BM, BN, NW, NS>::THREADS)) void gemm_w8a8_big_kernel(GemmArgs a, int64_t grid_blocks,
                                                                                 int64_t n_tiles) {
  static_assert(!SWCOL || MODE == ROWS_DENSE, "per-column weight scales: dense GEMM only");
  using C = BigCfg<BM, BN, NW, NS>;
  constexpr int S = C::STAGES, TI = C::TI, NT = 4 * TI, WROWS = C::WROWS;
  __shared__ __align__(1024) uint8_t sOps[S * C::STAGE_BYTES];  // stage s: A [BM][128] then W [BN][128]
  __shared__ __align__(16) float sS[S][BM];
  __shared__ int64_t sArow[BM];
  __shared__ int64_t sOrow[BM];
  __shared__ float sSW[2][kMaxKB];  // weight scales of the tile's (up to two) 128-wide column blocks
  __shared__ __align__(256) float sFill[NW * 64];  // landing area of the filler scale DMAs (never read)
  __shared__ __align__(16) float sSWc[SWCOL ? S : 1][SWCOL ? BN : 4];  // per-column weight scales

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
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
    // routed: bands of kRoutedBand consecutive work-list entries run all their column tiles
    // on one XCD (entries fastest), so a band's activation rows are shared across its column
    // tiles and each weight tile across the band's blocks of one expert (an expert's blocks are
    // adjacent in the list) in that XCD's L2; the bands are dealt round-robin over the XCDs, so
    // every XCD gets a mix of long and short blocks.  The live entry count is read first; the
    // grid covers the list's capacity.
    const int64_t count = *a.rt.work_count;
    const int64_t n_bands = cdiv(count, kRoutedBand);
    const int64_t band_tiles = kRoutedBand * n_tiles;
    const int64_t x = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int64_t band = (slot / band_tiles) * 8 + x;
    const int64_t in_band = slot % band_tiles;
    if (band >= n_bands) return;
    const int64_t band_rows = min<int64_t>(kRoutedBand, count - band * kRoutedBand);
    if (in_band >= band_rows * n_tiles) return;
    tile = band * kRoutedBand + in_band % band_rows;
    nt = in_band / band_rows;
  }
  const int64_t n0 = nt * BN;
  if (n0 >= a.N) return;

  TileInfo t;
  if (!tile_info<BM, MODE>(a, tile, t)) return;
  const int64_t expert = t.expert;
  const uint8_t* A = reinterpret_cast<const uint8_t*>(a.A);
  const uint8_t* Wb = a.W + expert * a.w_estride;
  const float* swb = reinterpret_cast<const float*>(a.ws) + expert * a.ws_estride;
  const int KB = int(a.K >> 7);
  // dense K split (blockIdx.y = chunk): K blocks [kb0, kb0 + nkb), fp32 partial sums to the
  // chunk's slice of `out`; an empty chunk writes zeros
  const int nsplit = MODE == ROWS_DENSE && a.k_split > 1 ? a.k_split : 1;
  const int split = nsplit > 1 ? int(blockIdx.y) : 0;
  const int kb0 = nsplit > 1 ? min(KB, split * int(a.k_chunk >> 7)) : 0;
  const int nkb = nsplit > 1 ? min(KB - kb0, int(a.k_chunk >> 7)) : KB;
  constexpr int NSB = BN > 128 ? 2 : 1;  // 128-wide weight-scale blocks the tile spans
  // staged once, after the first operand DMA is in flight so the two latencies overlap
  auto stage_weight_scales = [&]() __attribute__((always_inline)) {
    for (int i = tid; i < NSB * KB; i += C::THREADS) {
      const int blk = i / KB, kb = i - blk * KB;
      const int64_t nb = min<int64_t>((n0 >> 7) + blk, cdiv(a.N, 128) - 1);
      sSW[blk][kb] = swb[nb * a.ws_s0 + kb * a.ws_s1];
    }
  };
  const int sw_blk = (wn * 64) >> 7;  // the 128-wide scale block of this wave's columns
  // 16-byte stores need 16-byte aligned rows: the row stride and the base address
  const bool out_al16 = (reinterpret_cast<uintptr_t>(a.out) & 15) == 0;
  const bool vec_store = out_al16 && (a.ldo & 3) == 0;   // 16-byte fp32 stores
  const bool vec8_store = out_al16 && (a.ldo & 7) == 0;  // 16-byte bf16 stores

  for (int m_base = 0; m_base < t.m_total; m_base += BM) {
    const int m_size = min(BM, t.m_total - m_base);
    __syncthreads();
    fill_rows<BM, MODE>(a, t, m_base, sArow, sOrow);
    __syncthreads();

    // ---- per-lane DMA sources (32-bit byte offsets: the host routes operands below 4 GiB here)
    // cw: this wave's index among the copying waves (a wave that copies nothing computes
    // valid but unused offsets)
    const bool copier = wave >= NW / 2;
    const int cw = max(wave - NW / 2, 0);
    uint32_t oa[C::A_PIECES], ob[C::B_PIECES];
#pragma unroll
    for (int b = 0; b < C::A_PIECES; ++b) {
      const int row = (cw * C::A_PIECES + b) * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ swz(row);
      oa[b] = uint32_t(sArow[row] * a.lda + chunk * 16);
    }
#pragma unroll
    for (int b = 0; b < C::B_PIECES; ++b) {
      const int d = cw * C::B_PIECES + b;  // the tile's d-th 1 KB weight piece
      if (TILED) {
        // piece d = half (d & 1) of the tile of 16-row group d / 2
        const int64_t g16 = min<int64_t>(n0 / 16 + (d >> 1), a.N / 16 - 1);
        ob[b] = uint32_t(g16 * KB * 2048 + (d & 1) * 1024 + lane * 16);
      } else {
        const int row = d * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(row);
        const int64_t n = min<int64_t>(n0 + row, a.N - 1);
        ob[b] = uint32_t(n * a.ldw + chunk * 16);
      }
    }
    // activation scales: copying waves cw < BM/64 fetch 64 rows each; the other ones fetch a
    // filler dword into sFill so that every copying wave issues the same number of loads per
    // K block
    const bool sa_wave = cw < C::SA_WAVES;
    const uint32_t os = uint32_t(sArow[(cw % C::SA_WAVES) * 64 + lane] * a.lds * 4);

    auto stageA = [&](int s) -> uint8_t* { return sOps + s * C::STAGE_BYTES; };
    auto stageB = [&](int s) -> uint8_t* { return sOps + s * C::STAGE_BYTES + BM * kKS; };

    // one K block: A_PIECES + B_PIECES operand DMAs and one scale DMA per copying wave (one
    // more with per-column weight scales)
    auto issue = [&](int kb, int s) __attribute__((always_inline)) {
      if (!copier) return;
      const uint8_t* Ak = A + kb * kKS;
      const uint8_t* Wk = Wb + kb * (TILED ? 2048 : kKS);
      const uint32_t la = __builtin_amdgcn_readfirstlane(lds_addr(stageA(s)) + cw * C::A_PIECES * 1024);
      const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(stageB(s)) + cw * C::B_PIECES * 1024);
#pragma unroll
      for (int b = 0; b < C::A_PIECES; ++b) lds_dma16(Ak, oa[b], la + b * 1024);
#pragma unroll
      for (int b = 0; b < C::B_PIECES; ++b) lds_dma16(Wk, ob[b], lb + b * 1024);
      const uint32_t ls = sa_wave ? lds_addr(&sS[s][0]) + cw * 256 : lds_addr(sFill) + wave * 256;
      lds_dma4(a.sa + kb, os, __builtin_amdgcn_readfirstlane(ls));
      if constexpr (SWCOL) {
        // copying waves cw < BN / 64 fetch 64 column scales each; the others a filler dword
        const bool sw_wave = cw < BN / 64;
        const int64_t col = min<int64_t>(n0 + (cw % (BN / 64)) * 64 + lane, a.N - 1);
        const uint32_t lw = sw_wave ? lds_addr(&sSWc[s][0]) + cw * 256 : lds_addr(sFill) + wave * 256;
        lds_dma4(swb + col * a.ws_s0 + kb * a.ws_s1, __builtin_amdgcn_readfirstlane(lw));
      }
    };
    constexpr int kIssueOps = C::A_PIECES + C::B_PIECES + 1 + (SWCOL ? 1 : 0);  // per copying wave

    f32x4 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One K block: hold the wave's 4 weight fragments and stream the TI activation
    // fragments.  The products t = 4 i + j run as a software pipeline: step t issues the
    // MFMA of product t + 2 and then promotes product t (acc += partial * sa * sw), whose
    // MFMA went out two MFMAs earlier, from a ring of three partial-sum registers.
    // Scheduling fences around the promotion keep that order (left alone, the scheduler
    // moves each promotion right behind the MFMA that produces it and stalls on the
    // result).
    // `tie` (a compile-time count <= TI): the wave's leading 16-row sub-tiles that hold rows of
    // the block; the others are neither multiplied nor promoted (a short routed block in a
    // 128-row tile costs only its own rows' MFMAs).
    auto compute = [&](int kb, int s, auto tie) __attribute__((always_inline)) {
      constexpr int TIE = decltype(tie)::value;
      constexpr int NTE = 4 * TIE;
      const uint8_t* cA = stageA(s);
      const uint8_t* cB = stageB(s);
      const float* cS = sS[s];
      constexpr int DIST = 2, NB = DIST + 1;
      const int mrow = wm * WROWS;
      // the activation scales of all the wave's rows are read first, so that no wait for one
      // of them also waits for the fragment reads issued after it
      float cr[TI];  // combined scales of rows i
#pragma unroll
      for (int r = 0; r < TIE; ++r) cr[r] = cS[mrow + 16 * r + l16];
      i32x8 wf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wf[j] = TILED ? read_frag_tiled(cB, wn * 4 + j, lane) : read_frag(cB, wn * 64 + 16 * j + l16, q);
      const float sw = SWCOL ? 1.f : sSW[sw_blk][kb];
      f32x4 csw[4];  // SWCOL: the scales of this lane's 4 columns in each of the wave's 4 blocks
      if constexpr (SWCOL) {
#pragma unroll
        for (int j = 0; j < 4; ++j) csw[j] = *reinterpret_cast<const f32x4*>(&sSWc[s][wn * 64 + 16 * j + 4 * q]);
      }
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      i32x8 afr[2];  // activation fragments of rows i (slot i & 1)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (r >= TIE) break;
        afr[r] = read_frag(cA, mrow + 16 * r + l16, q);
      }
#pragma unroll
      for (int r = 0; r < TIE; ++r) cr[r] *= sw;
      f32x4 pb[NB];
#pragma unroll
      for (int u = 0; u < DIST; ++u) pb[u] = mfma_16x16x128_e4m3(wf[u & 3], afr[(u >> 2) & 1], zero);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NTE; ++u) {
        const int um = u + DIST;
        if (um < NTE) {
          const int im = um >> 2, jm = um & 3;
          pb[um % NB] = mfma_16x16x128_e4m3(wf[jm], afr[im & 1], zero);
          // the last MFMA of row im is out: its fragment slot takes row im + 2
          if (jm == 3 && im + 2 < TIE) afr[im & 1] = read_frag(cA, mrow + 16 * (im + 2) + l16, q);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int i = u >> 2, j = u & 3;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[i][j][r] = fmaf(pb[u % NB][r], SWCOL ? cr[i] * csw[j][r] : cr[i], acc[i][j][r]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // sub-tiles of this wave holding rows of the pass (routed blocks may be short; dense tiles
    // are full except possibly the last, which keeps the full product)
    const int n_ti = MODE == ROWS_DENSE ? TI : max(0, min(TI, (m_size - wm * WROWS + 15) / 16));
    auto compute_rows = [&](int kb, int s) __attribute__((always_inline)) {
      if (n_ti == TI) {
        compute(kb, s, std::integral_constant<int, TI>{});
        return;
      }
      switch (n_ti) {
        case 1: compute(kb, s, std::integral_constant<int, 1>{}); break;
        case 2: if constexpr (TI > 2) compute(kb, s, std::integral_constant<int, (TI > 2 ? 2 : TI)>{}); break;
        case 3: if constexpr (TI > 3) compute(kb, s, std::integral_constant<int, (TI > 3 ? 3 : TI)>{}); break;
        case 4: if constexpr (TI > 4) compute(kb, s, std::integral_constant<int, (TI > 4 ? 4 : TI)>{}); break;
        case 5: if constexpr (TI > 5) compute(kb, s, std::integral_constant<int, (TI > 5 ? 5 : TI)>{}); break;
        case 6: if constexpr (TI > 6) compute(kb, s, std::integral_constant<int, (TI > 6 ? 6 : TI)>{}); break;
        case 7: if constexpr (TI > 7) compute(kb, s, std::integral_constant<int, (TI > 7 ? 7 : TI)>{}); break;
        default: break;  // no rows of the pass in this wave's sub-tiles
      }
    };

    // ---- K loop.  Loads retire in issue order.  Each iteration waits for its own stage,
    // publishes it with a barrier (which also retires every wave's reads of the stage the
    // next DMA overwrites), issues the DMA S - 1 blocks ahead, and computes.
    // (j counts the workgroup's K blocks, kb0 + j is the block; without a split kb0 = 0, nkb = KB)
    if (S == 2) {
      if (nkb > 0) issue(kb0, 0);
      if (!SWCOL && m_base == 0) stage_weight_scales();
      for (int j = 0; j < nkb; ++j) {
        wait_vmcnt<0>();
        __syncthreads();
        if (j + 1 < nkb) issue(kb0 + j + 1, (j + 1) & 1);
        compute_rows(kb0 + j, j & 1);
      }
    } else {
      // ops a copying wave has issued after DMA(j) at the top of iteration j: DMA(j+1) when
      // it exists (the other waves have none outstanding)
      if (nkb > 0) issue(kb0, 0);
      if (nkb > 1) issue(kb0 + 1, 1);
      if (!SWCOL && m_base == 0) stage_weight_scales();
      int s = 0;
      for (int j = 0; j < nkb; ++j) {
        if (j + 1 < nkb)
          wait_vmcnt<kIssueOps>();
        else
          wait_vmcnt<0>();
        __syncthreads();
        if (j + 2 < nkb) issue(kb0 + j + 2, s == 0 ? 2 : s - 1);
        compute_rows(kb0 + j, s);
        s = s == S - 1 ? 0 : s + 1;
      }
    }
    wait_vmcnt<0>();

    // ---- epilogue: lane owns rows m = wm*WROWS + 16i + l16, columns n = wn*64 + 16j + 4q .. +3
    if (!OUT_F32) {
      // bf16: stage each wave's WROWS x 64 block through LDS (the operand stages are free
      // now) and write whole 128-byte row segments; 16-byte chunk c of row r sits at chunk
      // position c ^ (r & 7).
      __syncthreads();
      uint8_t* region = sOps + wave * WROWS * 128;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + 16 * j + 4 * q;
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if (HAS_BIAS && split == 0) {  // (a K split adds the bias on its first chunk only)
#pragma unroll
          for (int r = 0; r < 4; ++r) b[r] = (n + r < a.N) ? load_bias(a, expert, n + r) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < TI; ++i) {
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
      // all chunk reads first (the accumulators are dead, registers are free), then all
      // stores, so each wave keeps its whole block of writes in flight
      constexpr int CH = WROWS / 8;  // 16-byte chunks per lane
      i32x4 v[CH];
#pragma unroll
      for (int it = 0; it < CH; ++it) {
        const int id = it * 64 + lane;
        v[it] = *reinterpret_cast<const i32x4*>(region + (id >> 3) * 128 + (id & 7) * 16);
      }
#pragma unroll
      for (int it = 0; it < CH; ++it) {
        const int id = it * 64 + lane;
        const int row = id >> 3, pc = id & 7;
        const int c = pc ^ (row & 7);
        const int ml = wm * WROWS + row;
        if (ml >= m_size) continue;
        const int64_t n = n0 + wn * 64 + c * 8;
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + sOrow[ml] * a.ldo + n;
        if (vec8_store && n + 8 <= a.N) {
          // streaming store: the output is not re-read by this kernel
          __builtin_nontemporal_store(v[it], reinterpret_cast<i32x4*>(o));
        } else {
          const uint16_t* e = reinterpret_cast<const uint16_t*>(&v[it]);
          for (int r = 0; r < 8 && n + r < a.N; ++r) o[r] = e[r];
        }
      }
    } else {
      float* const outf = reinterpret_cast<float*>(a.out) + (nsplit > 1 ? split * a.split_stride : 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + 16 * j + 4 * q;
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if (HAS_BIAS && split == 0) {  // (a K split adds the bias on its first chunk only)
#pragma unroll
          for (int r = 0; r < 4; ++r) b[r] = (n + r < a.N) ? load_bias(a, expert, n + r) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int ml = wm * WROWS + 16 * i + l16;
          if (ml >= m_size) continue;
          const int64_t o = sOrow[ml] * a.ldo + n;
          const float v[4] = {acc[i][j][0] + b[0], acc[i][j][1] + b[1], acc[i][j][2] + b[2], acc[i][j][3] + b[3]};
          if (vec_store && n + 3 < a.N) {
            *reinterpret_cast<f32x4*>(outf + o) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < a.N) outf[o + r] = v[r];
          }
        }
      }
    }
  }
}

template <int BM, int BN, int NW, int NS, int MODE, bool TL, bool SWC = false>
static void launch_big_t(const GemmArgs& a, bool out_f32, int64_t grid_blocks, hipStream_t st) {
  const int64_t n_tiles = cdiv(a.N, int64_t(BN));
  // whole rounds over the 8 XCDs; routed: every XCD's share of bands at full width
  const int64_t nwg = MODE == ROWS_DENSE ? cdiv(grid_blocks * n_tiles, 8) * 8
                                         : 8 * cdiv(cdiv(grid_blocks, kRoutedBand), 8) * kRoutedBand * n_tiles;
  const unsigned chunks = MODE == ROWS_DENSE && a.k_split > 1 ? unsigned(a.k_split) : 1u;
  const dim3 grid(static_cast<unsigned>(nwg), chunks), block(BigCfg<BM, BN, NW, NS>::THREADS);
  const bool bias = a.bias != nullptr;
#define MXQ_BIG_GO(OF, HB)                                                                                     \
  hipLaunchKernelGGL((gemm_w8a8_big_kernel<BM, BN, NW, NS, MODE, OF, HB, TL, SWC>), grid, block, 0, st, a, grid_blocks, \
                     n_tiles)
  if (out_f32) { if (bias) MXQ_BIG_GO(true, true); else MXQ_BIG_GO(true, false); }
  else { if (bias) MXQ_BIG_GO(false, true); else MXQ_BIG_GO(false, false); }
#undef MXQ_BIG_GO
}

int big_tile_rows(int shape) { return shape == 0 ? 256 : 128; }

// Shapes: 0 = 256 x 256 (8 waves, 2 stages), 1 = 128 x 256 (8 waves, 3 stages),
// 2 = 128 x 128 (4 waves, 2 stages: two workgroups per CU), 3 = 128 x 128 (4 waves, 3 stages).
void launch_gemm_w8a8_big(const GemmArgs& a, int row_mode, int shape, bool out_f32, int64_t grid_blocks,
                          hipStream_t st) {
  if (grid_blocks <= 0 || a.N <= 0) return;
  if (row_mode == ROWS_DENSE) {
    // block_n == 1: per-column weight scales
    if (a.block_n == 1) {
      switch (shape) {
        case 0: launch_big_t<256, 256, 8, 2, ROWS_DENSE, false, true>(a, out_f32, grid_blocks, st); break;
        case 2: launch_big_t<128, 128, 4, 2, ROWS_DENSE, false, true>(a, out_f32, grid_blocks, st); break;
        case 3: launch_big_t<128, 128, 4, 3, ROWS_DENSE, false, true>(a, out_f32, grid_blocks, st); break;
        default: launch_big_t<128, 256, 8, 3, ROWS_DENSE, false, true>(a, out_f32, grid_blocks, st); break;
      }
      return;
    }
    switch (shape) {
      case 0: launch_big_t<256, 256, 8, 2, ROWS_DENSE, false>(a, out_f32, grid_blocks, st); break;
      case 2: launch_big_t<128, 128, 4, 2, ROWS_DENSE, false>(a, out_f32, grid_blocks, st); break;
      case 3: launch_big_t<128, 128, 4, 3, ROWS_DENSE, false>(a, out_f32, grid_blocks, st); break;
      default: launch_big_t<128, 256, 8, 3, ROWS_DENSE, false>(a, out_f32, grid_blocks, st); break;
    }
    return;
  }
  // routed blocks hold at most 128 rows: the 128 x 256 three-stage tile
  const bool tl = a.w_tiled != 0;
  if (row_mode == ROWS_GATHER_TOK) {
    if (tl) launch_big_t<128, 256, 8, 3, ROWS_GATHER_TOK, true>(a, out_f32, grid_blocks, st);
    else launch_big_t<128, 256, 8, 3, ROWS_GATHER_TOK, false>(a, out_f32, grid_blocks, st);
  } else {
    if (tl) launch_big_t<128, 256, 8, 3, ROWS_COMPACT_IN, true>(a, out_f32, grid_blocks, st);
    else launch_big_t<128, 256, 8, 3, ROWS_COMPACT_IN, false>(a, out_f32, grid_blocks, st);
  }
}

}  // namespace mxq
