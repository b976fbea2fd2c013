// Routed bf16-activation expert tiles (W8A16 block-FP8 and W4A16 MXFP4 weights) fed by a ring of
// LDS stages that direct global-to-LDS copies fill.
//
// What is computed is the block walk of "vLLM PR 50949 review" (moe_fp8.cpp listing): each
// expert block's rows times its expert's weights, the e4m3 partial sum of every 128-wide K block
// scaled by that block's weight scale before it joins the accumulator; MXFP4 weights carry an
// e8m0 scale per 32 elements, folded into the exact e2m1 -> bf16 decode.  The products run on
// V_MFMA_F32_16X16X32_BF16 after in-register decode of the weights (every e4m3 value and every
// scaled e2m1 value is a bf16 value).
//
// How it is fed: a 128-wide K step of a tile is one LDS stage (activation rows, 128 weight rows,
// MXFP4 scales).  GLOBAL_LOAD_LDS copies move the step straight from memory into its stage, so no
// register staging or second barrier sits between a step's arrival and its products; NS stages
// (three for 128-row tiles, four for smaller ones) keep NS - 1 steps in flight while one is being
// multiplied.  Every wave issues the same number of copies per step, so one vmcnt wait per step
// followed by one barrier publishes the step.  Eight waves (two per SIMD) let one wave's LDS
// reads overlap the other's products.  (Measured and dropped: issuing the first steps' weight
// copies before the row table is read; skipping the copies of activation rows past the block's
// row count, with per-wave vmcnt targets or as one-lane copies -- 1-5 % slower, the copies of
// the repeated last row hit in cache.)
//
// LDS layouts (per stage):
//  * activations: row-major 256-byte rows; the 16-byte chunk c of row r sits in slot c ^ (r % 16)
//    (the copying lane picks its source chunk by that rule), so the 16 rows an MFMA fragment read
//    touches fall in 16 different bank groups;
//  * e4m3 weights: per 16-row group a 2 KB block in fragment order -- half h, lane (q, r) holds
//    bytes [32 q + 16 h, +16) of row r's 128-byte step -- the layout the tiled prepack format
//    already has in memory, gathered the same way from the plain layout;
//  * e2m1 weights: per 16-row group 1 KB, half h = (K step offset / 16) % 2 of the 64-byte step;
//  * e8m0 scales: tiled, the 64 bytes of each group's scale tile for the step; plain, 4 bytes
//    per row.
// A ragged K tail (K a multiple of 32, not of 128) needs no zero fill: the sub-steps of 32 past K
// are not computed, and copies past a row's end read that row's first chunk instead.
#include <algorithm>
#include <type_traits>

#include "lds_dma.hpp"
#include "quant_common.hpp"
#include "tile_rows.hpp"


namespace mxq {

namespace {

constexpr int kRingThreads = 512;
constexpr int kRingMaxSteps = 128;  // K <= 16384: weight-block scales of the K range in LDS

template <int WFMT>
struct RingFmt {
  static constexpr bool MX = WFMT == W_E2M1_MX;
  static constexpr int w_bytes = MX ? 128 * 64 : 128 * 128;  // 128 weight rows of one K step
  static constexpr int s_bytes = MX ? 512 : 0;                // their e8m0 scales
};

template <int BM>
constexpr int ring_stages() { return BM == 128 ? 3 : 4; }

template <int BM, int WFMT>
constexpr int ring_stage_bytes() { return BM * 256 + RingFmt<WFMT>::w_bytes + RingFmt<WFMT>::s_bytes; }

template <int BM, int WFMT, bool OUT_F32>
constexpr size_t ring_lds_bytes() {
  const size_t ops = size_t(ring_stages<BM>()) * ring_stage_bytes<BM, WFMT>() + 2 * kRingMaxSteps * 4;
  const size_t out = OUT_F32 ? size_t(BM) * (128 + 4) * 4 : size_t(BM) * (128 + 8) * 2;
  return ops > out ? ops : out;
}

}  // namespace

// Self-routed block (small routings; every thread of the workgroup calls it): block `blk` of
// the routing as the sort kernel would lay the blocks out -- experts ascending, each expert's
// rows (flat ids ascending) cut into blocks of block_m -- found from the routing ids in LDS
// (`scratch`, R + E + 24 ints; on return its first R ints hold each routed row's expert, -1 when
// dropped).  Fills t and the block's flat routed ids s_rows (ascending) and
// returns the block's class from its own row count, or -1 (uniformly) when the block does not
// exist.
__device__ __forceinline__ int self_route_block(const BlockRouting& rt, int64_t blk, TileInfo& t, int32_t* scratch,
                                                int32_t* s_rows, int32_t* s_pick) {
  constexpr int NT = kRingThreads, NW = kRingThreads / 64;
  const int R = rt.route_R, E = rt.route_E, bm = rt.block_m;
  int32_t* s_ids = scratch;      // [R]: expert of each routed row, -1 when dropped
  int32_t* cnt = s_ids + R;      // [E]: rows per expert
  int32_t* wsum = cnt + E;       // [2 NW]: wave sums of the scans, then [NW] wave counts
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = tid; e < E; e += NT) cnt[e] = 0;
  if (tid == 0) s_pick[0] = -1;
  __syncthreads();
  for (int r = tid; r < R; r += NT) {
    int e = rt.route_ids[r];
    if (e < 0 || e >= E) e = -1;
    s_ids[r] = e;
    if (e >= 0) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // thread e (E <= NT): its expert's rows and blocks; exclusive scans of both over the experts
  // (thread order is expert order)
  const int my_rows = tid < E ? cnt[tid] : 0;
  const int my_blks = (my_rows + bm - 1) / bm;
  int sr = my_rows, sb = my_blks;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int tr = __shfl_up(sr, o, 64), tb = __shfl_up(sb, o, 64);
    if (lane >= o) {
      sr += tr;
      sb += tb;
    }
  }
  if (lane == 63) {
    wsum[2 * wave] = sr;
    wsum[2 * wave + 1] = sb;
  }
  __syncthreads();
  int pr = 0, pb = 0;
  for (int w = 0; w < wave; ++w) {
    pr += wsum[2 * w];
    pb += wsum[2 * w + 1];
  }
  const int row0 = pr + sr - my_rows, blk0 = pb + sb - my_blks;
  if (tid < E && blk >= blk0 && blk < blk0 + my_blks) {
    const int b = int(blk - blk0);
    const int m = min(bm, my_rows - b * bm);
    s_pick[0] = tid;
    s_pick[1] = b;
    s_pick[2] = m;
    s_pick[3] = row0 + b * bm;
    s_pick[4] = pick_class(rt.route_pol, m);
  }
  __syncthreads();
  const int pe = s_pick[0];
  if (pe < 0) return -1;
  const int r_lo = s_pick[1] * bm, m_size = s_pick[2];
  // the block's rows: the routed rows of expert pe whose rank among them lies in
  // [r_lo, r_lo + m_size) (ranks from ballots and wave counts, in flat-id order)
  int base = 0;
  int32_t* wcnt = wsum + 2 * NW;  // [NW]
  for (int r0 = 0; r0 < R; r0 += NT) {
    const int r = r0 + tid;
    const bool hit = r < R && s_ids[r] == pe;
    const uint64_t bal = __ballot(hit);
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int pre = base, tot = 0;
    for (int w = 0; w < NW; ++w) {
      pre += w < wave ? wcnt[w] : 0;
      tot += wcnt[w];
    }
    const int i = pre + __popcll(bal & lt) - r_lo;
    if (hit && i >= 0 && i < m_size) s_rows[i] = r;
    base += tot;
    __syncthreads();
  }
  t.expert = pe;
  t.m0 = 0;
  t.mb = 0;
  t.off = s_pick[3];
  t.m_total = m_size;
  return s_pick[4];
}

// The tile body: block t, column tile nt, K chunk `split`.  s_rows: the block's flat routed ids
// when the tile was self-routed, else NULL (rows from the sort's tables).
template <int BM, int MODE, int WFMT, bool OUT_F32, bool HAS_BIAS, bool TILED>
__device__ __forceinline__ void ring_body(const GemmArgs& a, const TileInfo& t, int64_t nt, int split, uint8_t* lds,
                                          const int32_t* s_rows) {
  constexpr int NT = kRingThreads, BN = 128, NS = ring_stages<BM>();
  constexpr int WAVES_M = BM == 128 ? 4 : (BM == 16 ? 1 : 2);
  constexpr int WAVES_N = (NT / 64) / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  static_assert(TM >= 1 && TN >= 1 && TM <= 2, "wave tile");
  constexpr bool MX = WFMT == W_E2M1_MX;
  // MXFP4 (scales folded into the decode) and per-tensor e4m3 (one scale, applied in the
  // epilogue) accumulate straight into acc; block e4m3 scales each K step's partial sum
  constexpr bool DIRECT = MX || WFMT == W_E4M3_TENSOR;
  constexpr int STAGE = ring_stage_bytes<BM, WFMT>();
  constexpr int W_OFF = BM * 256, S_OFF = W_OFF + RingFmt<WFMT>::w_bytes;
  constexpr int A_INS = BM == 16 ? 1 : BM / 32;  // activation copies per wave per step
  constexpr int P = A_INS + 2;                    // copies per wave per step (+ weights, scales)
  static_assert(NS - 2 <= 2, "vmcnt targets below cover at most two steps in flight");

  float* const sSw = reinterpret_cast<float*>(lds + NS * STAGE);  // weight-block scale per K step
  const uint32_t lbase = lds_addr(lds);  // LDS byte address of the stages, as copies take it
  __shared__ int64_t sArow[BM];
  __shared__ int64_t sOrow[BM];
  __shared__ float sWt[BM];  // top-1 fold: the routing weight of each output row

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int frow = lane & 15, fq = lane >> 4;
  const int nsplit = a.k_split > 1 ? a.k_split : 1;
  const int64_t n0 = nt * BN;
  const bool self_routed = s_rows != nullptr;
  // Paired tile (stage 1 with the SiLU-and-mul in its epilogue; no K split): tile nt holds ic1
  // columns [64 nt, +64), its weight-row groups 0..3 are the gate rows 64 nt + 16 g and groups
  // 4..7 the matching up rows I + 64 nt + 16 (g - 4) (N = 2 I, I a multiple of 64).
  const bool pair = a.silu_pair != 0;
  const int64_t half = a.N / 2;
  auto group_row0 = [&](int g) -> int64_t {
    return pair ? (g < 4 ? 64 * nt + 16 * g : half + 64 * nt + 16 * (g - 4)) : n0 + 16 * g;
  };
  const int64_t expert = t.expert;
  const int KS = int(cdiv(a.K, 128));
  int ks_b = 0, ks_e = KS;
  if (nsplit > 1) {
    const int cs = int(a.k_chunk >> 7);
    ks_b = min(KS, split * cs);
    ks_e = min(KS, ks_b + cs);
  }
  const int nsteps = ks_e - ks_b;

  // weight-block scales of the K range (read before any copy is in flight)
  if (WFMT == W_E4M3_BLOCK) {
    // paired: the gate half's 128-row scale block in sSw[0, steps), the up half's in
    // sSw[kRingMaxSteps, +steps)
    const float* sw0 = reinterpret_cast<const float*>(a.ws) + expert * a.ws_estride;
    const int64_t nb0 = group_row0(0) / 128, nb1 = group_row0(4) / 128;
    for (int i = tid; i < nsteps; i += NT) {
      sSw[i] = sw0[nb0 * a.ws_s0 + int64_t(ks_b + i) * a.ws_s1];
      if (pair) sSw[kRingMaxSteps + i] = sw0[nb1 * a.ws_s0 + int64_t(ks_b + i) * a.ws_s1];
    }
  }

  // ---- copies: wave w copies weight group w of the tile (16 rows) and the activation copies k
  // holding rows 4 (w + 8 k) .. +3 (BM = 16: rows 2 w, 2 w + 1 on lanes 0..31).  (Measured and
  // dropped, no gain: the upper wave of each SIMD issuing the lower wave's share too, so that
  // the lower one starts its products at once; the upper wave issuing its share after its
  // products instead of before them.)
  const uint8_t* Wb = a.W + expert * a.w_estride;
  const int64_t row_bytes = MX ? a.K / 2 : a.K;
  const int64_t tsteps = (row_bytes + 127) / 128;  // tiled layout: 128-byte row steps per group
  const int64_t grow0 = group_row0(wave);  // first weight row of this wave's 16-row group
  const int64_t grp16 = min<int64_t>(grow0 / 16, a.N / 16 - 1);
  const int64_t wrow = min<int64_t>(grow0 + frow, a.N - 1);
  const uint8_t* gw[2];
  int wbyte[2];  // plain layout: first byte of the lane's piece inside the row's K step
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (MX) {
      // one copy per step: lane (h, qq, r) = (lane / 32, lane / 16 % 2, lane % 16)
      const int hh = lane >> 5, qq = (lane >> 4) & 1;
      wbyte[h] = qq * 32 + hh * 16;
      gw[h] = TILED ? Wb + grp16 * tsteps * 2048 + hh * 1024 + (qq * 16 + frow) * 16 : Wb + wrow * a.ldw + wbyte[h];
    } else {
      // two copies per step (halves h): lane (qq, r) = (lane / 16, lane % 16)
      wbyte[h] = fq * 32 + h * 16;
      gw[h] = TILED ? Wb + grp16 * tsteps * 2048 + h * 1024 + lane * 16 : Wb + wrow * a.ldw + wbyte[h];
    }
  }
  const uint8_t* gs = nullptr;  // MXFP4 scale source (lanes 0..15)
  if (MX) {
    const uint8_t* se = reinterpret_cast<const uint8_t*>(a.ws) + expert * a.ws_estride;
    if (TILED)
      gs = se + grp16 * tsteps * 128 + (lane & 15) * 4;
    else
      gs = se + min<int64_t>(grow0 + (lane & 15), a.N - 1) * a.ws_s0;
  }

  for (int m_base = 0; m_base < t.m_total; m_base += BM) {
    const int m_size = min(BM, t.m_total - m_base);
    __syncthreads();  // the previous pass is done with the row tables and LDS

    auto issue_w = [&](int ks, int stage) __attribute__((always_inline)) {
      const uint32_t sb = lbase + uint32_t(stage * STAGE);
      const int64_t kbase = int64_t(ks) * 128;
      if (MX) {
        const int64_t step = TILED ? int64_t(ks >> 1) * 2048 + (ks & 1) * 512 : int64_t(ks) * 64;
        const uint8_t* src = gw[0] + step;
        if (!TILED && step + wbyte[0] >= row_bytes) src = gw[0] - wbyte[0];
        lds_dma16(src, sb + W_OFF + wave * 1024);
        const int64_t sstep = TILED ? int64_t(ks >> 1) * 128 + (ks & 1) * 64 : int64_t(ks) * 4;
        if (lane < 16) lds_dma4(gs + sstep, sb + S_OFF + wave * 64);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t step = TILED ? int64_t(ks) * 2048 : kbase;
          const uint8_t* src = gw[h] + step;
          if (!TILED && step + wbyte[h] >= row_bytes) src = gw[h] - wbyte[h];
          lds_dma16(src, sb + W_OFF + wave * 2048 + h * 1024);
        }
      }
    };

    if (self_routed) {
      // rows past the block repeat its last row and are never stored
      for (int i = tid; i < BM; i += NT) {
        const int ii = min(m_base + i, t.m_total - 1);
        const int32_t r = s_rows[ii];
        sArow[i] = MODE == ROWS_GATHER_TOK ? r / a.rt.topk : t.off + ii;
        sOrow[i] = MODE == ROWS_GATHER_TOK ? int64_t(t.off + ii) : int64_t(r);
        if (MODE == ROWS_COMPACT_IN && a.top1_w) sWt[i] = a.top1_w[r];
      }
    } else {
      fill_rows<BM, MODE>(a, t, m_base, sArow, sOrow);
    }
    __syncthreads();

    // activation copy sources; the lane's source chunk is its slot XOR the row's swizzle
    const uint8_t* ga[A_INS];
    int gac[A_INS];
#pragma unroll
    for (int k = 0; k < A_INS; ++k) {
      const int row = BM == 16 ? min(2 * wave + (lane >> 4), BM - 1) : 4 * (wave + 8 * k) + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);
      gac[k] = c;
      ga[k] = reinterpret_cast<const uint8_t*>(a.A) + sArow[row] * a.lda * 2 + c * 16;
    }
    auto issue_a = [&](int ks, int stage) __attribute__((always_inline)) {
      const uint32_t sb = lbase + uint32_t(stage * STAGE);
      const int64_t kbase = int64_t(ks) * 128;
#pragma unroll
      for (int k = 0; k < A_INS; ++k) {
        // a chunk past K re-reads the row's first chunk (its sub-step is never computed)
        const uint8_t* src = kbase + gac[k] * 8 < a.K ? ga[k] + kbase * 2 : ga[k] - gac[k] * 16;
        const uint32_t dst = sb + (BM == 16 ? wave * 512 : (wave + 8 * k) * 1024);
        if (BM != 16 || lane < 32) lds_dma16(src, dst);
      }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // products of one K step for the wave's first TL row tiles (those holding block rows);
    // FULL: all four 32-wide sub-steps lie inside K
    auto compute = [&](int ks, int stage, auto tl_c, auto full_c) __attribute__((always_inline)) {
      constexpr int TL = decltype(tl_c)::value;
      constexpr bool FULL = decltype(full_c)::value;
      const uint8_t* const sa = lds + stage * STAGE;
      const uint8_t* const sw = sa + W_OFF;
      const uint8_t* const ss = sa + S_OFF;
      const int nsub = FULL ? 4 : int(min<int64_t>(4, (a.K - int64_t(ks) * 128) >> 5));
      f32x4 part[TL][TN];
#pragma unroll
      for (int i = 0; i < TL; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (!FULL && s >= nsub) break;
        i32x4 af[TL], bfr[TN];
#pragma unroll
        for (int i = 0; i < TL; ++i) {
          const int r = wm * WM + 16 * i + frow;
          af[i] = *reinterpret_cast<const i32x4*>(sa + r * 256 + (((s * 4 + fq) ^ frow) << 4));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int g = (wn * WN >> 4) + j;  // 16-row weight group
          if (MX) {
            const uint32_t v =
                *reinterpret_cast<const uint32_t*>(sw + g * 1024 + (s & 1) * 512 + ((s >> 1) * 16 + frow) * 16 + fq * 4);
            const uint32_t e = TILED ? ss[g * 64 + (s >> 1) * 32 + frow * 2 + (s & 1)] : ss[(g * 16 + frow) * 4 + s];
            uint32_t o[4];
            e2m1x8_to_bf16(v, e8m0_to_f32(e), o);
            bfr[j] = i32x4{int(o[0]), int(o[1]), int(o[2]), int(o[3])};
          } else {
            const uint2 v =
                *reinterpret_cast<const uint2*>(sw + g * 2048 + (fq >> 1) * 1024 + (s * 16 + frow) * 16 + (fq & 1) * 8);
            uint32_t o0, o1, o2, o3;
            e4m3x4_to_bf16(v.x, o0, o1);
            e4m3x4_to_bf16(v.y, o2, o3);
            bfr[j] = i32x4{int(o0), int(o1), int(o2), int(o3)};
          }
        }
#pragma unroll
        for (int i = 0; i < TL; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if (DIRECT)
              acc[i][j] = mfma_16x16x32_bf16(af[i], bfr[j], acc[i][j]);
            else
              part[i][j] = mfma_16x16x32_bf16(af[i], bfr[j], part[i][j]);
          }
      }
      if (!DIRECT) {
        const float swv = sSw[(pair && wn * WN >= 64 ? kRingMaxSteps : 0) + ks - ks_b];
#pragma unroll
        for (int i = 0; i < TL; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(part[i][j][r], swv, acc[i][j][r]);
      }
    };

    // row tiles of this wave that hold rows of the block
    const int tl = min(TM, max(0, (m_size - wm * WM + 15) >> 4));

    for (int j = 0; j < NS - 1; ++j)
      if (j < nsteps) {
        issue_w(ks_b + j, j);
        issue_a(ks_b + j, j);
      }
    for (int j = 0; j < nsteps; ++j) {
      // this wave's copies of step j have landed once at most the copies of the steps issued
      // after it are outstanding (copies complete in issue order); the barrier then publishes
      // every wave's copies, and retires every wave's reads of the stage the next copies overwrite
      const int after = min(NS - 2, nsteps - 1 - j);
      if (after >= 2)
        wait_vmcnt<2 * P>();
      else if (after == 1)
        wait_vmcnt<P>();
      else
        wait_vmcnt<0>();
      __syncthreads();
      if (j + NS - 1 < nsteps) {
        issue_w(ks_b + j + NS - 1, (j + NS - 1) % NS);
        issue_a(ks_b + j + NS - 1, (j + NS - 1) % NS);
      }
      const int ks = ks_b + j;
      const bool full = int64_t(ks) * 128 + 128 <= a.K;
      if (tl == TM) {
        if (full) compute(ks, j % NS, std::integral_constant<int, TM>{}, std::true_type{});
        else compute(ks, j % NS, std::integral_constant<int, TM>{}, std::false_type{});
      } else if (TM == 2 && tl == 1) {
        if (full) compute(ks, j % NS, std::integral_constant<int, 1>{}, std::true_type{});
        else compute(ks, j % NS, std::integral_constant<int, 1>{}, std::false_type{});
      }
    }

    // ---- epilogue: the tile goes through LDS (free once every wave is past its last products)
    // and leaves as 16-byte row chunks; K-split chunks write fp32 partial sums to their own
    // slice, the bias rides on chunk 0
    constexpr int OE = OUT_F32 ? 4 : 2;
    constexpr int OROW = BN + (OUT_F32 ? 4 : 8);
    constexpr int CH = 16 / OE;
    static_assert(size_t(BM) * OROW * OE <= size_t(NS) * STAGE, "staged output fits the operand stages");
    uint8_t* const obase = static_cast<uint8_t*>(a.out) + (nsplit > 1 ? split * a.split_stride * OE : 0);
    const float tscale = WFMT == W_E4M3_TENSOR ? reinterpret_cast<const float*>(a.ws)[0] : 1.f;
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int cl = wn * WN + 16 * j + frow;
      const int64_t col = pair ? group_row0(cl >> 4) + (cl & 15) : n0 + cl;  // the weight row
      const float b = HAS_BIAS && split == 0 && col < a.N ? load_bias(a, expert, col) : 0.f;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = wm * WM + 16 * i + 4 * fq + r;
          float v = (WFMT == W_E4M3_TENSOR ? acc[i][j][r] * tscale : acc[i][j][r]) + b;
          // the top-1 combine, as the combine kernel evaluates it (an fma onto +0)
          if (MODE == ROWS_COMPACT_IN && !OUT_F32 && a.top1_w) v = fmaf(sWt[rl], v, 0.f);
          if (OUT_F32)
            reinterpret_cast<float*>(lds)[rl * OROW + cl] = v;
          else
            reinterpret_cast<uint16_t*>(lds)[rl * OROW + cl] = f2bf(v);
        }
    }
    __syncthreads();
    if (!OUT_F32 && pair) {
      // staged row: the bf16 ic0 values of gate columns [0, 64) and up columns [64, 128); out =
      // ic1 [rows, I], 8 outputs per 16-byte chunk
      for (int c = tid; c < m_size * 8; c += NT) {
        const int rl = c >> 3, ch = c & 7;
        const uint8_t* src = lds + (rl * OROW + ch * 8) * 2;
        const uint4 h = silu_mul8(*reinterpret_cast<const uint4*>(src), *reinterpret_cast<const uint4*>(src + 128));
        *reinterpret_cast<uint4*>(obase + (sOrow[rl] * a.ldo + 64 * nt + ch * 8) * 2) = h;
      }
      continue;  // next row pass (its first barrier orders these LDS reads before new writes)
    }
    const int64_t ncols = min<int64_t>(BN, a.N - n0);
    for (int c = tid; c < m_size * (BN / CH); c += NT) {
      const int rl = c / (BN / CH), ch = c % (BN / CH);
      const int64_t col = n0 + ch * CH;
      uint8_t* dst = obase + (sOrow[rl] * a.ldo + col) * OE;
      const uint8_t* src = lds + (rl * OROW + ch * CH) * OE;
      if (ch * CH + CH <= ncols) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int e = 0; e < CH * OE && ch * CH + e / OE < ncols; ++e) dst[e] = src[e];
      }
    }
  }  // row passes
}

// One tile of a class's work list: entry `tile`, column tile nt, K chunk split (K chunk
// fastest-varying, then the entry, then the column tile).
template <int BM, int MODE, int WFMT, bool OUT_F32, bool HAS_BIAS, bool TILED>
__device__ __forceinline__ void ring_tile(const GemmArgs& a, int64_t grid_blocks, int64_t bid, uint8_t* lds) {
  const int nsplit = a.k_split > 1 ? a.k_split : 1;
  const int split = int(bid % nsplit);
  const int64_t rest = bid / nsplit;
  const int64_t tile = rest % grid_blocks;
  const int64_t nt = rest / grid_blocks;
  if (nt * 128 >= a.N) return;
  TileInfo t;
  if (!tile_info<BM, MODE>(a, tile, t)) return;
  ring_body<BM, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(a, t, nt, split, lds, nullptr);
}

// Routed tile classes 16 / 32 / 64 / 128 rows in one launch; launch order 128, 64, 32, 16 rows
// (the longest tiles start first).
struct RingGroup {
  GemmArgs a[4];   // per class (16, 32, 64, 128 rows): the stage's arguments with its work list
  int64_t gb[4];   // per class: work-list capacity
  int64_t off[5];  // launch order 128, 64, 32, 16 rows: off[0] = 0, off[4] = grid size
};

template <int MODE, int WFMT, bool OUT_F32, bool HAS_BIAS, bool TILED>
__global__ __launch_bounds__(kRingThreads) void gemm_w16_ring_kernel(RingGroup g) {
  extern __shared__ __align__(1024) uint8_t ring_lds[];
  const int64_t b = blockIdx.x;
  if (b < g.off[1])
    ring_tile<128, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(g.a[3], g.gb[3], b - g.off[0], ring_lds);
  else if (b < g.off[2])
    ring_tile<64, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(g.a[2], g.gb[2], b - g.off[1], ring_lds);
  else if (b < g.off[3])
    ring_tile<32, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(g.a[1], g.gb[1], b - g.off[2], ring_lds);
  else
    ring_tile<16, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(g.a[0], g.gb[0], b - g.off[3], ring_lds);
}

// Self-routed small routings: workgroup (block, column tile, K chunk) -- K chunk fastest, then
// the column tile, then the block in the sort's order -- finds its block from the routing ids,
// then runs the tile class the block's row count picks.  Workgroups past the routing's blocks
// exit after the lookup; they come last in the grid, so a grid larger than the GPU holds never
// keeps a live workgroup waiting behind them.
template <int MODE, int WFMT, bool OUT_F32, bool HAS_BIAS, bool TILED>
__global__ __launch_bounds__(kRingThreads) void gemm_w16_ring_routed_kernel(GemmArgs a) {
  extern __shared__ __align__(1024) uint8_t ring_lds[];
  __shared__ int32_t s_rows[128];
  __shared__ int32_t s_pick[5];
  const int nsplit = a.k_split > 1 ? a.k_split : 1;
  const int64_t b = blockIdx.x;
  const int split = int(b % nsplit);
  const int64_t rest = b / nsplit;
  const int64_t n_tiles = cdiv(a.N, int64_t(128));
  const int64_t nt = rest % n_tiles;
  const int64_t blk = rest / n_tiles;
  TileInfo t;
  const int c = self_route_block(a.rt, blk, t, reinterpret_cast<int32_t*>(ring_lds), s_rows, s_pick);
  if (MODE == ROWS_COMPACT_IN && !OUT_F32 && a.top1_w && blk == 0 && split == 0) {
    // top-1 fold: the first block's workgroup of each column tile zeroes that tile's columns of
    // the tokens whose id was dropped (the lookup left each row's expert, -1 when dropped, in
    // the first R ints of the scratch); the barrier keeps those reads ahead of the tile's copies
    const int32_t* s_ids = reinterpret_cast<const int32_t*>(ring_lds);
    const int64_t n0 = nt * 128, ncols = min<int64_t>(128, a.N - n0);
    for (int e = threadIdx.x; e < a.rt.route_R * 16; e += kRingThreads) {
      const int r = e >> 4, ch = e & 15;
      if (s_ids[r] >= 0 || ch * 8 >= ncols) continue;
      uint16_t* o = static_cast<uint16_t*>(a.out) + int64_t(r) * a.ldo + n0 + ch * 8;
      if (ch * 8 + 8 <= ncols)
        *reinterpret_cast<uint4*>(o) = make_uint4(0, 0, 0, 0);
      else
        for (int k = 0; ch * 8 + k < ncols; ++k) o[k] = 0;
    }
    __syncthreads();
  }
  if (c < 0) return;
  if (c >= 4)
    ring_body<128, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(a, t, nt, split, ring_lds, s_rows);
  else if (c == 3)
    ring_body<64, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(a, t, nt, split, ring_lds, s_rows);
  else if (c == 2)
    ring_body<32, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(a, t, nt, split, ring_lds, s_rows);
  else
    ring_body<16, MODE, WFMT, OUT_F32, HAS_BIAS, TILED>(a, t, nt, split, ring_lds, s_rows);
}

// Dense per-tensor W8A16 products (bf16 out): row tile fastest, then the column tile; batch
// entry z = blockIdx.y reads A + z a_bstride, W + z w_estride, ws + z ws_estride, bias +
// z bias_estride and writes out + z o_bstride.
// (OUT_F32: a K split, chunk blockIdx.z, fp32 partial sums to the chunk's slice of out)
template <int BM, bool HAS_BIAS, bool OUT_F32 = false>
__global__ __launch_bounds__(kRingThreads) void gemm_w16_ring_dense_kernel(GemmArgs a, int64_t grid_blocks) {
  extern __shared__ __align__(1024) uint8_t ring_lds[];
  const int64_t z = blockIdx.y;
  a.A = static_cast<const uint16_t*>(a.A) + z * a.a_bstride;
  a.W += z * a.w_estride;
  a.ws = static_cast<const float*>(a.ws) + z * a.ws_estride;
  if (HAS_BIAS) a.bias = static_cast<const uint8_t*>(a.bias) + z * a.bias_estride * (a.bias_bf16 ? 2 : 4);
  a.out = static_cast<uint16_t*>(a.out) + z * a.o_bstride;
  const int64_t tile = blockIdx.x % grid_blocks, nt = blockIdx.x / grid_blocks;
  TileInfo t;
  if (!tile_info<BM, ROWS_DENSE>(a, tile, t)) return;
  ring_body<BM, ROWS_DENSE, W_E4M3_TENSOR, OUT_F32, HAS_BIAS, false>(a, t, nt, OUT_F32 ? int(blockIdx.z) : 0, ring_lds,
                                                                     nullptr);
}

template <int MODE, int WFMT, bool TL>
static void launch_ring_t(const RingGroup& g, bool out_f32, hipStream_t st) {
  size_t lds = 0;
  const size_t f32[4] = {ring_lds_bytes<128, WFMT, true>(), ring_lds_bytes<64, WFMT, true>(),
                         ring_lds_bytes<32, WFMT, true>(), ring_lds_bytes<16, WFMT, true>()};
  const size_t b16[4] = {ring_lds_bytes<128, WFMT, false>(), ring_lds_bytes<64, WFMT, false>(),
                         ring_lds_bytes<32, WFMT, false>(), ring_lds_bytes<16, WFMT, false>()};
  for (int i = 0; i < 4; ++i)
    if (g.off[i + 1] > g.off[i]) lds = std::max(lds, out_f32 ? f32[i] : b16[i]);
  const dim3 grid(unsigned(g.off[4])), block(kRingThreads);
  const bool bias = g.a[0].bias != nullptr;
#define MXQ_RING_GO(OF, HB) \
  hipLaunchKernelGGL((gemm_w16_ring_kernel<MODE, WFMT, OF, HB, TL>), grid, block, lds, st, g)
  if (out_f32) { if (bias) MXQ_RING_GO(true, true); else MXQ_RING_GO(true, false); }
  else { if (bias) MXQ_RING_GO(false, true); else MXQ_RING_GO(false, false); }
#undef MXQ_RING_GO
}

// live[i]: tile class i (16, 32, 64, 128 rows) can occur
template <int MODE, int WFMT, bool TL>
static void launch_ring_routed_t(const GemmArgs& g, int64_t max_blocks, const bool live[4], bool out_f32,
                                 hipStream_t st) {
  const size_t f32[4] = {ring_lds_bytes<16, WFMT, true>(), ring_lds_bytes<32, WFMT, true>(),
                         ring_lds_bytes<64, WFMT, true>(), ring_lds_bytes<128, WFMT, true>()};
  const size_t b16[4] = {ring_lds_bytes<16, WFMT, false>(), ring_lds_bytes<32, WFMT, false>(),
                         ring_lds_bytes<64, WFMT, false>(), ring_lds_bytes<128, WFMT, false>()};
  // the lookup keeps R + E + 24 routing ints in the same LDS
  size_t lds = sizeof(int32_t) * (size_t(g.rt.route_R) + size_t(g.rt.route_E) + 3 * (kRingThreads / 64));
  for (int i = 0; i < 4; ++i)
    if (live[i]) lds = std::max(lds, out_f32 ? f32[i] : b16[i]);
  const int64_t nblocks = max_blocks * cdiv(g.N, int64_t(128)) * std::max<int64_t>(g.k_split, 1);
  const dim3 grid{unsigned(nblocks)}, block{unsigned(kRingThreads)};
  const bool bias = g.bias != nullptr;
#define MXQ_RING_GO(OF, HB) \
  hipLaunchKernelGGL((gemm_w16_ring_routed_kernel<MODE, WFMT, OF, HB, TL>), grid, block, lds, st, g)
  if (out_f32) { if (bias) MXQ_RING_GO(true, true); else MXQ_RING_GO(true, false); }
  else { if (bias) MXQ_RING_GO(false, true); else MXQ_RING_GO(false, false); }
#undef MXQ_RING_GO
}

template <int MODE, int WFMT>
static void launch_ring_m(const RingGroup& g, bool out_f32, hipStream_t st) {
  if (g.a[0].w_tiled)
    launch_ring_t<MODE, WFMT, true>(g, out_f32, st);
  else
    launch_ring_t<MODE, WFMT, false>(g, out_f32, st);
}

bool w16_ring_shape_ok(const GemmArgs& a, int wfmt) {
  if (wfmt != W_E4M3_BLOCK && wfmt != W_E2M1_MX) return false;
  if (a.K <= 0 || a.K % 32 != 0 || a.K > int64_t(kRingMaxSteps) * 128) return false;
  if ((reinterpret_cast<uintptr_t>(a.A) & 15) != 0 || a.lda % 8 != 0) return false;
  return wfmt != W_E4M3_BLOCK || a.block_n == 128;
}

bool w16_ring_supported(const GemmArgs& a, int wfmt) {
  if (!w16_ring_shape_ok(a, wfmt)) return false;
  if (a.w_tiled) return a.N % 16 == 0;
  if ((reinterpret_cast<uintptr_t>(a.W) & 15) != 0 || a.ldw % 16 != 0 || a.w_estride % 16 != 0) return false;
  // plain e8m0 scales: one aligned dword per row per K step
  if (wfmt == W_E2M1_MX && (a.K % 128 != 0 || a.ws_s0 % 4 != 0 || a.ws_estride % 4 != 0 ||
                            (reinterpret_cast<uintptr_t>(a.ws) & 3) != 0))
    return false;
  return true;
}

void launch_gemm_w16_ring(const GemmArgs cls[4], const int64_t grid_blocks[4], int wfmt, int row_mode,
                          bool out_f32, hipStream_t stream) {
  RingGroup g{};
  for (int c = 0; c < 4; ++c) {
    g.a[c] = cls[c];
    g.gb[c] = std::max<int64_t>(grid_blocks[c], 0);
  }
  for (int i = 0; i < 4; ++i) {  // launch order: 128-, 64-, 32-, 16-row class
    const int c = 3 - i;
    g.off[i + 1] = g.off[i] + g.gb[c] * cdiv(cls[c].N, int64_t(128)) * std::max<int64_t>(cls[c].k_split, 1);
  }
  if (g.off[4] <= 0) return;
  const bool mx = wfmt == W_E2M1_MX;
  if (row_mode == ROWS_GATHER_TOK) {
    if (mx) launch_ring_m<ROWS_GATHER_TOK, W_E2M1_MX>(g, out_f32, stream);
    else launch_ring_m<ROWS_GATHER_TOK, W_E4M3_BLOCK>(g, out_f32, stream);
  } else {
    if (mx) launch_ring_m<ROWS_COMPACT_IN, W_E2M1_MX>(g, out_f32, stream);
    else launch_ring_m<ROWS_COMPACT_IN, W_E4M3_BLOCK>(g, out_f32, stream);
  }
}

void launch_gemm_w16_ring_routed(const GemmArgs& g, int64_t max_blocks, const bool live[4], int wfmt, int row_mode,
                                 bool out_f32, hipStream_t stream) {
  if (max_blocks <= 0 || g.N <= 0) return;
  const bool mx = wfmt == W_E2M1_MX;
#define MXQ_ROUTED(MODE, WF)                                                  \
  do {                                                                        \
    if (g.w_tiled) launch_ring_routed_t<MODE, WF, true>(g, max_blocks, live, out_f32, stream);   \
    else launch_ring_routed_t<MODE, WF, false>(g, max_blocks, live, out_f32, stream);            \
  } while (0)
  if (row_mode == ROWS_GATHER_TOK) {
    if (mx) MXQ_ROUTED(ROWS_GATHER_TOK, W_E2M1_MX);
    else MXQ_ROUTED(ROWS_GATHER_TOK, W_E4M3_BLOCK);
  } else {
    if (mx) MXQ_ROUTED(ROWS_COMPACT_IN, W_E2M1_MX);
    else MXQ_ROUTED(ROWS_COMPACT_IN, W_E4M3_BLOCK);
  }
#undef MXQ_ROUTED
}

bool w16_ring_dense_supported(const GemmArgs& a, int64_t batch) {
  const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (a.K <= 0 || a.K % 32 != 0 || a.N <= 0 || a.M <= 0) return false;
  if (!al16(a.A) || a.lda % 8 != 0 || !al16(a.W) || a.ldw % 16 != 0 || !al16(a.out) || a.ldo % 8 != 0) return false;
  return batch <= 1 || (a.a_bstride % 8 == 0 && a.w_estride % 16 == 0 && a.o_bstride % 8 == 0);
}

template <int BM>
static void launch_ring_dense_t(const GemmArgs& a, int64_t batch, hipStream_t st) {
  const int64_t gb = cdiv(a.M, int64_t(BM));
  // a K split (one 2-D product: batch 1) runs its chunks along the grid's third dimension
  const unsigned chunks = batch == 1 && a.k_split > 1 ? unsigned(a.k_split) : 1u;
  const dim3 grid{unsigned(gb * cdiv(a.N, int64_t(128))), unsigned(batch), chunks}, block{unsigned(kRingThreads)};
  if (chunks > 1) {
    const size_t lds = ring_lds_bytes<BM, W_E4M3_TENSOR, true>();
    if (a.bias)
      hipLaunchKernelGGL((gemm_w16_ring_dense_kernel<BM, true, true>), grid, block, lds, st, a, gb);
    else
      hipLaunchKernelGGL((gemm_w16_ring_dense_kernel<BM, false, true>), grid, block, lds, st, a, gb);
    return;
  }
  const size_t lds = ring_lds_bytes<BM, W_E4M3_TENSOR, false>();
  if (a.bias)
    hipLaunchKernelGGL((gemm_w16_ring_dense_kernel<BM, true>), grid, block, lds, st, a, gb);
  else
    hipLaunchKernelGGL((gemm_w16_ring_dense_kernel<BM, false>), grid, block, lds, st, a, gb);
}

void launch_gemm_w16_ring_dense(const GemmArgs& a, int tile, int64_t batch, hipStream_t stream) {
  if (batch <= 0 || a.M <= 0 || a.N <= 0) return;
  switch (tile) {
    case 0: launch_ring_dense_t<128>(a, batch, stream); break;
    case 1: launch_ring_dense_t<64>(a, batch, stream); break;
    case 2: launch_ring_dense_t<32>(a, batch, stream); break;
    default: launch_ring_dense_t<16>(a, batch, stream); break;
  }
}

}  // namespace mxq
