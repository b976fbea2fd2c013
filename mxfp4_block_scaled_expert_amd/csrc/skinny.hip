// Weight-streaming kernel for tiny routed expert blocks (at most 4 rows) on gfx950.
//
// "vLLM PR 50949 review" (implementation items 1-2, gemm.h listing): an expert
// block with few rows wants a fixed-row micro-kernel, not a large tile.  Such a
// block is bound by reading its expert's weights once, so this kernel is built
// around streaming them at HBM speed:
//
//  * each wave owns 16 weight rows and walks K in steps of 128 bytes per row;
//    lane (row r = lane % 16, q = lane / 16) loads the 32 contiguous bytes
//    [32q, 32q + 32) of row r's step straight into registers (whole 128-byte
//    lines per four lanes), through a 4-deep register ring, so ~6 KB per wave
//    are in flight and the weights never touch LDS;
//  * each 32-element K slice is one V_MFMA_F32_16X16X32_BF16.  The MFMA sums
//    over whatever K elements a lane supplies as long as both operands use the
//    same assignment, so slice s of lane group q takes the lane's own bytes
//    (elements 32q + 8s .. +8 of an e4m3 step, 64q + 8s .. +8 of an e2m1 step)
//    and the activation operand reads the same elements from LDS;
//  * weights are decoded to bf16 in registers (e4m3 exactly; e2m1 with its
//    e8m0 scale folded in), activation rows 4..15 of the MFMA are zero, and the
//    vector ALU only decodes: the K reduction happens in the matrix core;
//  * e4m3 block weights are promoted per 128-wide K block with their fp32
//    scale (times the per-token activation scale for W8A8); MXFP4 needs none.
#include "tile_rows.hpp"

namespace mxq {

namespace {
constexpr int kSkRows = 16;   // weight rows per wave
constexpr int kSkWaves = 4;
constexpr int kSkTileN = kSkRows * kSkWaves;
constexpr int kSkDepth = 4;   // register ring depth (steps)
constexpr int kSkActRows = 4;
}  // namespace

template <int WFMT, bool A_E4M3, int MODE, bool OUT_F32, bool HAS_BIAS>
__global__ __launch_bounds__(256) void skinny_kernel(GemmArgs a, int64_t grid_blocks) {
  constexpr bool MX = WFMT == W_E2M1_MX;
  constexpr int KSTEP = MX ? 256 : 128;  // K elements per 128-byte row step
  constexpr int SUBS = KSTEP / 32;       // MFMA K slices per step
  constexpr int EPL = KSTEP / 4;         // K elements per lane per step
  constexpr int AE = A_E4M3 ? 1 : 2;     // activation bytes per element

  extern __shared__ __align__(16) uint8_t smem[];
  float* s_sa = reinterpret_cast<float*>(smem);                 // W8A8: [4][K/128]
  uint8_t* act = smem + (A_E4M3 ? kSkActRows * ((a.K >> 7) + 4) * 4 : 0);  // [4][K] activations
  __shared__ int64_t s_arow[kSkActRows];
  __shared__ int64_t s_orow[kSkActRows];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t tile = blockIdx.x % grid_blocks;
  const int64_t nt = blockIdx.x / grid_blocks;
  const int64_t n0 = nt * kSkTileN;
  if (n0 >= a.N) return;
  TileInfo t;
  if (!tile_info<1, MODE>(a, tile, t)) return;
  const int64_t expert = t.expert;
  const int64_t K = a.K;
  const int nsteps = int(cdiv(K, KSTEP));
  const int KB = int(K >> 7);
  const int64_t nw = n0 + wave * kSkRows;
  const int64_t nrow = min<int64_t>(nw + l16, a.N - 1);
  const uint8_t* wrow = a.W + expert * a.w_estride + nrow * a.ldw;
  const int64_t row_bytes = MX ? K / 2 : K;
  const uint8_t* srow = MX ? reinterpret_cast<const uint8_t*>(a.ws) + expert * a.ws_estride + nrow * a.ws_s0 : nullptr;
  const float* swf = reinterpret_cast<const float*>(a.ws) + expert * a.ws_estride +
                     (min<int64_t>(nw, a.N - 1) >> 7) * a.ws_s0;

  for (int m_base = 0; m_base < t.m_total; m_base += kSkActRows) {
    const int m_size = min(kSkActRows, t.m_total - m_base);
    __syncthreads();
    if (tid < kSkActRows) {
      int64_t ar, orw;
      row_of<MODE>(a, t, m_base + min(tid, m_size - 1), ar, orw);
      s_arow[tid] = ar;
      s_orow[tid] = orw;
    }
    __syncthreads();
    // ---- stage the activation rows (and their per-token scales for W8A8) in LDS
    {
      const int64_t chunks = K * AE / 16;
      for (int64_t c = tid; c < kSkActRows * chunks; c += blockDim.x) {
        const int m = int(c / chunks);
        const int64_t cc = c - m * chunks;
        const uint8_t* g = reinterpret_cast<const uint8_t*>(a.A) + s_arow[m] * a.lda * AE + cc * 16;
        *reinterpret_cast<i32x4*>(act + m * K * AE + cc * 16) = *reinterpret_cast<const i32x4*>(g);
      }
      if (A_E4M3)
        for (int c = tid; c < kSkActRows * KB; c += blockDim.x) {
          const int m = c / KB, kb = c - m * KB;
          s_sa[m * KB + kb] = a.sa[s_arow[m] * a.lds + kb];
        }
    }
    __syncthreads();

    // ---- stream the wave's 16 weight rows through a register ring
    i32x4 wb[kSkDepth][2];
    uint32_t sb[kSkDepth][2];  // raw e8m0 bytes, combined only where used
    float swr[kSkDepth];
    auto load = [&](int st, int slot) __attribute__((always_inline)) {
      // 16-byte halves wholly past the row end (K tail) fetch the row's first line instead
      const int64_t off = int64_t(st) * 128 + q * 32;
      wb[slot][0] = *reinterpret_cast<const i32x4*>(wrow + (off + 16 <= row_bytes ? off : 0));
      wb[slot][1] = *reinterpret_cast<const i32x4*>(wrow + (off + 32 <= row_bytes ? off + 16 : 0));
      if (MX) {
        // this lane's two 32-element groups; indices past the row are clamped (never
        // branched around: a load under a branch would make the compiler drain the ring)
        const int64_t grp = int64_t(st) * 8 + 2 * q;
        const int64_t ng = row_bytes / 16;
        sb[slot][0] = srow[min(grp, ng - 1)];
        sb[slot][1] = srow[min(grp + 1, ng - 1)];
      } else {
        swr[slot] = swf[min(st, KB - 1) * a.ws_s1];
      }
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const bool arow_ok = l16 < m_size;
    const uint8_t* arow_lds = act + (arow_ok ? l16 : 0) * K * AE;
    auto compute = [&](int st, int slot) __attribute__((always_inline)) {
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < SUBS; ++s) {
        const int64_t k0 = int64_t(st) * KSTEP + q * EPL + 8 * s;
        // a lane's 8 elements lie wholly inside or wholly past K (K % 32 == 0)
        const bool kin = k0 + 8 <= K;
        i32x4 af = {0, 0, 0, 0};
        if (arow_ok && kin) {
          if (A_E4M3) {
            const uint2 v = *reinterpret_cast<const uint2*>(arow_lds + k0);
            uint32_t o0, o1, o2, o3;
            e4m3x4_to_bf16(v.x, o0, o1);
            e4m3x4_to_bf16(v.y, o2, o3);
            af = i32x4{int(o0), int(o1), int(o2), int(o3)};
          } else {
            af = *reinterpret_cast<const i32x4*>(arow_lds + k0 * 2);
          }
        }
        i32x4 bfr;
        if (MX) {
          const float sc = e8m0_to_f32(sb[slot][s >> 2]);
          uint32_t o[4];
          e2m1x8_to_bf16(uint32_t(wb[slot][s >> 2][s & 3]), sc, o);
          bfr = i32x4{int(o[0]), int(o[1]), int(o[2]), int(o[3])};
        } else {
          uint32_t o0, o1, o2, o3;
          e4m3x4_to_bf16(uint32_t(wb[slot][s >> 1][(2 * s) & 3]), o0, o1);
          e4m3x4_to_bf16(uint32_t(wb[slot][s >> 1][(2 * s + 1) & 3]), o2, o3);
          bfr = i32x4{int(o0), int(o1), int(o2), int(o3)};
        }
        if (MX)
          acc = mfma_16x16x32_bf16(af, bfr, acc);
        else
          part = mfma_16x16x32_bf16(af, bfr, part);
      }
      if (!MX) {
        const float sw = swr[slot];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float c = sw;
          if (A_E4M3) {
            const int m = 4 * q + r;
            c *= (m < m_size) ? s_sa[(m < kSkActRows ? m : 0) * KB + st] : 0.f;
          }
          acc[r] = fmaf(part[r], c, acc[r]);
        }
      }
    };

    // Loads are issued unconditionally (steps past the end read valid dummy addresses) and
    // the loop has no early exit, so the wait before each step's compute counts only the
    // newer steps' loads and the ring stays full.
#pragma unroll
    for (int u = 0; u < kSkDepth - 1; ++u) load(u, u);
    for (int st0 = 0; st0 < nsteps; st0 += kSkDepth) {
#pragma unroll
      for (int u = 0; u < kSkDepth; ++u) {
        load(st0 + u + kSkDepth - 1, (u + kSkDepth - 1) % kSkDepth);
        if (st0 + u < nsteps) compute(st0 + u, u);
      }
    }

    // ---- epilogue: lane holds D[m = 4q + r][n = l16]
    const int64_t col = nw + l16;
    if (col < a.N) {
      const float b = HAS_BIAS ? load_bias(a, expert, col) : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * q + r;
        if (m >= m_size) continue;
        const int64_t o = s_orow[m] * a.ldo + col;
        const float v = acc[r] + b;
        if (OUT_F32)
          reinterpret_cast<float*>(a.out)[o] = v;
        else
          reinterpret_cast<uint16_t*>(a.out)[o] = f2bf(v);
      }
    }
  }
}

size_t skinny_lds_bytes(bool a_e4m3, int64_t K) {
  return size_t(kSkActRows) * size_t(K) * (a_e4m3 ? 1 : 2) +
         (a_e4m3 ? size_t(kSkActRows) * size_t((K >> 7) + 4) * 4 : 0);
}

template <int WFMT, bool AE, int MODE>
static void launch_skinny_t(const GemmArgs& a, bool out_f32, int64_t gb, hipStream_t st) {
  const int64_t n_tiles = cdiv(a.N, kSkTileN);
  const dim3 grid(static_cast<unsigned>(gb * n_tiles)), block(256);
  const size_t lds = skinny_lds_bytes(AE, a.K);
  const bool bias = a.bias != nullptr;
#define MXQ_SK_GO(OF, HB) hipLaunchKernelGGL((skinny_kernel<WFMT, AE, MODE, OF, HB>), grid, block, lds, st, a, gb)
  if (out_f32) { if (bias) MXQ_SK_GO(true, true); else MXQ_SK_GO(true, false); }
  else { if (bias) MXQ_SK_GO(false, true); else MXQ_SK_GO(false, false); }
#undef MXQ_SK_GO
}

template <int MODE>
static void launch_skinny_mode(const GemmArgs& a, int wfmt, bool a_e4m3, bool out_f32, int64_t gb, hipStream_t st) {
  if (wfmt == W_E2M1_MX)
    launch_skinny_t<W_E2M1_MX, false, MODE>(a, out_f32, gb, st);
  else if (a_e4m3)
    launch_skinny_t<W_E4M3_BLOCK, true, MODE>(a, out_f32, gb, st);
  else
    launch_skinny_t<W_E4M3_BLOCK, false, MODE>(a, out_f32, gb, st);
}

void launch_skinny(const GemmArgs& a, int wfmt, bool a_e4m3, int row_mode, bool out_f32, int64_t grid_blocks,
                   hipStream_t stream) {
  if (grid_blocks <= 0 || a.N <= 0) return;
  if (row_mode == ROWS_GATHER_TOK)
    launch_skinny_mode<ROWS_GATHER_TOK>(a, wfmt, a_e4m3, out_f32, grid_blocks, stream);
  else
    launch_skinny_mode<ROWS_COMPACT_IN>(a, wfmt, a_e4m3, out_f32, grid_blocks, stream);
}

}  // namespace mxq
