// Weight-streaming kernel for tiny routed expert blocks on gfx950.
//
// "vLLM PR 50949 review" (implementation items 1-2, gemm.h listing): an expert
// block with few rows wants a fixed-row micro-kernel, not a large tile.  Such a
// block is bound by reading its expert's weights once, so this kernel is built
// around streaming them at HBM speed:
//
//  * a workgroup owns 64 * G weight rows of one expert block; wave w owns the
//    16-row groups w, w + 4, ..., and walks K in steps of 128 bytes per row,
//    K-outer: each step loads the step's bytes of all G groups, so one
//    activation fragment read from LDS feeds G MFMAs;
//  * lane (r = lane % 16, q = lane / 16) loads bytes [32q, 32q + 32) of row r's
//    step straight into registers through a D-deep ring (no LDS for weights);
//    loads are issued unconditionally (past-the-end steps read a valid dummy
//    address) so the compiler's wait before a step counts only newer loads;
//  * the first D - 1 steps are requested before the activation rows are staged,
//    so the staging latency overlaps the weight stream;
//  * e2m1 (MXFP4) and e4m3 weights with bf16 activations are decoded to bf16 and
//    reduced by V_MFMA_F32_16X16X32_BF16 (e8m0 scale folded into the decode;
//    e4m3 block scales applied per 128-wide K block); with e4m3 activations
//    (W8A8) both operands go to V_MFMA_F32_16X16X128_F8F6F4 undecoded and the
//    two block scales are applied per K block;
//  * MFMA rows past the block's row count read activation row 0 and are never
//    stored, so the loop needs no lane masking; activation rows are zero-padded
//    in LDS to a whole number of steps, which covers a ragged K tail;
//  * AR activation rows (4 or 8) are staged per pass; a taller block takes
//    several passes over the same weights;
//  * with weights in the tiled layout (prepack.hip) a step of one 16-row group
//    is 2 KB of contiguous memory, so each 64-lane load reads 1 KB in one piece;
//    the plain layout reads 16 rows x 64 bytes per load instead.
#include "quant_common.hpp"
#include "tile_rows.hpp"

namespace mxq {

namespace {
constexpr int kSkWaves = 4;
constexpr int kSkMaxRows = 8;

// Waves per SIMD the register budget targets, per weight format: MXFP4 (decode work per step
// is larger) 3, e4m3 4; chosen by measurement on the decode workloads, no register spills at
// these budgets.  Groups per wave and ring depth: G = 2, D = 3 for outputs of at least
// MXQ_SK_GSEL rows, else G = 1, D = 4 (see skinny_groups).
#ifndef MXQ_SK_MXW
#define MXQ_SK_MXW 3
#endif
#ifndef MXQ_SK_GSEL
#define MXQ_SK_GSEL 4096
#endif
template <int WFMT, bool AE>
struct SkinnyShape {
  static constexpr int W = WFMT == W_E2M1_MX ? MXQ_SK_MXW : 4;
};
}  // namespace

// LDS layout (bytes): activation rows [AR][row_stride] | weight scales [K/128][nb] | act scales [K/128][AR].
// A row holds the workgroup's own K range: kstage elements (a K chunk when K is split; 0: all of K).
struct SkinnyLds {
  int row_stride, kpad, kb, nb;
  uint32_t sw_off, sa_off, total;
};

// swcol: per-column weight scales (1 x 128 blocks) of the staged K steps, [steps][64 G]
__host__ __device__ inline SkinnyLds skinny_lds_layout(bool mx, bool a_e4m3, int64_t K, int G, int AR,
                                                      int64_t kstage = 0, bool swcol = false) {
  SkinnyLds L;
  const int kstep = mx ? 256 : 128;
  const int ae = a_e4m3 ? 1 : 2;
  L.kpad = int((K + kstep - 1) / kstep) * kstep;
  const int64_t ks = kstage > 0 && kstage < L.kpad ? kstage : L.kpad;
  L.row_stride = int((ks + kstep - 1) / kstep) * kstep * ae + 16;  // +16 B: rows read together fall in different banks
  L.kb = int(K >> 7);
  L.nb = G >= 2 ? G / 2 : 1;
  L.sw_off = uint32_t(AR * L.row_stride);
  const uint32_t sw_bytes = mx ? 0u : swcol ? uint32_t((L.row_stride - 16) / (kstep * ae) * 64 * G * 4)
                                              : uint32_t(L.kb * L.nb * 4);
  L.sa_off = (L.sw_off + sw_bytes + 15u) & ~15u;
  L.total = L.sa_off + (a_e4m3 ? uint32_t(L.kb * AR * 4) : 0u);
  return L;
}

template <int WFMT, bool A_E4M3, int MODE, bool OUT_F32, bool HAS_BIAS, bool TILED, int AR, int G, int D,
          bool SWCOL = false>
__global__ __launch_bounds__(256, (SkinnyShape<WFMT, A_E4M3>::W)) void skinny_kernel(GemmArgs a,
                                                                                     int64_t grid_blocks) {
  constexpr bool MX = WFMT == W_E2M1_MX;
  constexpr int KSTEP = MX ? 256 : 128;  // K elements per 128-byte row step
  constexpr int AE = A_E4M3 ? 1 : 2;     // activation bytes per element
  static_assert(!(MX && A_E4M3), "MXFP4 weights take bf16 activations");
  static_assert(AR == 4 || AR == 8, "four or eight activation rows per pass");

  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int64_t s_arow[AR];
  __shared__ int64_t s_orow[AR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t N = a.N, K = a.K;
  const int64_t ntiles = (N + 64 * G - 1) / (64 * G);
  // K split fastest (a tile's chunks run side by side), then n-tile: concurrently running
  // workgroups stream adjacent parts of one expert
  const int nsplit = a.k_split > 1 ? a.k_split : 1;
  const int split = int(blockIdx.x % unsigned(nsplit));
  const int64_t rest = blockIdx.x / unsigned(nsplit);
  const int64_t tile = rest / ntiles;
  const int64_t nt = rest - tile * ntiles;
  if (tile >= grid_blocks) return;
  TileInfo t;
  // dense: a tile is AR consecutive rows (one pass); routed: a tile is one expert block
  if (!tile_info<(MODE == ROWS_DENSE ? AR : 1), MODE>(a, tile, t)) return;

  static_assert(!SWCOL || (A_E4M3 && !MX && MODE == ROWS_DENSE), "per-column weight scales: dense W8A8 rows");
  const SkinnyLds L = skinny_lds_layout(MX, A_E4M3, K, G, AR, nsplit > 1 ? a.k_chunk : 0, SWCOL);
  const int nsteps = L.kpad / KSTEP;
  // this workgroup's K steps [st_b, st_e); an empty range (a chunk past K) stores zeros
  int st_b = 0, st_e = nsteps;
  if (nsplit > 1) {
    const int cs = int(a.k_chunk / KSTEP);
    st_b = min(nsteps, split * cs);
    st_e = min(nsteps, st_b + cs);
  }
  const int st_last = max(st_e, 1) - 1;  // loads past the range re-read its last step
  const int64_t n0 = nt * 64 * G;
  const int64_t row_bytes = MX ? K / 2 : K;
  const bool ragged = !TILED && MX && (row_bytes & 127) != 0;

  // per-group offsets inside the expert (32-bit: an expert's weights stay below 4 GB)
  const uint8_t* wexp = a.W + t.expert * a.w_estride;
  uint32_t woff[G];  // plain: row * ldw + 32 q;  tiled: first tile of the group + 16 lane
  uint32_t soff[G];  // MXFP4 scales.  plain: row * (K / 32);  tiled: first tile + 2 lane
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (TILED) {
      const int64_t grp16 = min<int64_t>(n0 / 16 + g * kSkWaves + wave, N / 16 - 1);
      woff[g] = uint32_t(grp16 * nsteps * 2048 + lane * 16);
      soff[g] = MX ? uint32_t(grp16 * nsteps * 128 + lane * 2) : 0u;
    } else {
      const int64_t row = min<int64_t>(n0 + (g * kSkWaves + wave) * 16 + l16, N - 1);
      woff[g] = uint32_t(row * a.ldw + q * 32);
      soff[g] = MX ? uint32_t(row * a.ws_s0) : 0u;
    }
  }
  const uint8_t* sexp = MX ? reinterpret_cast<const uint8_t*>(a.ws) + t.expert * a.ws_estride : nullptr;
  const int64_t ngroups = K / 32;  // MXFP4 scale groups per row

  i32x4 wb[D][G][2];
  // e8m0 scales of the lane's two 32-element groups: tiled, the two bytes as loaded (split where
  // used); plain, one byte each
  uint32_t sb[D][G][TILED ? 1 : 2];
  // tiled MXFP4 rows whose length is not a whole number of steps: in the last step, a lane
  // whose 16-byte chunk is padding reads its row's first chunk of that step instead (a line
  // lanes 0-15 fetch anyway), so the padding never travels from HBM; its activations are the
  // LDS zero padding, and e2m1 codes are finite, so the products are exact zeros
  uint32_t last_h0 = 0u, last_h1 = 1024u;
  if (TILED && MX) {
    const uint32_t rb_last = uint32_t(row_bytes - int64_t(nsteps - 1) * 128);
    if (32u * uint32_t(q) + 16u > rb_last) last_h0 = 0u - 256u * uint32_t(q);
    if (32u * uint32_t(q) + 32u > rb_last) last_h1 = 0u - 256u * uint32_t(q);
  }

  // all weight / scale addresses are a wave-uniform base plus a 32-bit lane offset
  auto load = [&](int st, int slot) __attribute__((always_inline)) {
    const uint32_t sc = uint32_t(min(st, st_last));
    if (TILED) {
      const bool last = MX && int(sc) == nsteps - 1;
      const uint32_t h0 = last ? last_h0 : 0u, h1 = last ? last_h1 : 1024u;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        wb[slot][g][0] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wexp + (woff[g] + sc * 2048u + h0)));
        wb[slot][g][1] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wexp + (woff[g] + sc * 2048u + h1)));
        if (MX) {
          const uint32_t v = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sexp + soff[g] + sc * 128u));
          sb[slot][g][0] = v;
        }
      }
      return;
    }
    const uint32_t in_row = sc * 128u + uint32_t(q) * 32u;
    const bool past0 = ragged && int64_t(in_row) + 16 > row_bytes;
    const bool past1 = ragged && int64_t(in_row) + 32 > row_bytes;
    const uint32_t g0 = min(sc * 8u + 2u * uint32_t(q), uint32_t(ngroups - 1));
    const uint32_t g1 = min(sc * 8u + 2u * uint32_t(q) + 1u, uint32_t(ngroups - 1));
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // 16-byte halves past the row end (ragged K) re-read the row's first bytes:
      // finite codes whose activations are the zero padding
      const uint32_t rowo = woff[g] - uint32_t(q) * 32u;
      const uint32_t o0 = past0 ? rowo : woff[g] + sc * 128u;
      const uint32_t o1 = past1 ? rowo : woff[g] + sc * 128u + 16u;
      wb[slot][g][0] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wexp + o0));
      wb[slot][g][1] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wexp + o1));
      if (MX) {
        sb[slot][g][0] = sexp[soff[g] + g0];
        sb[slot][g][TILED ? 0 : 1] = sexp[soff[g] + g1];
      }
    }
  };

  for (int m_base = 0; m_base < t.m_total; m_base += AR) {
    const int m_size = min(AR, t.m_total - m_base);
    __syncthreads();  // the previous pass is done with LDS

    // request the first steps of the weight stream before staging the activations
#pragma unroll
    for (int u = 0; u < D - 1; ++u) load(st_b + u, u);

    if (tid < AR) {
      int64_t ar, orw;
      row_of<MODE>(a, t, m_base + min(tid, m_size - 1), ar, orw);
      s_arow[tid] = ar;
      s_orow[tid] = orw;
    }
    __syncthreads();
    {
      // activation rows (rows >= m_size are never read) over the K steps of this workgroup,
      // zero-padded to whole steps
      const int cb = st_b * KSTEP * AE / 16, nc = (st_e - st_b) * KSTEP * AE / 16;
      const int kchunks = int(K * AE / 16);
      for (int c = tid; c < m_size * nc; c += 256) {
        const int m = c / nc, cc = cb + (c - m * nc);
        i32x4 v = {0, 0, 0, 0};
        if (cc < kchunks) {
          const uint8_t* src = reinterpret_cast<const uint8_t*>(a.A) + s_arow[m] * a.lda * AE + int64_t(cc) * 16;
          if (!A_E4M3 && a.a_silu) {
            // gate chunk and the matching up chunk K elements further along the row
            const uint4 g = *reinterpret_cast<const uint4*>(src);
            const uint4 u = *reinterpret_cast<const uint4*>(src + K * 2);
            const uint4 h = silu_mul8(g, u);
            v = i32x4{int(h.x), int(h.y), int(h.z), int(h.w)};
          } else {
            v = *reinterpret_cast<const i32x4*>(src);
          }
        }
        *reinterpret_cast<i32x4*>(smem + m * L.row_stride + (cc - cb) * 16) = v;
      }
      if (!MX) {
        // weight block scales of the workgroup's n-blocks, [kb][nb]
        float* s_sw = reinterpret_cast<float*>(smem + L.sw_off);
        const float* swe = reinterpret_cast<const float*>(a.ws) + t.expert * a.ws_estride;
        const int64_t nb_total = (N + 127) / 128;
        if constexpr (SWCOL) {
          // the scales of the workgroup's 64 G columns over its K steps, [step - st_b][column]
          constexpr int NCOL = 64 * G;
          for (int c = tid; c < (st_e - st_b) * NCOL; c += 256) {
            const int j = c / NCOL, cl = c - j * NCOL;
            const int64_t col = min<int64_t>(n0 + cl, N - 1);
            s_sw[c] = swe[col * a.ws_s0 + int64_t(st_b + j) * a.ws_s1];
          }
        } else
        for (int c = tid; c < L.kb * L.nb; c += 256) {
          const int kb = c / L.nb, nb = c - kb * L.nb;
          const int64_t gnb = min<int64_t>((n0 >> 7) + nb, nb_total - 1);
          s_sw[c] = swe[gnb * a.ws_s0 + kb * a.ws_s1];
        }
      }
      if (A_E4M3) {
        // per-token activation scales, [kb][AR]; rows past m_size repeat valid rows
        float* s_sa = reinterpret_cast<float*>(smem + L.sa_off);
        for (int c = tid; c < L.kb * AR; c += 256) {
          const int kb = c / AR, m = c - kb * AR;
          s_sa[c] = a.sa[s_arow[m] * a.lds + kb];
        }
      }
    }
    __syncthreads();

    f32x4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint8_t* arow = smem + (l16 < m_size ? l16 : 0) * L.row_stride;
    const float* s_sw = reinterpret_cast<const float*>(smem + L.sw_off);
    const float* s_sa = reinterpret_cast<const float*>(smem + L.sa_off);
    const int sa_q = min(q, AR / 4 - 1);  // lanes past the staged rows hold unused outputs

    auto compute = [&](int st, int slot) __attribute__((always_inline)) {
      if constexpr (MX) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const i32x4 af = *reinterpret_cast<const i32x4*>(arow + ((st - st_b) * KSTEP + q * 64 + 8 * s) * 2);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            uint32_t o[4];
            const uint32_t e = TILED ? (sb[slot][g][0] >> (8 * (s >> 2))) & 0xffu : sb[slot][g][(s >> 2) & (TILED ? 0 : 1)];
            e2m1x8_to_bf16(uint32_t(wb[slot][g][s >> 2][s & 3]), e8m0_to_f32(e), o);
            acc[g] = mfma_16x16x32_bf16(af, i32x4{int(o[0]), int(o[1]), int(o[2]), int(o[3])}, acc[g]);
          }
        }
      } else if constexpr (A_E4M3) {
        const i32x4 a0 = *reinterpret_cast<const i32x4*>(arow + (st - st_b) * KSTEP + q * 32);
        const i32x4 a1 = *reinterpret_cast<const i32x4*>(arow + (st - st_b) * KSTEP + q * 32 + 16);
        const i32x8 af = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const f32x4 sa = *reinterpret_cast<const f32x4*>(s_sa + st * AR + 4 * sa_q);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const i32x4 w0 = wb[slot][g][0];
          const i32x4 w1 = wb[slot][g][1];
          const i32x8 bf = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
          const f32x4 part = mfma_16x16x128_e4m3(af, bf, f32x4{0.f, 0.f, 0.f, 0.f});
          // (per-column scales: this lane's output column, (g * kSkWaves + wave) * 16 + l16)
          const float sw = SWCOL ? s_sw[(st - st_b) * (64 * G) + (g * kSkWaves + wave) * 16 + l16]
                                 : s_sw[st * L.nb + ((g * kSkWaves + wave) >> 3)];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[g][r] = fmaf(part[r], sw * sa[r], acc[g][r]);
        }
      } else {
        f32x4 part[G];
#pragma unroll
        for (int g = 0; g < G; ++g) part[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const i32x4 af = *reinterpret_cast<const i32x4*>(arow + ((st - st_b) * KSTEP + q * 32 + 8 * s) * 2);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            uint32_t o0, o1, o2, o3;
            e4m3x4_to_bf16(uint32_t(wb[slot][g][s >> 1][(2 * s) & 3]), o0, o1);
            e4m3x4_to_bf16(uint32_t(wb[slot][g][s >> 1][(2 * s + 1) & 3]), o2, o3);
            part[g] = mfma_16x16x32_bf16(af, i32x4{int(o0), int(o1), int(o2), int(o3)}, part[g]);
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float sw = s_sw[st * L.nb + ((g * kSkWaves + wave) >> 3)];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[g][r] = fmaf(part[g][r], sw, acc[g][r]);
        }
      }
    };

    for (int st0 = st_b; st0 < st_e; st0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        load(st0 + u + D - 1, (u + D - 1) % D);
        if (st0 + u < st_e) compute(st0 + u, u);
      }
    }

    // epilogue: lane (l16, q) holds D[4q + r][l16] of each group
    if (4 * q < m_size) {
      float* const outf = reinterpret_cast<float*>(a.out) + (nsplit > 1 ? split * a.split_stride : 0);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t col = n0 + (g * kSkWaves + wave) * 16 + l16;
        if (col >= N) continue;
        const float b = HAS_BIAS && split == 0 ? load_bias(a, t.expert, col) : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * q + r;
          if (m >= m_size) continue;
          const int64_t o = s_orow[m] * a.ldo + col;
          const float v = acc[g][r] + b;
          if (OUT_F32)
            outf[o] = v;
          else
            reinterpret_cast<uint16_t*>(a.out)[o] = f2bf(v);
        }
      }
    }
  }
}

// two 16-row groups per wave for wide outputs, one for narrow ones (more, smaller
// workgroups: less idle tail in the last round of a grid that is a few rounds deep)
static int skinny_groups(int64_t N) { return N >= MXQ_SK_GSEL ? 2 : 1; }

template <int WFMT, bool AE>
static size_t skinny_lds_t(int64_t K, int AR, int G) {
  return skinny_lds_layout(WFMT == W_E2M1_MX, AE, K, G, AR).total;
}

// Activation rows per pass: eight while the LDS stays within kSkLdsCap (so that several
// workgroups still share a compute unit), else four.
#ifndef MXQ_SK_AR8_CAP
#define MXQ_SK_AR8_CAP (32 * 1024)
#endif
constexpr size_t kSkLdsCap = MXQ_SK_AR8_CAP;
template <int WFMT, bool AE>
static int skinny_rows_t(int64_t K, int G) {
  return skinny_lds_t<WFMT, AE>(K, 8, G) <= kSkLdsCap ? 8 : 4;
}

size_t skinny_lds_bytes(int wfmt, bool a_e4m3, int64_t K) {
  // the larger of the two group counts (the weight-scale table grows with G)
  if (wfmt == W_E2M1_MX) return skinny_lds_t<W_E2M1_MX, false>(K, skinny_rows_t<W_E2M1_MX, false>(K, 2), 2);
  if (a_e4m3) return skinny_lds_t<W_E4M3_BLOCK, true>(K, skinny_rows_t<W_E4M3_BLOCK, true>(K, 2), 2);
  return skinny_lds_t<W_E4M3_BLOCK, false>(K, skinny_rows_t<W_E4M3_BLOCK, false>(K, 2), 2);
}

template <int WFMT, bool AE, int MODE, bool TL, int AR, int G, int D, bool SWC = false>
static void launch_skinny_ar(const GemmArgs& a, bool out_f32, int64_t gb, hipStream_t st, size_t lds_bytes = 0) {
  const int64_t n_tiles = cdiv(a.N, int64_t(64 * G));
  const int64_t nsplit = a.k_split > 1 ? a.k_split : 1;
  const dim3 grid(static_cast<unsigned>(gb * n_tiles * nsplit)), block(256);
  // (routed blocks: LDS for all of K, at least the chunk-sized layout the kernel uses)
  const size_t lds = lds_bytes > 0 ? lds_bytes : skinny_lds_t<WFMT, AE>(a.K, AR, G);
  const bool bias = a.bias != nullptr;
#define MXQ_SK_GO(OF, HB) \
  hipLaunchKernelGGL((skinny_kernel<WFMT, AE, MODE, OF, HB, TL, AR, G, D, SWC>), grid, block, lds, st, a, gb)
  if (out_f32) { if (bias) MXQ_SK_GO(true, true); else MXQ_SK_GO(true, false); }
  else { if (bias) MXQ_SK_GO(false, true); else MXQ_SK_GO(false, false); }
#undef MXQ_SK_GO
}

template <int WFMT, bool AE, int MODE, int G, int D>
static void launch_skinny_g(const GemmArgs& a, bool out_f32, int64_t gb, hipStream_t st) {
  const bool eight = skinny_rows_t<WFMT, AE>(a.K, G) == 8;
  if (a.w_tiled) {
    if (eight) launch_skinny_ar<WFMT, AE, MODE, true, 8, G, D>(a, out_f32, gb, st);
    else launch_skinny_ar<WFMT, AE, MODE, true, 4, G, D>(a, out_f32, gb, st);
  } else {
    if (eight) launch_skinny_ar<WFMT, AE, MODE, false, 8, G, D>(a, out_f32, gb, st);
    else launch_skinny_ar<WFMT, AE, MODE, false, 4, G, D>(a, out_f32, gb, st);
  }
}

template <int WFMT, bool AE, int MODE>
static void launch_skinny_t(const GemmArgs& a, bool out_f32, int64_t gb, hipStream_t st) {
  if (skinny_groups(a.N) == 2)
    launch_skinny_g<WFMT, AE, MODE, 2, 3>(a, out_f32, gb, st);
  else
    launch_skinny_g<WFMT, AE, MODE, 1, 4>(a, out_f32, gb, st);
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

// Dense W8A8 rows (e4m3 activations and weights in the plain layout, 128 x 128 weight blocks):
// tiles of AR rows (8, or 4 when eight rows of K would pass the LDS cap), all launched at once.
size_t skinny_dense_lds(int64_t N, int64_t K, int ar, int64_t kstage, bool a_e4m3, bool swcol) {
  return skinny_lds_layout(false, a_e4m3, K, skinny_groups(N), ar, kstage, swcol).total;
}

int64_t skinny_dense_col_tiles(int64_t N) { return cdiv(N, int64_t(64 * skinny_groups(N))); }

template <bool AE, bool SWC>
static void launch_skinny_dense_t(const GemmArgs& a, int ar, bool out_f32, hipStream_t st) {
  const int64_t tiles = cdiv(a.M, int64_t(ar));
  const size_t lds = skinny_dense_lds(a.N, a.K, ar, a.k_split > 1 ? a.k_chunk : 0, AE, SWC);
  if (skinny_groups(a.N) == 2) {
    if (ar == 8) launch_skinny_ar<W_E4M3_BLOCK, AE, ROWS_DENSE, false, 8, 2, 3, SWC>(a, out_f32, tiles, st, lds);
    else launch_skinny_ar<W_E4M3_BLOCK, AE, ROWS_DENSE, false, 4, 2, 3, SWC>(a, out_f32, tiles, st, lds);
  } else {
    if (ar == 8) launch_skinny_ar<W_E4M3_BLOCK, AE, ROWS_DENSE, false, 8, 1, 4, SWC>(a, out_f32, tiles, st, lds);
    else launch_skinny_ar<W_E4M3_BLOCK, AE, ROWS_DENSE, false, 4, 1, 4, SWC>(a, out_f32, tiles, st, lds);
  }
}

void launch_skinny_dense(const GemmArgs& a, int ar, bool a_e4m3, bool out_f32, hipStream_t st, bool swcol) {
  if (a.M <= 0 || a.N <= 0) return;
  if (swcol && a_e4m3)
    launch_skinny_dense_t<true, true>(a, ar, out_f32, st);
  else if (a_e4m3)
    launch_skinny_dense_t<true, false>(a, ar, out_f32, st);
  else
    launch_skinny_dense_t<false, false>(a, ar, out_f32, st);
}

// out[m, n] = bf16(sum over chunks c = 0 .. S-1, in that order, of part[c][m][n]); the bias rode
// on chunk 0.  Four columns per thread when N is a multiple of four.
__global__ __launch_bounds__(256) void dense_split_sum_kernel(const float* __restrict__ part, int32_t S, int64_t M,
                                                              int64_t N, uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t slice = M * N;
  const bool vec = (N & 3) == 0;
  const int64_t per = vec ? 4 : 1;
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * per;
  if (i >= slice) return;
  const int64_t m = i / N, n = i - m * N;
  if (vec) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
    for (int c = 1; c < S; ++c) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + c * slice + i);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += v[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) out[m * ldo + n + r] = f2bf(acc[r]);
  } else {
    float acc = part[i];
    for (int c = 1; c < S; ++c) acc += part[c * slice + i];
    out[m * ldo + n] = f2bf(acc);
  }
}

void launch_dense_split_sum(const float* part, int32_t S, int64_t M, int64_t N, uint16_t* out, int64_t ldo,
                            hipStream_t st) {
  if (M <= 0 || N <= 0) return;
  const int64_t per = (N & 3) == 0 ? 4 : 1;
  const dim3 grid{unsigned(cdiv(cdiv(M * N, per), int64_t(256)))}, block{256u};
  hipLaunchKernelGGL(dense_split_sum_kernel, grid, block, 0, st, part, S, M, N, out, ldo);
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
