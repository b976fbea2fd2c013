// Persistent expert-streaming kernel for routings whose experts all hold only a few rows
// (decode-sized batches).
//
// "vLLM PR 50949 review" (implementation items 1-2): a tiny expert block is bound by reading its
// expert's weights once; when every block of the routing is such a block, the sorted block
// tables are only bookkeeping between the routing ids and the weight stream.  So here each
// workgroup reads the routing ids once and groups the routed rows by expert in LDS (a counting
// pass, a prefix over the experts, a placement pass); it then walks a fixed share of the
// (touched expert, 64-column tile) items -- item i of workgroup b is b + i * gridDim.x -- and
// an expert with more than AR rows takes several passes over its weights.  Rows are named by
// their flat routed id (token * topk + k) in both stages: the intermediate and the stage-2
// output are indexed by it, and the top-k combine reads it back the same way.
//
//  * weights stream into registers through a D-deep ring, 128 bytes of a row per step, with the
//    operand layouts and decode of the tiny-block kernel (skinny.hip); the ring runs across
//    passes, so the first steps of the next pass are already requested while the current pass
//    finishes and a wave's weight stream does not stop between passes;
//  * the next pass's activation rows (and, for e4m3 weights, each wave's block-scale columns)
//    are copied into the second of two LDS buffers with GLOBAL_LOAD_LDS while the current pass
//    computes; a pass starts with a vmcnt wait and one barrier, and no dependent memory read
//    sits between two passes;
//  * stage 1 gives each wave a 16-row gate group and the matching up group, so its epilogue
//    adds the bias, rounds both halves to bf16 and writes h = bf16(silu(gate) * up) -- the
//    rounding points of the path that stores the gate / up rows first, bit for bit;
//  * stage 2 writes fp32 rows for the combine.
#include <algorithm>
#include <type_traits>

#include "lds_dma.hpp"
#include "quant_common.hpp"
#include "tile_rows.hpp"

namespace mxq {

namespace {
constexpr int kEsWaves = 4;

// Waves per SIMD the register budget targets (as for the tiny-block kernel).
template <int WFMT>
struct EsShape {
  static constexpr int W = WFMT == W_E2M1_MX ? 3 : 4;
};
}  // namespace

// LDS layout (bytes): routing tables (cnt, fill, start, touched: [E] each; rows [R]; touched
// count) | activation buffers [2][AR][row_stride] | e4m3 weight-scale columns
// [2 buffers][4 waves][G][kbp] fp32.
struct EsLds {
  int row_stride, kb, kbp;
  uint32_t act_off, buf_bytes, sw_off, total;
};

__host__ __device__ inline EsLds es_lds_layout(bool mx, int64_t K, int64_t E, int64_t R, int AR, int G) {
  EsLds L;
  const int64_t kstep = mx ? 256 : 128;
  const int64_t kpad = (K + kstep - 1) / kstep * kstep;
  L.row_stride = int(kpad * 2 + 16);  // +16 B: rows read together fall in different LDS banks
  L.kb = int(K >> 7);
  L.kbp = (L.kb + 63) / 64 * 64;
  const int64_t tab = 4 * (4 * E + R + 1);
  L.act_off = uint32_t((tab + 15) & ~int64_t(15));
  L.buf_bytes = uint32_t(AR * L.row_stride);
  L.sw_off = L.act_off + 2 * L.buf_bytes;
  L.total = L.sw_off + (mx ? 0u : uint32_t(2 * kEsWaves * G * L.kbp * 4));
  return L;
}

template <int WFMT, int STAGE, bool HAS_BIAS, bool TILED, int AR, int G, int D>
__global__ __launch_bounds__(256, (EsShape<WFMT>::W)) void expert_stream_kernel(GemmArgs a, EsRoute rt) {
  constexpr bool MX = WFMT == W_E2M1_MX;
  constexpr int KSTEP = MX ? 256 : 128;  // K elements per 128-byte row step
  static_assert(WFMT == W_E2M1_MX || WFMT == W_E4M3_BLOCK, "bf16 activations with e2m1 or e4m3 weights");
  static_assert(STAGE == 2 || G == 2, "stage 1 pairs a gate group with an up group");
  static_assert(AR == 4 || AR == 8, "four or eight rows per pass");
  static_assert(D >= 2 && (D - 1) * 2 * G < 64, "ring depth");

  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t N = a.N, K = a.K;
  const int E = rt.E;
  const int64_t R = rt.R;
  const EsLds L = es_lds_layout(MX, K, E, R, AR, G);
  int32_t* s_cnt = reinterpret_cast<int32_t*>(smem);
  int32_t* s_fill = s_cnt + E;
  int32_t* s_start = s_fill + E;
  int32_t* s_touch = s_start + E;
  int32_t* s_rows = s_touch + E;
  int32_t* s_ntouch = s_rows + R;

  // ---- 1. routed rows grouped by expert (experts outside [0, E) are dropped)
  for (int e = tid; e < E; e += 256) {
    s_cnt[e] = 0;
    s_fill[e] = 0;
  }
  {
    // both activation buffers start zeroed: the copies write [0, K) of a row, the padding up
    // to a whole step stays zero
    i32x4* p = reinterpret_cast<i32x4*>(smem + L.act_off);
    for (uint32_t i = tid; i < 2 * L.buf_bytes / 16; i += 256) p[i] = i32x4{0, 0, 0, 0};
  }
  __syncthreads();
  for (int64_t r = tid; r < R; r += 256) {
    const int e = rt.ids[r];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  if (wave == 0) {
    // lane l owns a run of experts; one wave-wide scan of (rows, touched experts)
    const int per = (E + 63) / 64;
    const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
    int nr = 0, nt = 0;
    for (int e = e0; e < e1; ++e) {
      nr += s_cnt[e];
      nt += s_cnt[e] > 0 ? 1 : 0;
    }
    int sr = nr, sn = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int tr = __shfl_up(sr, o, 64), tn = __shfl_up(sn, o, 64);
      if (lane >= o) {
        sr += tr;
        sn += tn;
      }
    }
    int rb = sr - nr, tb = sn - nt;
    for (int e = e0; e < e1; ++e) {
      s_start[e] = rb;
      rb += s_cnt[e];
      if (s_cnt[e] > 0) s_touch[tb++] = e;
    }
    if (lane == 63) *s_ntouch = sn;
  }
  __syncthreads();
  for (int64_t r = tid; r < R; r += 256) {
    const int e = rt.ids[r];
    // the order of an expert's rows does not matter: every output row is computed on its own
    if (e >= 0 && e < E) s_rows[s_start[e] + atomicAdd(&s_fill[e], 1)] = int32_t(r);
  }
  __syncthreads();

  // ---- 2. work items and passes
  const int64_t n_out = STAGE == 1 ? N / 2 : N;  // output columns
  const int64_t cols = STAGE == 1 ? 64 : 64 * G;  // output columns per item
  const int32_t ntiles = int32_t((n_out + cols - 1) / cols);
  const int32_t total = __builtin_amdgcn_readfirstlane(*s_ntouch) * ntiles;

  struct Unit {
    int32_t j, e, nt, row0, m;  // item, expert, column tile, first entry in s_rows, rows (0: none)
  };
  auto uni = [](int32_t v) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(v); };
  auto unit_at = [&](int32_t j) __attribute__((always_inline)) {
    Unit u{j, 0, 0, 0, 0};
    if (j < total) {
      const int32_t t = j / ntiles;
      u.e = uni(s_touch[t]);
      u.nt = j - t * ntiles;
      u.row0 = uni(s_start[u.e]);
      u.m = min(AR, uni(s_cnt[u.e]));
    }
    return u;
  };
  auto unit_next = [&](const Unit& u) __attribute__((always_inline)) {
    Unit v = u;
    if (u.m == 0) return v;
    const int32_t end = uni(s_start[u.e]) + uni(s_cnt[u.e]);
    if (u.row0 + AR < end) {
      v.row0 = u.row0 + AR;
      v.m = min(AR, end - v.row0);
      return v;
    }
    return unit_at(u.j + int32_t(gridDim.x));
  };

  Unit cu = unit_at(int32_t(blockIdx.x));
  if (cu.m == 0) return;  // uniform over the workgroup

  // ---- 3. weight geometry (as in the tiny-block kernel)
  const int nsteps = int((K + KSTEP - 1) / KSTEP);
  const int64_t row_bytes = MX ? K / 2 : K;
  const bool ragged = !TILED && MX && (row_bytes & 127) != 0;
  const int64_t ngroups = K / 32;  // MXFP4 scale groups per row
  const int64_t half16 = N / 32;   // stage 1: 16-row groups in the gate half

  // unclamped 16-row weight group of this wave's group g in column tile nt
  auto group_raw = [&](int32_t nt, int g) __attribute__((always_inline)) -> int64_t {
    if (STAGE == 1) {
      const int64_t gi = min<int64_t>(int64_t(nt) * 4 + wave, half16 - 1);
      return g == 0 ? gi : half16 + gi;
    }
    return int64_t(nt) * 4 * G + g * 4 + wave;
  };

  // where one pass's weights come from: expert base pointers (uniform) and this lane's offsets
  struct Geo {
    const uint8_t* w;
    const uint8_t* s;
    uint32_t woff[G];  // plain: row * ldw + 32 q;  tiled: first tile of the group + 16 lane
    uint32_t soff[G];  // MXFP4 scales.  plain: row * (K / 32);  tiled: first tile + 2 lane
  };
  auto geo_of = [&](const Unit& u) __attribute__((always_inline)) {
    Geo gm;
    gm.w = a.W + int64_t(u.e) * a.w_estride;
    gm.s = MX ? reinterpret_cast<const uint8_t*>(a.ws) + int64_t(u.e) * a.ws_estride : nullptr;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (TILED) {
        const int64_t grp16 = min<int64_t>(group_raw(u.nt, g), N / 16 - 1);
        gm.woff[g] = uint32_t(grp16 * nsteps * 2048 + lane * 16);
        gm.soff[g] = MX ? uint32_t(grp16 * nsteps * 128 + lane * 2) : 0u;
      } else {
        const int64_t row =
            min<int64_t>(group_raw(u.nt, g) * 16 + l16, STAGE == 1 ? (g == 0 ? N / 2 : N) - 1 : N - 1);
        gm.woff[g] = uint32_t(row * a.ldw + q * 32);
        gm.soff[g] = MX ? uint32_t(row * a.ws_s0) : 0u;
      }
    }
    return gm;
  };

  Unit nu = unit_next(cu);  // the pass whose operands are copied while cu computes
  Geo gc = geo_of(cu), gn = geo_of(nu.m > 0 ? nu : cu);

  i32x4 wb[D][G][2];
  // e8m0 scales of the lane's two 32-element groups: tiled, the two bytes as loaded; plain, one
  // byte each (kept at load width, so no instruction touches them before their step computes)
  uint16_t sb[D][G][TILED ? 1 : 2];
  // tiled MXFP4 rows that end inside the last step: padding chunks re-read the row's first chunk
  // of that step (a line lanes 0-15 fetch anyway); their activations are the LDS zero padding
  uint32_t last_h0 = 0u, last_h1 = 1024u;
  if (TILED && MX) {
    const uint32_t rb_last = uint32_t(row_bytes - int64_t(nsteps - 1) * 128);
    if (32u * uint32_t(q) + 16u > rb_last) last_h0 = 0u - 256u * uint32_t(q);
    if (32u * uint32_t(q) + 32u > rb_last) last_h1 = 0u - 256u * uint32_t(q);
  }

  // step st of a pass (steps past the row, the padding of a pass to whole ring turns, re-read
  // the last step and are never computed)
  // step st of the pass described by gc, or (nx) of the pass described by gn; steps past the
  // row -- the padding of a pass to whole turns of the ring -- re-read the last step and are
  // never computed.  The choice is a select, not a branch, so every ring slot is written on
  // one path.
  auto load = [&](bool nx, int st, int slot) __attribute__((always_inline)) {
    const uint32_t sc = uint32_t(min(st, nsteps - 1));
    const uint8_t* gw = nx ? gn.w : gc.w;
    const uint8_t* gs = nx ? gn.s : gc.s;
    uint32_t woff[G], soff[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      woff[g] = nx ? gn.woff[g] : gc.woff[g];
      soff[g] = nx ? gn.soff[g] : gc.soff[g];
    }
    if (TILED) {
      const bool last = MX && int(sc) == nsteps - 1;
      const uint32_t h0 = last ? last_h0 : 0u, h1 = last ? last_h1 : 1024u;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        wb[slot][g][0] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(gw + (woff[g] + sc * 2048u + h0)));
        wb[slot][g][1] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(gw + (woff[g] + sc * 2048u + h1)));
        if (MX)
          sb[slot][g][0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(gs + soff[g] + sc * 128u));
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
      // 16-byte halves past the row end (ragged K) re-read the row's first bytes: finite codes
      // whose activations are the zero padding
      const uint32_t rowo = woff[g] - uint32_t(q) * 32u;
      const uint32_t o0 = past0 ? rowo : woff[g] + sc * 128u;
      const uint32_t o1 = past1 ? rowo : woff[g] + sc * 128u + 16u;
      wb[slot][g][0] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(gw + o0));
      wb[slot][g][1] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(gw + o1));
      if (MX) {
        sb[slot][g][0] = gs[soff[g] + g0];
        sb[slot][g][TILED ? 0 : 1] = gs[soff[g] + g1];
      }
    }
  };

  // copies of one pass's operands into LDS buffer b
  const int64_t kbytes = K * 2;
  const int segs = int((kbytes + 1023) / 1024);
  auto issue_copies = [&](const Unit& u, int b) __attribute__((always_inline)) {
    uint8_t* base = smem + L.act_off + uint32_t(b) * L.buf_bytes;
    for (int i = wave; i < u.m * segs; i += kEsWaves) {  // 1 KB of one row per copy
      const int m = i / segs, s = i - m * segs;
      const int32_t r = uni(s_rows[u.row0 + m]);
      const int64_t arow = STAGE == 1 ? r / rt.topk : r;
      const int64_t cb = int64_t(s) * 1024 + lane * 16;
      if (cb < kbytes)
        lds_dma16(reinterpret_cast<const uint8_t*>(a.A) + arow * a.lda * 2 + cb,
                  lds_addr(base + m * L.row_stride + s * 1024));
    }
    if (!MX) {
      // this wave's block-scale columns: [kb] of the 128-row block holding each of its groups
      float* sw = reinterpret_cast<float*>(smem + L.sw_off) + (b * kEsWaves + wave) * G * L.kbp;
      const float* swe = reinterpret_cast<const float*>(a.ws) + int64_t(u.e) * a.ws_estride;
      const int64_t nb_last = (N - 1) >> 7;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t nb = min<int64_t>((group_raw(u.nt, g) * 16) >> 7, nb_last);
        for (int k0 = 0; k0 < L.kb; k0 += 64)
          if (k0 + lane < L.kb) lds_dma4(swe + nb * a.ws_s0 + (k0 + lane) * a.ws_s1, lds_addr(sw + g * L.kbp + k0));
      }
    }
  };

  f32x4 acc[G];
  float bias_r[G];
#pragma unroll
  for (int g = 0; g < G; ++g) bias_r[g] = 0.f;

  auto compute = [&](int st, int slot, int b, int m_size) __attribute__((always_inline)) {
    const uint8_t* arow = smem + L.act_off + uint32_t(b) * L.buf_bytes + (l16 < m_size ? l16 : 0) * L.row_stride;
    if constexpr (MX) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const i32x4 af = *reinterpret_cast<const i32x4*>(arow + (st * KSTEP + q * 64 + 8 * s) * 2);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          uint32_t o[4];
          const uint32_t e = TILED ? (uint32_t(sb[slot][g][0]) >> (8 * (s >> 2))) & 0xffu
                                   : uint32_t(sb[slot][g][(s >> 2) & (TILED ? 0 : 1)]);
          e2m1x8_to_bf16(uint32_t(wb[slot][g][s >> 2][s & 3]), e8m0_to_f32(e), o);
          acc[g] = mfma_16x16x32_bf16(af, i32x4{int(o[0]), int(o[1]), int(o[2]), int(o[3])}, acc[g]);
        }
      }
    } else {
      const float* sw = reinterpret_cast<const float*>(smem + L.sw_off) + (b * kEsWaves + wave) * G * L.kbp;
      f32x4 part[G];
#pragma unroll
      for (int g = 0; g < G; ++g) part[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const i32x4 af = *reinterpret_cast<const i32x4*>(arow + (st * KSTEP + q * 32 + 8 * s) * 2);
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
        const float s = sw[g * L.kbp + st];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[g][r] = fmaf(part[g][r], s, acc[g][r]);
      }
    }
  };

  // lane (l16, q) holds D[4q + r][l16] of each group: pass row 4q + r, output column l16
  auto epilogue = [&](const Unit& u) __attribute__((always_inline)) {
    if (4 * q >= u.m) return;
    if (STAGE == 1) {
      const int64_t I = N / 2;
      const int64_t col = int64_t(u.nt) * 64 + wave * 16 + l16;
      if (col >= I) return;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * q + r;
        if (m >= u.m) continue;
        const int64_t row = s_rows[u.row0 + m];
        const float gv = bf16f(f2bf(acc[0][r] + bias_r[0]));
        const float uv = bf16f(f2bf(acc[1][r] + bias_r[1]));
        reinterpret_cast<uint16_t*>(a.out)[row * a.ldo + col] = f2bf(silu_mul_f32(gv, uv));
      }
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t col = group_raw(u.nt, g) * 16 + l16;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * q + r;
          if (m >= u.m) continue;
          const int64_t row = s_rows[u.row0 + m];
          reinterpret_cast<float*>(a.out)[row * a.ldo + col] = acc[g][r] + bias_r[g];
        }
      }
    }
  };

  // ---- 4. the stream.  A pass is padded to whole turns of the ring (nsteps_pad steps, a
  // multiple of D), so step st of every pass sits in ring slot st % D.  The last turn of a pass
  // requests the first D - 1 steps of the next pass (or, after the last pass, re-reads its own
  // last step), so the ring never drains between passes.
  const int nsteps_pad = (nsteps + D - 1) / D * D;
  int buf = 0;
  issue_copies(cu, 0);
#pragma unroll
  for (int u = 0; u < D - 1; ++u) load(false, u, u);
  for (;;) {
    // this pass's copies were issued before at least D - 1 steps of ring loads (each at least
    // 2 G operations), so waiting down to (D - 1) * 2 G outstanding operations covers them;
    // after the barrier every wave's copies are in and the other buffer is free
    wait_vmcnt<(D - 1) * 2 * G>();
    __syncthreads();
    if (nu.m > 0) issue_copies(nu, buf ^ 1);
    if (HAS_BIAS && STAGE == 1) {
      // fp32 bias of this lane's gate and up columns (read now, used by the epilogue)
      const int64_t c = min<int64_t>(int64_t(cu.nt) * 64 + wave * 16 + l16, N / 2 - 1);
      const float* be = reinterpret_cast<const float*>(a.bias) + int64_t(cu.e) * a.bias_estride;
      bias_r[0] = be[c];
      bias_r[1] = be[N / 2 + c];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int m_size = cu.m;
    for (int st0 = 0; st0 < nsteps_pad; st0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        // in the last turn, step st0 + u + D - 1 is step u - 1 of the next pass (same slot)
        const int ls = st0 + u + D - 1;
        const bool nx = ls >= nsteps_pad;
        load(nx, nx ? ls - nsteps_pad : ls, (u + D - 1) % D);
        if (st0 + u < nsteps) compute(st0 + u, u, buf, m_size);
      }
    }
    epilogue(cu);
    if (nu.m == 0) break;
    cu = nu;
    gc = gn;
    nu = unit_next(cu);
    gn = geo_of(nu.m > 0 ? nu : cu);
    buf ^= 1;
  }
}

// ---------------------------------------------------------------- host side

namespace {
template <int WFMT>
size_t es_lds(int stage, int64_t K, int64_t E, int64_t R, int AR, int G) {
  return es_lds_layout(WFMT == W_E2M1_MX, K, E, R, AR, G).total;
}

int es_groups(int stage, int64_t N) { return stage == 1 ? 2 : (N >= 4096 ? 2 : 1); }

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int WFMT, int STAGE, bool TL, int AR, int G, int D>
void launch_es(const GemmArgs& a, const EsRoute& rt, hipStream_t st) {
  const size_t lds = es_lds<WFMT>(STAGE, a.K, rt.E, rt.R, AR, G);
  const int64_t n_out = STAGE == 1 ? a.N / 2 : a.N;
  const int64_t ntiles = cdiv(n_out, STAGE == 1 ? 64 : 64 * G);
  // two workgroups per compute unit: measured on the GPT-OSS decode shape, three (the LDS
  // allows it) keep more weight streams open than the memory system serves well
  const int per_cu = std::max<int>(1, std::min<int>(2, int((160 * 1024) / lds)));
  const int64_t items = std::min<int64_t>(rt.E, rt.R) * ntiles;  // touched experts <= min(E, R)
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(items, int64_t(device_cus()) * per_cu));
  // only stage 1 takes a bias
  if constexpr (STAGE == 1) {
    if (a.bias != nullptr) {
      hipLaunchKernelGGL((expert_stream_kernel<WFMT, STAGE, true, TL, AR, G, D>), dim3(unsigned(grid)), dim3(256),
                         lds, st, a, rt);
      return;
    }
  }
  hipLaunchKernelGGL((expert_stream_kernel<WFMT, STAGE, false, TL, AR, G, D>), dim3(unsigned(grid)), dim3(256), lds,
                     st, a, rt);
}

template <int WFMT, int STAGE, int G, int D>
void launch_es_g(const GemmArgs& a, const EsRoute& rt, hipStream_t st) {
  if (a.w_tiled)
    launch_es<WFMT, STAGE, true, 4, G, D>(a, rt, st);
  else
    launch_es<WFMT, STAGE, false, 4, G, D>(a, rt, st);
}

template <int WFMT, int STAGE>
void launch_es_s(const GemmArgs& a, const EsRoute& rt, hipStream_t st) {
  if constexpr (STAGE == 1)
    launch_es_g<WFMT, STAGE, 2, 3>(a, rt, st);
  else if (es_groups(STAGE, a.N) == 2)
    launch_es_g<WFMT, STAGE, 2, 3>(a, rt, st);
  else
    launch_es_g<WFMT, STAGE, 1, 4>(a, rt, st);
}
}  // namespace

size_t expert_stream_lds_bytes(int wfmt, int stage, int64_t N, int64_t K, int64_t E, int64_t R) {
  const int G = es_groups(stage, N);
  return wfmt == W_E2M1_MX ? es_lds<W_E2M1_MX>(stage, K, E, R, 4, G) : es_lds<W_E4M3_BLOCK>(stage, K, E, R, 4, G);
}

void launch_expert_stream(const GemmArgs& a, int wfmt, int stage, const EsRoute& rt, hipStream_t stream) {
  if (a.N <= 0 || rt.R <= 0) return;
  if (wfmt == W_E2M1_MX) {
    if (stage == 1)
      launch_es_s<W_E2M1_MX, 1>(a, rt, stream);
    else
      launch_es_s<W_E2M1_MX, 2>(a, rt, stream);
  } else {
    if (stage == 1)
      launch_es_s<W_E4M3_BLOCK, 1>(a, rt, stream);
    else
      launch_es_s<W_E4M3_BLOCK, 2>(a, rt, stream);
  }
}

}  // namespace mxq
