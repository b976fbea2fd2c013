// MX-scaled GEMM for gfx950: MXFP8 activations (e4m3 + one e8m0 scale per 32 columns of a
// row) times MXFP8 or MXFP4 weights (e4m3 / e2m1 + one e8m0 scale per 32 columns of a row),
// fp32 accumulation, bf16 output (+ optional bias), and the MXFP8 quantiser of its input.
//
// Arithmetic: out[m, n] = bf16( sum_k dec(qa[m,k]) 2^(sa[m,k/32]-127) dec(w[n,k]) 2^(sw[n,k/32]-127)
// + bias[n] ) -- the MXFP4 expert weights of "vLLM PR 50949 review" (summary and implementation
// item 2) and the [1, 32] activation block recipe of "SGLang PR 35605 review" (implementation
// item 1), multiplied on V_MFMA_SCALE_F32_16X16X128_F8F6F4, which applies both e8m0 scales
// itself: no promotion step between K blocks.
//
// The instruction's operand layout (measured on the device with a one-wave probe):
//  * lane l supplies row (l % 16) of its operand and the e8m0 scale of 32-column block l / 16
//    of the instruction's 128-column K step, for both operands;
//  * an e2m1 operand lane holds the 32 consecutive elements of that block (16 bytes, element
//    2j in the low nibble of byte j);
//  * an e4m3 operand lane holds elements [16q, 16q + 16) in its low 16 bytes and
//    [64 + 16q, 64 + 16q + 16) in its high 16 bytes (q = l / 16): so the fragment of a row is
//    16-byte chunks q and q + 4 of its 128-byte K step, and block b's scale (lane quarter b)
//    covers exactly memory columns [32b, 32b + 32).
//
// Tile: BM x 256 outputs per 512-thread workgroup (8 waves, 2 x 4, each BM/2 x 64), K step 128,
// two LDS stages filled by GLOBAL_LOAD_LDS (the upper four waves copy, the lower four start
// their products right after the barrier); per K step each row's four scale bytes ride the
// same copy (one dword per row).  MFMA A operand = weights, B = activations, so a lane owns 4
// consecutive output columns of one row.  XCD-aware raster as in the block-FP8 tile: bands of
// 4 row tiles run all their column tiles on one XCD.
#include "kernels.hpp"
#include "lds_dma.hpp"
#include "tile_rows.hpp"

namespace mxq {

namespace {

constexpr int kMxK = 128;  // K per step (four 32-column scale blocks)

template <int BM, int WFMT>
struct MxCfg {
  static constexpr int BN = 256, NW = 8, THREADS = NW * 64;
  static constexpr int WN = 4, WM = 2;
  static constexpr int WROWS = BM / WM, TI = WROWS / 16;
  static constexpr int WB = WFMT == MX_W_E2M1 ? 64 : 128;  // weight bytes per row per K step
  static constexpr int A_BYTES = BM * kMxK, B_BYTES = BN * WB;
  static constexpr int SA_BYTES = BM * 4, SB_BYTES = BN * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  static constexpr int COPY_WAVES = NW / 2;
  static constexpr int A_PIECES = A_BYTES / 1024 / COPY_WAVES;
  static constexpr int B_PIECES = B_BYTES / 1024 / COPY_WAVES;
  static constexpr int SA_DMAS = BM / 64, SB_DMAS = BN / 64;  // one dword per row
  static_assert(A_PIECES >= 1 && B_PIECES >= 1 && SA_DMAS <= COPY_WAVES && SB_DMAS <= COPY_WAVES, "tile");
};

// e4m3 rows (128 bytes per K step): 16-byte chunk c of row r stored at chunk c ^ swz8(r)
__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// e2m1 rows (64 bytes per K step): chunk c of row r stored at chunk c ^ ((r >> 2) & 3), so the
// 16 lanes reading one chunk of rows r .. r + 15 hit 16 different 16-byte bank groups
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

// MXFP8 fragment of `row`: chunks q and q + 4 of its 128-byte K step
__device__ __forceinline__ i32x8 frag_mx8(const uint8_t* tile, int row, int q) {
  const int s = swz8(row);
  const uint8_t* base = tile + row * kMxK;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + ((q ^ s) << 4));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + (((q + 4) ^ s) << 4));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// MXFP4 fragment of `row`: chunk q of its 64-byte K step (the upper half of the operand unused)
__device__ __forceinline__ i32x8 frag_mx4(const uint8_t* tile, int row, int q) {
  const i32x4 v = *reinterpret_cast<const i32x4*>(tile + row * 64 + ((q ^ swz4(row)) << 4));
  return i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
}

template <int WFMT>
__device__ __forceinline__ f32x4 mfma_mx(const i32x8& w, const i32x8& a, const f32x4& c, int sw, int sa) {
  // format codes of the instruction: 0 = e4m3, 4 = e2m1
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, c, WFMT == MX_W_E2M1 ? 4 : 0, 0, 0, sw, 0, sa);
}

}  // namespace

// OUT_F32: a K split -- chunk blockIdx.y runs its K steps and writes fp32 partial sums
template <int BM, int WFMT, bool HAS_BIAS, bool OUT_F32 = false>
__global__ __launch_bounds__(512) void gemm_mx_kernel(MxArgs a, int64_t row_tiles, int64_t n_tiles) {
  using C = MxCfg<BM, WFMT>;
  constexpr int TI = C::TI, WROWS = C::WROWS;
  // two operand stages; the epilogue reuses the space (8 waves x WROWS rows x 128 bytes)
  constexpr int kOps = 2 * C::STAGE > C::NW * WROWS * 128 ? 2 * C::STAGE : C::NW * WROWS * 128;
  __shared__ __align__(1024) uint8_t sOps[kOps];
  __shared__ int64_t sArow[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int l16 = lane & 15, q = lane >> 4;

  // XCD-aware raster (workgroup b runs on XCD b % 8): bands of 4 row tiles x all column tiles
  const int64_t total = row_tiles * n_tiles;
  const int64_t per_xcd = cdiv(total, 8);
  const int64_t t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (t >= total) return;
  const int64_t gm = min<int64_t>(4, row_tiles);
  const int64_t band = t / (gm * n_tiles);
  const int64_t band_rows = min<int64_t>(gm, row_tiles - band * gm);
  const int64_t in_band = t - band * gm * n_tiles;
  const int64_t m0 = (band * gm + in_band % band_rows) * BM;
  const int64_t n0 = (in_band / band_rows) * C::BN;
  if (m0 >= a.M || n0 >= a.N) return;
  const int m_size = int(min<int64_t>(BM, a.M - m0));

  for (int i = tid; i < BM; i += C::THREADS) sArow[i] = min<int64_t>(m0 + i, a.M - 1);
  __syncthreads();

  // per-lane copy sources (32-bit byte offsets: the host keeps every operand below 4 GiB)
  const bool copier = wave >= C::NW / 2;
  const int cw = max(wave - C::NW / 2, 0);
  uint32_t oa[C::A_PIECES], ob[C::B_PIECES];
#pragma unroll
  for (int b = 0; b < C::A_PIECES; ++b) {
    const int row = (cw * C::A_PIECES + b) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz8(row);
    oa[b] = uint32_t(sArow[row] * a.lda + chunk * 16);
  }
#pragma unroll
  for (int b = 0; b < C::B_PIECES; ++b) {
    const int d = cw * C::B_PIECES + b;
    int row, chunk;
    if (WFMT == MX_W_E2M1) {  // 16 rows of 64 bytes per 1 KB piece
      row = d * 16 + (lane >> 2);
      chunk = (lane & 3) ^ swz4(row);
    } else {
      row = d * 8 + (lane >> 3);
      chunk = (lane & 7) ^ swz8(row);
    }
    const int64_t n = min<int64_t>(n0 + row, a.N - 1);
    ob[b] = uint32_t(n * a.ldw + chunk * 16);
  }
  // scale rows: copying wave cw fetches activation-scale rows cw*64 + lane (cw < BM/64) and
  // weight-scale rows cw*64 + lane (cw < 4); one dword (four e8m0 bytes) per row per K step
  const bool sa_wave = cw < C::SA_DMAS;
  const uint32_t osa = uint32_t(sArow[(cw % C::SA_DMAS) * 64 + lane] * a.lds_bytes);
  const uint32_t osb = uint32_t(min<int64_t>(n0 + cw * 64 + lane, a.N - 1) * a.ldws_bytes);

  auto stA = [&](int s) { return sOps + s * C::STAGE; };
  auto stB = [&](int s) { return sOps + s * C::STAGE + C::A_BYTES; };
  auto stSA = [&](int s) { return sOps + s * C::STAGE + C::A_BYTES + C::B_BYTES; };
  auto stSB = [&](int s) { return sOps + s * C::STAGE + C::A_BYTES + C::B_BYTES + C::SA_BYTES; };
  const uint8_t* A = reinterpret_cast<const uint8_t*>(a.A);
  const uint8_t* W = reinterpret_cast<const uint8_t*>(a.W);
  const uint8_t* SA = reinterpret_cast<const uint8_t*>(a.sa);
  const uint8_t* SW = reinterpret_cast<const uint8_t*>(a.sw);

  auto issue = [&](int kb, int s) __attribute__((always_inline)) {
    if (!copier) return;
    const uint8_t* Ak = A + kb * kMxK;
    const uint8_t* Wk = W + kb * C::WB;
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds_addr(stA(s)) + cw * C::A_PIECES * 1024);
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(stB(s)) + cw * C::B_PIECES * 1024);
#pragma unroll
    for (int b = 0; b < C::A_PIECES; ++b) lds_dma16(Ak, oa[b], la + b * 1024);
#pragma unroll
    for (int b = 0; b < C::B_PIECES; ++b) lds_dma16(Wk, ob[b], lb + b * 1024);
    if (sa_wave) lds_dma4(SA + kb * 4, osa, __builtin_amdgcn_readfirstlane(lds_addr(stSA(s)) + cw * 256));
    lds_dma4(SW + kb * 4, osb, __builtin_amdgcn_readfirstlane(lds_addr(stSB(s)) + cw * 256));
  };

  f32x4 acc[TI][4];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int mrow = wm * WROWS;
  auto compute = [&](int s) __attribute__((always_inline)) {
    const uint8_t* cA = stA(s);
    const uint8_t* cB = stB(s);
    const uint8_t* cSA = stSA(s);
    const uint8_t* cSB = stSB(s);
    i32x8 wf[4];
    int wsc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 64 + 16 * j + l16;
      wf[j] = WFMT == MX_W_E2M1 ? frag_mx4(cB, r, q) : frag_mx8(cB, r, q);
      wsc[j] = cSB[r * 4 + q];
    }
    int asc[TI];
#pragma unroll
    for (int i = 0; i < TI; ++i) asc[i] = cSA[(mrow + 16 * i + l16) * 4 + q];
    i32x8 af[2];
    af[0] = frag_mx8(cA, mrow + l16, q);
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      if (i + 1 < TI) af[(i + 1) & 1] = frag_mx8(cA, mrow + 16 * (i + 1) + l16, q);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_mx<WFMT>(wf[j], af[i & 1], acc[i][j], wsc[j], asc[i]);
    }
  };

  // K loop: wait for this stage, publish it with a barrier (which also retires every wave's
  // reads of the stage the next copy overwrites), copy the next K step, compute
  const int KB = int(a.K / kMxK);
  // the workgroup's K steps [kb0, kb0 + nkb) (all of them without a split; an empty chunk
  // writes zeros)
  const int split = OUT_F32 ? int(blockIdx.y) : 0;
  const int kb0 = OUT_F32 ? min(KB, split * int(a.k_chunk / kMxK)) : 0;
  const int nkb = OUT_F32 ? min(KB - kb0, int(a.k_chunk / kMxK)) : KB;
  if (nkb > 0) issue(kb0, 0);
  for (int j = 0; j < nkb; ++j) {
    wait_vmcnt<0>();
    __syncthreads();
    if (j + 1 < nkb) issue(kb0 + j + 1, (j + 1) & 1);
    compute(j & 1);
  }
  wait_vmcnt<0>();

  if constexpr (OUT_F32) {
    // fp32 partial sums straight from the accumulators: lane owns rows mrow + 16 i + l16,
    // columns n0 + wn*64 + 16 j + 4 q .. + 3; the bias on chunk 0
    float* const outf = reinterpret_cast<float*>(a.out) + split * a.split_stride;
    const bool vec4 = (reinterpret_cast<uintptr_t>(outf) & 15) == 0 && (a.ldo & 3) == 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + 16 * j + 4 * q;
      float bias[4] = {0.f, 0.f, 0.f, 0.f};
      if (HAS_BIAS && split == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t c = min<int64_t>(n + r, a.N - 1);
          bias[r] = a.bias_bf16 ? bf16f(reinterpret_cast<const uint16_t*>(a.bias)[c])
                                : reinterpret_cast<const float*>(a.bias)[c];
        }
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int ml = mrow + 16 * i + l16;
        if (ml >= m_size) continue;
        float* o = outf + (m0 + ml) * a.ldo + n;
        const float v[4] = {acc[i][j][0] + bias[0], acc[i][j][1] + bias[1], acc[i][j][2] + bias[2],
                            acc[i][j][3] + bias[3]};
        if (vec4 && n + 4 <= a.N) {
          *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < a.N) o[r] = v[r];
        }
      }
    }
    return;
  }

  // epilogue: lane owns rows mrow + 16 i + l16, columns n0 + wn*64 + 16 j + 4 q .. + 3.  Each
  // wave's WROWS x 64 bf16 block goes through LDS (the operand stages are free) and leaves as
  // 16-byte row chunks; chunk c of row r sits at chunk c ^ (r & 7).
  __syncthreads();
  uint8_t* region = sOps + wave * WROWS * 128;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 64 + 16 * j + 4 * q;
    float bias[4] = {0.f, 0.f, 0.f, 0.f};
    if (HAS_BIAS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t c = min<int64_t>(n + r, a.N - 1);
        bias[r] = a.bias_bf16 ? bf16f(reinterpret_cast<const uint16_t*>(a.bias)[c])
                              : reinterpret_cast<const float*>(a.bias)[c];
      }
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = 16 * i + l16;
      const int pc = (2 * j + (q >> 1)) ^ (row & 7);
      uint2 pk;
      pk.x = pack_bf16x2(acc[i][j][0] + bias[0], acc[i][j][1] + bias[1]);
      pk.y = pack_bf16x2(acc[i][j][2] + bias[2], acc[i][j][3] + bias[3]);
      *reinterpret_cast<uint2*>(region + row * 128 + pc * 16 + (q & 1) * 8) = pk;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  const bool vec = (reinterpret_cast<uintptr_t>(a.out) & 15) == 0 && (a.ldo & 7) == 0;
  constexpr int CH = WROWS / 8;  // 16-byte chunks per lane
#pragma unroll
  for (int it = 0; it < CH; ++it) {
    const int id = it * 64 + lane;
    const int row = id >> 3, pc = id & 7;
    const i32x4 v = *reinterpret_cast<const i32x4*>(region + row * 128 + pc * 16);
    const int c = pc ^ (row & 7);
    const int ml = mrow + row;
    if (ml >= m_size) continue;
    const int64_t n = n0 + wn * 64 + c * 8;
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + (m0 + ml) * a.ldo + n;
    if (vec && n + 8 <= a.N) {
      __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(o));
    } else {
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
      for (int r = 0; r < 8 && n + r < a.N; ++r) o[r] = e[r];
    }
  }
}

template <int BM, int WFMT>
static void launch_mx_t(const MxArgs& a, hipStream_t st) {
  const int64_t row_tiles = cdiv(a.M, int64_t(BM)), n_tiles = cdiv(a.N, int64_t(256));
  const unsigned chunks = a.k_split > 1 ? unsigned(a.k_split) : 1u;
  const dim3 grid(static_cast<unsigned>(cdiv(row_tiles * n_tiles, 8) * 8), chunks), block(512);
  if (chunks > 1) {
    if (a.bias)
      hipLaunchKernelGGL((gemm_mx_kernel<BM, WFMT, true, true>), grid, block, 0, st, a, row_tiles, n_tiles);
    else
      hipLaunchKernelGGL((gemm_mx_kernel<BM, WFMT, false, true>), grid, block, 0, st, a, row_tiles, n_tiles);
    return;
  }
  if (a.bias)
    hipLaunchKernelGGL((gemm_mx_kernel<BM, WFMT, true>), grid, block, 0, st, a, row_tiles, n_tiles);
  else
    hipLaunchKernelGGL((gemm_mx_kernel<BM, WFMT, false>), grid, block, 0, st, a, row_tiles, n_tiles);
}

// 128-row tiles up to 128 rows, and wherever they fit the 256 compute units in one round: each
// tile runs its K range as one serial chain, so below a full GPU more, smaller tiles finish
// sooner; 256-row tiles otherwise.
#ifndef MXQ_MX_FILL
#define MXQ_MX_FILL 1
#endif
void launch_gemm_mx(const MxArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return;
  const bool small = a.M <= 128 || (MXQ_MX_FILL && cdiv(a.M, int64_t(128)) * cdiv(a.N, int64_t(256)) <= 256);
  if (a.w_fmt == MX_W_E2M1) {
    if (small) launch_mx_t<128, MX_W_E2M1>(a, st); else launch_mx_t<256, MX_W_E2M1>(a, st);
  } else {
    if (small) launch_mx_t<128, MX_W_E4M3>(a, st); else launch_mx_t<256, MX_W_E4M3>(a, st);
  }
}

// ---------------------------------------------------------------- MXFP8 quantiser

// Per row, per 32 columns: e = max(floor(log2(amax)) - 8, -127) (from amax's exponent field;
// zero and subnormal maxima give -127), scale code e + 127, codes e4m3_rne(clamp(x * 2^-e,
// +-448)) -- the multiplication by 2^-e is exact (a normal power of two: -127 <= e <= 119 for
// bf16 input).  Four lanes cover a 32-column block, eight values each.
__global__ __launch_bounds__(256) void quant_mx_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       int64_t ldx, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ s) {
  const int64_t per_row = K / 8;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool valid = idx < M * per_row;
  const int64_t ii = valid ? idx : 0;
  const int64_t row = ii / per_row, col = (ii - row * per_row) * 8;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (valid) raw = *reinterpret_cast<const uint4*>(x + row * ldx + col);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16lo(w[i]);
    v[2 * i + 1] = bf16hi(w[i]);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
  const int eb = int((__float_as_uint(amax) >> 23) & 0xffu);
  const int e = max(eb - 127 - 8, -127);
  const float inv = __uint_as_float(uint32_t(127 - e) << 23);  // 2^-e
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(v[i] * inv, -448.0f), 448.0f);
  if (valid) {
    uint2 qv;
    qv.x = cvt_pk_e4m3(v[0], v[1]) | (cvt_pk_e4m3(v[2], v[3]) << 16);
    qv.y = cvt_pk_e4m3(v[4], v[5]) | (cvt_pk_e4m3(v[6], v[7]) << 16);
    *reinterpret_cast<uint2*>(q + row * K + col) = qv;
    if ((threadIdx.x & 3) == 0) s[row * (K / 32) + col / 32] = uint8_t(e + 127);
  }
}

void launch_quant_mx(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, uint8_t* s,
                     hipStream_t stream) {
  const int64_t threads = M * (K / 8);
  if (threads == 0) return;
  hipLaunchKernelGGL(quant_mx_kernel, dim3(unsigned(cdiv(threads, 256))), dim3(256), 0, stream, x, M, K, ldx, q, s);
}

}  // namespace mxq
