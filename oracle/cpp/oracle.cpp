// Plain C++ CPU oracle of the scaled low-precision GEMM / routed fused-MoE path.
//
// TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's CPU baseline load
// it.  It shares no code, header, table or constant with the HIP library; every codec and
// every step is written out here from the definitions on the source pages, as explicit loops:
// operands decoded exactly and scaled in fp32, products and sums in double in ascending K
// order, one rounding to fp32, then bf16 (round to nearest even).  OpenMP splits output rows
// across threads; every output element is computed by one thread in a fixed order, so the
// results do not depend on the thread count.
//
// Sources (cited by title and section):
//  * "SGLang PR 35605 review" -- implementation item 1 and the fp8_utils.py listing: per-token
//    1x128 group quantisation (scale = amax / 448) and the block-FP8 W8A8 linear with
//    [ceil(N/block_n), K/128] weight scales;
//  * "SGLang PR 32618 review" -- implementation items 1-2 and the test_gemm.py listing: the
//    per-tensor FP8 W8A16 GEMM, out = bf16((A @ W^T) * scale + bias);
//  * "vLLM PR 50949 review" -- implementation item 2 and the moe_fp8.cpp listing: routed
//    experts, stage 1 into a 2I-wide gate/up intermediate (+ w1 bias), the activation, stage 2;
//    FP8 block and MXFP4 (e2m1 + e8m0 per 32) weights.
//
// Readings shared with the numpy oracle: eps 1e-10 for an all-zero group, IEEE fp32 divisions
// in the quantiser, clamp to +-448, e4m3 round to nearest even; w1 rows [0, I) gate and
// [I, 2I) up; silu(g) = g / (1 + exp(-g)) in double; ic0 and ic1 rounded to bf16; with W8A8
// both stage inputs quantised per token per 128 columns; y and the combine in fp32 / double;
// top-k weights applied at the combine, k ascending.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// ---------------------------------------------------------------- codecs

float bits_f32(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
uint32_t f32_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

float bf16_to_f32(uint16_t b) { return bits_f32(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest, ties to even (NaN -> quiet NaN)
uint16_t f32_to_bf16(float f) {
  const uint32_t u = f32_bits(f);
  if (std::isnan(f)) return uint16_t(((u >> 16) & 0x8000u) | 0x7FC0u);
  const uint32_t upper = u >> 16, lower = u & 0xFFFFu;
  const bool up = lower > 0x8000u || (lower == 0x8000u && (upper & 1u));
  return uint16_t(upper + (up ? 1u : 0u));
}

// e4m3 (OCP FP8 E4M3FN): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
// subnormal (m / 8) * 2^-6; 0x7F / 0xFF are NaN; no infinities.
double e4m3_value(uint8_t c) {
  const double sign = (c & 0x80) ? -1.0 : 1.0;
  const int e = (c >> 3) & 0xF, m = c & 0x7;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0) return sign * m * std::ldexp(1.0, -9);
  return sign * (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
}

struct E4m3Table {
  double v[256];
  E4m3Table() {
    for (int c = 0; c < 256; ++c) v[c] = e4m3_value(uint8_t(c));
  }
};
const E4m3Table& e4m3() {
  static const E4m3Table t;
  return t;
}

// |v| <= 448 -> nearest e4m3 code, ties to the even code, sign copied (-0 -> 0x80).
// Codes 0x00 .. 0x7E hold the finite non-negative values in ascending order.
uint8_t e4m3_encode(float v) {
  const double a = std::fabs(double(v));
  const double* t = e4m3().v;
  int lo = 0, hi = 0x7E;  // t[lo] <= a by construction after the search
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (t[mid] <= a) lo = mid; else hi = mid;
  }
  if (t[hi] <= a) lo = hi;
  int code = lo;
  if (t[lo] != a && lo < 0x7E) {
    const double mid = (t[lo] + t[lo + 1]) / 2.0;
    if (a > mid || (a == mid && ((lo + 1) % 2 == 0))) code = lo + 1;
  }
  return uint8_t(code | (std::signbit(v) ? 0x80 : 0));
}

// e2m1 (OCP MX FP4): sign, 2 exponent bits (bias 1), 1 mantissa bit
double e2m1_value(uint8_t nib) {
  const double sign = (nib & 0x8) ? -1.0 : 1.0;
  const int e = (nib >> 1) & 0x3, m = nib & 0x1;
  if (e == 0) return sign * m * 0.5;
  return sign * (1.0 + m / 2.0) * std::ldexp(1.0, e - 1);
}

// e8m0: 2^(c - 127); 0xFF is NaN
double e8m0_value(uint8_t c) { return c == 0xFF ? NAN : std::ldexp(1.0, int(c) - 127); }

// ---------------------------------------------------------------- quantisation

// One row of K values (K % 128 == 0) -> codes and K/128 scales:
// s = max(amax, 1e-10) / 448 (fp32 division), q = e4m3(clamp(x / s, +-448)) (fp32 division).
void quant_row_1x128(const float* x, int64_t K, uint8_t* q, float* s) {
  for (int64_t g = 0; g < K / 128; ++g) {
    float amax = 0.f;
    for (int i = 0; i < 128; ++i) amax = std::fmax(amax, std::fabs(x[g * 128 + i]));
    const float sc = std::fmax(amax, 1e-10f) / 448.0f;
    s[g] = sc;
    for (int i = 0; i < 128; ++i) {
      float v = x[g * 128 + i] / sc;
      v = std::fmin(std::fmax(v, -448.0f), 448.0f);
      q[g * 128 + i] = e4m3_encode(v);
    }
  }
}

// ---------------------------------------------------------------- expert weights

// Weight element (row n, column k) of one expert, decoded and scaled in fp32.
struct ExpertWeights {
  int fmt;             // 0: e4m3 + fp32 128x128 block scales; 1: packed e2m1 + e8m0 per 32
  const uint8_t* w;    // [N, K] codes or [N, K/2] packed
  const void* s;       // fp32 [ceil(N/128), K/128] or uint8 [N, K/32]
  int64_t N, K;
  float at(int64_t n, int64_t k) const {
    if (fmt == 0) {
      const float* sg = static_cast<const float*>(s);
      return float(e4m3().v[w[n * K + k]]) * sg[(n / 128) * (K / 128) + k / 128];
    }
    const uint8_t byte = w[n * (K / 2) + k / 2];
    const uint8_t nib = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    const uint8_t* se = static_cast<const uint8_t*>(s);
    return float(e2m1_value(nib) * e8m0_value(se[n * (K / 32) + k / 32]));
  }
  // the whole matrix in fp32 (row-major [N, K])
  std::vector<float> dequant() const {
    std::vector<float> out(size_t(N) * K);
    for (int64_t n = 0; n < N; ++n)
      for (int64_t k = 0; k < K; ++k) out[size_t(n) * K + k] = at(n, k);
    return out;
  }
};

// sum_k a[k] * w[k] in double, ascending k, rounded once to fp32
float dot_f32(const float* a, const float* w, int64_t K) {
  double acc = 0.0;
  for (int64_t k = 0; k < K; ++k) acc += double(a[k]) * double(w[k]);
  return float(acc);
}

}  // namespace

extern "C" {

int orc_threads() {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// bf16 [M, K] -> e4m3 [M, K] + fp32 [M, K/128]
void orc_quant_1x128(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    std::vector<float> row(K);
    for (int64_t k = 0; k < K; ++k) row[k] = bf16_to_f32(x[m * K + k]);
    quant_row_1x128(row.data(), K, q + m * K, s + m * (K / 128));
  }
}

// per-tensor W8A16: out_f32[m, n] = f32(sum_k a * dec(w)) * scale + bias[n]   (fp32 result)
void orc_fp8_scaled_mm_f32(const uint16_t* A, const uint8_t* W, int64_t M, int64_t N, int64_t K, float scale,
                           const float* bias, float* out) {
  const double* t = e4m3().v;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += double(bf16_to_f32(A[m * K + k])) * double(float(t[W[n * K + k]]));
      float v = float(acc) * scale;
      if (bias) v = v + bias[n];
      out[m * N + n] = v;
    }
  }
}

// block-FP8 W8A8 on pre-quantised activations:
// out_f32[m, n] = f32(sum_k (dec(qa) * sa[m, k/128]) * (dec(w) * sw[n/bn, k/128])) + bias[n]
void orc_block_fp8_linear_f32(const uint8_t* qa, const float* sa, const uint8_t* W, const float* sw, int64_t M,
                              int64_t N, int64_t K, int32_t block_n, const float* bias, float* out) {
  const double* t = e4m3().v;
  const int64_t KB = K / 128;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    std::vector<float> a(K);
    for (int64_t k = 0; k < K; ++k) a[k] = float(t[qa[m * K + k]]) * sa[m * KB + k / 128];
    std::vector<float> w(K);
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t k = 0; k < K; ++k) w[k] = float(t[W[n * K + k]]) * sw[(n / block_n) * KB + k / 128];
      float v = dot_f32(a.data(), w.data(), K);
      if (bias) v = v + bias[n];
      out[m * N + n] = v;
    }
  }
}

// bf16 activations: quantise per token per 128 columns, then the W8A8 linear; bf16 out
void orc_block_fp8_linear_bf16(const uint16_t* x, const uint8_t* W, const float* sw, int64_t M, int64_t N, int64_t K,
                               int32_t block_n, const float* bias, uint16_t* out) {
  std::vector<uint8_t> q(size_t(M) * K);
  std::vector<float> s(size_t(M) * (K / 128)), o(size_t(M) * N);
  orc_quant_1x128(x, M, K, q.data(), s.data());
  orc_block_fp8_linear_f32(q.data(), s.data(), W, sw, M, N, K, block_n, bias, o.data());
  for (size_t i = 0; i < o.size(); ++i) out[i] = f32_to_bf16(o[i]);
}

// Routed fused MoE: loops over experts e = 0 .. E-1 and, inside one expert, over its routed
// rows r = t * topk + k in ascending order.  wfmt 0: e4m3 weights with fp32 128x128 block
// scales (w1 [E, 2I, H], s1 [E, ceil(2I/128), H/128]; w2 [E, H, I], s2 [E, ceil(H/128), I/128]);
// wfmt 1: packed e2m1 with e8m0 per 32 (w1 [E, 2I, H/2], s1 [E, 2I, H/32]; w2 [E, H, I/2],
// s2 [E, H, I/32]).  b1: NULL or fp32 [E, 2I].  act_quant (e4m3 weights only): both stage
// inputs quantised per token per 128 columns.  Returns 0, or 1 for an expert id outside [0, E).
int orc_fused_moe(const uint16_t* x, int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk, const int32_t* ids,
                  const float* wts, int32_t wfmt, const uint8_t* w1, const void* s1, const uint8_t* w2,
                  const void* s2, const float* b1, int32_t act_quant, uint16_t* out) {
  const int64_t R = M * topk;
  for (int64_t r = 0; r < R; ++r)
    if (ids[r] < 0 || ids[r] >= E) return 1;
  // stage-1 input rows: bf16 values, or the dequantised 1x128 quantisation of x
  std::vector<float> xin(size_t(M) * H);
  for (int64_t i = 0; i < M * H; ++i) xin[i] = bf16_to_f32(x[i]);
  if (act_quant) {
    std::vector<uint8_t> q(size_t(M) * H);
    std::vector<float> s(size_t(M) * (H / 128));
    orc_quant_1x128(x, M, H, q.data(), s.data());
    for (int64_t t = 0; t < M; ++t)
      for (int64_t k = 0; k < H; ++k)
        xin[t * H + k] = float(e4m3().v[q[t * H + k]]) * s[t * (H / 128) + k / 128];
  }
  std::vector<float> y(size_t(R) * H, 0.f);
  const size_t w1_elems = wfmt == 0 ? size_t(2 * I) * H : size_t(2 * I) * (H / 2);
  const size_t w2_elems = wfmt == 0 ? size_t(H) * I : size_t(H) * (I / 2);
  const size_t s1_elems = wfmt == 0 ? size_t((2 * I + 127) / 128) * (H / 128) : size_t(2 * I) * (H / 32);
  const size_t s2_elems = wfmt == 0 ? size_t((H + 127) / 128) * (I / 128) : size_t(H) * (I / 32);
  const size_t sbytes = wfmt == 0 ? 4 : 1;
  for (int32_t e = 0; e < E; ++e) {
    std::vector<int64_t> rows;
    for (int64_t r = 0; r < R; ++r)
      if (ids[r] == e) rows.push_back(r);
    if (rows.empty()) continue;  // an expert with no rows is never read
    const ExpertWeights W1{wfmt, w1 + e * w1_elems, static_cast<const uint8_t*>(s1) + e * s1_elems * sbytes,
                           2 * I, H};
    const ExpertWeights W2{wfmt, w2 + e * w2_elems, static_cast<const uint8_t*>(s2) + e * s2_elems * sbytes, H, I};
    const std::vector<float> d1 = W1.dequant(), d2 = W2.dequant();
#pragma omp parallel for schedule(static)
    for (size_t ri = 0; ri < rows.size(); ++ri) {
      const int64_t r = rows[ri];
      const float* a = xin.data() + (r / topk) * H;
      // stage 1 (+ bias), rounded to bf16
      std::vector<float> ic0(2 * I);
      for (int64_t n = 0; n < 2 * I; ++n) {
        float v = dot_f32(a, d1.data() + n * H, H);
        if (b1) v = v + b1[e * 2 * I + n];
        ic0[n] = bf16_to_f32(f32_to_bf16(v));
      }
      // SiLU-and-mul in double, rounded fp64 -> fp32 -> bf16
      std::vector<float> ic1(I);
      for (int64_t j = 0; j < I; ++j) {
        const double g = ic0[j], u = ic0[I + j];
        const double act = g / (1.0 + std::exp(-g));
        ic1[j] = bf16_to_f32(f32_to_bf16(float(act * u)));
      }
      if (act_quant) {
        std::vector<uint8_t> q(I);
        std::vector<float> s(I / 128);
        quant_row_1x128(ic1.data(), I, q.data(), s.data());
        for (int64_t j = 0; j < I; ++j) ic1[j] = float(e4m3().v[q[j]]) * s[j / 128];
      }
      // stage 2 (fp32)
      for (int64_t n = 0; n < H; ++n) y[r * H + n] = dot_f32(ic1.data(), d2.data() + n * I, I);
    }
  }
  // top-k combine in double, k ascending, rounded once to fp32, then bf16
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < M; ++t)
    for (int64_t n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int32_t k = 0; k < topk; ++k) acc += double(wts[t * topk + k]) * double(y[(t * topk + k) * H + n]);
      out[t * H + n] = f32_to_bf16(float(acc));
    }
  return 0;
}

// fp32 -> bf16 bits (round to nearest even), for callers of the *_f32 entry points
void orc_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

// every e4m3 code's value (for the exhaustive table pin)
void orc_e4m3_table(double* out) {
  for (int c = 0; c < 256; ++c) out[c] = e4m3().v[c];
}

}  // extern "C"
